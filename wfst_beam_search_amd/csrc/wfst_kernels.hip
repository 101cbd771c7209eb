// gfx950 (CDNA4) kernels of the WFST Viterbi beam search.
//
// Semantics: page "GPU WFST Beam-Search Decoder" (OASR docs), sections 1, 3,
// 5.1-5.5 and 7. Design (ours, for 64-wide wavefronts):
//  * every frontier token owns a contiguous range of "slots" (its arcs of the
//    step's class); the ranges of all lanes form one flattened slot space cut
//    into 64-slot strips, and each wavefront walks a contiguous run of strips
//    with a forward token cursor resolved by a 6-shuffle search over a
//    register-held window of 64 token offsets (section 5.2/5.3 problem, wave64
//    solution);
//  * the slot pass (k_max) takes the exact per-lane maximum M with the
//    per-token upper-bound skip (section 5.3: (s+w)+lp <= (s+maxw)+maxlp holds
//    in IEEE fp32; a token whose state has at most kTopArcs emitting arcs
//    carries its exact best candidate instead), its running maximum seeded
//    with a lower bound the previous compaction posted; in the same walk it lists every candidate with
//    end > running max - b, a superset of the admitted ones (end > M - b), and
//    recombines them per destination in a direct-mapped per-lane table
//    best[state] with one posted u64 atomicMax of (ordered score | ~arc), so
//    the greatest score wins and, among equal scores, the smallest arc id;
//  * the compaction (k_finalize), with M known, admits from the list, keeps
//    the candidate of each destination whose key is the table entry (the
//    winner) and compacts the winners into the next frontier: one 64-bit
//    atomicAdd per wavefront allocates token positions and arc offsets
//    together (tokens in the low half, arcs in the high half), which is the
//    exclusive degree scan of the next step, done as the frontier is built;
//    the winners-log entry {source entry, arc} is written;
//  * epsilon closure passes (expand, then decide-and-apply) on TLG graphs;
//  * around the search: streams, the lattice and its backward prune,
//    winners-log compaction, blank-skip slicing.
// All fp32 arithmetic is single operations in the order the page fixes; the
// file is compiled with -ffp-contract=off.
#include <hip/hip_ext.h>
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "wfst_internal.h"

namespace wfst {

constexpr uint32_t kOrdNegInf = 0x007FFFFFu;  // ordered code of -inf

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t f2ord(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0.0 orders as +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float ord2f(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ unsigned long long cand_key(float score, int32_t arc)
{
    return ((unsigned long long)f2ord(score) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)arc);
}

// Epoch of recombination round (t, k): step t's slot pass is k = 0, closure
// pass k after it is k (t = -1: the start closure), counted on from the rounds
// of earlier sequences since the last clear. 1..epoch_period; 0 marks an empty
// entry. Kernels compute it once (the modulus is not a constant).
__device__ __forceinline__ uint32_t round_epoch(const Work &w, int t, int k)
{
    const uint32_t q = w.round_base + (uint32_t)((t + 1) * (1 + w.eps_iterations) + k);
    return 1u + q % w.epoch_period;
}

// State id of a destination field. When the graph stores ranks, arc records
// (and the candidates made from them) carry, above the state id, the arc's
// rank among its destination's incoming arcs, counted in arc id order.
__device__ __forceinline__ uint32_t dest_state(const Work &w, int32_t d) { return (uint32_t)d & w.dest_mask; }

// The graph's id of the arc at record position a; a redirect's virtual arc
// (num_arcs + state) keeps its offset past the graph's arcs.
__device__ __forceinline__ int32_t user_arc(const Work &w, int32_t a)
{
    if (a < 0) return a;
    return a < w.num_arcs ? w.arc_uid[a] : w.num_arcs_user + (a - w.num_arcs);
}

// Key of a candidate (arc, packed destination field pd) in the recombination
// table. With epochs: epoch << (32 + a) | ordered score << a | (2^a - 1 - tie),
// a = tie_bits <= 25, where the tie is the arc's rank among its destination's
// incoming arcs (when the graph stores ranks) or its arc id. Every key of an
// earlier round is smaller than every key of the current one, so no entry needs
// clearing (the host wipes the table before the epoch counter wraps). Within a
// round all keys of one entry share its destination, whose incoming arcs rank
// in arc id order, so the order is cand_key's either way: greater score, then
// smaller arc id.
__device__ __forceinline__ unsigned long long table_key(const Work &w, float score, int32_t arc, int32_t pd,
                                                        uint32_t ep)
{
    if (!w.epochs) return cand_key(score, arc);
    const uint32_t a = w.tie_bits;
    const uint32_t tie = w.rank_ties ? (uint32_t)pd >> w.dest_bits : (uint32_t)arc;
    return ((unsigned long long)ep << (32 + a)) | ((unsigned long long)f2ord(score) << a) |
           (unsigned long long)(((1u << a) - 1u) - tie);
}

// ------------------------------------------- recombination: table or hash
// Where the candidates of destination state ds (lane L, round epoch ep) meet:
// the direct-mapped table's entry best[L][ds], or a slot of the lane's
// open-addressing hash (page section 5.3: a hash keyed on the destination,
// one 64-bit atomicMax per candidate): linear probing from a multiplicative
// hash of ds; a slot whose claim is of an earlier round is empty, and the
// first candidate of ds to reach one claims it with a CAS. Every slot between
// ds's first probe and its slot belongs to another destination of this round,
// so a lookup stops at the first slot of an earlier round. Null: the hash is
// full (the lane retires with the hash bit).
__device__ __forceinline__ uint32_t hash_first(const Work &w, uint32_t ds)
{
    return (ds * 0x9E3779B1u) >> (32u - w.hash_bits);
}

// On graphs with epsilon arcs there are two tables (and two candidate lists):
// round (t, k) uses table k & 1, so a kernel that resolves closure pass k can
// relax pass k + 1 into the other one. (One table otherwise: k is always 0.)
__device__ __forceinline__ int round_tab(const Work &w, int k) { return k & (w.ntab - 1); }

// Lane L's row of table tb.
__device__ __forceinline__ size_t tab_row(const Work &w, int tb, int L)
{
    return (size_t)tb * (size_t)w.max_lanes + (size_t)L;
}

// (HASH: the kernels are compiled once per recombination structure, so the
// default table path carries no probing code)
template <bool HASH>
__device__ __forceinline__ unsigned long long *recomb_entry(const Work &w, int tb, int L, uint32_t ds, uint32_t ep)
{
    if (!HASH) return w.best + tab_row(w, tb, L) * (size_t)w.num_states + ds;
    HSlot *h = w.hash + (tab_row(w, tb, L) << w.hash_bits);
    const uint32_t mask = (1u << w.hash_bits) - 1u;
    const unsigned long long want = ((unsigned long long)ep << 32) | ds;
    uint32_t i = hash_first(w, ds);
    for (uint32_t n = 0; n <= mask; ++n, i = (i + 1u) & mask) {
        const unsigned long long c = __hip_atomic_load(&h[i].claim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (c == want) return &h[i].key;
        if ((uint32_t)(c >> 32) == ep) continue;   // another destination's, this round
        const unsigned long long old = atomicCAS(&h[i].claim, c, want);
        if (old == c || old == want) return &h[i].key;
        // (claimed meanwhile for another destination: the next slot)
    }
    return nullptr;
}

// The key recorded for destination ds in round ep after the round's atomics
// (0 when none: a table entry of an earlier round never equals a key of this one).
template <bool HASH>
__device__ __forceinline__ unsigned long long recomb_key(const Work &w, int tb, int L, uint32_t ds, uint32_t ep)
{
    if (!HASH) return w.best[tab_row(w, tb, L) * (size_t)w.num_states + ds];
    const HSlot *h = w.hash + (tab_row(w, tb, L) << w.hash_bits);
    const uint32_t mask = (1u << w.hash_bits) - 1u;
    const unsigned long long want = ((unsigned long long)ep << 32) | ds;
    uint32_t i = hash_first(w, ds);
    for (uint32_t n = 0; n <= mask; ++n, i = (i + 1u) & mask) {
        const HSlot v = h[i];
        if (v.claim == want) return v.key;
        if ((uint32_t)(v.claim >> 32) != ep) return 0ull;
    }
    return 0ull;
}

__device__ __forceinline__ int wlane() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ unsigned long long mask_lt() { return (1ull << wlane()) - 1ull; }

__device__ __forceinline__ uint32_t wave_excl_sum(uint32_t v, uint32_t *total)
{
    uint32_t x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t y = __shfl_up(x, d, kWave);
        if (wlane() >= d) x += y;
    }
    *total = __shfl(x, kWave - 1, kWave);
    return x - v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, kWave));
    return v;
}

__device__ __forceinline__ float lp_at(const float *row, uint32_t i) { return row[i]; }
__device__ __forceinline__ float lp_at(const __half *row, uint32_t i) { return __half2float(row[i]); }

__device__ __forceinline__ uint32_t *step_rec(const Work &w, int L, int t)
{
    return w.steps + ((size_t)L * (size_t)(w.max_frames + 2) + (size_t)(t + 1)) * kStepFields;
}

// Phase of lane c at step t of the sequence: real for t < T, final at t == T,
// none outside the lane's window of this sequence.
__device__ __forceinline__ int lane_phase(const LaneCtl &c, int t)
{
    if (c.status != kActive || t >= c.win) return kPhNone;
    if (t < c.T) return kPhReal;
    if (t == c.T) return kPhFinal;
    return kPhNone;
}

// Whether lane c has a result: a final-step winner, or the redirect's best token
// (whose entry is -1 when it is the start token: an empty path). A result's
// score is never -inf (it was admitted, or is a token's score).
__device__ __forceinline__ bool lane_has_result(const LaneCtl &c)
{
    return c.final_entry >= 0 || c.final_score > -__builtin_inff();
}

// A lattice node past the lane's node capacity (possible only with log
// compaction, which lets a lane hold more tokens over a decode than log
// entries): the lane's lattice is marked incomplete (its cursor past
// lat_cap, the arena bit) and gets no backward pass.
__device__ __forceinline__ void lat_node_overflow(const Work &w, LaneCtl &c)
{
    atomicOr(&c.overflow, kOvfArena);
    atomicMax(&c.lat_cursor, w.lat_cap + 1u);
}

// Parity of the frontier that feeds lane c's step t of the sequence.
__device__ __forceinline__ int lane_par(const LaneCtl &c, int t) { return (c.base + t) & 1; }

// Tag of the tokens a round makes: (the lane's frame << 5) | closure pass, the
// frame being the one step t builds (its closure included); the lane's frames
// count on across a stream's calls. Passes are at most 16, frames wrap at 2^27.
__device__ __forceinline__ uint32_t frame_tag(const LaneCtl &c, int t)
{
    return ((uint32_t)(c.base + t + 1) & ((1u << 27) - 1u)) << 5;
}


// Buffer of parity p (wavefront-uniform) out of a pair: a select between the two
// pointers, which a kernel loads once, instead of an indexed load per use.
template <typename T>
__device__ __forceinline__ T *pick(T *const (&a)[2], int p) { return p ? a[1] : a[0]; }

// Both parities of a per-lane pair in one load, then the one of parity p: no
// load of a kernel's prologue waits for the lane's parity.
__device__ __forceinline__ unsigned long long pair_at(const unsigned long long (&a)[2], int p)
{
    const ulonglong2 v = *reinterpret_cast<const ulonglong2 *>(a);
    return p ? v.y : v.x;
}
__device__ __forceinline__ uint32_t pair_at(const uint32_t (&a)[2], int p)
{
    const uint2 v = *reinterpret_cast<const uint2 *>(a);
    return p ? v.y : v.x;
}
__device__ __forceinline__ float pair_at(const float (&a)[2], int p)
{
    const float2 v = *reinterpret_cast<const float2 *>(a);
    return p ? v.y : v.x;
}

// A lane's parity from the LDS table, as a wavefront-uniform value.
__device__ __forceinline__ int upar(const int32_t *par, int L) { return __builtin_amdgcn_readfirstlane(par[L]); }

// Commits the compaction of step t that no closure followed: its token count n
// is its number of winners and of winners-log entries. Run by one thread of the
// next kernel that reads the log.
__device__ __forceinline__ void commit_log(const Work &w, LaneCtl &c, int L, int t, uint32_t n)
{
    if (!c.log_open) return;
    c.log_cursor += n;
    step_rec(w, L, t)[kRecDistinct] = n;
    c.log_open = 0u;
}

// Per-workgroup view of the lanes, built by wavefront 0 of every workgroup.
struct LaneTab {
    uint32_t base[kMaxLanes + 1];  // exclusive prefix of work units per lane
    uint32_t n[kMaxLanes];         // items (tokens / claims / sources)
    uint32_t arcs[kMaxLanes];      // slots of the step
    int32_t ph[kMaxLanes];
    int32_t T[kMaxLanes];
    float f0[kMaxLanes];           // finalize: 1 if the candidate list fits; closure apply: 1 if it does not
    float f1[kMaxLanes];           // cutoff, or the running max
    uint32_t fb[kMaxLanes];        // winners-log base of the sources' compaction
    int32_t par[kMaxLanes];        // parity of the frontier the kernel reads (k_max, k_finalize)
                                   //   or closes (closure passes)
    int32_t row[kMaxLanes];        // batch row of the lane's log-probs (k_max, k_finalize); in a
                                   //   compaction round, the frontier's winners-log base (bits)
    int32_t win[kMaxLanes];        // the lane's window of the sequence (k_finalize)
};

__device__ __forceinline__ void tab_publish(LaneTab &tab, int nl, uint32_t units)
{
    uint32_t tot;
    uint32_t ex = wave_excl_sum(units, &tot);
    const int L = (int)threadIdx.x;
    if (L < nl) tab.base[L] = ex;
    if (L == 0) tab.base[nl] = tot;
}

__device__ __forceinline__ int find_lane(const uint32_t *base, int nl, uint32_t s)
{
    int lo = 0, hi = nl - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (base[mid] <= s) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Next-step class of a token at state s: [abeg, abeg + deg) and score + the
// class's largest weight (the final class's bound; emitting classes add the
// frame's largest log-prob, or use the exact best candidate, where known).
__device__ __forceinline__ void class_of(const StateInfo &si, bool final_step, float score,
                                         int32_t *abeg, uint32_t *deg, float *ub)
{
    if (final_step) {
        *abeg = si.fin_b; *deg = (uint32_t)(si.end - si.fin_b); *ub = score + si.fin_maxw;
    } else {
        *abeg = si.emit_b; *deg = (uint32_t)(si.fin_b - si.emit_b); *ub = score + si.top_w[0];
    }
}

// Writes the strip map for tokens just allocated by one wavefront: the keepers
// of this wave got positions p0 + rank and slot offsets a0 + dpre (dpre is the
// exclusive scan of the keepers' degrees, so over all 64 lanes a0 + dpre is
// non-decreasing and a non-keeper acts as a token without arcs). For every
// strip whose first slot lies in [a0, a0 + dsum) the token holding that slot is
// the last lane whose offset is <= the slot.
__device__ __forceinline__ void write_strips(uint32_t *strip_tok, uint32_t strip_cap, uint32_t p0,
                                             uint32_t a0, uint32_t dpre, uint32_t dsum,
                                             unsigned long long keep_mask)
{
    const uint32_t o = a0 + dpre;
    const uint32_t rank = (uint32_t)__popcll(keep_mask & mask_lt());
    const uint32_t sb0 = (a0 + kWave - 1) / kWave;
    const uint32_t sb1 = (a0 + dsum + kWave - 1) / kWave;
    for (uint32_t sb = sb0 + (uint32_t)wlane(); sb - (uint32_t)wlane() < sb1; sb += kWave) {
        const uint32_t slot = sb * kWave;
        int i = 0;
#pragma unroll
        for (int st = 32; st >= 1; st >>= 1) {
            const uint32_t v = __shfl(o, i + st, kWave);
            if (v <= slot) i += st;
        }
        const uint32_t r = __shfl(rank, i, kWave);
        if (sb < sb1 && sb < strip_cap) strip_tok[sb] = p0 + r;
    }
}

// Per-wavefront LDS buffer of the listed candidates of the slot pass and the
// closure's expand passes (a unit lists at most kUnit of them; 8 KB per
// wavefront, so four units' worth between the flushes' list atomics).
constexpr uint32_t kClaimBuf = 384;

struct ClaimBuf {
    int32_t dest[kClaimBuf];
    int32_t arc[kClaimBuf];
    uint32_t tok[kClaimBuf];
    uint32_t score[kClaimBuf];
};

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Appends the wave's n buffered candidates to lane L's list: one atomic, then a
// coalesced copy out of LDS.
__device__ __forceinline__ void flush_claims(const Work &w, int tb, int L, uint32_t *counter, ClaimBuf &cb,
                                             uint32_t n)
{
    wave_lds_sync();
    uint32_t base = 0;
    if (wlane() == 0) base = atomicAdd(counter, n);
    base = __shfl(base, 0, kWave);
    Claim *dst = w.claims + tab_row(w, tb, L) * w.claims_cap;
    for (uint32_t i = (uint32_t)wlane(); i < n; i += kWave) {
        Claim c;
        c.dest = cb.dest[i];
        c.arc = cb.arc[i];
        c.tok = cb.tok[i];
        c.score = cb.score[i];
        if (base + i < w.claims_cap) dst[base + i] = c;
    }
    wave_lds_sync();
}

// Buffers the candidates of one round of a wavefront (lanes with `adm` set),
// flushing first if the round might not fit.
__device__ __forceinline__ void push_claims(const Work &w, int tb, int L, uint32_t *counter, ClaimBuf &cb,
                                            uint32_t &cb_n, bool adm, int32_t dest, int32_t arc,
                                            uint32_t tok, float score)
{
    const unsigned long long fm = __ballot(adm);
    if (!fm) return;
    if (cb_n + kWave > kClaimBuf) {
        flush_claims(w, tb, L, counter, cb, cb_n);
        cb_n = 0;
    }
    if (adm) {
        const uint32_t i = cb_n + (uint32_t)__popcll(fm & mask_lt());
        cb.dest[i] = dest;
        cb.arc[i] = arc;
        cb.tok[i] = tok;
        cb.score[i] = __float_as_uint(score);
    }
    cb_n += (uint32_t)__popcll(fm);
}

// Reads candidate i of lane L's list and decides whether it is the winner of
// its destination in round epoch ep: its key is the table entry after the
// closure's expand pass. Without epochs the winner clears the entry (a loser
// reading after that sees 0, never its key).
template <bool HASH>
__device__ __forceinline__ bool take_winner(const Work &w, int tb, int L, uint32_t i, uint32_t ep, Claim &cl)
{
    cl = w.claims[tab_row(w, tb, L) * w.claims_cap + i];
    const uint32_t ds = dest_state(w, cl.dest);
    if (ds >= (uint32_t)w.num_states) return false;
    const bool win = recomb_key<HASH>(w, tb, L, ds, ep) == table_key(w, __uint_as_float(cl.score), cl.arc, cl.dest, ep);
    if (win && !w.epochs) w.best[tab_row(w, tb, L) * (size_t)w.num_states + ds] = 0ull;
    return win;
}

// ---------------------------------------------------------------- k_clear
// k = 0 (start of a decode): clears the per-step records and the recombination
// tables — with epoch-tagged keys all of them when the host asks (the decode's
// rounds would pass an epoch wrap; otherwise they number on from the last
// sequence's and every older entry loses), else those of lanes whose
// candidate list overflowed in an earlier decode (the targeted clears cannot
// see those entries). k = 1: clears every table (before the epoch counter
// wraps). k = 2 (start of a stream sequence): the records of the lanes the
// plan names, and without epochs the table of a lane being opened after an
// overflow.
__global__ __launch_bounds__(kBlock) void k_clear(const Work *__restrict__ wp, int k)
{
    const Work &w = *wp;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k == 2) {
        const size_t per = (size_t)(w.max_frames + 2) * kStepFields;
        const size_t ns = (size_t)w.num_states;
        for (int L = 0; L < w.max_lanes; ++L) {
            const int cmd = w.plan[L * kPlanFields + kPlanCmd];
            if (cmd == kCmdPark) continue;
            for (size_t i = tid; i < per; i += stride) w.steps[(size_t)L * per + i] = 0u;
            if (cmd == kCmdOpen && !w.epochs && w.ctl[L].dirty) {
                for (int tb = 0; tb < w.ntab; ++tb) {
                    unsigned long long *tbl = w.best + tab_row(w, tb, L) * ns;
                    for (size_t i = tid; i < ns; i += stride) tbl[i] = 0ull;
                }
            }
        }
        return;
    }
    if (k == 0) {
        const size_t nrec = (size_t)w.max_lanes * (size_t)(w.max_frames + 2) * kStepFields;
        for (size_t i = tid; i < nrec; i += stride) w.steps[i] = 0u;
    }
    const size_t ns = (size_t)w.num_states;
    if (w.epochs) {
        if (k == 0 && !w.wipe) return;
        // non-temporal 16-byte stores over the whole [L][num_states] table
        // (hipMalloc'd: 256-byte aligned), an odd last entry singly: the
        // zeros bypass the caches instead of leaving them full of dirty lines
        // that later kernels would have to write back
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
        // (the hash: two u64 per slot)
        unsigned long long *base = w.hash_bits ? (unsigned long long *)w.hash : w.best;
        const size_t n = (size_t)w.ntab * (w.hash_bits ? ((size_t)w.max_lanes << w.hash_bits) * 2u
                                                       : (size_t)w.max_lanes * ns);
        v4u *t4 = (v4u *)base;
        const v4u z = {0u, 0u, 0u, 0u};
        for (size_t i = tid; i < n / 2; i += stride) __builtin_nontemporal_store(z, &t4[i]);
        if (tid == 0 && (n & 1)) base[n - 1] = 0ull;
        return;
    }
    if (k != 0) return;
    for (int L = 0; L < w.max_lanes; ++L) {
        if (!w.ctl[L].dirty) continue;
        for (int tb = 0; tb < w.ntab; ++tb) {
            unsigned long long *tbl = w.best + tab_row(w, tb, L) * ns;
            for (size_t i = tid; i < ns; i += stride) tbl[i] = 0ull;
        }
    }
}

// ----------------------------------------------------------------- k_init
// Lane control blocks and the start token (page section 2: InitKernel resets all
// state, so a decode is idempotent).
// Fresh search state of lane L with T frames (T = INT32_MAX: a stream, whose end
// is not known yet): control block and start token at parity 0.
__device__ void init_lane(const Work &w, int L, int T)
{
    LaneCtl &c = w.ctl[L];
    c.T = T;
    c.status = kActive;
    c.overflow = 0u;
    c.log_full = 0u;
    c.reached_final = 0;
    c.beam[0] = w.beam;
    c.beam[1] = w.beam;
    c.maxkey[0] = kOrdNegInf;
    c.maxkey[1] = kOrdNegInf;
    c.lbkey[0] = kOrdNegInf;
    c.lbkey[1] = kOrdNegInf;
    c.cutoff = 0.0f - w.beam;
    c.nclaims[0] = 0u;
    c.nclaims[1] = 0u;
    c.log_cursor = 0u;
    c.final_entry = -1;
    c.final_key = 0ull;
    c.final_score = -__builtin_inff();
    c.nclaims_eps[0] = 0u;
    c.nclaims_eps[1] = 0u;
    c.nclaims_eps[2] = 0u;
    c.nchanged[0] = 0ull;
    c.log_open = 0u;
    c.front_base[0] = 0xFFFFFFFFu;
    c.front_base[1] = 0xFFFFFFFFu;
    c.last_step = -1;
    c.phase_final = kPhNone;
    c.base = 0;
    c.frames = 0;
    c.lat_cursor = 0u;
    c.lat_out_n = 0u;
    c.sealed = 0u;
    c.gc_on = 0u;
    c.cnt[1] = 0ull;
    const int32_t s = w.start_state;
    const StateInfo si = w.sinfo[s];
    int32_t abeg; uint32_t deg; float ub;
    class_of(si, T == 0, 0.0f, &abeg, &deg, &ub);
    if (T != 0) ub = __builtin_inff();   // (its frame's log-probs are not known here)
    const size_t q = (size_t)L * w.frontier_cap;
    w.tok_state[0][q] = s;
    if (w.eps_iterations > 0) w.tok_tag[0][q] = 0u;   // frame 0 of the lane, made before any pass
    w.tok_score[0][q] = 0.0f;
    w.tok_entry[0][q] = -1;
    w.tok_last[0][q] = -1;
    w.tok_off[0][q] = 0u;
    w.tok_abeg[0][q] = abeg;
    w.tok_ub[0][q] = ub;
    // (the position map exists only where a kernel reads it: epsilon graphs, lattices)
    if (w.has_eps || w.lattice) w.pos[0][(size_t)L * w.num_states + s] = 0;
    // the start closure's sources: the start token, if it has epsilon arcs
    const bool eps_src = w.eps_iterations > 0 && si.emit_b > si.eps_b;
    if (eps_src) {
        w.changed[1][(size_t)L * w.chg_cap] = make_int4(si.eps_b, si.emit_b - si.eps_b, -1, (int)__float_as_uint(0.0f));
        if (w.lattice) w.chg_pos[1][(size_t)L * w.chg_cap] = 0;
    }
    c.nchanged[1] = eps_src ? 1ull : 0ull;
    if (w.lattice) {
        // frame 0's first node is the start token; the start closure's arcs
        // open the lattice (step -1)
        const size_t F = (size_t)w.max_frames + 3;
        w.lat_nbase[(size_t)L * F] = 0u;
        w.lat_aoff[(size_t)L * F] = 0u;
        w.lat_score[(size_t)L * w.lat_nodes] = 0.0f;
        w.lat_state[(size_t)L * w.lat_nodes] = s;
    }
    uint32_t *st = w.strip_tok[0] + (size_t)L * w.strip_cap;
    for (uint32_t sb = 0; sb * kWave < deg && sb < w.strip_cap; ++sb) st[sb] = 0u;
    c.cnt[0] = 1ull | ((unsigned long long)deg << 32);
}

// Start of a decode: lanes of the batch (their lengths) from their start state,
// the others idle.
__global__ __launch_bounds__(kWave) void k_init(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)threadIdx.x;
    if (L >= w.max_lanes) return;
    const LpDesc d = *w.lp;
    LaneCtl &c = w.ctl[L];
    const bool on = L < d.B;
    c.dirty = 0u;        // the clear at the start of the decode has run
    c.win = 0x7FFFFFFF;
    c.lp_row = on ? L : -1;
    c.want = on ? 1 : 0;
    if (on) {
        init_lane(w, L, w.lengths[L]);
    } else {
        c.T = 0;
        c.status = kDone;
        c.overflow = 0u;
        c.final_entry = -1;
        c.final_score = -__builtin_inff();
        c.log_open = 0u;
        c.base = 0;
        c.cnt[0] = 0ull;
        c.cnt[1] = 0ull;
        c.last_step = -1;
        c.phase_final = kPhNone;
        c.lat_cursor = 0u;
        c.lat_out_n = 0u;
    }
}

// ---------------------------------------------------------------- k_lpmax
// Max log-prob of every (lane, frame) row, for the upper-bound skip.
template <typename LPT>
__global__ __launch_bounds__(kBlock) void k_lpmax(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const LpDesc d = *w.lp;
    const int wpb = kBlock / kWave;
    const long long rows = (long long)w.max_lanes * w.max_frames;
    for (long long r = (long long)blockIdx.x * wpb + threadIdx.x / kWave; r < rows;
         r += (long long)gridDim.x * wpb) {
        const int L = (int)(r / w.max_frames), t = (int)(r % w.max_frames);
        const LaneCtl &c = w.ctl[L];
        // the real steps of the sequence that read a row of this input
        if (c.status != kActive || c.lp_row < 0 || t >= c.T || t >= c.win) continue;
        const LPT *row = (const LPT *)d.base + (long long)c.lp_row * d.stride_b + (long long)t * d.stride_t;
        // 16-byte loads over the row's aligned middle, single elements around it
        // (the maximum does not depend on the order)
        constexpr uint32_t kPer = 16 / sizeof(LPT);
        const uint32_t V = (uint32_t)w.vocab;
        const uint32_t mis = (uint32_t)(((uintptr_t)row & 15u) / sizeof(LPT));
        const uint32_t head = min(V, mis ? kPer - mis : 0u);
        const uint32_t nvec = (V - head) / kPer;
        float m = -__builtin_inff();
        for (uint32_t v = wlane(); v < head; v += kWave) m = fmaxf(m, lp_at(row, v));
        const uint4 *vp = (const uint4 *)(row + head);
        for (uint32_t k = wlane(); k < nvec; k += kWave) {
            const uint4 q = vp[k];
            const LPT *e = (const LPT *)&q;
#pragma unroll
            for (uint32_t j = 0; j < kPer; ++j) m = fmaxf(m, lp_at(e, j));
        }
        for (uint32_t v = head + nvec * kPer + wlane(); v < V; v += kWave) m = fmaxf(m, lp_at(row, v));
        m = wave_max(m);
        if (wlane() == 0) w.lpmax[(size_t)L * w.max_frames + t] = m;
    }
}

// ------------------------------------------------- slot walk (max / expand)

// A wavefront walks its run of the flattened slot space in units of kUnit slots:
// lane l owns slots j0 + r*64 + l for r < kR, so one window of token offsets and
// one round of independent arc loads serve kR strips (memory-level parallelism
// for the latency-bound gathers; two strips balance that against finer units
// best on the HLG-scale graph).
constexpr int kR = 2;
constexpr uint32_t kUnit = kWave * kR;

// Candidates of one unit as seen by one lane of the wavefront.
struct UnitData {
    float e[kR];          // end score (valid where bit r of `live` is set)
    uint32_t arc[kR];
    int32_t dst[kR];      // destination
    uint32_t tok[kR];     // source token
    uint32_t live;        // bit r: slot r is a candidate whose arc was loaded
};

// The lane of the batch a wavefront is working on.
struct LaneView {
    int L, ph;
    uint32_t n, arcs;
    const uint32_t *off;
    const int32_t *abeg;
    const float *score;
    const float *ubv;
    const void *row;      // log-prob row of the step (null on the final step)
};

__device__ __forceinline__ LaneView lane_view(const Work &w, const LaneTab &tab, int t, const LpDesc &d, int L)
{
    LaneView v;
    const int p = upar(tab.par, L);
    const size_t qo = (size_t)L * w.frontier_cap;
    v.L = L;
    v.ph = tab.ph[L];
    v.n = tab.n[L];
    v.arcs = tab.arcs[L];
    v.off = pick(w.tok_off, p) + qo;
    v.abeg = pick(w.tok_abeg, p) + qo;
    v.score = pick(w.tok_score, p) + qo;
    v.ubv = pick(w.tok_ub, p) + qo;
    const long long eoff = (long long)tab.row[L] * d.stride_b + (long long)t * d.stride_t;
    v.row = (v.ph == kPhReal)
        ? (const void *)((const char *)d.base + eoff * (w.lp_dtype == 1 ? 2 : 4)) : nullptr;
    return v;
}

// Loads unit u of lane v.L: lane l of the wavefront resolves slots
// j0 + r*64 + l against register-held windows of 64 token offsets (start token
// `cur`, moved forward), then issues every arc load of the unit before using
// any. Tokens whose bound ub <= skip are not expanded (exact: ub is at least
// every candidate through the token, so none of its arcs ends above skip).
// The window of 64 token offsets a wavefront last loaded (lane l: token wb + l),
// kept across the units of a lane segment: consecutive units continue in token
// order, so a unit whose slots lie within the window resolves them without a
// load (at HLG scale a window covers several units' slots).
struct SlotWin {
    bool valid;
    uint32_t wb, o, o_next;
    int32_t ab;
    float sc, ub;
};

template <typename LPT>
__device__ __forceinline__ void load_unit(const Work &w, const LaneView &v, uint32_t u, uint32_t &cur,
                                          float skip, UnitData &ud, SlotWin &sw)
{
    const int lane = wlane();
    const uint32_t n = v.n;
    const uint32_t j0 = u * kUnit;
    uint32_t j[kR], tok[kR], toff[kR];
    int32_t ab[kR];
    float sc[kR], ub[kR];
    bool valid[kR], resolved[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        j[r] = j0 + (uint32_t)(r * kWave + lane);
        valid[r] = j[r] < v.arcs;
        resolved[r] = !valid[r];
        tok[r] = cur; toff[r] = 0; ab[r] = 0; sc[r] = 0.0f; ub[r] = 0.0f;
    }
    // (a carried window starts at or before cur, the token of the last slot before this unit)
    bool have = sw.valid;
    uint32_t wb = have ? sw.wb : cur;
    uint32_t o = sw.o, o_next = sw.o_next;
    int32_t ab_l = sw.ab;
    float sc_l = sw.sc, ub_l = sw.ub;
    for (;;) {
        if (!have) {
            const uint32_t idx = wb + (uint32_t)lane;
            const bool in = idx < n;
            o = in ? v.off[idx] : 0xFFFFFFFFu;
            ab_l = in ? v.abeg[idx] : 0;
            sc_l = in ? v.score[idx] : 0.0f;
            ub_l = in ? v.ubv[idx] : 0.0f;
            o_next = (wb + kWave < n) ? v.off[wb + kWave] : 0xFFFFFFFFu;
        }
        have = false;
        bool pending = false;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            int i = 0;
#pragma unroll
            for (int st = 32; st >= 1; st >>= 1) {
                const uint32_t x = __shfl(o, i + st, kWave);
                if (x <= j[r]) i += st;
            }
            const uint32_t g_o = __shfl(o, i, kWave);
            const int32_t g_ab = __shfl(ab_l, i, kWave);
            const float g_sc = __shfl(sc_l, i, kWave);
            const float g_ub = __shfl(ub_l, i, kWave);
            if (!resolved[r] && (i < kWave - 1 || j[r] < o_next)) {
                tok[r] = wb + (uint32_t)i; toff[r] = g_o; ab[r] = g_ab; sc[r] = g_sc; ub[r] = g_ub;
                resolved[r] = true;
            }
            pending |= !resolved[r];
        }
        if (__ballot(pending) == 0ull) break;
        wb += kWave;
    }
    sw.valid = true;
    sw.wb = wb; sw.o = o; sw.o_next = o_next; sw.ab = ab_l; sw.sc = sc_l; sw.ub = ub_l;
    cur = __shfl(tok[kR - 1], kWave - 1, kWave);

    const LPT *row = (const LPT *)v.row;
    float wt[kR];
    uint32_t il[kR];
    ud.live = 0u;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        ud.arc[r] = (uint32_t)ab[r] + (j[r] - toff[r]);
        ud.tok[r] = tok[r];
        const bool go = valid[r] && tok[r] < n && ud.arc[r] < (uint32_t)w.num_arcs && ub[r] > skip;
        if (go) ud.live |= 1u << r;
        // {dest, ilabel, weight} in one 12-byte record
        ArcDLW a = {0, 0u, 0.0f};
        if (go) a = w.arc_dlw[ud.arc[r]];
        wt[r] = a.weight;
        il[r] = a.ilabel;
        ud.dst[r] = a.dest;
    }
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        float e = sc[r] + wt[r];
        if (row) e = e + (((ud.live >> r) & 1u) ? lp_at(row, il[r]) : 0.0f);
        ud.e[r] = e;
    }
}

__device__ __forceinline__ float unit_max(const UnitData &ud)
{
    float m = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < kR; ++r)
        if ((ud.live >> r) & 1u) m = fmaxf(m, ud.e[r]);
    return wave_max(m);
}

// Admits a unit's candidates into the step's superset (end > cut, strict, with
// cut = running max - b <= M - b, so every candidate the exact cutoff will admit
// is in) and recombines them: on a real step with one posted u64 atomicMax per
// candidate on the lane's direct-mapped table, on the final step with one
// wavefront-reduced atomicMax of the lane's final key. Every candidate of the
// superset goes to the wavefront's LDS buffer, then to the lane's list.
template <bool HASH>
__device__ __forceinline__ void admit_unit(const Work &w, int L, int ph, float cut, uint32_t ep,
                                           const UnitData &ud, uint32_t *counter, ClaimBuf *cb, uint32_t &cb_n)
{
    LaneCtl &c = w.ctl[L];
    const int lane = wlane();
    bool adm[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) adm[r] = ((ud.live >> r) & 1u) && ud.e[r] > cut;
    if (ph == kPhReal) {
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            if (!adm[r]) continue;
            unsigned long long *ent = recomb_entry<HASH>(w, 0, L, dest_state(w, ud.dst[r]), ep);
            if (ent) atomicMax(ent, table_key(w, ud.e[r], (int32_t)ud.arc[r], ud.dst[r], ep));
            else atomicOr(&c.overflow, kOvfHash);
        }
    } else {
        unsigned long long fkey = 0ull;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            if (adm[r]) {
                const unsigned long long k = cand_key(ud.e[r], (int32_t)ud.arc[r]);
                fkey = k > fkey ? k : fkey;
            }
        }
#pragma unroll
        for (int dd = kWave / 2; dd >= 1; dd >>= 1) {
            const unsigned long long o = __shfl_xor(fkey, dd, kWave);
            fkey = o > fkey ? o : fkey;
        }
        if (lane == 0 && fkey) atomicMax(&c.final_key, fkey);
    }
#pragma unroll
    for (int r = 0; r < kR; ++r)
        push_claims(w, 0, L, counter, *cb, cb_n, adm[r], ud.dst[r], (int32_t)ud.arc[r], ud.tok[r], ud.e[r]);
}

// XCD-aware block order: workgroups are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8), so block b takes virtual position
// (b % 8) * (grid / 8) + b / 8 and each XCD works on one contiguous eighth of a
// kernel's unit space. Lanes are laid out in the same order in every kernel's
// space, so a lane's tokens, strips and candidates are mostly written and read
// again on the same XCD, where they are still in that XCD's L2.
__device__ __forceinline__ uint32_t vblock()
{
    const uint32_t g = gridDim.x;
    if (g & 7u) return blockIdx.x;
    return (blockIdx.x & 7u) * (g >> 3) + (blockIdx.x >> 3);
}

// This wavefront's contiguous, equal share [s, s_end) of `total` units.
__device__ __forceinline__ void wave_share(uint32_t total, uint32_t *s, uint32_t *s_end)
{
    const uint32_t wpb = kBlock / kWave;
    const uint32_t nwaves = gridDim.x * wpb;
    const uint32_t wid = vblock() * wpb + threadIdx.x / kWave;
    *s = (uint32_t)(((unsigned long long)total * wid) / nwaves);
    *s_end = (uint32_t)(((unsigned long long)total * (wid + 1)) / nwaves);
}

// The end of the walk for the whole workgroup: each wavefront's last lane
// segment (lane L, n buffered candidates, running max run; L < 0: none) is
// posted with one list allocation and one maximum atomic per lane of the
// workgroup instead of one per wavefront, then every wavefront copies its
// buffer to its part of the allocation.
__device__ __forceinline__ void wg_post(const Work &w, const LaneTab &tab, int L, float run, uint32_t n,
                                        ClaimBuf *cb)
{
    constexpr int kW = kBlock / kWave;
    __shared__ int32_t agL[kW];
    __shared__ uint32_t agN[kW], agB[kW];
    __shared__ float agR[kW];
    const int wv = (int)(threadIdx.x / kWave);
    if (wlane() == 0) { agL[wv] = L; agN[wv] = n; agR[wv] = run; }
    __syncthreads();
    if (threadIdx.x < (unsigned)kW) {
        const int i = (int)threadIdx.x;
        const int Li = agL[i];
        bool first = Li >= 0;
        for (int j = 0; j < i; ++j) first = first && agL[j] != Li;
        if (first) {
            uint32_t tot = 0;
            float r = -__builtin_inff();
            for (int j = i; j < kW; ++j)
                if (agL[j] == Li) { tot += agN[j]; r = fmaxf(r, agR[j]); }
            const int p = tab.par[Li];
            LaneCtl &c = w.ctl[Li];
            uint32_t base = tot ? atomicAdd(&c.nclaims[p], tot) : 0u;
            if (r > -__builtin_inff()) atomicMax(&c.maxkey[p], f2ord(r));
            for (int j = i; j < kW; ++j)
                if (agL[j] == Li) { agB[j] = base; base += agN[j]; }
        }
    }
    __syncthreads();
    if (L >= 0 && n) {
        const uint32_t base = agB[wv];
        Claim *dst = w.claims + tab_row(w, 0, L) * w.claims_cap;
        for (uint32_t i = (uint32_t)wlane(); i < n; i += kWave) {
            Claim c;
            c.dest = cb->dest[i];
            c.arc = cb->arc[i];
            c.tok = cb->tok[i];
            c.score = cb->score[i];
            if (base + i < w.claims_cap) dst[base + i] = c;
        }
    }
}

// The workgroup's contiguous share [s, s_end) of `total` units: the union of
// its wavefronts' wave_share runs.
__device__ __forceinline__ void wg_share(uint32_t total, uint32_t *s, uint32_t *s_end)
{
    const uint32_t wpb = kBlock / kWave;
    const unsigned long long nwaves = (unsigned long long)gridDim.x * wpb;
    *s = (uint32_t)(((unsigned long long)total * (vblock() * wpb)) / nwaves);
    *s_end = (uint32_t)(((unsigned long long)total * (vblock() * wpb + wpb)) / nwaves);
}

// Units [s, s_end) of the flattened slot space, in one pass: the exact maximum
// (running max seeded with the lower bound the compaction posted, tokens whose
// bound ub <= running max - b skipped: exact for both results) and the
// superset admission against running max - b. Every thread of the workgroup
// calls it (the last segments are posted together, behind a barrier): per-lane
// counters that every wavefront hit with its own atomic serialize at the
// memory side (about 12 ns each on one address), so a lane's list allocation
// and maximum take one atomic per workgroup instead.
template <typename LPT, bool HASH>
__device__ __forceinline__ void walk_range(const Work &w, const LaneTab &tab, int t, const LpDesc &d,
                                           uint32_t s, uint32_t s_end, ClaimBuf *cbuf)
{
    const int nl = w.max_lanes;
    const uint32_t ep = round_epoch(w, t, 0);
    uint32_t cb_n = 0;
    int lastL = -1;
    float lastRun = -__builtin_inff();
    while (s < s_end) {
        const int L = find_lane(tab.base, nl, s);
        const int p = upar(tab.par, L);
        const uint32_t seg_end = min(s_end, tab.base[L + 1]);
        const LaneView v = lane_view(w, tab, t, d, L);
        LaneCtl &c = w.ctl[L];
        uint32_t cur = pick(w.strip_tok, p)[(size_t)L * w.strip_cap + (s - tab.base[L]) * kR];
        if (cur >= v.n) cur = 0;
        float run = ord2f(tab.fb[L]);
        const float b = tab.f1[L];
        SlotWin sw;
        sw.valid = false;
        sw.wb = 0u; sw.o = 0u; sw.o_next = 0u; sw.ab = 0; sw.sc = 0.0f; sw.ub = 0.0f;
        for (; s < seg_end; ++s) {
            UnitData ud;
            load_unit<LPT>(w, v, s - tab.base[L], cur, run - b, ud, sw);
            run = fmaxf(run, unit_max(ud));
            admit_unit<HASH>(w, L, v.ph, run - b, ep, ud, &c.nclaims[p], cbuf, cb_n);
        }
        // (the wavefront's last segment is posted by the whole workgroup)
        if (s >= s_end) { lastL = L; lastRun = run; break; }
        if (cb_n) flush_claims(w, 0, L, &c.nclaims[p], *cbuf, cb_n);
        cb_n = 0;
        if (run > -__builtin_inff() && wlane() == 0) atomicMax(&c.maxkey[p], f2ord(run));
    }
    wg_post(w, tab, lastL, lastRun, cb_n, cbuf);
}

template <typename LPT, bool HASH>
__device__ __forceinline__ void walk_slots(const Work &w, const LaneTab &tab, int t, const LpDesc &d,
                                           ClaimBuf *cbuf)
{
    uint32_t s, s_end;
    wave_share(tab.base[w.max_lanes], &s, &s_end);
    walk_range<LPT, HASH>(w, tab, t, d, s, s_end, cbuf);
}

// Dynamic beam b_t of a lane (page section 3), every operation one fp32
// rounding; n = frontier size entering the step. Every workgroup of the slot
// pass computes it (the same value workgroup 0 stores).
// T = the lane's frames, bp = the beam of its previous step.
__device__ __forceinline__ float step_beam(const Work &w, int T, float bp, int t, int ph, uint32_t n)
{
    if (ph == kPhFinal) return 1e10f;
    int mina = w.min_active;
    // a stream's T stays unbounded until it ends, so there this never applies
    if ((long long)T - t <= 5 && w.max_active / 2 > mina) mina = w.max_active / 2;
    if ((long long)n > (long long)w.max_active) return __fmul_rn(fminf(bp, w.beam), 0.8f);
    if ((long long)n < (long long)mina) return __fmul_rn(fmaxf(bp, w.beam), 1.25f);
    return __fadd_rn(__fmul_rn(0.8f, bp), __fmul_rn(0.2f, w.beam));
}

// Per-lane table of the slot pass of step t: units, row maximum, beam, and the
// compaction's lower bound of the step's maximum.
__device__ __forceinline__ void slot_prologue(const Work &w, LaneTab &tab, int t)
{
    if (threadIdx.x >= kWave) return;
    const int L = (int)threadIdx.x;
    uint32_t units = 0;
    if (L < w.max_lanes) {
        const LaneCtl &c = w.ctl[L];
        // every load first (none waits for another), then the decisions
        const int p = lane_par(c, t);
        int ph = lane_phase(c, t);
        const unsigned long long cn = pair_at(c.cnt, p);
        const uint32_t lbk = pair_at(c.lbkey, p);
        const float bprev = pair_at(c.beam, p ^ 1);
        const uint32_t n = (uint32_t)cn, arcs = (uint32_t)(cn >> 32);
        if (ph != kPhNone && (n > w.frontier_cap || arcs > w.strip_cap * (uint32_t)kWave)) ph = kPhNone;
        float b = 0.0f;
        uint32_t lb = kOrdNegInf;
        if (ph != kPhNone && n > 0u && arcs > 0u) {
            units = (arcs + kUnit - 1) / kUnit;
            b = step_beam(w, c.T, bprev, t, ph, n);
            if (ph == kPhReal) lb = lbk;
        }
        tab.n[L] = n;
        tab.arcs[L] = arcs;
        tab.ph[L] = ph;
        tab.T[L] = c.T;
        tab.f1[L] = b;
        tab.fb[L] = lb;
        tab.par[L] = p;
        tab.row[L] = c.lp_row;
    }
    tab_publish(tab, w.max_lanes, units);
}

// Step bookkeeping done once per step by thread L of workgroup 0 of k_max:
// retire overflowed / dead lanes, the dynamic beam, resets. Returns true when
// the lane's final step found no final arc and allow_partial asks for the
// redirect (done by a whole wavefront afterwards: redirect_lane).
__device__ __forceinline__ bool step_begin_lane(const Work &w, int t, int L)
{
    LaneCtl &c = w.ctl[L];
    const int p = lane_par(c, t);
    const unsigned long long cn = pair_at(c.cnt, p);
    const uint32_t n = (uint32_t)cn, arcs = (uint32_t)(cn >> 32);
    commit_log(w, c, L, t - 1, n);
    const int ph = lane_phase(c, t);
    if (ph == kPhNone) return false;
    uint32_t *rec = step_rec(w, L, t);
    c.last_step = t;
    if (w.lattice) w.lat_aoff[(size_t)L * (w.max_frames + 3) + t + 1] = c.lat_cursor;
    rec[kRecN] = n;
    rec[kRecArcs] = arcs;
    if (n > w.frontier_cap) { c.overflow |= kOvfFrontier; c.status = kDone; c.phase_final = kPhDead; rec[kRecPhase] = kPhDead; return false; }
    if (arcs > w.strip_cap * (uint32_t)kWave) { c.overflow |= kOvfSlots; c.status = kDone; c.phase_final = kPhDead; rec[kRecPhase] = kPhDead; return false; }
    if (n == 0u) { c.status = kDone; c.phase_final = kPhDead; rec[kRecPhase] = kPhDead; return false; }
    if (w.lattice) {
        // frame t holds n tokens (its closure is done): frame t + 1's first node
        const size_t F = (size_t)w.max_frames + 3;
        w.lat_nbase[(size_t)L * F + t + 1] = w.lat_nbase[(size_t)L * F + t] + n;
    }
    const float b = step_beam(w, c.T, c.beam[p ^ 1], t, ph, n);
    c.beam[p] = b;
    rec[kRecBeam] = __float_as_uint(b);
    rec[kRecPhase] = ph;
    c.phase_final = ph;
    c.nclaims[p ^ 1] = 0u;   // this step's list counter was cleared one step ago
    c.cnt[p ^ 1] = 0ull;
    c.nchanged[1] = 0ull;    // the closure's first sources, listed by this step's compaction
    c.maxkey[p ^ 1] = kOrdNegInf;
    c.lbkey[p ^ 1] = kOrdNegInf;
    if (arcs == 0u) {
        if (ph == kPhReal) {
            c.status = kDone; c.phase_final = kPhDead; rec[kRecPhase] = kPhDead;
        } else {
            c.status = kDone;
            if (w.allow_partial) return true;
        }
    }
    return false;
}

// The redirect of a final step without final arcs (page section 3, allow_partial;
// reading R10), by one wavefront: each token offers a virtual weight-0 arc
// num_arcs + state, and the greatest key(score, arc) wins (keys are unique: one
// token per state); a strided scan of the frontier, then a wavefront reduction.
__device__ __forceinline__ void redirect_lane(const Work &w, int t, int L)
{
    LaneCtl &c = w.ctl[L];
    const int p = lane_par(c, t);
    const uint32_t n = (uint32_t)pair_at(c.cnt, p);
    const size_t qo = (size_t)L * w.frontier_cap;
    unsigned long long bk = 0ull;
    uint32_t bi = 0xFFFFFFFFu;
    for (uint32_t i = (uint32_t)wlane(); i < n; i += kWave) {
        const float e = w.tok_score[p][qo + i] + 0.0f;
        const unsigned long long k = cand_key(e, (int32_t)((uint32_t)w.num_arcs + (uint32_t)w.tok_state[p][qo + i]));
        if (bi == 0xFFFFFFFFu || k > bk) { bk = k; bi = i; }
    }
    unsigned long long m = bi == 0xFFFFFFFFu ? 0ull : bk;
#pragma unroll
    for (int dd = kWave / 2; dd >= 1; dd >>= 1) {
        const unsigned long long o = __shfl_xor(m, dd, kWave);
        m = o > m ? o : m;
    }
    const unsigned long long who = __ballot(bi != 0xFFFFFFFFu && bk == m);
    if (!who) return;
    const int src = __ffsll((long long)who) - 1;
    if (wlane() != src) return;
    uint32_t *rec = step_rec(w, L, t);
    c.final_entry = w.tok_entry[p][qo + bi];
    c.final_score = w.tok_score[p][qo + bi] + 0.0f;
    c.reached_final = 0;
    rec[kRecPhase] = kPhRedirect;
    if (w.lattice) {
        // the redirect's virtual arc is the lattice's one final arc
        const uint32_t li = c.lat_cursor;
        if (li < w.lat_cap) {
            w.lat_arc[(size_t)L * w.lat_cap + li] =
                make_int4((int)bi, (int)((uint32_t)w.num_arcs + (uint32_t)w.tok_state[p][qo + bi]), w.super_final, 0);
            c.lat_cursor = li + 1u;
        } else {
            c.overflow |= kOvfArena;
        }
    }
    c.phase_final = kPhRedirect;
}

// Start of a step: the lane table of the step's slot space, then workgroup 0
// runs the per-lane bookkeeping (beam update, retirements, resets of the other
// parity's counters: the slot pass of this step is running beside it).
__device__ __forceinline__ void step_open(const Work &w, int t, LaneTab &tab)
{
    slot_prologue(w, tab, t);
    __syncthreads();
    if (blockIdx.x == 0) {
        // (block-uniform: the whole workgroup takes part in the barrier)
        __shared__ int32_t redir[kMaxLanes];
        if (threadIdx.x < (unsigned)w.max_lanes)
            redir[threadIdx.x] = step_begin_lane(w, t, (int)threadIdx.x) ? 1 : 0;
        __syncthreads();
        // one wavefront per lane that redirects
        for (int L = (int)(threadIdx.x / kWave); L < w.max_lanes; L += kBlock / kWave)
            if (redir[L]) redirect_lane(w, t, L);
    }
}

// The slot pass of step t: exact maximum and superset admission in one walk.
// (five workgroups per CU: the register budget is held to five wavefronts per SIMD)
template <typename LPT, bool HASH>
__global__ __launch_bounds__(kBlock, 5) void k_max(const Work *__restrict__ wp, int t)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    __shared__ ClaimBuf cbufs[kBlock / kWave];
    step_open(w, t, tab);
    const LpDesc d = *w.lp;
    walk_slots<LPT, HASH>(w, tab, t, d, &cbufs[threadIdx.x / kWave]);
}

// -------------------------------------------------------------- k_finalize

// The best next-step candidate through the state's kTopArcs largest-weight
// emitting arcs, (score + weight) + lp as the maximum pass adds them (unused
// entries weigh -inf); row = element offset of the next frame's log-prob row.
__device__ __forceinline__ float top_bound(const Work &w, const LpDesc &lpd, const StateInfo &si, float end,
                                           long long row)
{
    float lpk[kTopArcs];
    if (w.lp_dtype == 1) {
        const __half *r = (const __half *)lpd.base + row;
#pragma unroll
        for (int k = 0; k < kTopArcs; ++k) lpk[k] = __half2float(r[si.top_il[k]]);
    } else {
        const float *r = (const float *)lpd.base + row;
#pragma unroll
        for (int k = 0; k < kTopArcs; ++k) lpk[k] = r[si.top_il[k]];
    }
    float lbv = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < kTopArcs; ++k) lbv = fmaxf(lbv, (end + si.top_w[k]) + lpk[k]);
    return lbv;
}

// Result of the final step: the winners-log entry of the best final arc (key
// fk, source token stok of frontier parity p). Written by exactly one thread.
__device__ __forceinline__ void final_entry(const Work &w, LaneCtl &c, int L, int p,
                                            unsigned long long fk, int32_t stok)
{
    const float end = ord2f((uint32_t)(fk >> 32));
    const int32_t arc = (int32_t)(0xFFFFFFFFu - (uint32_t)fk);
    const int32_t esrc = (uint32_t)stok < w.frontier_cap
        ? pick(w.tok_entry, p)[(size_t)L * w.frontier_cap + stok] : -1;
    const uint32_t le = c.log_cursor;
    if (le < w.arena_lim) {
        const int32_t e = (int32_t)((uint32_t)L * w.arena + le);
        w.wlog[e] = make_int2(esrc, arc);
        c.log_cursor = le + 1u;
        c.final_entry = e;
        c.final_score = end;
        c.reached_final = 1;
    } else {
        atomicOr(&c.overflow, kOvfArena);
        c.log_full = 1u;
    }
}


// Lattice mode: the arcs the step before persisted (its own, then its
// closure's; the start closure's at step 0), whose destination states become
// positions in the frontier that step built. Its position map is still that
// frontier's here (this compaction writes the other parity's).
struct LatTab {
    uint32_t base[kMaxLanes + 1];  // exclusive prefix of work units per lane
    uint32_t n[kMaxLanes];         // arcs of the step before (and of its closure)
    uint32_t a0[kMaxLanes];        // the first of them
    uint32_t nb[kMaxLanes];        // first lattice node of the frame this compaction builds
};

template <bool HASH>
__device__ __forceinline__ void ph_finalize(const Work &w, int t, LaneTab &tab, LatTab &lt)
{
    const uint32_t ep = round_epoch(w, t, 0);
    const LpDesc lpd = *w.lp;
    // (the second wavefront builds the lattice table beside the first's lane
    // table; every load of a lane is issued before any decision)
    if (w.lattice && threadIdx.x >= kWave && threadIdx.x < 2 * kWave) {
        const int L = (int)threadIdx.x - kWave;
        uint32_t n = 0, a0 = 0, nb = 0;
        // a lane that began step t (whatever step t then did): the arcs of step
        // t - 1 (slot t of the offsets; step -1 is the start closure)
        if (L < w.max_lanes) {
            const size_t F = (size_t)w.max_frames + 3;
            const int ls = w.ctl[L].last_step;
            const uint32_t b0 = w.lat_aoff[(size_t)L * F + t];
            const uint32_t a1 = min(w.lat_aoff[(size_t)L * F + t + 1], w.lat_cap);
            const uint32_t nb0 = w.lat_nbase[(size_t)L * F + t + 1];
            if (ls == t) {
                a0 = b0;
                n = a1 > a0 ? a1 - a0 : 0u;
                nb = nb0;
            }
        }
        if (L < w.max_lanes) { lt.n[L] = n; lt.a0[L] = a0; lt.nb[L] = nb; }
        uint32_t tot;
        const uint32_t ex = wave_excl_sum((n + kWave - 1) / kWave, &tot);
        if (L < w.max_lanes) lt.base[L] = ex;
        if (L == 0) lt.base[w.max_lanes] = tot;
    }
    if (threadIdx.x < kWave) {
        const int L = (int)threadIdx.x;
        uint32_t units = 0;
        if (L < w.max_lanes) {
            const LaneCtl &c = w.ctl[L];
            const int ph = lane_phase(c, t);
            const int p = lane_par(c, t);
            const uint32_t nc = pair_at(c.nclaims, p);
            const uint32_t mk = pair_at(c.maxkey, p);
            const float bt = pair_at(c.beam, p);
            const uint32_t fbase = pair_at(c.front_base, p);
            // candidates past claims_cap were never written, or a full hash lost
            // some: the lane cannot be compacted (token and log capacity are
            // checked per wavefront)
            const bool fits = nc <= w.claims_cap && !(c.overflow & kOvfHash);
            if ((ph == kPhReal || ph == kPhFinal) && fits) units = (nc + kWave - 1) / kWave;
            tab.n[L] = nc;
            tab.arcs[L] = c.log_cursor;          // winners-log base of this compaction
            tab.ph[L] = ph;
            tab.T[L] = c.T;
            tab.f0[L] = fits ? 1.0f : 0.0f;
            tab.f1[L] = (ph != kPhNone) ? ord2f(mk) - bt : 0.0f;   // the exact cutoff
            tab.fb[L] = fbase;
            tab.par[L] = p;
            tab.row[L] = c.lp_row;
            tab.win[L] = c.win;
        }
        tab_publish(tab, w.max_lanes, units);
    }
    __syncthreads();

    if (blockIdx.x == 0 && threadIdx.x < (unsigned)w.max_lanes) {
        const int L = (int)threadIdx.x;
        LaneCtl &c = w.ctl[L];
        const int ph = tab.ph[L];
        const int p = tab.par[L], np = p ^ 1;
        const unsigned long long cn = c.cnt[p];
        if ((ph == kPhReal || ph == kPhFinal) && (uint32_t)cn > 0u && (uint32_t)(cn >> 32) > 0u) {
            // lanes with candidates: the exact maximum and the cutoff of the step
            step_rec(w, L, t)[kRecMax] = __float_as_uint(ord2f(c.maxkey[p]));
            step_rec(w, L, t)[kRecListed] = tab.n[L];
            if (ph == kPhReal) c.cutoff = tab.f1[L];
        }
        if (ph == kPhReal) {
            if (tab.f0[L] == 0.0f) {
                // the candidate list overflowed (or the hash was full): retire the
                // lane before writing any token; its table entries stay set, so
                // the table is cleared before the next decode
                if (tab.n[L] > w.claims_cap) c.overflow |= kOvfClaims;
                c.dirty = 1u; c.status = kDone; c.phase_final = kPhDead;
            } else {
                c.front_base[np] = tab.arcs[L];
                c.log_open = 1u;   // entries added to log_cursor by the next kernel
            }
            c.nclaims_eps[1] = 0u;   // (the closure's first two passes' lists)
            c.nclaims_eps[2] = 0u;
        } else if (ph == kPhFinal) {
            // the final key is the best of the superset: a result iff admitted
            const unsigned long long fk = c.final_key;
            const bool got = fk != 0ull && ord2f((uint32_t)(fk >> 32)) > tab.f1[L] && tab.f0[L] != 0.0f;
            step_rec(w, L, t)[kRecDistinct] = got ? 1u : 0u;
            if (tab.f0[L] == 0.0f && tab.n[L] > w.claims_cap) c.overflow |= kOvfClaims;
            c.status = kDone;
        }
    }

    const int nl = w.max_lanes;
    const uint32_t total = tab.base[nl];
    const int lane = wlane();
    const uint32_t Q = w.frontier_cap;
    // the workgroup's units, dealt round-robin to its wavefronts so that every
    // wavefront takes the same rounds: a round's lane counters (positions and
    // slot offsets, closure sources, admitted count, lower bound of the next
    // maximum) take one atomic per lane of the round instead of one per
    // wavefront (same-address atomics serialize at the memory side)
    constexpr int kW = kBlock / kWave;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    uint32_t g_beg, g_end;
    wg_share(total, &g_beg, &g_end);
    // (bounds, wavefront index and allocated bases as scalars: the loop holds
    // barriers, so the compiler must see it as uniform)
    g_beg = __builtin_amdgcn_readfirstlane(g_beg);
    g_end = __builtin_amdgcn_readfirstlane(g_end);
    __shared__ int32_t agL[kW];
    __shared__ uint32_t agA[kW], agN[kW], agD[kW], agE[kW], agPE[kW], agPR[kW];
    __shared__ unsigned long long agP[kW];
    __shared__ float agLB[kW];
    // lattice mode: the step before's unresolved arcs (its recombination losers
    // and its closure's epsilon arcs) get their destination's position among
    // the tokens of frame t (the parity this compaction reads). The wavefront's
    // first unit of them is read, and its position gathers issued, before the
    // compaction's own loads; the positions are written after them.
    uint32_t v_beg = 0, v_end = 0;
    int mL = -1;
    uint32_t mi = 0;
    int4 mr = make_int4(0, 0, 0, 0);
    int32_t mpos = 0;
    bool mpend = false, mun = false;
    if (w.lattice) {
        wave_share(lt.base[nl], &v_beg, &v_end);
        if (v_beg < v_end) {
            mL = find_lane(lt.base, nl, v_beg);
            mi = (v_beg - lt.base[mL]) * kWave + (uint32_t)lane;
            if (mi < lt.n[mL]) mr = w.lat_arc[(size_t)mL * w.lat_cap + lt.a0[mL] + mi];
            mpend = true;
        }
    }
    if (mpend) {
        const uint32_t d = (uint32_t)mr.z;
        if (mi < lt.n[mL] && (d & kLatUnresolved) && (d & ~kLatUnresolved) < (uint32_t)w.num_states) {
            mun = true;
            mpos = pick(w.pos, upar(tab.par, mL))[(size_t)mL * w.num_states + (d & ~kLatUnresolved)];
        }
    }
    for (uint32_t ur = g_beg; ur < g_end; ur += (uint32_t)kW) {
        const uint32_t u = ur + (uint32_t)wv;
        const bool has = u < g_end;                       // (wavefront-uniform)
        const int L = has ? find_lane(tab.base, nl, u) : 0;
        const int p = upar(tab.par, L), np = p ^ 1;
        const uint32_t nc = has ? tab.n[L] : 0u;
        const uint32_t i = has ? (u - tab.base[L]) * kWave + (uint32_t)lane : 0u;
        const bool valid = i < nc;
        const float cutoff = tab.f1[L];
        const bool next_final = (t + 1 == tab.T[L]);
        const bool fin = has && tab.ph[L] == kPhFinal;
        LaneCtl &c = w.ctl[L];
        bool keep = false;
        int32_t dst = 0, arc = 0, esrc = -1, abeg = 0, eps_b0 = 0;
        uint32_t deg = 0, eps_n = 0;
        float end = 0.0f, ub = 0.0f, lbv = -__builtin_inff();
        // the list is a superset: a candidate is admitted iff end > the exact
        // cutoff; the one whose key is its destination's entry owns the entry
        // (clears it) and becomes the token if admitted
        Claim cl;
        bool adm = false;
        if (valid) {
            cl = w.claims[tab_row(w, 0, L) * w.claims_cap + i];
            adm = __uint_as_float(cl.score) > cutoff;
        }
        const unsigned long long am = __ballot(adm);
        // lattice mode: every admitted candidate is a lattice arc {source
        // position, arc, destination, pass 0}, its record written once the
        // destination is known: a winner's position in the new frontier, else
        // (recombination losers, final arcs) its state marked unresolved
        // (kLatUnresolved), mapped to the position by the next compaction
        // (their positions are allocated with the round's counters below)
        uint32_t lat_i = 0xFFFFFFFFu;
        const uint32_t cds = valid ? dest_state(w, cl.dest) : 0u;
        int32_t lat_z = (int32_t)(cds | kLatUnresolved);
        if (fin) {
            if (adm && cand_key(__uint_as_float(cl.score), cl.arc) == c.final_key)
                final_entry(w, c, L, p, c.final_key, (int32_t)cl.tok);
        } else if (has) {
            // with epochs only admitted candidates need the table (stale entries of
            // earlier rounds always lose); without, every owner clears its entry
            if (valid && (adm || !w.epochs) && cds < (uint32_t)w.num_states) {
                if (recomb_key<HASH>(w, 0, L, cds, ep) == table_key(w, __uint_as_float(cl.score), cl.arc, cl.dest, ep)) {
                    if (!w.epochs) w.best[(size_t)L * (size_t)w.num_states + cds] = 0ull;
                    keep = adm;
                }
            }
            if (keep) {
                dst = (int32_t)cds;
                arc = cl.arc;
                end = __uint_as_float(cl.score);
                const StateInfo si = w.sinfo[dst];
                const int32_t stok = (int32_t)cl.tok;
                keep = (uint32_t)stok < Q;
                if (keep) {
                    // without epsilon arcs a token's entry is its compaction's base
                    // plus its position; the closure may give a token a fresh entry
                    const uint32_t fb = tab.fb[L];
                    esrc = w.has_eps ? pick(w.tok_entry, p)[(size_t)L * Q + stok]
                         : fb == 0xFFFFFFFFu ? -1 : (int32_t)((uint32_t)L * w.arena + fb + (uint32_t)stok);
                    class_of(si, next_final, end, &abeg, &deg, &ub);
                    eps_b0 = si.eps_b;
                    eps_n = (uint32_t)(si.emit_b - si.eps_b);
                    // (no bound past the sequence's window: its row is not in this input)
                    if (!next_final && deg > 0u && t + 1 < tab.win[L]) {
                        // candidates of the next step through the state's
                        // largest-weight arcs, (score + weight) + lp as the
                        // maximum pass adds them (unused entries weigh -inf)
                        lbv = top_bound(w, lpd, si, end, (long long)tab.row[L] * lpd.stride_b + (long long)(t + 1) * lpd.stride_t);
                        // the token's bound for the next step: its exact best candidate
                        // when these arcs are all it has, else (score + largest weight)
                        // + the frame's largest log-prob
                        ub = deg <= (uint32_t)kTopArcs
                            ? lbv : ub + w.lpmax[(size_t)L * w.max_frames + (size_t)(t + 1)];
                    } else if (!next_final) {
                        ub = __builtin_inff();   // (the next frame is not in this input)
                    }
                }
            }
        }
        const unsigned long long m = __ballot(keep);
        const uint32_t nkeep = (uint32_t)__popcll(m);
        const uint32_t rank = (uint32_t)__popcll(m & mask_lt());
        uint32_t dsum;
        const uint32_t dpre = wave_excl_sum(keep ? deg : 0u, &dsum);
        // on epsilon graphs the closure's first sources: the new tokens with
        // epsilon arcs
        const unsigned long long ml = (w.eps_iterations > 0) ? __ballot(keep && eps_n > 0u) : 0ull;
        // the round's allocation: per lane one 64-bit atomicAdd of positions
        // (low half) and slot offsets (high half), the wavefronts of the lane
        // taking consecutive parts in wavefront order
        // lower bound of the next step's maximum: the wavefront's best, posted
        // with the round's allocation
        const float lbw = wave_max(lbv);
        if (lane == 0) {
            agLB[wv] = lbw;
            agL[wv] = has ? L : -1;
            agA[wv] = (uint32_t)__popcll(am);
            agN[wv] = nkeep;
            agD[wv] = dsum;
            agE[wv] = (uint32_t)__popcll(ml);
        }
        __syncthreads();
        if (threadIdx.x < (unsigned)kW) {
            const int k = (int)threadIdx.x;
            const int Lk = agL[k];
            bool first = Lk >= 0;
            for (int j = 0; j < k; ++j) first = first && agL[j] != Lk;
            if (first) {
                uint32_t tA = 0, tN = 0, tD = 0, tE = 0;
                float tB = -__builtin_inff();
                for (int j = k; j < kW; ++j)
                    if (agL[j] == Lk) { tA += agA[j]; tN += agN[j]; tD += agD[j]; tE += agE[j]; tB = fmaxf(tB, agLB[j]); }
                LaneCtl &ck = w.ctl[Lk];
                const int npk = tab.par[Lk] ^ 1;
                unsigned long long old = 0ull;
                uint32_t e0 = 0u;
                if (tA) atomicAdd(step_rec(w, Lk, t) + kRecAdmitted, tA);
                uint32_t r0 = 0u;
                if (w.lattice && tA) r0 = atomicAdd(&ck.lat_cursor, tA);
                if (tB > -__builtin_inff()) atomicMax(&ck.lbkey[npk], f2ord(tB));
                if (tN) old = atomicAdd(&ck.cnt[npk], (unsigned long long)tN | ((unsigned long long)tD << 32));
                if (tE) e0 = (uint32_t)atomicAdd(&ck.nchanged[1], (unsigned long long)tE);
                for (int j = k; j < kW; ++j)
                    if (agL[j] == Lk) {
                        agP[j] = old;
                        agPE[j] = e0;
                        agPR[j] = r0;
                        r0 += agA[j];
                        old += (unsigned long long)agN[j] | ((unsigned long long)agD[j] << 32);
                        e0 += agE[j];
                    }
            }
        }
        __syncthreads();
        if (w.lattice && am) {
            const uint32_t lb0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)agPR[wv]);
            if ((unsigned long long)lb0 + (uint32_t)__popcll(am) > w.lat_cap) {
                if (lane == 0) atomicOr(&c.overflow, kOvfArena);
            } else if (adm) {
                lat_i = lb0 + (uint32_t)__popcll(am & mask_lt());
            }
        }
        if (m != 0ull) {
            const unsigned long long old = ((unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(agP[wv] >> 32)) << 32)
                                         | (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)agP[wv]);
            const uint32_t l0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)agPE[wv]);
            const int leader = __ffsll((long long)m) - 1;
            const uint32_t p0 = (uint32_t)old, a0 = (uint32_t)(old >> 32);
            // exact capacity of this wavefront's tokens and winners-log entries: on
            // overflow nothing is written and the lane retires (the frontier count
            // past frontier_cap keeps every later kernel off its tokens)
            const bool pos_ok = (unsigned long long)p0 + nkeep <= Q;
            if (!pos_ok || (unsigned long long)tab.arcs[L] + p0 + nkeep > w.arena_lim) {
                if (lane == leader) {
                    atomicOr(&c.overflow, pos_ok ? kOvfArena : kOvfFrontier);
                    if (pos_ok) c.log_full = 1u;
                    c.status = kDone;
                    c.phase_final = kPhDead;
                }
            } else {
                if (keep) {
                    const uint32_t pi = p0 + rank;
                    lat_z = (int32_t)pi;
                    const size_t q = (size_t)L * Q + pi;
                    const int32_t e = (int32_t)((uint32_t)L * w.arena + tab.arcs[L] + pi);
                    w.wlog[e] = make_int2(esrc, arc);
                    pick(w.tok_state, np)[q] = dst;
                    if (w.eps_iterations > 0) pick(w.tok_tag, np)[q] = frame_tag(c, t);   // made by the compaction
                    pick(w.tok_score, np)[q] = end;
                    pick(w.tok_entry, np)[q] = e;
                    pick(w.tok_last, np)[q] = arc;
                    pick(w.tok_off, np)[q] = a0 + dpre;
                    pick(w.tok_abeg, np)[q] = abeg;
                    pick(w.tok_ub, np)[q] = ub;
                    if (w.has_eps || w.lattice) pick(w.pos, np)[(size_t)L * w.num_states + dst] = (int32_t)pi;
                    if (w.lattice) {
                        // the token's lattice node (its closure may still raise the score)
                        const uint32_t ni = lt.nb[L] + pi;
                        if (ni < w.lat_nodes) {
                            w.lat_score[(size_t)L * w.lat_nodes + ni] = end;
                            w.lat_state[(size_t)L * w.lat_nodes + ni] = dst;
                        } else {
                            lat_node_overflow(w, c);
                        }
                    }
                    if ((ml >> lane) & 1ull) {
                        const size_t ci = (size_t)L * w.chg_cap + l0 + (uint32_t)__popcll(ml & mask_lt());
                        w.changed[1][ci] = make_int4(eps_b0, (int)eps_n, e, (int)__float_as_uint(end));
                        if (w.lattice) w.chg_pos[1][ci] = (int32_t)pi;
                    }
                }
                write_strips(pick(w.strip_tok, np) + (size_t)L * w.strip_cap, w.strip_cap, p0, a0, dpre, dsum, m);
            }
        }
        if (lat_i != 0xFFFFFFFFu) w.lat_arc[(size_t)L * w.lat_cap + lat_i] = make_int4((int)cl.tok, cl.arc, lat_z, 0);
    }
    if (w.lattice) {
        if (mun) w.lat_arc[(size_t)mL * w.lat_cap + lt.a0[mL] + mi].z = mpos;
        // (the wavefront's other units, if any)
        for (uint32_t u = v_beg + 1; u < v_end; ++u) {
            const int L = find_lane(lt.base, nl, u);
            const int p = upar(tab.par, L);
            const uint32_t i = (u - lt.base[L]) * kWave + (uint32_t)lane;
            if (i >= lt.n[L]) continue;
            int4 *r = w.lat_arc + (size_t)L * w.lat_cap + lt.a0[L] + i;
            const uint32_t d = (uint32_t)r->z;
            if ((d & kLatUnresolved) && (d & ~kLatUnresolved) < (uint32_t)w.num_states)
                r->z = pick(w.pos, p)[(size_t)L * w.num_states + (d & ~kLatUnresolved)];
        }
    }
}

template <bool HASH>
__global__ __launch_bounds__(kBlock) void k_finalize(const Work *__restrict__ wp, int t)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    __shared__ LatTab lt;
    ph_finalize<HASH>(w, t, tab, lt);
}

// ---------------------------------------------------------- epsilon closure
// Pass k of the closure that follows step t (t = -1: the start frontier). The
// frontier being closed feeds step t + 1 (parity lane_par(c, t + 1)).

// A lane whose winners log or frontier overflowed holds tokens that were
// counted but never written; it is skipped until the next step retires it.
// Capacity of the compaction before a closure was checked lane-wide before it
// wrote anything, and every apply kernel checks its own appends the same way,
// so an active lane never holds a counted but unwritten token.
__device__ __forceinline__ bool closure_lane(const LaneCtl &c, int t)
{
    return c.status == kActive && t < c.win && (t < 0 || t < c.T);
}

// Relaxes the epsilon arcs of a wavefront's sources in closure pass k of step
// t, at most one source per lane (src: first epsilon arc eb, ed arcs, winners-
// log entry ent, score sc, frontier position spos) of lane L: all their arcs, 64
// at a time (balanced within the wave), each admitted candidate posting its
// key to round (t, k)'s table and joining its list; in lattice mode each
// admitted one is a lattice arc of the frame being closed (nb: its first
// node), tagged with the pass. ep: the round's epoch.
template <bool HASH>
__device__ __forceinline__ void relax_sources(const Work &w, int L, int t, int k, uint32_t ep, float cutoff,
                                              uint32_t nb, bool src, int32_t eb, uint32_t ed, int32_t ent,
                                              float sc, int32_t spos, ClaimBuf *cbuf)
{
    LaneCtl &c = w.ctl[L];
    const int lane = wlane();
    const int tb = round_tab(w, k);
    uint32_t *counter = &c.nclaims_eps[k % 3];
    if (!src) ed = 0u;
    if (w.lattice && src) {
        // the source's node: this pass relaxes its epsilon arcs (a later pass
        // that relaxes them again admits a superset: the source's score only
        // grows)
        const uint32_t ni = nb + (uint32_t)spos;
        if (ni < w.lat_nodes) w.lat_epass[(size_t)L * w.lat_nodes + ni] = (uint8_t)k;
    }
    uint32_t dsum;
    const uint32_t dpre = wave_excl_sum(ed, &dsum);
    uint32_t n_adm = 0, cb_n = 0;
    for (uint32_t x0 = 0; x0 < dsum; x0 += kWave) {
        const uint32_t x = x0 + (uint32_t)lane;
        int sl = 0;
#pragma unroll
        for (int st = 32; st >= 1; st >>= 1) {
            const uint32_t v = __shfl(dpre, sl + st, kWave);
            if (v <= x) sl += st;
        }
        const int32_t a = __shfl(eb, sl, kWave) + (int32_t)(x - __shfl(dpre, sl, kWave));
        const float ssc = __shfl(sc, sl, kWave);
        // the source's winners-log entry as this pass found it (the resolving
        // kernel may give the source token a fresh one)
        const int32_t sen = __shfl(ent, sl, kWave);
        bool adm = false;
        int32_t dd = 0;
        float e = 0.0f;
        if (x < dsum) {
            const ArcDLW ar = w.arc_dlw[a];
            e = ssc + ar.weight;
            dd = ar.dest;
            adm = e > cutoff;
            if (adm) {
                ++n_adm;
                unsigned long long *slot = recomb_entry<HASH>(w, tb, L, dest_state(w, ar.dest), ep);
                if (slot) atomicMax(slot, table_key(w, e, a, ar.dest, ep));
                else atomicOr(&c.overflow, kOvfHash);
            }
        }
        if (w.lattice) {
            // every admitted epsilon candidate is a lattice arc of the frame
            // being closed: {source position, arc, destination state (unresolved
            // until the next compaction maps it), pass}
            const int32_t sps = __shfl(spos, sl, kWave);
            const unsigned long long am = __ballot(adm);
            if (am) {
                const int lead = __ffsll((long long)am) - 1;
                uint32_t lb0 = 0u;
                if (lane == lead) lb0 = atomicAdd(&c.lat_cursor, (uint32_t)__popcll(am));
                lb0 = __shfl(lb0, lead, kWave);
                if ((unsigned long long)lb0 + (uint32_t)__popcll(am) > w.lat_cap) {
                    if (lane == lead) atomicOr(&c.overflow, kOvfArena);
                } else if (adm) {
                    w.lat_arc[(size_t)L * w.lat_cap + lb0 + (uint32_t)__popcll(am & mask_lt())] =
                        make_int4(sps, a, (int32_t)(dest_state(w, dd) | kLatUnresolved), k);
                }
            }
        }
        push_claims(w, tb, L, counter, *cbuf, cb_n, adm, dd, a, (uint32_t)sen, e);
    }
    if (cb_n) flush_claims(w, tb, L, counter, *cbuf, cb_n);
    const uint32_t sd = wave_sum(n_adm);
    if (lane == 0 && dsum) {
        uint32_t *rec = step_rec(w, L, t);
        atomicAdd(rec + kRecEpsArcs, dsum);
        if (sd) atomicAdd(rec + kRecEpsAdmitted, sd);
    }
}

// Closure pass k's relaxation from the source list the kernel before wrote
// (pass 1: the compaction's new tokens with epsilon arcs; a pass after a
// resolving kernel that did not relax it itself: that kernel's changed tokens).
template <bool HASH>
__device__ __forceinline__ void ph_eps_expand(const Work &w, int t, int k, LaneTab &tab, ClaimBuf *cbuf)
{
    const uint32_t ep = round_epoch(w, t, k);
    if (threadIdx.x < kWave) {
        const int L = (int)threadIdx.x;
        uint32_t units = 0;
        if (L < w.max_lanes) {
            const LaneCtl &c = w.ctl[L];
            const int fp = lane_par(c, t + 1);
            tab.par[L] = fp;
            uint32_t ns = 0, srcs = 0;
            const uint32_t n = (uint32_t)pair_at(c.cnt, fp);
            const unsigned long long nch = c.nchanged[k & 1];
            if (closure_lane(c, t) && n <= w.frontier_cap) {
                ns = (uint32_t)nch;
                srcs = (k == 1) ? n : (uint32_t)(nch >> 32);
            }
            units = (ns + kWave - 1) / kWave;
            tab.n[L] = ns;
            tab.arcs[L] = srcs;
            tab.f1[L] = c.cutoff;
            // lattice mode: first node of the frame being closed
            tab.fb[L] = w.lattice ? w.lat_nbase[(size_t)L * ((size_t)w.max_frames + 3) + (size_t)(t + 1)] : 0u;
        }
        tab_publish(tab, w.max_lanes, units);
    }
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)w.max_lanes) {
        const int L = (int)threadIdx.x;
        LaneCtl &c = w.ctl[L];
        // the compaction before this closure (no closure token added yet)
        if (k == 1) commit_log(w, c, L, t, (uint32_t)c.cnt[tab.par[L]]);
        if (tab.arcs[L] > 0u) step_rec(w, L, t)[kRecEpsPasses] += 1u;   // a pass with sources
        // for the resolving kernel of this pass: an empty list of changed tokens
        c.nchanged[(k + 1) & 1] = 0ull;
    }
    const int nl = w.max_lanes;
    const uint32_t total = tab.base[nl];
    const int lane = wlane();
    uint32_t u_beg, u_end;
    wave_share(total, &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)lane;
        // the 64 sources of this unit: their epsilon ranges, entries and scores
        // as the kernel that made them wrote them
        int32_t eb = 0, ent = -1, spos = 0;
        uint32_t ed = 0;
        float sc = 0.0f;
        const bool src = i < tab.n[L];
        if (src) {
            const int4 ce = w.changed[k & 1][(size_t)L * w.chg_cap + i];
            eb = ce.x;
            ed = (uint32_t)ce.y;
            ent = ce.z;
            sc = __uint_as_float((uint32_t)ce.w);
            if (w.lattice) spos = w.chg_pos[k & 1][(size_t)L * w.chg_cap + i];
        }
        relax_sources<HASH>(w, L, t, k, ep, tab.f1[L], tab.fb[L], src, eb, ed, ent, sc, spos, cbuf);
    }
}

template <bool HASH>
__global__ __launch_bounds__(kBlock) void k_eps_expand(const Work *__restrict__ wp, int t, int k)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    __shared__ ClaimBuf cbufs[kBlock / kWave];
    ph_eps_expand<HASH>(w, t, k, tab, &cbufs[threadIdx.x / kWave]);
}

// Per claimed destination of pass k: the winner (its key is the table entry)
// is appended as a new token, replaces the destination's token if its key is
// greater, or does nothing; then the writes: fresh winners-log entries,
// appended tokens (with their next-step class and arc offsets), replaced
// tokens. Only a destination's winner reads or writes its token, and the
// existence test sees only the tokens of rounds before this pass (their tag:
// the frame's compaction or an earlier pass), so the decisions are those of a
// pass that reads everything before it writes. RELAX (k < passes): each
// wavefront then relaxes its changed tokens' epsilon arcs as pass k + 1 (into
// the other table and list: pass k's stay untouched); otherwise it lists them
// for the kernel of pass k + 1.
template <bool HASH, bool RELAX>
__device__ __forceinline__ void ph_eps_apply(const Work &w, int t, int k, LaneTab &tab, ClaimBuf *cbuf)
{
    const uint32_t ep = round_epoch(w, t, k);
    const uint32_t ep_next = RELAX ? round_epoch(w, t, k + 1) : 0u;
    const int tb = round_tab(w, k);
    if (threadIdx.x < kWave) {
        const int L = (int)threadIdx.x;
        uint32_t units = 0;
        if (L < w.max_lanes) {
            const LaneCtl &c = w.ctl[L];
            const int fp = lane_par(c, t + 1);
            tab.par[L] = fp;
            uint32_t nc = 0;
            const uint32_t nce = c.nclaims_eps[k % 3];
            // (a frontier past its capacity belongs to a lane that is retiring)
            const bool on = closure_lane(c, t) && (uint32_t)pair_at(c.cnt, fp) <= w.frontier_cap;
            if (on) nc = nce;
            // token and log capacity are checked per wavefront as it allocates;
            // a full hash lost candidates
            const bool fits = nc <= w.claims_cap && !(c.overflow & kOvfHash);
            if (fits) units = (nc + kWave - 1) / kWave;
            tab.n[L] = nc;
            tab.arcs[L] = frame_tag(c, t);
            tab.T[L] = c.T;
            tab.win[L] = c.win;
            tab.f1[L] = c.cutoff;
            tab.f0[L] = (on && !fits) ? 1.0f : 0.0f;
            // lattice mode: first node of the frame being closed
            tab.fb[L] = w.lattice ? w.lat_nbase[(size_t)L * ((size_t)w.max_frames + 3) + (size_t)(t + 1)] : 0u;
        }
        tab_publish(tab, w.max_lanes, units);
    }
    __syncthreads();
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)w.max_lanes) {
        const int L = (int)threadIdx.x;
        LaneCtl &c = w.ctl[L];
        // the list counters this launch does not fill and no later kernel has
        // filled yet: pass k + 2's (read last by pass k - 1), and when this
        // launch only lists pass k + 1's sources, pass k + 1's as well (its
        // relaxation runs next). A launch that relaxes pass k + 1 itself also
        // clears the source count a listing launch for pass k + 1 would add to.
        c.nclaims_eps[(k + 2) % 3] = 0u;
        if (!RELAX) c.nclaims_eps[(k + 1) % 3] = 0u;
        if (RELAX) c.nchanged[k & 1] = 0ull;
        if (tab.f0[L] != 0.0f) {
            // candidates past claims_cap were never listed (or the hash was
            // full): their table entries stay set, so the table is cleared
            // before the next decode
            if (tab.n[L] > w.claims_cap) c.overflow |= kOvfClaims;
            c.dirty = 1u;
            c.status = kDone; c.phase_final = kPhDead;
        }
    }
    const int nl = w.max_lanes;
    const uint32_t total = tab.base[nl];
    const int lane = wlane();
    const uint32_t Q = w.frontier_cap;
    uint32_t u_beg, u_end;
    wave_share(total, &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = (int)find_lane(tab.base, nl, u);
        const int fp = upar(tab.par, L);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)lane;
        const bool valid = i < tab.n[L];
        const bool next_final = (t + 1 == tab.T[L]);
        LaneCtl &c = w.ctl[L];
        // dd = {token replaced (-1: append, -2: nothing), score bits, arc, source entry}
        int4 dd = make_int4(-2, 0, 0, -1);
        int32_t dst = 0;
        Claim cl;
        const bool win = valid && take_winner<HASH>(w, tb, L, i, ep, cl);
        const unsigned long long wm = __ballot(win);
        if (wm && lane == __ffsll((long long)__ballot(valid)) - 1)
            atomicAdd(step_rec(w, L, t) + kRecEpsDistinct, (uint32_t)__popcll(wm));
        if (win && __uint_as_float(cl.score) > tab.f1[L]) {
            dst = (int32_t)dest_state(w, cl.dest);
            dd.y = (int)cl.score;
            dd.z = cl.arc;
            dd.w = (int32_t)cl.tok;
            // the destination's token, if a round before this pass made it
            const int32_t pd = pick(w.pos, fp)[(size_t)L * w.num_states + dst];
            bool exists = false;
            if ((uint32_t)pd < Q) {
                const size_t q = (size_t)L * Q + (uint32_t)pd;
                const uint32_t tg = pick(w.tok_tag, fp)[q];
                exists = pick(w.tok_state, fp)[q] == dst && tg >= tab.arcs[L] && tg < tab.arcs[L] + (uint32_t)k;
            }
            if (!exists) {
                dd.x = -1;
            } else {
                const size_t q = (size_t)L * Q + pd;
                if (cand_key(__uint_as_float(cl.score), cl.arc) > cand_key(pick(w.tok_score, fp)[q], pick(w.tok_last, fp)[q]))
                    dd.x = pd;
            }
        }
        const bool any = dd.x != -2;
        const bool isnew = dd.x == -1;
        const float end = __uint_as_float((uint32_t)dd.y);
        int32_t abeg = 0, eb = 0;
        uint32_t deg = 0, ed = 0;
        float ub = 0.0f;
        if (any) {
            const StateInfo si = w.sinfo[dst];
            class_of(si, next_final, end, &abeg, &deg, &ub);
            eb = si.eps_b;
            ed = (uint32_t)(si.emit_b - si.eps_b);
            // the bound of the next step's skip test: with the frame's largest
            // log-prob (unknown past the sequence's window)
            if (!next_final)
                ub = t + 1 < tab.win[L] ? ub + w.lpmax[(size_t)L * w.max_frames + (size_t)(t + 1)] : __builtin_inff();
        }
        const unsigned long long ma = __ballot(any);
        if (ma == 0ull) continue;
        const unsigned long long mn = __ballot(isnew);
        // the next pass's sources (none after the last pass): the changed tokens
        // with epsilon arcs
        const bool more = k < w.eps_iterations;
        const unsigned long long ml = more ? __ballot(any && ed > 0u) : 0ull;
        const int leader = __ffsll((long long)ma) - 1;
        uint32_t dsum;
        const uint32_t dpre = wave_excl_sum(isnew ? deg : 0u, &dsum);
        unsigned long long old = 0ull;
        uint32_t lb = 0u, cb = 0u;
        if (lane == leader) {
            lb = atomicAdd(&c.log_cursor, (uint32_t)__popcll(ma));
            if (RELAX) {
                // pass k + 1 has sources (the passes with sources are the first
                // few: one that changes nothing leaves the next none)
                atomicMax(step_rec(w, L, t) + kRecEpsPasses, (uint32_t)(k + 1));
            } else if (more) {
                // the list of pass k + 1 (low half), and the changed tokens (high)
                cb = (uint32_t)atomicAdd(&c.nchanged[(k + 1) & 1],
                                         (unsigned long long)__popcll(ml) | ((unsigned long long)__popcll(ma) << 32));
            }
            if (mn) old = atomicAdd(&c.cnt[fp], (unsigned long long)__popcll(mn) | ((unsigned long long)dsum << 32));
            uint32_t *rec = step_rec(w, L, t);
            if (mn) atomicAdd(rec + kRecEpsNew, (uint32_t)__popcll(mn));
            if (ma & ~mn) atomicAdd(rec + kRecEpsReplaced, (uint32_t)__popcll(ma & ~mn));
        }
        old = __shfl(old, leader, kWave);
        lb = __shfl(lb, leader, kWave);
        if (!RELAX) cb = __shfl(cb, leader, kWave);
        // exact capacity of this wavefront's appends and winners-log entries: on
        // overflow nothing is written and the lane retires (its table entries may
        // stay set by the relaxation of pass k + 1: the table is cleared before
        // the next decode)
        const bool pos_ok = (unsigned long long)(uint32_t)old + (uint32_t)__popcll(mn) <= Q;
        if (!pos_ok || (unsigned long long)lb + (uint32_t)__popcll(ma) > w.arena_lim) {
            if (lane == leader) {
                atomicOr(&c.overflow, pos_ok ? kOvfArena : kOvfFrontier);
                if (pos_ok) c.log_full = 1u;
                if (RELAX) c.dirty = 1u;
                c.status = kDone;
                c.phase_final = kPhDead;
            }
            continue;
        }
        if (mn) write_strips(pick(w.strip_tok, fp) + (size_t)L * w.strip_cap, w.strip_cap, (uint32_t)old,
                             (uint32_t)(old >> 32), dpre, dsum, mn);
        const uint32_t ra = (uint32_t)__popcll(ma & mask_lt());
        const uint32_t le = lb + ra;
        const int32_t e = (int32_t)((uint32_t)L * w.arena + le);
        uint32_t pi = 0u;
        if (any) {
            w.wlog[e] = make_int2(dd.w, dd.z);
            if (isnew) {
                pi = (uint32_t)old + (uint32_t)__popcll(mn & mask_lt());
                const size_t q = (size_t)L * Q + pi;
                pick(w.tok_state, fp)[q] = dst;
                pick(w.tok_tag, fp)[q] = tab.arcs[L] | (uint32_t)k;
                pick(w.tok_off, fp)[q] = (uint32_t)(old >> 32) + dpre;
                pick(w.tok_abeg, fp)[q] = abeg;
                pick(w.pos, fp)[(size_t)L * w.num_states + dst] = (int32_t)pi;
            } else {
                pi = (uint32_t)dd.x;
            }
            const size_t q = (size_t)L * Q + pi;
            pick(w.tok_score, fp)[q] = end;
            pick(w.tok_entry, fp)[q] = e;
            pick(w.tok_last, fp)[q] = dd.z;
            pick(w.tok_ub, fp)[q] = ub;
            if (w.lattice) {
                // the token's node (appended: a new one; replaced: its score rises)
                const uint32_t ni = tab.fb[L] + pi;
                if (ni < w.lat_nodes) {
                    w.lat_score[(size_t)L * w.lat_nodes + ni] = end;
                    if (isnew) w.lat_state[(size_t)L * w.lat_nodes + ni] = dst;
                } else {
                    lat_node_overflow(w, c);
                }
            }
        }
        const bool src = (ml >> lane) & 1ull;
        if (RELAX) {
            relax_sources<HASH>(w, L, t, k + 1, ep_next, tab.f1[L], tab.fb[L], src, eb, ed, e, end, (int32_t)pi, cbuf);
        } else if (src) {
            const uint32_t ci = cb + (uint32_t)__popcll(ml & mask_lt());
            if (ci < w.chg_cap) {
                w.changed[(k + 1) & 1][(size_t)L * w.chg_cap + ci] = make_int4(eb, (int)ed, e, (int)__float_as_uint(end));
                if (w.lattice) w.chg_pos[(k + 1) & 1][(size_t)L * w.chg_cap + ci] = (int32_t)pi;
            }
        }
    }
}

template <bool HASH>
__global__ __launch_bounds__(kBlock) void k_eps_apply(const Work *__restrict__ wp, int t, int k)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    ph_eps_apply<HASH, false>(w, t, k, tab, nullptr);
}

// Pass k's resolution and pass k + 1's relaxation in one launch (k < passes).
template <bool HASH>
__global__ __launch_bounds__(kBlock) void k_eps_apply_expand(const Work *__restrict__ wp, int t, int k)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    __shared__ ClaimBuf cbufs[kBlock / kWave];
    ph_eps_apply<HASH, true>(w, t, k, tab, &cbufs[threadIdx.x / kWave]);
}

// ------------------------------------------------------------------ lattice
// Lattice mode (page section 1 "Lattice mode", section 3 on output_beam,
// section 5.5 on persisting candidates after the closure, section 7
// "Lattice"): finalize persists every admitted candidate of a step, each closure
// pass every admitted epsilon candidate (tagged with its pass), as lattice arcs
// {source position, arc, destination}; a node is a frame's token (first node of
// the frame + its position), with its score after the frame's closure and its
// state. After the decode a backward pass over the frames (last to first)
// computes bwd(node) = the best s + bwd(destination) over its arcs, epsilon
// arcs staying inside their frame (a fixpoint per frame), and keeps the arcs
// with (fwd(source) + s) + bwd(destination) >= best - output_beam, where s is
// the arc's own score (weight + log-prob; a final or epsilon arc's weight; 0 for
// a redirect).

// Whether lane c's lattice holds every arc its search persisted: appends past
// lat_cap were dropped whole (arena bit) while the cursor still counted them,
// so a lane past its capacity has ranges with records never written; it gets
// no backward pass and no kept records.
__device__ __forceinline__ bool lat_complete(const Work &w, const LaneCtl &c) { return c.lat_cursor <= w.lat_cap; }

// Before the backward pass: every backward score of a lane with a result (and
// a complete lattice) is -inf (nodes of frames 0 .. its last step).
__global__ __launch_bounds__(kBlock) void k_lat_init(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t F = (size_t)w.max_frames + 3;
    for (int L = 0; L < w.max_lanes; ++L) {
        const LaneCtl &c = w.ctl[L];
        if (!lane_has_result(c) || !lat_complete(w, c) || c.last_step < 0) continue;
        const size_t n = min(w.lat_nbase[(size_t)L * F + (size_t)c.last_step + 1], w.lat_nodes);
        uint32_t *b = w.lat_bwd + (size_t)L * w.lat_nodes;
        for (size_t i = tid; i < n; i += stride) b[i] = kOrdNegInf;
    }
}

// Backward pass over the arcs of step t itself (launched for t = last .. 0;
// the epsilon arcs of its closure belong to frame t + 1, done before).
template <typename LPT>
__global__ __launch_bounds__(kBlock) void k_lat_back(const Work *__restrict__ wp, int t)
{
    const Work &w = *wp;
    const LpDesc d = *w.lp;
    __shared__ LaneTab tab;
    const size_t F = (size_t)w.max_frames + 3;
    if (threadIdx.x < kWave) {
        const int L = (int)threadIdx.x;
        uint32_t units = 0;
        if (L < w.max_lanes) {
            const LaneCtl &c = w.ctl[L];
            const bool on = lane_has_result(c) && t <= c.last_step && lat_complete(w, c);
            const bool fin = t == c.last_step;   // the lane's final step (or its redirect)
            const uint32_t a0 = w.lat_aoff[(size_t)L * F + t + 1];
            const uint32_t a1 = min(fin ? c.lat_cursor : w.lat_aoff[(size_t)L * F + t + 2], w.lat_cap);
            const uint32_t n = (on && a1 > a0) ? a1 - a0 : 0u;
            units = (n + kWave - 1) / kWave;
            tab.n[L] = n;
            tab.fb[L] = a0;
            tab.ph[L] = fin ? 1 : 0;
            tab.f1[L] = c.final_score - w.output_beam;
            tab.row[L] = c.lp_row;
            tab.arcs[L] = on ? w.lat_nbase[(size_t)L * F + t] : 0u;                      // frame t's first node
            tab.win[L] = (int32_t)((on && !fin) ? w.lat_nbase[(size_t)L * F + t + 1] : 0u);   // frame t + 1's
        }
        tab_publish(tab, w.max_lanes, units);
    }
    // (the flags of the frame's flat epsilon rounds start clear)
    if (blockIdx.x == 0 && threadIdx.x < (unsigned)w.max_lanes && w.lat_chg) w.lat_chg[threadIdx.x] = 0u;
    __syncthreads();
    const int nl = w.max_lanes;
    const int lane = wlane();
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)lane;
        const bool fin = tab.ph[L] != 0;
        uint32_t *bwd = w.lat_bwd + (size_t)L * w.lat_nodes;
        bool keep = false;
        int32_t rec[kLatFields];
        int4 r = make_int4(0, 0, 0, 1);
        if (i < tab.n[L]) r = w.lat_arc[(size_t)L * w.lat_cap + tab.fb[L] + i];
        if (r.w == 0) {   // (epsilon arcs of the step's closure, and lanes past their arcs, skip)
            const int32_t arc = r.y;
            const bool redirect = (uint32_t)arc >= (uint32_t)w.num_arcs;
            ArcDLW ad = {0, 0u, 0.0f};
            if (!redirect) ad = w.arc_dlw[arc];
            float sa;
            if (fin) {
                sa = redirect ? 0.0f : ad.weight;
            } else {
                const LPT *row = (const LPT *)d.base + (long long)tab.row[L] * d.stride_b + (long long)t * d.stride_t;
                sa = ad.weight + lp_at(row, ad.ilabel);
            }
            const size_t se = (size_t)tab.arcs[L] + (uint32_t)r.x;   // source node
            const float bd = fin ? 0.0f : ord2f(bwd[(uint32_t)tab.win[L] + (uint32_t)r.z]);
            const float v = sa + bd;
            if (v > -__builtin_inff()) atomicMax(&bwd[se], f2ord(v));
            const float fwd = w.lat_score[(size_t)L * w.lat_nodes + se];
            const float thr = (fwd + sa) + bd;
            keep = thr >= tab.f1[L];
            if (keep) {
                rec[kLatFrame] = t;
                rec[kLatSrc] = w.lat_state[(size_t)L * w.lat_nodes + se];
                rec[kLatDst] = (redirect || fin) ? w.super_final : (int32_t)dest_state(w, ad.dest);
                rec[kLatIlabel] = fin ? -1 : (int32_t)ad.ilabel;
                rec[kLatArc] = user_arc(w, arc);
                rec[kLatScore] = (int32_t)__float_as_uint(sa);
                rec[kLatLane] = L;
                rec[kLatFlags] = redirect ? 2 : (fin ? 1 : 0);
            }
        }
        const unsigned long long m = __ballot(keep);
        if (m == 0ull) continue;
        LaneCtl &c = w.ctl[L];
        const int leader = __ffsll((long long)m) - 1;
        uint32_t ob = 0u;
        if (lane == leader) ob = atomicAdd(&c.lat_out_n, (uint32_t)__popcll(m));
        ob = __shfl(ob, leader, kWave);
        if (keep) {
            const uint32_t oi = ob + (uint32_t)__popcll(m & mask_lt());
            if (oi < w.lat_cap) {
                int32_t *o = w.lat_out + ((size_t)L * w.lat_cap + oi) * kLatFields;
#pragma unroll
                for (int f = 0; f < kLatFields; ++f) o[f] = rec[f];
            }
        }
    }
}

// Backward sweeps of one workgroup per lane. The interval prune (k_lat_prune:
// the last 2N frames of a running lane) walks frames from the last to the
// first; for each frame f:
//  1. frame f's nodes start at -inf;
//  2. the arcs of step f (records of slot f + 1 with pass 0; their destinations
//     lie in frame f + 1, whose backward scores are final by now) raise
//     bwd(source) with one atomicMax each and are marked at once;
//  3. frame f's epsilon arcs (records of slot f with a pass > 0; both ends in
//     frame f) relax bwd(source) to the least fixpoint, then are marked.
// The final pass runs step 2 flat over lanes (k_lat_back, above) and step 3 as
// flat rounds over all lanes' records, finishing per lane only where a chain is
// still open (k_lat_eps_round, k_lat_eps_back, below). A sweep runs on as many
// workgroups as lanes, so its speed is set by the memory latency of each frame
// inside a workgroup. The prune's sweep therefore waits on no gather: a flat
// kernel over the whole chip (k_lat_prep) first turns every step arc of the
// window into a work record (positions, arc score, forward score of the
// source), and the sweep keeps the backward scores of the two frames it works
// on in LDS (a frame that does not fit beside the other in memory), so a frame
// costs one coalesced load of its work records, issued a frame ahead, and LDS
// operations. The final pass's per-lane epsilon fixpoint runs in LDS when the
// frame's nodes fit, else on the scores in memory.
constexpr int kLatSweepBlock = 1024;
constexpr int kLatBatch = 8;                  // records per thread per load round
constexpr int kLatEpsRegs = 8;                // epsilon-slot records per thread per load round (half in the prune)
constexpr uint32_t kLatEpsLdsNodes = 35840;   // frame nodes whose backward scores fit in LDS (140 KiB)
constexpr int kMaxPruneInterval = 512;        // 2N + 1 step offsets fit the workgroup's table
constexpr int kLatKeepBlocks = 256;           // workgroups of the final pass's flat epsilon keep
constexpr int kLatPrepBlock = 256;
constexpr int kLatPrepRecs = 4;              // prune work records per thread per load round

struct SweepShared {
    uint32_t bwd[kLatEpsLdsNodes];               // backward scores of one frame (final pass) or two (prune)
    uint32_t off0[2 * kMaxPruneInterval + 2];    // prune: step offsets of slots W .. F before compaction
    uint32_t nb0[2 * kMaxPruneInterval + 2];     // prune: first nodes of frames W .. F
    uint32_t exs[kLatSweepBlock];                // compaction: survivors before each thread's records
    uint32_t kmask[kLatSweepBlock];              // compaction: each thread's survivor bits
    uint32_t wtot[kLatSweepBlock / kWave];       // compaction: survivors per wavefront
};

// One lane's lattice arrays, and the keep threshold of the sweep: an arc is
// kept when (fwd(source) + s) + bwd(destination) >= thr.
struct SweepLane {
    int L;
    int4 *rec;
    uint32_t *bwd;
    const float *fwd;
    const int32_t *state;
    const uint8_t *epass;
    float thr;
};

__device__ __forceinline__ SweepLane sweep_lane(const Work &w, int L, float thr)
{
    const size_t nodes = (size_t)L * w.lat_nodes;
    return SweepLane{L, w.lat_arc + (size_t)L * w.lat_cap, w.lat_bwd + nodes, w.lat_score + nodes,
                     w.lat_state + nodes, w.lat_epass + nodes, thr};
}

__device__ __forceinline__ uint32_t load_bwd(const uint32_t *p)
{
    // (other threads of the workgroup raise these with atomics: read past L1)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Appends a wavefront's kept records (final pass) to lane L's output, one
// atomicAdd per wavefront. Every thread of the wavefront calls it.
__device__ __forceinline__ void lat_emit(const Work &w, LaneCtl &c, int L, bool keep, const int32_t (&o)[kLatFields])
{
    const unsigned long long m = __ballot(keep);
    if (m == 0ull) return;
    const int leader = __ffsll((long long)m) - 1;
    uint32_t ob = 0u;
    if (wlane() == leader) ob = atomicAdd(&c.lat_out_n, (uint32_t)__popcll(m));
    ob = __shfl(ob, leader, kWave);
    if (!keep) return;
    const uint32_t oi = ob + (uint32_t)__popcll(m & mask_lt());
    if (oi >= w.lat_cap) return;
    int32_t *dst = w.lat_out + ((size_t)L * w.lat_cap + oi) * kLatFields;
#pragma unroll
    for (int f = 0; f < kLatFields; ++f) dst[f] = o[f];
}

// Keeps (final pass) or marks (prune) one epsilon record of frame f with
// weight wt, source node se, the destination's backward score bd; fw = fwd(se),
// ep = the pass that last relaxed the source (final pass: a record is kept
// once, from that pass, which admitted every arc an earlier pass did, the
// source's score having only grown). Every thread of the wavefront calls it.
template <bool PRUNE>
__device__ __forceinline__ void eps_keep(const Work &w, LaneCtl &c, const SweepLane &s, int f, bool on,
                                         const int4 &r, uint32_t i, uint32_t se, float wt, float fw, float bd, int ep)
{
    const bool pass = on && ((fw + wt) + bd) >= s.thr;
    if (PRUNE) {
        if (on && !pass) s.rec[i].w = -1;
        return;
    }
    const bool keep = pass && ep == r.w;
    int32_t o[kLatFields] = {};
    if (keep) {
        const ArcDLW ad = w.arc_dlw[r.y];
        o[kLatFrame] = f;
        o[kLatSrc] = s.state[se];
        o[kLatDst] = (int32_t)dest_state(w, ad.dest);
        o[kLatIlabel] = (int32_t)ad.ilabel;
        o[kLatArc] = user_arc(w, r.y);
        o[kLatScore] = (int32_t)__float_as_uint(wt);
        o[kLatLane] = s.L;
        o[kLatFlags] = 4;
    }
    lat_emit(w, c, s.L, keep, o);
}

// Frame f's epsilon arcs: records [e0, e1) of slot f, those with a pass > 0,
// over nodes ns .. ns + nn - 1 (step 3 of the sweep). The fixpoint
// bwd(src) = max(bwd(src), weight + bwd(dst)) runs in rounds until one changes
// nothing (the least fixpoint: epsilon weights are <= 0 in lattice mode; a
// bound of one round per record + 1 ends them in any case). A round visits
// the records from the last to the first, a barrier after each 1024, so that
// later closure passes go first and most chains settle in one round. The
// scores live in LDS when the frame's nodes fit (bw = the LDS copy, indexed by
// position), else in memory (bw = the frame's first node); each round loads
// kLatEpsRegs records per thread at a time, or keeps them in registers when
// the frame has no more.
template <bool PRUNE, bool LDS, int R>
__device__ __forceinline__ void eps_fix(const Work &w, LaneCtl &c, const SweepLane &s, uint32_t *bw, int f,
                                        uint32_t e0, uint32_t e1, uint32_t ns, uint32_t nn)
{
    const uint32_t tid = threadIdx.x;
    constexpr uint32_t kSuper = (uint32_t)R * kLatSweepBlock;
    const uint32_t n = e1 - e0;
    const uint32_t nsup = (n + kSuper - 1) / kSuper;
    auto get = [&](uint32_t x) -> uint32_t { return LDS ? bw[x] : load_bwd(&bw[x]); };
    int4 r[R];
    float wt[R];
    auto load = [&](uint32_t q) {
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const uint32_t i = e0 + q * kSuper + (uint32_t)k * kLatSweepBlock + tid;
            r[k] = i < e1 ? s.rec[i] : make_int4(0, 0, 0, 0);
            if (!(r[k].w > 0 && (uint32_t)r[k].x < nn && (uint32_t)r[k].z < nn)) r[k].w = 0;
        }
#pragma unroll
        for (int k = 0; k < R; ++k) wt[k] = r[k].w > 0 ? w.arc_dlw[r[k].y].weight : 0.0f;
    };
    // relaxes the loaded records, last first; the number of 1024-record
    // groups present (kn) is workgroup-uniform. With `each`, a barrier follows
    // every group (a later group's raises are seen by the earlier ones: most
    // chains settle in one round); without, the loads of every group are
    // issued before any atomic and one barrier ends the batch (scores in
    // memory: one load and one atomic latency per batch instead of per group)
    auto relax = [&](uint32_t q, bool each) -> int {
        const uint32_t left = e1 - (e0 + q * kSuper);
        const int kn = (int)min((left + kLatSweepBlock - 1) / kLatSweepBlock, (uint32_t)R);
        int ch = 0;
        if (each) {
#pragma unroll
            for (int k = R - 1; k >= 0; --k) {
                if (k >= kn) continue;
                if (r[k].w > 0) {
                    const float v = wt[k] + ord2f(get((uint32_t)r[k].z));
                    if (v > -__builtin_inff()) {
                        const uint32_t o = f2ord(v);
                        if (atomicMax(&bw[(uint32_t)r[k].x], o) < o) ch = 1;
                    }
                }
                __syncthreads();
            }
        } else {
            float bd[R];
#pragma unroll
            for (int k = R - 1; k >= 0; --k)
                bd[k] = (k < kn && r[k].w > 0) ? ord2f(get((uint32_t)r[k].z)) : -__builtin_inff();
#pragma unroll
            for (int k = R - 1; k >= 0; --k) {
                const float v = wt[k] + bd[k];
                if (k < kn && r[k].w > 0 && v > -__builtin_inff()) {
                    const uint32_t o = f2ord(v);
                    if (atomicMax(&bw[(uint32_t)r[k].x], o) < o) ch = 1;
                }
            }
            __syncthreads();
        }
        return ch;
    };
    if (nsup == 1) load(0);
    for (uint32_t round = 0; round <= n + 1u; ++round) {
        // scores in LDS: a barrier per group in every round; in memory: in the
        // first round only (it settles most chains), later rounds batched
        const bool each = LDS || round == 0;
        int ch = 0;
        if (nsup == 1) {
            ch = relax(0, each);
        } else {
            for (uint32_t q = nsup; q-- > 0;) {
                load(q);
                ch |= relax(q, each);
            }
        }
        if (!__syncthreads_or(ch)) break;
    }
    // keep (final pass) or mark (prune)
    for (uint32_t q = 0; q < nsup; ++q) {
        if (nsup > 1) load(q);
        float fw[R];
        int ep[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const bool on = r[k].w > 0;
            fw[k] = on ? s.fwd[ns + (uint32_t)r[k].x] : 0.0f;
            ep[k] = (!PRUNE && on) ? (int)s.epass[ns + (uint32_t)r[k].x] : 0;
        }
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const uint32_t i = e0 + q * kSuper + (uint32_t)k * kLatSweepBlock;
            if (i >= e1) continue;   // (workgroup-uniform)
            const bool on = r[k].w > 0;
            const float bd = on ? ord2f(get((uint32_t)r[k].z)) : 0.0f;
            eps_keep<PRUNE>(w, c, s, f, on, r[k], i + tid, ns + (uint32_t)r[k].x, wt[k], fw[k], bd, ep[k]);
        }
    }
}

template <bool PRUNE, int R>
__device__ void sweep_eps(const Work &w, LaneCtl &c, const SweepLane &s, SweepShared &sh, int f,
                          uint32_t e0, uint32_t e1, uint32_t ns, uint32_t nn)
{
    if (e1 <= e0) return;
    const uint32_t tid = threadIdx.x;
    if (nn <= kLatEpsLdsNodes) {
        for (uint32_t i = tid; i < nn; i += kLatSweepBlock) sh.bwd[i] = load_bwd(&s.bwd[ns + i]);
        __syncthreads();
        eps_fix<PRUNE, true, R>(w, c, s, sh.bwd, f, e0, e1, ns, nn);
        for (uint32_t i = tid; i < nn; i += kLatSweepBlock) s.bwd[ns + i] = sh.bwd[i];
    } else {
        eps_fix<PRUNE, false, R>(w, c, s, s.bwd + ns, f, e0, e1, ns, nn);
    }
}

// The final pass over frame t's epsilon arcs (records of slot t with a pass
// > 0) on graphs with epsilon arcs, after k_lat_back(t): R flat rounds over
// every lane's records (k_lat_eps_round: each record once per round,
// bwd(src) = max(bwd(src), weight + bwd(dst)), any order; the last round
// records per lane whether it raised a score), then k_lat_eps_back: a lane
// whose last round raised nothing has reached the least fixpoint (no record can
// raise a score: each was tried against scores no one changed) and its records
// are kept flat over the grid; a lane whose last round raised a score gets a
// workgroup that runs the fixpoint to its end and keeps its records itself.
// Frames of tens of thousands of records (the largest lane's sets the time of
// a per-lane pass) are so spread over every CU; R = min(passes, 3) + 1 rounds
// settle chains of up to R - 1 epsilon arcs without a finishing workgroup.

// Lane table of the flat epsilon passes of frame t: records [aoff[t],
// aoff[t + 1]) of lanes with a result and a complete lattice (and, for the
// keep, whose last round raised no score); tab.fb = first record, tab.arcs =
// the frame's first node, tab.win = its node count, tab.f1 = the threshold.
__device__ __forceinline__ void eps_tab(const Work &w, LaneTab &tab, int t, bool keep)
{
    if (threadIdx.x >= kWave) return;
    const int L = (int)threadIdx.x;
    const size_t F = (size_t)w.max_frames + 3;
    uint32_t units = 0;
    if (L < w.max_lanes) {
        const LaneCtl &c = w.ctl[L];
        bool on = lane_has_result(c) && t <= c.last_step && lat_complete(w, c);
        if (keep && on) on = w.lat_chg[L] == 0u;
        const uint32_t a0 = on ? w.lat_aoff[(size_t)L * F + t] : 0u;
        const uint32_t a1 = on ? min(w.lat_aoff[(size_t)L * F + t + 1], w.lat_cap) : 0u;
        const uint32_t n = a1 > a0 ? a1 - a0 : 0u;
        const uint32_t nb = on ? w.lat_nbase[(size_t)L * F + t] : 0u;
        units = (n + kWave - 1) / kWave;
        tab.n[L] = n;
        tab.fb[L] = a0;
        tab.arcs[L] = nb;
        tab.win[L] = on ? (int32_t)(w.lat_nbase[(size_t)L * F + t + 1] - nb) : 0;
        tab.f1[L] = c.final_score - w.output_beam;
    }
    tab_publish(tab, w.max_lanes, units);
}

__global__ __launch_bounds__(kBlock) void k_lat_eps_round(const Work *__restrict__ wp, int t, int last)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    eps_tab(w, tab, t, false);
    __syncthreads();
    const int nl = w.max_lanes;
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)wlane();
        const uint32_t nn = (uint32_t)tab.win[L];
        int4 r = make_int4(0, 0, 0, 0);
        if (i < tab.n[L]) r = w.lat_arc[(size_t)L * w.lat_cap + tab.fb[L] + i];
        if (!(r.w > 0 && (uint32_t)r.x < nn && (uint32_t)r.z < nn)) continue;
        uint32_t *bwd = w.lat_bwd + (size_t)L * w.lat_nodes + tab.arcs[L];
        const float v = w.arc_dlw[r.y].weight + ord2f(load_bwd(&bwd[(uint32_t)r.z]));
        if (!(v > -__builtin_inff())) continue;
        const uint32_t o = f2ord(v);
        if (last) {
            if (atomicMax(&bwd[(uint32_t)r.x], o) < o) w.lat_chg[L] = 1u;
        } else {
            atomicMax(&bwd[(uint32_t)r.x], o);
        }
    }
}

// Workgroups 0 .. max_lanes - 1: the finishing workgroup of lane blockIdx.x
// (when its last round raised a score); the rest: the flat keep of every other
// lane's records.
__global__ __launch_bounds__(kLatSweepBlock) void k_lat_eps_back(const Work *__restrict__ wp, int t)
{
    const Work &w = *wp;
    __shared__ union {
        SweepShared sweep;
        LaneTab tab;
    } sh;
    const int nl = w.max_lanes;
    if ((int)blockIdx.x < nl) {
        const int L = (int)blockIdx.x;
        LaneCtl &c = w.ctl[L];
        if (w.lat_chg[L] == 0u || !lane_has_result(c) || t > c.last_step || !lat_complete(w, c)) return;
        const size_t FF = (size_t)w.max_frames + 3;
        const uint32_t *aoff = w.lat_aoff + (size_t)L * FF;
        const uint32_t *nbase = w.lat_nbase + (size_t)L * FF;
        const SweepLane s = sweep_lane(w, L, c.final_score - w.output_beam);
        sweep_eps<false, kLatEpsRegs>(w, c, s, sh.sweep, t, aoff[t], min(aoff[t + 1], w.lat_cap), nbase[t],
                                      nbase[t + 1] - nbase[t]);
        return;
    }
    LaneTab &tab = sh.tab;
    eps_tab(w, tab, t, true);
    __syncthreads();
    // this wavefront's equal share of the keep blocks' units
    const uint32_t wpb = kLatSweepBlock / kWave;
    const uint32_t nwaves = (gridDim.x - (uint32_t)nl) * wpb;
    const uint32_t wid = (blockIdx.x - (uint32_t)nl) * wpb + threadIdx.x / kWave;
    const uint32_t total = tab.base[nl];
    const uint32_t u_beg = (uint32_t)(((unsigned long long)total * wid) / nwaves);
    const uint32_t u_end = (uint32_t)(((unsigned long long)total * (wid + 1)) / nwaves);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)wlane();
        const uint32_t nn = (uint32_t)tab.win[L];
        const SweepLane s = sweep_lane(w, L, tab.f1[L]);
        int4 r = make_int4(0, 0, 0, 0);
        if (i < tab.n[L]) r = s.rec[tab.fb[L] + i];
        const bool on = r.w > 0 && (uint32_t)r.x < nn && (uint32_t)r.z < nn;
        const uint32_t se = tab.arcs[L] + (uint32_t)r.x;
        float wt = 0.0f, fw = 0.0f, bd = 0.0f;
        int ep = 0;
        if (on) {
            wt = w.arc_dlw[r.y].weight;
            fw = s.fwd[se];
            ep = (int)s.epass[se];
            bd = ord2f(s.bwd[tab.arcs[L] + (uint32_t)r.z]);
        }
        eps_keep<false>(w, w.ctl[L], s, t, on, r, tab.fb[L] + i, se, wt, fw, bd, ep);
    }
}

// Lanes the interval prune after real step t works on: running lanes with more
// real steps whose lattice has not overflowed.
__device__ __forceinline__ bool prune_lane(const Work &w, const LaneCtl &c, int t)
{
    return c.status == kActive && c.last_step == t && t + 1 < c.T && lat_complete(w, c);
}

// The prune's work records of lane L: its output area, unused until the final
// pass (which runs after every prune), holds one int4 per record index.
__device__ __forceinline__ int4 *lat_work(const Work &w, int L)
{
    return reinterpret_cast<int4 *>(w.lat_out + (size_t)L * w.lat_cap * kLatFields);
}

// Work records of the interval prune after real step t, flat over lanes and
// slots (blockIdx.y = lane, blockIdx.x = slot W + 1 + x, whose records hold
// step x + W's arcs and frame x + W + 1's epsilon arcs): for each record of the
// slot, {source position, destination position, s = weight + log-prob, fwd of
// the source} for a step arc (pass 0), y = -1 for any other. Step t's own arcs
// still hold destination states: their positions come from frame F's map.
template <typename LPT>
__global__ __launch_bounds__(kLatPrepBlock) void k_lat_prep(const Work *__restrict__ wp, int t)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.y;
    if (L >= w.max_lanes) return;
    const LaneCtl &c = w.ctl[L];
    if (!prune_lane(w, c, t)) return;
    const int F = t + 1, W = max(0, F - 2 * w.lat_prune_interval);
    const int sl = W + 1 + (int)blockIdx.x;
    if (sl > F) return;
    const size_t FF = (size_t)w.max_frames + 3;
    const uint32_t *aoff = w.lat_aoff + (size_t)L * FF;
    const uint32_t a0 = aoff[sl], a1 = sl < F ? aoff[sl + 1] : c.lat_cursor;
    const uint32_t ns = w.lat_nbase[(size_t)L * FF + (size_t)(sl - 1)];
    const int32_t *dpos = sl == F ? pick(w.pos, lane_par(c, F)) + (size_t)L * w.num_states : nullptr;
    const LpDesc d = *w.lp;
    const LPT *row = (const LPT *)d.base + (long long)c.lp_row * d.stride_b + (long long)(sl - 1) * d.stride_t;
    const int4 *rec = w.lat_arc + (size_t)L * w.lat_cap;
    const float *fwd = w.lat_score + (size_t)L * w.lat_nodes;
    int4 *work = lat_work(w, L);
    // kLatPrepRecs records per thread at a time, each level of loads issued
    // for all of them before any is used
    constexpr uint32_t kStride = (uint32_t)kLatPrepRecs * kLatPrepBlock;
    for (uint32_t b0 = a0; b0 < a1; b0 += kStride) {
        int4 r[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            const uint32_t i = b0 + (uint32_t)k * kLatPrepBlock + threadIdx.x;
            r[k] = i < a1 ? rec[i] : make_int4(0, 0, 0, 1);
        }
        ArcDLW ad[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) ad[k] = r[k].w == 0 ? w.arc_dlw[r[k].y] : ArcDLW{0, 0u, 0.0f};
        int4 o[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            o[k] = make_int4(0, -1, 0, 0);
            if (r[k].w != 0) continue;
            const float sa = ad[k].weight + lp_at(row, ad[k].ilabel);
            const uint32_t dz = (uint32_t)r[k].z;
            const uint32_t dp = (dpos && (dz & kLatUnresolved)) ? (uint32_t)dpos[dz & ~kLatUnresolved] : dz;
            o[k] = make_int4(r[k].x, (int)dp, (int)__float_as_uint(sa),
                             (int)__float_as_uint(fwd[ns + (uint32_t)r[k].x]));
        }
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            const uint32_t i = b0 + (uint32_t)k * kLatPrepBlock + threadIdx.x;
            if (i < a1) work[i] = o[k];
        }
    }
}

// LDS place of the prune sweep's frame of n nodes beside the live frame at
// [po, po + pn) (po == kNoLds: that one is in memory): right after it, else
// before it, else kNoLds (the frame's scores stay in memory).
constexpr uint32_t kNoLds = 0xFFFFFFFFu;
// Pass field of an arc the final pass keeps (it runs only without closure
// passes, so every other arc still holds pass 0).
constexpr int32_t kFinalKept = 1;
__device__ __forceinline__ uint32_t lds_place(uint32_t n, uint32_t po, uint32_t pn)
{
    if (n > kLatEpsLdsNodes) return kNoLds;
    if (po == kNoLds) return 0u;
    if (po + pn + n <= kLatEpsLdsNodes) return po + pn;
    return n <= po ? 0u : kNoLds;
}

// The prune's backward sweep over frames F - 1 .. W (steps 1-3 above) on the
// work records of slots W + 1 .. F (slot F's ending at `cursor`); frame F's
// scores are set, at LDS offset oF (or in memory). Returns frame W's LDS offset
// (kNoLds: its scores are in memory). The prune marks the arcs it drops (pass
// field -1), the final pass (FINAL) the ones it keeps (kFinalKept). Two
// frames are live at a time, f + 1 (read) and f (raised): each gets a place in
// the LDS array beside the other (lds_place), or the whole array when it fits
// alone (the other's scores then move to memory), or stays in memory. Without
// epsilon arcs the next frame's first batch of work records is loaded as this
// frame starts; with them, after the frame's fixpoint (whose loads need the
// registers).
template <bool EPS, bool FINAL = false>
__device__ __forceinline__ uint32_t prune_sweep(const Work &w, LaneCtl &c, const SweepLane &s, SweepShared &sh,
                                            const int4 *__restrict__ work, int F, int W, uint32_t nF, uint32_t oF,
                                            uint32_t cursor, int4 (&r)[kLatBatch])
{
    const uint32_t tid = threadIdx.x;
    auto nodes = [&](int f) -> uint32_t { return f == F ? nF : sh.nb0[f + 1 - W] - sh.nb0[f - W]; };
    auto load_work = [&](uint32_t b0, uint32_t a1, int4 (&x)[kLatBatch]) {
#pragma unroll
        for (int k = 0; k < kLatBatch; ++k) {
            const uint32_t i = b0 + (uint32_t)k * kLatSweepBlock + tid;
            x[k] = i < a1 ? work[i] : make_int4(0, -1, 0, 0);
        }
    };
    // frame g's nodes at -inf, at LDS offset o or in memory
    auto clear = [&](int g, uint32_t o) {
        const uint32_t n = nodes(g);
        if (o != kNoLds)
            for (uint32_t i = tid; i < n; i += kLatSweepBlock) sh.bwd[o + i] = kOrdNegInf;
        else
            for (uint32_t i = tid; i < n; i += kLatSweepBlock) s.bwd[sh.nb0[g - W] + i] = kOrdNegInf;
    };
    // a frame that fits the LDS array alone but not beside the frame it reads
    // takes the whole array; that frame's scores move to memory first (the
    // step that reads them, the next one, gathers them there)
    auto evict = [&](uint32_t o, uint32_t n, uint32_t nbase) {
        for (uint32_t i = tid; i < n; i += kLatSweepBlock) s.bwd[nbase + i] = sh.bwd[o + i];
        __syncthreads();
    };
    uint32_t od = oF, os = lds_place(nodes(F - 1), oF, nF);
    if (os == kNoLds && od != kNoLds && nodes(F - 1) <= kLatEpsLdsNodes) {
        evict(od, nF, sh.nb0[F - W]);
        od = kNoLds;
        os = 0u;
    }
    clear(F - 1, os);
    load_work(sh.off0[F - W], cursor, r);   // step F - 1's first batch
    __syncthreads();
    for (int f = F - 1; f >= W; --f) {
        const uint32_t ns = sh.nb0[f - W], nd = sh.nb0[f + 1 - W], nn = nodes(f);
        const bool ls = os != kNoLds, ld = od != kNoLds;
        const uint32_t a0 = sh.off0[f + 1 - W], a1 = (f + 1 < F) ? sh.off0[f + 2 - W] : cursor;
        const uint32_t n0 = f > W ? sh.off0[f - W] : 0u, n1 = f > W ? sh.off0[f + 1 - W] : 0u;
        int4 nx[kLatBatch];
        if (!EPS) load_work(n0, n1, nx);
        for (uint32_t b0 = a0; b0 < a1; b0 += (uint32_t)kLatBatch * kLatSweepBlock) {
            if (b0 != a0) load_work(b0, a1, r);
            float bv[kLatBatch];
            if (ld) {
#pragma unroll
                for (int k = 0; k < kLatBatch; ++k) bv[k] = r[k].y != -1 ? ord2f(sh.bwd[od + (uint32_t)r[k].y]) : 0.0f;
            } else {
#pragma unroll
                for (int k = 0; k < kLatBatch; ++k)
                    bv[k] = r[k].y != -1 ? ord2f(load_bwd(&s.bwd[nd + (uint32_t)r[k].y])) : 0.0f;
            }
#pragma unroll
            for (int k = 0; k < kLatBatch; ++k) {
                if (r[k].y == -1) continue;   // (also positions past a1)
                const float sa = __int_as_float(r[k].z), fw = __int_as_float(r[k].w);
                const float v = sa + bv[k];
                if (v > -__builtin_inff()) {
                    if (ls) atomicMax(&sh.bwd[os + (uint32_t)r[k].x], f2ord(v));
                    else atomicMax(&s.bwd[ns + (uint32_t)r[k].x], f2ord(v));
                }
                const bool kept = ((fw + sa) + bv[k]) >= s.thr;
                if (FINAL ? kept : !kept) s.rec[b0 + (uint32_t)k * kLatSweepBlock + tid].w = FINAL ? kFinalKept : -1;
            }
        }
        if (EPS) {
            __syncthreads();
            const uint32_t e0 = sh.off0[f - W], e1 = sh.off0[f + 1 - W];
            if (e1 > e0) {
                if (ls) eps_fix<true, true, kLatEpsRegs / 2>(w, c, s, sh.bwd + os, f, e0, e1, ns, nn);
                else eps_fix<true, false, kLatEpsRegs / 2>(w, c, s, s.bwd + ns, f, e0, e1, ns, nn);
            }
            load_work(n0, n1, nx);
        }
#pragma unroll
        for (int k = 0; k < kLatBatch; ++k) r[k] = nx[k];
        if (f > W) {
            __syncthreads();   // frame f final, frame f + 1 no longer read
            uint32_t o = lds_place(nodes(f - 1), os, nn);
            if (o == kNoLds && ls && nodes(f - 1) <= kLatEpsLdsNodes) {
                evict(os, nn, ns);
                os = kNoLds;
                o = 0u;
            }
            clear(f - 1, o);
            od = os;
            os = o;
            __syncthreads();
        }
    }
    return os;
}

// Interval prune (page section 7, lat_prune_interval = N: a window-loose prune
// that bounds the lattice, the exact final pass unchanged), after real step t
// with (t + 1) % N == 0 for lanes with more real steps, one workgroup per lane,
// after k_lat_prep(t). With F = t + 1 the frontier's frame and
// W = max(0, F - 2N): the sweep over frames F - 1 .. W starts from
// bwd(u) = -fwd(u) at every frontier token u (no complete path through u can
// score more than the final best) and marks (pass field -1) the arcs of steps
// W .. F - 1 and the epsilon arcs of frames W .. F - 1 with
// (fwd(src) + s) + bwd(dst) < 0 - output_beam; then the records from step
// W - 1's first to the cursor are compacted in place, in order, with the step
// offsets rewritten.
__global__ __launch_bounds__(kLatSweepBlock) void k_lat_prune(const Work *__restrict__ wp, int t)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.x;
    if (L >= w.max_lanes) return;
    LaneCtl &c = w.ctl[L];
    if (!prune_lane(w, c, t)) return;
    __shared__ SweepShared sh;
    const int F = t + 1;
    const int W = max(0, F - 2 * w.lat_prune_interval);
    const size_t FF = (size_t)w.max_frames + 3;
    uint32_t *aoff = w.lat_aoff + (size_t)L * FF;
    const uint32_t *nbase = w.lat_nbase + (size_t)L * FF;
    const SweepLane s = sweep_lane(w, L, 0.0f - w.output_beam);
    const uint32_t nF = (uint32_t)c.cnt[lane_par(c, F)];
    const uint32_t cursor = c.lat_cursor;
    const uint32_t tid = threadIdx.x;
    const int nslot = F - W + 1;
    for (int i = (int)tid; i < nslot; i += kLatSweepBlock) {
        sh.off0[i] = aoff[W + i];
        sh.nb0[i] = nbase[W + i];
    }
    const uint32_t nf0 = nbase[F], oF = lds_place(nF, kNoLds, 0u);
    if (oF != kNoLds)
        for (uint32_t i = tid; i < nF; i += kLatSweepBlock) sh.bwd[oF + i] = f2ord(0.0f - s.fwd[nf0 + i]);
    else
        for (uint32_t i = nf0 + tid; i < nf0 + nF; i += kLatSweepBlock) s.bwd[i] = f2ord(0.0f - s.fwd[i]);
    __syncthreads();   // (sh.nb0 and sh.off0 too)
    int4 r[kLatBatch];
    if (w.has_eps) prune_sweep<true>(w, c, s, sh, lat_work(w, L), F, W, nF, oF, cursor, r);
    else prune_sweep<false>(w, c, s, sh, lat_work(w, L), F, W, nF, oF, cursor, r);
    __syncthreads();   // the last frame's marks (slots W and W + 1) before any is read
    // in-place compaction of [off0[0], cursor), kLatBatch records per thread (a
    // contiguous run) per chunk: every record of a chunk is read before any is
    // written, and survivors only move down, so no unread record is overwritten;
    // the next chunk's records are loaded while this one's are written (they lie
    // past every position this chunk writes)
    constexpr uint32_t kChunk = (uint32_t)kLatBatch * kLatSweepBlock;
    const uint32_t wv = tid / kWave;
    uint32_t out = sh.off0[0];
    auto load_chunk = [&](uint32_t b, int4 (&x)[kLatBatch]) {
#pragma unroll
        for (int k = 0; k < kLatBatch; ++k) {
            const uint32_t i = b + tid * (uint32_t)kLatBatch + (uint32_t)k;
            x[k] = i < cursor ? s.rec[i] : make_int4(0, 0, 0, -1);
        }
    };
    load_chunk(sh.off0[0], r);
    for (uint32_t b0 = sh.off0[0]; b0 < cursor; b0 += kChunk) {
        uint32_t km = 0u;
#pragma unroll
        for (int k = 0; k < kLatBatch; ++k)
            if (r[k].w != -1) km |= 1u << k;
        __syncthreads();
        int4 nx[kLatBatch];
        load_chunk(b0 + kChunk, nx);
        uint32_t tot;
        const uint32_t ex = wave_excl_sum((uint32_t)__popc(km), &tot);
        if (wlane() == 0) sh.wtot[wv] = tot;
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (uint32_t x = 0; x < (uint32_t)(kLatSweepBlock / kWave); ++x) {
            if (x < wv) before += sh.wtot[x];
            all += sh.wtot[x];
        }
        sh.exs[tid] = before + ex;
        sh.kmask[tid] = km;
        uint32_t o = out + before + ex;
#pragma unroll
        for (int k = 0; k < kLatBatch; ++k)
            if ((km >> k) & 1u) s.rec[o++] = r[k];
        __syncthreads();
        // slots whose first record lies in this chunk start at its survivors' place
        for (int sl = 1 + (int)tid; sl < nslot; sl += kLatSweepBlock) {
            const uint32_t p = sh.off0[sl];
            if (p >= b0 && p < b0 + kChunk && p < cursor) {
                const uint32_t j = p - b0, th = j / (uint32_t)kLatBatch, q = j % (uint32_t)kLatBatch;
                aoff[W + sl] = out + sh.exs[th] + (uint32_t)__popc(sh.kmask[th] & ((1u << q) - 1u));
            }
        }
        out += all;
#pragma unroll
        for (int k = 0; k < kLatBatch; ++k) r[k] = nx[k];
        __syncthreads();
    }
    for (int sl = 1 + (int)tid; sl < nslot; sl += kLatSweepBlock)
        if (sh.off0[sl] >= cursor) aoff[W + sl] = out;
    if (tid == 0) c.lat_cursor = out;
}

// Final pass on a graph without closure passes, as three launches instead of
// one per frame: every persisted arc is a step arc, so the backward scores
// follow from one sweep over the frames per lane (the interval prune's sweep,
// prune_sweep, over the whole lattice), fed by work records a flat kernel
// makes first, and a flat kernel then writes the kept arcs out. The arcs kept,
// their fields and their scores are those of k_lat_back.

// A lane that gets the final pass: it has a result, every arc it persisted was
// written, and it ran a step.
__device__ __forceinline__ bool lat_final_lane(const Work &w, const LaneCtl &c)
{
    return lane_has_result(c) && lat_complete(w, c) && c.last_step >= 0;
}

// Records of step ts of lane L: [a0, a1) of its lattice arcs; fin: ts is the
// lane's final step (its arcs are final arcs, or the redirect).
struct FinalStep {
    uint32_t a0, a1, ns;   // ns: first node of frame ts (the sources)
    bool fin;
};

__device__ __forceinline__ FinalStep final_step(const Work &w, const LaneCtl &c, int L, int ts)
{
    const size_t FF = (size_t)w.max_frames + 3;
    const uint32_t *aoff = w.lat_aoff + (size_t)L * FF;
    const bool fin = ts == c.last_step;
    return FinalStep{aoff[ts + 1], min(fin ? c.lat_cursor : aoff[ts + 2], w.lat_cap),
                     w.lat_nbase[(size_t)L * FF + (size_t)ts], fin};
}

// s of an arc of step ts as the backward pass adds it: weight + log-prob of
// frame ts; on the final step the final arc's weight, 0 for the redirect.
template <typename LPT>
__device__ __forceinline__ float final_arc_score(bool fin, bool redirect, const ArcDLW &ad, const LPT *row)
{
    if (fin) return redirect ? 0.0f : ad.weight;
    return ad.weight + lp_at(row, ad.ilabel);
}

// Work records of the final pass (blockIdx.y = lane, blockIdx.x = step ts):
// for each arc of step ts, {source position, destination position, s, fwd of
// the source}; the final step's arcs (and the redirect) all lead to the
// super-final node (position 0, unused).
template <typename LPT>
__global__ __launch_bounds__(kLatPrepBlock) void k_lat_fprep(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.y;
    if (L >= w.max_lanes) return;
    const LaneCtl &c = w.ctl[L];
    const int ts = (int)blockIdx.x;
    if (!lat_final_lane(w, c) || ts > c.last_step) return;
    const FinalStep st = final_step(w, c, L, ts);
    const LpDesc d = *w.lp;
    const LPT *row = (const LPT *)d.base + (long long)c.lp_row * d.stride_b + (long long)ts * d.stride_t;
    const int4 *rec = w.lat_arc + (size_t)L * w.lat_cap;
    const float *fwd = w.lat_score + (size_t)L * w.lat_nodes;
    int4 *work = lat_work(w, L);
    constexpr uint32_t kStride = (uint32_t)kLatPrepRecs * kLatPrepBlock;
    for (uint32_t b0 = st.a0; b0 < st.a1; b0 += kStride) {
        int4 r[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            const uint32_t i = b0 + (uint32_t)k * kLatPrepBlock + threadIdx.x;
            r[k] = i < st.a1 ? rec[i] : make_int4(0, 0, 0, 1);
        }
        ArcDLW ad[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k)
            ad[k] = (r[k].w == 0 && (uint32_t)r[k].y < (uint32_t)w.num_arcs) ? w.arc_dlw[r[k].y] : ArcDLW{0, 0u, 0.0f};
        int4 o[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            o[k] = make_int4(0, -1, 0, 0);
            if (r[k].w != 0) continue;
            const bool redirect = (uint32_t)r[k].y >= (uint32_t)w.num_arcs;
            const float sa = final_arc_score(st.fin, redirect, ad[k], row);
            o[k] = make_int4(r[k].x, st.fin ? 0 : r[k].z, (int)__float_as_uint(sa),
                             (int)__float_as_uint(fwd[st.ns + (uint32_t)r[k].x]));
        }
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            const uint32_t i = b0 + (uint32_t)k * kLatPrepBlock + threadIdx.x;
            if (i < st.a1) work[i] = o[k];
        }
    }
}

// The final pass's backward sweep, one workgroup per lane (after k_lat_fprep),
// with the keep threshold final_score - output_beam: the final step's arcs set
// the scores of frame last_step (bwd(u) = the best s of u's final arcs; their
// destination, the super-final node, scores 0), then prune_sweep walks frames
// last_step - 1 .. 0; every arc kept is marked (kFinalKept). Frames go
// in windows of at most 2 * kMaxPruneInterval (the workgroup's table of step
// offsets and first nodes), each starting from the scores the window above
// left (in LDS or in memory).
__global__ __launch_bounds__(kLatSweepBlock) void k_lat_fsweep(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.x;
    if (L >= w.max_lanes) return;
    LaneCtl &c = w.ctl[L];
    if (!lat_final_lane(w, c)) return;
    __shared__ SweepShared sh;
    const size_t FF = (size_t)w.max_frames + 3;
    const uint32_t *aoff = w.lat_aoff + (size_t)L * FF;
    const uint32_t *nbase = w.lat_nbase + (size_t)L * FF;
    const SweepLane s = sweep_lane(w, L, c.final_score - w.output_beam);
    const int4 *work = lat_work(w, L);
    const uint32_t tid = threadIdx.x;
    int F = c.last_step;
    const FinalStep st = final_step(w, c, L, F);
    const uint32_t nF = nbase[F + 1] - st.ns, oF = lds_place(nF, kNoLds, 0u);
    uint32_t *bf = oF != kNoLds ? sh.bwd + oF : s.bwd + st.ns;
    for (uint32_t i = tid; i < nF; i += kLatSweepBlock) bf[i] = kOrdNegInf;
    __syncthreads();
    for (uint32_t i = st.a0 + tid; i < st.a1; i += kLatSweepBlock) {
        const int4 r = work[i];
        if (r.y == -1) continue;
        const float sa = __int_as_float(r.z), fw = __int_as_float(r.w);
        const float v = sa + 0.0f;
        if (v > -__builtin_inff()) atomicMax(&bf[(uint32_t)r.x], f2ord(v));
        if (((fw + sa) + 0.0f) >= s.thr) s.rec[i].w = kFinalKept;
    }
    uint32_t o = oF, end = st.a0;
    while (F > 0) {
        const int W = max(0, F - 2 * kMaxPruneInterval);
        __syncthreads();   // (frame F's scores; the window above no longer reads the table)
        for (int i = (int)tid; i <= F - W; i += kLatSweepBlock) {
            sh.off0[i] = aoff[W + i];
            sh.nb0[i] = nbase[W + i];
        }
        __syncthreads();
        const uint32_t n = nbase[F + 1] - nbase[F];
        int4 r[kLatBatch];
        o = prune_sweep<false, true>(w, c, s, sh, work, F, W, n, o, end, r);
        end = sh.off0[1];
        F = W;
    }
}

// The final pass's output (after k_lat_fsweep): every arc of step ts
// (blockIdx.x) of lane blockIdx.y that the sweep kept, written as k_lat_back
// writes it.
template <typename LPT>
__global__ __launch_bounds__(kLatPrepBlock) void k_lat_femit(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.y;
    if (L >= w.max_lanes) return;
    LaneCtl &c = w.ctl[L];
    const int ts = (int)blockIdx.x;
    if (!lat_final_lane(w, c) || ts > c.last_step) return;
    const FinalStep st = final_step(w, c, L, ts);
    const LpDesc d = *w.lp;
    const LPT *row = (const LPT *)d.base + (long long)c.lp_row * d.stride_b + (long long)ts * d.stride_t;
    const int4 *rec = w.lat_arc + (size_t)L * w.lat_cap;
    const int32_t *state = w.lat_state + (size_t)L * w.lat_nodes;
    constexpr uint32_t kStride = (uint32_t)kLatPrepRecs * kLatPrepBlock;
    // (the block's loop count is uniform: every wavefront takes part in each
    // lat_emit)
    for (uint32_t b0 = st.a0; b0 < st.a1; b0 += kStride) {
        int4 r[kLatPrepRecs];
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            const uint32_t i = b0 + (uint32_t)k * kLatPrepBlock + threadIdx.x;
            r[k] = i < st.a1 ? rec[i] : make_int4(0, 0, 0, -1);
        }
#pragma unroll
        for (int k = 0; k < kLatPrepRecs; ++k) {
            const bool keep = r[k].w == kFinalKept;
            int32_t o[kLatFields];
            if (keep) {
                const int32_t arc = r[k].y;
                const bool redirect = (uint32_t)arc >= (uint32_t)w.num_arcs;
                ArcDLW ad = {0, 0u, 0.0f};
                if (!redirect) ad = w.arc_dlw[arc];
                o[kLatFrame] = ts;
                o[kLatSrc] = state[st.ns + (uint32_t)r[k].x];
                o[kLatDst] = (redirect || st.fin) ? w.super_final : (int32_t)dest_state(w, ad.dest);
                o[kLatIlabel] = st.fin ? -1 : (int32_t)ad.ilabel;
                o[kLatArc] = user_arc(w, arc);
                o[kLatScore] = (int32_t)__float_as_uint(final_arc_score(st.fin, redirect, ad, row));
                o[kLatLane] = L;
                o[kLatFlags] = redirect ? 2 : (st.fin ? 1 : 0);
            }
            lat_emit(w, c, L, keep, o);
        }
    }
}

// ---------------------------------------------------------- stream sequences
// A stream (page section 8) holds one lane for its lifetime; every call is a
// short sequence of the same step kernels, framed by these three. The host
// writes one plan record per lane first (kPlan*).

// Applies the plan: parks the lanes it does not name (their state is kept),
// opens a lane (fresh start token; the start closure that follows runs for it
// alone, at t = -1 < win = 0), opens the window of an advancing lane on its next
// `len` frames (row `row` of this call's log_prob; T stays unbounded), or arms a
// lane's end (T = 0: step 0 of the sequence is its final step).
__global__ __launch_bounds__(kWave) void k_stream_begin(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)threadIdx.x;
    if (L >= w.max_lanes) return;
    const int32_t *pl = w.plan + L * kPlanFields;
    LaneCtl &c = w.ctl[L];
    c.want = 0;
    if (pl[kPlanCmd] != kCmdPark) c.last_step = -1;   // steps of this sequence not run yet
    switch (pl[kPlanCmd]) {
    case kCmdOpen:
        init_lane(w, L, 0x7FFFFFFF);
        c.dirty = 0u;     // k_clear ran first for this lane
        c.win = 0;
        c.lp_row = -1;
        break;
    case kCmdAdvance:
        c.base = c.frames;
        c.win = pl[kPlanLen];
        c.lp_row = pl[kPlanRow];
        c.want = pl[kPlanWant] ? 2 : 0;
        break;
    case kCmdFinish:
        c.base = c.frames;
        c.T = 0;
        c.win = 1;
        c.lp_row = -1;
        c.want = 1;
        break;
    default:
        c.win = -1;
        break;
    }
}

// End of a sequence: commits the last compaction of an advancing lane and moves
// its frame count past the window.
__global__ __launch_bounds__(kWave) void k_stream_end(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)threadIdx.x;
    if (L >= w.max_lanes) return;
    const int cmd = w.plan[L * kPlanFields + kPlanCmd];
    if (cmd != kCmdAdvance) return;
    LaneCtl &c = w.ctl[L];
    const int n = c.win;
    commit_log(w, c, L, n - 1, (uint32_t)c.cnt[lane_par(c, n)]);
    c.frames = c.base + n;
    // the steps this sequence ran, for the caller's records
    int32_t *R = w.res + (size_t)L * w.res_stride;
    R[6] = c.phase_final;
    R[7] = c.last_step;
}

// Before a stream's final step: its tokens hold the class of an emitting step
// (T was unbounded when they were made); one workgroup per ending lane gives
// them the final class in place — first arc, degree and bound of the final arcs,
// slot offsets by a workgroup scan in token order, strip map, slot count.
constexpr int kReclassBlock = 1024;

__global__ __launch_bounds__(kReclassBlock) void k_reclass(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.x;
    if (L >= w.max_lanes || w.plan[L * kPlanFields + kPlanCmd] != kCmdFinish) return;
    LaneCtl &c = w.ctl[L];
    if (c.status != kActive) return;
    const int par = lane_par(c, 0);
    const uint32_t n = (uint32_t)c.cnt[par];
    const uint32_t Q = w.frontier_cap;
    if (n > Q) return;   // an overflowed lane: its step retires it
    __shared__ uint32_t wtot[kReclassBlock / kWave];
    const int wid = (int)(threadIdx.x / kWave);
    uint32_t *strips = w.strip_tok[par] + (size_t)L * w.strip_cap;
    unsigned long long run = 0;
    for (uint32_t i0 = 0; i0 < n; i0 += kReclassBlock) {
        const uint32_t i = i0 + threadIdx.x;
        int32_t abeg = 0;
        uint32_t deg = 0;
        float ub = 0.0f;
        const size_t q = (size_t)L * Q + i;
        if (i < n) class_of(w.sinfo[w.tok_state[par][q]], true, w.tok_score[par][q], &abeg, &deg, &ub);
        uint32_t tot;
        const uint32_t dpre = wave_excl_sum(deg, &tot);
        if (wlane() == 0) wtot[wid] = tot;
        __syncthreads();
        unsigned long long before = 0, all = 0;
        for (int x = 0; x < kReclassBlock / kWave; ++x) {
            if (x < wid) before += wtot[x];
            all += wtot[x];
        }
        const unsigned long long off = run + before + dpre;
        if (i < n) {
            w.tok_off[par][q] = (uint32_t)off;
            w.tok_abeg[par][q] = abeg;
            w.tok_ub[par][q] = ub;
            // strips whose first slot this token holds
            for (unsigned long long sb = (off + kWave - 1) / kWave; sb * kWave < off + deg && sb < w.strip_cap; ++sb)
                strips[sb] = i;
        }
        run += all;
        __syncthreads();
    }
    // more slots than the lane's slot space: its final step retires it
    if (threadIdx.x == 0) c.cnt[par] = (unsigned long long)n | ((unsigned long long)min(run, 0xFFFFFFFFull) << 32);
}

// -------------------------------------------------------------- k_backtrack
// One wavefront per lane that wants a result: its result entry (want 1), or the
// best token of its current frontier (want 2: a stream's partial hypothesis,
// the greatest key(score, arc that gave the token its score)). Lane 0 walks the
// winners chain from there (newest arc first), then the wavefront reverses it in
// place and gathers the word ids (page sections 7 and 8).
__global__ __launch_bounds__(kWave) void k_backtrack(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.x;
    if (L >= w.max_lanes) return;
    const LaneCtl &c = w.ctl[L];
    const int want = c.want;
    if (want == 0) return;
    int32_t *R = w.res + (size_t)L * w.res_stride;
    int32_t *arcs = R + kResHeader;
    int32_t *words = arcs + w.path_cap;
    const int lane = wlane();
    uint32_t len = 0;
    uint32_t ovf = c.overflow;
    int32_t start = c.final_entry;
    float score = c.final_score;
    int32_t reached = c.reached_final;
    bool has_path = lane_has_result(c);
    if (want == 2) {
        start = -1;
        score = -__builtin_inff();
        reached = 0;
        const int par = lane_par(c, c.win);
        const uint32_t n = (uint32_t)c.cnt[par];
        unsigned long long bk = 0ull;
        int32_t be = -1;
        float bs = 0.0f;
        if (c.status == kActive && n <= w.frontier_cap) {
            const size_t qo = (size_t)L * w.frontier_cap;
            for (uint32_t i = (uint32_t)lane; i < n; i += kWave) {
                const unsigned long long k = cand_key(w.tok_score[par][qo + i], w.tok_last[par][qo + i]);
                if (k > bk) { bk = k; be = w.tok_entry[par][qo + i]; bs = w.tok_score[par][qo + i]; }
            }
        }
        unsigned long long m = bk;
#pragma unroll
        for (int dd = kWave / 2; dd >= 1; dd >>= 1) {
            const unsigned long long o = __shfl_xor(m, dd, kWave);
            m = o > m ? o : m;
        }
        const unsigned long long who = __ballot(bk == m && m != 0ull);
        has_path = who != 0ull;
        if (has_path) {
            const int src = __ffsll((long long)who) - 1;
            start = __shfl(be, src, kWave);
            score = __shfl(bs, src, kWave);
        }
    }
    // The walk goes back entry by entry (newest arc first) until it reaches the
    // lane's sealed prefix: compaction keeps there the path every live token
    // shares, one chain in log order (each entry's predecessor is the one
    // before it, the first one's the start token), so the path ends with
    // entries tail - 1, ..., 0, read in one sweep.
    uint32_t tail = 0;
    if (lane == 0 && has_path) {
        const long long limit = (long long)w.max_lanes * w.arena;
        const long long lbase = (long long)L * w.arena, sb = lbase + c.sealed;
        int32_t e = start;   // -1: the start token (empty path)
        while (e >= 0 && e < limit) {
            if (e < sb) { tail = (uint32_t)(e - lbase) + 1u; break; }
            const int2 r = w.wlog[e];
            if (len < w.path_cap) arcs[len] = r.y;
            ++len;
            e = r.x;
            if (len > (uint32_t)w.arena) break;
        }
    }
    len = __shfl(len, 0, kWave);
    tail = __shfl(tail, 0, kWave);
    for (uint32_t x = (uint32_t)lane; x < tail && len + x < w.path_cap; x += kWave)
        arcs[len + x] = w.wlog[(long long)L * w.arena + (tail - 1u - x)].y;
    len += tail;
    if (len > w.path_cap) ovf |= kOvfPath;
    ovf = __shfl(ovf, 0, kWave);
    const uint32_t ns = min(len, w.path_cap);
    __syncthreads();
    for (uint32_t i = (uint32_t)lane; i < ns / 2; i += kWave) {
        const int32_t a = arcs[i], b = arcs[ns - 1 - i];
        arcs[i] = b;
        arcs[ns - 1 - i] = a;
    }
    __syncthreads();
    uint32_t nw = 0;
    for (uint32_t i0 = 0; i0 < ns; i0 += kWave) {
        const uint32_t i = i0 + (uint32_t)lane;
        int32_t ol = 0;
        if (i < ns) {
            ol = w.olabel[arcs[i]];
            arcs[i] = user_arc(w, arcs[i]);   // (the graph's arc ids in the result)
        }
        const unsigned long long m = __ballot(ol != 0);
        if (ol != 0) words[nw + (uint32_t)__popcll(m & mask_lt())] = ol;
        nw += (uint32_t)__popcll(m);
    }
    if (lane == 0) {
        R[kResOk] = ovf == 0u ? 1 : 0;
        R[kResReached] = reached;
        R[kResOverflow] = (int32_t)ovf;
        R[kResArcLen] = (int32_t)len;
        R[kResWordLen] = (int32_t)nw;
        R[kResScore] = (int32_t)__float_as_uint(has_path ? score : -__builtin_inff());
        R[6] = c.phase_final;
        R[7] = c.last_step;
    }
}

// ------------------------------------------------------ winners-log compaction
// A compaction round (page section 8.1 and the page's winners-log GC: memory
// bounded, results bit-identical) keeps only the winners-log entries a live
// token still reaches, renumbered in log order, and extends the lane's sealed
// prefix: the path every live token shares, which later rounds neither walk nor
// move. Entries hold global ids (lane * arena + local) or -1. A round's window
// is [sealed, log_cursor) in local ids; bit j of the live map is local entry
// sealed + j; a live entry's compacted position is the count of live bits before
// it. Kernels, in order: begin, mark, scan, compact, commit, roots, clear, end.

// Whether lane c's round runs: it ran a real step in this sequence and is
// active (lattice nodes are frame positions, never log entries, so lattices
// do not hold the log back).
__device__ __forceinline__ bool gc_due(const LaneCtl &c)
{
    return c.status == kActive && c.last_step >= 0 && c.last_step < c.T;
}

// Round set-up, one thread per lane: the compaction of the lane's last step is
// committed (its entries are the roots' own), counters reset.
__global__ __launch_bounds__(kWave) void k_gc_begin(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)threadIdx.x;
    if (L >= w.max_lanes) return;
    LaneCtl &c = w.ctl[L];
    const bool on = gc_due(c);
    c.gc_on = on ? 1u : 0u;
    if (!on) return;
    const int p = lane_par(c, c.last_step + 1);
    commit_log(w, c, L, c.last_step, (uint32_t)pair_at(c.cnt, p));
    c.gc_base_children = 0u;
    c.gc_k = 0xFFFFFFFFu;
    c.gc_live = 0u;
}

// Per-lane table of a round: units of `what` (0: the frontier's tokens, 1: the
// window's entries, 2: the live entries, 3: the window's 32-entry words), the
// frontier parity, the window [sealed, cursor).
__device__ __forceinline__ void gc_prologue(const Work &w, LaneTab &tab, int what)
{
    if (threadIdx.x < kWave) {
        const int L = (int)threadIdx.x;
        uint32_t units = 0;
        if (L < w.max_lanes) {
            const LaneCtl &c = w.ctl[L];
            const int p = lane_par(c, c.last_step + 1);
            const uint32_t n = (uint32_t)pair_at(c.cnt, p);
            const uint32_t win = c.log_cursor > c.sealed ? c.log_cursor - c.sealed : 0u;
            uint32_t items = 0;
            if (c.gc_on && n <= w.frontier_cap && c.log_cursor <= w.arena_lim)
                items = what == 0 ? n : what == 1 ? win : what == 2 ? c.gc_live : max((win + 31u) / 32u, c.gc_live);
            units = (items + kWave - 1) / kWave;
            tab.n[L] = items;
            tab.win[L] = (int32_t)c.gc_live;
            tab.arcs[L] = c.sealed;
            tab.par[L] = p;
            tab.fb[L] = c.log_cursor;
            tab.row[L] = (int32_t)pair_at(c.front_base, p);
        }
        tab_publish(tab, w.max_lanes, units);
    }
    __syncthreads();
}

__device__ __forceinline__ size_t gc_words(const Work &w) { return (size_t)w.arena / 32 + 1; }

// Compacted position of live window entry j.
__device__ __forceinline__ uint32_t gc_pos(const uint32_t *mark, const uint32_t *wpre, uint32_t j)
{
    return wpre[j >> 5] + (uint32_t)__popc(mark[j >> 5] & ((1u << (j & 31u)) - 1u));
}

// Marking: every frontier token marks its own entry, then walks its chain back
// through the window, setting live bits, and stops at the first entry already
// marked (or sealed, or -1). Without epsilon arcs the frontier's entries are its
// compaction's base plus the token's position, so a wavefront's 64 consecutive
// tokens set their bits with one atomic per 32-entry word; every walk step
// issues its predecessor load beside its atomic.
__global__ __launch_bounds__(kBlock) void k_gc_mark(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    gc_prologue(w, tab, 0);
    const int nl = w.max_lanes;
    const int lane = wlane();
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const int p = upar(tab.par, L);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)lane;
        const bool valid = i < tab.n[L];
        const uint32_t sealed = tab.arcs[L], cursor = tab.fb[L];
        uint32_t *mark = w.gc_mark + (size_t)L * gc_words(w);
        const long long lbase = (long long)L * w.arena;
        const uint32_t fb = (uint32_t)tab.row[L];
        long long e = -1;                           // the token's own entry (local), -1: none
        if (!w.has_eps) {
            if (valid && fb != 0xFFFFFFFFu) e = (long long)fb + i;   // (the start token has no entry)
        } else if (valid) {
            const int32_t ge = pick(w.tok_entry, p)[(size_t)L * w.frontier_cap + i];
            e = ge < 0 ? -1 : (long long)ge - lbase;
        }
        const bool own = e >= (long long)sealed && e < (long long)cursor;
        const uint32_t j0 = own ? (uint32_t)(e - sealed) : 0u;
        int32_t prev = own ? w.wlog[lbase + e].x : -1;
        if (!w.has_eps) {
            // consecutive tokens own consecutive entries: each word's bits form one
            // run over a run of lanes
            const unsigned long long om = __ballot(own);
            if (om) {
                const uint32_t wfirst = __shfl(j0 >> 5, __ffsll((long long)om) - 1, kWave);
#pragma unroll
                for (uint32_t q = 0; q < 3u; ++q) {
                    const unsigned long long bm = __ballot(own && (j0 >> 5) == wfirst + q);
                    if (!bm) continue;
                    const int la = __ffsll((long long)bm) - 1, lb = 63 - __clzll((long long)bm);
                    const uint32_t ba = __shfl(j0 & 31u, la, kWave), bb = __shfl(j0 & 31u, lb, kWave);
                    if (lane == la) atomicOr(&mark[wfirst + q], ((2u << bb) - 1u) & ~((1u << ba) - 1u));
                }
            }
        } else if (own) {
            atomicOr(&mark[j0 >> 5], 1u << (j0 & 31u));
        }
        if (!own) continue;
        e = prev < 0 ? -1 : (long long)prev - lbase;
        while (e >= (long long)sealed && e < (long long)cursor) {
            const uint32_t j = (uint32_t)(e - sealed), bit = 1u << (j & 31u);
            prev = w.wlog[lbase + e].x;
            if (atomicOr(&mark[j >> 5], bit) & bit) break;
            e = prev < 0 ? -1 : (long long)prev - lbase;
        }
    }
}

// Prefix counts of live entries by 32-entry word, one workgroup per lane.
constexpr int kGcScanBlock = 1024;

__global__ __launch_bounds__(kGcScanBlock) void k_gc_scan(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)blockIdx.x;
    if (L >= w.max_lanes) return;
    LaneCtl &c = w.ctl[L];
    const int p = lane_par(c, c.last_step + 1);
    if (!c.gc_on || c.log_cursor > w.arena_lim || (uint32_t)pair_at(c.cnt, p) > w.frontier_cap) return;
    const uint32_t win = c.log_cursor > c.sealed ? c.log_cursor - c.sealed : 0u;
    const uint32_t nw = (win + 31u) / 32u;
    const uint32_t *mark = w.gc_mark + (size_t)L * gc_words(w);
    uint32_t *wpre = w.gc_wpre + (size_t)L * gc_words(w);
    __shared__ uint32_t wtot[kGcScanBlock / kWave];
    const int wid = (int)(threadIdx.x / kWave);
    uint32_t run = 0;
    for (uint32_t x0 = 0; x0 < nw; x0 += kGcScanBlock) {
        const uint32_t x = x0 + threadIdx.x;
        const uint32_t cnt = x < nw ? (uint32_t)__popc(mark[x]) : 0u;
        uint32_t tot;
        const uint32_t pre = wave_excl_sum(cnt, &tot);
        if (wlane() == 0) wtot[wid] = tot;
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (int k = 0; k < kGcScanBlock / kWave; ++k) {
            if (k < wid) before += wtot[k];
            all += wtot[k];
        }
        if (x < nw) wpre[x] = run + before + pre;
        run += all;
        __syncthreads();
    }
    if (threadIdx.x == 0) c.gc_live = run;
}

// Compaction into the lane's buffer: each live window entry at its position,
// its predecessor renumbered; live-children counts by position (children of the
// sealed prefix's last entry, or of the start token, counted apart).
__global__ __launch_bounds__(kBlock) void k_gc_compact(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    gc_prologue(w, tab, 1);
    const int nl = w.max_lanes;
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t j = (u - tab.base[L]) * kWave + (uint32_t)wlane();
        if (j >= tab.n[L]) continue;
        const uint32_t *mark = w.gc_mark + (size_t)L * gc_words(w);
        if (!((mark[j >> 5] >> (j & 31u)) & 1u)) continue;
        const uint32_t *wpre = w.gc_wpre + (size_t)L * gc_words(w);
        const uint32_t sealed = tab.arcs[L];
        const long long lbase = (long long)L * w.arena;
        const int2 r = w.wlog[lbase + sealed + j];
        int32_t np = r.x;
        const long long pe = r.x < 0 ? -1 : (long long)r.x - lbase;
        if (pe >= (long long)sealed) {
            const uint32_t pp = gc_pos(mark, wpre, (uint32_t)(pe - sealed));
            np = (int32_t)(lbase + sealed + pp);
            atomicAdd(&w.gc_child[(size_t)L * w.arena + pp], 1u);
        } else {
            atomicAdd(&w.ctl[L].gc_base_children, 1u);
        }
        w.gc_buf[(size_t)L * w.arena + gc_pos(mark, wpre, j)] = make_int2(np, r.y);
    }
}

// The buffer back into the log; a position without exactly one live child ends
// the shared path (one atomic per 64 positions: the first such one).
__global__ __launch_bounds__(kBlock) void k_gc_commit(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    gc_prologue(w, tab, 2);
    const int nl = w.max_lanes;
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)wlane();
        const bool valid = i < tab.n[L];
        bool ends = false;
        if (valid) {
            const size_t q = (size_t)L * w.arena + i;
            w.wlog[(long long)L * w.arena + tab.arcs[L] + i] = w.gc_buf[q];
            ends = w.gc_child[q] != 1u;
        }
        const unsigned long long m = __ballot(ends);
        if (m && wlane() == __ffsll((long long)m) - 1) atomicMin(&w.ctl[L].gc_k, i);
    }
}

// The frontier's entries renumbered (an epsilon-free frontier's base too). Every
// frontier token's entry lies at or after its compaction's base, so the base's
// position bounds the shared path.
__global__ __launch_bounds__(kBlock) void k_gc_roots(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    gc_prologue(w, tab, 0);
    const int nl = w.max_lanes;
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const int p = upar(tab.par, L);
        const uint32_t i = (u - tab.base[L]) * kWave + (uint32_t)wlane();
        if (i >= tab.n[L]) continue;
        const uint32_t sealed = tab.arcs[L], cursor = tab.fb[L];
        const uint32_t *mark = w.gc_mark + (size_t)L * gc_words(w);
        const uint32_t *wpre = w.gc_wpre + (size_t)L * gc_words(w);
        const long long lbase = (long long)L * w.arena;
        LaneCtl &c = w.ctl[L];
        int32_t *te = pick(w.tok_entry, p) + (size_t)L * w.frontier_cap + i;
        const int32_t ge = *te;
        if (ge >= 0) {
            const long long e = (long long)ge - lbase;
            if (e >= (long long)sealed && e < (long long)cursor)
                *te = (int32_t)(lbase + sealed + gc_pos(mark, wpre, (uint32_t)(e - sealed)));
        }
        if (i == 0) {
            const uint32_t fb = c.front_base[p];
            if (fb != 0xFFFFFFFFu && fb >= sealed && fb < cursor) {
                // live entries before the base (the base itself may be dead on an
                // epsilon lane whose first token was replaced)
                const uint32_t pos = gc_pos(mark, wpre, fb - sealed);
                atomicMin(&c.gc_k, pos);
                // the epsilon-free frontier's entries are its base plus the token's
                // position: the base moves with token 0's entry
                if (!w.has_eps) c.front_base[p] = sealed + pos;
            }
        }
    }
}

// Clears the round's live map (the window's words) and child counts (set only
// at the live entries' compacted positions), each with one coalesced store per
// item.
__global__ __launch_bounds__(kBlock) void k_gc_clear(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    __shared__ LaneTab tab;
    gc_prologue(w, tab, 3);
    const int nl = w.max_lanes;
    uint32_t u_beg, u_end;
    wave_share(tab.base[nl], &u_beg, &u_end);
    for (uint32_t u = u_beg; u < u_end; ++u) {
        const int L = find_lane(tab.base, nl, u);
        const uint32_t x = (u - tab.base[L]) * kWave + (uint32_t)wlane();
        if (x >= tab.n[L]) continue;
        const uint32_t win = tab.fb[L] > tab.arcs[L] ? tab.fb[L] - tab.arcs[L] : 0u;
        if (x < (win + 31u) / 32u) w.gc_mark[(size_t)L * gc_words(w) + x] = 0u;
        if (x < (uint32_t)tab.win[L] && x < w.arena) w.gc_child[(size_t)L * w.arena + x] = 0u;
    }
}

// End of a round, one thread per lane: the log ends after the live entries, and
// the sealed prefix grows by the shared path (positions 0 .. k of the window,
// when exactly one live entry hangs off the old prefix).
__global__ __launch_bounds__(kWave) void k_gc_end(const Work *__restrict__ wp)
{
    const Work &w = *wp;
    const int L = (int)threadIdx.x;
    if (L >= w.max_lanes) return;
    LaneCtl &c = w.ctl[L];
    const int p = lane_par(c, c.last_step + 1);
    if (!c.gc_on || c.log_cursor > w.arena_lim || (uint32_t)pair_at(c.cnt, p) > w.frontier_cap) return;
    const uint32_t live = c.gc_live;
    uint32_t grow = 0;
    if (c.gc_base_children == 1u && live > 0u) grow = min(c.gc_k, live - 1u) + 1u;
    c.log_cursor = c.sealed + live;
    c.sealed += grow;
    c.gc_on = 0u;
}

// -------------------------------------------------------- blank-skip slicing
// Frame pre-slicing before a decode (page section 3: the search itself never
// skips frames; the caller slices them first, as WeNet does): a frame t < length is dropped iff its blank
// log-prob exceeds lthr = log(threshold); the kept frames keep their order.

// One workgroup per lane: keep flags, a workgroup scan in frame order, the
// source frame of every kept row and the kept count.
constexpr int kSkipBlock = 1024;

template <typename LPT>
__global__ __launch_bounds__(kSkipBlock) void k_blank_scan(const Work *__restrict__ wp, float lthr, int blank, int T)
{
    const Work &w = *wp;
    const LpDesc d = *w.lp;
    const int b = (int)blockIdx.x;
    if (b >= d.B) return;
    const int len = w.lengths[b];
    __shared__ uint32_t wtot[kSkipBlock / kWave];
    const int wid = (int)(threadIdx.x / kWave);
    int32_t *src = w.bs_src + (size_t)b * w.max_frames;
    uint32_t run = 0;
    for (int t0 = 0; t0 < T; t0 += kSkipBlock) {
        const int t = t0 + (int)threadIdx.x;
        bool keep = false;
        if (t < len) {
            const LPT *row = (const LPT *)d.base + (long long)b * d.stride_b + (long long)t * d.stride_t;
            keep = !(lp_at(row, (uint32_t)blank) > lthr);
        }
        const unsigned long long m = __ballot(keep);
        if (wlane() == 0) wtot[wid] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (int x = 0; x < kSkipBlock / kWave; ++x) {
            if (x < wid) before += wtot[x];
            all += wtot[x];
        }
        if (keep) src[run + before + (uint32_t)__popcll(m & mask_lt())] = t;
        run += all;
        __syncthreads();
    }
    if (threadIdx.x == 0) w.bs_len[b] = (int32_t)run;
}

// One wavefront per output row: the kept row's copy, or zeros past the count;
// 16-byte accesses when every row of both tensors starts 16-byte aligned.
template <typename LPT>
__global__ __launch_bounds__(kBlock) void k_blank_copy(const Work *__restrict__ wp, LPT *__restrict__ out, int T)
{
    const Work &w = *wp;
    const LpDesc d = *w.lp;
    const int wpb = kBlock / kWave;
    const long long rows = (long long)d.B * T;
    constexpr uint32_t kPer = 16 / sizeof(LPT);
    const bool vec = ((uintptr_t)d.base & 15u) == 0 && ((uintptr_t)out & 15u) == 0 && d.stride_t % kPer == 0 &&
                     d.stride_b % kPer == 0;
    const uint32_t V = (uint32_t)w.vocab, nvec = vec ? V / kPer : 0u;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (long long r = (long long)blockIdx.x * wpb + threadIdx.x / kWave; r < rows; r += (long long)gridDim.x * wpb) {
        const int b = (int)(r / T), i = (int)(r % T);
        LPT *o = out + (long long)b * d.stride_b + (long long)i * d.stride_t;
        uint4 *o4 = (uint4 *)o;
        if (i < w.bs_len[b]) {
            const LPT *row = (const LPT *)d.base + (long long)b * d.stride_b +
                             (long long)w.bs_src[(size_t)b * w.max_frames + i] * d.stride_t;
            const uint4 *r4 = (const uint4 *)row;
            // four loads in flight per lane before their stores
            uint32_t k = wlane();
            for (; k + 3u * kWave < nvec; k += 4u * kWave) {
                const uint4 a0 = r4[k], a1 = r4[k + kWave], a2 = r4[k + 2u * kWave], a3 = r4[k + 3u * kWave];
                o4[k] = a0; o4[k + kWave] = a1; o4[k + 2u * kWave] = a2; o4[k + 3u * kWave] = a3;
            }
            for (; k < nvec; k += kWave) o4[k] = r4[k];
            for (uint32_t v = nvec * kPer + wlane(); v < V; v += kWave) o[v] = row[v];
        } else {
            for (uint32_t k = wlane(); k < nvec; k += kWave) o4[k] = z4;
            for (uint32_t v = nvec * kPer + wlane(); v < V; v += kWave) o[v] = (LPT)0.0f;
        }
    }
}

hipError_t launch_blank_skip(const Work &w, const Work *dw, void *out, float lthr, int blank, int B, int T,
                             int grid, hipStream_t s)
{
    if (w.lp_dtype == 1) {
        hipLaunchKernelGGL(k_blank_scan<__half>, dim3(B), dim3(kSkipBlock), 0, s, dw, lthr, blank, T);
        hipLaunchKernelGGL(k_blank_copy<__half>, dim3(grid), dim3(kBlock), 0, s, dw, (__half *)out, T);
    } else {
        hipLaunchKernelGGL(k_blank_scan<float>, dim3(B), dim3(kSkipBlock), 0, s, dw, lthr, blank, T);
        hipLaunchKernelGGL(k_blank_copy<float>, dim3(grid), dim3(kBlock), 0, s, dw, (float *)out, T);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

// Plain launch, or with timing events recorded by the dispatch itself (start and
// end of the kernel's execution) when e0 is given.
template <typename... A>
static void go(void (*kern)(A...), dim3 g, dim3 b, hipStream_t s, hipEvent_t e0, hipEvent_t e1, A... args)
{
    if (e0) hipExtLaunchKernelGGL(kern, g, b, 0, s, e0, e1, 0, args...);
    else hipLaunchKernelGGL(kern, g, b, 0, s, args...);
}

hipError_t launch_kernel(int id, const Work &w, const Work *dw, int t, int k, int grid, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1)
{
    const bool f16 = w.lp_dtype == 1;
    const bool hash = w.hash_bits != 0;
    const dim3 G(grid), B(kBlock);
    switch (id) {
    case kKClear: go(k_clear, G, B, s, e0, e1, dw, k); break;
    case kKInit: go(k_init, dim3(1), dim3(kWave), s, e0, e1, dw); break;
    case kKLpmax:
        if (f16) go(k_lpmax<__half>, G, B, s, e0, e1, dw);
        else go(k_lpmax<float>, G, B, s, e0, e1, dw);
        break;
    case kKMax: {
        const dim3 GW(w.walk_grid > 0 ? w.walk_grid : grid);
        if (hash) {
            if (f16) go(k_max<__half, true>, GW, B, s, e0, e1, dw, t);
            else go(k_max<float, true>, GW, B, s, e0, e1, dw, t);
        } else {
            if (f16) go(k_max<__half, false>, GW, B, s, e0, e1, dw, t);
            else go(k_max<float, false>, GW, B, s, e0, e1, dw, t);
        }
        break;
    }
    case kKFinalize:
        if (hash) go(k_finalize<true>, G, B, s, e0, e1, dw, t);
        else go(k_finalize<false>, G, B, s, e0, e1, dw, t);
        break;
    case kKEpsExpand:
        if (hash) go(k_eps_expand<true>, G, B, s, e0, e1, dw, t, k);
        else go(k_eps_expand<false>, G, B, s, e0, e1, dw, t, k);
        break;
    case kKEpsApply:
        if (hash) go(k_eps_apply<true>, G, B, s, e0, e1, dw, t, k);
        else go(k_eps_apply<false>, G, B, s, e0, e1, dw, t, k);
        break;
    case kKEpsApplyExpand:
        if (k < 1 || k >= w.eps_iterations || w.ntab != 2) return hipErrorInvalidValue;
        if (hash) go(k_eps_apply_expand<true>, G, B, s, e0, e1, dw, t, k);
        else go(k_eps_apply_expand<false>, G, B, s, e0, e1, dw, t, k);
        break;
    case kKBacktrack: go(k_backtrack, dim3(w.max_lanes), dim3(kWave), s, e0, e1, dw); break;
    case kKStreamBegin: go(k_stream_begin, dim3(1), dim3(kWave), s, e0, e1, dw); break;
    case kKStreamEnd: go(k_stream_end, dim3(1), dim3(kWave), s, e0, e1, dw); break;
    case kKReclass: go(k_reclass, dim3(w.max_lanes), dim3(kReclassBlock), s, e0, e1, dw); break;
    case kKLatInit: go(k_lat_init, G, B, s, e0, e1, dw); break;
    case kKLatBack:
        if (f16) go(k_lat_back<__half>, G, B, s, e0, e1, dw, t);
        else go(k_lat_back<float>, G, B, s, e0, e1, dw, t);
        break;
    case kKLatEpsRound: go(k_lat_eps_round, G, B, s, e0, e1, dw, t, k); break;
    case kKLatEpsBack:
        go(k_lat_eps_back, dim3(w.max_lanes + kLatKeepBlocks), dim3(kLatSweepBlock), s, e0, e1, dw, t);
        break;
    case kKGcBegin: go(k_gc_begin, dim3(1), dim3(kWave), s, e0, e1, dw); break;
    case kKGcMark: go(k_gc_mark, G, B, s, e0, e1, dw); break;
    case kKGcScan: go(k_gc_scan, dim3(w.max_lanes), dim3(kGcScanBlock), s, e0, e1, dw); break;
    case kKGcCompact: go(k_gc_compact, G, B, s, e0, e1, dw); break;
    case kKGcCommit: go(k_gc_commit, G, B, s, e0, e1, dw); break;
    case kKGcRoots: go(k_gc_roots, G, B, s, e0, e1, dw); break;
    case kKGcClear: go(k_gc_clear, G, B, s, e0, e1, dw); break;
    case kKGcEnd: go(k_gc_end, dim3(1), dim3(kWave), s, e0, e1, dw); break;
    case kKLatPrep:
        if (w.lat_prune_interval < 1 || w.lat_prune_interval > kMaxPruneInterval) return hipErrorInvalidValue;
        if (f16) go(k_lat_prep<__half>, dim3(2 * w.lat_prune_interval, w.max_lanes), dim3(kLatPrepBlock), s, e0, e1, dw, t);
        else go(k_lat_prep<float>, dim3(2 * w.lat_prune_interval, w.max_lanes), dim3(kLatPrepBlock), s, e0, e1, dw, t);
        break;
    case kKLatPrune:
        if (w.lat_prune_interval < 1 || w.lat_prune_interval > kMaxPruneInterval) return hipErrorInvalidValue;
        go(k_lat_prune, dim3(w.max_lanes), dim3(kLatSweepBlock), s, e0, e1, dw, t);
        break;
    case kKLatFPrep:   // t: the decode's steps
        if (t < 1 || t > w.max_frames + 1) return hipErrorInvalidValue;
        if (f16) go(k_lat_fprep<__half>, dim3(t, w.max_lanes), dim3(kLatPrepBlock), s, e0, e1, dw);
        else go(k_lat_fprep<float>, dim3(t, w.max_lanes), dim3(kLatPrepBlock), s, e0, e1, dw);
        break;
    case kKLatSweep: go(k_lat_fsweep, dim3(w.max_lanes), dim3(kLatSweepBlock), s, e0, e1, dw); break;
    case kKLatEmit:
        if (t < 1 || t > w.max_frames + 1) return hipErrorInvalidValue;
        if (f16) go(k_lat_femit<__half>, dim3(t, w.max_lanes), dim3(kLatPrepBlock), s, e0, e1, dw);
        else go(k_lat_femit<float>, dim3(t, w.max_lanes), dim3(kLatPrepBlock), s, e0, e1, dw);
        break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace wfst
