// Internal layout shared by the host orchestration (wfst_api.cpp) and the
// gfx950 kernels (wfst_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace wfst {

constexpr int kWave = 64;           // CDNA wavefront width
constexpr int kBlock = 256;         // threads per workgroup of the frame-loop kernels
constexpr int kMaxLanes = 64;       // one wavefront scans the per-lane table
constexpr int kStepFields = 16;     // u32 fields of one per-step record
constexpr uint32_t kMaxEpochArcBits = 25;  // epoch-tagged table keys need arc ids below 2^25
constexpr uint16_t kFinalLabel = 0xFFFF;

// Lane status.
enum : int32_t { kActive = 0, kDone = 1 };

// Step phase of a lane.
enum : int32_t { kPhNone = -1, kPhReal = 0, kPhFinal = 1, kPhRedirect = 2, kPhDead = 3 };

// Overflow bits (same values as the public WFST_OVF_*).
enum : uint32_t {
    kOvfSlots = 1, kOvfHash = 2, kOvfArena = 4, kOvfClaims = 8, kOvfFrontier = 16, kOvfPath = 32
};

// Per-step record fields (u32).
enum : int {
    kRecN = 0, kRecBeam, kRecMax, kRecArcs, kRecAdmitted, kRecDistinct, kRecEpsArcs,
    kRecEpsAdmitted, kRecEpsDistinct, kRecEpsNew, kRecEpsReplaced, kRecEpsPasses, kRecPhase,
    kRecListed    // candidates the slot pass listed (its superset of the admitted ones)
};

// Emitting arcs per state whose (label, weight) the state's record keeps for
// the lower bound of the next step's maximum and the exact bound of the skip.
// A random read of a state record costs one 128-byte line whatever its size,
// so the record fills the line; 15 of the 18 that would fit measured best
// (each is one more log-prob gather per new token).
constexpr int kTopArcs = 15;

// Per-state arc ranges and weights, one 128-byte record per state: arcs
// [eps_b, emit_b) are epsilon, [emit_b, fin_b) emitting, [fin_b, end) final.
// top_w / top_il are the kTopArcs largest-weight emitting arcs, by weight
// descending (top_w[0] is the largest emitting weight, -inf if none); unused
// entries have weight -inf and label 0.
struct alignas(128) StateInfo {
    int32_t eps_b, emit_b, fin_b, end;
    float fin_maxw;              // largest weight over the final arcs (-inf if none)
    float top_w[kTopArcs];
    uint16_t top_il[kTopArcs];
};
static_assert(sizeof(StateInfo) == 128, "one state record is one 128-byte line");

// Arc records {dest, ilabel, weight}, one contiguous run per state (the CSR
// order of the graph), so the fields a pass reads for a token's arcs share
// cache lines; each state's run starts after up to 31 padding records, placed
// so that its emitting arcs span the fewest 128-byte lines. On the device an
// arc is named by its record's position, which grows with the graph's arc id
// (a tie between arcs resolves the same on either); results and lattice
// records carry the graph's ids (Work::arc_uid). Final arcs carry kFinalLabel.
// When the graph stores ranks, dest
// holds the arc's rank among its destination's incoming non-final arcs (in arc
// id order) above the state id's bits (Work::dest_bits).
struct ArcDLW {
    int32_t dest;
    uint32_t ilabel;
    float weight;
};

// An admitted candidate: destination (the arc record's field: the state id,
// with the arc's rank above it when the graph stores ranks), arc, source (the
// source token's position in the frontier being read; for a closure candidate,
// the source token's winners-log entry) and end score. Its key (score, then arc
// id or rank) is unique per destination, so exactly one candidate of each
// destination finds its own key in the table once the pass is over: the winner.
struct alignas(16) Claim {
    int32_t dest;
    int32_t arc;
    uint32_t tok;
    uint32_t score;   // binary32 bits of the end score
};

// A slot of the per-lane open-addressing recombination hash (the alternative to
// the direct-mapped table): claim = epoch << 32 | destination state (a slot of
// an earlier round counts as empty), key = the table key of its best candidate.
struct alignas(16) HSlot {
    unsigned long long claim;
    unsigned long long key;
};

// Per-lane control block. Device-scope atomics on one 128-byte line serialize
// even on different words, so every counter that many wavefronts of one kernel
// update atomically has a line of its own; the first line holds the fields the
// kernels only read, or that one thread writes.
struct alignas(128) LaneCtl {
    int32_t T;                 // frames of this lane
    int32_t status;            // kActive / kDone
    uint32_t overflow;         // kOvf* bits
    int32_t reached_final;
    float beam[2];             // b_t by step parity (beam[1] = search beam before step 0)
    uint32_t front_base[2];    // winners-log base of the compaction that built the frontier of each
                               //   parity (0xFFFFFFFF: the start frontier, whose token has entry -1)
    unsigned long long final_key;  // best final candidate key of the final step
    float cutoff;              // cutoff of the latest real step (closure passes use it)
    int32_t final_entry;       // winners-log entry of the result (-1 none)
    float final_score;
    uint32_t dirty;            // recombination table may hold stale entries (claims overflow)
    int32_t last_step;         // last step this lane ran
    int32_t phase_final;       // phase code of the lane's last step
    uint32_t log_open;         // 1: the last compaction's entries (its token count) are not yet
                               //   in log_cursor; the next kernel that reads the log adds them
    // Steps of one launch sequence (a decode, a stream's chunk or its end) are
    // numbered t = 0, 1, ... in every lane; a lane's own step is base + t, and the
    // frontier feeding it has parity (base + t) & 1.
    int32_t base;              // the lane's steps before this sequence (0 for a decode)
    int32_t win;               // the lane runs steps t < win of this sequence (-1: parked)
    int32_t lp_row;            // batch row of the lane's frames in this sequence's log_prob (-1 none)
    int32_t frames;            // a stream's frames so far
    int32_t want;              // result wanted after the sequence: 0 none, 1 the lane's result,
                               //   2 the partial hypothesis (best current token)
    // winners-log compaction: entries [0, sealed) of the lane's region are the
    // path every live token shares (never moved again); a round compacts the
    // live entries of [sealed, log_cursor)
    uint32_t sealed;
    uint32_t gc_on;            // this round compacts the lane
    uint32_t gc_live;          // live entries of the window (after the scan)
    uint32_t log_full;         // 1: the winners log's committed bound stopped the lane
    alignas(128) unsigned long long cnt[2];  // frontier counter by parity: tokens | (arcs of the
                                             //   step's class) << 32
    alignas(128) uint32_t nclaims[2];        // candidate-list length of the slot pass by step parity
    alignas(128) uint32_t maxkey[2];         // ordered exact maximum M_t by step parity (slot pass)
    uint32_t lbkey[2];                       // ordered lower bound of M_t by step parity: the best
                                             //   candidate through each token's largest-weight arcs
                                             //   (posted by the compaction of the step before)
    alignas(128) uint32_t log_cursor;        // winners-log entries used in this lane's region
    alignas(128) uint32_t nclaims_eps[3];    // listed candidates of closure pass k at [k % 3] (three,
                                             //   so a kernel that reads pass k's and appends pass
                                             //   k + 1's can clear pass k + 2's)
    alignas(128) unsigned long long nchanged[2];  // closure pass k's sources at [k & 1]: entries of
                                                  //   its list (low half) | tokens appended or replaced
                                                  //   by the pass before it (high half; pass 1: unused)
    alignas(128) uint32_t lat_cursor;        // lattice arcs persisted (lattice mode)
    alignas(128) uint32_t lat_out_n;         // lattice records kept by the prune (lattice mode)
    alignas(128) uint32_t gc_base_children;  // live window entries whose predecessor is sealed
    uint32_t gc_k;                           // first window position that ends the shared path
};

// Device-resident description of the caller's log_prob tensor, rewritten before
// every decode so that a captured graph stays valid across decodes.
struct LpDesc {
    const void *base;
    long long stride_b;   // elements between lanes
    long long stride_t;   // elements between frames
    int32_t B;
    int32_t dtype;        // 0 f32, 1 f16
};

// Everything a kernel needs, passed by value.
struct Work {
    // graph (read-only)
    const StateInfo *sinfo;
    const ArcDLW *arc_dlw;
    const int32_t *olabel;        // by record position
    const int32_t *arc_uid;       // record position -> the graph's arc id (-1: padding)
    int32_t num_states, num_arcs, start_state, vocab, super_final;   // num_arcs: records, padding included
    int32_t num_arcs_user;        // the graph's arcs
    int32_t has_eps;
    int32_t epochs;           // table keys carry the round's epoch: entries are never cleared singly
    uint32_t tie_bits;        // tie bits of an epoch-tagged key (the epoch takes 32 - tie_bits)
    uint32_t rank_ties;       // ties by the arc's rank among its destination's incoming arcs (else arc id)
    uint32_t dest_bits;       // state id bits of a destination field holding a rank above them (0: none)
    uint32_t dest_mask;       // state id of a destination field: field & dest_mask
    uint32_t epoch_period;    // rounds between full clears of the table
    uint32_t round_base;      // epoch count of the sequence's round 0 (its rounds' offset into the period)
    uint32_t wipe;            // 1: the decode's first clear wipes the table (written with round_base)
    // search settings
    float beam;
    int32_t min_active, max_active, allow_partial, eps_iterations;
    int32_t lp_dtype;         // 0 f32, 1 f16
    // capacities
    int32_t max_lanes;        // lanes held by the workspace
    int32_t max_frames;
    uint32_t frontier_cap;    // Q
    uint32_t claims_cap;      // CC
    uint32_t arena;           // winners-log entries per lane (region stride, global id = L * arena + local)
    uint32_t arena_lim;       // winners-log entries per lane backed by memory (<= arena): the append bound
    uint32_t path_cap;        // device path buffer per lane
    uint32_t strip_cap;       // 64-slot strips per lane and step (slot space = 64 * strip_cap)
    uint32_t res_stride;      // int32 per lane in the result buffer
    // workspace
    LaneCtl *ctl;             // [L]
    const LpDesc *lp;         // device descriptor
    const int32_t *lengths;   // [L] device copy of the batch lengths
    float *lpmax;             // [L][max_frames]
    int32_t *tok_state[2];    // [L][Q] by parity
    uint32_t *tok_tag[2];     // [L][Q] (graphs with epsilon arcs) the round that made the token:
                              //   (the lane's frame << 5) | closure pass (0: the compaction)
    float *tok_score[2];
    int32_t *tok_entry[2];
    int32_t *tok_last[2];
    uint32_t *tok_off[2];     // exclusive arc offset of the token in the step's slot space
    uint32_t *strip_tok[2];   // [L][strip_cap] token holding the first slot of each 64-slot strip
    int32_t *tok_abeg[2];     // first arc of the step's class
    float *tok_ub[2];         // bound on every candidate through the token in the step it feeds:
                              //   its exact best candidate (states with at most kTopArcs emitting
                              //   arcs), else (score + largest weight) + the frame's largest log-prob;
                              //   score + largest final weight before a final step; +inf if unknown
    int32_t *pos[2];          // [L][num_states] state -> token index (validated on read)
    unsigned long long *best; // [ntab][L][num_states] recombination keys (0 = unclaimed); null with
                              //   the hash; round (t, k) uses table k & (ntab - 1)
    HSlot *hash;              // [ntab][L][1 << hash_bits] recombination hash (hash_bits > 0), else null
    uint32_t hash_bits;       // 0: the direct-mapped table; else log2 of the hash slots per lane
    Claim *claims;            // [ntab][L][CC] candidate lists: round (t, k) uses list k & (ntab - 1)
    int32_t ntab;             // recombination tables and candidate lists: 2 on graphs with epsilon
                              //   arcs (a kernel that resolves closure pass k while it relaxes pass
                              //   k + 1 reads one and fills the other), else 1
    int4 *changed[2];         // [L][chg_cap] closure source lists by pass parity: the tokens with
                              //   epsilon arcs, {first epsilon arc, epsilon arcs, entry, score bits}
    uint32_t chg_cap;         // max(claims_cap, frontier_cap)
    int2 *wlog;               // [L][arena] winners log {prev entry, arc}
    int32_t *res;             // [L][res_stride] results
    uint32_t *steps;          // [L][max_frames + 2][kStepFields]
    const int32_t *plan;      // [L][kPlanFields] stream commands of the next sequence
    // lattice mode: every admitted candidate of every step and closure pass. A
    // lattice node is a token of one frame (after the frame's closure): node id
    // = the frame's first node + the token's position in that frame's frontier.
    int32_t lattice;          // 1: persist and prune the lattice
    float output_beam;        // the prune's beam
    int32_t lat_prune_interval;  // > 0: the interval prune runs after every that many steps
    uint32_t lat_cap;         // lattice arcs (and kept records) per lane
    uint32_t lat_nodes;       // lattice nodes per lane: max(arena, lat_cap) + 1 (without log compaction every
                              //   token but the start one has its own entry, so arena + 1 suffice; a lane
                              //   past it has an incomplete lattice)
    int4 *lat_arc;            // [L][lat_cap] {source position, arc, destination position (its state |
                              //   kLatUnresolved until the next compaction maps it), closure pass
                              //   (0: an arc of the step itself)}
    uint32_t *lat_aoff;       // [L][max_frames + 3] first lattice arc of step t at [t + 1] (t = -1: the
                              //   start closure); step t's arcs are followed by its closure's
    uint32_t *lat_nbase;      // [L][max_frames + 3] first node of each frame
    float *lat_score;         // [L][lat_nodes] token score of each node (after its frame's closure)
    int32_t *lat_state;       // [L][lat_nodes] state of each node
    uint32_t *lat_bwd;        // [L][lat_nodes] ordered backward score of each node
    uint8_t *lat_epass;       // [L][lat_nodes] last closure pass whose sources included the node
    uint32_t *lat_chg;        // [L] the last flat epsilon round of the final pass raised a score
    int32_t *lat_out;         // [L][lat_cap][kLatFields] kept records
    int32_t *chg_pos[2];      // [L][chg_cap] frontier position of each closure source (lattice mode)
    // blank-skip pre-slicing
    int32_t *bs_src;          // [L][max_frames] source frame of each kept row
    int32_t *bs_len;          // [L] kept rows
    // winners-log compaction (gc_interval > 0), per lane over its arena region
    int32_t gc_interval;      // steps between compaction rounds (0: none)
    uint32_t *gc_mark;        // [L][arena / 32 + 1] live bits
    uint32_t *gc_wpre;        // [L][arena / 32 + 1] live entries before each 32-entry word
    uint32_t *gc_child;       // [L][arena] live children by compacted position
    int2 *gc_buf;             // [L][arena] compacted entries
    // launch shape (host side): workgroups of the slot walk (0: the frame-loop grid)
    int32_t walk_grid;
};

// Fields of a kept lattice record (int32 each).
enum : int32_t { kLatFrame = 0, kLatSrc, kLatDst, kLatIlabel, kLatArc, kLatScore, kLatLane, kLatFlags,
                 kLatFields = 8 };

// A persisted lattice arc's destination field while it still holds a state
// (state | kLatUnresolved) rather than the destination's frontier position.
constexpr uint32_t kLatUnresolved = 0x80000000u;

// Per-lane stream command of a launch sequence (written by the host).
enum : int32_t { kPlanCmd = 0, kPlanLen, kPlanRow, kPlanWant, kPlanFields = 4 };
enum : int32_t { kCmdPark = 0, kCmdOpen = 1, kCmdAdvance = 2, kCmdFinish = 3 };

// Kernels of a decode, in launch order within a step (ids match WFST_K_*).
enum : int {
    kKClear = 0, kKInit, kKLpmax, kKMax, kKExpand, kKFinalize, kKEpsExpand, kKEpsResolve,
    kKEpsApply, kKBacktrack, kKStreamBegin, kKStreamEnd, kKReclass, kKLatResolve, kKLatInit,
    kKLatBack, kKGcBegin, kKGcMark, kKGcScan, kKGcCompact, kKGcCommit, kKGcRoots, kKGcClear, kKGcEnd,
    kKLatEpsBack, kKLatPrune, kKLatEpsRound, kKEpsApplyExpand, kKLatPrep, kKLatFPrep, kKLatSweep,
    kKLatEmit, kKCount
};

// Host-side launchers (wfst_kernels.hip): t = step (-1 before step 0), k = closure pass.
// With e0 / e1 given, the dispatch records the kernel's start and end in them.
// Kernels receive `dw`, the device copy of `w` (a kernel argument of one pointer:
// dispatch cost grows with argument size); `w` gives host-side launch shapes.
hipError_t launch_kernel(int id, const Work &w, const Work *dw, int t, int k, int grid, hipStream_t s,
                         hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);

// Blank-skip pre-slicing of the log_prob the device descriptor names (B lanes,
// T frames, lengths in Work::lengths) into `out` (same shape): rows whose blank
// log-prob exceeds lthr are dropped, the kept rows packed first, zeros after.
hipError_t launch_blank_skip(const Work &w, const Work *dw, void *out, float lthr, int blank, int B, int T,
                             int grid, hipStream_t s);

// Allocation-free decode (wfst_noalloc.hip): the per-device static
// scratch every such call lays its workspace out in, its address on `device`
// (looked up once per device, with the device current), the mutex that keeps
// those calls one at a time per device, and the kernel that writes a call's
// Work, log-prob descriptor and lengths (n <= kMaxLanes) into the scratch.
constexpr size_t kScratchBytes = 64ull << 20;   // WFST_NOALLOC_SCRATCH_BYTES
hipError_t scratch_region(int device, void **ptr);
std::mutex &scratch_call_mutex(int device);
hipError_t launch_noalloc_put(const Work &w, const LpDesc &d, const int32_t *lengths, int n, Work *dw, LpDesc *dd,
                              int32_t *dl, hipStream_t s);

// Result buffer header (int32 per lane, then arcs[path_cap], words[path_cap]).
enum : int { kResOk = 0, kResReached, kResOverflow, kResArcLen, kResWordLen, kResScore, kResHeader = 8 };

}  // namespace wfst
