// C ABI of the MI355X WFST decoder: graph validation and upload, decoder
// workspace, hipGraph capture of the frame loop, decode, statistics.
// Page "GPU WFST Beam-Search Decoder" (OASR docs): section 4 (validation, SoA
// split, per-state upper-bound weights), section 6.1 (workspace), section 9
// (whole-decode graph replay, plain launches when disabled), section 10 (API).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "wfst.h"
#include "wfst_internal.h"

using namespace wfst;

namespace {

thread_local std::string g_err;

constexpr uint64_t kNoRound = ~0ull;   // no recombination round used since the table was wiped

int fail(int code, const std::string &msg)
{
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(e == hipErrorOutOfMemory ? WFST_ENOMEM : WFST_EDEVICE,
                std::string(what) + ": " + hipGetErrorString(e));
}

#define HIP_TRY(expr)                                              \
    do {                                                           \
        hipError_t _e = (expr);                                    \
        if (_e != hipSuccess) return hip_fail(_e, #expr);          \
    } while (0)

template <typename T>
int dalloc(T **p, size_t count, std::vector<void *> *owned, size_t *bytes)
{
    *p = nullptr;
    const size_t nb = std::max<size_t>(count, 1) * sizeof(T);
    hipError_t e = hipMalloc((void **)p, nb);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc");
    owned->push_back(*p);
    *bytes += nb;
    return WFST_OK;
}


// A caller's buffer of `bytes` bytes at p that the kernels will read or write
// (page section 4: a bad tensor fails with an error, never an out-of-bounds
// access): device (or managed) memory of `device`, inside one allocation.
int check_device_buffer(const void *p, size_t bytes, int device, const char *what)
{
    if (bytes == 0) return WFST_OK;
    hipPointerAttribute_t a{};
    if (!p || hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(WFST_EINVAL, std::string(what) + " is not device memory");
    }
    if (!a.isManaged && (a.type != hipMemoryTypeDevice || a.device != device))
        return fail(WFST_EINVAL, std::string(what) + " is not device memory of the decoder's device");
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess && base) {
        if ((const char *)p + bytes > (const char *)base + size)
            return fail(WFST_EINVAL, std::string(what) + " ends past its allocation");
    } else {
        (void)hipGetLastError();
    }
    return WFST_OK;
}

// The winners log as a lazily committed region (page section 6.2): the whole
// max_lanes x arena range is reserved as device address space once, so every
// pointer a kernel or a captured graph holds stays valid, and physical chunks
// are mapped behind it only where the lanes' logs reach. Lane L's region is
// [L * arena, L * arena + lim) in entries; the chunks covering those ranges for
// the current lim are mapped (a chunk may straddle two lanes' ranges).
struct LogRegion {
    bool vmm = false;                 // false: one plain allocation, all committed
    int device = 0;
    char *va = nullptr;
    size_t va_bytes = 0;
    size_t chunk = 0;                 // mapping unit, bytes
    std::vector<hipMemGenericAllocationHandle_t> h;   // by chunk, null = unmapped
    size_t mapped = 0;                // chunks mapped
    uint32_t lanes = 0, arena = 0, lim = 0;

    // Reserves the range (falls back to a plain allocation when the device has
    // no virtual memory management) and commits lim0 entries per lane.
    hipError_t init(int dev, uint32_t L, uint32_t arena_entries, uint32_t lim0, bool lazy)
    {
        device = dev; lanes = L; arena = arena_entries;
        const size_t need = (size_t)L * arena * sizeof(int2);
        int vmm_ok = 0;
        if (lazy && hipDeviceGetAttribute(&vmm_ok, hipDeviceAttributeVirtualMemoryManagementSupported, dev) != hipSuccess)
            vmm_ok = 0;
        size_t gran = 0;
        hipMemAllocationProp prop = props();
        if (vmm_ok && (hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum) != hipSuccess ||
                       gran == 0))
            vmm_ok = 0;
        if (vmm_ok) {
            // 4 MiB units: few mappings for a large log, little waste for a small one
            chunk = ((std::max<size_t>(4u << 20, gran) + gran - 1) / gran) * gran;
            va_bytes = (need + chunk - 1) / chunk * chunk;
            void *p = nullptr;
            if (hipMemAddressReserve(&p, va_bytes, chunk, nullptr, 0) == hipSuccess) {
                vmm = true;
                va = (char *)p;
                h.assign(va_bytes / chunk, hipMemGenericAllocationHandle_t{});
                return commit(lim0);
            }
        }
        vmm = false;
        va_bytes = need;
        void *p = nullptr;
        hipError_t e = hipMalloc(&p, std::max<size_t>(need, 1));
        if (e != hipSuccess) return e;
        va = (char *)p;
        lim = arena;
        return hipSuccess;
    }

    static hipMemAllocationProp props_for(int dev)
    {
        hipMemAllocationProp p{};
        p.type = hipMemAllocationTypePinned;
        p.location.type = hipMemLocationTypeDevice;
        p.location.id = dev;
        return p;
    }
    hipMemAllocationProp props() const { return props_for(device); }

    // Maps the chunks covering every lane's first n entries (lim never shrinks).
    hipError_t commit(uint32_t n)
    {
        n = std::min(n, arena);
        if (!vmm || n <= lim) return hipSuccess;
        const hipMemAllocationProp prop = props();
        hipMemAccessDesc acc{};
        acc.location = prop.location;
        acc.flags = hipMemAccessFlagsProtReadWrite;
        for (uint32_t L = 0; L < lanes; ++L) {
            const size_t b0 = ((size_t)L * arena + lim) * sizeof(int2);
            const size_t b1 = ((size_t)L * arena + n) * sizeof(int2);
            for (size_t k = b0 / chunk; k < (b1 + chunk - 1) / chunk; ++k) {
                if (h[k]) continue;
                hipMemGenericAllocationHandle_t x{};
                hipError_t e = hipMemCreate(&x, chunk, &prop, 0);
                if (e != hipSuccess) return e;
                e = hipMemMap(va + k * chunk, chunk, 0, x, 0);
                if (e != hipSuccess) { (void)hipMemRelease(x); return e; }
                h[k] = x;
                ++mapped;
                e = hipMemSetAccess(va + k * chunk, chunk, &acc, 1);
                if (e != hipSuccess) return e;
            }
        }
        lim = n;
        return hipSuccess;
    }

    // Maps the chunks covering lane L's whole region (a stream's: it cannot
    // grow and run again). Other lanes' bounds stay as they are.
    hipError_t commit_lane(uint32_t L)
    {
        if (!vmm || lim >= arena) return hipSuccess;
        const hipMemAllocationProp prop = props();
        hipMemAccessDesc acc{};
        acc.location = prop.location;
        acc.flags = hipMemAccessFlagsProtReadWrite;
        const size_t b0 = (size_t)L * arena * sizeof(int2), b1 = ((size_t)L + 1) * arena * sizeof(int2);
        for (size_t k = b0 / chunk; k < (b1 + chunk - 1) / chunk; ++k) {
            if (h[k]) continue;
            hipMemGenericAllocationHandle_t x{};
            hipError_t e = hipMemCreate(&x, chunk, &prop, 0);
            if (e != hipSuccess) return e;
            e = hipMemMap(va + k * chunk, chunk, 0, x, 0);
            if (e != hipSuccess) { (void)hipMemRelease(x); return e; }
            h[k] = x;
            ++mapped;
            e = hipMemSetAccess(va + k * chunk, chunk, &acc, 1);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }

    size_t committed_bytes() const { return vmm ? mapped * chunk : va_bytes; }

    void release()
    {
        if (!va) return;
        if (vmm) {
            for (size_t k = 0; k < h.size(); ++k)
                if (h[k]) { (void)hipMemUnmap(va + k * chunk, chunk); (void)hipMemRelease(h[k]); }
            (void)hipMemAddressFree(va, va_bytes);
        } else {
            (void)hipFree(va);
        }
        va = nullptr;
        h.clear();
        mapped = 0;
    }
};

}  // namespace

struct wfst_graph_s {
    std::atomic<int> refs{1};
    int device = 0;
    int32_t num_states = 0, num_arcs = 0, start = 0, vocab = 0, eps_id = -1;
    int32_t num_records = 0;      // arc records on the device, padding included
    uint32_t max_class_deg = 0;   // most arcs of one class leaving one state
    uint32_t dest_bits = 0;       // arc records hold the in-rank above this many state id bits (0: no ranks)
    uint32_t rank_bits = 0;       // bits of the largest in-rank
    bool eps_positive = false;    // some epsilon arc has a weight > 0 (lattice mode refuses the graph)
    std::vector<void *> owned;
    size_t bytes = 0;
    StateInfo *sinfo = nullptr;
    ArcDLW *arc_dlw = nullptr;
    int32_t *olabel = nullptr, *arc_uid = nullptr;

    ~wfst_graph_s()
    {
        if (!owned.empty()) {
            (void)hipSetDevice(device);
            for (void *p : owned) (void)hipFree(p);
        }
    }
};

struct wfst_decoder_s {
    std::mutex mu;
    wfst_graph_s *g = nullptr;
    wfst_decoder_config cfg{};
    Work w{};
    int grid = 0;
    int passes = 0;                 // closure passes run per step (0 without epsilon arcs)
    std::vector<void *> owned;
    size_t bytes = 0;
    LaneCtl *ctl = nullptr;
    Work *d_work = nullptr;         // device copy of w: the kernels' one pointer argument
    LpDesc *d_desc = nullptr;
    int32_t *d_lengths = nullptr;
    void *h_in = nullptr;           // pinned: LpDesc + lengths
    int32_t *h_res = nullptr;       // pinned: results
    hipStream_t cap_stream = nullptr;
    std::map<int, hipGraphExec_t> graphs;
    std::map<int, hipGraphExec_t> stream_graphs;   // stream sequences by (kind, steps)
    std::vector<int32_t> last_len;   // per lane: frames of the last call (-1: not in it)
    // streams (page section 8): a stream holds one lane for its lifetime
    std::vector<uint8_t> chan_open;
    int open_streams = 0;
    int32_t *d_plan = nullptr;       // [L][kPlanFields] device copy of the plan
    int32_t *h_plan = nullptr;       // pinned: plan, then the sequence's round base
    // recombination rounds are numbered on across decodes and stream sequences;
    // the epoch of round q is 1 + q mod epoch_period, and the table is wiped
    // before the first round used past a multiple of the period
    uint64_t round_next = 0;         // round 0 of the next sequence
    uint64_t round_last = kNoRound;  // last round used since the table was last wiped
    uint32_t dev_round_base = 0;     // round base and wipe flag the device-side Work holds
    uint32_t dev_wipe = 0;
    int last_steps = 0;
    bool prof_on = false;            // time every launch with a start / end event pair
    bool last_profiled = false;
    std::vector<hipEvent_t> ev;
    std::vector<int> ev_kind;
    size_t ev_used = 0;
    LogRegion log;                   // the winners log (w.wlog)
    uint32_t dev_arena_lim = 0;      // append bound the device-side Work holds (log.lim, or the whole region
                                     //   while streams are open: only their lanes append, each fully mapped)
    int last_regrows = 0;            // re-decodes of the last decode after the log grew

    ~wfst_decoder_s()
    {
        (void)hipSetDevice(g ? g->device : 0);
        for (auto &kv : graphs) (void)hipGraphExecDestroy(kv.second);
        for (auto &kv : stream_graphs) (void)hipGraphExecDestroy(kv.second);
        for (hipEvent_t e : ev) (void)hipEventDestroy(e);
        if (cap_stream) (void)hipStreamDestroy(cap_stream);
        if (h_in) (void)hipHostFree(h_in);
        if (h_res) (void)hipHostFree(h_res);
        if (h_plan) (void)hipHostFree(h_plan);
        for (void *p : owned) (void)hipFree(p);
        log.release();
        if (g && g->refs.fetch_sub(1) == 1) delete g;
    }
};

// ------------------------------------------------------------- validation

// Checks every rule of wfst_graph_desc (page section 4: every index the decoder
// later follows without a check) and derives the per-state ranges and
// upper-bound weights. Pure host code: no device call.
static int validate_graph(const wfst_graph_desc *g, std::vector<StateInfo> *info, uint32_t *max_deg)
{
    if (!g) return fail(WFST_EINVAL, "graph descriptor is null");
    const int32_t S = g->num_states, A = g->num_arcs;
    if (S < 2) return fail(WFST_ECORRUPT, "corrupt graph: num_states must be >= 2 (a real state and the super-final state)");
    if (A < 0 || A == INT32_MAX) return fail(WFST_ECORRUPT, "corrupt graph: num_arcs out of range");
    if (!g->row_splits || (A > 0 && (!g->dest || !g->ilabel || !g->olabel || !g->weight)))
        return fail(WFST_EINVAL, "graph array pointer is null");
    if (g->vocab_size < 1 || g->vocab_size >= 65535)
        return fail(WFST_ECORRUPT, "corrupt graph: vocab_size must lie in [1, 65535)");
    if (g->epsilon_id < -1 || g->epsilon_id >= g->vocab_size)
        return fail(WFST_ECORRUPT, "corrupt graph: epsilon_id must be -1 or lie in [0, vocab_size)");
    if (g->start_state < 0 || g->start_state >= S - 1)
        return fail(WFST_ECORRUPT, "corrupt graph: start_state must be a real state");
    const int32_t *rs = g->row_splits;
    if (rs[0] != 0 || rs[S] != A) return fail(WFST_ECORRUPT, "corrupt graph: row_splits must start at 0 and end at num_arcs");
    for (int32_t s = 0; s < S; ++s)
        if (rs[s + 1] < rs[s]) return fail(WFST_ECORRUPT, "corrupt graph: row_splits decreases at state " + std::to_string(s));
    if (rs[S - 1] != rs[S]) return fail(WFST_ECORRUPT, "corrupt graph: the super-final state (last) must have no out-arcs");
    const int32_t sf = S - 1, V = g->vocab_size, eps = g->epsilon_id;
    info->assign((size_t)S, StateInfo{});
    uint32_t md = 0;
    for (int32_t s = 0; s < S; ++s) {
        int32_t a = rs[s];
        const int32_t e = rs[s + 1];
        StateInfo si{};
        si.eps_b = a;
        if (eps >= 0)
            while (a < e && g->ilabel[a] == eps) ++a;
        si.emit_b = a;
        float fmax = -INFINITY;
        for (int k = 0; k < kTopArcs; ++k) { si.top_w[k] = -INFINITY; si.top_il[k] = 0; }
        while (a < e && g->ilabel[a] >= 0 && g->ilabel[a] < V && g->ilabel[a] != eps) {
            // keep the kTopArcs largest-weight emitting arcs, by weight descending
            // (their candidates give the lower bound of the next step's maximum)
            const float wa = g->weight[a];
            const int filled = std::min(a - si.emit_b, kTopArcs);
            int k = filled;
            while (k > 0 && si.top_w[k - 1] < wa) --k;
            if (k < kTopArcs) {
                for (int j = kTopArcs - 1; j > k; --j) { si.top_w[j] = si.top_w[j - 1]; si.top_il[j] = si.top_il[j - 1]; }
                si.top_w[k] = wa;
                si.top_il[k] = (uint16_t)g->ilabel[a];
            }
            ++a;
        }
        si.fin_b = a;
        while (a < e && g->ilabel[a] == -1) {
            fmax = std::max(fmax, g->weight[a]);
            ++a;
        }
        si.end = e;
        if (a != e) {
            const int32_t il = g->ilabel[a];
            if (il == -1 || il == eps || (il >= 0 && il < V))
                return fail(WFST_ECORRUPT, "corrupt graph: arcs of state " + std::to_string(s) +
                                               " are not ordered [epsilon][emitting][final] (arc " + std::to_string(a) + ")");
            return fail(WFST_ECORRUPT, "corrupt graph: arc " + std::to_string(a) + " has ilabel " + std::to_string(il) +
                                           " outside {-1, epsilon_id} and [0, vocab_size)");
        }
        si.fin_maxw = fmax;
        md = std::max(md, (uint32_t)(si.fin_b - si.emit_b));
        md = std::max(md, (uint32_t)(si.end - si.fin_b));
        md = std::max(md, (uint32_t)(si.emit_b - si.eps_b));
        (*info)[(size_t)s] = si;
    }
    for (int32_t a = 0; a < A; ++a) {
        const int32_t d = g->dest[a];
        if (d < 0 || d >= S) return fail(WFST_ECORRUPT, "corrupt graph: arc " + std::to_string(a) + " has dest outside [0, num_states)");
        if ((g->ilabel[a] == -1) != (d == sf))
            return fail(WFST_ECORRUPT, "corrupt graph: arc " + std::to_string(a) +
                                           ": an arc must enter the super-final state iff its ilabel is -1");
        if (g->olabel[a] < 0) return fail(WFST_ECORRUPT, "corrupt graph: arc " + std::to_string(a) + " has a negative olabel");
        const float w = g->weight[a];
        if (std::isnan(w) || (std::isinf(w) && w > 0)) return fail(WFST_ECORRUPT, "corrupt graph: arc " + std::to_string(a) + " has a NaN or +inf weight");
    }
    *max_deg = md;
    return WFST_OK;
}

extern "C" const char *wfst_last_error(void) { return g_err.c_str(); }

extern "C" int wfst_graph_upload(const wfst_graph_desc *g, int device, wfst_graph_t *out)
{
    if (!out) return fail(WFST_EINVAL, "out is null");
    *out = nullptr;
    std::vector<StateInfo> info;
    uint32_t md = 0;
    int rc = validate_graph(g, &info, &md);
    if (rc != WFST_OK) return rc;
    int ndev = 0;
    HIP_TRY(hipGetDeviceCount(&ndev));
    if (device < 0 || device >= ndev) return fail(WFST_EINVAL, "device index out of range");
    HIP_TRY(hipSetDevice(device));

    const int32_t S = g->num_states, A = g->num_arcs;
    // interleaved arc records in CSR order (section 4's split, regrouped so that
    // the fields a pass reads for one arc share a cache line). State s's run
    // starts k <= 31 records after the one before ends, k the least that puts
    // its emitting arcs on the fewest 128-byte lines (12-byte records: a run
    // can start at a line's start only every 32 records); without such a k, or
    // if the records would pass 2^31 - 1, k = 0.
    std::vector<int64_t> first((size_t)S + 1);
    auto lay = [&](bool pad) {
        int64_t p = 0;
        for (int32_t s = 0; s < S; ++s) {
            const StateInfo &si = info[(size_t)s];
            const int64_t ne = si.emit_b - si.eps_b, n = si.fin_b - si.emit_b;
            int k = 0;
            if (pad && n > 0) {
                const int64_t need = (12 * n + 127) / 128 * 128;
                while (k < 32 && (12 * (p + k + ne)) % 128 + 12 * n > need) ++k;
                if (k == 32) k = 0;
            }
            first[(size_t)s] = p + k;
            p += k + (si.end - si.eps_b);
        }
        first[(size_t)S] = p;
        return p;
    };
    if (lay(true) >= INT32_MAX) lay(false);
    const int32_t R = (int32_t)first[(size_t)S];
    auto pos_of = [&](int32_t s, int32_t a) -> int32_t { return (int32_t)(first[(size_t)s] + (a - g->row_splits[s])); };
    std::vector<ArcDLW> dlw((size_t)R, ArcDLW{0, 0u, 0.0f});
    std::vector<int32_t> ol((size_t)R, 0), uid((size_t)R, -1);
    // each non-final arc's rank among its destination's incoming non-final arcs,
    // in arc id order: a table key may break ties by it instead of the arc id
    // (same order among one destination's candidates, far fewer bits), stored
    // above the state id when both fit in 31 bits
    std::vector<uint32_t> rank((size_t)A, 0u);
    uint32_t max_rank = 0;
    {
        std::vector<uint32_t> seen((size_t)S, 0u);
        for (int32_t a = 0; a < A; ++a) {
            if (g->ilabel[a] == -1) continue;
            rank[(size_t)a] = seen[(size_t)g->dest[a]]++;
            max_rank = std::max(max_rank, rank[(size_t)a]);
        }
    }
    uint32_t db = 1, rb = 1;
    while ((1ull << db) < (unsigned long long)S) ++db;
    while ((1ull << rb) <= (unsigned long long)max_rank) ++rb;
    const bool ranks = db + rb <= 31;
    for (int32_t s = 0; s < S; ++s) {
        for (int32_t a = g->row_splits[s]; a < g->row_splits[s + 1]; ++a) {
            const uint32_t il = g->ilabel[a] == -1 ? (uint32_t)kFinalLabel : (uint32_t)g->ilabel[a];
            const uint32_t dfield = (uint32_t)g->dest[a] | (ranks ? rank[(size_t)a] << db : 0u);
            const int32_t q = pos_of(s, a);
            dlw[(size_t)q] = ArcDLW{(int32_t)dfield, il, g->weight[a]};
            ol[(size_t)q] = g->olabel[a];
            uid[(size_t)q] = a;
        }
        // the state's class ranges, as record positions
        StateInfo &si = info[(size_t)s];
        const int32_t d = (int32_t)(first[(size_t)s] - g->row_splits[s]);
        si.eps_b += d; si.emit_b += d; si.fin_b += d; si.end += d;
    }

    wfst_graph_s *h = new wfst_graph_s();
    h->device = device;
    h->num_states = S;
    h->num_arcs = A;
    h->num_records = R;
    h->start = g->start_state;
    h->vocab = g->vocab_size;
    h->eps_id = g->epsilon_id;
    h->max_class_deg = md;
    h->dest_bits = ranks ? db : 0u;
    h->rank_bits = ranks ? rb : 0u;
    if (g->epsilon_id >= 0)
        for (int32_t a = 0; a < A; ++a)
            if (g->ilabel[a] == g->epsilon_id && g->weight[a] > 0.0f) { h->eps_positive = true; break; }
    int r = WFST_OK;
    if ((r = dalloc(&h->sinfo, (size_t)S, &h->owned, &h->bytes)) ||
        (r = dalloc(&h->arc_dlw, (size_t)R, &h->owned, &h->bytes)) ||
        (r = dalloc(&h->olabel, (size_t)R, &h->owned, &h->bytes)) ||
        (r = dalloc(&h->arc_uid, (size_t)R, &h->owned, &h->bytes))) {
        delete h;
        return r;
    }
    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = hipMemcpy(h->sinfo, info.data(), sizeof(StateInfo) * (size_t)S, hipMemcpyHostToDevice);
    if (R > 0) {
        if (e == hipSuccess) e = hipMemcpy(h->arc_dlw, dlw.data(), sizeof(ArcDLW) * (size_t)R, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(h->olabel, ol.data(), 4 * (size_t)R, hipMemcpyHostToDevice);
        if (e == hipSuccess) e = hipMemcpy(h->arc_uid, uid.data(), 4 * (size_t)R, hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) {
        delete h;
        return hip_fail(e, "graph upload");
    }
    *out = h;
    return WFST_OK;
}

extern "C" int wfst_graph_release(wfst_graph_t g)
{
    if (g && g->refs.fetch_sub(1) == 1) delete g;
    return WFST_OK;
}

// ---------------------------------------------------------------- decoder

// Capacities of a decoder's workspace, derived from its config (page section
// 6.1: every buffer sized once from the configuration).
struct Sizes {
    uint64_t Q = 0, slots = 0, strip_cap = 0, CC = 0, arena = 0, lat_cap = 0, path_cap = 0;
    int P = 0;   // closure passes per step (0 without epsilon arcs)
};

// Validates a config against graph g and derives the capacities (0 = derive).
static int derive_sizes(const wfst_graph_s *g, const wfst_decoder_config &c, Sizes *z)
{
    if (!(c.beam > 0.0f) || std::isinf(c.beam)) return fail(WFST_EINVAL, "beam must be positive and finite");
    if (c.max_active < 1 || c.min_active < 0) return fail(WFST_EINVAL, "max_active must be >= 1 and min_active >= 0");
    if (c.max_lanes < 1 || c.max_lanes > kMaxLanes) return fail(WFST_EINVAL, "max_lanes must lie in [1, 64]");
    if (c.max_frames < 1 || c.max_frames > (1 << 20)) return fail(WFST_EINVAL, "max_frames must lie in [1, 2^20]");
    if (c.lp_dtype != WFST_LP_F32 && c.lp_dtype != WFST_LP_F16) return fail(WFST_EINVAL, "lp_dtype must be WFST_LP_F32 or WFST_LP_F16");
    if (c.eps_iterations < 0 || c.eps_iterations > 16) return fail(WFST_EINVAL, "eps_iterations must lie in [0, 16]");
    if (c.frontier_cap < 0 || c.claims_cap < 0 || c.arena_entries < 0 || c.grid_blocks < 0 ||
        c.slot_cap < 0 || c.slot_cap > (1ll << 31))
        return fail(WFST_EINVAL, "capacities must be >= 0");
    if (c.plain_keys < 0 || c.plain_keys > 2) return fail(WFST_EINVAL, "plain_keys must be 0, 1 or 2");
    if (c.epoch_period < 0) return fail(WFST_EINVAL, "epoch_period must be >= 0");
    const int P = (g->eps_id >= 0) ? c.eps_iterations : 0;

    const uint64_t Q = c.frontier_cap ? (uint64_t)c.frontier_cap : std::min<uint64_t>(64ull * (uint64_t)c.max_active, 1ull << 28);
    if (Q < 1 || Q > (1ull << 28)) return fail(WFST_EINVAL, "frontier_cap must lie in [1, 2^28]");
    const uint64_t slots = c.slot_cap ? (uint64_t)c.slot_cap
                                      : std::min<uint64_t>(std::max<uint64_t>(512ull * (uint64_t)c.max_active, 1ull << 16), 1ull << 31);
    const uint64_t strip_cap = (slots + kWave - 1) / kWave;
    // admitted candidates of one pass are at most its candidate arcs; past a
    // million per lane the default stops following slot_cap
    const uint64_t CC = c.claims_cap ? (uint64_t)c.claims_cap
                                     : std::min<uint64_t>(slots, std::max<uint64_t>(Q, 1ull << 20));
    if (CC < 1 || CC > (1ull << 28)) return fail(WFST_EINVAL, "claims_cap must lie in [1, 2^28]");
    const uint64_t maxdeg = std::max<uint32_t>(g->max_class_deg, 1);
    // a live lane holds at most frontier_cap tokens, and their arcs must fit the
    // 32-bit slot space of one lane
    if (Q * maxdeg >= (1ull << 32))
        return fail(WFST_EINVAL, "frontier_cap * (largest out-degree of one arc class) must stay below 2^32 (32-bit slot offsets)");
    uint64_t arena = c.arena_entries ? (uint64_t)c.arena_entries
                   : c.gc_interval > 0
                       ? std::max<uint64_t>(1ull << 20, 8ull * (uint64_t)c.max_active * (uint64_t)(c.gc_interval + 2) * (uint64_t)(1 + P))
                       : std::max<uint64_t>(1ull << 20, 4ull * (uint64_t)c.max_active * (uint64_t)(c.max_frames + 2) * (uint64_t)(1 + P));
    if ((uint64_t)c.max_lanes * arena >= (1ull << 31)) {
        if (c.arena_entries) return fail(WFST_EINVAL, "max_lanes * arena_entries must stay below 2^31");
        arena = ((1ull << 31) - 1) / (uint64_t)c.max_lanes;
    }
    if (c.path_cap < 0 || c.path_cap > (1 << 26)) return fail(WFST_EINVAL, "path_cap must lie in [0, 2^26]");
    if (c.lattice != 0 && c.lattice != 1) return fail(WFST_EINVAL, "lattice must be 0 or 1");
    if (c.lattice && P > 0 && g->eps_positive)
        return fail(WFST_EINVAL, "lattice mode on a graph with epsilon arcs needs every epsilon weight <= 0 "
                                 "(a frame's backward scores are a fixpoint over its epsilon arcs)");
    if (c.lattice && (!(c.output_beam >= 0.0f) || std::isinf(c.output_beam))) return fail(WFST_EINVAL, "output_beam must be finite and >= 0");
    if (c.lattice_cap < 0 || c.lattice_cap > (1ll << 28)) return fail(WFST_EINVAL, "lattice_cap must lie in [0, 2^28]");
    if (c.gc_interval < 0) return fail(WFST_EINVAL, "gc_interval must be >= 0");
    if (c.arena_commit < -1) return fail(WFST_EINVAL, "arena_commit must be >= -1");
    if (c.lat_prune_interval < 0 || c.lat_prune_interval > 512 || (c.lat_prune_interval > 0 && !c.lattice))
        return fail(WFST_EINVAL, "lat_prune_interval must lie in [0, 512] and needs lattice mode");
    if (c.recomb_slots != 0 && (c.recomb_slots < 64 || c.recomb_slots > (1ll << 28) ||
                                (c.recomb_slots & (c.recomb_slots - 1)) != 0))
        return fail(WFST_EINVAL, "recomb_slots must be 0 (direct-mapped table) or a power of 2 in [64, 2^28]");
    z->lat_cap = !c.lattice ? 0 : c.lattice_cap ? (uint64_t)c.lattice_cap
        : std::min<uint64_t>(std::max<uint64_t>(2ull * (uint64_t)c.max_active * (uint64_t)(c.max_frames + 2), 1ull << 20),
                             1ull << 28);
    z->path_cap = c.path_cap ? (uint64_t)c.path_cap : (uint64_t)(c.max_frames + 2) * (uint64_t)(1 + P);
    z->Q = Q; z->slots = slots; z->strip_cap = strip_cap; z->CC = CC; z->arena = arena; z->P = P;
    return WFST_OK;
}

// The scalar fields of a decoder's Work (graph, keys, search settings,
// capacities); pointers are laid out by lay_out.
static int init_work(Work &w, const wfst_graph_s *g, const wfst_decoder_config &c, const Sizes &z)
{
    w = Work{};
    w.sinfo = g->sinfo; w.arc_dlw = g->arc_dlw;
    w.olabel = g->olabel; w.arc_uid = g->arc_uid;
    w.num_states = g->num_states; w.num_arcs = g->num_records; w.num_arcs_user = g->num_arcs;
    w.start_state = g->start;
    w.vocab = g->vocab; w.super_final = g->num_states - 1; w.has_eps = g->eps_id >= 0;
    uint32_t ab = 1;
    while (ab < 31 && (1ll << ab) < (long long)g->num_records) ++ab;
    const bool ranks = g->dest_bits > 0 && c.plain_keys == 0;
    const uint32_t tb = ranks ? g->rank_bits : ab;
    w.tie_bits = tb;
    w.rank_ties = ranks ? 1u : 0u;
    w.dest_bits = g->dest_bits;
    w.dest_mask = g->dest_bits ? (1u << g->dest_bits) - 1u : 0xFFFFFFFFu;
    w.epochs = (tb <= kMaxEpochArcBits && c.plain_keys != 1) ? 1 : 0;
    // more than 2^16 rounds between clears would gain nothing measurable
    const uint32_t pmax = (uint32_t)std::min<uint64_t>((1ull << (32 - tb)) - 1, 65535);
    if (c.epoch_period != 0 && (c.epoch_period < 2 || (uint32_t)c.epoch_period > pmax))
        return fail(WFST_EINVAL, "epoch_period must be 0 or lie in [2, 2^(32 - key tie bits) - 1] (at most 65535)");
    w.epoch_period = c.epoch_period ? (uint32_t)c.epoch_period : pmax;
    if (c.recomb_slots > 0) {
        // the hash's claims carry the round's epoch: it needs epoch-tagged keys
        if (!w.epochs)
            return fail(WFST_EINVAL, "recomb_slots needs epoch-tagged table keys (plain_keys != 1 and key ties of at most 25 bits)");
        uint32_t hb = 0;
        while ((1ll << hb) < c.recomb_slots) ++hb;
        w.hash_bits = hb;
    }
    w.beam = c.beam; w.min_active = c.min_active; w.max_active = c.max_active;
    w.allow_partial = c.allow_partial ? 1 : 0; w.eps_iterations = z.P; w.lp_dtype = c.lp_dtype;
    w.max_lanes = c.max_lanes; w.max_frames = c.max_frames;
    w.frontier_cap = (uint32_t)z.Q; w.claims_cap = (uint32_t)z.CC;
    w.arena = (uint32_t)z.arena; w.path_cap = (uint32_t)z.path_cap; w.strip_cap = (uint32_t)z.strip_cap;
    w.res_stride = (uint32_t)(kResHeader + 2 * z.path_cap);
    w.lattice = c.lattice;
    w.output_beam = c.lattice ? c.output_beam : 0.0f;
    w.lat_cap = (uint32_t)z.lat_cap;
    w.lat_nodes = c.lattice ? (uint32_t)(std::max(z.arena, z.lat_cap) + 1) : 0u;
    w.lat_prune_interval = c.lattice ? c.lat_prune_interval : 0;
    w.gc_interval = c.gc_interval;
    w.chg_cap = (uint32_t)std::max<uint64_t>(z.CC, z.Q);
    // two recombination tables and candidate lists where closure passes run
    // (a kernel resolves pass k from one while it relaxes pass k + 1 into the other)
    w.ntab = z.P > 0 ? 2 : 1;
    w.round_base = 0;
    w.wipe = 0;
    return WFST_OK;
}

// Device buffers of a decode beside the ones Work points to.
struct Extra {
    LaneCtl *ctl = nullptr;
    Work *d_work = nullptr;
    LpDesc *d_desc = nullptr;
    int32_t *d_lengths = nullptr;
    int32_t *d_plan = nullptr;   // streams only
};

// Lays out every device buffer a decode touches through take(&ptr, count),
// called once per buffer in a fixed order. `full`: also the buffers of streams,
// blank-skip, log compaction and lattices (a decoder's), and the winners log is
// not taken here (a decoder maps it as a lazily committed region).
template <typename Take>
static void lay_out(Work &w, Extra &x, const wfst_decoder_config &c, const Sizes &z, size_t S, bool full, Take &&take)
{
    const size_t L = (size_t)c.max_lanes;
    const uint64_t Q = z.Q;
    take(&x.ctl, L);
    take(&x.d_work, 1);
    take(&x.d_desc, 1);
    take(&x.d_lengths, L);
    take(&w.lpmax, L * (size_t)c.max_frames);
    for (int p = 0; p < 2; ++p) {
        take(&w.tok_state[p], L * Q); take(&w.tok_score[p], L * Q); take(&w.tok_entry[p], L * Q);
        take(&w.tok_last[p], L * Q); take(&w.tok_off[p], L * Q); take(&w.tok_abeg[p], L * Q);
        take(&w.tok_ub[p], L * Q); take(&w.strip_tok[p], L * z.strip_cap);
        if (z.P > 0) take(&w.tok_tag[p], L * Q);
        // state -> position maps: read by the closure and the lattice only
        if (w.has_eps || c.lattice) take(&w.pos[p], L * S);
        if (z.P > 0) take(&w.changed[p], L * std::max<uint64_t>(z.CC, Q));
    }
    const size_t nt = (size_t)w.ntab;
    if (w.hash_bits) take(&w.hash, nt * (L << w.hash_bits));
    else take(&w.best, nt * L * S);
    take(&w.claims, nt * L * z.CC);
    take(&w.res, L * (size_t)w.res_stride);
    take(&w.steps, L * (size_t)(c.max_frames + 2) * kStepFields);
    if (!full) {
        take(&w.wlog, L * (size_t)z.arena);
        return;
    }
    take(&x.d_plan, L * kPlanFields);
    take(&w.bs_src, L * (size_t)c.max_frames);
    take(&w.bs_len, L);
    if (c.gc_interval > 0) {
        const size_t words = (size_t)z.arena / 32 + 1;
        take(&w.gc_mark, L * words);
        take(&w.gc_wpre, L * words);
        take(&w.gc_child, L * (size_t)z.arena);
        take(&w.gc_buf, L * (size_t)z.arena);
    }
    if (c.lattice) {
        const size_t F = (size_t)c.max_frames + 3, nodes = (size_t)std::max(z.arena, z.lat_cap) + 1;
        take(&w.lat_arc, L * z.lat_cap);
        take(&w.lat_aoff, L * F);
        take(&w.lat_nbase, L * F);
        take(&w.lat_score, L * nodes);
        take(&w.lat_state, L * nodes);
        take(&w.lat_bwd, L * nodes);
        take(&w.lat_epass, L * nodes);
        take(&w.lat_chg, L);
        take(&w.lat_out, L * z.lat_cap * kLatFields);
        if (z.P > 0)
            for (int p = 0; p < 2; ++p) take(&w.chg_pos[p], L * std::max<uint64_t>(z.CC, Q));
    }
}

// Frame-loop grid: every workgroup first builds the lane table, so 4 workgroups
// per CU (16 wavefronts) is measured best on MI355X for most kernels; the slot
// walk (per = 5) fits five per CU (its register budget is held to five
// wavefronts per SIMD, its candidate buffers to 24 KiB per workgroup) and
// gains from the fifth on the HLG-scale batch.
static int default_grid(const wfst_decoder_config &c, int device, int per = 4)
{
    int ncu = 256;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
        ncu = prop.multiProcessorCount;
    // (a multiple of 8: the kernels deal workgroups to the 8 XCDs in equal runs)
    const long long want = (((long long)c.max_lanes * c.max_active + 127) / 128 + 7) / 8 * 8;
    return c.grid_blocks ? c.grid_blocks : (int)std::min<long long>(std::max<long long>(want, 8), (long long)per * ncu);
}

extern "C" int wfst_decoder_create(wfst_graph_t g, const wfst_decoder_config *cp, wfst_decoder_t *out)
{
    if (!out) return fail(WFST_EINVAL, "out is null");
    *out = nullptr;
    if (!g || !cp) return fail(WFST_EINVAL, "graph or config is null");
    const wfst_decoder_config c = *cp;
    Sizes z;
    int rz = derive_sizes(g, c, &z);
    if (rz != WFST_OK) return rz;
    Work w0;
    rz = init_work(w0, g, c, z);
    if (rz != WFST_OK) return rz;
    HIP_TRY(hipSetDevice(g->device));
    wfst_decoder_s *d = new wfst_decoder_s();
    d->g = g;
    g->refs.fetch_add(1);
    d->cfg = c;
    d->passes = z.P;
    d->grid = default_grid(c, g->device);
    Work &w = d->w;
    w = w0;
    w.walk_grid = default_grid(c, g->device, 5);

    const size_t L = (size_t)c.max_lanes, S = (size_t)g->num_states;
    const uint64_t arena = z.arena;
    int r = WFST_OK;
    Extra x;
    lay_out(w, x, c, z, S, true, [&](auto **p, size_t n) { if (r == WFST_OK) r = dalloc(p, n, &d->owned, &d->bytes); });
    d->ctl = x.ctl; d->d_work = x.d_work; d->d_desc = x.d_desc; d->d_lengths = x.d_lengths; d->d_plan = x.d_plan;
    if (r != WFST_OK) { delete d; return r; }
    {
        const uint64_t lim0 = c.arena_commit < 0 ? arena
                            : c.arena_commit > 0 ? std::min<uint64_t>((uint64_t)c.arena_commit, arena)
                                                 : std::min<uint64_t>(arena, 1ull << 19);
        hipError_t e = d->log.init(g->device, (uint32_t)L, (uint32_t)arena, (uint32_t)lim0, c.arena_commit >= 0);
        if (e != hipSuccess) { delete d; return hip_fail(e, "winners-log region"); }
        w.wlog = (int2 *)d->log.va;
        w.arena_lim = d->log.lim;
        d->dev_arena_lim = d->log.lim;
    }
    w.ctl = d->ctl; w.lp = d->d_desc; w.lengths = d->d_lengths; w.plan = d->d_plan;
    d->chan_open.assign(L, 0);
    d->last_len.assign(L, -1);

    hipError_t e = hipMemset(d->ctl, 0, sizeof(LaneCtl) * L);
    if (e == hipSuccess) e = hipMemcpy(d->d_work, &w, sizeof(Work), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = w.hash_bits ? hipMemset(w.hash, 0, sizeof(HSlot) * w.ntab * (L << w.hash_bits))
                                          : hipMemset(w.best, 0, sizeof(unsigned long long) * w.ntab * L * S);
    for (int p = 0; p < 2 && e == hipSuccess && w.pos[p]; ++p) e = hipMemset(w.pos[p], 0xFF, 4 * L * S);
    if (e == hipSuccess) e = hipHostMalloc(&d->h_in, sizeof(LpDesc) + 4 * L, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void **)&d->h_res, 4 * L * (size_t)w.res_stride, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void **)&d->h_plan, 4 * (L * kPlanFields + 2), hipHostMallocDefault);
    if (e == hipSuccess) e = hipMemset(d->d_plan, 0, 4 * L * kPlanFields);
    if (e == hipSuccess && c.gc_interval > 0) {
        const size_t words = (size_t)arena / 32 + 1;
        e = hipMemset(w.gc_mark, 0, 4 * L * words);
        if (e == hipSuccess) e = hipMemset(w.gc_child, 0, 4 * L * (size_t)arena);
    }
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&d->cap_stream, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) { delete d; return hip_fail(e, "decoder workspace"); }
    *out = d;
    return WFST_OK;
}

extern "C" int wfst_decoder_destroy(wfst_decoder_t d)
{
    delete d;
    return WFST_OK;
}

// One launch of the decode; with profiling on, an event is recorded before it
// (events between consecutive launches bound each kernel's time).
static hipError_t launch(wfst_decoder_s *d, int id, int t, int k, hipStream_t s)
{
    if (d->prof_on) {
        if (2 * d->ev_used + 1 >= d->ev.size()) return hipErrorInvalidValue;
        const size_t i = d->ev_used++;
        d->ev_kind[i] = id;
        return launch_kernel(id, d->w, d->d_work, t, k, d->grid, s, d->ev[2 * i], d->ev[2 * i + 1]);
    }
    return launch_kernel(id, d->w, d->d_work, t, k, d->grid, s);
}

// Queue one whole decode of `steps` frame-loop steps: go(id, t, k) launches one
// kernel. With epoch-tagged table keys the epoch of round (t, k) restarts at 1
// every epoch_period rounds: the whole table is cleared before such a round (a
// decode whose rounds pass a multiple of the period starts at one, with the
// table wiped, and uses every round after its round 0).
// Closure passes 1..P of step t (t = -1: the start closure). Pass k + 1's
// relaxation runs in pass k's resolving launch (kKEpsApplyExpand) unless a
// table clear is due before round (t, k + 1): the clear must fall between the
// two. clear(t, k) enqueues the clear due before round (t, k), if any;
// clear_due(t, k) says whether one is.
template <typename Go, typename Due, typename Clear>
static hipError_t enqueue_closure(int t, int P, Go &&go, Due &&clear_due, Clear &&clear)
{
    hipError_t e;
    bool relaxed = false;   // pass k's relaxation ran in the launch before
    for (int k = 1; k <= P; ++k) {
        if (!relaxed) {
            if ((e = clear(t, k)) != hipSuccess) return e;
            if ((e = go(kKEpsExpand, t, k)) != hipSuccess) return e;
        }
        const bool fuse = k < P && !clear_due(t, k + 1);
        if (fuse && (e = clear(t, k + 1)) != hipSuccess) return e;   // (none due: bookkeeping only)
        if ((e = go(fuse ? kKEpsApplyExpand : kKEpsApply, t, k)) != hipSuccess) return e;
        relaxed = fuse;
    }
    return hipSuccess;
}

template <typename Go>
static hipError_t enqueue_decode_with(const Work &w, int passes, int steps, Go &&go)
{
    hipError_t e;
    auto clear_due = [&](int t, int k) -> bool {
        if (!w.epochs) return false;
        const long long q = (long long)(t + 1) * (1 + passes) + k;
        return q > 0 && q % w.epoch_period == 0;
    };
    auto wrap_clear = [&](int t, int k) -> hipError_t {
        return clear_due(t, k) ? go(kKClear, t, 1) : hipSuccess;
    };
    if ((e = go(kKClear, 0, 0)) != hipSuccess) return e;
    if ((e = go(kKInit, 0, 0)) != hipSuccess) return e;
    // (the row maxima first: the start closure's tokens carry frame 0's in their bound)
    if ((e = go(kKLpmax, 0, 0)) != hipSuccess) return e;
    if ((e = enqueue_closure(-1, passes, go, clear_due, wrap_clear)) != hipSuccess) return e;
    for (int t = 0; t < steps; ++t) {
        if ((e = wrap_clear(t, 0)) != hipSuccess) return e;
        if ((e = go(kKMax, t, 0)) != hipSuccess) return e;
        if ((e = go(kKFinalize, t, 0)) != hipSuccess) return e;
        if ((e = enqueue_closure(t, passes, go, clear_due, wrap_clear)) != hipSuccess) return e;
        if (w.lat_prune_interval > 0 && (t + 1) % w.lat_prune_interval == 0 && t + 1 < steps &&
            ((e = go(kKLatPrep, t, 0)) != hipSuccess || (e = go(kKLatPrune, t, 0)) != hipSuccess)) return e;
        if (w.gc_interval > 0 && (t + 1) % w.gc_interval == 0 && t + 1 < steps) {
            static const int ids[] = {kKGcBegin, kKGcMark, kKGcScan, kKGcCompact, kKGcCommit, kKGcRoots, kKGcClear, kKGcEnd};
            for (int id : ids)
                if ((e = go(id, 0, 0)) != hipSuccess) return e;
        }
    }
    if (w.lattice && passes <= 0) {
        // without a closure every lattice arc is a step arc: work records, one
        // backward sweep per lane over all its frames, the kept arcs
        if (steps > 0 && ((e = go(kKLatFPrep, steps, 0)) != hipSuccess || (e = go(kKLatSweep, 0, 0)) != hipSuccess ||
                          (e = go(kKLatEmit, steps, 0)) != hipSuccess)) return e;
    } else if (w.lattice) {
        if ((e = go(kKLatInit, 0, 0)) != hipSuccess) return e;
        for (int t = steps - 1; t >= 0; --t) {
            if ((e = go(kKLatBack, t, 0)) != hipSuccess) return e;
            if (passes <= 0) continue;
            const int rounds = std::min(passes, 3) + 1;
            for (int k = 1; k <= rounds; ++k)
                if ((e = go(kKLatEpsRound, t, k == rounds ? 1 : 0)) != hipSuccess) return e;
            if ((e = go(kKLatEpsBack, t, 0)) != hipSuccess) return e;
        }
    }
    return go(kKBacktrack, 0, 0);
}

// One winners-log compaction round (lanes that ran a real step).
static hipError_t gc_round(wfst_decoder_s *d, hipStream_t s)
{
    static const int ids[] = {kKGcBegin, kKGcMark, kKGcScan, kKGcCompact, kKGcCommit, kKGcRoots, kKGcClear, kKGcEnd};
    for (int id : ids) {
        hipError_t e = launch(d, id, 0, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Queue one whole decode of `steps` frame-loop steps on stream s.
static hipError_t enqueue_decode(wfst_decoder_s *d, int steps, hipStream_t s)
{
    d->ev_used = 0;
    return enqueue_decode_with(d->w, d->passes, steps, [&](int id, int t, int k) { return launch(d, id, t, k, s); });
}

static int graph_for(wfst_decoder_s *d, int steps, hipGraphExec_t *exec)
{
    const int key = steps * 2 + (d->prof_on ? 1 : 0);
    auto it = d->graphs.find(key);
    if (it != d->graphs.end()) { *exec = it->second; return WFST_OK; }
    hipGraph_t graph = nullptr;
    HIP_TRY(hipStreamBeginCapture(d->cap_stream, hipStreamCaptureModeThreadLocal));
    hipError_t e = enqueue_decode(d, steps, d->cap_stream);
    hipError_t e2 = hipStreamEndCapture(d->cap_stream, &graph);
    if (e != hipSuccess) { if (graph) (void)hipGraphDestroy(graph); return hip_fail(e, "kernel launch during capture"); }
    if (e2 != hipSuccess) return hip_fail(e2, "hipStreamEndCapture");
    hipGraphExec_t ex = nullptr;
    e = hipGraphInstantiate(&ex, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
    d->graphs[key] = ex;
    *exec = ex;
    return WFST_OK;
}

// Round base (the sequence's round 0 modulo the epoch period) and the decode's
// wipe flag, held by the device-side Work.
static int set_round_base(wfst_decoder_s *d, uint32_t v, uint32_t wipe, hipStream_t s)
{
    static_assert(offsetof(Work, wipe) == offsetof(Work, round_base) + 4, "round_base and wipe are adjacent");
    if (d->dev_round_base == v && d->dev_wipe == wipe) return WFST_OK;
    uint32_t *h = (uint32_t *)(d->h_plan + (size_t)d->cfg.max_lanes * kPlanFields);
    h[0] = v;
    h[1] = wipe;
    HIP_TRY(hipMemcpyAsync((char *)d->d_work + offsetof(Work, round_base), h, 8, hipMemcpyHostToDevice, s));
    d->dev_round_base = v;
    d->dev_wipe = wipe;
    return WFST_OK;
}

// Whether rounds first..last (absolute numbers, in use order) need a table wipe
// before some of them: the last round used since the last wipe (or, with none,
// the first of them) lies in an earlier epoch period than the last of them.
static bool rounds_wrap(const wfst_decoder_s *d, uint64_t first, uint64_t last)
{
    const uint64_t P = d->w.epoch_period;
    const uint64_t ref = d->round_last == kNoRound ? first : d->round_last;
    return ref / P != last / P;
}

// Publishes append bound v to the kernels (their Work copy). The caller has no
// kernel of this decoder in flight that the bound could matter to.
static int set_arena_lim(wfst_decoder_s *d, uint32_t v)
{
    if (d->dev_arena_lim == v) return WFST_OK;
    d->w.arena_lim = v;
    HIP_TRY(hipMemcpy((char *)d->d_work + offsetof(Work, arena_lim), &v, 4, hipMemcpyHostToDevice));
    d->dev_arena_lim = v;
    return WFST_OK;
}

// Commits n winners-log entries per lane and publishes the bound to the
// kernels. Same precondition.
static int grow_log(wfst_decoder_s *d, uint32_t n)
{
    if (n <= d->log.lim) return set_arena_lim(d, d->log.lim);
    hipError_t e = d->log.commit(n);
    if (e != hipSuccess) return hip_fail(e, "winners-log commit");
    return set_arena_lim(d, d->log.lim);
}

// Copies result block `lane` (already in h_res) to output row j.
static void copy_result(const wfst_decoder_s *d, int lane, int j, int32_t *out_words, int32_t words_cap,
                        int32_t *out_word_lens, int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens,
                        float *out_scores, int32_t *out_meta)
{
    const int32_t *R = d->h_res + (size_t)d->w.res_stride * (size_t)lane;
    const int32_t *arcs = R + kResHeader;
    const int32_t *words = arcs + d->w.path_cap;
    const int32_t alen = R[kResArcLen], wlen = R[kResWordLen];
    const int32_t astored = std::min<int32_t>(alen, (int32_t)d->w.path_cap);
    out_meta[3 * j + 0] = R[kResOk];
    out_meta[3 * j + 1] = R[kResReached];
    out_meta[3 * j + 2] = R[kResOverflow];
    uint32_t sb = (uint32_t)R[kResScore];
    float sc;
    std::memcpy(&sc, &sb, 4);
    out_scores[j] = sc;
    out_arc_lens[j] = alen;
    out_word_lens[j] = wlen;
    if (arcs_cap > 0) std::memcpy(out_arcs + (size_t)j * arcs_cap, arcs, 4 * (size_t)std::min(astored, arcs_cap));
    if (words_cap > 0) std::memcpy(out_words + (size_t)j * words_cap, words, 4 * (size_t)std::min(wlen, words_cap));
}

extern "C" int wfst_decode(wfst_decoder_t d, const void *log_prob, int32_t B, int32_t T, int32_t V,
                           const int32_t *lengths_host, void *stream, int32_t *out_words, int32_t words_cap,
                           int32_t *out_word_lens, int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens,
                           float *out_scores, int32_t *out_meta)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    const wfst_decoder_config &c = d->cfg;
    if (B < 1 || B > c.max_lanes) return fail(WFST_EINVAL, "B must lie in [1, max_lanes]");
    if (T < 0 || T > c.max_frames) return fail(WFST_EINVAL, "T must lie in [0, max_frames]");
    if (V != d->g->vocab) return fail(WFST_EINVAL, "V differs from the graph's vocab_size");
    if (!lengths_host || !out_word_lens || !out_arc_lens || !out_scores || !out_meta)
        return fail(WFST_EINVAL, "an output or lengths pointer is null");
    if (words_cap < 0 || arcs_cap < 0 || (words_cap > 0 && !out_words) || (arcs_cap > 0 && !out_arcs))
        return fail(WFST_EINVAL, "bad words/arcs buffer");
    int32_t maxlen = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (lengths_host[b] < 0 || lengths_host[b] > T) return fail(WFST_EINVAL, "lengths must lie in [0, T]");
        maxlen = std::max(maxlen, lengths_host[b]);
    }
    if (maxlen > 0 && !log_prob) return fail(WFST_EINVAL, "log_prob is null");

    std::lock_guard<std::mutex> lock(d->mu);
    if (d->open_streams > 0) return fail(WFST_EINVAL, "the decoder has open streams (release them first)");
    HIP_TRY(hipSetDevice(d->g->device));
    {
        // (streams left the kernels' bound at their lanes' whole regions)
        const int rcl = set_arena_lim(d, d->log.lim);
        if (rcl != WFST_OK) return rcl;
    }
    const size_t elem = c.lp_dtype == WFST_LP_F16 ? 2 : 4;
    if (maxlen > 0) {
        const int rcb = check_device_buffer(log_prob, (size_t)B * (size_t)T * (size_t)V * elem, d->g->device, "log_prob");
        if (rcb != WFST_OK) return rcb;
    }
    hipStream_t s = (hipStream_t)stream;
    const size_t L = (size_t)c.max_lanes;
    LpDesc *hd = (LpDesc *)d->h_in;
    hd->base = log_prob;
    hd->stride_t = V;
    hd->stride_b = (long long)T * V;
    hd->B = B;
    hd->dtype = c.lp_dtype;
    int32_t *hl = (int32_t *)((char *)d->h_in + sizeof(LpDesc));
    for (size_t b = 0; b < L; ++b) hl[b] = (int32_t)b < B ? lengths_host[b] : 0;
    HIP_TRY(hipMemcpyAsync(d->d_desc, hd, sizeof(LpDesc), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(d->d_lengths, hl, 4 * L, hipMemcpyHostToDevice, s));

    const int steps = maxlen + 1;
    const size_t rs = d->w.res_stride;
    d->last_regrows = 0;
    for (;;) {
        // timing events cannot be read back from a replayed graph: a profiled
        // decode runs the same kernels as plain launches
        const bool replay = c.use_graphs && !d->prof_on;
        int bucket = steps <= 256 ? (steps + 31) / 32 * 32 : (steps + 63) / 64 * 64;
        bucket = std::min(bucket, c.max_frames + 1);
        const int nsteps = replay ? bucket : steps;
        // rounds 1 .. R - 1 of the decode are used (round 0 is not). They number
        // on from the last sequence's unless they would pass an epoch wrap: then
        // the decode starts at the next multiple of the period with the table
        // wiped, and clears it again at each later multiple. (A decode run again
        // after the log grew takes fresh rounds: its first run's entries lose.)
        const uint64_t R = (uint64_t)(nsteps + 1) * (uint64_t)(1 + d->passes);
        uint64_t base = d->round_next;
        uint32_t wipe = 0;
        if (d->w.epochs) {
            const uint64_t P = d->w.epoch_period;
            if (R > P || rounds_wrap(d, base + 1, base + R - 1)) {
                base = (base + P - 1) / P * P;
                wipe = 1;
            }
        }
        int rc0 = set_round_base(d, d->w.epochs ? (uint32_t)(base % d->w.epoch_period) : 0u, wipe, s);
        if (rc0 != WFST_OK) return rc0;
        if (replay) {
            hipGraphExec_t ex = nullptr;
            int rc = graph_for(d, bucket, &ex);
            if (rc != WFST_OK) return rc;
            HIP_TRY(hipGraphLaunch(ex, s));
            d->last_steps = bucket;
        } else {
            hipError_t e = enqueue_decode(d, steps, s);
            if (e != hipSuccess) return hip_fail(e, "kernel launch");
            d->last_steps = steps;
        }
        d->round_next = base + R;
        d->round_last = base + R - 1;
        d->last_profiled = d->prof_on;
        HIP_TRY(hipMemcpyAsync(d->h_res, d->w.res, 4 * rs * (size_t)B, hipMemcpyDeviceToHost, s));
        HIP_TRY(hipStreamSynchronize(s));
        // a lane whose log outgrew the committed part of its region: commit more
        // (page section 6.2: grow and decode again; a decode starts from nothing,
        // so the result is the one a fully committed region gives)
        if (d->log.lim >= d->w.arena) break;
        bool grow = false;
        for (int32_t b = 0; b < B; ++b)
            grow |= (d->h_res[rs * (size_t)b + kResOverflow] & kOvfArena) != 0;
        if (!grow) break;
        // (the arena bit also reports a full lattice: only lanes the log's bound
        // stopped count)
        std::vector<LaneCtl> ctl((size_t)c.max_lanes);
        HIP_TRY(hipMemcpy(ctl.data(), d->ctl, sizeof(LaneCtl) * ctl.size(), hipMemcpyDeviceToHost));
        grow = false;
        for (int32_t b = 0; b < B; ++b) grow |= ctl[(size_t)b].log_full != 0u;
        if (!grow) break;
        // the log grows about linearly with the frames: aim at the longest lane's
        // end from the step where the first one stopped, at least doubling
        uint64_t want = 2ull * d->log.lim;
        for (int32_t b = 0; b < B; ++b) {
            if (!ctl[(size_t)b].log_full) continue;
            const uint64_t done = (uint64_t)std::max(ctl[(size_t)b].last_step, 0) + 1;
            want = std::max<uint64_t>(want, (uint64_t)d->log.lim * ((uint64_t)lengths_host[b] + 2) * 5 / (4 * done));
        }
        int rc = grow_log(d, (uint32_t)std::min<uint64_t>(want, d->w.arena));
        if (rc != WFST_OK) return rc;
        d->last_regrows += 1;
    }

    d->last_len.assign(L, -1);
    for (int32_t b = 0; b < B; ++b) d->last_len[(size_t)b] = lengths_host[b];
    for (int32_t b = 0; b < B; ++b)
        copy_result(d, b, b, out_words, words_cap, out_word_lens, out_arcs, arcs_cap, out_arc_lens, out_scores, out_meta);
    return WFST_OK;
}

// ------------------------------------------------------ allocation-free decode

static_assert(kScratchBytes == (size_t)WFST_NOALLOC_SCRATCH_BYTES, "one scratch size in the header and the library");

extern "C" int wfst_decode_noalloc(wfst_graph_t g, const wfst_decoder_config *cp, const void *log_prob, int32_t B,
                                   int32_t T, int32_t V, const int32_t *lengths_host, void *stream,
                                   int32_t *out_words, int32_t words_cap, int32_t *out_word_lens,
                                   int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens, float *out_scores,
                                   int32_t *out_meta)
{
    if (!g || !cp) return fail(WFST_EINVAL, "graph or config is null");
    const wfst_decoder_config &c = *cp;
    if (c.lattice) return fail(WFST_EINVAL, "the allocation-free decode has no lattice mode");
    if (c.gc_interval > 0) return fail(WFST_EINVAL, "the allocation-free decode runs without log compaction (gc_interval 0)");
    Sizes z;
    int rc = derive_sizes(g, c, &z);
    if (rc != WFST_OK) return rc;
    if (B < 1 || B > c.max_lanes) return fail(WFST_EINVAL, "B must lie in [1, max_lanes]");
    if (T < 0 || T > c.max_frames) return fail(WFST_EINVAL, "T must lie in [0, max_frames]");
    if (V != g->vocab) return fail(WFST_EINVAL, "V differs from the graph's vocab_size");
    if (!lengths_host || !out_word_lens || !out_arc_lens || !out_scores || !out_meta)
        return fail(WFST_EINVAL, "an output or lengths pointer is null");
    if (words_cap < 0 || arcs_cap < 0 || (words_cap > 0 && !out_words) || (arcs_cap > 0 && !out_arcs))
        return fail(WFST_EINVAL, "bad words/arcs buffer");
    int32_t maxlen = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (lengths_host[b] < 0 || lengths_host[b] > T) return fail(WFST_EINVAL, "lengths must lie in [0, T]");
        maxlen = std::max(maxlen, lengths_host[b]);
    }
    if (maxlen > 0 && !log_prob) return fail(WFST_EINVAL, "log_prob is null");
    Work w;
    rc = init_work(w, g, c, z);
    if (rc != WFST_OK) return rc;

    // the workspace, laid out in the device's scratch (256-byte aligned pieces)
    const size_t L = (size_t)c.max_lanes, S = (size_t)g->num_states;
    size_t need = 0;
    bool over = false;
    auto place = [&](char *base) {
        need = 0;
        Extra x;
        lay_out(w, x, c, z, S, false, [&](auto **p, size_t n) {
            using E = std::remove_pointer_t<std::remove_pointer_t<decltype(p)>>;
            const size_t nb = std::max<size_t>(n, 1) * sizeof(E);
            need = (need + 255) & ~(size_t)255;
            if (nb > kScratchBytes || need > kScratchBytes - nb) over = true;
            *p = (base && !over) ? (E *)(base + need) : nullptr;
            need += nb;
        });
        return x;
    };
    place(nullptr);
    if (over || need > kScratchBytes)
        return fail(WFST_EINVAL, "the workspace needs " + std::to_string(need) + " bytes; the allocation-free decode has " +
                                     std::to_string(kScratchBytes) +
                                     " (lower max_lanes, frontier_cap, claims_cap, slot_cap, arena_entries or path_cap)");
    HIP_TRY(hipSetDevice(g->device));
    const size_t elem = c.lp_dtype == WFST_LP_F16 ? 2 : 4;
    if (maxlen > 0) {
        const int rcb = check_device_buffer(log_prob, (size_t)B * (size_t)T * (size_t)V * elem, g->device, "log_prob");
        if (rcb != WFST_OK) return rcb;
    }
    void *base = nullptr;
    HIP_TRY(scratch_region(g->device, &base));
    std::lock_guard<std::mutex> lock(scratch_call_mutex(g->device));
    const Extra x = place((char *)base);
    w.ctl = x.ctl; w.lp = x.d_desc; w.lengths = x.d_lengths; w.plan = nullptr;
    w.arena_lim = w.arena;   // the whole region is backed: nothing to commit later
    hipStream_t s = (hipStream_t)stream;
    LpDesc hd{};
    hd.base = log_prob;
    hd.stride_t = V;
    hd.stride_b = (long long)T * V;
    hd.B = B;
    hd.dtype = c.lp_dtype;
    int32_t lens[kMaxLanes] = {0};
    for (int32_t b = 0; b < B; ++b) lens[b] = lengths_host[b];
    const int grid = default_grid(c, g->device);
    w.walk_grid = default_grid(c, g->device, 5);
    const int steps = maxlen + 1;
    // the scratch holds whatever the last call left: the control blocks and the
    // recombination table start at zero, the position maps at -1
    auto run = [&]() -> hipError_t {
        hipError_t e = hipMemsetAsync(x.ctl, 0, sizeof(LaneCtl) * L, s);
        if (e == hipSuccess)
            e = w.hash_bits ? hipMemsetAsync(w.hash, 0, sizeof(HSlot) * w.ntab * (L << w.hash_bits), s)
                            : hipMemsetAsync(w.best, 0, sizeof(unsigned long long) * w.ntab * L * S, s);
        for (int p = 0; p < 2 && e == hipSuccess && w.pos[p]; ++p) e = hipMemsetAsync(w.pos[p], 0xFF, 4 * L * S, s);
        if (e == hipSuccess) e = launch_noalloc_put(w, hd, lens, (int)L, x.d_work, x.d_desc, x.d_lengths, s);
        if (e == hipSuccess)
            e = enqueue_decode_with(w, z.P, steps, [&](int id, int t, int k) {
                return launch_kernel(id, w, x.d_work, t, k, grid, s);
            });
        return e;
    };
    hipError_t e = run();
    // result headers, then each lane's arcs and words straight into the
    // caller's rows (entries past a row's length are unspecified)
    int32_t hdr[kMaxLanes][kResHeader];
    const size_t rs = 4 * (size_t)w.res_stride;
    if (e == hipSuccess) e = hipMemcpy2DAsync(hdr, sizeof(hdr[0]), w.res, rs, sizeof(hdr[0]), (size_t)B, hipMemcpyDeviceToHost, s);
    const size_t acopy = std::min<size_t>((size_t)arcs_cap, w.path_cap), wcopy = std::min<size_t>((size_t)words_cap, w.path_cap);
    if (e == hipSuccess && acopy > 0)
        e = hipMemcpy2DAsync(out_arcs, 4 * (size_t)arcs_cap, w.res + kResHeader, rs, 4 * acopy, (size_t)B,
                             hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && wcopy > 0)
        e = hipMemcpy2DAsync(out_words, 4 * (size_t)words_cap, w.res + kResHeader + w.path_cap, rs, 4 * wcopy, (size_t)B,
                             hipMemcpyDeviceToHost, s);
    // (also on failure: no work of this call may still run when the next one starts)
    const hipError_t es = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "allocation-free decode");
    if (es != hipSuccess) return hip_fail(es, "hipStreamSynchronize");
    for (int32_t b = 0; b < B; ++b) {
        const int32_t *R = hdr[b];
        out_meta[3 * b + 0] = R[kResOk];
        out_meta[3 * b + 1] = R[kResReached];
        out_meta[3 * b + 2] = R[kResOverflow];
        uint32_t sb = (uint32_t)R[kResScore];
        float sc;
        std::memcpy(&sc, &sb, 4);
        out_scores[b] = sc;
        out_arc_lens[b] = R[kResArcLen];
        out_word_lens[b] = R[kResWordLen];
    }
    return WFST_OK;
}

// ----------------------------------------------------------------- streams

enum { kSeqOpen = 0, kSeqAdvance, kSeqFinish };

// Queues one stream sequence (plan already in d_plan): records cleared, plan
// applied, then the start closure (open), the final class (finish) or the row
// maxima (advance), `steps` steps, the commit and the wanted results. Its
// recombination rounds continue the count of earlier sequences, with the table
// cleared before the epoch wraps.
static hipError_t enqueue_stream(wfst_decoder_s *d, int kind, int steps, hipStream_t s)
{
    hipError_t e;
    d->ev_used = 0;
    const uint64_t base = d->round_next;
    uint64_t last = d->round_last;
    // before each round it uses: a wipe when the round lies in a later epoch
    // period than the last round used (a captured sequence has none: see
    // stream_wraps)
    auto wrap_due = [&](int t, int k) -> bool {
        if (!d->w.epochs) return false;
        const uint64_t q = base + (uint64_t)((long long)(t + 1) * (1 + d->passes) + k);
        const uint64_t P = d->w.epoch_period;
        return last != kNoRound && last / P != q / P;
    };
    auto wrap = [&](int t, int k) -> hipError_t {
        if (!d->w.epochs) return hipSuccess;
        const bool clear = wrap_due(t, k);
        last = base + (uint64_t)((long long)(t + 1) * (1 + d->passes) + k);
        return clear ? launch(d, kKClear, t, 1, s) : hipSuccess;
    };
    auto go = [&](int id, int t, int k) -> hipError_t { return launch(d, id, t, k, s); };
    if ((e = launch(d, kKClear, 0, 2, s)) != hipSuccess) return e;
    if ((e = launch(d, kKStreamBegin, 0, 0, s)) != hipSuccess) return e;
    if (kind == kSeqOpen && (e = enqueue_closure(-1, d->passes, go, wrap_due, wrap)) != hipSuccess) return e;
    if (kind == kSeqFinish && (e = launch(d, kKReclass, 0, 0, s)) != hipSuccess) return e;
    if (kind == kSeqAdvance && steps > 0 && (e = launch(d, kKLpmax, 0, 0, s)) != hipSuccess) return e;
    for (int t = 0; t < steps; ++t) {
        if ((e = wrap(t, 0)) != hipSuccess) return e;
        if ((e = launch(d, kKMax, t, 0, s)) != hipSuccess) return e;
        if ((e = launch(d, kKFinalize, t, 0, s)) != hipSuccess) return e;
        if (kind != kSeqAdvance) continue;
        if ((e = enqueue_closure(t, d->passes, go, wrap_due, wrap)) != hipSuccess) return e;
        // every gc_interval steps and at the end of the chunk
        if (d->w.gc_interval > 0 && ((t + 1) % d->w.gc_interval == 0 || t + 1 == steps) &&
            (e = gc_round(d, s)) != hipSuccess) return e;
    }
    if ((e = launch(d, kKStreamEnd, 0, 0, s)) != hipSuccess) return e;
    if ((e = launch(d, kKBacktrack, 0, 0, s)) != hipSuccess) return e;
    return hipSuccess;
}

// Recombination rounds a stream sequence uses.
static uint64_t stream_rounds(const wfst_decoder_s *d, int kind, int steps)
{
    return (uint64_t)((kind == kSeqOpen ? 0 : steps) + 1) * (uint64_t)(1 + d->passes);
}

// The first and last rounds a stream sequence uses, as offsets from its round
// 0 (false when it uses none): the start closure's passes (open), the steps'
// slot passes and closure passes (advance), the steps' slot passes (finish).
static bool stream_used(const wfst_decoder_s *d, int kind, int steps, uint64_t *first, uint64_t *last)
{
    const uint64_t p1 = 1 + (uint64_t)d->passes;
    if (kind == kSeqOpen) {
        *first = 1;
        *last = (uint64_t)d->passes;
        return d->passes > 0;
    }
    *first = p1;
    *last = kind == kSeqFinish ? (uint64_t)steps * p1 : (uint64_t)(steps + 1) * p1 - 1;
    return steps > 0;
}

// Whether the sequence needs a table wipe before one of its rounds (then it
// runs as plain launches, with the wipe before that round).
static bool stream_wraps(const wfst_decoder_s *d, int kind, int steps)
{
    uint64_t f = 0, l = 0;
    if (!d->w.epochs || !stream_used(d, kind, steps, &f, &l)) return false;
    return rounds_wrap(d, d->round_next + f, d->round_next + l);
}

// Runs a stream sequence with the plan in h_plan and waits for it; copies the
// result blocks of `lanes` (the lanes whose result is wanted) to h_res. With
// use_graphs the sequence replays a graph captured once per (kind, steps).
static int run_stream(wfst_decoder_s *d, int kind, int steps, hipStream_t s, const std::vector<int> &lanes)
{
    const size_t L = (size_t)d->cfg.max_lanes;
    const uint32_t rb = d->w.epochs ? (uint32_t)(d->round_next % d->w.epoch_period) : 0u;
    int rc = set_round_base(d, rb, 0u, s);
    if (rc != WFST_OK) return rc;
    HIP_TRY(hipMemcpyAsync(d->d_plan, d->h_plan, 4 * L * kPlanFields, hipMemcpyHostToDevice, s));
    if (d->cfg.use_graphs && !d->prof_on && !stream_wraps(d, kind, steps)) {
        const int key = steps * 4 + kind;
        auto it = d->stream_graphs.find(key);
        hipGraphExec_t ex = nullptr;
        if (it != d->stream_graphs.end()) {
            ex = it->second;
        } else {
            hipGraph_t graph = nullptr;
            HIP_TRY(hipStreamBeginCapture(d->cap_stream, hipStreamCaptureModeThreadLocal));
            hipError_t e = enqueue_stream(d, kind, steps, d->cap_stream);
            hipError_t e2 = hipStreamEndCapture(d->cap_stream, &graph);
            if (e != hipSuccess) { if (graph) (void)hipGraphDestroy(graph); return hip_fail(e, "kernel launch during capture"); }
            if (e2 != hipSuccess) return hip_fail(e2, "hipStreamEndCapture");
            e = hipGraphInstantiate(&ex, graph, nullptr, nullptr, 0);
            (void)hipGraphDestroy(graph);
            if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
            d->stream_graphs[key] = ex;
        }
        HIP_TRY(hipGraphLaunch(ex, s));
    } else {
        hipError_t e = enqueue_stream(d, kind, steps, s);
        if (e != hipSuccess) return hip_fail(e, "kernel launch");
    }
    if (!lanes.empty()) {
        // one copy over the span of wanted lanes
        const size_t rs = d->w.res_stride;
        const int lo = *std::min_element(lanes.begin(), lanes.end());
        const int hi = *std::max_element(lanes.begin(), lanes.end());
        HIP_TRY(hipMemcpyAsync(d->h_res + rs * (size_t)lo, d->w.res + rs * (size_t)lo, 4 * rs * (size_t)(hi - lo + 1),
                               hipMemcpyDeviceToHost, s));
    }
    HIP_TRY(hipStreamSynchronize(s));
    uint64_t uf = 0, ul = 0;
    if (stream_used(d, kind, steps, &uf, &ul)) d->round_last = d->round_next + ul;
    d->round_next += stream_rounds(d, kind, steps);
    d->last_profiled = d->prof_on;
    d->last_steps = steps;
    return WFST_OK;
}

static void plan_clear(wfst_decoder_s *d)
{
    std::memset(d->h_plan, 0, 4 * (size_t)d->cfg.max_lanes * kPlanFields);   // kCmdPark
}

// Opens up to n streams in one open sequence: channels[0 .. *opened) receive
// the lanes, lowest free lanes first.
static int open_lanes(wfst_decoder_s *d, int32_t n, void *stream, int32_t *channels, int32_t *opened)
{
    *opened = 0;
    if (d->w.lattice) return fail(WFST_EINVAL, "a lattice-mode decoder does not stream");
    std::lock_guard<std::mutex> lock(d->mu);
    std::vector<int> lanes;
    for (int L = 0; L < d->cfg.max_lanes && (int32_t)lanes.size() < n; ++L)
        if (!d->chan_open[(size_t)L]) lanes.push_back(L);
    if (lanes.empty()) return WFST_OK;   // every lane holds a stream
    HIP_TRY(hipSetDevice(d->g->device));
    // a stream cannot be decoded again: the whole region of each lane that
    // opens one is committed now (page section 6.2: a channel's slice at
    // CreateStream), and while streams are open the kernels' bound is the
    // whole region (only open streams' lanes append); the chunks stay mapped
    // after release, for the lane's next stream (streams wait for the device
    // before a commit, see grow_log)
    if (d->log.lim < d->w.arena || d->dev_arena_lim != d->w.arena) {
        HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
        for (int L : lanes) {
            const hipError_t e = d->log.commit_lane((uint32_t)L);
            if (e != hipSuccess) return hip_fail(e, "winners-log commit");
        }
        int rc0 = set_arena_lim(d, d->w.arena);
        if (rc0 != WFST_OK) return rc0;
    }
    plan_clear(d);
    for (int L : lanes) d->h_plan[L * kPlanFields + kPlanCmd] = kCmdOpen;
    int rc = run_stream(d, kSeqOpen, 0, (hipStream_t)stream, {});
    if (rc != WFST_OK) return rc;
    d->last_len.assign((size_t)d->cfg.max_lanes, -1);
    for (int L : lanes) {
        d->last_len[(size_t)L] = 0;
        d->chan_open[(size_t)L] = 1;
        channels[(*opened)++] = L;
    }
    d->open_streams += (int)lanes.size();
    return WFST_OK;
}

extern "C" int wfst_create_stream(wfst_decoder_t d, void *stream, int32_t *channel)
{
    if (!d || !channel) return fail(WFST_EINVAL, "decoder or channel is null");
    *channel = -1;
    int32_t opened = 0;
    return open_lanes(d, 1, stream, channel, &opened);
}

extern "C" int wfst_create_streams(wfst_decoder_t d, int32_t n, void *stream, int32_t *channels, int32_t *opened)
{
    if (!d || !channels || !opened || n < 0) return fail(WFST_EINVAL, "bad arguments");
    *opened = 0;
    if (n == 0) return WFST_OK;
    return open_lanes(d, n, stream, channels, opened);
}

extern "C" int wfst_advance_chunk(wfst_decoder_t d, const int32_t *channels, int32_t C, const void *log_prob,
                                  int32_t T, int32_t V, const int32_t *lengths_host, void *stream,
                                  int32_t want_partial, int32_t *out_words, int32_t words_cap,
                                  int32_t *out_word_lens, int32_t *out_arcs, int32_t arcs_cap,
                                  int32_t *out_arc_lens, float *out_scores, int32_t *out_meta)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    const wfst_decoder_config &c = d->cfg;
    if (C < 1 || C > c.max_lanes || !channels || !lengths_host) return fail(WFST_EINVAL, "C must lie in [1, max_lanes] with channels and lengths given");
    if (T < 0 || T > c.max_frames) return fail(WFST_EINVAL, "T (chunk frames) must lie in [0, max_frames]");
    if (V != d->g->vocab) return fail(WFST_EINVAL, "V differs from the graph's vocab_size");
    if (want_partial && (!out_word_lens || !out_arc_lens || !out_scores || !out_meta ||
                         words_cap < 0 || arcs_cap < 0 || (words_cap > 0 && !out_words) || (arcs_cap > 0 && !out_arcs)))
        return fail(WFST_EINVAL, "want_partial needs the output buffers");
    std::lock_guard<std::mutex> lock(d->mu);
    std::vector<uint8_t> seen((size_t)c.max_lanes, 0);
    int32_t steps = 0;
    for (int32_t j = 0; j < C; ++j) {
        const int32_t ch = channels[j];
        if (ch < 0 || ch >= c.max_lanes || !d->chan_open[(size_t)ch]) return fail(WFST_EINVAL, "a channel is not an open stream");
        if (seen[(size_t)ch]) return fail(WFST_EINVAL, "a channel appears twice");
        seen[(size_t)ch] = 1;
        if (lengths_host[j] < 0 || lengths_host[j] > T) return fail(WFST_EINVAL, "lengths must lie in [0, T]");
        steps = std::max(steps, lengths_host[j]);
    }
    if (steps > 0 && !log_prob) return fail(WFST_EINVAL, "log_prob is null");
    HIP_TRY(hipSetDevice(d->g->device));
    if (steps > 0) {
        const size_t elem = c.lp_dtype == WFST_LP_F16 ? 2 : 4;
        const int rcb = check_device_buffer(log_prob, (size_t)C * (size_t)T * (size_t)V * elem, d->g->device, "log_prob");
        if (rcb != WFST_OK) return rcb;
    }
    hipStream_t s = (hipStream_t)stream;
    LpDesc *hd = (LpDesc *)d->h_in;
    hd->base = log_prob;
    hd->stride_t = V;
    hd->stride_b = (long long)T * V;
    hd->B = C;
    hd->dtype = c.lp_dtype;
    HIP_TRY(hipMemcpyAsync(d->d_desc, hd, sizeof(LpDesc), hipMemcpyHostToDevice, s));
    plan_clear(d);
    std::vector<int> lanes;
    for (int32_t j = 0; j < C; ++j) {
        int32_t *pl = d->h_plan + channels[j] * kPlanFields;
        pl[kPlanCmd] = kCmdAdvance;
        pl[kPlanLen] = lengths_host[j];
        pl[kPlanRow] = j;
        pl[kPlanWant] = want_partial ? 1 : 0;
        if (want_partial) lanes.push_back(channels[j]);
    }
    int rc = run_stream(d, kSeqAdvance, steps, s, lanes);
    if (rc != WFST_OK) return rc;
    d->last_len.assign((size_t)c.max_lanes, -1);
    for (int32_t j = 0; j < C; ++j) d->last_len[(size_t)channels[j]] = lengths_host[j];
    if (want_partial)
        for (int32_t j = 0; j < C; ++j)
            copy_result(d, channels[j], j, out_words, words_cap, out_word_lens, out_arcs, arcs_cap, out_arc_lens,
                        out_scores, out_meta);
    return WFST_OK;
}

// Ends channels[0 .. C) in one finish sequence and copies each result to its row.
static int finalize_lanes(wfst_decoder_s *d, const int32_t *channels, int32_t C, void *stream, int32_t *out_words,
                          int32_t words_cap, int32_t *out_word_lens, int32_t *out_arcs, int32_t arcs_cap,
                          int32_t *out_arc_lens, float *out_scores, int32_t *out_meta)
{
    if (!out_word_lens || !out_arc_lens || !out_scores || !out_meta || words_cap < 0 || arcs_cap < 0 ||
        (words_cap > 0 && !out_words) || (arcs_cap > 0 && !out_arcs))
        return fail(WFST_EINVAL, "an output pointer is null");
    const int nl = d->cfg.max_lanes;
    if (!channels || C < 1 || C > nl) return fail(WFST_EINVAL, "C must lie in [1, max_lanes] with channels given");
    std::lock_guard<std::mutex> lock(d->mu);
    std::vector<uint8_t> seen((size_t)nl, 0);
    for (int32_t j = 0; j < C; ++j) {
        const int32_t ch = channels[j];
        if (ch < 0 || ch >= nl || !d->chan_open[(size_t)ch]) return fail(WFST_EINVAL, "channel is not an open stream");
        if (seen[(size_t)ch]) return fail(WFST_EINVAL, "a channel appears twice");
        seen[(size_t)ch] = 1;
    }
    HIP_TRY(hipSetDevice(d->g->device));
    plan_clear(d);
    std::vector<int> lanes;
    for (int32_t j = 0; j < C; ++j) {
        d->h_plan[channels[j] * kPlanFields + kPlanCmd] = kCmdFinish;
        lanes.push_back(channels[j]);
    }
    int rc = run_stream(d, kSeqFinish, 1, (hipStream_t)stream, lanes);
    if (rc != WFST_OK) return rc;
    d->last_len.assign((size_t)nl, -1);
    for (int32_t j = 0; j < C; ++j) {
        d->last_len[(size_t)channels[j]] = 0;
        copy_result(d, channels[j], j, out_words, words_cap, out_word_lens, out_arcs, arcs_cap, out_arc_lens,
                    out_scores, out_meta);
    }
    return WFST_OK;
}

extern "C" int wfst_finalize_stream(wfst_decoder_t d, int32_t channel, void *stream, int32_t *out_words,
                                    int32_t words_cap, int32_t *out_word_len, int32_t *out_arcs, int32_t arcs_cap,
                                    int32_t *out_arc_len, float *out_score, int32_t *out_meta)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    return finalize_lanes(d, &channel, 1, stream, out_words, words_cap, out_word_len, out_arcs, arcs_cap,
                          out_arc_len, out_score, out_meta);
}

extern "C" int wfst_finalize_streams(wfst_decoder_t d, const int32_t *channels, int32_t C, void *stream,
                                     int32_t *out_words, int32_t words_cap, int32_t *out_word_lens,
                                     int32_t *out_arcs, int32_t arcs_cap, int32_t *out_arc_lens, float *out_scores,
                                     int32_t *out_meta)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    return finalize_lanes(d, channels, C, stream, out_words, words_cap, out_word_lens, out_arcs, arcs_cap,
                          out_arc_lens, out_scores, out_meta);
}

extern "C" int wfst_release_stream(wfst_decoder_t d, int32_t channel)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    std::lock_guard<std::mutex> lock(d->mu);
    if (channel < 0 || channel >= d->cfg.max_lanes || !d->chan_open[(size_t)channel])
        return fail(WFST_EINVAL, "channel is not an open stream");
    d->chan_open[(size_t)channel] = 0;
    d->open_streams -= 1;
    return WFST_OK;
}

static int fetch_records(wfst_decoder_s *d, std::vector<uint32_t> *rec)
{
    const size_t per = (size_t)(d->cfg.max_frames + 2) * kStepFields;
    rec->resize(per * (size_t)d->cfg.max_lanes);
    HIP_TRY(hipSetDevice(d->g->device));
    HIP_TRY(hipMemcpy(rec->data(), d->w.steps, 4 * rec->size(), hipMemcpyDeviceToHost));
    return WFST_OK;
}

extern "C" int wfst_decoder_stats(wfst_decoder_t d, int64_t *out, int32_t n)
{
    if (!d || !out || n < 0) return fail(WFST_EINVAL, "bad arguments");
    std::lock_guard<std::mutex> lock(d->mu);
    int64_t v[17] = {0};
    bool any = false;
    for (int32_t x : d->last_len) any |= x >= 0;
    if (any) {
        std::vector<uint32_t> rec;
        int rc = fetch_records(d, &rec);
        if (rc != WFST_OK) return rc;
        const size_t per = (size_t)(d->cfg.max_frames + 2);
        for (int b = 0; b < d->cfg.max_lanes; ++b) {
            if (d->last_len[(size_t)b] < 0) continue;
            for (size_t r = 0; r < per; ++r) {
                const uint32_t *x = rec.data() + ((size_t)b * per + r) * kStepFields;
                v[0] += x[kRecArcs]; v[1] += x[kRecAdmitted]; v[2] += x[kRecDistinct]; v[3] += x[kRecN];
                v[4] += x[kRecEpsArcs]; v[5] += x[kRecEpsAdmitted]; v[6] += x[kRecEpsDistinct];
                v[7] += (int64_t)x[kRecEpsNew] + x[kRecEpsReplaced];
                v[10] = std::max<int64_t>(v[10], x[kRecN]);
                if (r >= 1 && x[kRecPhase] == (uint32_t)kPhReal && x[kRecN] > 0) v[12] += 1;
                v[13] += x[kRecListed];
            }
        }
        std::vector<LaneCtl> ctl((size_t)d->cfg.max_lanes);
        HIP_TRY(hipMemcpy(ctl.data(), d->ctl, sizeof(LaneCtl) * ctl.size(), hipMemcpyDeviceToHost));
        for (int b = 0; b < d->cfg.max_lanes; ++b)
            if (d->last_len[(size_t)b] >= 0) v[8] += ctl[(size_t)b].log_cursor;
    }
    v[9] = d->last_steps;
    v[11] = (int64_t)(d->bytes + d->log.committed_bytes() + d->g->bytes);
    v[14] = (int64_t)d->log.va_bytes;
    v[15] = (int64_t)d->log.committed_bytes();
    v[16] = d->last_regrows;
    for (int32_t i = 0; i < n && i < 17; ++i) out[i] = v[i];
    return WFST_OK;
}

extern "C" int wfst_decoder_mem_stats(wfst_decoder_t d, int64_t out[4])
{
    if (!d || !out) return fail(WFST_EINVAL, "bad arguments");
    std::lock_guard<std::mutex> lock(d->mu);
    int64_t hw = 0;
    bool any = false;
    for (int32_t x : d->last_len) any |= x >= 0;
    if (any) {
        std::vector<LaneCtl> ctl((size_t)d->cfg.max_lanes);
        HIP_TRY(hipSetDevice(d->g->device));
        HIP_TRY(hipMemcpy(ctl.data(), d->ctl, sizeof(LaneCtl) * ctl.size(), hipMemcpyDeviceToHost));
        for (int b = 0; b < d->cfg.max_lanes; ++b)
            if (d->last_len[(size_t)b] >= 0)
                hw = std::max<int64_t>(hw, std::min<int64_t>(ctl[(size_t)b].log_cursor, d->w.arena));
    }
    out[0] = (int64_t)(d->bytes + d->log.va_bytes);
    out[1] = (int64_t)(d->bytes + d->log.committed_bytes());
    out[2] = (int64_t)d->bytes;
    out[3] = hw * (int64_t)sizeof(int2);
    return WFST_OK;
}

extern "C" int wfst_decoder_step_stats(wfst_decoder_t d, int32_t lane, int64_t *out, int32_t steps_cap)
{
    if (!d || !out || steps_cap < 0) return fail(WFST_EINVAL, "bad arguments");
    std::lock_guard<std::mutex> lock(d->mu);
    if (lane < 0 || lane >= d->cfg.max_lanes || d->last_len[(size_t)lane] < 0)
        return fail(WFST_EINVAL, "lane not in the last decode or stream call");
    std::vector<uint32_t> rec;
    int rc = fetch_records(d, &rec);
    if (rc != WFST_OK) return rc;
    // the lane's last step of the call (its result header on the device)
    int32_t last = -1;
    HIP_TRY(hipMemcpy(&last, d->w.res + (size_t)d->w.res_stride * (size_t)lane + 7, 4, hipMemcpyDeviceToHost));
    const size_t per = (size_t)(d->cfg.max_frames + 2);
    const int32_t nrec = std::min<int32_t>(steps_cap, d->last_len[(size_t)lane] + 2);
    for (int32_t r = 0; r < nrec; ++r) {
        const uint32_t *x = rec.data() + ((size_t)lane * per + (size_t)r) * kStepFields;
        for (int f = 0; f < kStepFields; ++f) out[(size_t)r * kStepFields + f] = x[f];
        if (r >= 1 && r - 1 > last) out[(size_t)r * kStepFields + kRecPhase] = -1;
        if (r == 0) out[kRecPhase] = -1;
    }
    return nrec;
}

extern "C" int wfst_decoder_profile(wfst_decoder_t d, int32_t enable)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    std::lock_guard<std::mutex> lock(d->mu);
    HIP_TRY(hipSetDevice(d->g->device));
    if (enable && d->ev.empty()) {
        const size_t rounds = (size_t)(d->cfg.max_frames + 2) * (size_t)(1 + d->passes);
        const size_t n = 18 + (size_t)(d->cfg.max_frames + 2) * (size_t)(5 + 3 * d->passes + 8) + rounds / d->w.epoch_period;
        d->ev.resize(2 * n, nullptr);
        d->ev_kind.assign(n, -1);
        for (size_t i = 0; i < 2 * n; ++i) HIP_TRY(hipEventCreateWithFlags(&d->ev[i], hipEventDefault));
    }
    d->prof_on = enable != 0;
    return WFST_OK;
}

extern "C" int wfst_decoder_kernel_times(wfst_decoder_t d, double *out, int32_t n)
{
    if (!d || !out || n < 0) return fail(WFST_EINVAL, "bad arguments");
    std::lock_guard<std::mutex> lock(d->mu);
    if (!d->last_profiled) return fail(WFST_EINVAL, "the last decode was not profiled");
    HIP_TRY(hipSetDevice(d->g->device));
    std::vector<double> v(2 * kKCount, 0.0);
    for (size_t i = 0; i < d->ev_used; ++i) {
        float ms = 0.0f;
        HIP_TRY(hipEventElapsedTime(&ms, d->ev[2 * i], d->ev[2 * i + 1]));
        const int id = d->ev_kind[i];
        if (id >= 0 && id < kKCount) { v[2 * id] += ms; v[2 * id + 1] += 1.0; }
    }
    for (int32_t i = 0; i < n && i < 2 * kKCount; ++i) out[i] = v[(size_t)i];
    return WFST_OK;
}

extern "C" int wfst_lattice_records(wfst_decoder_t d, int32_t lane, int32_t *out, int64_t cap, int64_t *n)
{
    if (!d || !n || cap < 0 || (cap > 0 && !out)) return fail(WFST_EINVAL, "bad arguments");
    std::lock_guard<std::mutex> lock(d->mu);
    *n = 0;
    if (!d->w.lattice) return fail(WFST_EINVAL, "the decoder is not in lattice mode");
    if (lane < 0 || lane >= d->cfg.max_lanes || d->last_len[(size_t)lane] < 0)
        return fail(WFST_EINVAL, "lane not in the last decode");
    HIP_TRY(hipSetDevice(d->g->device));
    uint32_t kept = 0;
    HIP_TRY(hipMemcpy(&kept, (const char *)(d->ctl + lane) + offsetof(LaneCtl, lat_out_n), 4, hipMemcpyDeviceToHost));
    *n = kept;
    const int64_t m = std::min<int64_t>(std::min<int64_t>(kept, cap), (int64_t)d->w.lat_cap);
    if (m > 0)
        HIP_TRY(hipMemcpy(out, d->w.lat_out + (size_t)lane * d->w.lat_cap * kLatFields,
                          4 * (size_t)m * kLatFields, hipMemcpyDeviceToHost));
    return WFST_OK;
}

extern "C" int wfst_blank_skip(wfst_decoder_t d, const void *log_prob, int32_t B, int32_t T, int32_t V,
                               const int32_t *lengths_host, int32_t blank_id, float threshold, void *out_log_prob,
                               int32_t *out_lengths_host, void *stream)
{
    if (!d) return fail(WFST_EINVAL, "decoder is null");
    const wfst_decoder_config &c = d->cfg;
    if (B < 1 || B > c.max_lanes) return fail(WFST_EINVAL, "B must lie in [1, max_lanes]");
    if (T < 0 || T > c.max_frames) return fail(WFST_EINVAL, "T must lie in [0, max_frames]");
    if (V != d->g->vocab) return fail(WFST_EINVAL, "V differs from the graph's vocab_size");
    if (blank_id < 0 || blank_id >= V) return fail(WFST_EINVAL, "blank_id must lie in [0, V)");
    if (!(threshold > 0.0f) || std::isinf(threshold)) return fail(WFST_EINVAL, "threshold must be positive and finite");
    if (!lengths_host || !out_lengths_host || (T > 0 && (!log_prob || !out_log_prob)))
        return fail(WFST_EINVAL, "a pointer is null");
    if (T > 0 && out_log_prob == log_prob) return fail(WFST_EINVAL, "out_log_prob must not alias log_prob");
    for (int32_t b = 0; b < B; ++b)
        if (lengths_host[b] < 0 || lengths_host[b] > T) return fail(WFST_EINVAL, "lengths must lie in [0, T]");
    std::lock_guard<std::mutex> lock(d->mu);
    HIP_TRY(hipSetDevice(d->g->device));
    if (T > 0) {
        const size_t nb = (size_t)B * (size_t)T * (size_t)V * (c.lp_dtype == WFST_LP_F16 ? 2 : 4);
        int rcb = check_device_buffer(log_prob, nb, d->g->device, "log_prob");
        if (rcb == WFST_OK) rcb = check_device_buffer(out_log_prob, nb, d->g->device, "out_log_prob");
        if (rcb != WFST_OK) return rcb;
    }
    hipStream_t s = (hipStream_t)stream;
    const size_t L = (size_t)c.max_lanes;
    LpDesc *hd = (LpDesc *)d->h_in;
    hd->base = log_prob;
    hd->stride_t = V;
    hd->stride_b = (long long)T * V;
    hd->B = B;
    hd->dtype = c.lp_dtype;
    int32_t *hl = (int32_t *)((char *)d->h_in + sizeof(LpDesc));
    for (size_t b = 0; b < L; ++b) hl[b] = (int32_t)b < B ? lengths_host[b] : 0;
    HIP_TRY(hipMemcpyAsync(d->d_desc, hd, sizeof(LpDesc), hipMemcpyHostToDevice, s));
    HIP_TRY(hipMemcpyAsync(d->d_lengths, hl, 4 * L, hipMemcpyHostToDevice, s));
    if (T > 0) {
        // the threshold as a log-probability, rounded once to binary32
        const float lthr = (float)std::log((double)threshold);
        HIP_TRY(launch_blank_skip(d->w, d->d_work, out_log_prob, lthr, blank_id, B, T, d->grid, s));
        HIP_TRY(hipMemcpyAsync(out_lengths_host, d->w.bs_len, 4 * (size_t)B, hipMemcpyDeviceToHost, s));
    } else {
        for (int32_t b = 0; b < B; ++b) out_lengths_host[b] = 0;
    }
    HIP_TRY(hipStreamSynchronize(s));
    return WFST_OK;
}
