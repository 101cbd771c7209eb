// Machine probes for the decoder's roofline discussion: what one MI355X gives
// to the access shapes the search is made of. Not part of the decoder (a
// separate library, libwfst_probe.so, run by bench.py --probe):
//   - random 4-byte gathers (four independent loads per lane) over footprints
//     from 4 MiB to 4 GiB: lines per second where nothing is reused;
//   - dependent load chains (x = a[x]): the latency of one level;
//   - posted 64-bit atomicMax on random slots of a small and a large table;
//   - the launch floor: empty kernels back to back, eager and replayed from a
//     captured graph;
//   - hot counters: one returning 64-bit atomicAdd per wavefront on few
//     addresses (as per-lane counters are), timed inside the kernel.
// Every index is masked into its array; every kernel is a plain grid with no
// waits between workgroups.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

namespace {

__device__ __forceinline__ uint32_t mix(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(256) void p_fill(uint32_t *a, uint32_t n)
{
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) a[i] = mix(i * 2654435761u + 7u);
}

// four independent random dword loads per lane over [0, mask]
__global__ __launch_bounds__(256) void p_gather4(const uint32_t *a, uint32_t mask, uint32_t seed, uint32_t *out)
{
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = a[mix(gid * 4u + (uint32_t)k + seed) & mask];
    const uint32_t s = v[0] + v[1] + v[2] + v[3];
    if (s == 0x12345678u) out[gid] = s;
}

// a dependent chain of D loads per lane
template <int D>
__global__ __launch_bounds__(256) void p_chain(const uint32_t *a, uint32_t mask, uint32_t seed, uint32_t *out)
{
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    uint32_t x = mix(gid + seed) & mask;
#pragma unroll
    for (int d = 0; d < D; ++d) x = a[x] & mask;
    if (x == 0x12345678u) out[gid] = x;
}

// one posted u64 atomicMax per lane on a random slot of [0, nslots) (nslots a power of 2)
__global__ __launch_bounds__(256) void p_atomic_max(unsigned long long *slots, uint32_t mask, uint32_t seed)
{
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    atomicMax(&slots[mix(gid + seed) & mask], (unsigned long long)gid * 7u + seed);
}

// one returning u64 atomicAdd per wavefront (lane 0) on counter (wave % nctr),
// counters 256 bytes apart; each wavefront records the wall-clock ticks its
// atomic took (out[3 * wave]), its start tick and the value the atomic returned
__global__ __launch_bounds__(256) void p_hot(unsigned long long *ctr, unsigned long long *out, uint32_t nctr)
{
    const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) / 64u;
    const unsigned long long t0 = wall_clock64();
    unsigned long long v = 0;
    if ((threadIdx.x & 63u) == 0u) v = atomicAdd(&ctr[(size_t)(wave % nctr) * 32u], 1ull);
    v = __shfl(v, 0, 64);
    const unsigned long long t1 = wall_clock64();
    if ((threadIdx.x & 63u) == 0u) {
        out[3 * (size_t)wave] = t1 - t0;
        out[3 * (size_t)wave + 1] = t0;
        out[3 * (size_t)wave + 2] = v;
    }
}

__global__ __launch_bounds__(64) void p_empty(uint32_t *out)
{
    if (threadIdx.x == 1000u) out[0] = 1u;
}

#define PCK(x)                                                                                   \
    do {                                                                                         \
        const hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                                  \
            fprintf(stderr, "wfst_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
            return 1;                                                                            \
        }                                                                                        \
    } while (0)

}  // namespace

// Runs every probe on the current device. out (n doubles) receives, in order:
//   for each footprint of 4, 32, 128, 512, 1024, 4096 MiB (6 x 3 values):
//     microseconds per gather launch (262144 lanes x 4 loads), G random lines/s,
//     microseconds per chain level (chain of 4 minus chain of 1, over 3);
//   posted atomicMax on 8 MiB of slots: us per launch (262144 atomics), G atomics/s;
//   the same on 512 MiB;
//   launch floor: us per empty launch eager, us per empty launch in a graph replay;
//   hot counters, 4096 wavefronts on 1, 8, 32 and 4096 counters (4 x 2 values):
//     mean and largest latency of the wavefronts' returning atomics (us).
// Returns 0 on success, 1 on a HIP error, 2 if n is too small (n >= 32).
extern "C" int wfst_probe_run(double *out, int n)
{
    if (!out || n < 32) return 2;
    const size_t maxb = (size_t)4 << 30;
    uint32_t *a = nullptr, *sink = nullptr;
    unsigned long long *slots = nullptr;
    PCK(hipMalloc(&a, maxb));
    PCK(hipMalloc(&sink, (size_t)1024 * 256 * 4));
    PCK(hipMalloc(&slots, (size_t)512 << 20));
    PCK(hipMemset(slots, 0, (size_t)512 << 20));
    p_fill<<<4096, 256>>>(a, (uint32_t)(maxb / 4));
    PCK(hipGetLastError());
    PCK(hipDeviceSynchronize());
    hipStream_t s;
    PCK(hipStreamCreate(&s));
    hipEvent_t e0, e1;
    PCK(hipEventCreate(&e0));
    PCK(hipEventCreate(&e1));
    const int reps = 20;
    const uint32_t G = 1024;
    const double lanes = (double)G * 256.0;
    auto timeit = [&](auto f) -> double {
        f(0u);
        (void)hipStreamSynchronize(s);
        (void)hipEventRecord(e0, s);
        for (int i = 0; i < reps; ++i) f((uint32_t)(i + 1) * 977u);
        (void)hipEventRecord(e1, s);
        (void)hipEventSynchronize(e1);
        float ms = 0.0f;
        (void)hipEventElapsedTime(&ms, e0, e1);
        return (double)ms * 1000.0 / reps;
    };
    int o = 0;
    for (size_t mb : {4, 32, 128, 512, 1024, 4096}) {
        const uint32_t mask = (uint32_t)(mb * 1024 * 1024 / 4 - 1);
        const double g = timeit([&](uint32_t sd) { p_gather4<<<G, 256, 0, s>>>(a, mask, sd, sink); });
        const double c1 = timeit([&](uint32_t sd) { p_chain<1><<<G, 256, 0, s>>>(a, mask, sd, sink); });
        const double c4 = timeit([&](uint32_t sd) { p_chain<4><<<G, 256, 0, s>>>(a, mask, sd, sink); });
        out[o++] = g;
        out[o++] = lanes * 4.0 / (g * 1e3);
        out[o++] = (c4 - c1) / 3.0;
    }
    for (size_t mb : {8, 512}) {
        const uint32_t mask = (uint32_t)(mb * 1024 * 1024 / 8 - 1);
        const double t = timeit([&](uint32_t sd) { p_atomic_max<<<G, 256, 0, s>>>(slots, mask, sd); });
        out[o++] = t;
        out[o++] = lanes / (t * 1e3);
    }
    PCK(hipGetLastError());
    // launch floor: 1000 empty launches, eager and from a captured graph
    const int nl = 1000;
    {
        p_empty<<<1, 64, 0, s>>>(sink);
        PCK(hipStreamSynchronize(s));
        PCK(hipEventRecord(e0, s));
        for (int i = 0; i < nl; ++i) p_empty<<<1, 64, 0, s>>>(sink);
        PCK(hipEventRecord(e1, s));
        PCK(hipEventSynchronize(e1));
        float ms = 0.0f;
        PCK(hipEventElapsedTime(&ms, e0, e1));
        out[o++] = (double)ms * 1000.0 / nl;
    }
    {
        hipGraph_t gr;
        hipGraphExec_t ge;
        PCK(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
        for (int i = 0; i < nl; ++i) p_empty<<<1, 64, 0, s>>>(sink);
        PCK(hipStreamEndCapture(s, &gr));
        PCK(hipGraphInstantiate(&ge, gr, nullptr, nullptr, 0));
        PCK(hipGraphLaunch(ge, s));
        PCK(hipStreamSynchronize(s));
        PCK(hipEventRecord(e0, s));
        PCK(hipGraphLaunch(ge, s));
        PCK(hipEventRecord(e1, s));
        PCK(hipEventSynchronize(e1));
        float ms = 0.0f;
        PCK(hipEventElapsedTime(&ms, e0, e1));
        out[o++] = (double)ms * 1000.0 / nl;
        PCK(hipGraphExecDestroy(ge));
        PCK(hipGraphDestroy(gr));
    }
    {
        // hot counters: 1024 workgroups of 4 wavefronts, one atomic each
        const uint32_t nw = G * 4u;
        unsigned long long *ctr = nullptr, *lat = nullptr;
        PCK(hipMalloc(&ctr, (size_t)4096 * 32 * 8));
        PCK(hipMalloc(&lat, (size_t)nw * 3 * 8));
        PCK(hipMemset(ctr, 0, (size_t)4096 * 32 * 8));
        int khz = 0;
        PCK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, 0));
        const double us_per_tick = khz > 0 ? 1000.0 / (double)khz : 0.01;
        unsigned long long *h = (unsigned long long *)malloc((size_t)nw * 3 * 8);
        if (!h) return 1;
        for (uint32_t nc : {1u, 8u, 32u, 4096u}) {
            for (int r = 0; r < 3; ++r) p_hot<<<G, 256, 0, s>>>(ctr, lat, nc);
            PCK(hipGetLastError());
            PCK(hipStreamSynchronize(s));
            PCK(hipMemcpy(h, lat, (size_t)nw * 3 * 8, hipMemcpyDeviceToHost));
            double sum = 0.0, mx = 0.0;
            for (uint32_t wv = 0; wv < nw; ++wv) {
                const double d = (double)h[3 * (size_t)wv] * us_per_tick;
                sum += d;
                if (d > mx) mx = d;
            }
            out[o++] = sum / nw;
            out[o++] = mx;
        }
        free(h);
        PCK(hipFree(lat));
        PCK(hipFree(ctr));
    }
    PCK(hipEventDestroy(e0));
    PCK(hipEventDestroy(e1));
    PCK(hipStreamDestroy(s));
    PCK(hipFree(slots));
    PCK(hipFree(sink));
    PCK(hipFree(a));
    return 0;
}
