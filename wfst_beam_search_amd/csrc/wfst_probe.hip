// Machine probes for the decoder's roofline discussion: what one MI355X gives
// to the access shapes the search is made of. Not part of the decoder (a
// separate library, libwfst_probe.so, run by bench.py --probe):
//   - random 4-byte gathers (four independent loads per lane) over footprints
//     from 4 MiB to 4 GiB: lines per second where nothing is reused;
//   - dependent load chains (x = a[x]): the latency of one level;
//   - posted 64-bit atomicMax on random slots of a small and a large table;
//   - the launch floor: empty kernels back to back, eager and replayed from a
//     captured graph.
// Every index is masked into its array; every kernel is a plain grid with no
// waits between workgroups.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

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
//   launch floor: us per empty launch eager, us per empty launch in a graph replay.
// Returns 0 on success, 1 on a HIP error, 2 if n is too small (n >= 24).
extern "C" int wfst_probe_run(double *out, int n)
{
    if (!out || n < 24) return 2;
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
    PCK(hipEventDestroy(e0));
    PCK(hipEventDestroy(e1));
    PCK(hipStreamDestroy(s));
    PCK(hipFree(slots));
    PCK(hipFree(sink));
    PCK(hipFree(a));
    return 0;
}
