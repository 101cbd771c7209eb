// Device scratch of the allocation-free decode (wfst_decode_noalloc): one
// file-scope array per device, of a fixed size, that every such call carves
// its whole workspace from. The array is held by each device the library's
// code object is loaded on until the process ends.
//
// Host code never takes the array's name as a device address: its address on a
// device is looked up once, with that device current, by hipGetSymbolAddress,
// and kept per device; kernels and copies receive that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wfst_internal.h"

namespace wfst {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_lookup_mu;
void *g_scratch_ptr[kMaxDevices];      // address of `scratch` on each device (null: not looked up)
std::mutex g_call_mu[kMaxDevices];     // one allocation-free call at a time per device

}  // namespace

hipError_t scratch_region(int device, void **ptr)
{
    *ptr = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_lookup_mu);
    if (!g_scratch_ptr[device]) {
        // the caller has made `device` current
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    return hipSuccess;
}

std::mutex &scratch_call_mutex(int device) { return g_call_mu[device]; }

// Writes a call's Work, log-prob descriptor and lengths into its scratch
// buffers from kernel arguments (no host staging buffer is needed).
struct NoallocLens {
    int32_t v[kMaxLanes];
};

__global__ __launch_bounds__(kWave) void k_noalloc_put(Work w, LpDesc d, NoallocLens lens, Work *dw, LpDesc *dd,
                                                       int32_t *dl, int n)
{
    const int i = (int)threadIdx.x;
    if (i < n) dl[i] = lens.v[i];
    if (i == 0) {
        *dw = w;
        *dd = d;
    }
}

hipError_t launch_noalloc_put(const Work &w, const LpDesc &d, const int32_t *lengths, int n, Work *dw, LpDesc *dd,
                              int32_t *dl, hipStream_t s)
{
    if (n < 0 || n > kMaxLanes) return hipErrorInvalidValue;
    NoallocLens lens{};
    for (int i = 0; i < n; ++i) lens.v[i] = lengths[i];
    hipLaunchKernelGGL(k_noalloc_put, dim3(1), dim3(kWave), 0, s, w, d, lens, dw, dd, dl, n);
    return hipGetLastError();
}

}  // namespace wfst
