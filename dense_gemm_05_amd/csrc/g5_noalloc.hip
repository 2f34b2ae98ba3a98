// g5_noalloc.hip -- the library's own scratch memory for gemm_run_noalloc,
// the entry point for callers that cannot allocate a workspace: a
// file-scope device array of kScratchBytes, one copy per GPU the library
// runs on (it lives until the process ends), shared by every such call on
// that GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "g5_kernels.h"

namespace g5 {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[64];   // device address of `scratch` on each device, once looked up
}  // namespace

// Device address of this GPU's copy of `scratch` (the current device's),
// looked up once per device with that device current.  In host code the
// array's name is only a stand-in for the symbol; its device address comes
// from hipGetSymbolAddress, and only that address is ever passed to a kernel.
hipError_t noalloc_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// Zero n arrival counters (a fill kernel rather than a memset, so that the
// call stays correct when a caller records it into a HIP graph).
__global__ void __launch_bounds__(256) k_clear_counters(unsigned *c, int n)
{
    for (int i = threadIdx.x + blockIdx.x * 256; i < n; i += 256 * gridDim.x) c[i] = 0u;
}

hipError_t launch_clear_counters(void *base, int64_t n, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int blocks = (int)((n + 255) / 256 < 64 ? (n + 255) / 256 : 64);
    hipLaunchKernelGGL(k_clear_counters, dim3(blocks), dim3(256), 0, s, (unsigned *)base, (int)n);
    return hipGetLastError();
}

}  // namespace g5
