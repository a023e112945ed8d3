// noalloc.hip -- split-K scratch of the allocation-free GEMM entry point
// (w4a16_gemm_noalloc): a fixed device array instead of library allocations.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy from module load until the process ends.  In
// host code its name is only a stand-in: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// is the only handle host code passes on.  The first region holds the
// zero-initialised counters and fixed-point slots (cleared by a fill kernel
// at set-up, and left zero by the last arrival of every call), the second the
// fp32 split partials.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace w4a16 {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocCounterBytes + kNoAllocPartialBytes];

__global__ __launch_bounds__(256) void zero_words(uint32_t *__restrict__ p, uint32_t n) {
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, uint32_t **counters, float **partials) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        // counters and slots must start at zero; a kernel, not a memset, so a
        // first call made under graph capture records a plain kernel node
        const uint32_t words = kNoAllocCounterBytes / 4;
        hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, stream, static_cast<uint32_t *>(ptr), words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_ptr[dev] = ptr;
    }
    *counters = static_cast<uint32_t *>(g_ptr[dev]);
    *partials = reinterpret_cast<float *>(static_cast<uint8_t *>(g_ptr[dev]) + kNoAllocCounterBytes);
    return hipSuccess;
}

}  // namespace w4a16
