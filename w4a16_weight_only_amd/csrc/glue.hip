// glue.hip -- row re-normalisation and SwiGLU between the linears of a decode
// step (fp16 in/out, fp32 math, one workgroup per row, fixed reduction order).
//
// The pages give no glue; the step chains the linears with
//   rn(v)      = v / sqrt(mean(v^2) + 1e-6)   per row
//   swiglu(gu) = silu(gu[:, :I]) * gu[:, I:],  silu(x) = x / (1 + exp(-x))
// and stores each intermediate as fp16.
#include "device.h"
#include "kernels.h"

namespace w4a16 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum(float v, float *sh) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) s += sh[w];
    return s;
}

__device__ __forceinline__ float load_f16(const uint16_t *p) { return f16_bits_to_f32(*p); }

__global__ __launch_bounds__(kThreads) void rownorm_kernel(const uint16_t *__restrict__ x, int ldx,
                                                           int width, uint16_t *__restrict__ y) {
    __shared__ float sh[kThreads / 64];
    const uint16_t *xr = x + (size_t)blockIdx.x * ldx;
    float ss = 0.f;
    for (int j = threadIdx.x; j < width; j += kThreads) {
        const float v = load_f16(xr + j);
        ss = __builtin_fmaf(v, v, ss);
    }
    const float tot = block_sum(ss, sh);
    const float inv = 1.0f / sqrtf(tot / (float)width + 1e-6f);
    uint16_t *yr = y + (size_t)blockIdx.x * width;
    for (int j = threadIdx.x; j < width; j += kThreads) yr[j] = f32_to_f16_bits(load_f16(xr + j) * inv);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__global__ __launch_bounds__(kThreads) void swiglu_rownorm_kernel(const uint16_t *__restrict__ gu,
                                                                  int I, uint16_t *__restrict__ y) {
    __shared__ float sh[kThreads / 64];
    const uint16_t *gr = gu + (size_t)blockIdx.x * 2 * I;
    float ss = 0.f;
    for (int i = threadIdx.x; i < I; i += kThreads) {
        const float t = silu_mul(load_f16(gr + i), load_f16(gr + I + i));
        ss = __builtin_fmaf(t, t, ss);
    }
    const float tot = block_sum(ss, sh);
    const float inv = 1.0f / sqrtf(tot / (float)I + 1e-6f);
    uint16_t *yr = y + (size_t)blockIdx.x * I;
    for (int i = threadIdx.x; i < I; i += kThreads)
        yr[i] = f32_to_f16_bits(silu_mul(load_f16(gr + i), load_f16(gr + I + i)) * inv);
}

}  // namespace

hipError_t launch_rownorm(const uint16_t *x, int64_t M, int64_t ldx, int64_t width, uint16_t *y,
                          hipStream_t stream) {
    hipLaunchKernelGGL(rownorm_kernel, dim3((unsigned)M), dim3(kThreads), 0, stream, x, (int)ldx,
                       (int)width, y);
    return hipGetLastError();
}

hipError_t launch_swiglu_rownorm(const uint16_t *gu, int64_t M, int64_t I, uint16_t *y,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(swiglu_rownorm_kernel, dim3((unsigned)M), dim3(kThreads), 0, stream, gu,
                       (int)I, y);
    return hipGetLastError();
}

}  // namespace w4a16
