// glue.hip -- row re-normalisation and SwiGLU between the linears of a decode
// step (fp16 in/out, fp32 math, one workgroup per row, fixed reduction order).
//
// The pages give no glue; the step chains the linears with
//   rn(v)      = v / sqrt(mean(v^2) + 1e-6)   per row
//   swiglu(gu) = silu(gu[:, :I]) * gu[:, I:],  silu(x) = x / (1 + exp(-x))
// and stores each intermediate as fp16.
//
// A row is at most kThreads * 8 * kMaxVec fp16 values.  Each thread issues all
// of its 16-byte loads before using any of them, keeps the row in registers
// through the reduction and writes it back from there, so a launch costs one
// HBM/L2 round trip for the loads and one for the stores rather than one per
// element.
#include "device.h"
#include "kernels.h"

namespace w4a16 {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Sum over the workgroup: a lane-xor butterfly inside each wave (wave_sum),
// then every thread adds the per-wave sums in wave order (the same order in
// every thread and run).
__device__ __forceinline__ float block_sum(float v, float *sh) {
    v = wave_sum(v, threadIdx.x & 63);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += sh[w];
    return s;
}

__device__ __forceinline__ float lane_f32(const u32x4 &v, int e) {
    return f16_bits_to_f32((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
}

__device__ __forceinline__ u32x4 load16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ void store_scaled(uint16_t *p, const float (&t)[8], float inv) {
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = scaled_f16(t[2 * w], inv) | (scaled_f16(t[2 * w + 1], inv) << 16);
    *reinterpret_cast<u32x4 *>(p) = o;
}

// y[m][0..width) = rn(x[m][0..width)), x row stride ldx; V 16-byte vectors
// per thread (width <= 8 * kThreads * V, width % 8 == 0).
template <int V>
__global__ __launch_bounds__(kThreads) void rownorm_kernel(const uint16_t *__restrict__ x, int ldx,
                                                           int width, uint16_t *__restrict__ y) {
    __shared__ float sh[kWaves];
    const uint16_t *xr = x + (size_t)blockIdx.x * ldx;
    const int nvec = width >> 3;
    u32x4 v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int i = threadIdx.x + j * kThreads;
        v[j] = i < nvec ? load16(xr + 8 * i) : u32x4{0u, 0u, 0u, 0u};
    }
    float ss = 0.f;
    float t[V][8];
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            t[j][e] = lane_f32(v[j], e);
            ss = __builtin_fmaf(t[j][e], t[j][e], ss);
        }
    const float tot = block_sum(ss, sh);
    const float inv = row_inv(tot, width);
    uint16_t *yr = y + (size_t)blockIdx.x * width;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < nvec) store_scaled(yr + 8 * i, t[j], inv);
    }
}

// y[m][i] = rn_row(silu(gu[m][i]) * gu[m][I + i]), gu rows ld >= 2I elements
// apart; same vector layout as rownorm_kernel over the I outputs.
template <int V>
__global__ __launch_bounds__(kThreads) void swiglu_rownorm_kernel(const uint16_t *__restrict__ gu, int ld,
                                                                  int I, uint16_t *__restrict__ y) {
    __shared__ float sh[kWaves];
    const uint16_t *gr = gu + (size_t)blockIdx.x * ld;
    const int nvec = I >> 3;
    u32x4 g[V], u[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int i = threadIdx.x + j * kThreads;
        const bool in = i < nvec;
        g[j] = in ? load16(gr + 8 * i) : u32x4{0u, 0u, 0u, 0u};
        u[j] = in ? load16(gr + I + 8 * i) : u32x4{0u, 0u, 0u, 0u};
    }
    float ss = 0.f;
    float t[V][8];
#pragma unroll
    for (int j = 0; j < V; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            t[j][e] = silu_mul(lane_f32(g[j], e), lane_f32(u[j], e));
            ss = __builtin_fmaf(t[j][e], t[j][e], ss);
        }
    const float tot = block_sum(ss, sh);
    const float inv = row_inv(tot, I);
    uint16_t *yr = y + (size_t)blockIdx.x * I;
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < nvec) store_scaled(yr + 8 * i, t[j], inv);
    }
}

int vectors_per_thread(int64_t width) {
    const int64_t per = (width / 8 + kThreads - 1) / kThreads;
    return per <= 1 ? 1 : per <= 2 ? 2 : 4;
}

}  // namespace

hipError_t launch_rownorm(const uint16_t *x, int64_t M, int64_t ldx, int64_t width, uint16_t *y,
                          hipStream_t stream) {
    if (width % 8 != 0 || ldx % 8 != 0 || width > kGlueMaxWidth) return hipErrorInvalidValue;
    const dim3 grid((unsigned)M), block(kThreads);
    switch (vectors_per_thread(width)) {
        case 1: hipLaunchKernelGGL(rownorm_kernel<1>, grid, block, 0, stream, x, (int)ldx, (int)width, y); break;
        case 2: hipLaunchKernelGGL(rownorm_kernel<2>, grid, block, 0, stream, x, (int)ldx, (int)width, y); break;
        default: hipLaunchKernelGGL(rownorm_kernel<4>, grid, block, 0, stream, x, (int)ldx, (int)width, y); break;
    }
    return hipGetLastError();
}

hipError_t launch_swiglu_rownorm(const uint16_t *gu, int64_t M, int64_t ld, int64_t I, uint16_t *y,
                                 hipStream_t stream) {
    if (I % 8 != 0 || ld % 8 != 0 || ld < 2 * I || I > kGlueMaxWidth) return hipErrorInvalidValue;
    const dim3 grid((unsigned)M), block(kThreads);
    switch (vectors_per_thread(I)) {
        case 1: hipLaunchKernelGGL(swiglu_rownorm_kernel<1>, grid, block, 0, stream, gu, (int)ld, (int)I, y); break;
        case 2: hipLaunchKernelGGL(swiglu_rownorm_kernel<2>, grid, block, 0, stream, gu, (int)ld, (int)I, y); break;
        default: hipLaunchKernelGGL(swiglu_rownorm_kernel<4>, grid, block, 0, stream, gu, (int)ld, (int)I, y); break;
    }
    return hipGetLastError();
}

}  // namespace w4a16
