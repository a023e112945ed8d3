// repack.hip -- checkpoint layout [N, K/8] -> kernel layout [K, N/8] (gfx950).
//
// vLLM PR #37352 write-up, "Code analysis" item 2: the compressed-tensors
// weight is packed along K ([N, K//8]); the GEMM wants it packed along N
// ([K, N//8]).  Element (k, n) sits at nibble k%8 of source word (n, k/8) and
// must land at nibble n%8 of destination word (k, n/8).  Bit-exact.
//
// Work unit: an 8x8 nibble block = source words (8*nb + i, kb), i = 0..7, and
// destination words (8*kb + j, nb), j = 0..7; it is an 8x8 transpose of 4-bit
// elements, done in registers with three rounds of masked block swaps (16-,
// 8- and 4-bit blocks; the recursive bit-matrix transpose of Warren,
// "Hacker's Delight", section 7-3, at nibble granularity).
//
// A workgroup covers 32x32 blocks (256 rows of K x 256 columns of N).  Loads
// put consecutive lanes on consecutive kb, so each load instruction reads
// whole 128-byte source row segments.  Results go through LDS with an XOR
// swizzle (column nb ^ kb) that keeps both the scattered block writes and the
// row-wise read-back conflict-free, and leave as 128-byte destination rows.
// Every word is read once and written once: both use the non-temporal cache
// policy (measured on MI355X: 15.6 -> 13.0 us at K = 4096, N = 12800).
#include "device.h"
#include "kernels.h"

namespace w4a16 {
namespace {

constexpr int kBlk = 32;  // blocks per tile edge

__device__ __forceinline__ void swap_masked(uint32_t &x, uint32_t &y, int shift, uint32_t mask) {
    const uint32_t t = ((x >> shift) ^ y) & mask;
    x ^= t << shift;
    y ^= t;
}

// In: w[i] holds row i of an 8x8 nibble matrix (element (i, j) at nibble j).
// Out: w[j] holds column j (element (i, j) at nibble i).
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t (&w)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) swap_masked(w[i], w[i + 4], 16, 0x0000FFFFu);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if ((i & 2) == 0) swap_masked(w[i], w[i + 2], 8, 0x00FF00FFu);
#pragma unroll
    for (int i = 0; i < 8; i += 2) swap_masked(w[i], w[i + 1], 4, 0x0F0F0F0Fu);
}

__global__ __launch_bounds__(256) void repack_kernel(const uint32_t *__restrict__ src,
                                                     uint32_t *__restrict__ dst, int K8, int N8) {
    // src: [N][K8] words, dst: [K][N8] words (K8 = K/8, N8 = N/8).
    __shared__ uint32_t tile[8 * kBlk][kBlk];  // destination rows x destination words (swizzled)
    const int tid = threadIdx.x;
    const int kb_local = tid & 31;
    const int kb = blockIdx.x * kBlk + kb_local;
    const int nb0 = blockIdx.y * kBlk;

#pragma unroll
    for (int r = 0; r < kBlk / 8; ++r) {
        const int nb_local = (tid >> 5) + 8 * r;
        const int nb = nb0 + nb_local;
        uint32_t w[8];
        if (kb < K8 && nb < N8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = __builtin_nontemporal_load(&src[(size_t)(8 * nb + i) * K8 + kb]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = 0u;
        }
        transpose8x8_nibbles(w);
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[8 * kb_local + j][nb_local ^ kb_local] = w[j];
    }
    __syncthreads();

    // Write back: one destination row of 32 words per 32 lanes.
    const int kb0 = blockIdx.x * kBlk;
#pragma unroll 4
    for (int it = 0; it < (8 * kBlk * kBlk) / 256; ++it) {
        const int row = it * 8 + (tid >> 5);  // 0 .. 255
        const int phys = tid & 31;
        const int nb_local = phys ^ (row >> 3);
        const int k = 8 * kb0 + row;
        const int nb = nb0 + nb_local;
        if (k < 8 * K8 && nb < N8) __builtin_nontemporal_store(tile[row][phys], &dst[(size_t)k * N8 + nb]);
    }
}

// Group scales, checkpoint [N, G_n] -> kernel [G_n, N] (G_n = K/G groups): a
// transpose of 16-bit values through a 64 x 64 LDS tile, so that the reads
// (along a checkpoint row) and the writes (along a kernel row) both take 64
// consecutive values per wave.  Tiles are numbered along G_n first in a 1-D
// grid.  Bit-exact.
constexpr int kTr = 64;

__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t *__restrict__ src,
                                                          uint16_t *__restrict__ dst, int rows, int cols,
                                                          int tiles_c) {
    __shared__ uint16_t tile[kTr][kTr + 2];
    const int tc = blockIdx.x % tiles_c, tr = blockIdx.x / tiles_c;
    const int c0 = tc * kTr, r0 = tr * kTr;
    const int tx = threadIdx.x & (kTr - 1), ty = threadIdx.x / kTr;  // 64 x 4 threads
    for (int i = ty; i < kTr; i += 256 / kTr) {
        const int r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < kTr; i += 256 / kTr) {
        const int c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) dst[(size_t)c * rows + r] = tile[tx][i];
    }
}

}  // namespace

hipError_t launch_repack_scales(const uint16_t *src, uint16_t *dst, int64_t Gn, int64_t N, hipStream_t stream) {
    const int tiles_c = (int)((Gn + kTr - 1) / kTr);
    const int64_t blocks = (int64_t)tiles_c * ((N + kTr - 1) / kTr);
    hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, (int)N, (int)Gn,
                       tiles_c);
    return hipGetLastError();
}

hipError_t launch_repack(const int32_t *src, int32_t *dst, int64_t K, int64_t N, hipStream_t stream) {
    const int K8 = (int)(K / 8), N8 = (int)(N / 8);
    dim3 grid((unsigned)((K8 + kBlk - 1) / kBlk), (unsigned)((N8 + kBlk - 1) / kBlk), 1);
    hipLaunchKernelGGL(repack_kernel, grid, dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t *>(src), reinterpret_cast<uint32_t *>(dst), K8, N8);
    return hipGetLastError();
}

}  // namespace w4a16
