// gemm_mfma.hip -- W4A16 GEMM for M >= 9 on the CDNA4 matrix cores (gfx950).
//
// out = a . ((q - z) * s)  (vLLM PR #37352 write-up, "Code analysis" item 1),
// computed with v_mfma_f32_16x16x32_f16: fp16 operands, fp32 accumulation.
//
// Operand mapping.  In a 16x16x32 MFMA each lane supplies 8 consecutive k of
// one row of A (lane%16 = row, lane/16 = which 8-k slice) and 8 consecutive k
// of one column of B.  The packed weight word holds 8 *columns* of one row, so
// a lane loads the same word index from 8 consecutive rows (a column of words)
// and, for each nibble position t = 0..7, forms the B operand of a different
// MFMA column tile: tile t's column j is matrix column 8*(word0 + j) + t.  The
// dequantised weights therefore never leave registers -- no LDS round trip and
// no transpose -- and lane j of every tile owns 8 adjacent output columns, so
// the epilogue stores 16 contiguous bytes per row.  Dequantisation is
// (q - z) exact in fp16 (device.h), times the group scale rounded to fp16.
//
// A wave computes (16*MT rows) x (128 columns) over its K-split; NWN waves side
// by side make a workgroup read whole 128-byte weight lines.  K-splits across
// workgroups meet in an fp32 partials buffer; the last workgroup to arrive at a
// tile's counter sums them in split order (deterministic) and resets it.
#include "device.h"
#include "kernels.h"

namespace w4a16 {
namespace {

// Dequantise the 8 B operands (one per nibble position) from the 8 words of
// rows k0+8*kq .. +7 of one packed column-of-words.
template <int B>
__device__ __forceinline__ void dequant_byte(const uint32_t (&wd)[8], const f16x2 (&zc)[8],
                                             const f16x2 (&sp)[8], f16x8 (&bop)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t pr = gather_byte_pair<B>(wd[2 * j], wd[2 * j + 1]);
        const f16x2 v0 = (as_f16x2(biased_pair<0>(pr)) - zc[2 * B]) * sp[2 * B];
        const f16x2 v1 = (as_f16x2(biased_pair<1>(pr)) - zc[2 * B + 1]) * sp[2 * B + 1];
        bop[2 * B][2 * j] = v0.x;
        bop[2 * B][2 * j + 1] = v0.y;
        bop[2 * B + 1][2 * j] = v1.x;
        bop[2 * B + 1][2 * j + 1] = v1.y;
    }
}

template <int MT, int NWN, bool ASYM>
__global__ __launch_bounds__(64 * NWN) void mfma_kernel(
    const uint16_t *__restrict__ a, const uint32_t *__restrict__ b,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros, int M, int K, int N,
    int G, uint32_t zp, int split_len, int splits, uint16_t *__restrict__ out,
    float *__restrict__ partials, uint32_t *__restrict__ counters) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j16 = lane & 15;  // A row within the tile / B column within the tile
    const int kq = lane >> 4;   // 8-row slice of the 32-row step
    const int N8 = N >> 3;
    const int tile_n = blockIdx.x;
    const int tile_m = blockIdx.y;
    const int split = blockIdx.z;
    const int word = (tile_n * NWN + wave) * 16 + j16;
    const bool col_ok = word < N8;
    const int m0 = tile_m * 16 * MT;
    const int nsteps = K / 32;
    const int s_begin = split * split_len;
    const int s_end = min(s_begin + split_len, nsteps);

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    f16x2 sp[8], zc[8];
    int gcur = -1;
    for (int st = s_begin; st < s_end; ++st) {
        const int k0 = st * 32;
        const int g = k0 / G;
        if (g != gcur) {
            gcur = g;
            u32x4 sv = {0u, 0u, 0u, 0u};
            if (col_ok) sv = *reinterpret_cast<const u32x4 *>(scales + (size_t)g * N + word * 8);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t lo = sv[x] & 0xffffu, hi = sv[x] >> 16;
                sp[2 * x] = as_f16x2(lo | (lo << 16));
                sp[2 * x + 1] = as_f16x2(hi | (hi << 16));
            }
            if (ASYM) {
                const uint32_t zw = col_ok ? qzeros[(size_t)g * N8 + word] : 0u;
                zc[0] = zero_pair_from_word<0>(zw);
                zc[1] = zero_pair_from_word<1>(zw);
                zc[2] = zero_pair_from_word<2>(zw);
                zc[3] = zero_pair_from_word<3>(zw);
                zc[4] = zero_pair_from_word<4>(zw);
                zc[5] = zero_pair_from_word<5>(zw);
                zc[6] = zero_pair_from_word<6>(zw);
                zc[7] = zero_pair_from_word<7>(zw);
            } else {
                zc[0] = zero_pair_const<0>(zp);
                zc[1] = zero_pair_const<1>(zp);
                zc[2] = zero_pair_const<2>(zp);
                zc[3] = zero_pair_const<3>(zp);
                zc[4] = zero_pair_const<4>(zp);
                zc[5] = zero_pair_const<5>(zp);
                zc[6] = zero_pair_const<6>(zp);
                zc[7] = zero_pair_const<7>(zp);
            }
        }

        uint32_t wd[8];
        if (col_ok) {
            const uint32_t *bp = b + (size_t)(k0 + 8 * kq) * N8 + word;
#pragma unroll
            for (int r = 0; r < 8; ++r) wd[r] = bp[(size_t)r * N8];
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) wd[r] = 0x88888888u;
        }
        f16x8 av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = m0 + 16 * mt + j16;
            if (row < M)
                av[mt] = *reinterpret_cast<const f16x8 *>(a + (size_t)row * K + k0 + 8 * kq);
            else
                av[mt] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }

        f16x8 bop[8];
        dequant_byte<0>(wd, zc, sp, bop);
        dequant_byte<1>(wd, zc, sp, bop);
        dequant_byte<2>(wd, zc, sp, bop);
        dequant_byte<3>(wd, zc, sp, bop);

#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], bop[t], acc[mt][t], 0, 0, 0);
    }

    // acc[mt][t][v] = C[m0 + 16*mt + 4*kq + v][8*word + t].
    if (splits == 1) {
        if (!col_ok) return;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + 16 * mt + 4 * kq + v;
                if (row >= M) continue;
                f16x8 o;
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t] = (f16)acc[mt][t][v];
                *reinterpret_cast<f16x8 *>(out + (size_t)row * N + word * 8) = o;
            }
        return;
    }

    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + 16 * mt + 4 * kq + v;
                if (row >= M) continue;
                f32x4 *dst = reinterpret_cast<f32x4 *>(partials + ((size_t)split * M + row) * N + word * 8);
                dst[0] = f32x4{acc[mt][0][v], acc[mt][1][v], acc[mt][2][v], acc[mt][3][v]};
                dst[1] = f32x4{acc[mt][4][v], acc[mt][5][v], acc[mt][6][v], acc[mt][7][v]};
            }
    }
    fence_release_agent();
    __syncthreads();
    __shared__ uint32_t last;
    const int tile_id = tile_m * gridDim.x + tile_n;
    if (threadIdx.x == 0) last = (arrive_agent(&counters[tile_id]) == (uint32_t)(splits - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    fence_acquire_agent();
    if (col_ok) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + 16 * mt + 4 * kq + v;
                if (row >= M) continue;
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
                for (int sp_i = 0; sp_i < splits; ++sp_i) {
                    const f32x4 *src = reinterpret_cast<const f32x4 *>(
                        partials + ((size_t)sp_i * M + row) * N + word * 8);
                    s0 += src[0];
                    s1 += src[1];
                }
                f16x8 o = {(f16)s0.x, (f16)s0.y, (f16)s0.z, (f16)s0.w,
                           (f16)s1.x, (f16)s1.y, (f16)s1.z, (f16)s1.w};
                *reinterpret_cast<f16x8 *>(out + (size_t)row * N + word * 8) = o;
            }
    }
    if (threadIdx.x == 0) reset_counter_agent(&counters[tile_id]);
}

template <int MT>
hipError_t launch_mt(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    constexpr int NWN = 2;
    dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)p.splits);
    dim3 block(64 * NWN, 1, 1);
    const uint32_t *b = reinterpret_cast<const uint32_t *>(g.b);
    const uint32_t *qz = reinterpret_cast<const uint32_t *>(g.qzeros);
    if (g.qzeros)
        hipLaunchKernelGGL((mfma_kernel<MT, NWN, true>), grid, block, 0, stream, g.a, b, g.scales,
                           qz, (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp,
                           (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    else
        hipLaunchKernelGGL((mfma_kernel<MT, NWN, false>), grid, block, 0, stream, g.a, b, g.scales,
                           qz, (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp,
                           (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    switch (p.mt) {
        case 1: return launch_mt<1>(g, p, stream);
        case 2: return launch_mt<2>(g, p, stream);
        case 4: return launch_mt<4>(g, p, stream);
        case 8: return launch_mt<8>(g, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
