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
// Work split.  A wave computes (16*MT rows) x (128 columns) over a share of
// the K range.  A workgroup has NWN waves side by side along N and NWK waves
// dividing its K range (contiguous blocks of 32-row steps, loads issued two
// steps ahead of use); the NWK partial tiles are
// summed through LDS in fixed order.  When the grid also splits K across
// workgroups, each split writes fp32 partials and a second, fully parallel
// kernel sums the splits in split order (deterministic; the kernel boundary
// orders the two).  Workgroup indices are remapped so that neighbouring
// column tiles run on the same XCD and share its L2.
#include "device.h"
#include "kernels.h"

namespace w4a16 {
namespace {

// Dequantise the 8 B operands (one per nibble position) from the 8 words of
// rows k0+8*kq .. +7 of one packed column-of-words.
template <int B>
__device__ __forceinline__ void dequant_byte(const uint32_t (&wd)[8], const f16x2 (&zc)[8],
                                             const f16x2 (&sp)[8], const NibbleConsts &nk,
                                             f16x8 (&bop)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t pr = gather_byte_pair<B>(wd[2 * j], wd[2 * j + 1]);
        const f16x2 v0 = (as_f16x2(biased_pair<0>(pr, nk)) - zc[2 * B]) * sp[2 * B];
        const f16x2 v1 = (as_f16x2(biased_pair<1>(pr, nk)) - zc[2 * B + 1]) * sp[2 * B + 1];
        bop[2 * B][2 * j] = v0.x;
        bop[2 * B][2 * j + 1] = v0.y;
        bop[2 * B + 1][2 * j] = v1.x;
        bop[2 * B + 1][2 * j + 1] = v1.y;
    }
}

template <int MT, int NWN, int NWK, bool ASYM>
__global__ __launch_bounds__(64 * NWN * NWK) void mfma_kernel(
    const uint16_t *__restrict__ a, const uint32_t *__restrict__ b,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros, int M, int K, int N,
    int G, uint32_t zp, int tiles_n, int tiles_m, int split_len, int splits,
    uint16_t *__restrict__ out, float *__restrict__ partials) {
    // Logical workgroup: XCD-contiguous runs (grid is a multiple of 8).
    const int logical = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (logical >= tiles_n * tiles_m * splits) return;
    const int tile_n = logical % tiles_n;
    const int tile_m = (logical / tiles_n) % tiles_m;
    const int split = logical / (tiles_n * tiles_m);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % NWN;
    const int wk = wave / NWN;
    const int j16 = lane & 15;  // A row within the tile / B column within the tile
    const int kq = lane >> 4;   // 8-row slice of the 32-row step
    const int N8 = N >> 3;
    const int word = (tile_n * NWN + wn) * 16 + j16;
    const bool col_ok = word < N8;
    const int wordc = col_ok ? word : N8 - 1;  // clamped: loads stay in bounds
    const int m0 = tile_m * 16 * MT;
    const int nsteps = K / 32;
    const int s_begin = split * split_len;
    const int s_end = min(s_begin + split_len, nsteps);
    const NibbleConsts nk = nibble_consts();

    f32x4 acc[MT][8];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This K-wave's contiguous block of 32-row steps (groups change rarely).
    const int per_wave = (s_end - s_begin + NWK - 1) / NWK;
    const int w_begin = min(s_begin + wk * per_wave, s_end);
    const int w_end = min(w_begin + per_wave, s_end);

    // Software pipeline: weight words two steps ahead, activations and the
    // group's scale/zero words one step ahead, so the loop never waits on a
    // load issued in the same iteration.
    auto load_w = [&](int st, uint32_t (&wd)[8]) {
        const uint32_t *bp = b + (size_t)(st * 32 + 8 * kq) * N8 + wordc;
#pragma unroll
        for (int r = 0; r < 8; ++r) wd[r] = bp[(size_t)r * N8];
    };
    auto load_a = [&](int st, f16x8 (&av)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = m0 + 16 * mt + j16;
            av[mt] = row < M ? *reinterpret_cast<const f16x8 *>(a + (size_t)row * K + st * 32 + 8 * kq)
                             : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    };
    auto load_sz = [&](int st, u32x4 &sv, uint32_t &zw) {
        const int g = st * 32 / G;
        sv = *reinterpret_cast<const u32x4 *>(scales + (size_t)g * N + wordc * 8);
        zw = ASYM ? qzeros[(size_t)g * N8 + wordc] : 0u;
    };

    uint32_t w0[8], w1[8];
    f16x8 a0[MT];
    u32x4 sv0;
    uint32_t zw0;
    if (w_begin < w_end) {
        load_w(w_begin, w0);
        load_a(w_begin, a0);
        load_sz(w_begin, sv0, zw0);
    }
    if (w_begin + 1 < w_end) load_w(w_begin + 1, w1);

    f16x2 sp[8], zc[8];
    int gcur = -1;
    for (int st = w_begin; st < w_end; ++st) {
        // prefetch
        uint32_t w2[8];
        f16x8 a1[MT];
        u32x4 sv1;
        uint32_t zw1;
        const bool more1 = st + 1 < w_end, more2 = st + 2 < w_end;
        if (more2) load_w(st + 2, w2);
        if (more1) {
            load_a(st + 1, a1);
            load_sz(st + 1, sv1, zw1);
        }

        const int g = st * 32 / G;
        if (g != gcur) {
            gcur = g;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t lo = sv0[x] & 0xffffu, hi = sv0[x] >> 16;
                sp[2 * x] = as_f16x2(lo | (lo << 16));
                sp[2 * x + 1] = as_f16x2(hi | (hi << 16));
            }
            if (ASYM) {
                zc[0] = zero_pair_from_word<0>(zw0, nk);
                zc[1] = zero_pair_from_word<1>(zw0, nk);
                zc[2] = zero_pair_from_word<2>(zw0, nk);
                zc[3] = zero_pair_from_word<3>(zw0, nk);
                zc[4] = zero_pair_from_word<4>(zw0, nk);
                zc[5] = zero_pair_from_word<5>(zw0, nk);
                zc[6] = zero_pair_from_word<6>(zw0, nk);
                zc[7] = zero_pair_from_word<7>(zw0, nk);
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

        f16x8 bop[8];
        dequant_byte<0>(w0, zc, sp, nk, bop);
        dequant_byte<1>(w0, zc, sp, nk, bop);
        dequant_byte<2>(w0, zc, sp, nk, bop);
        dequant_byte<3>(w0, zc, sp, nk, bop);

#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0[mt], bop[t], acc[mt][t], 0, 0, 0);

        // rotate the pipeline
#pragma unroll
        for (int r = 0; r < 8; ++r) { w0[r] = w1[r]; w1[r] = w2[r]; }
        if (more1) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a0[mt] = a1[mt];
            sv0 = sv1;
            zw0 = zw1;
        }
    }

    // Sum the NWK partial tiles in order wk = 0, 1, ... through LDS, one
    // K-wave at a time (each round moves MT * 8 KB per N-wave).
    if constexpr (NWK > 1) {
        __shared__ f32x4 red[NWN][MT * 8][64];
#pragma unroll
        for (int r = 1; r < NWK; ++r) {
            if (wk == r) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int t = 0; t < 8; ++t) red[wn][mt * 8 + t][lane] = acc[mt][t];
            }
            __syncthreads();
            if (wk == 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int t = 0; t < 8; ++t) acc[mt][t] += red[wn][mt * 8 + t][lane];
            }
            __syncthreads();
        }
        if (wk != 0) return;
    }
    if (!col_ok) return;

    // acc[mt][t][v] = C[m0 + 16*mt + 4*kq + v][8*word + t].
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = m0 + 16 * mt + 4 * kq + v;
            if (row >= M) continue;
            if (splits == 1) {
                f16x8 o;
#pragma unroll
                for (int t = 0; t < 8; ++t) o[t] = (f16)acc[mt][t][v];
                *reinterpret_cast<f16x8 *>(out + (size_t)row * N + word * 8) = o;
            } else {
                f32x4 *dst = reinterpret_cast<f32x4 *>(partials + ((size_t)split * M + row) * N + word * 8);
                dst[0] = f32x4{acc[mt][0][v], acc[mt][1][v], acc[mt][2][v], acc[mt][3][v]};
                dst[1] = f32x4{acc[mt][4][v], acc[mt][5][v], acc[mt][6][v], acc[mt][7][v]};
            }
        }
}

// out[m][8c .. 8c+7] = fp16(sum over s of partials[s][m][8c .. 8c+7]), s in order.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ partials, int splits,
                                                            int M, int N, uint16_t *__restrict__ out) {
    const int N8 = N >> 3;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * N8) return;
    const int64_t row = idx / N8, c8 = idx % N8;
    const size_t plane = (size_t)M * N;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(partials + (size_t)row * N + c8 * 8);
    f32x4 s0 = src[0], s1 = src[1];
    for (int s = 1; s < splits; ++s) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(partials + s * plane + (size_t)row * N + c8 * 8);
        s0 += p[0];
        s1 += p[1];
    }
    const f16x8 o = {(f16)s0.x, (f16)s0.y, (f16)s0.z, (f16)s0.w, (f16)s1.x, (f16)s1.y, (f16)s1.z, (f16)s1.w};
    *reinterpret_cast<f16x8 *>(out + (size_t)row * N + c8 * 8) = o;
}

template <int MT, int NWN, int NWK>
hipError_t launch_cfg(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    dim3 grid((unsigned)p.grid, 1, 1);
    dim3 block(64 * NWN * NWK, 1, 1);
    const uint32_t *b = reinterpret_cast<const uint32_t *>(g.b);
    const uint32_t *qz = reinterpret_cast<const uint32_t *>(g.qzeros);
    if (g.qzeros)
        hipLaunchKernelGGL((mfma_kernel<MT, NWN, NWK, true>), grid, block, 0, stream, g.a, b, g.scales, qz,
                           (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp, (int)p.tiles_n,
                           (int)p.tiles_m, (int)p.split_len, p.splits, g.out, g.partials);
    else
        hipLaunchKernelGGL((mfma_kernel<MT, NWN, NWK, false>), grid, block, 0, stream, g.a, b, g.scales, qz,
                           (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp, (int)p.tiles_n,
                           (int)p.tiles_m, (int)p.split_len, p.splits, g.out, g.partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t n = g.M * (g.N / 8);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       g.partials, p.splits, (int)g.M, (int)g.N, g.out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    // (MT, NWN, NWK) combinations the planner emits.
    if (p.mt == 1 && p.waves == 2 && p.kwaves == 4) return launch_cfg<1, 2, 4>(g, p, stream);
    if (p.mt == 2 && p.waves == 2 && p.kwaves == 4) return launch_cfg<2, 2, 4>(g, p, stream);
    if (p.mt == 4 && p.waves == 2 && p.kwaves == 2) return launch_cfg<4, 2, 2>(g, p, stream);
    if (p.mt == 8 && p.waves == 1 && p.kwaves == 4) return launch_cfg<8, 1, 4>(g, p, stream);
    if (p.mt == 8 && p.waves == 2 && p.kwaves == 2) return launch_cfg<8, 2, 2>(g, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace w4a16
