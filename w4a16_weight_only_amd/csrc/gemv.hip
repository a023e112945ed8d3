// gemv.hip -- W4A16 split-K GEMV for M <= 8 rows (gfx950), in two forms that
// share the tiles, the K-split hand-off and the glue folding: the dot2 form
// below (vector ALUs) and the matrix-core form further down (the default).
//
// out = a . ((q - z) * s)  (vLLM PR #37352 write-up, "Code analysis" item 1).
// Decode is bound by streaming the weights once (inference-engine article,
// section 1.2), so the kernel is organised around that stream:
//
//  * A workgroup owns a 256-column tile (32 packed words = one 128-byte line
//    of every weight row) and a K range.  In a wave, CL column lanes cover the
//    line with WORDS-word loads (16 bytes when WORDS = 4) and RL = 64/CL row
//    lanes take different 16-row chunks, so each load instruction reads whole
//    lines (narrower tiles that split lines between workgroups cost up to 60%
//    more time on MI355X), with the non-temporal cache policy (read once).  Loads are unconditional -- lanes past N read a
//    clamped, valid address and their columns are never stored -- so the
//    compiler can wait for each row pair as it lands.
//  * Each lane converts nibbles two rows at a time (device.h) and accumulates
//    a_k * (q - z) for the row pair with one v_dot2_f32_f16 into fp32.  In the
//    exact form the zero point is subtracted in fp16 before the dot (exact:
//    small integers); in the folded form the dot takes (bias + q) and the
//    zero term is removed once per 16-row chunk (one VALU op fewer per pair,
//    fp32 rounding of the biased sums).  The group scale is applied
//    once per chunk (a chunk lies in one K-group).  No matrix cores.
//  * Row lanes are reduced with a transpose-reduce over lane-xor shuffles
//    (each step halves the values a lane holds), waves through LDS.  K-splits
//    meet in one 64-bit slot per output: each split adds its fp32 partial as
//    an exact fixed-point integer together with an arrival count, and the
//    split whose atomic completes the count writes the fp16 output from the
//    value the atomic returned (device.h).  Integer addition is associative,
//    so the result is the same whatever the arrival order (no float atomics,
//    the lesson of the same article's section 3.4), and the hand-off costs
//    one atomic round trip instead of store, counter and reload.
#include "device.h"
#include "kernels.h"

#include <type_traits>

namespace w4a16 {
namespace {

constexpr int kTileWords = 32;  // 256 columns per workgroup tile
constexpr int kTileCols = 256;
constexpr int kChunkRows = 16;  // rows per lane chunk = 8 row pairs

template <int W>
struct Words {
    uint32_t v[W];
};

template <int W>
__device__ __forceinline__ Words<W> buffer_words(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
template <>
__device__ __forceinline__ Words<4> buffer_words<4>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 t = buffer_load_x4_nt(r, voff, soff);
    return Words<4>{{t.x, t.y, t.z, t.w}};
}
template <>
__device__ __forceinline__ Words<2> buffer_words<2>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x2 t = buffer_load_x2_nt(r, voff, soff);
    return Words<2>{{t.x, t.y}};
}
template <>
__device__ __forceinline__ Words<1> buffer_words<1>(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return Words<1>{{buffer_load_x1_nt(r, voff, soff)}};
}

template <int W>
__device__ __forceinline__ Words<W> load_words(const uint32_t *p);
template <>
__device__ __forceinline__ Words<4> load_words<4>(const uint32_t *p) {
    u32x4 t = *reinterpret_cast<const u32x4 *>(p);
    return Words<4>{{t.x, t.y, t.z, t.w}};
}
template <>
__device__ __forceinline__ Words<2> load_words<2>(const uint32_t *p) {
    u32x2 t = *reinterpret_cast<const u32x2 *>(p);
    return Words<2>{{t.x, t.y}};
}
template <>
__device__ __forceinline__ Words<1> load_words<1>(const uint32_t *p) {
    return Words<1>{{*p}};
}

// One byte position B of one word pair: columns col0+2B, col0+2B+1, two rows.
template <int M, int COLS, int B, bool FOLD, bool FIRST>
__device__ __forceinline__ void dot_byte(uint32_t lo, uint32_t hi, int col0, const f16x2 *zc,
                                         const uint32_t (&apair)[M], const NibbleConsts &nk,
                                         float (&p)[M][COLS]) {
    const uint32_t pr = gather_byte_pair<B>(lo, hi);
    f16x2 v0 = as_f16x2(biased_pair<0>(pr, nk));
    f16x2 v1 = as_f16x2(biased_pair<1>(pr, nk));
    if (!FOLD) {
        v0 = v0 - zc[col0 + 2 * B];
        v1 = v1 - zc[col0 + 2 * B + 1];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const f16x2 av = as_f16x2(apair[m]);
        if (FIRST) {
            p[m][col0 + 2 * B] = dot2_first(v0, av);
            p[m][col0 + 2 * B + 1] = dot2_first(v1, av);
        } else {
            p[m][col0 + 2 * B] = __builtin_amdgcn_fdot2(v0, av, p[m][col0 + 2 * B], false);
            p[m][col0 + 2 * B + 1] = __builtin_amdgcn_fdot2(v1, av, p[m][col0 + 2 * B + 1], false);
        }
    }
}

template <int T>
__device__ __forceinline__ f16x2 zero_pair(bool asym, uint32_t zword, uint32_t zp, const NibbleConsts &nk) {
    return asym ? zero_pair_from_word<T>(zword, nk) : zero_pair_const<T>(zp);
}

// Logical workgroup index for hardware index `bid` (grid a multiple of 8):
// workgroups are dealt to the 8 XCDs round-robin, so this gives each XCD a
// contiguous run of logical indices (neighbouring tiles and their scales).
__device__ __forceinline__ int xcd_local_index(int bid, int grid) {
    return (bid & 7) * (grid >> 3) + (bid >> 3);
}

// Activation transform applied as the activations are loaded (the decode
// step's glue between linears, folded into the consuming GEMV):
//   ACT 0: a as given
//   ACT 1: a[m][k] = fp16(src[m][k] * inv_m),  inv_m = 1/sqrt(mean_{k<K} src[m][k]^2 + 1e-6)
//   ACT 2: t[m][k] = silu(src[m][k]) * src[m][K + k],  a[m][k] = fp16(t * inv_m), inv over t
// src rows are `ld` elements apart; math in fp32, one RNE rounding to fp16.
template <int ACT>
__device__ __forceinline__ float act_value(const u32x4 &x, const u32x4 &y, int e) {
    const float v = f16_bits_to_f32((x[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    if constexpr (ACT == 2) return silu_mul(v, f16_bits_to_f32((y[e >> 1] >> (16 * (e & 1))) & 0xffffu));
    else return v;
}

// Row sums of squares of the transformed activations, in the glue kernels'
// order (glue.hip): 1024 virtual threads, virtual thread i accumulates vectors
// i + 1024 j (j = 0, 1, ...) element by element with fma, each wave of 64
// reduces with an xor-shuffle and the 16 wave sums are added in order.  Thread
// t of the 512-thread workgroup plays virtual threads t (chain 0) and t + 512
// (chain 1), so the row scale is bit for bit the standalone glue kernel's and
// the fused and unfused decode steps agree exactly.
template <int ACT>
__device__ __forceinline__ float sq_chain(const u32x4 &x, const u32x4 &y, float ss) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float t = act_value<ACT>(x, y, e);
        ss = __builtin_fmaf(t, t, ss);
    }
    return ss;
}

// Row sums of squares of the glue-transformed rows (ACT 1, 2) for a
// 512-thread workgroup, in the glue kernels' order (sq_chain).  With EARLY
// (M <= 2) load() requests the row's vectors before the weight stream and
// holds them in registers (RV 16-byte vectors per virtual thread); otherwise
// partials() streams them.  partials() is the per-lane part; reduce() the
// cross-lane part, to be called where every lane of the wave is active; the
// 16 per-wave sums of each row meet in s_part, which inv() reads.
template <int M, int ACT, int RV, bool EARLY>
struct RowSums {
    static constexpr int kRM = EARLY ? M : 1, kRV = EARLY ? RV : 1;
    u32x4 rx[kRM][2][kRV], ry[kRM][2][kRV];
    float ss[M][2];

    __device__ __forceinline__ void load(const uint16_t *src, int ld, int K) {
        if constexpr (EARLY) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(src + (size_t)m * ld, (uint32_t)K * 2u);
                const __amdgpu_buffer_rsrc_t ur =
                    buffer_rsrc(src + (size_t)m * ld + K, ACT == 2 ? (uint32_t)K * 2u : 0u);
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < RV; ++j) {
                        // a vector past the row reads zeros (adds exactly 0)
                        const uint32_t off = ((uint32_t)threadIdx.x + 512u * h + 1024u * j) * 16u;
                        rx[m][h][j] = buffer_load_x4(gr, off, 0);
                        ry[m][h][j] = rx[m][h][j];
                        if constexpr (ACT == 2) ry[m][h][j] = buffer_load_x4(ur, off, 0);
                    }
            }
        }
    }
    __device__ __forceinline__ void partials(const uint16_t *src, int ld, int K) {
        if constexpr (EARLY) {
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float t = 0.f;
#pragma unroll
                    for (int j = 0; j < RV; ++j) t = sq_chain<ACT>(rx[m][h][j], ry[m][h][j], t);
                    ss[m][h] = t;
                }
        } else {
            // Pass j requests vector j of both chains of every row at once (one
            // round trip per pass rather than one per row and chain), then
            // extends each chain; every chain still runs in increasing j.
            const int passes = (K / 8 + 1023) / 1024;
#pragma unroll
            for (int m = 0; m < M; ++m) ss[m][0] = ss[m][1] = 0.f;
            for (int j = 0; j < passes; ++j) {
                u32x4 x[M][2], y[M][2];
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const __amdgpu_buffer_rsrc_t gr = buffer_rsrc(src + (size_t)m * ld, (uint32_t)K * 2u);
                    const __amdgpu_buffer_rsrc_t ur =
                        buffer_rsrc(src + (size_t)m * ld + K, ACT == 2 ? (uint32_t)K * 2u : 0u);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // a vector past the row reads zeros (adds exactly 0)
                        const uint32_t off = ((uint32_t)threadIdx.x + 512u * h + 1024u * j) * 16u;
                        x[m][h] = buffer_load_x4(gr, off, 0);
                        y[m][h] = x[m][h];
                        if constexpr (ACT == 2) y[m][h] = buffer_load_x4(ur, off, 0);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int h = 0; h < 2; ++h) ss[m][h] = sq_chain<ACT>(x[m][h], y[m][h], ss[m][h]);
            }
        }
    }
    __device__ __forceinline__ void reduce(float (&s_part)[16][M], int lane, int wave) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float v = wave_sum(ss[m][h], lane);
                if (lane == 0) s_part[8 * h + wave][m] = v;
            }
    }
    static __device__ __forceinline__ float inv(const float (&s_part)[16][M], int m, int K) {
        float q = 0.f;
#pragma unroll
        for (int w = 0; w < 16; ++w) q += s_part[w][m];
        return row_inv(q, K);
    }
};

// Sums the workgroup's per-wave partials of a TC-column tile (red) in wave
// order, multiplies row m by row_scale(m), and writes the tile: directly with
// one K-split, else through one fixed-point slot per output (device.h), every
// atomic issued before the first result is looked at.
template <int M, int NW, typename RowScale, int TC = kTileCols>
__device__ __forceinline__ void finish_tile(const float (&red)[NW][M][TC], RowScale row_scale, int tile,
                                            int N, int splits, uint16_t *__restrict__ out,
                                            uint32_t *__restrict__ counters) {
    // One (row, column) per thread and pass.
    constexpr int PASSES = (M * TC + 64 * NW - 1) / (64 * NW);
    const int col_base = tile * TC;
    float sums[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int t = threadIdx.x + i * 64 * NW;
        float s = 0.f;
        if (t < M * TC) {
#pragma unroll
            for (int wv = 0; wv < NW; ++wv) s += red[wv][t / TC][t % TC];
            s *= row_scale(t / TC);
        }
        sums[i] = s;
    }
    if (splits == 1) {
#pragma unroll
        for (int i = 0; i < PASSES; ++i) {
            const int t = threadIdx.x + i * 64 * NW;
            const int col = col_base + t % TC;
            if (t < M * TC && col < N) out[(size_t)(t / TC) * N + col] = f32_to_f16_bits(sums[i]);
        }
        return;
    }
    uint64_t *slots = reinterpret_cast<uint64_t *>(counters);
    uint64_t add[PASSES], old[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int t = threadIdx.x + i * 64 * NW;
        const int col = col_base + t % TC;
        add[i] = slot_contribution(sums[i]);
        old[i] = 0;
        if (t < M * TC && col < N) old[i] = slot_add(&slots[(size_t)(t / TC) * N + col], add[i]);
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
        const int t = threadIdx.x + i * 64 * NW;
        const int col = col_base + t % TC;
        if (t < M * TC && col < N && slot_last(old[i], splits)) {
            const size_t o = (size_t)(t / TC) * N + col;
            out[o] = slot_result_f16(old[i] + add[i], splits);
            slot_reset(&slots[o]);
        }
    }
}

template <int M, int WORDS, int NW, bool ASYM, bool FOLD, int ACT, int RV>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ src, int ld, const uint32_t *__restrict__ b,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros, int K, int N, int G,
    uint32_t zp, int tiles, int split_len, int splits, uint16_t *__restrict__ out,
    uint32_t *__restrict__ counters) {
    constexpr int CL = kTileWords / WORDS;  // column lanes per row segment
    constexpr int RL = 64 / CL;             // row lanes
    constexpr int COLS = 8 * WORDS;         // columns per lane
    static_assert(COLS == 4 * RL, "four columns per lane after the row-lane reduction");

    const int logical = xcd_local_index(blockIdx.x, gridDim.x);
    if (logical >= tiles * splits) return;
    const int tile = logical % tiles;
    const int split = logical / tiles;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cl = lane % CL;
    const int rl = lane / CL;
    const int N8 = N >> 3;
    // Lanes past N read a valid (clamped) address; their columns are never stored.
    const int word0 = min(tile * kTileWords + cl * WORDS, N8 - WORDS);
    const int nchunks = K / kChunkRows;
    const int c_begin = split * split_len;
    const int c_end = min(c_begin + split_len, nchunks);
    const NibbleConsts nk = nibble_consts();
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(b, (uint32_t)((uint64_t)K * N8 * 4));
    const uint32_t row_bytes = (uint32_t)N8 * 4u;

    float acc[M][COLS];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < COLS; ++j) acc[m][j] = 0.f;

    // Glue transform (ACT != 0).  The row-norm is a per-row scalar, so it is
    // applied to the products in the epilogue: the GEMV takes the raw row
    // (ACT 1) or fp16(silu(g) * u) (ACT 2) and each output is multiplied by
    // its row's 1/sqrt(mean(t^2) + 1e-6).  The row sums run off the weight
    // stream's critical path: at M <= 2 the row's vectors are requested
    // before the weights (loads complete in issue order, so they never wait
    // for the weight stream), are summed while the first weights are in
    // flight, and meet at the epilogue's barrier.  (Summing the rows before the weight stream
    // starts costs an L2 round trip and two barriers per launch.)
    __shared__ float s_part[16][M];
    constexpr bool kEarlyRows = ACT != 0 && M <= 2;
    RowSums<M, ACT, RV, kEarlyRows> rows;
    if constexpr (kEarlyRows) {
        rows.load(src, ld, K);
        __builtin_amdgcn_sched_barrier(0);
    }

    struct Chunk {
        u32x4 ax[M][2], ay[M][2];  // raw activations (ACT 2: gate in ax, up in ay)
        uint32_t sw[COLS / 2];     // scale bits, two columns per word
        Words<WORDS> zw;           // packed zeros (ASYM)
        Words<WORDS> w[kChunkRows];
    };
    // Small loads first, the weight stream last, so that row pairs are
    // consumed in order as they land.
    auto load_chunk = [&](int c, Chunk &d) __attribute__((always_inline)) {
        const int k0 = c * kChunkRows;
        const int g = k0 / G;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const uint16_t *row = ACT == 0 ? a + (size_t)m * K + k0 : src + (size_t)m * ld + k0;
            d.ax[m][0] = *reinterpret_cast<const u32x4 *>(row);
            d.ax[m][1] = *reinterpret_cast<const u32x4 *>(row + 8);
            if constexpr (ACT == 2) {
                d.ay[m][0] = *reinterpret_cast<const u32x4 *>(row + K);
                d.ay[m][1] = *reinterpret_cast<const u32x4 *>(row + K + 8);
            }
        }
        const u32x4 *sp = reinterpret_cast<const u32x4 *>(scales + (size_t)g * N + word0 * 8);
#pragma unroll
        for (int x = 0; x < WORDS; ++x) {
            const u32x4 t = sp[x];
            d.sw[4 * x] = t.x; d.sw[4 * x + 1] = t.y; d.sw[4 * x + 2] = t.z; d.sw[4 * x + 3] = t.w;
        }
#pragma unroll
        for (int x = 0; x < WORDS; ++x) d.zw.v[x] = 0u;
        if (ASYM) d.zw = load_words<WORDS>(qzeros + (size_t)g * N8 + word0);
        // keep the scale and zero requests ahead of the weight stream (the
        // scheduler otherwise sinks them towards their late use)
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t voff = ((uint32_t)k0 * (uint32_t)N8 + (uint32_t)word0) * 4u;
#pragma unroll
        for (int r = 0; r < kChunkRows; ++r) d.w[r] = buffer_words<WORDS>(brs, voff, (uint32_t)r * row_bytes);
    };
    auto compute_chunk = [&](const Chunk &d) __attribute__((always_inline)) {
        uint32_t av[M][8];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if constexpr (ACT != 2) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    av[m][4 * h] = d.ax[m][h].x; av[m][4 * h + 1] = d.ax[m][h].y;
                    av[m][4 * h + 2] = d.ax[m][h].z; av[m][4 * h + 3] = d.ax[m][h].w;
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        av[m][4 * h + j] =
                            (uint32_t)f32_to_f16_bits(act_value<2>(d.ax[m][h], d.ay[m][h], 2 * j)) |
                            ((uint32_t)f32_to_f16_bits(act_value<2>(d.ax[m][h], d.ay[m][h], 2 * j + 1)) << 16);
            }
        }
        const uint32_t(&sw)[COLS / 2] = d.sw;
        const Words<WORDS> &zw = d.zw;
        const Words<WORDS>(&w)[kChunkRows] = d.w;

        f16x2 zc[COLS];
        if (!FOLD) {
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                zc[8 * x + 0] = zero_pair<0>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 1] = zero_pair<1>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 2] = zero_pair<2>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 3] = zero_pair<3>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 4] = zero_pair<4>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 5] = zero_pair<5>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 6] = zero_pair<6>(ASYM, zw.v[x], zp, nk);
                zc[8 * x + 7] = zero_pair<7>(ASYM, zw.v[x], zp, nk);
            }
        }

        float p[M][COLS];
        {  // row pair (k0, k0 + 1) starts the sums
            uint32_t apair[M];
#pragma unroll
            for (int m = 0; m < M; ++m) apair[m] = av[m][0];
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                const uint32_t lo = w[0].v[x], hi = w[1].v[x];
                dot_byte<M, COLS, 0, FOLD, true>(lo, hi, 8 * x, zc, apair, nk, p);
                dot_byte<M, COLS, 1, FOLD, true>(lo, hi, 8 * x, zc, apair, nk, p);
                dot_byte<M, COLS, 2, FOLD, true>(lo, hi, 8 * x, zc, apair, nk, p);
                dot_byte<M, COLS, 3, FOLD, true>(lo, hi, 8 * x, zc, apair, nk, p);
            }
        }
#pragma unroll
        for (int j = 1; j < 8; ++j) {  // row pair (k0 + 2j, k0 + 2j + 1)
            uint32_t apair[M];
#pragma unroll
            for (int m = 0; m < M; ++m) apair[m] = av[m][j];
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                const uint32_t lo = w[2 * j].v[x], hi = w[2 * j + 1].v[x];
                dot_byte<M, COLS, 0, FOLD, false>(lo, hi, 8 * x, zc, apair, nk, p);
                dot_byte<M, COLS, 1, FOLD, false>(lo, hi, 8 * x, zc, apair, nk, p);
                dot_byte<M, COLS, 2, FOLD, false>(lo, hi, 8 * x, zc, apair, nk, p);
                dot_byte<M, COLS, 3, FOLD, false>(lo, hi, 8 * x, zc, apair, nk, p);
            }
        }

        // Folded form: remove (bias + z) * sum(a) per chunk.  Symmetric zero
        // point: the correction is the same dot2 chain as the sums, run on the
        // constant (bias + zp) pair, so a column whose nibbles all equal zp
        // cancels to exactly 0.  Packed zeros vary by column: (bias + z) times
        // the chunk's activation sum.
        float corr[M][2], asum[M];
        if (FOLD) {
            if constexpr (!ASYM) {
                const f16x2 b0 = zero_pair_const<0>(zp), b1 = zero_pair_const<1>(zp);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float c0 = dot2_first(b0, as_f16x2(av[m][0])), c1 = dot2_first(b1, as_f16x2(av[m][0]));
#pragma unroll
                    for (int j = 1; j < 8; ++j) {
                        c0 = __builtin_amdgcn_fdot2(b0, as_f16x2(av[m][j]), c0, false);
                        c1 = __builtin_amdgcn_fdot2(b1, as_f16x2(av[m][j]), c1, false);
                    }
                    corr[m][0] = c0;
                    corr[m][1] = c1;
                }
            } else {
                const f16x2 ones = as_f16x2(0x3c003c00u);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float s = 0.f;
#pragma unroll
                    for (int j = 0; j < 8; ++j) s = __builtin_amdgcn_fdot2(as_f16x2(av[m][j]), ones, s, false);
                    asum[m] = s;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < COLS; ++j) {
            const uint32_t bits = (j & 1) ? (sw[j >> 1] >> 16) : (sw[j >> 1] & 0xffffu);
            const float s = f16_bits_to_f32(bits);
            if (FOLD && !ASYM) {
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m][j] = __builtin_fmaf(s, p[m][j] - corr[m][j & 1], acc[m][j]);
            } else if (FOLD) {
                const uint32_t zq = (zw.v[j >> 3] >> (4 * (j & 7))) & 0xfu;
                const float zb = (float)((j & 1) ? 64u + zq : 1024u + zq);
#pragma unroll
                for (int m = 0; m < M; ++m)
                    acc[m][j] = __builtin_fmaf(s, __builtin_fmaf(-zb, asum[m], p[m][j]), acc[m][j]);
            } else {
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m][j] = __builtin_fmaf(s, p[m][j], acc[m][j]);
            }
        }
    };

    const int c0 = c_begin + wave * RL + rl;
    constexpr int kStride = NW * RL;
    // Row sums: the per-lane part (row_partials) and the cross-lane part
    // (row_reduce, where every lane of the wave is active), then across waves
    // in the epilogue.  With the row held in registers (M <= 2) the per-lane
    // part runs while the first chunk's weights are in flight; otherwise
    // after the chunk loop.
    auto row_partials = [&]() __attribute__((always_inline)) {
        if constexpr (ACT != 0) {
            static_assert(NW == 8, "the row sums map 1024 virtual threads onto 512");
            rows.partials(src, ld, K);
        }
    };
    auto row_reduce = [&]() __attribute__((always_inline)) {
        if constexpr (ACT != 0) rows.reduce(s_part, lane, wave);
    };

    if constexpr (kEarlyRows) {
        // first chunk peeled: its weights are requested, then the per-lane row
        // sums run on the row vectors (requested earlier, so already waited
        // for without waiting for the weights).  Whether a lane holds a chunk
        // differs between the lanes of a wave when a split holds fewer chunks
        // than row lanes, so the cross-lane reduction waits until after the
        // branch, where every lane takes part.
        if (c0 < c_end) {
            Chunk d;
            load_chunk(c0, d);
            row_partials();
            compute_chunk(d);
        } else {
            row_partials();
        }
        row_reduce();
        for (int c = c0 + kStride; c < c_end; c += kStride) {
            Chunk d;
            load_chunk(c, d);
            compute_chunk(d);
        }
    } else {
        for (int c = c0; c < c_end; c += kStride) {
            Chunk d;
            load_chunk(c, d);
            compute_chunk(d);
        }
        row_partials();
        row_reduce();
    }

    // Transpose-reduce over the row lanes (lane bits 5 .. log2(CL)): after the
    // step with mask 2^b the lanes with that bit set hold the sums of the
    // upper half of the columns they held.  Lane (cl, rl) ends with columns
    // cl*COLS + 4*rl + 0..3.
    if constexpr (CL <= 32) {
#pragma unroll
        for (int i = 0; i < COLS / 2; ++i)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m][i] = swap_add<32>(acc[m][i], acc[m][COLS / 2 + i], lane);
    }
    if constexpr (CL <= 16) {
#pragma unroll
        for (int i = 0; i < COLS / 4; ++i)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m][i] = swap_add<16>(acc[m][i], acc[m][COLS / 4 + i], lane);
    }
    if constexpr (CL <= 8) {
#pragma unroll
        for (int i = 0; i < COLS / 8; ++i)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m][i] = swap_add<8>(acc[m][i], acc[m][COLS / 8 + i], lane);
    }
    static_assert(CL >= 8, "at most three row-lane reduction steps");

    __shared__ float red[NW][M][kTileCols];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const f32x4 v = {acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        *reinterpret_cast<f32x4 *>(&red[wave][m][cl * COLS + 4 * rl]) = v;
    }
    __syncthreads();
    finish_tile<M, NW>(
        red,
        [&](int m) __attribute__((always_inline)) {
            if constexpr (ACT != 0) return RowSums<M, ACT, RV, kEarlyRows>::inv(s_part, m, K);
            else return 1.0f;
        },
        tile, N, splits, out, counters);
}

// ------------------------------------------------------------- MFMA form ---
// The same tiles, K-splits and hand-off with the k-reduction on the matrix
// cores: per 16-row set one v_mfma_f32_16x16x32_f16 takes the weights of 16
// lanes' columns as B and the activations as A.  Measured against the dot2
// form above, the vector ALUs then do about 0.8 instructions per weight
// instead of 1.4 (M = 1) to 4.75 (M = 8):
//
//  * Weights as biased fp16.  One AND-OR of a packed word gives nibbles 0 and
//    4 in the two fp16 halves as 1024 + q (device.h), another nibbles 1 and 5
//    as 64 + q; the word shifted right by 8 gives nibbles 2, 6 and 3, 7 the
//    same way: exact values, one instruction per two weights.  (Subnormal
//    weights, q * 2^-24 with no bias, lost precision on the matrix cores: 4-9
//    times the dot2 form's error.)
//  * Two columns per register.  A register of the B operand holds (column c,
//    column c + 4) of one weight row: its two k-slots.  Activation row mu
//    occupies A rows 2 mu and 2 mu + 1, which hold the row's activations in
//    the even and in the odd k-slots only, so D row 2 mu + e collects column
//    c + 4e.  Up to 8 activation rows fill the 16 A rows.
//  * Zero point.  By default (and always with packed zeros) the zero word is
//    unpacked like a weight word and one packed subtraction per register
//    leaves the exact integer (q - z) in fp16 before the MFMA: the products
//    are exact, so a column whose nibbles all equal its zero point sums to
//    exactly 0, and packed zeros that all equal zp give bit for bit the
//    symmetric result.  Measured on MI355X the subtraction costs nothing
//    visible (headline 8.24 -> 8.22 us).  Folded form (a symmetric zero point
//    with the tuning key gemv_mma_exact=0): B holds the biased weights and the
//    zero term sum(a) * (bias + zp) runs the same MFMA chain as the products,
//    on two B operands that hold (bias + zp) in every k-slot (bias 1024 and
//    64); the chunk's (q - z) sums are D minus that term, scaled by the group
//    scale into an fp32 total (the per-group factorisation out = sum_g s
//    (sum a q' - z' sum a)).  An all-zp column gets the same MFMA inputs
//    twice and cancels to exactly 0, but the biased sums (about 1000x the
//    result) carry fp32 rounding of their own size.
//  * Non-finite activations.  In the folded form the biased sums would turn
//    an infinite activation into inf - inf; when the zero term of a chunk is
//    not finite (exactly when one of its activations is not), the wave
//    recomputes all its chunks after the loop in the exact form, so
//    infinities keep their sign and a zero weight times an infinity gives
//    NaN, as in the definition (and as the exact form gives directly).
//
// Lane (j, g) = (lane % 16, lane / 16) loads words 2j, 2j+1 of the tile (8
// bytes of each row) for rows 16 s + 4 g + i (i < 4) of set s, and the
// activations of row mu = j / 2 at those rows.  A wave takes chunks of CH rows
// (CH divides G, so a chunk lies in one group) and issues all of a chunk's
// loads before its first wait.
// Zero-point forms of the matrix-core GEMV (template argument ZM).
enum ZeroMode { kZeroFolded = 0, kZeroPacked = 1, kZeroExact = 2 };

template <int M, int ZM, int ACT, int RV, int WL = 2>
__global__ __launch_bounds__(512) void gemv_mma_kernel(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ src, int ld, const uint32_t *__restrict__ b,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros, int K, int N, int G, uint32_t zp,
    int tiles, int split_len, int splits, uint16_t *__restrict__ out, uint32_t *__restrict__ counters) {
    static_assert(M >= 1 && M <= 8, "two A rows per activation row");
    constexpr bool ASYM = ZM == kZeroPacked;  // packed zero points
    constexpr bool kExact = ZM != kZeroFolded;  // B holds exact (q - z)
    constexpr int NW = 8;
    constexpr int CH = kMmaChunkRows;
    constexpr int SETS = CH / 16;
    constexpr int DV = M >= 2 ? 4 : 2;  // D elements that can hold rows < M (D row 4 g + v)
    constexpr int TW = 16 * WL, TC = 8 * TW;  // tile words and columns
    const int logical = xcd_local_index(blockIdx.x, gridDim.x);
    if (logical >= tiles * splits) return;
    const int tile = logical % tiles;
    const int split = logical / tiles;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;
    const int g = lane >> 4;
    const int N8 = N >> 3;
    // Lanes past N read a valid (clamped) address; their columns are never stored.
    const int word = min(tile * TW + WL * j, N8 - WL);
    const int nchunks = K / CH;
    const int c_begin = split * split_len;
    const int c_end = min(c_begin + split_len, nchunks);
    const uint32_t row_bytes = (uint32_t)N8 * 4u;
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(b, (uint32_t)((uint64_t)K * N8 * 4));
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(scales, (uint32_t)((uint64_t)(K / G) * N * 2));
    const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(qzeros, ASYM ? (uint32_t)((uint64_t)(K / G) * row_bytes) : 0u);
    // Activations: `a` (row stride K), or with the glue folded in (ACT 1, 2)
    // the raw rows of `src` (row stride ld; ACT 2: gate then up, K each).
    const int lda = ACT == 0 ? K : ld;
    const __amdgpu_buffer_rsrc_t ars =
        buffer_rsrc(ACT == 0 ? a : src, (uint32_t)(((uint64_t)(M - 1) * lda + (ACT == 2 ? 2 : 1) * K) * 2));
    const uint32_t b_voff = ((uint32_t)(4 * g) * (uint32_t)N8 + (uint32_t)word) * 4u;
    const int mu = j >> 1;
    const uint32_t a_voff = ((uint32_t)min(mu, M - 1) * (uint32_t)lda + 4u * (uint32_t)g) * 2u;
    // v_perm selectors placing activation 2r (sel0) or 2r + 1 (sel1) of a
    // loaded pair in fp16 half (j & 1) of an A register, the other half zero;
    // lanes of rows mu >= M give zeros.
    const NibbleConsts nk = nibble_consts();
    uint32_t sel0 = (j & 1) ? 0x01000c0cu : 0x0c0c0100u;
    uint32_t sel1 = (j & 1) ? 0x03020c0cu : 0x0c0c0302u;
    if (mu >= M) sel0 = sel1 = 0x0c0c0c0cu;
    // Symmetric zero term: B operands holding (1024 + zp) and (64 + zp) in
    // every k-slot (the biased weights' values where q == zp).
    const uint32_t zb0 = kMagicLo | zp | (zp << 16), zb1 = kMagicHi | (zp << 4) | (zp << 20);
    const f16x8 zb_lo = __builtin_bit_cast(f16x8, u32x4{zb0, zb0, zb0, zb0});
    const f16x8 zb_hi = __builtin_bit_cast(f16x8, u32x4{zb1, zb1, zb1, zb1});

    f32x4 tot[WL][4];
#pragma unroll
    for (int x = 0; x < WL; ++x)
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[x][q] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Glue folded in: the row scale 1/sqrt(mean(t^2) + 1e-6) multiplies the
    // products in the epilogue, as in the dot2 form (row sums in the glue
    // kernels' order; at M <= 2 the row's vectors requested first).
    __shared__ float s_part[16][M];
    constexpr bool kEarlyRows = ACT != 0 && M <= 2;
    RowSums<M, ACT, RV, kEarlyRows> rows;
    if constexpr (kEarlyRows) {
        rows.load(src, ld, K);
        __builtin_amdgcn_sched_barrier(0);
    }

    struct Chunk {
        u32x4 sv[WL];    // scales of the lane's 8 WL columns
        uint32_t zw[WL]; // packed zeros of its words (ASYM)
        u32x2 av[SETS];  // activations of row mu at the lane's 4 rows of each set (ACT 2: gate)
        u32x2 au[SETS];  // ACT 2: up
        uint32_t w[SETS][4][WL];
    };
    auto load_chunk = [&](int c, Chunk &d) __attribute__((always_inline)) {
        const uint32_t k0 = (uint32_t)c * CH;
        const uint32_t grp = k0 / (uint32_t)G;
#pragma unroll
        for (int x = 0; x < WL; ++x) {
            d.sv[x] = buffer_load_x4(srs, (uint32_t)word * 16u + 16u * x, grp * (uint32_t)N * 2u);
            d.zw[x] = 0u;
        }
        if constexpr (ASYM) {
            if constexpr (WL == 4) {
                const u32x4 z4 = buffer_load_x4(zrs, (uint32_t)word * 4u, grp * row_bytes);
                d.zw[0] = z4.x; d.zw[1] = z4.y; d.zw[2] = z4.z; d.zw[3] = z4.w;
            } else {
                const u32x2 z2 = buffer_load_x2(zrs, (uint32_t)word * 4u, grp * row_bytes);
                d.zw[0] = z2.x; d.zw[1] = z2.y;
            }
        }
#pragma unroll
        for (int s = 0; s < SETS; ++s) {
            d.av[s] = buffer_load_x2(ars, a_voff, (k0 + 16u * s) * 2u);
            if constexpr (ACT == 2) d.au[s] = buffer_load_x2(ars, a_voff + (uint32_t)K * 2u, (k0 + 16u * s) * 2u);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < SETS; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (WL == 4) {
                    const u32x4 v = buffer_load_x4_nt(brs, b_voff, (k0 + 16u * s + i) * row_bytes);
                    d.w[s][i][0] = v.x; d.w[s][i][1] = v.y; d.w[s][i][2] = v.z; d.w[s][i][3] = v.w;
                } else {
                    const u32x2 v = buffer_load_x2_nt(brs, b_voff, (k0 + 16u * s + i) * row_bytes);
                    d.w[s][i][0] = v.x; d.w[s][i][1] = v.y;
                }
            }
        // every load of the chunk is issued before its first use: left free,
        // the scheduler placed the A operand's perms (and with them a wait for
        // the activations) ahead of the weight requests in the glue-fused
        // variants, one memory round trip per chunk
        __builtin_amdgcn_sched_barrier(0);
    };
    // Products of one chunk into acc (per word x and nibble pair q) and, with a
    // symmetric zero point, the zero term into cz (one accumulator per bias).
    f32x4 acc[WL][4], cz[2];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < WL; ++x)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[x][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        cz[0] = cz[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // (bias + z) pairs of word x, nibble pair q (the weights' own unpacking
    // applied to the zero word; symmetric: the same for every word).
    auto zero_pair_q = [&](const Chunk &d, int x, int q) __attribute__((always_inline)) {
        if constexpr (ASYM) {
            const uint32_t zw = q >= 2 ? d.zw[x] >> 8 : d.zw[x];
            return (q & 1) ? ((zw & nk.mask_hi) | nk.bias_hi) : ((zw & nk.mask_lo) | nk.bias_lo);
        } else {
            return (q & 1) ? (kMagicHi | (zp << 4) | (zp << 20)) : (kMagicLo | zp | (zp << 16));
        }
    };
    // EXACT: B holds (q - z) (packed zeros, and the rare non-finite redo);
    // otherwise bias + q and the zero term in cz.
    auto mma_chunk = [&](const Chunk &d, auto exact_c) __attribute__((always_inline)) {
        constexpr bool EXACT = decltype(exact_c)::value;
#pragma unroll
        for (int s = 0; s < SETS; ++s) {
            uint32_t lo = d.av[s].x, hi = d.av[s].y;
            if constexpr (ACT == 2) {
                // a = fp16(silu(g) * u), the dot2 form's rounding
                auto t2 = [](uint32_t g2, uint32_t u2) __attribute__((always_inline)) {
                    const float t0 = silu_mul(f16_bits_to_f32(g2 & 0xffffu), f16_bits_to_f32(u2 & 0xffffu));
                    const float t1 = silu_mul(f16_bits_to_f32(g2 >> 16), f16_bits_to_f32(u2 >> 16));
                    return (uint32_t)f32_to_f16_bits(t0) | ((uint32_t)f32_to_f16_bits(t1) << 16);
                };
                lo = t2(lo, d.au[s].x);
                hi = t2(hi, d.au[s].y);
            }
            const f16x8 av = __builtin_bit_cast(
                f16x8, u32x4{__builtin_amdgcn_perm(0u, lo, sel0), __builtin_amdgcn_perm(0u, lo, sel1),
                             __builtin_amdgcn_perm(0u, hi, sel0), __builtin_amdgcn_perm(0u, hi, sel1)});
#pragma unroll
            for (int x = 0; x < WL; ++x) {
                uint32_t p[4][4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w = d.w[s][i][x];
                    const uint32_t sh = w >> 8;
                    p[0][i] = (w & nk.mask_lo) | nk.bias_lo;
                    p[1][i] = (w & nk.mask_hi) | nk.bias_hi;
                    p[2][i] = (sh & nk.mask_lo) | nk.bias_lo;
                    p[3][i] = (sh & nk.mask_hi) | nk.bias_hi;
                }
                if constexpr (EXACT) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f16x2 zq = as_f16x2(zero_pair_q(d, x, q));
#pragma unroll
                        for (int i = 0; i < 4; ++i) p[q][i] = as_u32(as_f16x2(p[q][i]) - zq);
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[x][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        av, __builtin_bit_cast(f16x8, u32x4{p[q][0], p[q][1], p[q][2], p[q][3]}), acc[x][q], 0, 0, 0);
            }
            if constexpr (!EXACT) {
                cz[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, zb_lo, cz[0], 0, 0, 0);
                cz[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, zb_hi, cz[1], 0, 0, 0);
            }
        }
    };
    // Products of one chunk (packed zeros: the exact form).  With a
    // symmetric zero point `nonfinite` records a zero term that is not finite
    // (the wave then redoes its chunks in the exact form after the loop, where
    // the loop's registers are free).
    bool nonfinite = false;
    auto chunk = [&](const Chunk &d) __attribute__((always_inline)) {
        zero_acc();
        mma_chunk(d, std::integral_constant<bool, kExact>{});
        if constexpr (!kExact) {
#pragma unroll
            for (int v = 0; v < DV; ++v) nonfinite |= !__builtin_isfinite(cz[0][v]);
        }
    };
    // End of a group: (q - z) sums times the group scale into tot.  acc[x][q]
    // element v is D row 4 g + v = (row 2 g + v / 2, half e = v & 1), column
    // 8 (word + x) + q + 4 e of the lane's words.
    auto flush = [&](const u32x4 (&sv)[WL]) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < WL; ++x) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int v = 0; v < DV; ++v) {
                    const int c = q + 4 * (v & 1);  // column within the word
                    const float s = f16_bits_to_f32((sv[x][c >> 1] >> (16 * (c & 1))) & 0xffffu);
                    const float d = kExact ? acc[x][q][v] : acc[x][q][v] - cz[q & 1][v];
                    tot[x][q][v] = __builtin_fmaf(s, d, tot[x][q][v]);
                }
        }
    };

    // chunks c_begin + wave, + 8, ...: the workgroup's waves read consecutive
    // rows.  With the row held in registers the per-lane row sums run while
    // the first chunk's weights are in flight (first chunk peeled); the
    // cross-lane part follows where every lane of the wave is active.
    const int c0 = c_begin + wave;
    int c = c0;
    if constexpr (kEarlyRows) {
        // (c is the same in every lane of the wave, so each branch below runs
        // with the whole wave active)
        if (c0 < c_end) {
            Chunk d;
            load_chunk(c0, d);
            rows.partials(src, ld, K);
            chunk(d);
            flush(d.sv);
        } else {
            rows.partials(src, ld, K);
        }
        c += NW;
        // the cross-lane row sums while the second chunk's loads are in flight
        if (c < c_end) {
            Chunk d;
            load_chunk(c, d);
            rows.reduce(s_part, lane, wave);
            chunk(d);
            flush(d.sv);
            c += NW;
        } else {
            rows.reduce(s_part, lane, wave);
        }
    }
    for (; c < c_end; c += NW) {
        Chunk d;
        load_chunk(c, d);
        chunk(d);
        flush(d.sv);
    }
    // Rare: some activation of the wave's chunks was not finite.  Redo them
    // all with exact (q - z) weights (wave-uniform branch).
    if (!kExact && __builtin_amdgcn_ballot_w64(nonfinite) != 0) {
#pragma unroll
        for (int x = 0; x < WL; ++x)
#pragma unroll
            for (int q = 0; q < 4; ++q) tot[x][q] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ce = c0; ce < c_end; ce += NW) {
            Chunk d;
            load_chunk(ce, d);
            zero_acc();
            mma_chunk(d, std::true_type{});
            flush(d.sv);
        }
    }
    if constexpr (ACT != 0 && !kEarlyRows) {
        rows.partials(src, ld, K);
        rows.reduce(s_part, lane, wave);
    }

    auto row_scale_fn = [&](int m) __attribute__((always_inline)) {
        if constexpr (ACT != 0) return RowSums<M, ACT, RV, kEarlyRows>::inv(s_part, m, K);
        else return 1.0f;
    };
    __shared__ float red[NW][M][TC];
#pragma unroll
    for (int v = 0; v < DV; ++v) {
        const int m = 2 * g + (v >> 1);
        if (m < M) {
#pragma unroll
            for (int x = 0; x < WL; ++x) {
                const f32x4 o = {tot[x][0][v], tot[x][1][v], tot[x][2][v], tot[x][3][v]};
                *reinterpret_cast<f32x4 *>(&red[wave][m][8 * WL * j + 8 * x + 4 * (v & 1)]) = o;
            }
        }
    }
    __syncthreads();
    finish_tile<M, NW, decltype(row_scale_fn), TC>(red, row_scale_fn, tile, N, splits, out, counters);
}

template <int M, int WORDS, int NW, bool ASYM, bool FOLD, int ACT, int RV = 1>
hipError_t launch_k(const GemmArgs &g, const GemmPlan &p, const uint16_t *src, int ld, hipStream_t stream) {
    hipLaunchKernelGGL((gemv_kernel<M, WORDS, NW, ASYM, FOLD, ACT, RV>), dim3((unsigned)p.grid), dim3(64 * NW), 0,
                       stream, g.a, src, ld, reinterpret_cast<const uint32_t *>(g.b), g.scales,
                       reinterpret_cast<const uint32_t *>(g.qzeros), (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp,
                       (int)p.tiles_n, (int)p.split_len, p.splits, g.out, g.counters);
    return hipGetLastError();
}

// Glue-fused variants.  With a symmetric zero point at M <= 2 they take the
// folded form, like the plain GEMV there (measured on MI355X: the 40-layer
// 8B-class decode step 1691 -> 1622 us at M = 1, 2354 -> 2229 us at M = 2);
// with packed zeros, and at M >= 3, the exact form.  At M <= 2 the row's
// vectors are held in registers from the start: RV per virtual thread, the
// glue kernels' own count for a row of K values.
template <int M>
constexpr bool kFoldAct = M <= 2;
template <int M, int WORDS, int ACT>
hipError_t launch_act(const GemmArgs &g, const GemmPlan &p, const uint16_t *src, int ld, hipStream_t stream) {
    const int64_t per = (g.K / 8 + 1023) / 1024;
    if (M <= 2 && per > 2)
        return g.qzeros ? launch_k<M, WORDS, 8, true, false, ACT, 4>(g, p, src, ld, stream)
                        : launch_k<M, WORDS, 8, false, kFoldAct<M>, ACT, 4>(g, p, src, ld, stream);
    if (M <= 2 && per > 1)
        return g.qzeros ? launch_k<M, WORDS, 8, true, false, ACT, 2>(g, p, src, ld, stream)
                        : launch_k<M, WORDS, 8, false, kFoldAct<M>, ACT, 2>(g, p, src, ld, stream);
    return g.qzeros ? launch_k<M, WORDS, 8, true, false, ACT, 1>(g, p, src, ld, stream)
                    : launch_k<M, WORDS, 8, false, kFoldAct<M>, ACT, 1>(g, p, src, ld, stream);
}

template <int M, int WORDS, int NW>
hipError_t launch_v(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    if (g.qzeros)
        return p.fold_asym ? launch_k<M, WORDS, NW, true, true, 0>(g, p, nullptr, 0, stream)
                           : launch_k<M, WORDS, NW, true, false, 0>(g, p, nullptr, 0, stream);
    return p.fold ? launch_k<M, WORDS, NW, false, true, 0>(g, p, nullptr, 0, stream)
                  : launch_k<M, WORDS, NW, false, false, 0>(g, p, nullptr, 0, stream);
}

template <int M, int WORDS>
hipError_t launch_m(const GemmArgs &g, const GemmPlan &p, int act, const uint16_t *src, int ld, hipStream_t stream) {
    if (act == 1) return launch_act<M, WORDS, 1>(g, p, src, ld, stream);
    if (act == 2) return launch_act<M, WORDS, 2>(g, p, src, ld, stream);
    return p.waves == 8 ? launch_v<M, WORDS, 8>(g, p, stream) : launch_v<M, WORDS, 4>(g, p, stream);
}

template <int M, int ZM, int ACT, int RV>
hipError_t launch_mma_k(const GemmArgs &g, const GemmPlan &p, const uint16_t *src, int ld, hipStream_t stream) {
    if constexpr (M <= 2 && ACT <= 1) {
        // 512-column tiles (4 words per lane), planned at M <= 2 where they fill more of the chip
        if (p.words == 4) {
            hipLaunchKernelGGL((gemv_mma_kernel<M, ZM, ACT, RV, 4>), dim3((unsigned)p.grid), dim3(512), 0, stream,
                               g.a, src, ld, reinterpret_cast<const uint32_t *>(g.b), g.scales,
                               reinterpret_cast<const uint32_t *>(g.qzeros), (int)g.K, (int)g.N, (int)g.G,
                               (uint32_t)g.zp, (int)p.tiles_n, (int)p.split_len, p.splits, g.out, g.counters);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemv_mma_kernel<M, ZM, ACT, RV>), dim3((unsigned)p.grid), dim3(512), 0, stream, g.a, src,
                       ld, reinterpret_cast<const uint32_t *>(g.b), g.scales,
                       reinterpret_cast<const uint32_t *>(g.qzeros), (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp,
                       (int)p.tiles_n, (int)p.split_len, p.splits, g.out, g.counters);
    return hipGetLastError();
}

// Packed zeros: the exact form; symmetric zero point: folded (default) or,
// with plan.exact, the exact form.
template <int M, int ACT, int RV>
hipError_t launch_mma_z(const GemmArgs &g, const GemmPlan &p, const uint16_t *src, int ld, hipStream_t stream) {
    if (g.qzeros) return launch_mma_k<M, kZeroPacked, ACT, RV>(g, p, src, ld, stream);
    return p.exact ? launch_mma_k<M, kZeroExact, ACT, RV>(g, p, src, ld, stream)
                   : launch_mma_k<M, kZeroFolded, ACT, RV>(g, p, src, ld, stream);
}

// Glue-fused variants: at M <= 2 the row's vectors are held in registers
// from the start, RV per virtual thread (the glue kernels' own count).
template <int M, int ACT>
hipError_t launch_mma_act(const GemmArgs &g, const GemmPlan &p, const uint16_t *src, int ld, hipStream_t stream) {
    const int64_t per = (g.K / 8 + 1023) / 1024;
    if (M <= 2 && per > 2) return launch_mma_z<M, ACT, 4>(g, p, src, ld, stream);
    if (M <= 2 && per > 1) return launch_mma_z<M, ACT, 2>(g, p, src, ld, stream);
    return launch_mma_z<M, ACT, 1>(g, p, src, ld, stream);
}

template <int M>
hipError_t launch_mma(const GemmArgs &g, const GemmPlan &p, int act, const uint16_t *src, int ld, hipStream_t stream) {
    if (act == 1) return launch_mma_act<M, 1>(g, p, src, ld, stream);
    if (act == 2) return launch_mma_act<M, 2>(g, p, src, ld, stream);
    return launch_mma_z<M, 0, 1>(g, p, nullptr, 0, stream);
}

}  // namespace

hipError_t launch_gemv(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    return launch_gemv_act(g, p, 0, nullptr, 0, stream);
}

hipError_t launch_gemv_act(const GemmArgs &g, const GemmPlan &p, int act, const uint16_t *src, int64_t ld,
                           hipStream_t stream) {
    if (p.splits > kGemvMaxSplits) return hipErrorInvalidValue;
    if (act != 0 && (p.waves != 8 || !src || ld % 8 != 0 || g.K % 8 != 0 || g.K > kGlueMaxWidth))
        return hipErrorInvalidValue;
    if (p.mma) {
        if (p.waves != 8 || g.N % 32 != 0 || g.G % kMmaChunkRows != 0 || (p.words == 4 && (g.M > 2 || act == 2)))
            return hipErrorInvalidValue;
        switch (g.M) {
            case 1: return launch_mma<1>(g, p, act, src, (int)ld, stream);
            case 2: return launch_mma<2>(g, p, act, src, (int)ld, stream);
            case 3: return launch_mma<3>(g, p, act, src, (int)ld, stream);
            case 4: return launch_mma<4>(g, p, act, src, (int)ld, stream);
            case 5: return launch_mma<5>(g, p, act, src, (int)ld, stream);
            case 6: return launch_mma<6>(g, p, act, src, (int)ld, stream);
            case 7: return launch_mma<7>(g, p, act, src, (int)ld, stream);
            case 8: return launch_mma<8>(g, p, act, src, (int)ld, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (g.M) {
        case 1: return launch_m<1, 4>(g, p, act, src, (int)ld, stream);
        case 2: return launch_m<2, 4>(g, p, act, src, (int)ld, stream);
        case 3: return launch_m<3, 2>(g, p, act, src, (int)ld, stream);
        case 4: return launch_m<4, 2>(g, p, act, src, (int)ld, stream);
        case 5: return launch_m<5, 1>(g, p, act, src, (int)ld, stream);
        case 6: return launch_m<6, 1>(g, p, act, src, (int)ld, stream);
        case 7: return launch_m<7, 1>(g, p, act, src, (int)ld, stream);
        case 8: return launch_m<8, 1>(g, p, act, src, (int)ld, stream);
        default: return hipErrorInvalidValue;
    }
}

int gemv_words_for_m(int64_t M) { return M <= 2 ? 4 : (M <= 4 ? 2 : 1); }

}  // namespace w4a16
