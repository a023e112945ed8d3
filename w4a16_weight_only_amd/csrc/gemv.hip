// gemv.hip -- W4A16 split-K GEMV for M <= 8 rows on the vector ALUs (gfx950).
//
// out = a . ((q - z) * s)  (vLLM PR #37352 write-up, "Code analysis" item 1).
// Decode is bound by streaming the weights once (inference-engine article,
// section 1.2), so this kernel is built around the weight stream:
//
//  * A workgroup owns a 256-column tile (32 packed words = 128 bytes of every
//    weight row) and a K-split.  In a wave, CL "column lanes" cover the 128
//    bytes of a row with WORDS-word loads (16 bytes when WORDS = 4) and RL =
//    64/CL "row lanes" take different 16-row chunks, so every load
//    instruction reads whole 128-byte lines.
//  * Each lane unpacks its nibbles in registers two rows at a time (see
//    device.h), subtracts the zero point exactly in fp16 and accumulates
//    a_k*(q-z) for the row pair with one v_dot2_f32_f16 (fp32 accumulate).
//    The 16-row chunk lies inside one K-group, so the group scale is applied
//    once per chunk in fp32.  No matrix cores: at M <= 8 the work is a
//    bandwidth-bound matrix-vector product.
//  * Row lanes are reduced with a transpose-reduce over lane-xor shuffles
//    (each step halves the values a lane holds), waves through LDS, and
//    K-splits through an fp32 partials buffer: the last workgroup to arrive at
//    a tile's counter sums the splits in split order (deterministic; the
//    reduce-in-shared-memory-not-float-atomics lesson of the same article,
//    section 3.4) and resets the counter for the next call.
#include "device.h"
#include "kernels.h"

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

// One byte position B of one word pair: two columns (nibbles 2B, 2B+1) x two
// rows, accumulated into p[m][col0 + 2B], p[m][col0 + 2B + 1].
template <int M, int COLS, int B>
__device__ __forceinline__ void dot_byte(uint32_t lo, uint32_t hi, const f16x2 *zc, int col0,
                                         const uint32_t (&apair)[M], float (&p)[M][COLS]) {
    uint32_t pr = gather_byte_pair<B>(lo, hi);
    f16x2 v0 = as_f16x2(biased_pair<0>(pr)) - zc[col0 + 2 * B];
    f16x2 v1 = as_f16x2(biased_pair<1>(pr)) - zc[col0 + 2 * B + 1];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        f16x2 av = as_f16x2(apair[m]);
        p[m][col0 + 2 * B] = __builtin_amdgcn_fdot2(v0, av, p[m][col0 + 2 * B], false);
        p[m][col0 + 2 * B + 1] = __builtin_amdgcn_fdot2(v1, av, p[m][col0 + 2 * B + 1], false);
    }
}

template <int M, int WORDS, int NWAVES, bool ASYM>
__global__ __launch_bounds__(64 * NWAVES) void gemv_kernel(
    const uint16_t *__restrict__ a, const uint32_t *__restrict__ b,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros, int K, int N, int G,
    uint32_t zp, int split_len, int splits, uint16_t *__restrict__ out,
    float *__restrict__ partials, uint32_t *__restrict__ counters) {
    constexpr int CL = kTileWords / WORDS;  // column lanes per row segment
    constexpr int RL = 64 / CL;             // row lanes
    constexpr int COLS = 8 * WORDS;         // columns per lane
    static_assert(COLS == 4 * RL, "four columns per lane after the row-lane reduction");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cl = lane % CL;
    const int rl = lane / CL;
    const int N8 = N >> 3;
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int word0 = tile * kTileWords + cl * WORDS;
    const bool col_ok = word0 < N8;  // N % 32 == 0: a lane's words are all in or all out
    const int nchunks = K / kChunkRows;
    const int c_begin = split * split_len;
    const int c_end = min(c_begin + split_len, nchunks);

    float acc[M][COLS];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int j = 0; j < COLS; ++j) acc[m][j] = 0.f;

    for (int c = c_begin + wave * RL + rl; c < c_end; c += NWAVES * RL) {
        const int k0 = c * kChunkRows;
        const int g = k0 / G;

        Words<WORDS> w[kChunkRows];
        if (col_ok) {
#pragma unroll
            for (int r = 0; r < kChunkRows; ++r)
                w[r] = load_words<WORDS>(b + (size_t)(k0 + r) * N8 + word0);
        } else {
#pragma unroll
            for (int r = 0; r < kChunkRows; ++r)
#pragma unroll
                for (int x = 0; x < WORDS; ++x) w[r].v[x] = 0u;
        }
        // a[m][k0 .. k0+15] as 8 fp16 pairs per row.
        uint32_t av[M][8];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const u32x4 *ap = reinterpret_cast<const u32x4 *>(a + (size_t)m * K + k0);
            u32x4 lo = ap[0], hi = ap[1];
            av[m][0] = lo.x; av[m][1] = lo.y; av[m][2] = lo.z; av[m][3] = lo.w;
            av[m][4] = hi.x; av[m][5] = hi.y; av[m][6] = hi.z; av[m][7] = hi.w;
        }
        // Scales of the lane's COLS columns in group g (COLS fp16 = WORDS x 16 bytes).
        uint32_t sw[COLS / 2];
        if (col_ok) {
            const u32x4 *sp = reinterpret_cast<const u32x4 *>(scales + (size_t)g * N + word0 * 8);
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                u32x4 t = sp[x];
                sw[4 * x] = t.x; sw[4 * x + 1] = t.y; sw[4 * x + 2] = t.z; sw[4 * x + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int x = 0; x < COLS / 2; ++x) sw[x] = 0u;
        }
        f16x2 zc[COLS];
        if (ASYM) {
            Words<WORDS> zw;
            if (col_ok) {
                zw = load_words<WORDS>(qzeros + (size_t)g * N8 + word0);
            } else {
#pragma unroll
                for (int x = 0; x < WORDS; ++x) zw.v[x] = 0u;
            }
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                zc[8 * x + 0] = zero_pair_from_word<0>(zw.v[x]);
                zc[8 * x + 1] = zero_pair_from_word<1>(zw.v[x]);
                zc[8 * x + 2] = zero_pair_from_word<2>(zw.v[x]);
                zc[8 * x + 3] = zero_pair_from_word<3>(zw.v[x]);
                zc[8 * x + 4] = zero_pair_from_word<4>(zw.v[x]);
                zc[8 * x + 5] = zero_pair_from_word<5>(zw.v[x]);
                zc[8 * x + 6] = zero_pair_from_word<6>(zw.v[x]);
                zc[8 * x + 7] = zero_pair_from_word<7>(zw.v[x]);
            }
        } else {
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                zc[8 * x + 0] = zero_pair_const<0>(zp);
                zc[8 * x + 1] = zero_pair_const<1>(zp);
                zc[8 * x + 2] = zero_pair_const<2>(zp);
                zc[8 * x + 3] = zero_pair_const<3>(zp);
                zc[8 * x + 4] = zero_pair_const<4>(zp);
                zc[8 * x + 5] = zero_pair_const<5>(zp);
                zc[8 * x + 6] = zero_pair_const<6>(zp);
                zc[8 * x + 7] = zero_pair_const<7>(zp);
            }
        }

        float p[M][COLS];
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int j = 0; j < COLS; ++j) p[m][j] = 0.f;

#pragma unroll
        for (int j = 0; j < 8; ++j) {  // row pair (k0 + 2j, k0 + 2j + 1)
            uint32_t apair[M];
#pragma unroll
            for (int m = 0; m < M; ++m) apair[m] = av[m][j];
#pragma unroll
            for (int x = 0; x < WORDS; ++x) {
                const uint32_t lo = w[2 * j].v[x], hi = w[2 * j + 1].v[x];
                dot_byte<M, COLS, 0>(lo, hi, zc, 8 * x, apair, p);
                dot_byte<M, COLS, 1>(lo, hi, zc, 8 * x, apair, p);
                dot_byte<M, COLS, 2>(lo, hi, zc, 8 * x, apair, p);
                dot_byte<M, COLS, 3>(lo, hi, zc, 8 * x, apair, p);
            }
        }
#pragma unroll
        for (int j = 0; j < COLS; ++j) {
            const uint32_t bits = (j & 1) ? (sw[j >> 1] >> 16) : (sw[j >> 1] & 0xffffu);
            const float s = f16_bits_to_f32(bits);
#pragma unroll
            for (int m = 0; m < M; ++m) acc[m][j] = __builtin_fmaf(s, p[m][j], acc[m][j]);
        }
    }

    // Transpose-reduce over the row lanes (lane bits 5 .. log2(CL)): after the
    // step with mask 2^b the lanes with that bit set keep the upper half of
    // their values.  Lane (cl, rl) ends with columns cl*COLS + 4*rl + 0..3.
#pragma unroll
    for (int step = 0; (32 >> step) >= CL; ++step) {
        const int mask = 32 >> step;
        const int half = COLS >> (step + 1);
        const bool upper = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float lo = acc[m][i], hi = acc[m][half + i];
                const float keep = upper ? hi : lo;
                const float send = upper ? lo : hi;
                acc[m][i] = keep + __shfl_xor(send, mask);
            }
        }
    }

    __shared__ float red[NWAVES][M][kTileCols];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        f32x4 v = {acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        *reinterpret_cast<f32x4 *>(&red[wave][m][cl * COLS + 4 * rl]) = v;
    }
    __syncthreads();

    const int col_base = tile * kTileCols;
    for (int t = threadIdx.x; t < kTileCols; t += 64 * NWAVES) {
        const int col = col_base + t;
        if (col >= N) continue;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float s = 0.f;
#pragma unroll
            for (int wv = 0; wv < NWAVES; ++wv) s += red[wv][m][t];
            if (splits == 1)
                out[(size_t)m * N + col] = f32_to_f16_bits(s);
            else
                partials[((size_t)split * M + m) * N + col] = s;
        }
    }
    if (splits == 1) return;

    // Split-K: the last workgroup to arrive sums every split in split order.
    fence_release_agent();
    __syncthreads();
    __shared__ uint32_t last;
    if (threadIdx.x == 0) last = (arrive_agent(&counters[tile]) == (uint32_t)(splits - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    fence_acquire_agent();
    for (int t = threadIdx.x; t < kTileCols; t += 64 * NWAVES) {
        const int col = col_base + t;
        if (col >= N) continue;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float s = 0.f;
            for (int sp = 0; sp < splits; ++sp) s += partials[((size_t)sp * M + m) * N + col];
            out[(size_t)m * N + col] = f32_to_f16_bits(s);
        }
    }
    if (threadIdx.x == 0) reset_counter_agent(&counters[tile]);
}

template <int M, int WORDS>
hipError_t launch_m(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    constexpr int NW = 4;
    dim3 grid((unsigned)p.tiles_n, (unsigned)p.splits, 1);
    dim3 block(64 * NW, 1, 1);
    const uint32_t *b = reinterpret_cast<const uint32_t *>(g.b);
    const uint32_t *qz = reinterpret_cast<const uint32_t *>(g.qzeros);
    if (g.qzeros)
        hipLaunchKernelGGL((gemv_kernel<M, WORDS, NW, true>), grid, block, 0, stream, g.a, b,
                           g.scales, qz, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp,
                           (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    else
        hipLaunchKernelGGL((gemv_kernel<M, WORDS, NW, false>), grid, block, 0, stream, g.a, b,
                           g.scales, qz, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp,
                           (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    switch (g.M) {
        case 1: return launch_m<1, 4>(g, p, stream);
        case 2: return launch_m<2, 4>(g, p, stream);
        case 3: return launch_m<3, 2>(g, p, stream);
        case 4: return launch_m<4, 2>(g, p, stream);
        case 5: return launch_m<5, 1>(g, p, stream);
        case 6: return launch_m<6, 1>(g, p, stream);
        case 7: return launch_m<7, 1>(g, p, stream);
        case 8: return launch_m<8, 1>(g, p, stream);
        default: return hipErrorInvalidValue;
    }
}

int gemv_words_for_m(int64_t M) { return M <= 2 ? 4 : (M <= 4 ? 2 : 1); }

}  // namespace w4a16
