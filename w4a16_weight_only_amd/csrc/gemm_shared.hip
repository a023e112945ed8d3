// gemm_shared.hip -- W4A16 GEMM for larger M on the CDNA4 matrix cores
// (gfx950), with each K-step's dequantised weights shared through LDS by the
// waves that cover different rows.
//
// out = a . ((q - z) * s)  (vLLM PR #37352 write-up, "Code analysis" item 1),
// with v_mfma_f32_16x16x32_f16 on the exact integers (q - z) in fp16 and each
// group's scale applied to that group's fp32 sums, as in gemm_mfma.hip.
//
// Workgroup: 8 waves = WM row waves x WK = 8 / WM K-waves.  A wave computes 32
// rows x 128 columns (two 16-row MFMA tiles x eight 16-column tiles); the WM
// row waves of a K-wave work on the same K-steps in lockstep.  In the MFMA
// B operand of column tile o a lane holds column 8 * word + o (word = the
// lane's packed word) for the eight rows 8 kq .. 8 kq + 7 of the step
// (kq = lane / 16), two rows per register.  Per 32-row K-step of a K-wave:
//   * row wave wm loads, three steps ahead (with the step's activations,
//     scales and zeros), only the packed rows of the registers it converts: rows 8 kq + 2 j and 8 kq + 2 j + 1 for
//     j = wm (and j = wm + 2 when WM = 2);
//   * it converts them to exact fp16 (q - z) for all eight column tiles --
//     register j of each of the eight B operands -- and writes them to an LDS
//     fragment buffer (double-buffered by step), so each weight is converted
//     once per workgroup instead of once per row wave;
//   * after the step's barrier every row wave reads the eight B operands back
//     (lane-contiguous reads) and issues its 16 MFMAs, then converts its share
//     of the next step.
// The first MFMA of each group starts from an inline zero accumulator (no
// zeroing instructions); at the group's last step the group sums are scaled
// into the running totals.  The K-waves meet through LDS at the end, and
// K-splits across workgroups meet in split order through fp32 partials (the
// last arriving workgroup sums them), as in gemm_mfma.hip.
#include "device.h"
#include "kernels.h"
#include "store.h"

namespace w4a16 {
namespace {

// LDS bytes: fragment buffers, each K-wave's group scales and packed zeros
// (staged once per workgroup), and the K-wave reduction after the loop (which
// reuses the same memory).
template <int WM, int WK>
struct SharedCfg {
    static constexpr int kThreads = 64 * WM * WK;
    static constexpr int kFragBytes = 2 * WK * 8 * 4 * 256;            // [buf][kw][op][j][lane] u32
    static constexpr int kGM = kSharedGroupSlots / WK;                 // group slots per K-wave
    static constexpr int kScaleBytes = kSharedGroupSlots * 256;        // [kw][group][128 columns] fp16
    static constexpr int kZeroBytes = kSharedGroupSlots * 64;          // [kw][group][16 words] u32
    static constexpr int kLoopBytes = kFragBytes + kScaleBytes + kZeroBytes;
    static constexpr int kRedBytes = (WK - 1) * WM * 32 * 128 * 4;     // K-waves 1.. totals
    static constexpr int kLds = kLoopBytes > kRedBytes ? kLoopBytes : kRedBytes;
    // ring of steps in flight in registers: deeper with one wave per SIMD
    static constexpr int kRing = WK == 1 ? 8 : 4;
};

// Workgroup barrier for waves that keep global loads in flight: waits for
// this wave's LDS accesses only (__syncthreads would also drain the
// prefetched global loads), then s_barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int WM, int WK, int SPG, bool ASYM>
__global__ __launch_bounds__(64 * WM * WK) void mfma_shared_kernel(
    const uint16_t *__restrict__ a, const uint32_t *__restrict__ b, const uint16_t *__restrict__ scales,
    const uint32_t *__restrict__ qzeros, int M, int K, int N, int G, uint32_t zp, int tiles_n, int tiles_m,
    int m_group, int split_len, int splits, uint16_t *__restrict__ out, float *__restrict__ partials,
    uint32_t *__restrict__ counters) {
    using C = SharedCfg<WM, WK>;
    constexpr int NT = C::kThreads;
    constexpr int R = C::kRing;           // loads R - 1 steps ahead
    constexpr int U = SPG > R ? SPG : R;  // steps per loop iteration (ring indices stay static)
    constexpr int JPW = 4 / WM;           // row pairs (B registers per operand) each row wave converts
    constexpr int GM = C::kGM;
    static_assert(WM == 2 || WM == 4, "two or four row waves");
    static_assert(U % R == 0 && U % 2 == 0 && U % SPG == 0, "static ring slots per iteration");

    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kLds];
    uint32_t *const frag = reinterpret_cast<uint32_t *>(smem);  // [2][WK][8][4][64]
    uint16_t *const sl = reinterpret_cast<uint16_t *>(smem + C::kFragBytes);                   // [WK][GM][128]
    uint32_t *const zl = reinterpret_cast<uint32_t *>(smem + C::kFragBytes + C::kScaleBytes);  // [WK][GM][16]

    // Logical workgroup (XCD-contiguous runs; grid is a multiple of 8), split,
    // then bands of m_group row tiles per column tile, as in gemm_mfma.hip.
    const int logical = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (logical >= tiles_n * tiles_m * splits) return;  // whole workgroup
    const int split = logical / (tiles_n * tiles_m);
    const int in_split = logical - split * (tiles_n * tiles_m);
    const int band = in_split / (m_group * tiles_n);
    const int in_band = in_split - band * (m_group * tiles_n);
    const int band_rows = min(m_group, tiles_m - band * m_group);
    const int tile_n = in_band / band_rows;
    const int tile_m = band * m_group + (in_band - tile_n * band_rows);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % WM;
    const int kw = wave / WM;
    const int j16 = lane & 15;
    const int kq = lane >> 4;
    const int N8 = N >> 3;
    const int word = tile_n * 16 + j16;
    const bool col_ok = word < N8;
    const int wordc = col_ok ? word : N8 - 1;  // clamped: loads stay in bounds
    const int m0 = tile_m * 32 * WM + 32 * wm;  // this wave's first row
    const NibbleConsts nk = nibble_consts();

    // This K-wave's contiguous run of whole groups within the split; every
    // wave runs the same number of loop steps (whole iterations of U), the
    // steps past its run being dummies that compute nothing but keep the
    // barriers in step.
    const int nsteps = K / 32;
    const int s_begin = split * split_len;
    const int s_end = min(s_begin + split_len, nsteps);
    const int ngroups = (s_end - s_begin) / SPG;
    const int per_kw = (ngroups + WK - 1) / WK;
    const int g_begin = min(kw * per_kw, ngroups);
    const int n_my = SPG * (min(g_begin + per_kw, ngroups) - g_begin);   // valid steps (multiple of SPG)
    const int n_loop = ((SPG * per_kw + U - 1) / U) * U;                  // uniform across the workgroup
    const int st0 = s_begin + SPG * g_begin;
    // step index of loop step t, clamped into this wave's run (or the split's
    // last step when the run is empty): loads of dummy steps stay in bounds
    auto stc = [&](int t) __attribute__((always_inline)) {
        return n_my > 0 ? st0 + min(t, n_my - 1) : s_end - 1;
    };

    const uint32_t row_bytes = (uint32_t)N8 * 4u;
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(b, (uint32_t)((uint64_t)K * N8 * 4));
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a, (uint32_t)((uint64_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(scales, (uint32_t)((uint64_t)(K / G) * N * 2));
    const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(qzeros, ASYM ? (uint32_t)((uint64_t)(K / G) * row_bytes) : 0u);
    // A rows past M read row M - 1, packed words past the tile's last word read
    // on into the next row or (past the end) zeros: their results are never
    // stored

    // ---- loads ----
    // Global loads use lane patterns that touch few cache lines per quarter
    // wave; lane permutes (ds_bpermute) then bring the data into the MFMA
    // operand layout, where each quarter wave would touch 16 rows.
    //  * packed weights: per row pair jj, lane l reads two adjacent words
    //    (2 (l & 7), +1 of the tile) of row (l >> 3) of this wave's 8 rows
    //    8 kq + 2 j + h (kq = (l >> 3) >> 1, h = (l >> 3) & 1);
    //  * activations: per 16-row tile mt, lane l reads 8 k values
    //    (8 (l & 3) ..) of row m0 + 16 mt + (l >> 2).
    u32x2 braw[R][JPW];
    uint32_t b_voff2[JPW];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
        const int rr = lane >> 3;
        b_voff2[jj] = ((uint32_t)(8 * (rr >> 1) + 2 * (wm + WM * jj) + (rr & 1)) * (uint32_t)N8 +
                       (uint32_t)(tile_n * 16 + 2 * (lane & 7))) * 4u;
    }
    auto issue_b = [&](int t, int slot) __attribute__((always_inline)) {
        const uint32_t base = (uint32_t)stc(t) * 32u * row_bytes;
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) braw[slot][jj] = buffer_load_x2(brs, b_voff2[jj], base);
    };
    u32x4 araw[R][2];
    uint32_t a_voff2[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
        a_voff2[mt] = ((uint32_t)min(m0 + 16 * mt + (lane >> 2), M - 1) * (uint32_t)K + 8u * (lane & 3)) * 2u;
    auto issue_a = [&](int t, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) araw[slot][mt] = buffer_load_x4(ars, a_voff2[mt], (uint32_t)stc(t) * 64u);
    };
    // Group scales and packed zeros of this K-wave's run, staged in LDS once
    // (the K-wave's row waves share the loads): lane l of a wave takes the
    // scale pair of columns 2 l, 2 l + 1 of the tile, lanes 0..15 the zero word.
    // (every load issued before the first store: one round trip)
    {
        const int ng = n_my / SPG, g0 = st0 / SPG;
        constexpr int kPer = GM / WM;
        uint32_t sw[kPer], zw0[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int gi = wm + WM * i;
            const uint32_t g = (uint32_t)(g0 + min(gi, max(ng - 1, 0)));
            sw[i] = buffer_load_x1(srs, (uint32_t)(tile_n * 128 + 2 * lane) * 2u, g * (uint32_t)N * 2u);
            if constexpr (ASYM) zw0[i] = buffer_load_x1(zrs, (uint32_t)(tile_n * 16 + (lane & 15)) * 4u, g * row_bytes);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int gi = wm + WM * i;
            if (gi < ng) {
                *reinterpret_cast<uint32_t *>(sl + (kw * GM + gi) * 128 + 2 * lane) = sw[i];
                if constexpr (ASYM) {
                    if (lane < 16) zl[(kw * GM + gi) * 16 + lane] = zw0[i];
                }
            }
        }
    }
    // A operand of row tile mt: lane (j16, kq) takes row j16, k 8 kq .. from
    // lane 4 j16 + kq.
    const int a_src = (4 * j16 + kq) * 4;
    f16x8 av[2][2];  // [step parity][row tile]
    auto permute_a = [&](int slot, int par) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            u32x4 v;
#pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(a_src, (int)araw[slot][mt][d]);
            av[par][mt] = __builtin_bit_cast(f16x8, v);
        }
    };
    // Packed words of rows 8 kq + 2 j + h, word j16: from lane 8 (2 kq + h) +
    // j16 / 2, its word j16 & 1.
    const int b_src0 = (8 * (2 * kq) + (j16 >> 1)) * 4, b_src1 = (8 * (2 * kq + 1) + (j16 >> 1)) * 4;
    const bool b_odd = (j16 & 1) != 0;
    auto permute_b = [&](int slot, int jj, int h) __attribute__((always_inline)) {
        const int src = h ? b_src1 : b_src0;
        const uint32_t x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)braw[slot][jj].x);
        const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)braw[slot][jj].y);
        return b_odd ? y : x;
    };

    // ---- this wave's share of a step's dequantisation ----
    // Register j of every B operand o: (q - z) of rows 2j, 2j+1 of the lane's
    // slice at nibble o.
    // t: the loop step converted (its group's zeros come from LDS)
    auto convert = [&](int t, int slot, int buf) __attribute__((always_inline)) {
        f16x2 zc[8];
        if constexpr (ASYM) {
            const uint32_t zw = zl[(kw * GM + min(t / SPG, GM - 1)) * 16 + j16];
            zc[0] = zero_pair_from_word<0>(zw, nk); zc[1] = zero_pair_from_word<1>(zw, nk);
            zc[2] = zero_pair_from_word<2>(zw, nk); zc[3] = zero_pair_from_word<3>(zw, nk);
            zc[4] = zero_pair_from_word<4>(zw, nk); zc[5] = zero_pair_from_word<5>(zw, nk);
            zc[6] = zero_pair_from_word<6>(zw, nk); zc[7] = zero_pair_from_word<7>(zw, nk);
        } else {
            zc[0] = zero_pair_const<0>(zp); zc[1] = zero_pair_const<1>(zp);
            zc[2] = zero_pair_const<2>(zp); zc[3] = zero_pair_const<3>(zp);
            zc[4] = zero_pair_const<4>(zp); zc[5] = zero_pair_const<5>(zp);
            zc[6] = zero_pair_const<6>(zp); zc[7] = zero_pair_const<7>(zp);
        }
        uint32_t *fd = frag + ((buf * WK + kw) * 8) * 4 * 64 + lane;
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
            const int j = wm + WM * jj;
            const uint32_t lo = permute_b(slot, jj, 0), hi = permute_b(slot, jj, 1);
            uint32_t v[8];
            auto byte = [&](auto bc) __attribute__((always_inline)) {
                constexpr int B = decltype(bc)::value;
                const uint32_t pr = gather_byte_pair<B>(lo, hi);
                v[2 * B] = as_u32(as_f16x2(biased_pair<0>(pr, nk)) - zc[2 * B]);
                v[2 * B + 1] = as_u32(as_f16x2(biased_pair<1>(pr, nk)) - zc[2 * B + 1]);
            };
            byte(std::integral_constant<int, 0>{});
            byte(std::integral_constant<int, 1>{});
            byte(std::integral_constant<int, 2>{});
            byte(std::integral_constant<int, 3>{});
#pragma unroll
            for (int o = 0; o < 8; ++o) fd[(o * 4 + j) * 64] = v[o];
        }
    };

    // ---- accumulators ----
    f32x4 acc[2][8], tot[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int o = 0; o < 8; ++o) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+v"(z));
            tot[mt][o] = z;
            acc[mt][o] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // ---- prologue: steps 0 .. R-2 issued (in the loop's order, so that the
    // waits the compiler derives for the first iteration hold for all), step
    // 0 converted ----
    __syncthreads();  // scales and zeros are in LDS
    static_for<0, R - 1>([&](auto tc) __attribute__((always_inline)) {
        constexpr int t = decltype(tc)::value;
        issue_b(t, t);
        asm volatile("" ::: "memory");
        issue_a(t, t);
        asm volatile("" ::: "memory");
    });
    permute_a(0, 0);
    convert(0, 0, 0);
    lds_barrier();  // step 0's operands are in the fragment buffer

    // ---- main loop: U steps per iteration, ring slots static; at least one
    // iteration (every K-wave's share is at least one group), so the
    // prologue's loads stay ahead of the loop ----
    int t0 = 0;
    do {
        static_for<0, U>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            const int t = t0 + u;
            const bool valid = t < n_my;
            issue_b(t + R - 1, (u + R - 1) % R);
            __builtin_amdgcn_sched_barrier(0);
            issue_a(t + R - 1, (u + R - 1) % R);
            __builtin_amdgcn_sched_barrier(0);
            // this step's operands (written before the last barrier)
            f16x8 bop[8];
            const uint32_t *fs = frag + (((u & 1) * WK + kw) * 8) * 4 * 64 + lane;
#pragma unroll
            for (int o = 0; o < 8; ++o)
                bop[o] = __builtin_bit_cast(f16x8, u32x4{fs[(o * 4 + 0) * 64], fs[(o * 4 + 1) * 64],
                                                        fs[(o * 4 + 2) * 64], fs[(o * 4 + 3) * 64]});
            if (valid) {
#pragma unroll
                for (int o = 0; o < 8; ++o)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        if constexpr (u % SPG == 0)
                            acc[mt][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[u & 1][mt], bop[o],
                                                                                f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        else
                            acc[mt][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[u & 1][mt], bop[o], acc[mt][o],
                                                                                0, 0, 0);
                    }
            }
            // the next step's activations and share of the conversion (into
            // the other fragment buffer)
            permute_a((u + 1) % R, (u + 1) & 1);
            convert(t + 1, (u + 1) % R, (u + 1) & 1);
            if constexpr (u % SPG == SPG - 1) {
                if (valid) {
                    const u32x4 scl = *reinterpret_cast<const u32x4 *>(sl + (kw * GM + min(t / SPG, GM - 1)) * 128 + 8 * j16);
#pragma unroll
                    for (int o = 0; o < 8; ++o) {
                        const float so = f16_bits_to_f32((scl[o >> 1] >> (16 * (o & 1))) & 0xffffu);
#pragma unroll
                        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                            for (int v = 0; v < 4; ++v) tot[mt][o][v] = __builtin_fmaf(so, acc[mt][o][v], tot[mt][o][v]);
                    }
                }
            }
            lds_barrier();  // next step's operands written, this step's read
        });
        t0 += U;
    } while (t0 < n_loop);

    // ---- K-wave reduction: K-waves 1.. write their totals, K-wave 0 sums in
    // order and stores (fp16, or fp32 partials with K-splits) ----
    lds_barrier();  // fragment buffers, scales and zeros are free
    float *red = reinterpret_cast<float *>(smem);  // [(kw-1)][wm][slot 0..7][2 halves][64 lanes] f32x4
    auto red_at = [&](int k, int q, int h) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4 *>(red) + ((((k - 1) * WM + wm) * 8 + q) * 2 + h) * 64 + lane;
    };
    // row slot q = (mt, v): row m0 + 16 mt + 4 kq + v, columns 8 word + 0..7
    auto slot_lo = [&](int q) __attribute__((always_inline)) {
        const int mt = q >> 2, v = q & 3;
        return f32x4{tot[mt][0][v], tot[mt][1][v], tot[mt][2][v], tot[mt][3][v]};
    };
    auto slot_hi = [&](int q) __attribute__((always_inline)) {
        const int mt = q >> 2, v = q & 3;
        return f32x4{tot[mt][4][v], tot[mt][5][v], tot[mt][6][v], tot[mt][7][v]};
    };
    if constexpr (WK > 1) {
        if (kw > 0) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                *red_at(kw, q, 0) = slot_lo(q);
                *red_at(kw, q, 1) = slot_hi(q);
            }
        }
        lds_barrier();
    }
    const int tile = tile_m * tiles_n + tile_n;
    const uint32_t plane = (uint32_t)M * (uint32_t)N * 4u;
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(partials, splits > 1 ? (uint32_t)splits * plane : 0u);
    typedef f16 f16x8_t __attribute__((ext_vector_type(8)));
    if (kw == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            f32x4 lo = slot_lo(q), hi = slot_hi(q);
#pragma unroll
            for (int k = 1; k < WK; ++k) {
                lo += *red_at(k, q, 0);
                hi += *red_at(k, q, 1);
            }
            const int row = m0 + 16 * (q >> 2) + 4 * kq + (q & 3);
            if (row < M && col_ok) {
                if (splits == 1) {
                    f16x8_t o;
                    o[0] = (f16)lo.x; o[1] = (f16)lo.y; o[2] = (f16)lo.z; o[3] = (f16)lo.w;
                    o[4] = (f16)hi.x; o[5] = (f16)hi.y; o[6] = (f16)hi.z; o[7] = (f16)hi.w;
                    *reinterpret_cast<f16x8_t *>(out + (size_t)row * N + word * 8) = o;
                } else {
                    const uint32_t off = ((uint32_t)row * (uint32_t)N + (uint32_t)word * 8u) * 4u;
                    store_partial_x4(lo, prs, off, (uint32_t)split * plane);
                    store_partial_x4(hi, prs, off + 16u, (uint32_t)split * plane);
                }
            }
        }
    }
    if (splits == 1) return;

    // Split-K: the last workgroup of the tile sums every split's fp32 tile in
    // split order and writes fp16.
    wait_vm_zero();
    __syncthreads();
    __shared__ uint32_t last;
    if (threadIdx.x == 0) last = (arrive_agent(&counters[tile]) == (uint32_t)(splits - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    // Every thread sums kUnits 16-byte units of the tile over the splits, in
    // split order; per chunk of units every split's load is issued before the
    // first add.
    constexpr int kRows = 32 * WM, kRowUnits = 128 / 4;  // f32x4 units per tile row
    constexpr int kUnits = kRows * kRowUnits / NT, kChunk = kUnits < 4 ? kUnits : 4;
    static_assert(kUnits % kChunk == 0, "whole chunks");
    const int row0 = tile_m * kRows, col0 = tile_n * 128;
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int u0 = 0; u0 < kUnits; u0 += kChunk) {
        f32x4 v[kChunk][kSharedMaxSplits];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int idx = threadIdx.x + (u0 + u) * NT;
            const int row = row0 + idx / kRowUnits;
            const int col = col0 + 4 * (idx % kRowUnits);
            const bool ok = row < M && col < N;
            const uint32_t off = ok ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 4u : 0u;
#pragma unroll
            for (int sp = 0; sp < kSharedMaxSplits; ++sp)
                v[u][sp] = (ok && sp < splits) ? buffer_load_f32x4_sc1(prs, off, (uint32_t)sp * plane)
                                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int idx = threadIdx.x + (u0 + u) * NT;
            const int row = row0 + idx / kRowUnits;
            const int col = col0 + 4 * (idx % kRowUnits);
            if (row >= M || col >= N) continue;
            f32x4 s = v[u][0];
#pragma unroll
            for (int sp = 1; sp < kSharedMaxSplits; ++sp)
                if (sp < splits) s += v[u][sp];
            const u16x4 o = {f32_to_f16_bits(s.x), f32_to_f16_bits(s.y), f32_to_f16_bits(s.z),
                             f32_to_f16_bits(s.w)};
            *reinterpret_cast<u16x4 *>(out + (size_t)row * N + col) = o;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (threadIdx.x == 0) reset_counter_agent(&counters[tile]);
}

template <int WM, int WK, int SPG>
hipError_t launch_shared_spg(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    constexpr int NT = SharedCfg<WM, WK>::kThreads;
    if (g.qzeros)
        hipLaunchKernelGGL((mfma_shared_kernel<WM, WK, SPG, true>), dim3((unsigned)p.grid), dim3(NT), 0, stream, g.a,
                           reinterpret_cast<const uint32_t *>(g.b), g.scales, reinterpret_cast<const uint32_t *>(g.qzeros),
                           (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp, (int)p.tiles_n, (int)p.tiles_m,
                           p.m_group, (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    else
        hipLaunchKernelGGL((mfma_shared_kernel<WM, WK, SPG, false>), dim3((unsigned)p.grid), dim3(NT), 0, stream, g.a,
                           reinterpret_cast<const uint32_t *>(g.b), g.scales, reinterpret_cast<const uint32_t *>(g.qzeros),
                           (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp, (int)p.tiles_n, (int)p.tiles_m,
                           p.m_group, (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    return hipGetLastError();
}

template <int WM, int WK>
hipError_t launch_shared_wm(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    switch (g.G / 32) {
        case 1: return launch_shared_spg<WM, WK, 1>(g, p, stream);
        case 2: return launch_shared_spg<WM, WK, 2>(g, p, stream);
        case 4: return launch_shared_spg<WM, WK, 4>(g, p, stream);
        case 8: return launch_shared_spg<WM, WK, 8>(g, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace


inline int64_t cdiv_groups(int64_t a, int64_t b) { return (a + b - 1) / b; }

hipError_t launch_mfma_shared(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    if (p.splits > 1 && (!g.partials || !g.counters)) return hipErrorInvalidValue;
    if (!shared_supports(g.G) || p.split_len % (g.G / 32) != 0 || p.splits > kSharedMaxSplits)
        return hipErrorInvalidValue;
    // every K-wave's run of groups fits its LDS scale slots
    const int64_t spg = g.G / 32, groups = p.split_len / spg;
    if (p.kwaves < 1 || cdiv_groups(groups, p.kwaves) > kSharedGroupSlots / p.kwaves) return hipErrorInvalidValue;
    if (p.wm == 4 && p.kwaves == 2) return launch_shared_wm<4, 2>(g, p, stream);
    if (p.wm == 2 && p.kwaves == 4) return launch_shared_wm<2, 4>(g, p, stream);
    if (p.wm == 4 && p.kwaves == 1) return launch_shared_wm<4, 1>(g, p, stream);
    if (p.wm == 2 && p.kwaves == 1) return launch_shared_wm<2, 1>(g, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace w4a16
