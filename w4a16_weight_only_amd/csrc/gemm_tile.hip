// gemm_tile.hip -- W4A16 GEMM for larger M on the CDNA4 matrix cores
// (gfx950): 128-row x 256-column workgroup tiles whose activations and
// dequantised weights are both shared through LDS, every global load reading
// whole 128-byte lines.
//
// out = a . ((q - z) * s)  (vLLM PR #37352 write-up, "Code analysis" item 1),
// with v_mfma_f32_16x16x32_f16 on the exact integers (q - z) in fp16 and each
// group's scale applied to that group's fp32 sums.
//
// Workgroup: 8 waves = 4 row waves (wm, 32 rows each) x 2 column waves (wn,
// 128 columns each); one K stream per workgroup.  The operand mapping is the
// other MFMA kernels': in the B operand of column tile o a lane (j16, kq)
// holds column 8 * word + o of its word for rows 8 kq .. 8 kq + 7 of the
// 32-row step, two rows per register.  Per step:
//   * activations: the workgroup's 128 rows x 64 bytes are loaded two steps at a
//     time (128 bytes of a row = one line; lane l reads 16 bytes of row
//     (l >> 3) of an 8-row block), written once into an LDS buffer (XOR-
//     swizzled so the MFMA-layout reads hit distinct banks) and read back by
//     the row waves that need them -- each byte crosses the load units once
//     per workgroup instead of once per column wave;
//   * packed weights: 32 rows x 128 bytes (a whole line per row); wave
//     (wm, wn) loads rows 8 kq + 2 wm + h for kq in {2 wn, 2 wn + 1} (a line
//     per quarter wave), and converts register wm of all eight B operands of
//     both column halves for those kq, writing them to a double-buffered LDS
//     fragment tile: each weight is converted once per workgroup;
//   * after the step's barrier each wave reads its half's eight B operands and
//     its two A operands and issues 16 MFMAs, then converts its share of the
//     next step.
// Group scales and packed zeros of the workgroup's K range are staged in LDS
// once.  K-splits across workgroups meet in split order through fp32
// partials (the last arriving workgroup of a tile sums them).
#include "device.h"
#include "kernels.h"
#include "store.h"

namespace w4a16 {
namespace {

constexpr int kRows = 128, kWords = 32;  // 256 columns
constexpr int kGS = kTileGroupSlots;

// LDS layout (bytes)
constexpr int kFragBytes = 2 * 2 * 8 * 4 * 256;  // [buf][half][op][j][lane] u32
constexpr int kABytes = 2 * kRows * 128;         // [buf][row][128 B] (two steps of k)
constexpr int kScaleBytes = kGS * 512;           // [group][256 columns] fp16
constexpr int kZeroBytes = kGS * 128;            // [group][32 words] u32
constexpr int kTileLds = kFragBytes + kABytes + kScaleBytes + kZeroBytes;

__device__ __forceinline__ void lds_barrier_t() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16-byte slot of chunk c (0..7) in row r of an activation buffer: rows r and
// r + 1 share a 256-byte bank window, so 16 consecutive rows at one chunk
// land on 16 distinct slots.
__device__ __forceinline__ int a_slot(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int SPG, bool ASYM>
__global__ __launch_bounds__(512) void mfma_tile_kernel(
    const uint16_t *__restrict__ a, const uint32_t *__restrict__ b, const uint16_t *__restrict__ scales,
    const uint32_t *__restrict__ qzeros, int M, int K, int N, int G, uint32_t zp, int tiles_n, int tiles_m,
    int m_group, int split_len, int splits, uint16_t *__restrict__ out, float *__restrict__ partials,
    uint32_t *__restrict__ counters) {
    constexpr int RB = 4;                 // packed-weight ring: loads three steps ahead
    constexpr int U = SPG > 4 ? SPG : 4;  // steps per loop iteration: static ring slots
    static_assert(U % RB == 0 && U % 4 == 0 && U % SPG == 0, "static ring slots per iteration");

    __shared__ __attribute__((aligned(16))) uint8_t smem[kTileLds];
    uint32_t *const frag = reinterpret_cast<uint32_t *>(smem);
    uint8_t *const abuf = smem + kFragBytes;
    uint16_t *const sl = reinterpret_cast<uint16_t *>(smem + kFragBytes + kABytes);
    uint32_t *const zl = reinterpret_cast<uint32_t *>(smem + kFragBytes + kABytes + kScaleBytes);

    // Logical workgroup (XCD-contiguous runs; grid is a multiple of 8), split,
    // then bands of m_group row tiles per column tile.
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
    const int wm = wave & 3;
    const int wn = wave >> 2;
    const int j16 = lane & 15;
    const int kq = lane >> 4;
    const int N8 = N >> 3;
    const int word0 = tile_n * kWords;
    const int word = word0 + 16 * wn + j16;  // this lane's output word
    const bool col_ok = word < N8;
    const int m0 = tile_m * kRows + 32 * wm;
    const NibbleConsts nk = nibble_consts();

    const int nsteps = K / 32;
    const int s_begin = split * split_len;
    const int s_end = min(s_begin + split_len, nsteps);
    const int n_my = s_end - s_begin;                 // steps of this split (whole groups)
    const int n_loop = ((n_my + U - 1) / U) * U;      // uniform across the workgroup
    auto stc = [&](int t) __attribute__((always_inline)) { return s_begin + min(t, n_my - 1); };

    const uint32_t row_bytes = (uint32_t)N8 * 4u;
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(b, (uint32_t)((uint64_t)K * N8 * 4));
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a, (uint32_t)((uint64_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(scales, (uint32_t)((uint64_t)(K / G) * N * 2));
    const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(qzeros, ASYM ? (uint32_t)((uint64_t)(K / G) * row_bytes) : 0u);

    // ---- group scales and packed zeros of the split, staged once ----
    // (every load issued before the first store: one round trip)
    {
        const int ng = n_my / SPG, g0 = s_begin / SPG;
        constexpr int kPer = kGS / 8;
        u32x2 sw[kPer];
        uint32_t zw[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int gi = wave + 8 * i;
            const uint32_t g = (uint32_t)(g0 + min(gi, ng - 1));
            sw[i] = buffer_load_x2(srs, (uint32_t)(word0 * 8 + 4 * lane) * 2u, g * (uint32_t)N * 2u);
            if constexpr (ASYM) zw[i] = buffer_load_x1(zrs, (uint32_t)(word0 + (lane & 31)) * 4u, g * row_bytes);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int gi = wave + 8 * i;
            if (gi < ng) {
                *reinterpret_cast<u32x2 *>(sl + gi * 256 + 4 * lane) = sw[i];
                if constexpr (ASYM) {
                    if (lane < 32) zl[gi * 32 + lane] = zw[i];
                }
            }
        }
    }

    // ---- loads ----
    // Activations of super-step S (steps 2S, 2S + 1): wave w loads rows
    // 16 w + 8 i + (lane >> 3), bytes 16 (lane & 7) .. of the 128 (rows past M
    // read row M - 1; k past the split reads on, unused).
    u32x4 araw[2][2];  // [ring slot][i]
    uint32_t a_voff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        a_voff[i] = ((uint32_t)min(tile_m * kRows + 16 * wave + 8 * i + (lane >> 3), M - 1) * (uint32_t)K +
                     8u * (uint32_t)(lane & 7)) * 2u;
    auto issue_a = [&](int S, int slot) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)stc(2 * S) * 64u;
#pragma unroll
        for (int i = 0; i < 2; ++i) araw[slot][i] = buffer_load_x4(ars, a_voff[i], soff);
    };
    auto write_a = [&](int slot, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 16 * wave + 8 * i + (lane >> 3);
            *reinterpret_cast<u32x4 *>(abuf + buf * (kRows * 128) + a_slot(r, lane & 7)) = araw[slot][i];
        }
    };
    // Packed weights of step t: rows 8 kq' + 2 wm + h, kq' = 2 wn + (r' >> 1),
    // h = r' & 1 for r' = lane >> 4; words 2 (lane & 15), + 1 of the tile
    // (words past the matrix's last read on or, past its end, zeros: unused).
    u32x2 braw[RB];
    const int rb = lane >> 4;
    const uint32_t b_voff = ((uint32_t)(8 * (2 * wn + (rb >> 1)) + 2 * wm + (rb & 1)) * (uint32_t)N8 +
                             (uint32_t)(word0 + 2 * (lane & 15))) * 4u;
    auto issue_b = [&](int t, int slot) __attribute__((always_inline)) {
        braw[slot] = buffer_load_x2(brs, b_voff, (uint32_t)stc(t) * 32u * row_bytes);
    };

    // ---- this wave's share of a step's dequantisation ----
    // Lane L makes register wm of the eight operands of half hc = L >> 5 at
    // fragment lane (j16, kq' = 2 wn + ((L >> 4) & 1)): tile word w = 16 hc +
    // j16 of rows 8 kq' + 2 wm + h, held by lane 16 (2 ((L >> 4) & 1) + h) +
    // w / 2 (its word w & 1).
    const int c_hc = lane >> 5, c_sel = (lane >> 4) & 1;
    const int c_w = 16 * c_hc + j16;
    const int c_src0 = (16 * (2 * c_sel) + (c_w >> 1)) * 4, c_src1 = (16 * (2 * c_sel + 1) + (c_w >> 1)) * 4;
    const bool c_odd = (c_w & 1) != 0;
    const int c_lane = j16 + 16 * (2 * wn + c_sel);
    auto convert = [&](int t, int slot, int buf) __attribute__((always_inline)) {
        f16x2 zc[8];
        if constexpr (ASYM) {
            const uint32_t zw = zl[min(t / SPG, kGS - 1) * 32 + c_w];
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
        const uint32_t x0 = (uint32_t)__builtin_amdgcn_ds_bpermute(c_src0, (int)braw[slot].x);
        const uint32_t y0 = (uint32_t)__builtin_amdgcn_ds_bpermute(c_src0, (int)braw[slot].y);
        const uint32_t x1 = (uint32_t)__builtin_amdgcn_ds_bpermute(c_src1, (int)braw[slot].x);
        const uint32_t y1 = (uint32_t)__builtin_amdgcn_ds_bpermute(c_src1, (int)braw[slot].y);
        const uint32_t lo = c_odd ? y0 : x0, hi = c_odd ? y1 : x1;
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
        uint32_t *fd = frag + ((buf * 2 + c_hc) * 8) * 4 * 64 + c_lane;
#pragma unroll
        for (int o = 0; o < 8; ++o) fd[(o * 4 + wm) * 64] = v[o];
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

    // ---- prologue: weights of steps 0..2 and activations of super-steps 0,
    // 1 issued in the loop's order; super-step 0 written, step 0 converted ----
    __syncthreads();  // scales and zeros are in LDS
    issue_b(0, 0);
    asm volatile("" ::: "memory");
    issue_a(0, 0);
    asm volatile("" ::: "memory");
    issue_b(1, 1);
    asm volatile("" ::: "memory");
    issue_b(2, 2);
    asm volatile("" ::: "memory");
    issue_a(1, 1);
    asm volatile("" ::: "memory");
    write_a(0, 0);
    convert(0, 0, 0);
    lds_barrier_t();  // step 0's operands and super-step 0's activations are in LDS

    // ---- main loop: U steps per iteration, ring slots static; at least one
    // iteration ----
    int t0 = 0;
    do {
        static_for<0, U>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = decltype(uc)::value;
            const int t = t0 + u;
            const bool valid = t < n_my;
            issue_b(t + 3, (u + 3) % RB);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (u % 2 == 0) {
                // super-step S = t / 2: activations of S + 2 into slot S % 2
                // (written to LDS one step after S + 1's)
                issue_a(t / 2 + 2, (u / 2) % 2);
                __builtin_amdgcn_sched_barrier(0);
            }
            // this step's operands (written before the last barrier)
            f16x8 bop[8], av[2];
            const uint32_t *fs = frag + (((u & 1) * 2 + wn) * 8) * 4 * 64 + lane;
#pragma unroll
            for (int o = 0; o < 8; ++o)
                bop[o] = __builtin_bit_cast(f16x8, u32x4{fs[(o * 4 + 0) * 64], fs[(o * 4 + 1) * 64],
                                                        fs[(o * 4 + 2) * 64], fs[(o * 4 + 3) * 64]});
            const uint8_t *ab = abuf + ((u / 2) % 2) * (kRows * 128);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                av[mt] = *reinterpret_cast<const f16x8 *>(ab + a_slot(32 * wm + 16 * mt + j16, 4 * (u & 1) + kq));
            if (valid) {
#pragma unroll
                for (int o = 0; o < 8; ++o)
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        if constexpr (u % SPG == 0)
                            acc[mt][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], bop[o],
                                                                                f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                        else
                            acc[mt][o] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], bop[o], acc[mt][o], 0, 0, 0);
                    }
            }
            // the next step's share of the conversion (other fragment buffer)
            convert(t + 1, (u + 1) % RB, (u + 1) & 1);
            if constexpr (u % 2 == 1) {
                // activations of super-step t / 2 + 1 (issued two super-steps
                // ago) into the buffer super-step t / 2 - 1 used
                write_a((u / 2 + 1) % 2, (u / 2 + 1) % 2);
            }
            if constexpr (u % SPG == SPG - 1) {
                if (valid) {
                    const u32x4 scl = *reinterpret_cast<const u32x4 *>(sl + min(t / SPG, kGS - 1) * 256 +
                                                                       8 * (16 * wn + j16));
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
            lds_barrier_t();
        });
        t0 += U;
    } while (t0 < n_loop);

    // ---- store: fp16, or fp32 partials with K-splits ----
    const int tile = tile_m * tiles_n + tile_n;
    const uint32_t plane = (uint32_t)M * (uint32_t)N * 4u;
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(partials, splits > 1 ? (uint32_t)splits * plane : 0u);
    typedef f16 f16x8_t __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int mt = q >> 2, v = q & 3;
        const f32x4 lo = {tot[mt][0][v], tot[mt][1][v], tot[mt][2][v], tot[mt][3][v]};
        const f32x4 hi = {tot[mt][4][v], tot[mt][5][v], tot[mt][6][v], tot[mt][7][v]};
        const int row = m0 + 16 * mt + 4 * kq + v;
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
    if (splits == 1) return;

    // Split-K: the last workgroup of the tile sums every split's fp32 tile in
    // split order and writes fp16; per chunk of units every split's load is
    // issued before the first add.
    wait_vm_zero();
    __syncthreads();
    __shared__ uint32_t last;
    if (threadIdx.x == 0) last = (arrive_agent(&counters[tile]) == (uint32_t)(splits - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last) return;
    constexpr int kRowUnits = 256 / 4;                  // f32x4 units per tile row
    constexpr int kUnits = kRows * kRowUnits / 512, kChunk = 4;
    const int row0 = tile_m * kRows, col0 = tile_n * 256;
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int u0 = 0; u0 < kUnits; u0 += kChunk) {
        f32x4 v[kChunk][kSharedMaxSplits];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int idx = threadIdx.x + (u0 + u) * 512;
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
            const int idx = threadIdx.x + (u0 + u) * 512;
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

template <int SPG>
hipError_t launch_tile_spg(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    if (g.qzeros)
        hipLaunchKernelGGL((mfma_tile_kernel<SPG, true>), dim3((unsigned)p.grid), dim3(512), 0, stream, g.a,
                           reinterpret_cast<const uint32_t *>(g.b), g.scales, reinterpret_cast<const uint32_t *>(g.qzeros),
                           (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp, (int)p.tiles_n, (int)p.tiles_m,
                           p.m_group, (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    else
        hipLaunchKernelGGL((mfma_tile_kernel<SPG, false>), dim3((unsigned)p.grid), dim3(512), 0, stream, g.a,
                           reinterpret_cast<const uint32_t *>(g.b), g.scales, reinterpret_cast<const uint32_t *>(g.qzeros),
                           (int)g.M, (int)g.K, (int)g.N, (int)g.G, (uint32_t)g.zp, (int)p.tiles_n, (int)p.tiles_m,
                           p.m_group, (int)p.split_len, p.splits, g.out, g.partials, g.counters);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_tile(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    if (p.splits > 1 && (!g.partials || !g.counters)) return hipErrorInvalidValue;
    if (!shared_supports(g.G) || p.splits > kSharedMaxSplits) return hipErrorInvalidValue;
    const int64_t spg = g.G / 32;
    if (p.split_len % spg != 0 || p.split_len / spg > kTileGroupSlots) return hipErrorInvalidValue;
    switch (spg) {
        case 1: return launch_tile_spg<1>(g, p, stream);
        case 2: return launch_tile_spg<2>(g, p, stream);
        case 4: return launch_tile_spg<4>(g, p, stream);
        case 8: return launch_tile_spg<8>(g, p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
