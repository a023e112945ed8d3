// gemm_tall.hip -- W4A16 GEMM for the prefill regime (many rows) on the CDNA4
// matrix cores (gfx950): each wave dequantises a narrow column strip once and
// multiplies it against every row tile of the workgroup.
//
// out = a . ((q - z) * s)  (vLLM PR #37352 write-up, "Code analysis" item 1),
// with v_mfma_f32_16x16x32_f16: fp16 operands, fp32 accumulation.  As in the
// other MFMA kernels the B operands are the exact integers (q - z) in fp16
// and each group's fp32 sums are multiplied by the group scale when the
// group ends, so no weight is rounded.
//
// Where the work goes.  At 256 rows the product is bound by the matrix cores
// (about 750 flops per HBM byte), and what competes with them for issue slots
// is the per-weight conversion work and the operand traffic through LDS.  A
// workgroup here owns 128 rows x 128 columns and a K range; each of its four
// waves owns all 128 rows of a 32-column strip (8 row tiles x 2 column tiles
// of 16x16).  So a weight is converted by one wave, once, and feeds 8 MFMAs
// (20 conversion instructions per 16 MFMAs), and the activations, which every
// wave needs, are staged in LDS once per workgroup and read as whole MFMA
// fragments (one ds_read_b128 per row tile and K-step).  Two K-groups of four
// waves can share a workgroup (below), halving the split partials.
//
// B operand mapping.  A 16x16x32 MFMA takes, in lane (j, kq) = (lane % 16,
// lane / 16), eight consecutive k of column j of B.  A packed word holds 8
// columns of one weight row.  Lane j of a wave reads word (j % 4) of the
// wave's four words at rows 8 kq .. 8 kq + 7, and takes byte (j / 4) of each:
// nibble 2 (j / 4) feeds column tile 0 and nibble 2 (j / 4) + 1 column tile 1,
// so the lane's two output columns are adjacent: 8 word + 2 (j / 4) + {0, 1}.
// The byte is gathered with a per-lane v_perm selector and turned into exact
// fp16 (bias + q) by one AND-OR (device.h); one packed subtraction of
// (bias + z) leaves q - z.
//
// Staging.  Per stage of two 32-row K-steps the workgroup copies the A tile
// (128 rows x 64 k, 16 KB) and the packed words (64 rows x 16 words, 4 KB)
// into one of two LDS buffers: the global reads are whole 128-byte lines (two
// rows per quarter wave), requested two stages ahead into one of two register
// sets, and written to LDS at the end of the stage before their own, followed
// by the stage's single barrier.  A fragments sit in LDS in MFMA lane order
// with the slot index XOR-swizzled by the fragment's k-octet and step (lane L
// of block (row tile, step) at slot L ^ (2 (L / 16) + step)), so neither the
// fragment reads nor the line-wise writes meet bank conflicts.  Weight rows
// are 17 words apart in LDS, so the four k-octets of a wave's reads fall in
// different banks.
//
// Reduction.  With K split across workgroups each split writes its fp32 tile
// with device-coherent stores and bumps the tile's arrival counter; the last
// workgroup to arrive sums the splits in split order (deterministic), writes
// fp16 and resets the counter.
#include "device.h"
#include "kernels.h"

#include <type_traits>

namespace w4a16 {
namespace {

constexpr int kThreads = 256;          // four waves
constexpr int kWords = 16;             // workgroup tile: 16 packed words = 128 columns
constexpr int kKS = 2;                 // 32-row K-steps per LDS stage
constexpr int kABlock = 1024;          // one A fragment block: 16 rows x 32 k of fp16
constexpr int kBRowWords = kWords + 1;                // padded LDS row of packed words
constexpr int kBStageWords = 32 * kKS * kBRowWords;
static_assert(32 * kKS * kWords / 4 == kThreads, "one 16-byte B piece per thread per stage");

// Sizes of a workgroup tile of RT MFMA row tiles (16 RT rows; RT = 8 for the
// prefill sizes, fewer for small M).
template <int RT>
struct TallRows {
    static constexpr int kRowTiles = RT;
    static constexpr int kRows = 16 * RT;
    static constexpr int kAStage = RT * kKS * kABlock;
    static constexpr int kAChunks = kRows * kKS * 4 / kThreads;  // 16-byte A pieces per thread per stage
    static constexpr int kTileUnits = kRows * (kWords * 8 / 4);  // f32x4 units of a tile (last arrival)
    static_assert(kAChunks >= 1 && kAChunks * kThreads == kRows * kKS * 4, "whole A pieces per thread");
};

// KG K-groups of four waves per workgroup: each group takes its own part of
// the workgroup's K range with its own LDS stage buffers, and the groups'
// totals meet in LDS (group 0 + group 1) before the split hand-off, so two
// groups halve the fp32 partials of a given number of workgroups per CU.
template <bool ASYM, int KG, int RT>
__global__ __launch_bounds__(kThreads * KG, 2) void tall_kernel(
    const uint16_t *__restrict__ a, const uint32_t *__restrict__ b, const uint16_t *__restrict__ scales,
    const uint32_t *__restrict__ qzeros, int M, int K, int N, int G, uint32_t zp, int tiles_n, int tiles_m,
    int split_len, int splits, uint16_t *__restrict__ out, float *__restrict__ partials,
    uint32_t *__restrict__ counters) {
    using R = TallRows<RT>;
    constexpr int kRows = R::kRows, kRowTiles = R::kRowTiles, kAStage = R::kAStage, kAChunks = R::kAChunks;
    __shared__ __attribute__((aligned(16))) uint8_t s_a[KG][2][kAStage];
    __shared__ uint32_t s_b[KG][2][kBStageWords];

    // Logical workgroup: XCD-contiguous runs (grid a multiple of 8); within a
    // split, the row tiles of one column tile are consecutive (same weights).
    const int logical = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (logical >= tiles_n * tiles_m * splits) return;  // whole workgroup
    const int split = logical / (tiles_n * tiles_m);
    const int rem = logical - split * (tiles_n * tiles_m);
    const int tile_n = rem / tiles_m;
    const int tile_m = rem - tile_n * tiles_m;

    const int tid_all = threadIdx.x;
    const int kg = __builtin_amdgcn_readfirstlane(tid_all >> 8);  // K-group
    const int tid = tid_all & (kThreads - 1);                    // thread within the group
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j16 = lane & 15;
    const int kq = lane >> 4;
    const int wsub = j16 & 3;   // word of the wave's four
    const int bsel = j16 >> 2;  // byte of that word: columns 2 bsel, 2 bsel + 1
    const int N8 = N >> 3;
    const int word = tile_n * kWords + wave * 4 + wsub;
    const bool col_ok = word < N8;
    const int wordc = col_ok ? word : N8 - 1;
    const int m0 = tile_m * kRows;
    const int nsteps = K / 32;
    // The split's steps, then this K-group's share of them (whole stages; every
    // group runs the same number of stages, a group past the split's end none
    // of their steps).
    const int sp_begin = split * split_len;
    const int sp_end = min(sp_begin + split_len, nsteps);
    const int nstages = ((sp_end - sp_begin + kKS - 1) / kKS + KG - 1) / KG;
    const int s_begin = min(sp_begin + kg * nstages * kKS, sp_end);
    const int s_end = min(s_begin + nstages * kKS, sp_end);
    const NibbleConsts nk = nibble_consts();
    // v_perm selector: byte bsel of the first word into byte 0, of the second
    // into byte 2 (bytes 1 and 3 zero)
    const uint32_t sel = 0x0c000c00u | ((4u + (uint32_t)bsel) << 16) | (uint32_t)bsel;

    const uint32_t row_bytes = (uint32_t)N8 * 4u;
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a, (uint32_t)((uint64_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(b, (uint32_t)((uint64_t)K * N8 * 4));
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(scales, (uint32_t)((uint64_t)(K / G) * N * 2));
    const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(qzeros, ASYM ? (uint32_t)((uint64_t)(K / G) * row_bytes) : 0u);

    // A pieces of this thread: piece c = p * 256 + tid is row c / 8, k-octet
    // c % 8 of the stage (step c % 8 / 4, octet kq' = c % 4 within the step).
    // Rows past M read row M - 1 (valid memory, results never stored).  The
    // per-lane part of every staged load's offset is fixed; the stage's first
    // step moves only the wave-uniform part (an SGPR).  Steps past the split's
    // end read other valid bytes or, past the buffer, zeros: never used.
    uint32_t a_voff[kAChunks], a_lds[kAChunks];
#pragma unroll
    for (int p = 0; p < kAChunks; ++p) {
        const int c = p * kThreads + tid;
        const int row = c >> 3, o = c & 7, ks = o >> 2, okq = o & 3;
        a_voff[p] = ((uint32_t)min(m0 + row, M - 1) * (uint32_t)K + 8u * (uint32_t)o) * 2u;
        const int L = (row & 15) + 16 * okq;
        const int slot = L ^ (2 * okq + ks);
        a_lds[p] = (uint32_t)(((row >> 4) * kKS + ks) * kABlock + 16 * slot);
    }
    // B piece of this thread: stage row tid / 4, words 4 (tid % 4) .. + 3 of
    // the tile (pieces wholly past N read the tile's last in-range piece).
    const int b_row = tid >> 2;
    const int b_word = min(tile_n * kWords + 4 * (tid & 3), N8 - 4);
    const uint32_t b_voff = (uint32_t)b_word * 4u + (uint32_t)b_row * row_bytes;
    const int b_lds = b_row * kBRowWords + 4 * (tid & 3);
    // Reads: A fragment slot of this lane per step, B words of its k-octet.
    uint32_t a_frag[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) a_frag[ks] = (uint32_t)(ks * kABlock + 16 * (lane ^ (2 * kq + ks)));
    const int b_rd = (8 * kq) * kBRowWords + wave * 4 + wsub;
    const uint32_t s_voff = ((uint32_t)wordc * 8u + 2u * (uint32_t)bsel) * 2u;
    const uint32_t z_voff = (uint32_t)wordc * 4u;

    // Two register sets of staged loads: stage s travels in set s % 2, is
    // requested two stages before it is computed and written to LDS buffer
    // s % 2 at the end of the stage before.  Every iteration issues the same
    // loads (past the split's last stage they read unused bytes), so the
    // compiler can count them exactly.
    u32x4 a_st[2][kAChunks];
    u32x4 b_st[2];
    auto stage_load = [&](int stg, u32x4 (&ast)[kAChunks], u32x4 &bst) __attribute__((always_inline)) {
        const uint32_t st0 = (uint32_t)(s_begin + stg * kKS);
#pragma unroll
        for (int p = 0; p < kAChunks; ++p) ast[p] = buffer_load_x4(ars, a_voff[p], st0 * 64u);
        bst = buffer_load_x4_nt(brs, b_voff, st0 * 32u * row_bytes);
    };
    auto stage_store = [&](int buf, const u32x4 (&ast)[kAChunks], const u32x4 &bst) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < kAChunks; ++p) *reinterpret_cast<u32x4 *>(&s_a[kg][buf][a_lds[p]]) = ast[p];
        s_b[kg][buf][b_lds + 0] = bst.x;
        s_b[kg][buf][b_lds + 1] = bst.y;
        s_b[kg][buf][b_lds + 2] = bst.z;
        s_b[kg][buf][b_lds + 3] = bst.w;
    };
    // Group scale pair (this lane's two columns) and zero word of group g.
    auto load_sz = [&](int g, uint32_t &sc, uint32_t &zw) __attribute__((always_inline)) {
        sc = buffer_load_x1(srs, s_voff, (uint32_t)g * (uint32_t)N * 2u);
        if constexpr (ASYM) zw = buffer_load_x1(zrs, z_voff, (uint32_t)g * row_bytes);
    };

    // acc: the current group's sums (the group's first step starts them from
    // an inline zero); tot: the scaled totals of the groups before.
    f32x4 acc[kRowTiles][2], tot[kRowTiles][2];
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+v"(z));
            tot[r][c] = z;
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // Group position of a step, tracked without division: (g, r) = (st / G32,
    // st % G32), advanced one step at a time (wave-uniform).
    const int G32 = G >> 5;
    struct Pos {
        int g, r;
    };
    auto advance = [&](Pos q) __attribute__((always_inline)) {
        if (++q.r == G32) {
            q.r = 0;
            ++q.g;
        }
        return q;
    };

    // Products of one K-step from LDS buffer P; FIRST: the first step of a
    // group (or of the split), whose MFMAs start from zero.
    auto step_mfma = [&](const uint8_t *abase, int ks, const f16x8 &b0, const f16x8 &b1, auto first)
        __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < kRowTiles; ++r) {
            const f16x8 af = *reinterpret_cast<const f16x8 *>(abase + r * kKS * kABlock + a_frag[ks]);
            acc[r][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b0, FIRST ? zero : acc[r][0], 0, 0, 0);
            acc[r][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b1, FIRST ? zero : acc[r][1], 0, 0, 0);
        }
    };

    uint32_t sc[kKS], zw[kKS] = {};
    Pos pos0 = {s_begin / G32, s_begin % G32};  // the current stage's first step
    // One stage: compute stage i from LDS buffer P = i % 2 while stage i + 2
    // is requested into register set P and the next stage's scales and zeros
    // arrive (requested first, so waiting for them never waits for stage
    // i + 2); then stage i + 1 goes from set P ^ 1 into buffer P ^ 1, and one
    // barrier.
    auto body = [&](int i, auto par) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;
        const int st0 = s_begin + i * kKS;
        Pos pos[kKS + 1];
        pos[0] = pos0;
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) pos[ks + 1] = advance(pos[ks]);
        // next stage's scales and zeros
        uint32_t scn[kKS], zwn[kKS] = {};
        {
            Pos q = pos[kKS];
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) {
                load_sz(q.g, scn[ks], zwn[ks]);
                q = advance(q);
            }
        }
        stage_load(i + 2, a_st[P], b_st[P]);
        const uint8_t *abase = s_a[kg][P];
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            const int st = st0 + ks;
            if (st >= s_end) break;  // (wave-uniform) last stage of an odd step count
            // this lane's 8 packed words: rows 8 kq .. 8 kq + 7 of the step
            uint32_t w[8];
#pragma unroll
            for (int r = 0; r < 8; ++r) w[r] = s_b[kg][P][b_rd + (32 * ks + r) * kBRowWords];
            f16x2 zc0, zc1;
            if constexpr (ASYM) {
                const uint32_t pz = __builtin_amdgcn_perm(zw[ks], zw[ks], sel);
                zc0 = as_f16x2(biased_pair<0>(pz, nk));
                zc1 = as_f16x2(biased_pair<1>(pz, nk));
            } else {
                zc0 = zero_pair_const<0>(zp);
                zc1 = zero_pair_const<1>(zp);
            }
            f16x8 bop0, bop1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t pr = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], sel);
                const f16x2 v0 = as_f16x2(biased_pair<0>(pr, nk)) - zc0;
                const f16x2 v1 = as_f16x2(biased_pair<1>(pr, nk)) - zc1;
                bop0[2 * j] = v0.x;
                bop0[2 * j + 1] = v0.y;
                bop1[2 * j] = v1.x;
                bop1[2 * j + 1] = v1.y;
            }
            if (pos[ks].r == 0 || st == s_begin)
                step_mfma(abase, ks, bop0, bop1, std::true_type{});
            else
                step_mfma(abase, ks, bop0, bop1, std::false_type{});
            // the group of step st ends here, or the split does
            if (pos[ks].r == G32 - 1 || st + 1 == s_end) {
                const float s0 = f16_bits_to_f32(sc[ks] & 0xffffu), s1 = f16_bits_to_f32(sc[ks] >> 16);
#pragma unroll
                for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        tot[r][0][v] = __builtin_fmaf(s0, acc[r][0][v], tot[r][0][v]);
                        tot[r][1][v] = __builtin_fmaf(s1, acc[r][1][v], tot[r][1][v]);
                    }
            }
        }
        stage_store(P ^ 1, a_st[P ^ 1], b_st[P ^ 1]);
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
            sc[ks] = scn[ks];
            zw[ks] = zwn[ks];
        }
        pos0 = pos[kKS];
        __syncthreads();
    };

    if (nstages > 0) {
        {
            Pos q = pos0;
#pragma unroll
            for (int ks = 0; ks < kKS; ++ks) {
                load_sz(q.g, sc[ks], zw[ks]);
                q = advance(q);
            }
        }
        stage_load(0, a_st[0], b_st[0]);
        stage_load(1, a_st[1], b_st[1]);
        stage_store(0, a_st[0], b_st[0]);
        __syncthreads();
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        int i = 0;
        for (; i + 2 <= nstages; i += 2) {
            body(i, I0{});
            body(i + 1, I1{});
        }
        if (i < nstages) body(i, I0{});
    }

    if constexpr (KG == 2) {
        // Group 1's totals to LDS (the stage buffers are free: every stage ended
        // with a barrier), added to group 0's in that order.
        static_assert(sizeof(s_a) >= sizeof(float) * kRowTiles * 2 * 4 * kThreads, "totals fit the stage buffers");
        float *red = reinterpret_cast<float *>(&s_a[0][0][0]);
        if (kg == 1) {
#pragma unroll
            for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int v = 0; v < 4; ++v) red[((r * 2 + c) * 4 + v) * kThreads + tid] = tot[r][c][v];
        }
        __syncthreads();
        if (kg == 0) {
#pragma unroll
            for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int v = 0; v < 4; ++v) tot[r][c][v] += red[((r * 2 + c) * 4 + v) * kThreads + tid];
        }
    }

    // Epilogue (group 0): lane (j16, kq) holds rows m0 + 16 r + 4 kq + v, columns
    // 8 word + 2 bsel + {0, 1}.
    const int col = word * 8 + 2 * bsel;
    const uint32_t plane = (uint32_t)M * (uint32_t)N * 4u;
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(partials, splits > 1 ? (uint32_t)splits * plane : 0u);
#pragma unroll
    for (int r = 0; r < kRowTiles; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = m0 + 16 * r + 4 * kq + v;
            if (kg != 0 || row >= M || !col_ok) continue;
            if (splits == 1) {
                const uint32_t o = (uint32_t)f32_to_f16_bits(tot[r][0][v]) |
                                   ((uint32_t)f32_to_f16_bits(tot[r][1][v]) << 16);
                *reinterpret_cast<uint32_t *>(out + (size_t)row * N + col) = o;
            } else {
                const uint32_t off = ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 4u;
                buffer_store_f32_sc1(tot[r][0][v], prs, off, (uint32_t)split * plane);
                buffer_store_f32_sc1(tot[r][1][v], prs, off + 4u, (uint32_t)split * plane);
            }
        }
    if (splits == 1) return;

    wait_vm_zero();
    __syncthreads();
    __shared__ uint32_t last;
    const int tile = tile_m * tiles_n + tile_n;
    if (tid_all == 0) last = (arrive_agent(&counters[tile]) == (uint32_t)(splits - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last) return;

    // Last arrival: every thread sums kUnits 16-byte units of the tile over
    // all splits, in split order; per chunk of units every split's load is
    // issued before the first add.
    constexpr int kRowUnits = kWords * 8 / 4;
    const int col0 = tile_n * kWords * 8;
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
    constexpr int kT = kThreads * KG;
    constexpr int kUnits = R::kTileUnits / kT;  // f32x4 units per thread
    constexpr int kChunk = kUnits < 4 ? kUnits : 4;
    static_assert(kUnits * kT == R::kTileUnits && kUnits % kChunk == 0, "whole chunks");
#pragma unroll
    for (int u0 = 0; u0 < kUnits; u0 += kChunk) {
        f32x4 v[kChunk][kTallMaxSplits];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int idx = tid_all + (u0 + u) * kT;
            const int row = m0 + idx / kRowUnits;
            const int c4 = col0 + 4 * (idx % kRowUnits);
            const bool ok = row < M && c4 < N;
            const uint32_t off = ok ? ((uint32_t)row * (uint32_t)N + (uint32_t)c4) * 4u : 0u;
#pragma unroll
            for (int sp = 0; sp < kTallMaxSplits; ++sp)
                v[u][sp] = (ok && sp < splits) ? buffer_load_f32x4_sc1(prs, off, (uint32_t)sp * plane)
                                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int idx = tid_all + (u0 + u) * kT;
            const int row = m0 + idx / kRowUnits;
            const int c4 = col0 + 4 * (idx % kRowUnits);
            if (row >= M || c4 >= N) continue;
            f32x4 s = v[u][0];
#pragma unroll
            for (int sp = 1; sp < kTallMaxSplits; ++sp) s += v[u][sp];
            const u16x4 o = {f32_to_f16_bits(s.x), f32_to_f16_bits(s.y), f32_to_f16_bits(s.z),
                             f32_to_f16_bits(s.w)};
            *reinterpret_cast<u16x4 *>(out + (size_t)row * N + c4) = o;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (tid_all == 0) reset_counter_agent(&counters[tile]);
}

}  // namespace

hipError_t launch_mfma_tall(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    if (p.splits > kTallMaxSplits || p.splits < 1) return hipErrorInvalidValue;
    if (p.splits > 1 && (!g.partials || !g.counters)) return hipErrorInvalidValue;
    if (g.N % 32 != 0 || g.G % 32 != 0) return hipErrorInvalidValue;
    if (p.kwaves != 1 && p.kwaves != 2) return hipErrorInvalidValue;
    auto go = [&](auto kern, int kgroups) {
        hipLaunchKernelGGL(kern, dim3((unsigned)p.grid), dim3(kThreads * kgroups), 0, stream, g.a,
                           reinterpret_cast<const uint32_t *>(g.b), g.scales,
                           reinterpret_cast<const uint32_t *>(g.qzeros), (int)g.M, (int)g.K, (int)g.N, (int)g.G,
                           (uint32_t)g.zp, (int)p.tiles_n, (int)p.tiles_m, (int)p.split_len, p.splits, g.out,
                           g.partials, g.counters);
    };
    auto by_rt = [&](auto rt) {
        constexpr int RT = decltype(rt)::value;
        if (p.kwaves == 2) {
            if (g.qzeros) go(tall_kernel<true, 2, RT>, 2);
            else go(tall_kernel<false, 2, RT>, 2);
        } else {
            if (g.qzeros) go(tall_kernel<true, 1, RT>, 1);
            else go(tall_kernel<false, 1, RT>, 1);
        }
    };
    if (p.mt == 8) by_rt(std::integral_constant<int, 8>{});
    else if (p.mt == 4) by_rt(std::integral_constant<int, 4>{});
    else if (p.mt == 2) by_rt(std::integral_constant<int, 2>{});
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace w4a16
