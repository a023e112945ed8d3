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
// the epilogue stores 16 contiguous bytes per row.  The operands are the exact
// integers (q - z) in fp16 (device.h); the group scale multiplies the fp32
// sums of each group (group accumulators flushed into running totals when a
// group ends), so no weight is rounded: the same per-group factorisation
// out = sum_g s_g (sum_k a_k (q_k - z_g)) the definition allows, with fp32
// rounding only in the sums.
//
// Pipeline.  A wave computes (16*MT rows) x (128 columns) over a contiguous
// block of 32-row K-steps.  The loop is unrolled by two over a ring of two
// packed-word slots and two A-operand slots, so nothing is copied between
// iterations: the MFMAs of step s run while the VALU dequantises step s+1
// into the B operand registers the MFMAs have just read (explicit scheduling
// regions keep that order), A for step s+1 and B for step s+2 are in flight.
// Loads are issued in the order they are consumed, so waiting for the data of
// one step never waits for a later prefetch.  All loads are buffer loads whose
// per-row/per-step offset is an SGPR: no vector address arithmetic.
//
// Reduction.  A workgroup has NWN waves side by side along N and NWK waves
// dividing its K range; the NWK partial tiles are summed through LDS in fixed
// order.  When the grid also splits K across workgroups, every split writes
// its fp32 tile with device-coherent stores and bumps the tile's arrival
// counter; the workgroup that arrives last reads all splits back and sums
// them in split order (deterministic), writes fp16 and resets the counter.
#include "device.h"
#include "kernels.h"
#include "store.h"

#include <type_traits>

namespace w4a16 {
namespace {

// The last workgroup of a split-K tile keeps at most kSplitLoads 16-byte
// partial loads in flight per thread (a chunk of units x every split).
constexpr int kSplitLoads = 32;

template <int MT, int NWN, int NWK>
struct Cfg {
    static constexpr int kThreads = 64 * NWN * NWK;
    static constexpr int kTileRows = 16 * MT;
    static constexpr int kTileCols = 128 * NWN;
    // f32x4 units of the workgroup tile per thread in the split-K reduction.
    static constexpr int kUnits = kTileRows * (kTileCols / 4) / kThreads;
    static constexpr int kMaxSplits = 8;  // in-flight loads of the last workgroup
    static constexpr int kChunk = kSplitLoads / kMaxSplits < kUnits ? kSplitLoads / kMaxSplits : kUnits;
    static_assert(kUnits >= 1 && kTileRows * (kTileCols / 4) % kThreads == 0, "whole units per thread");
    static_assert(kChunk >= 1 && kUnits % kChunk == 0, "whole chunks");
    // Row tiles per K-wave reduction round: every wave's share of a round
    // (MTC * 8 KB) for all NWN * NWK waves within 128 KB of LDS.
    static constexpr int kRedTiles = (NWN * NWK * MT * 8 <= 128) ? MT : (NWN * NWK * 8 * 2 <= 128 ? 2 : 1);
};

// Values a region must produce where it stands: an empty asm that reads and
// "rewrites" them keeps IR passes from sinking their computation into a
// later region (emits no instruction).
__device__ __forceinline__ void pin(f16x8 &a, f16x8 &b) { asm volatile("" : "+v"(a), "+v"(b)); }
__device__ __forceinline__ void pin2(f16x2 &a, f16x2 &b, f16x2 &c, f16x2 &d) {
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// Scheduling pattern for one region: (one MFMA, then V VALU) NMFMA times.
template <int NMFMA, int V>
__device__ __forceinline__ void interleave() {
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);  // VALU
    }
}

template <int A, int B>
struct Gcd : Gcd<B, A % B> {};
template <int A>
struct Gcd<A, 0> : std::integral_constant<int, A> {};

// Pipeline depths: steps of B (packed words, scales, zeros) and of A in
// flight.  Two B slots: with each group's sums and the scaled totals (128
// accumulator registers at 32-row wave tiles), a third or fourth slot spills.
template <int MT, int NWK>
struct RingW : std::integral_constant<int, 2> {};
template <int MT>
struct RingA : std::integral_constant<int, 2> {};

template <bool ASYM>
__device__ __forceinline__ void zero_pairs(uint32_t zw, uint32_t zp, const NibbleConsts &nk, f16x2 (&zc)[8]) {
    if constexpr (ASYM) {
        zc[0] = zero_pair_from_word<0>(zw, nk);
        zc[1] = zero_pair_from_word<1>(zw, nk);
        zc[2] = zero_pair_from_word<2>(zw, nk);
        zc[3] = zero_pair_from_word<3>(zw, nk);
        zc[4] = zero_pair_from_word<4>(zw, nk);
        zc[5] = zero_pair_from_word<5>(zw, nk);
        zc[6] = zero_pair_from_word<6>(zw, nk);
        zc[7] = zero_pair_from_word<7>(zw, nk);
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

// Dequantise byte position B (nibbles 2B, 2B+1) of the 8 words of rows
// k0+8*kq .. +7 of one packed column-of-words into B operands 2B and 2B+1:
// the exact integers q - z in fp16.
template <int B>
__device__ __forceinline__ void dequant_byte(const uint32_t (&wd)[8], const f16x2 (&zc)[8],
                                             const NibbleConsts &nk, f16x8 (&bop)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t pr = gather_byte_pair<B>(wd[2 * j], wd[2 * j + 1]);
        const f16x2 v0 = as_f16x2(biased_pair<0>(pr, nk)) - zc[2 * B];
        const f16x2 v1 = as_f16x2(biased_pair<1>(pr, nk)) - zc[2 * B + 1];
        bop[2 * B][2 * j] = v0.x;
        bop[2 * B][2 * j + 1] = v0.y;
        bop[2 * B + 1][2 * j] = v1.x;
        bop[2 * B + 1][2 * j + 1] = v1.y;
    }
}


// RN: the decode step's row-norm folded in.  A is the raw row (row stride
// lda); each output is multiplied by its row's 1/sqrt(mean(a^2) + 1e-6) over
// the K values, a per-row scalar, so it is applied to the products: each wave
// sums the squares of the A operands it already holds, the K-waves meet in
// the LDS reduction, and with K-splits the per-row partial sums travel with
// the fp32 partials (after the output planes) to the last workgroup.
template <int MT, int NWN, int NWK, bool ASYM, bool RN>
__global__ __launch_bounds__(64 * NWN * NWK) void mfma_kernel(
    const uint16_t *__restrict__ a, int lda, const uint32_t *__restrict__ b,
    const uint16_t *__restrict__ scales, const uint32_t *__restrict__ qzeros, int M, int K, int N,
    int G, uint32_t zp, int tiles_n, int tiles_m, int m_group, int split_len, int splits,
    uint16_t *__restrict__ out, float *__restrict__ partials, uint32_t *__restrict__ counters) {
    static_assert(!RN || NWK > 1, "the row sums meet in the K-wave reduction");
    using C = Cfg<MT, NWN, NWK>;
    // Logical workgroup: XCD-contiguous runs (grid is a multiple of 8), so the
    // workgroups one XCD runs together are consecutive logical indices.
    const int logical = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (logical >= tiles_n * tiles_m * splits) return;  // whole workgroup
    // Within a split: bands of m_group row tiles; inside a band the row tiles
    // of one column tile are consecutive (they read the same weights), the
    // last band possibly shorter.
    const int split = logical / (tiles_n * tiles_m);
    const int in_split = logical - split * (tiles_n * tiles_m);
    const int band = in_split / (m_group * tiles_n);
    const int in_band = in_split - band * (m_group * tiles_n);
    const int band_rows = min(m_group, tiles_m - band * m_group);
    const int tile_n = in_band / band_rows;
    const int tile_m = band * m_group + (in_band - tile_n * band_rows);

    const int lane = threadIdx.x & 63;
    // Wave-uniform (the compiler cannot prove threadIdx.x >> 6 is): keeps the
    // per-step buffer offsets in SGPRs.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave % NWN;
    const int wk = wave / NWN;
    const int j16 = lane & 15;  // A row within the tile / B column within the tile
    const int kq = lane >> 4;   // 8-row slice of the 32-row step
    const int N8 = N >> 3;
    const int word = (tile_n * NWN + wn) * 16 + j16;
    const bool col_ok = word < N8;
    const int wordc = col_ok ? word : N8 - 1;  // clamped: loads stay in bounds
    const int m0 = tile_m * C::kTileRows;
    const int nsteps = K / 32;
    const int s_begin = split * split_len;
    const int s_end = min(s_begin + split_len, nsteps);
    const NibbleConsts nk = nibble_consts();

    const uint32_t row_bytes = (uint32_t)N8 * 4u;
    const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(b, (uint32_t)((uint64_t)K * N8 * 4));
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a, (uint32_t)(((uint64_t)(M - 1) * lda + K) * 2));
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(scales, (uint32_t)((uint64_t)(K / G) * N * 2));
    const __amdgpu_buffer_rsrc_t zrs = buffer_rsrc(qzeros, ASYM ? (uint32_t)((uint64_t)(K / G) * row_bytes) : 0u);
    const uint32_t b_voff = ((uint32_t)(8 * kq) * (uint32_t)N8 + (uint32_t)wordc) * 4u;
    const uint32_t s_voff = (uint32_t)wordc * 16u;
    const uint32_t z_voff = (uint32_t)wordc * 4u;
    // A row tile mt of this wave starts 16*mt rows below row tile 0: a
    // wave-uniform byte offset, so one lane offset serves every tile.  Rows
    // past M read row M-1 instead (valid memory; results never stored), which
    // only happens in a workgroup's last row tiles when 16*MT does not divide M.
    const uint32_t a_row_bytes = (uint32_t)lda * 2u;
    const bool a_full = m0 + C::kTileRows <= M;
    const uint32_t a_voff0 = ((uint32_t)(m0 + j16) * (uint32_t)lda + 8u * kq) * 2u;
    uint32_t a_voff_tail[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        a_voff_tail[mt] = ((uint32_t)min(m0 + 16 * mt + j16, M - 1) * (uint32_t)lda + 8u * kq) * 2u;

    // Accumulators start from distinct (opaque) zeros: with one shared zero
    // constant the register allocator gave MFMA results and their srcC
    // different registers and copied the accumulators every step.
    // acc: the current group's sums; tot: the scaled totals of the groups
    // before it.
    static_assert(MT <= 2, "group sums and totals of 64-row wave tiles do not fit the registers");
    f32x4 acc[MT][8], tot[MT][8];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                asm volatile("" : "+v"(z));
                acc[mt][t] = z;
            }
    };
    zero_acc();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+v"(z));
            tot[mt][t] = z;
        }

    // This K-wave's contiguous block of 32-row steps (groups change rarely).
    const int per_wave = (s_end - s_begin + NWK - 1) / NWK;
    const int w_begin = min(s_begin + wk * per_wave, s_end);
    const int n = min(w_begin + per_wave, s_end) - w_begin;
    auto stc = [&](int i) __attribute__((always_inline)) { return w_begin + min(i, n - 1); };  // clamped step index

    auto load_b = [&](int st, uint32_t (&w)[8]) {
        const uint32_t base = (uint32_t)st * 32u * row_bytes;
#pragma unroll
        for (int r = 0; r < 8; ++r) w[r] = buffer_load_x1(brs, b_voff, base + (uint32_t)r * row_bytes);
    };
    auto load_a = [&](int st, f16x8 (&av)[MT]) {
        if (a_full) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                av[mt] = __builtin_bit_cast(
                    f16x8, buffer_load_x4(ars, a_voff0, (uint32_t)st * 64u + (uint32_t)(16 * mt) * a_row_bytes));
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                av[mt] = __builtin_bit_cast(f16x8, buffer_load_x4(ars, a_voff_tail[mt], (uint32_t)st * 64u));
        }
    };
    auto load_sz = [&](int st, u32x4 &sv, uint32_t &zw) __attribute__((always_inline)) {
        const uint32_t g = (uint32_t)(st * 32 / G);
        sv = buffer_load_x4(srs, s_voff, g * (uint32_t)N * 2u);
        if constexpr (ASYM) zw = buffer_load_x1(zrs, z_voff, g * row_bytes);
    };
    // MFMAs for B operand pair (T, T+1) of one step, every row tile.
    auto mfma_pair = [&](const f16x8 (&av)[MT], const f16x8 (&bop)[8], auto tc) {
        constexpr int T = decltype(tc)::value;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            acc[mt][T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], bop[T], acc[mt][T], 0, 0, 0);
            acc[mt][T + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[mt], bop[T + 1], acc[mt][T + 1], 0, 0, 0);
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I6 = std::integral_constant<int, 6>;

    // Ring of packed-word / scale / zero slots (B data for steps s, s+1) and
    // two A-operand slots; one set of B operands `bop`.
    constexpr int kRing = RingW<MT, NWK>::value;  // B / scale / zero slots
    constexpr int kRingA = RingA<MT>::value;  // A slots
    constexpr int kUnroll = kRing * kRingA / Gcd<kRing, kRingA>::value;
    uint32_t w[kRing][8];
    u32x4 sv[kRing];
    uint32_t zw[kRing] = {};
    f16x8 av[kRingA][MT], bop[8];
    f16x2 zc[8];
    // End of a group: totals += group scale * group sums (tile t of the lane
    // is column 8 * word + t, scale element t of the word's scale vector).
    auto flush = [&](const u32x4 &scl) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float st = f16_bits_to_f32((scl[t >> 1] >> (16 * (t & 1))) & 0xffffu);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) tot[mt][t][v] = __builtin_fmaf(st, acc[mt][t][v], tot[mt][t][v]);
        }
        zero_acc();
    };

    // One K-step s held in ring slot U (A slot U & 1).  Four scheduling
    // regions, each issuing the MFMAs of one B operand pair of step s next to
    // the VALU work that rewrites the pair the previous region consumed:
    //   1: MFMA pair 0,1 | dequantise pair 6,7 of step s; zeros of s+1
    //   2: MFMA pair 2,3 | dequantise pair 0,1 of step s+1
    //   3: MFMA pair 4,5 | dequantise pair 2,3 of step s+1
    //   4: MFMA pair 6,7 | dequantise pair 4,5 of step s+1
    // then, when step s ends a group, the group flush.  A for s+1 is
    // requested at the top, B/scale/zero for s+2 after region 1 frees slot U.
    // Steps past the block clamp their loads (data unused).  Inside a region,
    // alternate one MFMA with a share of the region's VALU work (20
    // conversion ops per operand pair; the first region also builds the next
    // step's zero pairs), so that the matrix core and the VALU stay busy
    // together; left alone the scheduler clusters them.
    constexpr int kValuPair = (20 + 2 * MT - 1) / (2 * MT);
    constexpr int kValuFirst = (20 + (ASYM ? 16 : 0) + (RN ? 8 * MT : 0) + 2 * MT - 1) / (2 * MT);
    float sq[MT];  // RN: this lane's sum of squares of its A values (row m0 + 16 mt + j16)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sq[mt] = 0.f;
    auto step = [&](int s, auto uc) __attribute__((always_inline)) {
        constexpr int U = decltype(uc)::value;
        constexpr int AC = U % kRingA, AN = (U + kRingA - 1) % kRingA, WC = U % kRing, WN = (U + 1) % kRing;
        load_a(stc(s + kRingA - 1), av[AN]);
        const u32x4 scl = sv[WC];  // this step's group scales (the slot is refilled below)
        f16x2 zcn[8];
        mfma_pair(av[AC], bop, I0{});
        if constexpr (RN) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 8; ++e) sq[mt] = __builtin_fmaf((float)av[AC][mt][e], (float)av[AC][mt][e], sq[mt]);
        }
        dequant_byte<3>(w[WC], zc, nk, bop);
        zero_pairs<ASYM>(zw[WN], zp, nk, zcn);
        interleave<2 * MT, kValuFirst>();
        pin(bop[6], bop[7]);
#pragma unroll
        for (int x = 0; x < 8; x += 4) pin2(zcn[x], zcn[x + 1], zcn[x + 2], zcn[x + 3]);
        __builtin_amdgcn_sched_barrier(0);
        load_b(stc(s + kRing), w[WC]);
        load_sz(stc(s + kRing), sv[WC], zw[WC]);
        mfma_pair(av[AC], bop, I2{});
        dequant_byte<0>(w[WN], zcn, nk, bop);
        interleave<2 * MT, kValuPair>();
        pin(bop[0], bop[1]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_pair(av[AC], bop, I4{});
        dequant_byte<1>(w[WN], zcn, nk, bop);
        interleave<2 * MT, kValuPair>();
        pin(bop[2], bop[3]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_pair(av[AC], bop, I6{});
        dequant_byte<2>(w[WN], zcn, nk, bop);
        interleave<2 * MT, kValuPair>();
        pin(bop[4], bop[5]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 8; ++x) zc[x] = zcn[x];
        // the group of step s ends here (G is a multiple of 32), or the block does
        if (s + 1 == n || ((w_begin + s + 1) * 32) % G == 0) flush(scl);
    };

    if (n > 0) {
        // Issue order = consumption order: B(0), A(0 .. kRingA-2), B(1 ..).
        load_b(stc(0), w[0]);
        load_sz(stc(0), sv[0], zw[0]);
#pragma unroll
        for (int r = 0; r + 1 < kRingA; ++r) load_a(stc(r), av[r]);
#pragma unroll
        for (int r = 1; r < kRing; ++r) {
            load_b(stc(r), w[r]);
            load_sz(stc(r), sv[r], zw[r]);
        }
        zero_pairs<ASYM>(zw[0], zp, nk, zc);
        dequant_byte<0>(w[0], zc, nk, bop);
        dequant_byte<1>(w[0], zc, nk, bop);
        dequant_byte<2>(w[0], zc, nk, bop);
        int i = 0;
        for (; i + kUnroll <= n; i += kUnroll)
            static_for<0, kUnroll>([&](auto uc) __attribute__((always_inline)) { step(i + decltype(uc)::value, uc); });
        static_for<0, kUnroll - 1>([&](auto uc) __attribute__((always_inline)) {
            if (i + decltype(uc)::value < n) step(i + decltype(uc)::value, uc);
        });
    }

    // K-wave reduction and tile store.  A "row slot" (mt, v) is the row
    // m0 + 16*mt + 4*kq + v of every lane, 8 columns 8*word + 0..7 per lane:
    // tot[mt][0..7][v].  Every wave writes its slots to LDS at once (in rounds
    // of MTC row tiles, so the buffer stays within LDS); after one barrier,
    // each K-wave of an N-wave group sums its share of the slots over the
    // group's NWK waves in order wk = 0, 1, ... (deterministic) and stores
    // those rows itself: fp16 when the grid does not split K, else fp32 with
    // device-coherent stores into partials[split].
    typedef f16 f16x8_t __attribute__((ext_vector_type(8)));
    const int tile = tile_m * tiles_n + tile_n;
    // RN with K-splits: per (split, tile) the kTileRows row sums of squares,
    // after the splits' output planes.
    const uint32_t sq_base = (uint32_t)splits * (uint32_t)M * (uint32_t)N * 4u;
    const uint32_t sq_bytes = RN ? (uint32_t)splits * (uint32_t)(tiles_n * tiles_m) * C::kTileRows * 4u : 0u;
    const __amdgpu_buffer_rsrc_t prs = buffer_rsrc(partials, splits > 1 ? sq_base + sq_bytes : 0u);
    const uint32_t plane = (uint32_t)M * (uint32_t)N * 4u;
    auto store_slot = [&](int mt, int v, const f32x4 &lo, const f32x4 &hi) __attribute__((always_inline)) {
        const int row = m0 + 16 * mt + 4 * kq + v;
        if (row >= M || !col_ok) return;
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
    };
    auto slot_lo = [&](int mt, int v) __attribute__((always_inline)) {
        return f32x4{tot[mt][0][v], tot[mt][1][v], tot[mt][2][v], tot[mt][3][v]};
    };
    auto slot_hi = [&](int mt, int v) __attribute__((always_inline)) {
        return f32x4{tot[mt][4][v], tot[mt][5][v], tot[mt][6][v], tot[mt][7][v]};
    };
    if constexpr (NWK == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int v = 0; v < 4; ++v) store_slot(mt, v, slot_lo(mt, v), slot_hi(mt, v));
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        constexpr int MTC = C::kRedTiles;               // row tiles per round
        constexpr int SLOTS = MTC * 4;                  // row slots per round
        constexpr int PER = (SLOTS + NWK - 1) / NWK;    // slots per reducing wave
        static_assert(MT % MTC == 0, "whole rounds");
        __shared__ f32x4 red[NWN][NWK][SLOTS][2][64];
        __shared__ float sq_red[NWN][NWK][MT][16];  // RN: per K-wave row sums of squares
        if constexpr (RN) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                float v = sq[mt];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                if (kq == 0) sq_red[wn][wk][mt][j16] = v;
            }
        }
#pragma unroll
        for (int r0 = 0; r0 < MT; r0 += MTC) {
            if (r0 > 0) __syncthreads();  // previous round's reads are done
#pragma unroll
            for (int q = 0; q < SLOTS; ++q) {
                red[wn][wk][q][0][lane] = slot_lo(r0 + q / 4, q % 4);
                red[wn][wk][q][1][lane] = slot_hi(r0 + q / 4, q % 4);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int q = wk * PER + i;
                if (q < SLOTS) {
                    f32x4 lo = red[wn][0][q][0][lane], hi = red[wn][0][q][1][lane];
#pragma unroll
                    for (int src = 1; src < NWK; ++src) {
                        lo += red[wn][src][q][0][lane];
                        hi += red[wn][src][q][1][lane];
                    }
                    if constexpr (RN) {
                        const int mt = r0 + q / 4, rl = 4 * kq + q % 4;  // row m0 + 16 mt + rl
                        float rs = sq_red[wn][0][mt][rl];
#pragma unroll
                        for (int src = 1; src < NWK; ++src) rs += sq_red[wn][src][mt][rl];
                        if (splits == 1) {
                            const float inv = row_inv(rs, K);
                            lo *= inv;
                            hi *= inv;
                        } else if (wn == 0 && j16 == 0 && m0 + 16 * mt + rl < M) {
                            buffer_store_f32_sc1(rs, prs,
                                                 sq_base + (((uint32_t)split * (uint32_t)(tiles_n * tiles_m) +
                                                             (uint32_t)tile) * C::kTileRows + 16u * mt + rl) * 4u,
                                                 0u);
                        }
                    }
                    store_slot(r0 + q / 4, q % 4, lo, hi);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (splits == 1) return;

    wait_vm_zero();
    __syncthreads();
    __shared__ uint32_t last;
    if (threadIdx.x == 0) last = (arrive_agent(&counters[tile]) == (uint32_t)(splits - 1)) ? 1u : 0u;
    __syncthreads();
    if (!last) return;

    // Last arrival: every thread sums kUnits 16-byte units of the tile over
    // all splits, in split order; per chunk of units every split's load is
    // issued before the first add.
    constexpr int kRowUnits = C::kTileCols / 4;
    const int col0 = tile_n * C::kTileCols;
    typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int u0 = 0; u0 < C::kUnits; u0 += C::kChunk) {
        f32x4 v[C::kChunk][C::kMaxSplits];
        float rq[C::kChunk][C::kMaxSplits];  // RN: the splits' row sums of squares
#pragma unroll
        for (int u = 0; u < C::kChunk; ++u) {
            const int idx = threadIdx.x + (u0 + u) * C::kThreads;
            const int row = m0 + idx / kRowUnits;
            const int col = col0 + 4 * (idx % kRowUnits);
            const bool ok = row < M && col < N;
            const uint32_t off = ok ? ((uint32_t)row * (uint32_t)N + (uint32_t)col) * 4u : 0u;
            const uint32_t roff = ((uint32_t)tile * C::kTileRows + (uint32_t)(idx / kRowUnits)) * 4u;
#pragma unroll
            for (int sp = 0; sp < C::kMaxSplits; ++sp) {
                v[u][sp] = (ok && sp < splits) ? buffer_load_f32x4_sc1(prs, off, (uint32_t)sp * plane)
                                               : f32x4{0.f, 0.f, 0.f, 0.f};
                rq[u][sp] = 0.f;
                if constexpr (RN)
                    if (ok && sp < splits)
                        rq[u][sp] = buffer_load_f32_sc1(
                            prs, sq_base + (uint32_t)sp * (uint32_t)(tiles_n * tiles_m) * C::kTileRows * 4u + roff, 0u);
            }
        }
#pragma unroll
        for (int u = 0; u < C::kChunk; ++u) {
            const int idx = threadIdx.x + (u0 + u) * C::kThreads;
            const int row = m0 + idx / kRowUnits;
            const int col = col0 + 4 * (idx % kRowUnits);
            if (row >= M || col >= N) continue;
            f32x4 s = v[u][0];
#pragma unroll
            for (int sp = 1; sp < C::kMaxSplits; ++sp) s += v[u][sp];
            if constexpr (RN) {
                float rs = rq[u][0];
#pragma unroll
                for (int sp = 1; sp < C::kMaxSplits; ++sp) rs += rq[u][sp];  // zero past `splits`
                s *= row_inv(rs, K);
            }
            const u16x4 o = {f32_to_f16_bits(s.x), f32_to_f16_bits(s.y), f32_to_f16_bits(s.z),
                             f32_to_f16_bits(s.w)};
            *reinterpret_cast<u16x4 *>(out + (size_t)row * N + col) = o;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (threadIdx.x == 0) reset_counter_agent(&counters[tile]);
}

template <int MT, int NWN, int NWK, bool ASYM, bool RN>
hipError_t launch_k(const GemmArgs &g, const GemmPlan &p, const uint16_t *a, int64_t lda, hipStream_t stream) {
    hipLaunchKernelGGL((mfma_kernel<MT, NWN, NWK, ASYM, RN>), dim3((unsigned)p.grid), dim3(64 * NWN * NWK), 0, stream,
                       a, (int)lda, reinterpret_cast<const uint32_t *>(g.b), g.scales,
                       reinterpret_cast<const uint32_t *>(g.qzeros), (int)g.M, (int)g.K, (int)g.N, (int)g.G,
                       (uint32_t)g.zp, (int)p.tiles_n, (int)p.tiles_m, p.m_group, (int)p.split_len, p.splits, g.out,
                       g.partials, g.counters);
    return hipGetLastError();
}

template <int MT, int NWN, int NWK>
hipError_t launch_cfg(const GemmArgs &g, const GemmPlan &p, bool rn, const uint16_t *a, int64_t lda,
                      hipStream_t stream) {
    if (p.splits > Cfg<MT, NWN, NWK>::kMaxSplits) return hipErrorInvalidValue;
    if (p.splits > 1 && (!g.partials || !g.counters)) return hipErrorInvalidValue;
    if (rn)
        return g.qzeros ? launch_k<MT, NWN, NWK, true, true>(g, p, a, lda, stream)
                        : launch_k<MT, NWN, NWK, false, true>(g, p, a, lda, stream);
    return g.qzeros ? launch_k<MT, NWN, NWK, true, false>(g, p, a, lda, stream)
                    : launch_k<MT, NWN, NWK, false, false>(g, p, a, lda, stream);
}


}  // namespace

int mfma_max_splits(int mt, int waves, int kwaves) {
    if (mt == 1 && waves == 2 && kwaves == 4) return Cfg<1, 2, 4>::kMaxSplits;
    if (mt == 2 && waves == 2 && kwaves == 4) return Cfg<2, 2, 4>::kMaxSplits;
    if (mt == 2 && waves == 1 && kwaves == 8) return Cfg<2, 1, 8>::kMaxSplits;
    return 1;
}

hipError_t launch_mfma_rn(const GemmArgs &g, const GemmPlan &p, bool rn, const uint16_t *a, int64_t lda,
                          hipStream_t stream) {
    if (p.wm != 0 || p.wide || p.tall) return hipErrorInvalidValue;  // a plan of an LDS-sharing kernel
    // (MT, NWN, NWK) combinations the planner emits.
    if (p.mt == 1 && p.waves == 2 && p.kwaves == 4) return launch_cfg<1, 2, 4>(g, p, rn, a, lda, stream);
    if (p.mt == 2 && p.waves == 2 && p.kwaves == 4) return launch_cfg<2, 2, 4>(g, p, rn, a, lda, stream);
    if (p.mt == 2 && p.waves == 1 && p.kwaves == 8) return launch_cfg<2, 1, 8>(g, p, rn, a, lda, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_mfma(const GemmArgs &g, const GemmPlan &p, hipStream_t stream) {
    if (p.tall) return launch_mfma_tall(g, p, stream);
    if (p.wide) return launch_mfma_tile(g, p, stream);
    if (p.wm != 0) return launch_mfma_shared(g, p, stream);
    return launch_mfma_rn(g, p, false, g.a, g.K, stream);
}

size_t mfma_rn_extra_floats(const GemmPlan &p) {
    return p.splits > 1 ? (size_t)p.splits * (size_t)(p.tiles_n * p.tiles_m) * (size_t)(16 * p.mt) : 0;
}

}  // namespace w4a16
