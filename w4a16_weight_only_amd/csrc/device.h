// device.h -- gfx950 device helpers shared by the W4A16 kernels.
//
// Nibble -> fp16 conversion uses the binary16 layout directly: OR-ing a 4-bit
// value into the fraction field of a power of two whose fraction LSB is worth
// the nibble's LSB gives (2^e + q) exactly, and one packed subtraction of
// (2^e + z) leaves the exact integer q - z.  Low nibbles of a byte sit in
// fraction bits 0..3 under 1024 (0x6400, LSB = 1); high nibbles sit in bits
// 4..7 under 64 (0x5400, LSB = 1/16, so 16*q/16 = q).  The dot2 GEMV converts
// two rows per 32-bit register: v_perm_b32 gathers byte b of row k and of row
// k+1 into bytes 0 and 2, one AND-OR then forms both fp16 lanes.  The
// matrix-core GEMV applies the AND-OR to a packed word as loaded (columns c
// and c + 4 of one row) and keeps the bias, removing it per chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr uint32_t kMagicLo = 0x64006400u;  // fp16 1024 in both halves
constexpr uint32_t kMagicHi = 0x54005400u;  // fp16 64 in both halves
constexpr uint32_t kMaskLo = 0x000F000Fu;
constexpr uint32_t kMaskHi = 0x00F000F0u;

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// Byte B of `lo` into byte 0 and byte B of `hi` into byte 2 (bytes 1, 3 zero).
template <int B>
__device__ __forceinline__ uint32_t gather_byte_pair(uint32_t lo, uint32_t hi) {
    // v_perm_b32: selector values 0..3 pick bytes of the second operand,
    // 4..7 bytes of the first, 0x0c yields zero.
    constexpr uint32_t sel = 0x0c000c00u | ((4u + B) << 16) | (uint32_t)B;
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Masks and biases for the nibble -> fp16 conversion, held in VGPRs whose
// values the compiler cannot see (an empty asm with a "+v" operand emits no
// instruction).  gfx9 VOP3 encodings take no literal constants, so with
// literals the compiler splits AND-OR into v_and + v_or; with register
// operands it selects one v_and_or_b32 per pair.
struct NibbleConsts {
    uint32_t mask_lo, mask_hi, bias_lo, bias_hi;
};

__device__ __forceinline__ NibbleConsts nibble_consts() {
    uint32_t a = kMaskLo, b = kMaskHi, c = kMagicLo, d = kMagicHi;
    asm volatile("" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
    return NibbleConsts{a, b, c, d};
}

// Biased fp16 pair for nibble 2B (H = 0) or 2B+1 (H = 1) of the gathered pair
// `p`: lanes hold (bias + q_lo_row, bias + q_hi_row), bias 1024 or 64.
template <int H>
__device__ __forceinline__ uint32_t biased_pair(uint32_t p, const NibbleConsts &k) {
    return H ? ((p & k.mask_hi) | k.bias_hi) : ((p & k.mask_lo) | k.bias_lo);
}

// Bias-plus-zero constant for nibble position T (0..7) of a packed zero word:
// (1024 + z) for even T, (64 + z) for odd T, in both fp16 lanes.
template <int T>
__device__ __forceinline__ f16x2 zero_pair_from_word(uint32_t zword, const NibbleConsts &k) {
    constexpr int B = T / 2;
    uint32_t p = gather_byte_pair<B>(zword, zword);
    return as_f16x2(biased_pair<T & 1>(p, k));
}

// Same constant for a symmetric zero point z in [0, 15].
template <int T>
__device__ __forceinline__ f16x2 zero_pair_const(uint32_t z) {
    uint32_t v = (T & 1) ? (kMagicHi | (z << 4) | (z << 20)) : (kMagicLo | z | (z << 16));
    return as_f16x2(v);
}

// Raw buffer resource over `bytes` bytes (< 2^32) at `base`: loads take a
// per-lane byte offset plus a wave-uniform byte offset held in an SGPR, so a
// stream of rows at a uniform stride costs no vector address arithmetic.
// Out-of-range reads return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load_x4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x2 buffer_load_x2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buffer_load_x1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
// Non-temporal (nt) forms for data read exactly once, the weight stream: on
// MI355X they shorten the M = 1 GEMV by about 7% against the default policy.
constexpr int kCpolNt = 2;
__device__ __forceinline__ u32x4 buffer_load_x4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCpolNt));
}
__device__ __forceinline__ u32x2 buffer_load_x2_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kCpolNt));
}
__device__ __forceinline__ uint32_t buffer_load_x1_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kCpolNt));
}

// Device-coherent (sc1) 16-byte buffer accesses, for data handed between
// workgroups that may sit on different XCDs: the same cache policy the
// compiler gives agent-scope atomic loads and stores on gfx950.
constexpr int kCpolSc1 = 16;
__device__ __forceinline__ f32x4 buffer_load_f32x4_sc1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCpolSc1));
}
__device__ __forceinline__ void buffer_store_f32x4_sc1(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)voff, (int)soff, kCpolSc1);
}
__device__ __forceinline__ float buffer_load_f32_sc1(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kCpolSc1));
}
__device__ __forceinline__ void buffer_store_f32_sc1(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, (int)soff, kCpolSc1);
}

// dot(x, y) + 0 into a fresh register (VOP3P form: no zeroing move first).
__device__ __forceinline__ float dot2_first(f16x2 x, f16x2 y) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(x), "v"(y));
    return r;
}

// Exchange for one transpose-reduce step across lane halves: returns
// lo + hi where, in lanes whose `mask` bit is clear, lo/hi are this lane's
// lower-half value and the partner's lower-half value, and in the other lanes
// the two upper-half values.  mask 32 and 16 use the gfx950 lane-swap
// instructions; mask 8 uses a DPP row rotation by 8 (lane ^ 8 in a row).
template <int MASK>
__device__ __forceinline__ float swap_add(float lo, float hi, int lane) {
    if constexpr (MASK == 32 || MASK == 16) {
        // Written as asm with both registers as in/out operands: with the
        // two-result builtin this compiler added the first result to itself.
        // The s_nops keep the swap clear of neighbouring VALU writes/reads,
        // which the compiler cannot see through the asm.
        float a = lo, b = hi;
        if constexpr (MASK == 32)
            asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
        else
            asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
        return a + b;
    } else {
        static_assert(MASK == 8, "lane-xor 8 within a 16-lane row");
        const float pl = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                             0u, __builtin_bit_cast(uint32_t, lo), 0x128, 0xf, 0xf, false));
        const float ph = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                             0u, __builtin_bit_cast(uint32_t, hi), 0x128, 0xf, 0xf, false));
        return (lane & 8) ? hi + ph : lo + pl;
    }
}

// Sum over the 64 lanes of a wave, every lane getting the total, with the
// pairing of a lane-xor butterfly (32, 16, 8, 4, 2, 1): bit for bit what
// `for (off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off)` gives (each
// step adds the same two values in every lane of a pair, and fp32 addition is
// commutative), on lane swaps and DPP instead of six LDS permutes.  After the
// xor-8 step lanes 8 apart hold equal values, so a rotation by 4 inside the
// 16-lane row reads a lane holding the xor-4 partner's value.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, v), CTRL, 0xf,
                                                                 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v, int lane) {
    v = swap_add<32>(v, v, lane);
    v = swap_add<16>(v, v, lane);
    v = swap_add<8>(v, v, lane);
    v += dpp_f32<0x124>(v);  // row_ror:4
    v += dpp_f32<0x4e>(v);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    v += dpp_f32<0xb1>(v);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    return v;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(f16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (f16)x);  // round-to-nearest-even
}

// Decode-step glue arithmetic, shared by the standalone glue kernels and the
// GEMVs that apply the glue as they load activations, so that both round the
// same way bit for bit.  A value passed through an empty asm is opaque to the
// optimiser: it is rounded to fp32 on its own and cannot be fused with what
// follows (left alone, the compiler turned fp16(t * inv) into one
// mixed-precision multiply that rounds once in one kernel and into a multiply
// plus a conversion, two roundings, in another).
__device__ __forceinline__ float opaque(float x) {
    asm volatile("" : "+v"(x));
    return x;
}
// fp16(t * inv): the product rounded to fp32, then to fp16 (RNE).
__device__ __forceinline__ uint32_t scaled_f16(float t, float inv) { return f32_to_f16_bits(opaque(t * inv)); }
// 1 / sqrt(sum_sq / width + 1e-6).
__device__ __forceinline__ float row_inv(float sum_sq, int width) {
    return 1.0f / sqrtf(opaque(sum_sq / (float)width) + 1e-6f);
}
// silu(g) * u with silu(g) = g / (1 + exp(-g)), on the hardware base-2
// exponential (exp(-g) = 2^(-g log2 e)) and reciprocal: a few instructions per
// element where the correctly rounded expf and division take about thirty; the
// relative error (about 1e-7 near |g| = 10, growing with |g|) stays far below
// the fp16 rounding that follows.  Limits: g -> -inf gives -0, g -> +inf gives
// g, NaN stays NaN.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(opaque(-g * 1.44269504088896341f));
    const float r = __builtin_amdgcn_rcpf(opaque(1.0f + e));
    return opaque(g * r) * u;
}

// Split-K hand-off between workgroups that may sit on different XCDs (each
// with its own L2).  Partial sums are written with device-scope stores (sc1:
// coherent at device scope by themselves) and read back with device-scope
// loads (sc1), so no whole-L2 write-back or invalidate is needed: a writer
// waits for its stores to complete (vmcnt(0)) before it bumps the tile's
// arrival counter, and the workgroup that brings the counter to `splits`
// reads every split's partials.  An agent-scope release/acquire fence pair
// would instead write back and invalidate the XCD's whole L2 once per wave.
__device__ __forceinline__ void store_partial(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_partial(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Split-K reduction in exact fixed point, so the result does not depend on the
// order in which splits arrive.  Each output owns one zero-initialised 64-bit
// slot, and each split adds its fp32 partial p with one atomic:
//   bits 60..63  arrivals
//   bits 55..59  "positive beyond range" partials: +inf, or finite p >= 2^17
//   bits 50..54  "negative beyond range" partials: -inf, or finite p <= -2^17
//                (a NaN partial counts in both fields)
//   bits  0..49  splits * 2^45 + the sum over the other partials of
//                round(p * 2^28)
// The arrival that brings the count to `splits` holds the total (the value it
// got back plus its own addition), writes the output and zeroes the slot for
// the next call.  At most kGemvMaxSplits (16) splits, so no field carries into
// the next.  Every partial with |p| < 2^17 (twice the fp16 range) enters the
// sum exactly up to its 2^-28 rounding; beyond that the result is exact or
// loud: an infinite partial gives that infinity (NaN with both signs, as fp32
// addition does), and a finite partial past 2^17 gives the infinity of its
// sign when the rest cannot pull the sum back inside fp16 range (the other
// partials sum to less than 2^16 against it), NaN otherwise.
constexpr int kFixFracBits = 28;
constexpr int kSlotNegShift = 50;
constexpr int kSlotPosShift = 55;
constexpr int kSlotCountShift = 60;
constexpr int64_t kFixBias = 1ll << 45;
constexpr float kFixMax = 131072.0f;  // 2^17

__device__ __forceinline__ uint64_t slot_contribution(float p) {
    // every split adds the bias once, so the sum field holds splits * bias
    // plus the fixed-point partials of the splits in range
    uint64_t add = (1ull << kSlotCountShift) + (uint64_t)kFixBias;
    if (__builtin_fabsf(p) < kFixMax) {
        add += (uint64_t)(int64_t)rintf(p * (float)(1 << kFixFracBits));
    } else {
        // +-inf, a finite partial beyond 2^17, or NaN (both fields)
        if (!(p < 0.f)) add += 1ull << kSlotPosShift;
        if (!(p > 0.f)) add += 1ull << kSlotNegShift;
    }
    return add;
}
__device__ __forceinline__ uint64_t slot_add(uint64_t *slot, uint64_t v) {
    return __hip_atomic_fetch_add(slot, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool slot_last(uint64_t old, int splits) {
    return (old >> kSlotCountShift) == (uint64_t)(splits - 1);
}
// fp16 output for a slot's final value.
__device__ __forceinline__ uint16_t slot_result_f16(uint64_t total, int splits) {
    const uint32_t pos = (uint32_t)(total >> kSlotPosShift) & 31u;
    const uint32_t neg = (uint32_t)(total >> kSlotNegShift) & 31u;
    const int64_t s = (int64_t)(total & ((1ull << kSlotNegShift) - 1)) - (int64_t)splits * kFixBias;
    constexpr int64_t kRange = 1ll << (16 + kFixFracBits);  // 2^16 in fixed point
    if (pos && neg) return 0x7e00u;
    if (pos) return s > -kRange ? 0x7c00u : 0x7e00u;
    if (neg) return s < kRange ? 0xfc00u : 0x7e00u;
    return f32_to_f16_bits((float)((double)s * (1.0 / (double)(1ll << kFixFracBits))));
}
__device__ __forceinline__ void slot_reset(uint64_t *slot) {
    __hip_atomic_store(slot, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vm_zero() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ uint32_t arrive_agent(uint32_t *counter) {
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter_agent(uint32_t *counter) {
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace w4a16
