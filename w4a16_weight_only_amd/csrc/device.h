// device.h -- gfx950 device helpers shared by the W4A16 kernels.
//
// Nibble -> fp16 conversion uses the binary16 layout directly: OR-ing a 4-bit
// value into the fraction field of a power of two whose fraction LSB is worth
// the nibble's LSB gives (2^e + q) exactly, and one packed subtraction of
// (2^e + z) leaves the exact integer q - z.  Low nibbles of a byte sit in
// fraction bits 0..3 under 1024 (0x6400, LSB = 1); high nibbles sit in bits
// 4..7 under 64 (0x5400, LSB = 1/16, so 16*q/16 = q).  Two rows are converted
// per 32-bit register: v_perm_b32 gathers byte b of row k and of row k+1 into
// bytes 0 and 2, one AND-OR then forms both fp16 lanes.
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

// Biased fp16 pair for nibble 2B (H = 0) or 2B+1 (H = 1) of the gathered pair
// `p`: lanes hold (bias + q_lo_row, bias + q_hi_row), bias 1024 or 64.
template <int H>
__device__ __forceinline__ uint32_t biased_pair(uint32_t p) {
    return H ? ((p & kMaskHi) | kMagicHi) : ((p & kMaskLo) | kMagicLo);
}

// Bias-plus-zero constant for nibble position T (0..7) of a packed zero word:
// (1024 + z) for even T, (64 + z) for odd T, in both fp16 lanes.
template <int T>
__device__ __forceinline__ f16x2 zero_pair_from_word(uint32_t zword) {
    constexpr int B = T / 2;
    uint32_t p = gather_byte_pair<B>(zword, zword);
    return as_f16x2(biased_pair<T & 1>(p));
}

// Same constant for a symmetric zero point z in [0, 15].
template <int T>
__device__ __forceinline__ f16x2 zero_pair_const(uint32_t z) {
    uint32_t v = (T & 1) ? (kMagicHi | (z << 4) | (z << 20)) : (kMagicLo | z | (z << 16));
    return as_f16x2(v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(f16, (uint16_t)bits16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (f16)x);  // round-to-nearest-even
}

// Device-scope release/acquire around the split-K arrival counter: partial
// sums written by workgroups on other XCDs must be visible through their L2s.
__device__ __forceinline__ void fence_release_agent() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire_agent() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}
__device__ __forceinline__ uint32_t arrive_agent(uint32_t *counter) {
    return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_counter_agent(uint32_t *counter) {
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace w4a16
