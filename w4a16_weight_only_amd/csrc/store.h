// store.h -- wide device-coherent stores of fp32 split partials.
//
// A buffer store of more than 64 bits reads its data registers after it
// issues.  With the byte offset in an SGPR the compiler places no wait
// between such a store and an instruction that overwrites its data registers,
// and on gfx950 an fp32 partial stored that way was observed to reach memory
// holding the value written next into the same register (an intermittent
// split-K error: one split's column c summed with its column c + 4).  The
// store below keeps its data registers live through a few wait states of its
// own, so nothing can reuse them before the store has read them.
#pragma once

#include "device.h"

namespace w4a16 {

__device__ __forceinline__ void store_partial_x4(f32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    buffer_store_f32x4_sc1(v, r, voff, soff);
    asm volatile("s_nop 4" ::"v"(v));
}

}  // namespace w4a16
