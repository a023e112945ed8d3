// kernels.h -- host-side plan and launch interface between the C ABI layer
// (api.cpp) and the gfx950 kernels.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a16 {

enum GemmPath { kPathGemv = 1, kPathMfma = 2 };
// Rows per chunk of the matrix-core GEMV (a multiple of 16 dividing every G,
// which is a multiple of 32).
constexpr int kMmaChunkRows = 32;
// Most K-splits of a GEMV: its fixed-point split-K slots count arrivals in
// four bits (device.h).
constexpr int kGemvMaxSplits = 16;

// Everything a GEMM launch needs besides the tensors; computed on the host
// from (M, K, N, G) alone so that it can be inspected without a GPU.
struct GemmPlan {
    int path = 0;
    // GEMV: `words` packed words (8 columns each) per lane (matrix-core form:
    // 2, or 4 for 512-column tiles), `waves` waves per workgroup.  MFMA: `mt`
    // 16-row tiles per wave, `waves` along N.
    int words = 4;
    int waves = 4;
    int mt = 1;
    int kwaves = 1;           // MFMA: waves dividing a workgroup's K range (LDS-reduced)
    bool wide = false;        // MFMA: the 128 x 256 kernel sharing activations and weights
                              // through LDS (gemm_tile.hip)
    bool tall = false;        // MFMA: the 128 x 128 kernel whose waves each own a 32-column strip
                              // of all 128 rows, activations staged in LDS (gemm_tall.hip)
    int wm = 0;               // MFMA: row waves sharing each step's dequantised weights through
                              // LDS (2 or 4; mt = 2, waves = 1, kwaves = 8 / wm); 0: the
                              // register-direct kernel
    bool mma = false;         // GEMV with the k-reduction on the matrix cores (split_len in
                              // kMmaChunkRows-row chunks); false: the dot2 GEMV
    bool fold = false;        // GEMV, symmetric zero point: remove bias and zero per chunk, not per pair
    bool fold_asym = false;   // the same with packed zeros
    bool exact = false;       // matrix-core GEMV, symmetric zero point: exact (q - z) weights
                              // instead of biased weights with the zero term folded per chunk
    int64_t tiles_n = 0;      // workgroup tiles along N
    int64_t tiles_m = 1;      // workgroup tiles along M (MFMA)
    int m_group = 1;          // MFMA: consecutive workgroups walk this many row tiles of one
                              // column tile before the next column tile (shared weights in L2)
    int splits = 1;           // K-splits across workgroups
    int64_t split_len = 0;    // K-units per split (GEMV: 16-row chunks, 32 with mma; MFMA:
                              // 32-row steps)
    int64_t grid = 0;         // workgroups launched
    size_t partial_floats = 0;  // fp32 split-K partials needed (0 when splits == 1)
    size_t counters = 0;        // zero-initialised words needed: MFMA arrival counters,
                                // GEMV 64-bit fixed-point slots (two words per output)
};

struct GemmArgs {
    const uint16_t *a;
    const int32_t *b;
    const uint16_t *scales;
    const int32_t *qzeros;
    int64_t M, K, N, G;
    int32_t zp;
    uint16_t *out;
    float *partials;     // plan.partial_floats floats (or null when unused)
    uint32_t *counters;  // plan.counters zero-initialised words (or null)
};

// allow_mma = false keeps a GEMV plan on the dot2 kernel; allow_wide = false
// keeps the matrix-core GEMV on 256-column tiles (its SwiGLU variant has no
// 512-column form); allow_shared = false keeps an MFMA plan on the
// register-direct kernel (the one with the folded row-norm).  MFMA K-splits
// stop where their fp32 partials would pass partial_cap_bytes (>= 0).
GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int64_t G, bool allow_mma = true, bool allow_wide = true,
                   bool allow_shared = true, int64_t partial_cap_bytes = -1);

hipError_t launch_gemv(const GemmArgs &args, const GemmPlan &plan, hipStream_t stream);
// GEMV with the decode step's glue folded in: act 1: out = (src . W) * inv_row,
// act 2: out = (fp16(silu(g) * u) . W) * inv_row with g = src[:, :K],
// u = src[:, K:2K]; inv_row = 1/sqrt(mean(t^2) + 1e-6) over the row's
// transformed values t (summed in the glue kernels' order).  The row scale is
// applied to the products, so the normalised activations are not rounded to
// fp16 on their own (one rounding fewer than the separate glue kernels).
// src rows ld elements apart (ld and K multiples of 8, K <= kGlueMaxWidth).
// Needs plan.waves == 8.
hipError_t launch_gemv_act(const GemmArgs &args, const GemmPlan &plan, int act, const uint16_t *src,
                           int64_t ld, hipStream_t stream);
// Runs the LDS-shared kernel (gemm_shared.hip) when plan.wm is set.
hipError_t launch_mfma(const GemmArgs &args, const GemmPlan &plan, hipStream_t stream);
// MFMA GEMM whose row waves share each step's dequantised weights through LDS
// (plan.wm = 2 or 4 row waves of 32 rows, plan.kwaves = 8 / wm K-waves or 1,
// 128-column tiles).  G must be 32, 64, 128 or 256, split_len whole groups,
// at most kSharedGroupSlots / kwaves groups per K-wave (each K-wave's group
// scales and zeros are staged in LDS) and kSharedMaxSplits K-splits.
constexpr int kSharedMaxSplits = 8;
constexpr int kSharedGroupSlots = 128;
inline bool shared_supports(int64_t G) { return G == 32 || G == 64 || G == 128 || G == 256; }
hipError_t launch_mfma_shared(const GemmArgs &args, const GemmPlan &plan, hipStream_t stream);
// MFMA GEMM on 128-row x 256-column workgroup tiles whose activations and
// dequantised weights are both shared through LDS (gemm_tile.hip; plan.wide).
// G must be 32, 64, 128 or 256, split_len whole groups, at most
// kTileGroupSlots groups per split and kSharedMaxSplits K-splits.
constexpr int kTileGroupSlots = 64;
hipError_t launch_mfma_tile(const GemmArgs &args, const GemmPlan &plan, hipStream_t stream);
// MFMA GEMM on 128 x 128 workgroup tiles, each wave dequantising one
// 32-column strip for all 128 rows, the activations staged in LDS per
// workgroup (gemm_tall.hip; plan.tall).  N and G multiples of 32, at most
// kTallMaxSplits K-splits.
constexpr int kTallMaxSplits = 8;
hipError_t launch_mfma_tall(const GemmArgs &args, const GemmPlan &plan, hipStream_t stream);
// MFMA GEMM on A = `a` with row stride lda (>= K); with rn, the decode step's
// row-norm folded in: out = (a . W) * inv_row, inv_row = 1/sqrt(mean(a_row^2)
// + 1e-6) over the row's K values, applied to the products (the partials
// buffer then needs mfma_rn_extra_floats(plan) more floats).
hipError_t launch_mfma_rn(const GemmArgs &args, const GemmPlan &plan, bool rn, const uint16_t *a, int64_t lda,
                          hipStream_t stream);
size_t mfma_rn_extra_floats(const GemmPlan &plan);
// Largest K-split count the MFMA kernel's in-kernel reduction takes for a
// (mt, waves, kwaves) configuration.
int mfma_max_splits(int mt, int waves, int kwaves);
hipError_t launch_repack(const int32_t *src, int32_t *dst, int64_t K, int64_t N, hipStream_t stream);

// Split-K scratch of the allocation-free GEMM entry point (noalloc.hip): a
// fixed device array per GPU, counters and slots first, fp32 partials after.
constexpr size_t kNoAllocCounterBytes = (size_t)4 << 20;
constexpr size_t kNoAllocPartialBytes = (size_t)12 << 20;
// Device addresses of this GPU's array (taken once per device, the counter
// region cleared by a kernel on `stream` the first time).
hipError_t noalloc_scratch(hipStream_t stream, uint32_t **counters, float **partials);
// fp16 [N, Gn] -> [Gn, N] (checkpoint group scales to the kernel layout).
hipError_t launch_repack_scales(const uint16_t *src, uint16_t *dst, int64_t Gn, int64_t N, hipStream_t stream);

// Decode-step glue (fp16 in/out, fp32 math).  Widths (and row strides) must
// be multiples of 8 and at most kGlueMaxWidth; the launchers return
// hipErrorInvalidValue otherwise.
constexpr int64_t kGlueMaxWidth = 32768;
// y[m][0..width) = rn(x[m][0..width)) with x row stride ldx.
hipError_t launch_rownorm(const uint16_t *x, int64_t M, int64_t ldx, int64_t width, uint16_t *y,
                          hipStream_t stream);
// y[m][i] = rn_row(silu(gu[m][i]) * gu[m][I + i]), gu rows ld >= 2I apart.
hipError_t launch_swiglu_rownorm(const uint16_t *gu, int64_t M, int64_t ld, int64_t I, uint16_t *y,
                                 hipStream_t stream);

}  // namespace w4a16
