/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 weight-only-quantized linear
 * layer library (libw4a16.so).
 *
 * The operation (vLLM PR #37352 write-up, "Code analysis" item 1: the reference
 * dequantize-then-matmul formula and the kernel call taking group_size, qzeros
 * and zp_bias):
 *
 *     out[m][n] = sum_k a[m][k] * (q[k][n] - z[k/G][n]) * s[k/G][n]
 *
 * with q the unsigned 4-bit weight, z the zero point of the (K-group, column)
 * and s its fp16 scale; out is rounded to fp16.  Accumulation is fp32.
 *
 * Conventions for every entry point:
 *   - fp16 values travel as their 16-bit patterns (uint16_t).
 *   - Packed int4: 8 nibbles per 32-bit word, nibble j (bits 4j..4j+3) is the
 *     j-th lowest index of the 8 elements the word packs; nibbles are unsigned
 *     0..15 and words are used as raw bit patterns (negative int32 is normal).
 *   - All tensors are dense row-major; pointers marked "device" must be device
 *     memory of the current HIP device; the caller owns every buffer it passes.
 *   - Work is enqueued on `stream` (NULL = the default stream).  A return of
 *     W4A16_OK means "validated and enqueued"; faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Every argument is validated on the host before any HIP call; a rejected
 *     call touches nothing and enqueues nothing.
 *   - No function throws or aborts; each returns a w4a16_status code and, on
 *     failure, records a message readable with w4a16_last_error() on the same
 *     host thread.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, bad divisibility, overlap */
    W4A16_ERR_UNSUPPORTED = 2, /* legal shape the kernels do not cover (see each call) */
    W4A16_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed */
    W4A16_ERR_WORKSPACE = 4    /* library-owned scratch could not be allocated */
} w4a16_status;

/* Static, human-readable name of a status code (never NULL). */
const char *w4a16_status_string(int status);

/* Message describing the last failing call on this host thread ("" if none).
 * The pointer stays valid until the next library call on the same thread. */
const char *w4a16_last_error(void);

/*
 * Repack checkpoint-layout weights into the kernel layout.
 * Defined by: vLLM PR #37352 write-up, "Code analysis" item 2 -- the loaded
 * compressed-tensors weight [N, K/8] becomes [K, N/8] before the kernel runs.
 *
 *   src_nk8  device, int32 [N, K/8]: word (n, k/8) holds element (k, n) at
 *            nibble k%8.
 *   dst_kn8  device, int32 [K, N/8]: word (k, n/8) receives element (k, n) at
 *            nibble n%8.  Must not overlap src (no in-place repack).
 *   K, N     > 0, both multiples of 8.
 * Bit-exact.  Errors: INVALID_ARG for NULL pointers, K or N <= 0 or not a
 * multiple of 8, or overlapping buffers; HIP if the launch fails.
 */
int w4a16_repack(const int32_t *src_nk8, int32_t *dst_kn8, int64_t K, int64_t N,
                 hipStream_t stream);

/*
 * Repack checkpoint-layout group scales into the kernel layout.
 * Defined by: vLLM PR #37352 write-up, "Code analysis" item 2 -- after loading,
 * the scale tensor has shape (K/G, N).  The page does not print the
 * checkpoint's own scale layout; this call reads it as per output column,
 * [N, K/G] (the weights' own orientation), and transposes.  Packed zero
 * points in the checkpoint, read the same way as packed along the group axis
 * ([N, (K/G)/8]), become [K/G, N/8] through w4a16_repack(src, dst, K/G, N).
 *
 *   src_ng   device, fp16 bits [N, Gn]: scale of (column n, group g).
 *   dst_gn   device, fp16 bits [Gn, N]: receives it at (g, n).  Must not
 *            overlap src.
 *   Gn       number of groups K/G, > 0.  N > 0, a multiple of 8.
 * Bit-exact.  Errors: INVALID_ARG for NULL pointers, Gn <= 0, N <= 0 or not a
 * multiple of 8, or overlapping buffers; UNSUPPORTED beyond 32-bit indexing;
 * HIP if the launch fails.
 */
int w4a16_repack_scales(const uint16_t *src_ng, uint16_t *dst_gn, int64_t Gn, int64_t N,
                        hipStream_t stream);

/*
 * out = a . ((q - z) * s).
 * Defined by: vLLM PR #37352 write-up, "Code analysis" item 1 (formula and call
 * signature) and "Why it is good" item 3 (contiguous inputs, N % 8 == 0).
 *
 *   a        device, fp16 [M, K] activations.
 *   b_packed device, int32 [K, N/8] weights (kernel layout, see w4a16_repack).
 *   scales   device, fp16 [K/G, N]: scale of (group k/G, column n).
 *   qzeros   device, int32 [K/G, N/8] packed zero points (nibble n%8 of word
 *            (g, n/8)), or NULL for the symmetric case z = zp_bias.  When given,
 *            zp_bias is ignored.
 *   M        >= 0 rows (M == 0 is a no-op returning W4A16_OK; a and out may
 *            then be NULL).
 *   K        > 0, a multiple of G.
 *   N        > 0, a multiple of 8.
 *   G        group size along K; must be a multiple of 32 (UNSUPPORTED else).
 *   zp_bias  symmetric zero point in [0, 15] (8 for signed int4), used only when
 *            qzeros is NULL.
 *   out      device, fp16 [M, N], caller-allocated; must not overlap any input.
 *
 * Paths (w4a16_gemm_plan reports which): M <= 8 (with N % 32 == 0) runs a
 * split-K GEMV whose k-reduction runs on the matrix cores
 * (v_mfma_f32_16x16x32_f16 on the exact integers q - z in fp16; with the
 * tuning key gemv_mma_exact=0 and a symmetric zero point, on biased weights
 * 1024 + q or 64 + q with the zero term removed per 32-row chunk by the same
 * MFMA chain); the tuning key gemv_mma=0 selects the same GEMV with
 * v_dot2_f32_f16 on the vector ALUs.  M >= 9 runs an MFMA GEMM on exact
 * (q - z) fp16 operands that applies each group's scale to the fp32 sums of
 * that group: below M = 161 each wave dequantises its own operands in
 * registers for 32 rows; from M = 161 (tuning key mfma_tall_m) a workgroup
 * owns 128 rows x 128 columns, each wave converts the weights of one
 * 32-column strip once for all 128 rows, and the activations are staged in
 * LDS once per workgroup.  (A third form, tuning key mfma_shared_m, shares
 * each K-step's dequantised weights between row waves through LDS.)
 * Accumulation is fp32 throughout.  K-splits across workgroups meet in
 * fixed point (GEMV) or in split order (MFMA GEMM), so the result is
 * deterministic for a given shape and plan.
 *
 * Scratch: split-K partials and counters live in buffers the library
 * allocates per (device, stream) on the first call that needs them; a call
 * that needs more allocates a larger set and keeps the old one (graphs that
 * captured it stay valid) until w4a16_release().  An allocation cannot be
 * captured: a call that would need one while its stream is capturing returns
 * W4A16_ERR_WORKSPACE, so run a shape once on the stream before capturing
 * it.  Calls on one stream from several host threads at once are not
 * supported.
 *
 * Errors: INVALID_ARG for NULL b_packed/scales (or a/out with M > 0), M < 0, K/N/G <= 0,
 * N % 8 != 0, K % G != 0, zp_bias outside [0, 15] without qzeros, or `out`
 * overlapping an input; UNSUPPORTED for G % 32 != 0, a pointer that is not
 * 16-byte aligned, or sizes past the kernels' 32-bit ranges (M > 2^20,
 * K or N > 2^26, M*K or M*N >= 2^31, K*N/8 >= 2^30); WORKSPACE if scratch
 * allocation fails; HIP on launch failure.
 */
int w4a16_gemm(const uint16_t *a, const int32_t *b_packed, const uint16_t *scales,
               const int32_t *qzeros, int64_t M, int64_t K, int64_t N, int64_t G,
               int32_t zp_bias, uint16_t *out, hipStream_t stream);

/*
 * w4a16_gemm without any allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture that has not run the shape before,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * plans, kernels and results as w4a16_gemm (bit for bit); the split-K scratch
 * is a fixed array of 4 MiB (counters and fixed-point slots) + 12 MiB (fp32
 * partials) in the library's device data, one per GPU, held until the
 * process ends.  Its device address is taken on the first call on each
 * device, which also clears the counters with a kernel on `stream` (no
 * allocation, no memset); every call leaves them zero again.  All calls on
 * one GPU share the array: calls that overlap in time on one GPU (several
 * streams or threads) race and must not be issued.
 * Errors: as w4a16_gemm; UNSUPPORTED when the shape's plan needs more scratch
 * than the array holds (M * N * 8 bytes of slots for the GEMV; splits * M * N
 * * 4 bytes of partials for the MFMA GEMM), with the sizes in the message.
 */
int w4a16_gemm_noalloc(const uint16_t *a, const int32_t *b_packed, const uint16_t *scales,
                       const int32_t *qzeros, int64_t M, int64_t K, int64_t N, int64_t G,
                       int32_t zp_bias, uint16_t *out, hipStream_t stream);

/* One W4A16 linear of a decode stack (host struct; pointers are device). */
typedef struct {
    const int32_t *b_packed;  /* [K, N/8] */
    const uint16_t *scales;   /* [K/G, N] fp16 */
    const int32_t *qzeros;    /* [K/G, N/8] or NULL */
    int64_t K, N, G;
    int32_t zp_bias;
} w4a16_linear;

/* Glue applied to a linear's input by w4a16_gemm_glue. */
typedef enum {
    W4A16_GLUE_NONE = 0,    /* out = x[:, :K] . W                                   */
    W4A16_GLUE_RMSNORM = 1, /* out = rn(x[:, :K]) . W                               */
    W4A16_GLUE_SWIGLU = 2   /* out = rn(silu(x[:, :K]) * x[:, K:2K]) . W            */
} w4a16_glue;

/*
 * One W4A16 linear on glue-transformed activations: the linears of the decode
 * step (w4a16_decode_step is exactly a sequence of these calls, below).
 * Follows: the vLLM PR #37352 write-up, "Code analysis" item 1, for the
 * product; the glue between the linears of a decode pass (the inference-
 * engine article, section 1.1, gives the blocks but no glue) is this
 * library's reading:
 *     rn(v)   = v / sqrt(mean(v^2) + 1e-6) per row, in fp32
 *     silu(g) = g / (1 + exp(-g))
 * Where the glue runs inside the GEMM (the default for the GEMV of M <= 8:
 * the row-norm, and SwiGLU below 3 rows) the row scale multiplies the
 * products, so the normalised activations are not rounded to fp16 on their
 * own; where it runs as a kernel of its own (the default for the MFMA GEMM
 * of M >= 9), its fp16 output goes through `workspace` and the GEMM reads it.
 *
 *   glue       a w4a16_glue value.
 *   x          device fp16 rows of ldx elements: NONE reads [M, K] (ldx must
 *              equal K), RMSNORM [M, K], SWIGLU [M, 2K] (gate, then up).
 *   ldx        row stride in elements, a multiple of 8.
 *   lin        host pointer to the linear (weights as for w4a16_gemm).
 *   M          >= 0 rows (0: no-op).
 *   out        device fp16 [M, N]; must not overlap x, the weights or
 *              workspace.
 *   workspace  device scratch of w4a16_gemm_glue_workspace_bytes() bytes
 *              (0 when the glue runs inside the GEMM; NULL is then allowed),
 *              caller-owned, not overlapping x or out.
 * Errors: as w4a16_gemm; INVALID_ARG for a bad glue value, ldx, overlap or a
 * short workspace; UNSUPPORTED for glue with K % 8 != 0 or K > 32768.
 */
size_t w4a16_gemm_glue_workspace_bytes(int glue, int64_t M, const w4a16_linear *lin);
int w4a16_gemm_glue(int glue, const uint16_t *x, int64_t ldx, const w4a16_linear *lin, int64_t M,
                    uint16_t *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * y[m][0..width) = rn(x[m][0..width)) (rn as for w4a16_gemm_glue), rounded to
 * fp16: the last step of w4a16_decode_step.  x device fp16 rows of ldx
 * elements (ldx >= width, both multiples of 8, width <= 32768); y device fp16
 * [M, width], not overlapping x.  Errors: INVALID_ARG / UNSUPPORTED for bad
 * sizes, HIP on launch failure.
 */
int w4a16_rownorm(const uint16_t *x, int64_t ldx, int64_t M, int64_t width, uint16_t *y, hipStream_t stream);

/*
 * Scratch bytes w4a16_decode_step needs for M rows and this stack (0 if the
 * stack is malformed): three buffers of M x (widest linear output) fp16.
 * Host-only, no HIP calls.
 */
size_t w4a16_decode_workspace_bytes(int64_t M, const w4a16_linear *lin, int64_t n_layers);

/*
 * One decode step through n_layers transformer layers' linears.
 * Follows: the decode phase of the from-scratch C++/CUDA inference-engine
 * article (pt.news.hada.io topic 18295, section 1.1: one pass through the
 * stack of blocks per generated token) with every linear a W4A16 GEMM.  The
 * pages give no glue between the linears; this step uses, per layer with
 * hidden H and MLP width I (both read from the stack):
 *     q  = lin[4l+0](x)                  [M, Nq], Nq >= H
 *     h1 = rn(q[:, :H])                  (stands in for attention)
 *     h2 = rn(lin[4l+1](h1))             [M, H]
 *     gu = lin[4l+2](h2)                 [M, 2I]
 *     h3 = rn(silu(gu[:, :I]) * gu[:, I:])
 *     x  = rn(lin[4l+3](h3))             [M, H]
 * rn(v) = v / sqrt(mean(v^2) + 1e-6) per row, computed in fp32; silu(x) =
 * x / (1 + exp(-x)).  The step is exactly these calls (P, Q, R the three
 * workspace buffers, glue scratch in R):
 *     layer 0:   w4a16_gemm_glue(NONE, x_in, H, qkv)          -> P
 *     layer l>0: w4a16_gemm_glue(RMSNORM, Q, H, qkv)          -> P
 *                w4a16_gemm_glue(RMSNORM, P, Nq, o)           -> Q
 *                w4a16_gemm_glue(RMSNORM, Q, H, gate_up)      -> P
 *                w4a16_gemm_glue(SWIGLU, P, 2I, down)         -> Q
 *     then       w4a16_rownorm(Q, H, M, H)                    -> x_out
 * so each row-norm and SwiGLU folds into the GEMM that consumes it where
 * that GEMM can take it (see w4a16_gemm_glue).  Intermediates are stored as
 * fp16.
 *
 *   lin        host array of 4*n_layers linears: qkv, o, gate_up, down per layer
 *              (shapes must chain as above, else INVALID_ARG; H and I must be
 *              multiples of 8 and at most 32768, else UNSUPPORTED).
 *   x_in       device fp16 [M, H]; x_out device fp16 [M, H] (may equal x_in).
 *   M          1..8192 rows.
 *   workspace  device scratch of at least w4a16_decode_workspace_bytes(...)
 *              bytes, caller-owned, not shared with a concurrent call.
 * Errors: INVALID_ARG for a malformed stack, NULL pointers, M out of range or
 * a workspace smaller than required; otherwise as w4a16_gemm.
 */
int w4a16_decode_step(const w4a16_linear *lin, int64_t n_layers, const uint16_t *x_in,
                      uint16_t *x_out, int64_t M, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Describe the plan w4a16_gemm would run for a shape (host-only, no HIP calls):
 * path 1 = GEMV on the vector ALUs (dot2), 3 = GEMV with its k-reduction on
 * the matrix cores (M <= 8, the default there), 2 = MFMA GEMM (tiles of 16+
 * rows); splits = K-splits across workgroups;
 * grid = workgroups launched.  Returns the status w4a16_gemm would return from
 * validation of the sizes alone (pointers are not examined).
 */
int w4a16_gemm_plan(int64_t M, int64_t K, int64_t N, int64_t G, int32_t *path,
                    int32_t *splits, int64_t *grid);

/* Replace the planner's tuning overrides (the same "key=value,..." form the
 * environment variable W4A16_TUNE gives at first use; NULL or "" restores the
 * defaults).  Keys: gemv_mma (1 default: the matrix-core GEMV at M <= 8;
 * 0: the dot2 GEMV), gemv_mma_exact (1 default: the matrix-core GEMV takes
 * exact (q - z) weights; 0: with a symmetric zero point, biased weights and
 * the zero term folded per chunk), gemv_mma_words (2 or 4
 * words per lane: 256- or 512-column tiles, M <= 2; 0 by fill),
 * gemv_target_waves (the dot2 GEMV's M <= 2 wave target),
 * gemv_waves (4 or 8; 4 selects the dot2 GEMV), gemv_splits,
 * gemv_fold (dot2 GEMV: 1 folded form, 0 exact form, -1 folded for symmetric
 * zero point at M <= 2), gemv_max_m,
 * mfma_target_waves, mfma_splits, mfma_cfg (1..3: 16-row x 256-column, 32 x 256,
 * 32 x 128 wave tiles), mfma_mgroup (row tiles
 * walked per column tile by consecutive workgroups), max_partial_bytes,
 * decode_fuse (0: the decode step runs its glue as separate kernels),
 * decode_swiglu_m (GEMV route: from this many rows on, default 3, SwiGLU +
 * row-norm runs as a kernel of its own instead of inside the down GEMV),
 * decode_rn_mfma (1: the MFMA GEMMs of M >= 9 fold the row-norm, applying the
 * row scale to the products, instead of reading the row-norm kernel's fp16
 * output), mfma_tall_m (the M from which the 128 x 128 MFMA GEMM whose waves
 * each convert a 32-column strip runs, default 161; 0: never; at most 8
 * K-splits), mfma_tall_kg (its K-groups of four waves per workgroup, 1 or 2;
 * default 0: two where the grid still fits one round of the chip),
 * mfma_tall_rt (its MFMA row tiles per workgroup tile, 2, 4 or 8; default 0: 8), mfma_shared_m (the M from which the MFMA GEMM sharing
 * dequantised weights between row waves through LDS runs, default 0:
 * never), mfma_wm (its row waves per workgroup, 2 or 4; 0:
 * 4 above 64 rows), mfma_shared_kw (1: one K-wave per workgroup, one wave
 * per SIMD with a deeper load ring), mfma_tile_m (the M from which a
 * 128-row x 256-column workgroup tile runs that also stages the activations
 * in LDS; default 0: never; groups of at most 64 per K-split).  Every
 * choice computes the same product; they differ in speed and in fp32
 * rounding.  Unknown keys or malformed values: W4A16_ERR_INVALID_ARG and the
 * current settings stay.  Affects calls planned after it returns; not
 * meant to race with calls in flight on other threads. */
int w4a16_set_tuning(const char *spec);

/* Free library-owned scratch on every device (current and retired sets) after
 * synchronising the streams that used it.  Safe to call at any time no w4a16
 * call is in flight; graphs that captured w4a16 calls must not be replayed
 * afterwards (their scratch is gone). */
int w4a16_release(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
