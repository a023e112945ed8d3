/*
 * w4a16_oracle.c -- plain, slow, obviously-correct CPU oracle for the W4A16
 * weight-only-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library under
 * w4a16_weight_only_amd/) includes, links or calls this file; only the tests,
 * the smoke check and the benchmark's CPU-baseline leg do.  It shares no code,
 * header, table or constant with the GPU path.
 *
 * Sources (the pages this follows):
 *   [VLLM-37352] "vLLM PR #37352: Triton-based W4A16 kernel for AMD ROCm"
 *                (blog.secrett2633.cloud PR analysis), section "Code analysis"
 *                item 1 (the reference dequantize-then-matmul formula and the
 *                kernel call with group_size / qzeros / zp_bias) and item 2
 *                (checkpoint [N, K/8] -> kernel [K, N/8] repack with the
 *                weight [K, N/8] and scale [K/G, N] shape assertions).
 *
 * What is computed (the plain definition, no blocking or reordering):
 *   W[k][n]   = (q[k][n] - z[k/G][n]) * s[k/G][n]      (exact in double)
 *   out[m][n] = fp16_rne( sum_{k=0..K-1} A[m][k] * W[k][n] )   ascending k,
 *               accumulated in double, rounded once to fp16.
 * The page's formula converts (q - z) to fp32, multiplies by the scale and
 * does an fp32 matmul; every product here is exact in double and the sum is
 * far more precise than fp32, so this is the page's formula evaluated closer
 * to the exact value.
 *
 * Readings where the page is silent (each one also listed in the design notes):
 *   - packed words hold 8 unsigned nibbles; nibble j (bits 4j..4j+3) is the
 *     lowest-index element j of the 8 it packs (column for [K, N/8], row k for
 *     the checkpoint [N, K/8]); words are handled as uint32 bit patterns;
 *   - qzeros, when given, is [K/G, N/8] packed like the weights and the stored
 *     nibble is the zero point itself; it overrides zp_bias;
 *   - the group of row k is floor(k / G); scales are fp16 [K/G, N];
 *   - output is fp16 [M, N] row-major, round-to-nearest-even.
 *
 * fp16 handling is written here from the IEEE-754 binary16 definition
 * (1 sign, 5 exponent bits biased by 15, 10 fraction bits).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define W4O_OK 0
#define W4O_EINVAL 1

/* ---------------------------------------------------------------- fp16 --- */

/* binary16 bits -> double (exact for every input). */
double w4o_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* 1.f * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* Round a non-negative double holding an integer-plus-fraction to the nearest
 * integer, ties to even. */
static double rne_int(double q)
{
    double r = floor(q);
    double d = q - r;                              /* exact */
    if (d > 0.5 || (d == 0.5 && fmod(r, 2.0) != 0.0))
        r += 1.0;
    return r;
}

/* double -> binary16 bits, round to nearest even; overflow -> inf;
 * NaN -> quiet NaN with the input's sign. */
uint16_t w4o_f64_to_f16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    if (isinf(x))
        return (uint16_t)(sign | 0x7c00);
    if (ax == 0.0)
        return sign;
    if (ax < ldexp(1.0, -14)) {                    /* subnormal range */
        double q = rne_int(ldexp(ax, 24));         /* units of 2^-24 */
        return (uint16_t)(sign | (uint16_t)q);     /* q == 1024 -> min normal */
    }
    int E;
    frexp(ax, &E);                                 /* ax = f*2^E, f in [0.5,1) */
    int e = E - 1;                                 /* ax in [2^e, 2^(e+1)) */
    double q = rne_int(ldexp(ax, 10 - e));         /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7c00);          /* overflow -> inf */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

/* ------------------------------------------------------------- unpack --- */

/* Nibble j of a packed word, treated as an unsigned 32-bit pattern. */
static int nibble(int32_t word, int j)
{
    return (int)(((uint32_t)word >> (4 * j)) & 0xfu);
}

/* q[k][n] from the kernel layout [K, N/8]. */
static int q_kn8(const int32_t *b, int64_t N, int64_t k, int64_t n)
{
    return nibble(b[k * (N / 8) + n / 8], (int)(n % 8));
}

/* q[k][n] from the checkpoint layout [N, K/8]. */
static int q_nk8(const int32_t *src, int64_t K, int64_t k, int64_t n)
{
    return nibble(src[n * (K / 8) + k / 8], (int)(k % 8));
}

/* Zero point of (group g, column n). */
static int zero_of(const int32_t *qzeros, int32_t zp_bias, int64_t N, int64_t g, int64_t n)
{
    if (qzeros)
        return nibble(qzeros[g * (N / 8) + n / 8], (int)(n % 8));
    return (int)zp_bias;
}

static int check_shape(int64_t M, int64_t K, int64_t N, int64_t G)
{
    if (M < 0 || K <= 0 || N <= 0 || G <= 0) return W4O_EINVAL;
    if (N % 8 != 0 || K % G != 0) return W4O_EINVAL;
    return W4O_OK;
}

/* One output element, straight from the definition.  `layout_nk8` selects
 * where the weight nibble is read from, so that the repacked and the
 * checkpoint layouts can be checked against each other. */
static double dot_one(const double *arow, const int32_t *b, int layout_nk8,
                      const double *scol_by_group, const int32_t *qzeros,
                      int32_t zp_bias, int64_t K, int64_t N, int64_t G, int64_t n)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        int64_t g = k / G;
        int q = layout_nk8 ? q_nk8(b, K, k, n) : q_kn8(b, N, k, n);
        int z = zero_of(qzeros, zp_bias, N, g, n);
        double w = (double)(q - z) * scol_by_group[g];  /* exact */
        acc += arow[k] * w;                             /* exact product */
    }
    return acc;
}

static int gemm_impl(const uint16_t *a, const int32_t *b, int layout_nk8,
                     const uint16_t *scales, const int32_t *qzeros,
                     int64_t M, int64_t K, int64_t N, int64_t G, int32_t zp_bias,
                     uint16_t *out, double *acc_out)
{
    if (check_shape(M, K, N, G) != W4O_OK) return W4O_EINVAL;
    if (!a || !b || !scales || !out) return W4O_EINVAL;
    if (M == 0) return W4O_OK;
    int64_t NG = K / G;
    double *A = (double *)malloc(sizeof(double) * (size_t)(M * K));
    double *scol = (double *)malloc(sizeof(double) * (size_t)NG);
    if (!A || !scol) { free(A); free(scol); return W4O_EINVAL; }
    for (int64_t i = 0; i < M * K; ++i) A[i] = w4o_f16_to_f64(a[i]);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < NG; ++g) scol[g] = w4o_f16_to_f64(scales[g * N + n]);
        for (int64_t m = 0; m < M; ++m) {
            double acc = dot_one(A + m * K, b, layout_nk8, scol, qzeros, zp_bias, K, N, G, n);
            if (acc_out) acc_out[m * N + n] = acc;
            out[m * N + n] = w4o_f64_to_f16(acc);
        }
    }
    free(A);
    free(scol);
    return W4O_OK;
}

/* out = a . ((q - z) * s) with b in the kernel layout [K, N/8].
 * a: fp16 bits [M, K]; scales: fp16 bits [K/G, N]; qzeros: [K/G, N/8] or NULL
 * (then z = zp_bias); out: fp16 bits [M, N]; acc_out: optional double [M, N]
 * holding the unrounded sums. */
int w4o_gemm(const uint16_t *a, const int32_t *b_kn8, const uint16_t *scales,
             const int32_t *qzeros, int64_t M, int64_t K, int64_t N, int64_t G,
             int32_t zp_bias, uint16_t *out, double *acc_out)
{
    return gemm_impl(a, b_kn8, 0, scales, qzeros, M, K, N, G, zp_bias, out, acc_out);
}

/* Same product, reading the weight nibbles from the checkpoint layout [N, K/8]
 * (K % 8 == 0).  Used to check that repacking preserves the operator. */
int w4o_gemm_nk8(const uint16_t *a, const int32_t *b_nk8, const uint16_t *scales,
                 const int32_t *qzeros, int64_t M, int64_t K, int64_t N, int64_t G,
                 int32_t zp_bias, uint16_t *out, double *acc_out)
{
    if (K % 8 != 0) return W4O_EINVAL;
    return gemm_impl(a, b_nk8, 1, scales, qzeros, M, K, N, G, zp_bias, out, acc_out);
}

/* A sample of output elements (m_idx[i], n_idx[i]) of w4o_gemm, computed one
 * by one; for checking full-size problems without the whole product. */
int w4o_gemm_sample(const uint16_t *a, const int32_t *b_kn8, const uint16_t *scales,
                    const int32_t *qzeros, int64_t M, int64_t K, int64_t N, int64_t G,
                    int32_t zp_bias, const int64_t *m_idx, const int64_t *n_idx,
                    int64_t count, uint16_t *out, double *acc_out)
{
    if (check_shape(M, K, N, G) != W4O_OK) return W4O_EINVAL;
    int64_t NG = K / G;
    double *arow = (double *)malloc(sizeof(double) * (size_t)K);
    double *scol = (double *)malloc(sizeof(double) * (size_t)NG);
    if (!arow || !scol) { free(arow); free(scol); return W4O_EINVAL; }
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = m_idx[i], n = n_idx[i];
        if (m < 0 || m >= M || n < 0 || n >= N) { free(arow); free(scol); return W4O_EINVAL; }
        for (int64_t k = 0; k < K; ++k) arow[k] = w4o_f16_to_f64(a[m * K + k]);
        for (int64_t g = 0; g < NG; ++g) scol[g] = w4o_f16_to_f64(scales[g * N + n]);
        double acc = dot_one(arow, b_kn8, 0, scol, qzeros, zp_bias, K, N, G, n);
        if (acc_out) acc_out[i] = acc;
        out[i] = w4o_f64_to_f16(acc);
    }
    free(arow);
    free(scol);
    return W4O_OK;
}

/* ------------------------------------------------------------- repack --- */

/* Checkpoint [N, K/8] -> kernel [K, N/8]: the nibble of (row k, column n)
 * moves from word (n, k/8) position k%8 to word (k, n/8) position n%8.
 * Bit-exact; dst must not alias src. */
int w4o_repack(const int32_t *src_nk8, int32_t *dst_kn8, int64_t K, int64_t N)
{
    if (K <= 0 || N <= 0 || K % 8 != 0 || N % 8 != 0) return W4O_EINVAL;
    memset(dst_kn8, 0, sizeof(int32_t) * (size_t)(K * (N / 8)));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            uint32_t nib = (uint32_t)q_nk8(src_nk8, K, k, n);
            uint32_t *w = (uint32_t *)&dst_kn8[k * (N / 8) + n / 8];
            *w |= nib << (4 * (n % 8));
        }
    }
    return W4O_OK;
}

/* Checkpoint group scales [N, Gn] -> kernel [Gn, N] (vLLM PR #37352 write-up,
 * "Code analysis" item 2: the loaded scale tensor has shape (K/G, N); the
 * checkpoint's own orientation, per output column, is this library's reading).
 * The value of (column n, group g) moves from src[n][g] to dst[g][n]: 16-bit
 * patterns copied unchanged.  dst must not alias src. */
int w4o_repack_scales(const uint16_t *src_ng, uint16_t *dst_gn, int64_t Gn, int64_t N)
{
    if (Gn <= 0 || N <= 0) return W4O_EINVAL;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t g = 0; g < Gn; ++g) dst_gn[g * N + n] = src_ng[n * Gn + g];
    return W4O_OK;
}

/* ------------------------------------------------------ decode-step glue --- */
/*
 * The decode step chains four linears per layer (QKV, O, gate+up, down) with
 * row re-normalisation between them.  The pages give no glue; the reading used
 * (documented with the design) is, per layer with hidden H and MLP width I:
 *   q  = lin0(x)            [M, Nq]   (Nq >= H)
 *   h1 = rn(q[:, :H])                 (stand-in for attention)
 *   o  = lin1(h1)           [M, H];  h2 = rn(o)
 *   gu = lin2(h2)           [M, 2I]; h3 = rn(silu(gu[:, :I]) * gu[:, I:])
 *   d  = lin3(h3)           [M, H];  x' = rn(d)
 * rn(v) = v / sqrt(mean(v^2) + 1e-6) per row; silu(x) = x / (1 + exp(-x)).
 * Every intermediate is rounded to fp16 where it is stored.
 */

/* y[m][0..width) = rn(x[m][0..width)), x with row stride ldx (elements). */
int w4o_rownorm(const uint16_t *x, int64_t M, int64_t ldx, int64_t width, uint16_t *y)
{
    if (M < 0 || width <= 0 || ldx < width) return W4O_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t j = 0; j < width; ++j) {
            double v = w4o_f16_to_f64(x[m * ldx + j]);
            ss += v * v;
        }
        double inv = 1.0 / sqrt(ss / (double)width + 1e-6);
        for (int64_t j = 0; j < width; ++j)
            y[m * width + j] = w4o_f64_to_f16(w4o_f16_to_f64(x[m * ldx + j]) * inv);
    }
    return W4O_OK;
}

/* y[m][i] = rn_row( silu(gu[m][i]) * gu[m][I + i] ), gu is [M, 2I]. */
int w4o_swiglu_rownorm(const uint16_t *gu, int64_t M, int64_t I, uint16_t *y)
{
    if (M < 0 || I <= 0) return W4O_EINVAL;
    double *t = (double *)malloc(sizeof(double) * (size_t)I);
    if (!t) return W4O_EINVAL;
    for (int64_t m = 0; m < M; ++m) {
        double ss = 0.0;
        for (int64_t i = 0; i < I; ++i) {
            double g = w4o_f16_to_f64(gu[m * 2 * I + i]);
            double u = w4o_f16_to_f64(gu[m * 2 * I + I + i]);
            t[i] = g / (1.0 + exp(-g)) * u;
            ss += t[i] * t[i];
        }
        double inv = 1.0 / sqrt(ss / (double)I + 1e-6);
        for (int64_t i = 0; i < I; ++i)
            y[m * I + i] = w4o_f64_to_f16(t[i] * inv);
    }
    free(t);
    return W4O_OK;
}

/* One linear of a decode stack, host pointers. */
typedef struct {
    const int32_t *b_packed;   /* [K, N/8] */
    const uint16_t *scales;    /* [K/G, N] */
    const int32_t *qzeros;     /* [K/G, N/8] or NULL */
    int64_t K, N, G;
    int32_t zp_bias;
} w4o_linear;

/* Full decode step over n_layers layers (lin has 4*n_layers entries in the
 * order qkv, o, gate_up, down).  x_in/x_out: fp16 [M, H].  Slow: meant for
 * small stacks.  Intermediates are rounded to fp16 at each store. */
int w4o_decode_step(const w4o_linear *lin, int64_t n_layers, const uint16_t *x_in,
                    uint16_t *x_out, int64_t M)
{
    if (n_layers <= 0 || M <= 0) return W4O_EINVAL;
    int64_t H = lin[0].K;
    int64_t maxN = 0;
    for (int64_t i = 0; i < 4 * n_layers; ++i)
        if (lin[i].N > maxN) maxN = lin[i].N;
    uint16_t *x = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * H));
    uint16_t *t = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * maxN));
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)(M * maxN));
    int rc = W4O_OK;
    if (!x || !t || !h) { rc = W4O_EINVAL; goto done; }
    memcpy(x, x_in, sizeof(uint16_t) * (size_t)(M * H));
    for (int64_t l = 0; l < n_layers && rc == W4O_OK; ++l) {
        const w4o_linear *L = lin + 4 * l;
        int64_t I = L[2].N / 2;
        if (L[0].K != H || L[0].N < H || L[1].K != H || L[1].N != H || L[2].K != H ||
            L[2].N % 2 != 0 || L[3].K != I || L[3].N != H) { rc = W4O_EINVAL; break; }
        rc |= w4o_gemm(x, L[0].b_packed, L[0].scales, L[0].qzeros, M, H, L[0].N, L[0].G, L[0].zp_bias, t, NULL);
        rc |= w4o_rownorm(t, M, L[0].N, H, h);
        rc |= w4o_gemm(h, L[1].b_packed, L[1].scales, L[1].qzeros, M, H, H, L[1].G, L[1].zp_bias, t, NULL);
        rc |= w4o_rownorm(t, M, H, H, h);
        rc |= w4o_gemm(h, L[2].b_packed, L[2].scales, L[2].qzeros, M, H, 2 * I, L[2].G, L[2].zp_bias, t, NULL);
        rc |= w4o_swiglu_rownorm(t, M, I, h);
        rc |= w4o_gemm(h, L[3].b_packed, L[3].scales, L[3].qzeros, M, I, H, L[3].G, L[3].zp_bias, t, NULL);
        rc |= w4o_rownorm(t, M, H, H, x);
    }
    if (rc == W4O_OK) memcpy(x_out, x, sizeof(uint16_t) * (size_t)(M * H));
done:
    free(x);
    free(t);
    free(h);
    return rc;
}
