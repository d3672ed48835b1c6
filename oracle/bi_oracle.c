/*
 * bi_oracle.c -- plain, slow, fixed-order CPU oracle for the batch-invariant
 * reductions (dense matmul, group-quantized matmul, RMSNorm, decode/verify
 * attention) and the pointwise pieces of a Llama-style decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file.  It is used by the tests, by the package's smoke
 * check and by the benchmark's CPU-baseline leg.  It shares no code, header,
 * table or constant with the HIP kernels.
 *
 * Arithmetic conventions (the oracle's own fixed order):
 *   - every input is widened to fp32 exactly (bf16 / fp16 / e2m1 / e4m3 are
 *     subsets of fp32);
 *   - every reduction is a sequential left fold in fp32 in ascending index
 *     order, one rounded multiply then one rounded add per term (the file is
 *     compiled with -ffp-contract=off so no fused multiply-add is formed);
 *   - results are returned as raw fp32; rounding to a 16-bit output type is a
 *     separate, explicit step (bo_round) using round-to-nearest-even.
 * The sequential fp32 fold is the reduction the "Batch-invariant kernels"
 * chapter uses in its worked examples (Case 2 `sequential`, Case 4
 * `sum_sq_ordered`); a fixed order is all batch invariance asks for, and the
 * parity tests hold the GPU to this result within the stated tolerance.
 *
 * Parallelism: OpenMP splits only independent outputs (rows, column blocks,
 * attention rows); no single output's fold is ever split.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { BO_BF16 = 0, BO_F16 = 1, BO_F32 = 2 };
enum { BO_AFFINE = 0, BO_NVFP4 = 1, BO_MXFP4 = 2, BO_MXFP8 = 3 };

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the upper half of an fp32 word. */
float bo_bf16_to_f32(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* fp32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t bo_f32_to_bf16(float f)
{
    uint32_t u = f32_to_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)               /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;                                /* carries into the exponent on overflow -> inf */
    return (uint16_t)(u >> 16);
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
float bo_f16_to_f32(uint16_t h)
{
    uint32_t s = (uint32_t)(h >> 15) & 1u;
    uint32_t e = (uint32_t)(h >> 10) & 0x1fu;
    uint32_t m = (uint32_t)h & 0x3ffu;
    float v;
    if (e == 0) {
        v = ldexpf((float)m, -24);                     /* zero or subnormal: m * 2^-24 */
    } else if (e == 31) {
        v = m ? bits_to_f32(0x7fc00000u) : INFINITY;
    } else {
        v = bits_to_f32(((e + 112u) << 23) | (m << 13)); /* rebias 15 -> 127 */
    }
    return s ? -v : v;
}

/* fp32 -> binary16, round to nearest, ties to even (subnormals included,
 * overflow to infinity). */
uint16_t bo_f32_to_f16(float f)
{
    uint32_t u = f32_to_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);      /* NaN */
    uint32_t e8 = a >> 23;
    if (e8 >= 143u) return (uint16_t)(sign | 0x7c00u);          /* |f| >= 2^16: inf */
    if (e8 >= 113u) {                                           /* normal binary16 range */
        uint32_t m23 = a & 0x7fffffu;
        uint32_t h = ((e8 - 112u) << 10) | (m23 >> 13);
        uint32_t rem = m23 & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
        if (h >= 0x7c00u) h = 0x7c00u;
        return (uint16_t)(sign | h);
    }
    /* subnormal or zero: value = n * 2^-24 with n an integer in [0, 1024] */
    float scaled = ldexpf(bits_to_f32(a), 24);                  /* exact */
    float n = nearbyintf(scaled);                               /* default mode: ties to even */
    return (uint16_t)(sign | (uint16_t)n);                      /* n == 1024 is the smallest normal */
}

/* OCP e2m1 (4-bit): 1 sign, 2 exponent (bias 1), 1 mantissa; no inf/NaN. */
float bo_e2m1_to_f32(uint8_t c)
{
    uint32_t s = (c >> 3) & 1u, e = (c >> 1) & 3u, m = c & 1u;
    float v = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
    return s ? -v : v;
}

/* OCP e4m3 "fn": 1 sign, 4 exponent (bias 7), 3 mantissa; S.1111.111 is NaN,
 * no infinities, subnormals m/8 * 2^-6. */
float bo_e4m3_to_f32(uint8_t c)
{
    uint32_t s = (c >> 7) & 1u, e = (c >> 3) & 0xfu, m = c & 7u;
    float v;
    if (e == 15u && m == 7u) v = bits_to_f32(0x7fc00000u);
    else if (e == 0) v = ldexpf((float)m / 8.0f, -6);
    else v = ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
    return s ? -v : v;
}

/* OCP MX e8m0 scale: an unsigned biased exponent, value 2^(e - 127); the
 * byte 0xFF is NaN.  2^-127 is an fp32 subnormal, so every value is exact. */
float bo_e8m0_to_f32(uint8_t e)
{
    if (e == 0xffu) return bits_to_f32(0x7fc00000u);
    return ldexpf(1.0f, (int)e - 127);
}

static float load_elem(const void *p, int64_t i, int dtype)
{
    switch (dtype) {
    case BO_BF16: return bo_bf16_to_f32(((const uint16_t *)p)[i]);
    case BO_F16:  return bo_f16_to_f32(((const uint16_t *)p)[i]);
    default:      return ((const float *)p)[i];
    }
}

static int valid_dtype(int dtype) { return dtype == BO_BF16 || dtype == BO_F16 || dtype == BO_F32; }

/* Round fp32 values to the storage type (RNE); F32 is a plain copy. */
int bo_round(const float *in, void *out, int64_t n, int dtype)
{
    if (!valid_dtype(dtype) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == BO_BF16) ((uint16_t *)out)[i] = bo_f32_to_bf16(in[i]);
        else if (dtype == BO_F16) ((uint16_t *)out)[i] = bo_f32_to_f16(in[i]);
        else ((float *)out)[i] = in[i];
    }
    return 0;
}

int bo_widen(const void *in, float *out, int64_t n, int dtype)
{
    if (!valid_dtype(dtype) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = load_elem(in, i, dtype);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Fold primitives: the reduction trees of the chapter's Case 1 and Case 2.  */
/* ------------------------------------------------------------------------ */

/* sequential left fold, one rounded add per element */
float bo_fold_seq_f32(const float *a, int64_t n)
{
    float s = 0.0f;
    for (int64_t i = 0; i < n; ++i) s = s + a[i];
    return s;
}

double bo_fold_seq_f64(const double *a, int64_t n)
{
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s = s + a[i];
    return s;
}

/* pairwise: add adjacent pairs level by level; an odd last element is carried
 * to the next level unchanged. */
float bo_fold_pairwise_f32(const float *a, int64_t n)
{
    if (n <= 0) return 0.0f;
    float *t = (float *)malloc((size_t)n * sizeof(float));
    if (!t) return NAN;
    memcpy(t, a, (size_t)n * sizeof(float));
    while (n > 1) {
        int64_t h = 0;
        for (int64_t i = 0; i + 1 < n; i += 2) t[h++] = t[i] + t[i + 1];
        if (n & 1) t[h++] = t[n - 1];
        n = h;
    }
    float r = t[0];
    free(t);
    return r;
}

/* split reduction: `splits` contiguous chunks, the first n % splits of them one
 * element longer; each chunk folded sequentially, then the partials folded
 * sequentially in chunk order. */
float bo_fold_split_f32(const float *a, int64_t n, int64_t splits)
{
    if (splits < 1) return NAN;
    float *part = (float *)calloc((size_t)splits, sizeof(float));
    if (!part) return NAN;
    int64_t base = n / splits, extra = n % splits, at = 0;
    for (int64_t c = 0; c < splits; ++c) {
        int64_t len = base + (c < extra ? 1 : 0);
        part[c] = bo_fold_seq_f32(a + at, len);
        at += len;
    }
    float r = bo_fold_seq_f32(part, splits);
    free(part);
    return r;
}

/* ------------------------------------------------------------------------ */
/* Dense matmul  y[m,n] = sum_k x[m,k] * W[n,k]                             */
/* ------------------------------------------------------------------------ */

/* x: [M,K] of dtype; w: [N,K] when w_transposed else [K,N]; y: fp32 [M,N].
 * Each y[m,n] is the sequential fp32 fold over k = 0..K-1 of the rounded
 * product x*w (descending: k = K-1..0, the chapter's Case 4 "reverse" order,
 * a second valid fixed tree).  Work is vectorised across n, which leaves every
 * output's own order untouched. */
static int matmul_fold(const void *x, const void *w, float *y, int64_t M, int64_t N, int64_t K,
                       int dtype, int w_transposed, int descending)
{
    if (!x || !w || !y || M < 0 || N < 0 || K < 0 || !valid_dtype(dtype)) return -1;
    if (M == 0 || N == 0) return 0;
    float *xf = (float *)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(float));
    if (!xf) return -2;
    for (int64_t i = 0; i < M * K; ++i) xf[i] = load_elem(x, i, dtype);
    const int64_t NB = 256, MB = 8;
    const int64_t nblocks = (N + NB - 1) / NB;
    int err = 0;
#pragma omp parallel
    {
        float *wt = (float *)malloc((size_t)(K > 0 ? K : 1) * NB * sizeof(float));
        float *acc = (float *)malloc((size_t)(MB * NB) * sizeof(float));
        if (!wt || !acc) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic)
            for (int64_t b = 0; b < nblocks; ++b) {
                int64_t n0 = b * NB, nb = (N - n0 < NB) ? N - n0 : NB;
                for (int64_t k = 0; k < K; ++k)
                    for (int64_t j = 0; j < nb; ++j)
                        wt[k * NB + j] = w_transposed ? load_elem(w, (n0 + j) * K + k, dtype)
                                                      : load_elem(w, k * N + (n0 + j), dtype);
                /* Up to MB rows share one pass over the weight block; each
                 * output still folds k = 0..K-1 in order in its own acc. */
                for (int64_t m0 = 0; m0 < M; m0 += MB) {
                    const int64_t mb = (M - m0 < MB) ? M - m0 : MB;
                    for (int64_t i = 0; i < mb * NB; ++i) acc[i] = 0.0f;
                    for (int64_t kk = 0; kk < K; ++kk) {
                        const int64_t k = descending ? K - 1 - kk : kk;
                        const float *wr = wt + k * NB;
                        for (int64_t i = 0; i < mb; ++i) {
                            const float xv = xf[(m0 + i) * K + k];
                            float *ai = acc + i * NB;
                            for (int64_t j = 0; j < nb; ++j) ai[j] = ai[j] + xv * wr[j];
                        }
                    }
                    for (int64_t i = 0; i < mb; ++i)
                        for (int64_t j = 0; j < nb; ++j) y[(m0 + i) * N + n0 + j] = acc[i * NB + j];
                }
            }
        }
        free(wt);
        free(acc);
    }
    free(xf);
    return err;
}

int bo_matmul(const void *x, const void *w, float *y, int64_t M, int64_t N, int64_t K,
              int dtype, int w_transposed)
{
    return matmul_fold(x, w, y, M, N, K, dtype, w_transposed, 0);
}

int bo_matmul_desc(const void *x, const void *w, float *y, int64_t M, int64_t N, int64_t K,
                   int dtype, int w_transposed)
{
    return matmul_fold(x, w, y, M, N, K, dtype, w_transposed, 1);
}

/* ------------------------------------------------------------------------ */
/* Group-quantized weights: dequantize, then the dense matmul above.         */
/* ------------------------------------------------------------------------ */

/* Packed layout: every stored row is a little-endian bit stream of `bits`-bit
 * codes in 32-bit words: code j of the row occupies bits [j*bits, (j+1)*bits)
 * of the stream, bit i of the stream being bit i % 32 of word i / 32.  At 4
 * bits this is 8 codes per word with the lowest index in bits 0..3; at 8 bits
 * the codes are the row's bytes in order.
 * rows x cols is the weight matrix as stored, quantized along cols:
 *   transposed weights [N,K]: rows = N, cols = K;
 *   natural weights    [K,N]: rows = K, cols = N.
 * wq: [rows, cols*bits/32] words; scales: [rows, cols/gs]; biases: [rows, cols/gs].
 * Affine (2 to 8 bits): w = s*q + b with q in 0..2^bits-1 and binary16 s, b.
 *   The product s*q is exact in fp32 (at most 11 + 8 significant bits); the
 *   add rounds once in fp32; the result is rounded to binary16 (the
 *   activation type the weights are multiplied against).
 * NVFP4: w = e2m1(q) * e4m3(s), one scale byte per 16 elements; the product
 *   is exact in fp32 and exactly representable in binary16.
 * MXFP4: w = e2m1(q) * e8m0(s), one scale byte per 32 elements; the product is
 *   exact in fp32 (a power-of-two scaling of a 2-bit significand) and is then
 *   rounded to binary16 (values beyond its range become +-inf, tiny ones
 *   round to subnormals or zero).
 * MXFP8: w = e4m3(q) * e8m0(s), one byte code per element and one scale byte
 *   per 32; the product is exact in fp32 (a 4-bit significand scaled by a
 *   power of two, never below 2^-136) or overflows to inf, and is then
 *   rounded to binary16 as for MXFP4.
 * Output: binary16 bits, same [rows, cols] layout as the stored matrix. */
int bo_dequantize(const uint32_t *wq, const void *scales, const uint16_t *biases,
                  uint16_t *out, int64_t rows, int64_t cols, int qmode, int bits, int group_size)
{
    if (!wq || !scales || !out || rows < 0 || cols < 0) return -1;
    if (qmode == BO_AFFINE) {
        if (bits < 2 || bits > 8) return -3;
        if (group_size != 32 && group_size != 64 && group_size != 128) return -3;
        if (!biases) return -1;
    } else if (qmode == BO_NVFP4) {
        if (bits != 4 || group_size != 16) return -3;
    } else if (qmode == BO_MXFP4) {
        if (bits != 4 || group_size != 32) return -3;
    } else if (qmode == BO_MXFP8) {
        if (bits != 8 || group_size != 32) return -3;
    } else {
        return -1;
    }
    if (cols % group_size || (cols * bits) % 32) return -3;
    const int64_t words = cols * bits / 32, groups = cols / group_size;
    const uint32_t mask = (1u << bits) - 1u;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            /* the code's bits, one at a time from the row's stream */
            uint32_t q = 0;
            for (int i = 0; i < bits; ++i) {
                int64_t bit = c * bits + i;
                uint32_t word = wq[r * words + bit / 32];
                q |= ((word >> (bit % 32)) & 1u) << i;
            }
            q &= mask;
            int64_t g = r * groups + c / group_size;
            float v;
            if (qmode == BO_AFFINE) {
                float s = bo_f16_to_f32(((const uint16_t *)scales)[g]);
                float b = bo_f16_to_f32(biases[g]);
                float sq = s * (float)q;
                v = sq + b;
            } else if (qmode == BO_NVFP4) {
                v = bo_e2m1_to_f32((uint8_t)q) * bo_e4m3_to_f32(((const uint8_t *)scales)[g]);
            } else if (qmode == BO_MXFP4) {
                v = bo_e2m1_to_f32((uint8_t)q) * bo_e8m0_to_f32(((const uint8_t *)scales)[g]);
            } else {
                v = bo_e4m3_to_f32((uint8_t)q) * bo_e8m0_to_f32(((const uint8_t *)scales)[g]);
            }
            out[r * cols + c] = bo_f32_to_f16(v);
        }
    }
    return 0;
}

/* y = x @ dequantize(W)^T (transposed) or x @ dequantize(W) (natural);
 * x binary16 [M,K]; y fp32 [M,N]. */
int bo_qmatmul(const uint16_t *x, const uint32_t *wq, const void *scales, const uint16_t *biases,
               float *y, int64_t M, int64_t N, int64_t K, int qmode, int bits, int group_size, int w_transposed)
{
    if (!x || !y || M < 0 || N < 0 || K < 0) return -1;
    int64_t rows = w_transposed ? N : K, cols = w_transposed ? K : N;
    uint16_t *wd = (uint16_t *)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * 2);
    if (!wd) return -2;
    int rc = bo_dequantize(wq, scales, biases, wd, rows, cols, qmode, bits, group_size);
    if (rc == 0) rc = bo_matmul(x, wd, y, M, N, K, BO_F16, w_transposed);
    free(wd);
    return rc;
}

/* Expert ("gather") matmul of a mixture-of-experts layer:
 *   y[m, :] = x[lhs[m], :] @ dequantize(W[rhs[m]])^T   (transposed weights)
 *   y[m, :] = x[lhs[m], :] @ dequantize(W[rhs[m]])     (natural weights)
 * W holds E quantized matrices back to back, each stored as bo_dequantize
 * describes (codes, scales and biases each [E, ...]); lhs NULL reads x[m].
 * Every row is its own sequential fp32 fold over k, so a row's value does not
 * depend on the other rows or on their order.  A row whose lhs or rhs index is
 * out of range is NaN.  x binary16 [x_rows, K]; y fp32 [M, N]. */
int bo_gather_qmatmul(const uint16_t *x, const int32_t *lhs, const int32_t *rhs, const uint32_t *wq,
                      const void *scales, const uint16_t *biases, float *y, int64_t M, int64_t x_rows,
                      int64_t N, int64_t K, int64_t E, int qmode, int bits, int group_size, int w_transposed)
{
    if (!x || !rhs || !wq || !scales || !y || M < 0 || x_rows < 0 || N < 0 || K < 0 || E < 1) return -1;
    if (!lhs && x_rows < M) return -1;
    const int64_t rows = w_transposed ? N : K, cols = w_transposed ? K : N;
    if (group_size < 1 || cols % group_size || (cols * bits) % 32) return -3;
    const int64_t words_e = rows * cols * bits / 32, groups_e = rows * cols / group_size;
    const size_t ssz = qmode == BO_AFFINE ? 2 : 1;
    uint16_t *wd = (uint16_t *)malloc((size_t)(E * rows * cols > 0 ? E * rows * cols : 1) * 2);
    if (!wd) return -2;
    for (int64_t e = 0; e < E; ++e) {
        int rc = bo_dequantize(wq + e * words_e, (const uint8_t *)scales + e * groups_e * ssz,
                               biases ? biases + e * groups_e : NULL, wd + e * rows * cols, rows, cols, qmode, bits,
                               group_size);
        if (rc) {
            free(wd);
            return rc;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const int64_t xr = lhs ? lhs[m] : m, e = rhs[m];
        if (xr < 0 || xr >= x_rows || e < 0 || e >= E) {
            for (int64_t n = 0; n < N; ++n) y[m * N + n] = bits_to_f32(0x7fc00000u);
            continue;
        }
        const uint16_t *w = wd + e * rows * cols;
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                const float wv = bo_f16_to_f32(w_transposed ? w[n * K + k] : w[k * N + n]);
                acc = acc + bo_f16_to_f32(x[xr * K + k]) * wv;
            }
            y[m * N + n] = acc;
        }
    }
    free(wd);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm  y = (x * inv) * w,  inv = 1 / sqrt(sum(x^2) / H + eps)          */
/* ------------------------------------------------------------------------ */

/* x [rows,H] and w [H] of dtype; y fp32 [rows,H]; ss (optional) fp32 [rows]
 * receives each row's sequential sum of squares (ascending i; descending: the
 * chapter's Case 4 "reverse" order, a second valid fixed tree). */
static int rmsnorm_fold(const void *x, const void *w, float *y, float *ss, int64_t rows, int64_t H,
                        float eps, int dtype, int descending)
{
    if (!x || !w || !y || rows < 0 || H < 1 || !valid_dtype(dtype)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float s = 0.0f;
        for (int64_t ii = 0; ii < H; ++ii) {
            const int64_t i = descending ? H - 1 - ii : ii;
            float v = load_elem(x, r * H + i, dtype);
            s = s + v * v;
        }
        if (ss) ss[r] = s;
        float mean = s / (float)H;
        float inv = 1.0f / sqrtf(mean + eps);
        for (int64_t i = 0; i < H; ++i) {
            float v = load_elem(x, r * H + i, dtype);
            y[r * H + i] = (v * inv) * load_elem(w, i, dtype);
        }
    }
    return 0;
}

int bo_rmsnorm(const void *x, const void *w, float *y, float *ss, int64_t rows, int64_t H,
               float eps, int dtype)
{
    return rmsnorm_fold(x, w, y, ss, rows, H, eps, dtype, 0);
}

int bo_rmsnorm_desc(const void *x, const void *w, float *y, float *ss, int64_t rows, int64_t H,
                    float eps, int dtype)
{
    return rmsnorm_fold(x, w, y, ss, rows, H, eps, dtype, 1);
}

/* ------------------------------------------------------------------------ */
/* Scaled dot-product attention for decode / verify blocks.                  */
/* ------------------------------------------------------------------------ */

/* q [B,Q,Hq,D]; k, v [B,Lcap,Hkv,D] (dtype); kv_len [B]; o fp32 [B,Q,Hq,D].
 * Query j of sequence b sits at position p = kv_len[b] - Q + j.  With
 * `causal` it sees keys 0..p, otherwise keys 0..kv_len[b]-1.  Query head h
 * reads key/value head h / (Hq / Hkv).
 * Plain two-pass softmax: s_t = (q . k_t) * scale (sequential over d),
 * m = max s, p_t = exp(s_t - m), l = sum p_t, o_d = (sum_t p_t * v_td) / l,
 * every sum sequential in ascending index (descending: every sum -- over d
 * and over keys -- in descending index, a second valid fixed tree). */
static int sdpa_fold(const void *q, const void *k, const void *v, float *o, const int32_t *kv_len,
                     int64_t B, int64_t Q, int64_t Lcap, int64_t Hq, int64_t Hkv, int64_t D,
                     float scale, int causal, int dtype, int descending)
{
    if (!q || !k || !v || !o || !kv_len || B < 0 || Q < 1 || Lcap < 1 || Hq < 1 || Hkv < 1 || D < 1)
        return -1;
    if (Hq % Hkv) return -4;
    if (!valid_dtype(dtype)) return -1;
    for (int64_t b = 0; b < B; ++b)
        if (kv_len[b] < Q || kv_len[b] > Lcap) return -4;
    const int64_t G = Hq / Hkv;
    const int64_t rows = B * Q * Hq;
    int err = 0;
#pragma omp parallel
    {
        float *sc = (float *)malloc((size_t)Lcap * sizeof(float));
        float *qf = (float *)malloc((size_t)D * sizeof(float));
        float *acc = (float *)malloc((size_t)D * sizeof(float));
        if (!sc || !qf || !acc) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic)
            for (int64_t r = 0; r < rows; ++r) {
                int64_t h = r % Hq, j = (r / Hq) % Q, b = r / (Hq * Q);
                int64_t g = h / G;
                int64_t last = causal ? (int64_t)kv_len[b] - Q + j : (int64_t)kv_len[b] - 1;
                for (int64_t d = 0; d < D; ++d) qf[d] = load_elem(q, r * D + d, dtype);
                float m = -INFINITY;
                for (int64_t t = 0; t <= last; ++t) {
                    int64_t kb = ((b * Lcap + t) * Hkv + g) * D;
                    float dot = 0.0f;
                    for (int64_t dd = 0; dd < D; ++dd) {
                        const int64_t d = descending ? D - 1 - dd : dd;
                        dot = dot + qf[d] * load_elem(k, kb + d, dtype);
                    }
                    sc[t] = dot * scale;
                    if (sc[t] > m) m = sc[t];
                }
                for (int64_t t = 0; t <= last; ++t) sc[t] = expf(sc[t] - m);
                float l = 0.0f;
                for (int64_t tt = 0; tt <= last; ++tt) l = l + sc[descending ? last - tt : tt];
                for (int64_t d = 0; d < D; ++d) acc[d] = 0.0f;
                for (int64_t tt = 0; tt <= last; ++tt) {
                    const int64_t t = descending ? last - tt : tt;
                    int64_t vb = ((b * Lcap + t) * Hkv + g) * D;
                    for (int64_t d = 0; d < D; ++d) acc[d] = acc[d] + sc[t] * load_elem(v, vb + d, dtype);
                }
                for (int64_t d = 0; d < D; ++d) o[r * D + d] = acc[d] / l;
            }
        }
        free(sc);
        free(qf);
        free(acc);
    }
    return err;
}

int bo_sdpa(const void *q, const void *k, const void *v, float *o, const int32_t *kv_len,
            int64_t B, int64_t Q, int64_t Lcap, int64_t Hq, int64_t Hkv, int64_t D,
            float scale, int causal, int dtype)
{
    return sdpa_fold(q, k, v, o, kv_len, B, Q, Lcap, Hq, Hkv, D, scale, causal, dtype, 0);
}

int bo_sdpa_desc(const void *q, const void *k, const void *v, float *o, const int32_t *kv_len,
                 int64_t B, int64_t Q, int64_t Lcap, int64_t Hq, int64_t Hkv, int64_t D,
                 float scale, int causal, int dtype)
{
    return sdpa_fold(q, k, v, o, kv_len, B, Q, Lcap, Hq, Hkv, D, scale, causal, dtype, 1);
}

/* ------------------------------------------------------------------------ */
/* Pointwise pieces of the Llama-style decoder.                              */
/* ------------------------------------------------------------------------ */

/* Rotary embedding, rotate-half form, on x [T, nh, D] (dtype) with per-token
 * positions pos [T] and fp32 tables cos/sin [*, D/2]:
 *   out[i]       = x[i] * c_i - x[i+D/2] * s_i
 *   out[i+D/2]   = x[i+D/2] * c_i + x[i] * s_i           (i < D/2)
 * out fp32 [T, nh, D]. */
int bo_rope(const void *x, float *out, const int32_t *pos, const float *cos_t, const float *sin_t,
            int64_t T, int64_t nh, int64_t D, int dtype)
{
    if (!x || !out || !pos || !cos_t || !sin_t || D % 2 || !valid_dtype(dtype)) return -1;
    const int64_t half = D / 2;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < nh; ++h) {
            int64_t base = (t * nh + h) * D;
            const float *c = cos_t + (int64_t)pos[t] * half, *s = sin_t + (int64_t)pos[t] * half;
            for (int64_t i = 0; i < half; ++i) {
                float a = load_elem(x, base + i, dtype), bb = load_elem(x, base + i + half, dtype);
                out[base + i] = a * c[i] - bb * s[i];
                out[base + i + half] = bb * c[i] + a * s[i];
            }
        }
    return 0;
}

/* SwiGLU gate: out = silu(g) * u with silu(g) = g / (1 + exp(-g)). */
int bo_silu_mul(const void *g, const void *u, float *out, int64_t n, int dtype)
{
    if (!g || !u || !out || !valid_dtype(dtype)) return -1;
    for (int64_t i = 0; i < n; ++i) {
        float gv = load_elem(g, i, dtype);
        float sg = gv / (1.0f + expf(-gv));
        out[i] = sg * load_elem(u, i, dtype);
    }
    return 0;
}

/* Index of the largest element of each row; the lowest index wins ties. */
int bo_argmax(const void *x, int32_t *idx, int64_t rows, int64_t cols, int dtype)
{
    if (!x || !idx || cols < 1 || !valid_dtype(dtype)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t best = 0;
        float bv = load_elem(x, r * cols, dtype);
        for (int64_t c = 1; c < cols; ++c) {
            float v = load_elem(x, r * cols + c, dtype);
            if (v > bv) { bv = v; best = c; }
        }
        idx[r] = (int32_t)best;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Row log-softmax, token log-probability and row mean                     */
/* ------------------------------------------------------------------------ */

/* y[r, c] = (x[r, c] - m) - logf(s), m = max_c x[r, c], s = sum_c expf(x[r, c] - m)
 * summed in ascending c in fp32 (the textbook log-softmax, written out). */
int bo_log_softmax(const void *x, float *y, int64_t rows, int64_t cols, int dtype)
{
    if (!x || !y || cols < 1 || !valid_dtype(dtype)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float m = load_elem(x, r * cols, dtype);
        for (int64_t c = 1; c < cols; ++c) {
            float v = load_elem(x, r * cols + c, dtype);
            if (v > m) m = v;
        }
        float s = 0.0f;
        for (int64_t c = 0; c < cols; ++c) s = s + expf(load_elem(x, r * cols + c, dtype) - m);
        const float ls = logf(s);
        for (int64_t c = 0; c < cols; ++c) y[r * cols + c] = (load_elem(x, r * cols + c, dtype) - m) - ls;
    }
    return 0;
}

/* y[r] = (sum_c x[r, c], ascending c, fp32) / cols. */
int bo_row_mean(const void *x, float *y, int64_t rows, int64_t cols, int dtype)
{
    if (!x || !y || cols < 1 || !valid_dtype(dtype)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        float s = 0.0f;
        for (int64_t c = 0; c < cols; ++c) s = s + load_elem(x, r * cols + c, dtype);
        y[r] = s / (float)cols;
    }
    return 0;
}

/* Threads the oracle's parallel loops use from now on (n >= 1); returns the
 * count in effect.  Each output's fold is sequential whatever n is. */
int bo_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

int bo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
