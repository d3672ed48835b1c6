// glue.hip -- pointwise pieces of a Llama-style decoder (bf16), plus the
// library's status and build-info strings.
//
// Source: "Batch-invariant kernels: why temperature-0 decoding is still
// nondeterministic", Mental model (pointwise ops are batch-invariant; only the
// three reductions need care) and Case 6 (the KV cache is updated before the
// attention kernel runs, so cached and new tokens share one layout).
// Every output element here depends only on its own inputs; argmax is a
// max-with-lowest-index selection, whose result does not depend on the order
// in which candidates are compared.
#include "common.hpp"

namespace bi {

__global__ void embed_kernel(const int32_t *__restrict__ ids, const uint4 *__restrict__ table,
                             uint4 *__restrict__ out, int64_t T, int64_t V, int64_t H16)
{
    const int64_t t = blockIdx.x;
    const int32_t id = ids[t];
    const bool ok = id >= 0 && id < V;
    for (int64_t i = threadIdx.x; i < H16; i += blockDim.x)
        out[t * H16 + i] = ok ? table[(int64_t)id * H16 + i] : make_uint4(0, 0, 0, 0);
}

// One thread per (token, head, pair i < D/2).
__global__ void rope_kv_kernel(const uint16_t *__restrict__ qkv, uint16_t *__restrict__ q_out,
                               uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
                               const int32_t *__restrict__ kv_len, const float *__restrict__ cos_t,
                               const float *__restrict__ sin_t, int64_t B, int64_t Q, int64_t Lcap,
                               int Hq, int Hkv, int D, int64_t max_pos)
{
    const int half = D / 2;
    const int heads = Hq + 2 * Hkv;
    const int64_t n = B * Q * heads * half;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int i = (int)(idx % half);
        const int hh = (int)((idx / half) % heads);
        const int64_t tok = idx / ((int64_t)half * heads);       // b * Q + j
        const int64_t b = tok / Q, j = tok % Q;
        const int64_t pos = (int64_t)kv_len[b] - Q + j;
        if (pos < 0 || pos >= Lcap || pos >= max_pos) continue;   // out-of-range positions write nothing
        const uint16_t *src = qkv + tok * (int64_t)heads * D + (int64_t)hh * D;
        const float a = BF16::widen(src[i]), bb = BF16::widen(src[i + half]);
        if (hh >= Hq + Hkv) {                                      // v: copied to the cache unchanged
            uint16_t *dst = vc + ((b * Lcap + pos) * Hkv + (hh - Hq - Hkv)) * (int64_t)D;
            dst[i] = src[i];
            dst[i + half] = src[i + half];
            continue;
        }
        const float c = cos_t[pos * half + i], s = sin_t[pos * half + i];
        const float lo = a * c - bb * s;
        const float hi = bb * c + a * s;
        uint16_t *dst = hh < Hq ? q_out + tok * (int64_t)Hq * D + (int64_t)hh * D
                                : kc + ((b * Lcap + pos) * Hkv + (hh - Hq)) * (int64_t)D;
        dst[i] = BF16::narrow(lo);
        dst[i + half] = BF16::narrow(hi);
    }
}

__global__ void silu_mul_kernel(const uint16_t *__restrict__ gu, uint16_t *__restrict__ out, int64_t rows, int64_t F)
{
    const int64_t n = rows * F;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / F, i = idx % F;
        const float g = BF16::widen(gu[r * 2 * F + i]);
        const float u = BF16::widen(gu[r * 2 * F + F + i]);
        const float sg = g / (1.0f + expf(-g));
        out[idx] = BF16::narrow(sg * u);
    }
}

__global__ void add_kernel(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t n)
{
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x)
        out[idx] = BF16::narrow(BF16::widen(a[idx]) + BF16::widen(b[idx]));
}

__device__ inline bool better(float v, int64_t i, float bv, int64_t bi)
{
    return v > bv || (v == bv && i < bi);
}

constexpr int kArgmaxThreads = 256;

__global__ __launch_bounds__(kArgmaxThreads)
void argmax_kernel(const uint16_t *__restrict__ x, int32_t *__restrict__ idx, int64_t rows, int64_t cols)
{
    __shared__ float sv[kArgmaxThreads];
    __shared__ int64_t si[kArgmaxThreads];
    const int64_t r = blockIdx.x;
    float bv = -INFINITY;
    int64_t bi = cols;                          // sentinel: loses every comparison with a real index
    for (int64_t cc = threadIdx.x; cc < cols; cc += kArgmaxThreads) {
        const float v = BF16::widen(x[r * cols + cc]);
        if (bi == cols || better(v, cc, bv, bi)) { bv = v; bi = cc; }
    }
    sv[threadIdx.x] = bv;
    si[threadIdx.x] = bi;
    __syncthreads();
    for (int off = kArgmaxThreads / 2; off > 0; off >>= 1) {
        if (threadIdx.x < off) {
            const float v = sv[threadIdx.x + off];
            const int64_t i = si[threadIdx.x + off];
            if (i < cols && (si[threadIdx.x] == cols || better(v, i, sv[threadIdx.x], si[threadIdx.x]))) {
                sv[threadIdx.x] = v;
                si[threadIdx.x] = i;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) idx[r] = (int32_t)si[0];
}

inline unsigned grid_for(int64_t n, int threads)
{
    const int64_t g = cdiv(n, threads);
    return (unsigned)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

}  // namespace bi

using namespace bi;

extern "C" bi_status bi_embed(const int32_t *ids, const void *table, void *out, int64_t T, int64_t V, int64_t H,
                              hipStream_t stream)
{
    if (!ids || !table || !out) return BI_ERR_NULL;
    if (T < 1 || V < 1 || H < 1 || H % 8 || T > (1ll << 31) - 1) return BI_ERR_SHAPE;
    if (!host_aligned16(table) || !host_aligned16(out) || ((uintptr_t)ids & 3u)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)T), dim3(256), 0, stream, ids, (const uint4 *)table,
                       (uint4 *)out, T, V, H / 8);
    return launch_status();
}

extern "C" bi_status bi_rope_kv_write(const void *qkv, void *q_out, void *kc, void *vc, const int32_t *kv_len,
                                      const float *cos_t, const float *sin_t, int64_t B, int64_t Q, int64_t Lcap,
                                      int32_t Hq, int32_t Hkv, int32_t D, int64_t max_pos, hipStream_t stream)
{
    if (!qkv || !q_out || !kc || !vc || !kv_len || !cos_t || !sin_t) return BI_ERR_NULL;
    if (B < 1 || Q < 1 || Lcap < 1 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 || max_pos < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(qkv) || !host_aligned16(q_out) || !host_aligned16(kc) || !host_aligned16(vc) ||
        !host_aligned16(cos_t) || !host_aligned16(sin_t) || ((uintptr_t)kv_len & 3u))
        return BI_ERR_ALIGN;
    (void)hipGetLastError();
    const int64_t n = B * Q * (Hq + 2 * Hkv) * (D / 2);
    hipLaunchKernelGGL(rope_kv_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, (const uint16_t *)qkv,
                       (uint16_t *)q_out, (uint16_t *)kc, (uint16_t *)vc, kv_len, cos_t, sin_t, B, Q, Lcap,
                       Hq, Hkv, D, max_pos);
    return launch_status();
}

extern "C" bi_status bi_silu_mul(const void *gu, void *out, int64_t rows, int64_t F, hipStream_t stream)
{
    if (!gu || !out) return BI_ERR_NULL;
    if (rows < 1 || F < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(gu) || !host_aligned16(out)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    hipLaunchKernelGGL(silu_mul_kernel, dim3(grid_for(rows * F, 256)), dim3(256), 0, stream,
                       (const uint16_t *)gu, (uint16_t *)out, rows, F);
    return launch_status();
}

extern "C" bi_status bi_add(const void *a, const void *b, void *out, int64_t n, hipStream_t stream)
{
    if (!a || !b || !out) return BI_ERR_NULL;
    if (n < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(a) || !host_aligned16(b) || !host_aligned16(out)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    hipLaunchKernelGGL(add_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, (const uint16_t *)a,
                       (const uint16_t *)b, (uint16_t *)out, n);
    return launch_status();
}

extern "C" bi_status bi_argmax(const void *x, int32_t *idx, int64_t rows, int64_t cols, hipStream_t stream)
{
    if (!x || !idx) return BI_ERR_NULL;
    if (rows < 1 || cols < 1 || rows > (1ll << 31) - 1 || cols > (1ll << 31) - 1) return BI_ERR_SHAPE;
    if (!host_aligned16(x) || ((uintptr_t)idx & 3u)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)rows), dim3(kArgmaxThreads), 0, stream,
                       (const uint16_t *)x, idx, rows, cols);
    return launch_status();
}

extern "C" const char *bi_status_str(int32_t status)
{
    switch (status) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE: a dimension is out of range or inconsistent";
    case BI_ERR_DTYPE: return "BI_ERR_DTYPE: unsupported data type";
    case BI_ERR_GROUP: return "BI_ERR_GROUP: illegal quantization mode, group size or bit width for this shape";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN: a base pointer is not 16-byte aligned";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE: workspace missing or too small";
    case BI_ERR_LAUNCH: return "BI_ERR_LAUNCH: the HIP runtime rejected a launch";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: not implemented in this build";
    default: return "unknown bi_status";
    }
}

extern "C" const char *bi_build_info(void)
{
    return "libbi gfx950;"
           " matmul: v_mfma_f32_16x16x32_bf16/f16 and v_mfma_f32_16x16x4_f32 for every M,"
           " K blocks of 128 (16-bit) / 16 (f32), block b owned by wave b%8 of 8, wave partials added in order;"
           " qmatmul: dequantize to binary16 in registers, v_mfma_f32_16x16x32_f16, same K slicing;"
           " rmsnorm: one wave per row, 16-byte chunk v to lane v%64, per-lane fma fold, xor butterfly 32..1;"
           " sdpa: chunks of 256 keys, 4 waves x 64 keys, bf16 P in MFMA, pass-2 weights exp(m_c-M) summed in chunk order";
}
