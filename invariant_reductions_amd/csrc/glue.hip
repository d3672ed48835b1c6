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

// One thread per (token, head, group of G pairs): G = 8 with 16-byte accesses
// when D / 2 is a multiple of 8, else G = 1.  Pair i of a head rotates
// elements i and i + D/2.
template <int G>
__global__ void rope_kv_kernel(const uint16_t *__restrict__ qkv, uint16_t *__restrict__ q_out,
                               uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
                               const int32_t *__restrict__ kv_len, const float *__restrict__ cos_t,
                               const float *__restrict__ sin_t, int64_t B, int64_t Q, int64_t Lcap,
                               int Hq, int Hkv, int D, int64_t max_pos, int head_major)
{
    // cache element offset of (sequence b, position pos, KV head h)
    auto cache_at = [&](int64_t b, int64_t pos, int64_t h) {
        return (head_major ? (b * Hkv + h) * Lcap + pos : (b * Lcap + pos) * Hkv + h) * (int64_t)D;
    };
    typedef uint16_t vec_t __attribute__((ext_vector_type(G)));
    const int half = D / 2, ng = half / G;
    const int heads = Hq + 2 * Hkv;
    const int64_t per_tok = (int64_t)heads * ng;
    const int64_t n = B * Q * per_tok;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < n; it += (int64_t)gridDim.x * blockDim.x) {
        const int64_t tok = it / per_tok;                          // b * Q + j
        const int rem = (int)(it - tok * per_tok);
        const int hh = rem / ng, i = (rem - hh * ng) * G;
        const int64_t b = tok / Q, j = tok - b * Q;
        // the qkv row is requested before the position is known (it is in bounds either way)
        const uint16_t *src = qkv + tok * (int64_t)heads * D + (int64_t)hh * D;
        const vec_t lo_in = *reinterpret_cast<const vec_t *>(src + i);
        const vec_t hi_in = *reinterpret_cast<const vec_t *>(src + i + half);
        const int64_t pos = (int64_t)kv_len[b] - Q + j;
        if (pos < 0 || pos >= Lcap || pos >= max_pos) continue;   // out-of-range positions write nothing
        if (hh >= Hq + Hkv) {                                      // v: copied to the cache unchanged
            uint16_t *dst = vc + cache_at(b, pos, hh - Hq - Hkv);
            *reinterpret_cast<vec_t *>(dst + i) = lo_in;
            *reinterpret_cast<vec_t *>(dst + i + half) = hi_in;
            continue;
        }
        vec_t lo_out, hi_out;
#pragma unroll
        for (int e = 0; e < G; ++e) {
            const float a = BF16::widen(lo_in[e]), bb = BF16::widen(hi_in[e]);
            const float c = cos_t[pos * half + i + e], sn = sin_t[pos * half + i + e];
            lo_out[e] = BF16::narrow(a * c - bb * sn);
            hi_out[e] = BF16::narrow(bb * c + a * sn);
        }
        uint16_t *dst = hh < Hq ? q_out + tok * (int64_t)Hq * D + (int64_t)hh * D
                                : kc + cache_at(b, pos, hh - Hq);
        *reinterpret_cast<vec_t *>(dst + i) = lo_out;
        *reinterpret_cast<vec_t *>(dst + i + half) = hi_out;
    }
}

// VEC: F % 8 == 0 and 16-byte aligned rows; thread = 8 consecutive outputs.
template <bool VEC>
__global__ void silu_mul_kernel(const uint16_t *__restrict__ gu, uint16_t *__restrict__ out, int64_t rows, int64_t F)
{
    if (VEC) {
        const int64_t fc = F / 8, n = rows * fc;
        for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (int64_t)gridDim.x * blockDim.x) {
            const int64_t r = c / fc, i = (c - r * fc) * 8;
            const uint4 gv = *reinterpret_cast<const uint4 *>(gu + r * 2 * F + i);
            const uint4 uv = *reinterpret_cast<const uint4 *>(gu + r * 2 * F + F + i);
            const uint16_t *g8 = reinterpret_cast<const uint16_t *>(&gv), *u8 = reinterpret_cast<const uint16_t *>(&uv);
            uint16_t o8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = silu_mul1(g8[e], u8[e]);
            *reinterpret_cast<uint4 *>(out + r * F + i) = __builtin_bit_cast(uint4, o8);
        }
    } else {
        const int64_t n = rows * F;
        for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
            const int64_t r = idx / F, i = idx % F;
            out[idx] = silu_mul1(gu[r * 2 * F + i], gu[r * 2 * F + F + i]);
        }
    }
}

// VEC: n % 8 == 0 (pointers are 16-byte aligned by contract); out may alias a or b.
template <bool VEC>
__global__ void add_kernel(const uint16_t *a, const uint16_t *b, uint16_t *out, int64_t n)
{
    if (VEC) {
        for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n / 8; c += (int64_t)gridDim.x * blockDim.x) {
            const uint4 av = reinterpret_cast<const uint4 *>(a)[c], bv = reinterpret_cast<const uint4 *>(b)[c];
            const uint16_t *a8 = reinterpret_cast<const uint16_t *>(&av), *b8 = reinterpret_cast<const uint16_t *>(&bv);
            uint16_t o8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o8[e] = BF16::narrow(BF16::widen(a8[e]) + BF16::widen(b8[e]));
            reinterpret_cast<uint4 *>(out)[c] = __builtin_bit_cast(uint4, o8);
        }
    } else {
        for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x)
            out[idx] = BF16::narrow(BF16::widen(a[idx]) + BF16::widen(b[idx]));
    }
}

__device__ inline bool better(float v, int64_t i, float bv, int64_t bi)
{
    return v > bv || (v == bv && i < bi);
}

constexpr int kArgmaxThreads = 1024;
constexpr int kArgmaxUnroll = 4;           // independent 16-byte loads in flight per thread

__device__ inline void argmax_take(float v, int i, float &bv, int &bi, int none)
{
    if (i != none && (bi == none || better(v, i, bv, bi))) {
        bv = v;
        bi = i;
    }
}

// One workgroup per row.  VEC (cols % 8 == 0): thread t reads the 16-byte
// chunks t, t + 1024, ... of the row, kArgmaxUnroll loads at a time.  The
// winner -- the largest value, lowest index among equals -- is the same for
// any order of comparison, so the wave butterfly and the cross-wave step may
// meet candidates in any order.
template <bool VEC>
__global__ __launch_bounds__(kArgmaxThreads)
void argmax_kernel(const uint16_t *__restrict__ x, int32_t *__restrict__ idx, int64_t rows, int64_t cols,
                   int32_t *__restrict__ ids_next, int32_t *__restrict__ kv_len)
{
    __shared__ float sv[kArgmaxThreads / kWave];
    __shared__ int si[kArgmaxThreads / kWave];
    const int none = (int)cols;                 // sentinel: loses every comparison with a real index
    const uint16_t *xr = x + (int64_t)blockIdx.x * cols;
    float bv = -INFINITY;
    int bi = none;
    if (VEC) {
        const int nch = (int)(cols / 8);
        for (int c0 = threadIdx.x; c0 < nch; c0 += kArgmaxThreads * kArgmaxUnroll) {
            uint4 v[kArgmaxUnroll];
#pragma unroll
            for (int u = 0; u < kArgmaxUnroll; ++u) {
                const int ch = c0 + u * kArgmaxThreads;
                v[u] = ch < nch ? reinterpret_cast<const uint4 *>(xr)[ch] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < kArgmaxUnroll; ++u) {
                const int ch = c0 + u * kArgmaxThreads;
                if (ch >= nch) break;
                const uint16_t *e8 = reinterpret_cast<const uint16_t *>(&v[u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) argmax_take(BF16::widen(e8[e]), ch * 8 + e, bv, bi, none);
            }
        }
    } else {
        for (int c = threadIdx.x; c < (int)cols; c += kArgmaxThreads) argmax_take(BF16::widen(xr[c]), c, bv, bi, none);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, kWave);
        const int oi = __shfl_xor(bi, off, kWave);
        argmax_take(ov, oi, bv, bi, none);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (wave == 0) {
        bv = lane < kArgmaxThreads / kWave ? sv[lane] : -INFINITY;
        bi = lane < kArgmaxThreads / kWave ? si[lane] : none;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            argmax_take(ov, oi, bv, bi, none);
        }
        if (lane == 0) {
            idx[blockIdx.x] = bi;
            // greedy decode bookkeeping: the token is the sequence's next input
            // and its cache grows by one position
            if (ids_next) ids_next[blockIdx.x] = bi;
            if (kv_len) kv_len[blockIdx.x] = kv_len[blockIdx.x] + 1;
        }
    }
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
    launch_kernel(embed_kernel, dim3((unsigned)T), dim3(256), 0, stream, ids, (const uint4 *)table,
                       (uint4 *)out, T, V, H / 8);
    return launch_status();
}

extern "C" bi_status bi_rope_kv_write(const void *qkv, void *q_out, void *kc, void *vc, const int32_t *kv_len,
                                      const float *cos_t, const float *sin_t, int64_t B, int64_t Q, int64_t Lcap,
                                      int32_t Hq, int32_t Hkv, int32_t D, int64_t max_pos, int32_t kv_layout,
                                      hipStream_t stream)
{
    if (!qkv || !q_out || !kc || !vc || !kv_len || !cos_t || !sin_t) return BI_ERR_NULL;
    if (B < 1 || Q < 1 || Lcap < 1 || Hq < 1 || Hkv < 1 || D < 2 || D % 2 || max_pos < 1) return BI_ERR_SHAPE;
    if (kv_layout != 0 && kv_layout != 1) return BI_ERR_SHAPE;
    if (!host_aligned16(qkv) || !host_aligned16(q_out) || !host_aligned16(kc) || !host_aligned16(vc) ||
        !host_aligned16(cos_t) || !host_aligned16(sin_t) || ((uintptr_t)kv_len & 3u))
        return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if ((int64_t)(Hq + 2 * Hkv) * D > (1ll << 31) - 1) return BI_ERR_SHAPE;
    const bool vec = (D / 2) % 8 == 0;
    const int64_t n = B * Q * (Hq + 2 * Hkv) * (vec ? D / 16 : D / 2);
    if (vec)
        launch_kernel(rope_kv_kernel<8>, dim3(grid_for(n, 256)), dim3(256), 0, stream, (const uint16_t *)qkv,
                           (uint16_t *)q_out, (uint16_t *)kc, (uint16_t *)vc, kv_len, cos_t, sin_t, B, Q, Lcap,
                           Hq, Hkv, D, max_pos, kv_layout);
    else
        launch_kernel(rope_kv_kernel<1>, dim3(grid_for(n, 256)), dim3(256), 0, stream, (const uint16_t *)qkv,
                           (uint16_t *)q_out, (uint16_t *)kc, (uint16_t *)vc, kv_len, cos_t, sin_t, B, Q, Lcap,
                           Hq, Hkv, D, max_pos, kv_layout);
    return launch_status();
}

extern "C" bi_status bi_silu_mul(const void *gu, void *out, int64_t rows, int64_t F, hipStream_t stream)
{
    if (!gu || !out) return BI_ERR_NULL;
    if (rows < 1 || F < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(gu) || !host_aligned16(out)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (F % 8 == 0)
        launch_kernel(silu_mul_kernel<true>, dim3(grid_for(rows * F / 8, 256)), dim3(256), 0, stream,
                           (const uint16_t *)gu, (uint16_t *)out, rows, F);
    else
        launch_kernel(silu_mul_kernel<false>, dim3(grid_for(rows * F, 256)), dim3(256), 0, stream,
                           (const uint16_t *)gu, (uint16_t *)out, rows, F);
    return launch_status();
}

extern "C" bi_status bi_add(const void *a, const void *b, void *out, int64_t n, hipStream_t stream)
{
    if (!a || !b || !out) return BI_ERR_NULL;
    if (n < 1) return BI_ERR_SHAPE;
    if (!host_aligned16(a) || !host_aligned16(b) || !host_aligned16(out)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (n % 8 == 0)
        launch_kernel(add_kernel<true>, dim3(grid_for(n / 8, 256)), dim3(256), 0, stream, (const uint16_t *)a,
                           (const uint16_t *)b, (uint16_t *)out, n);
    else
        launch_kernel(add_kernel<false>, dim3(grid_for(n, 256)), dim3(256), 0, stream, (const uint16_t *)a,
                           (const uint16_t *)b, (uint16_t *)out, n);
    return launch_status();
}

static bi_status run_argmax(const void *x, int32_t *idx, int32_t *ids_next, int32_t *kv_len, int64_t rows,
                            int64_t cols, hipStream_t stream)
{
    if (!x || !idx) return BI_ERR_NULL;
    if (rows < 1 || cols < 1 || rows > (1ll << 31) - 1 || cols > (1ll << 31) - 1) return BI_ERR_SHAPE;
    if (!host_aligned16(x) || (((uintptr_t)idx | (uintptr_t)ids_next | (uintptr_t)kv_len) & 3u)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (cols % 8 == 0)
        launch_kernel(argmax_kernel<true>, dim3((unsigned)rows), dim3(kArgmaxThreads), 0, stream,
                           (const uint16_t *)x, idx, rows, cols, ids_next, kv_len);
    else
        launch_kernel(argmax_kernel<false>, dim3((unsigned)rows), dim3(kArgmaxThreads), 0, stream,
                           (const uint16_t *)x, idx, rows, cols, ids_next, kv_len);
    return launch_status();
}

extern "C" bi_status bi_argmax(const void *x, int32_t *idx, int64_t rows, int64_t cols, hipStream_t stream)
{
    return run_argmax(x, idx, nullptr, nullptr, rows, cols, stream);
}

extern "C" bi_status bi_argmax_advance(const void *x, int32_t *idx, int32_t *ids_next, int32_t *kv_len, int64_t rows,
                                       int64_t cols, hipStream_t stream)
{
    if (!ids_next || !kv_len) return BI_ERR_NULL;
    return run_argmax(x, idx, ids_next, kv_len, rows, cols, stream);
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
           " K blocks of 128 (16-bit) / 16 (f32), block b in slot b%8 of 8, each slot summed in block order,"
           " slots added pairwise ((0+1)+(2+3))+((4+5)+(6+7));"
           " qmatmul: dequantize to binary16 in registers, v_mfma_f32_16x16x32_f16, same K slicing,"
           " each dequantized word feeding every row tile of up to 32 rows;"
           " rmsnorm: one wave per row, 16-byte chunk v to lane v%64, per-lane fma fold, xor butterfly 32..1;"
           " sdpa: scores in base-2 units (scale*log2e rounded once), exponentials 2^x by v_exp_f32,"
           " chunks of 256 keys, 4 waves x 64 keys, P as hi+lo 16-bit parts in MFMA (lo first),"
           " chunk partials merged in ranges of 16 chunks (weights 2^(m_c-M_r), ascending), ranges merged"
           " in ascending order (weights 2^(M_r-M)); many short groups: one launch, the merge in the"
           " workgroup; prompts (>= 128 query rows per KV head, <= 8192 keys):"
           " the same tree in one launch, one wave playing the 4 quarters of a chunk;"
           " dense M > 64: the same K tree walked slot by slot, x/W tiles shared through LDS";
}
