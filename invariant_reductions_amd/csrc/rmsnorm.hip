// rmsnorm.hip -- batch-invariant RMSNorm on gfx950.
//
// Source: "Batch-invariant kernels: why temperature-0 decoding is still
// nondeterministic", Case 4 (the sum-of-squares order must not follow the
// batch) and Case 6 (RMSNorm stays data-parallel, one row never split, idle
// compute units accepted at batch 1).
//
// Reduction tree of one row (frozen; depends on H only):
//   * the row is cut into 16-byte chunks (8 bf16/f16 or 4 f32 elements);
//     chunk v belongs to lane v mod 64 of the row's wavefront;
//   * each lane folds x*x of its chunks in ascending chunk order, elements in
//     ascending order, with fused multiply-add in fp32;
//   * the 64 lane sums are combined by a xor butterfly (offsets 32, 16, 8, 4,
//     2, 1); every step adds two equal-shaped partials, so all lanes end with
//     the same bits;
//   * inv = 1 / sqrt(ss / H + eps) with IEEE division and square root;
//     y = (x * inv) * w, each product rounded in fp32, then RNE to the storage
//     type.
// One wavefront owns one row; how many rows share a workgroup or a launch
// does not enter the computation.
#include "common.hpp"

namespace bi {

constexpr int kNormRowsPerBlock = 1;      // free: rows per workgroup (one per wave); one row spreads short batches over more CUs
constexpr int kNormCached = 8;            // free: chunks per lane kept in registers

template <typename S>
__device__ inline void chunk_vals(uint4 v, float *out)
{
    constexpr int E = S::kElemsPer16B;
    const typename S::store_t *p = reinterpret_cast<const typename S::store_t *>(&v);
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = S::widen(p[e]);
}

template <typename S, bool VEC>
__device__ inline void store_chunk(typename S::store_t *row, int64_t k, int64_t limit, const float *vals)
{
    constexpr int E = S::kElemsPer16B;
    typename S::store_t tmp[E];
#pragma unroll
    for (int e = 0; e < E; ++e) tmp[e] = S::narrow(vals[e]);
    if (VEC) {
        if (k < limit) *reinterpret_cast<uint4 *>(row + k) = __builtin_bit_cast(uint4, tmp);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            if (k + e < limit) row[k + e] = tmp[e];
    }
}

__device__ inline float wave_sum_butterfly(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, kWave);
    return v;
}

// Partial sum of squares of chunks [c0, c1) owned by this lane (lane mapping
// as above, relative to c0).
template <typename S, bool VEC>
__device__ inline float lane_sumsq(const typename S::store_t *xr, int64_t H, int64_t c0, int64_t c1, int lane)
{
    constexpr int E = S::kElemsPer16B;
    float ss = 0.0f;
    for (int64_t v = c0 + lane; v < c1; v += kWave) {
        float xv[E];
        chunk_vals<S>(load_chunk<S, VEC>(xr, v * E, H, true), xv);
#pragma unroll
        for (int e = 0; e < E; ++e) ss = __builtin_fmaf(xv[e], xv[e], ss);
    }
    return ss;
}

template <typename S, bool VEC>
__device__ inline void normalize_chunks(const typename S::store_t *xr, const typename S::store_t *w,
                                        typename S::store_t *yr, int64_t H, int64_t c0, int64_t c1,
                                        int lane, float inv)
{
    constexpr int E = S::kElemsPer16B;
    for (int64_t v = c0 + lane; v < c1; v += kWave) {
        float xv[E], wv[E], yv[E];
        chunk_vals<S>(load_chunk<S, VEC>(xr, v * E, H, true), xv);
        chunk_vals<S>(load_chunk<S, VEC>(w, v * E, H, true), wv);
#pragma unroll
        for (int e = 0; e < E; ++e) yv[e] = (xv[e] * inv) * wv[e];
        store_chunk<S, VEC>(yr, v * E, H, yv);
    }
}

// Chunk v of the row as the norm sees it: x itself, or with ADD the residual
// sum RNE(x + r) (the bits bi_add produces), which is also stored to xo.
template <typename S, bool VEC, bool ADD>
__device__ inline uint4 row_chunk(const typename S::store_t *xr, const typename S::store_t *rr,
                                  typename S::store_t *xor_, int64_t v, int64_t H, bool ok)
{
    constexpr int E = S::kElemsPer16B;
    const uint4 a = load_chunk<S, VEC>(xr, v * E, H, ok);
    if constexpr (!ADD) {
        return a;
    } else {
        float av[E], bv[E], sv[E];
        chunk_vals<S>(a, av);
        chunk_vals<S>(load_chunk<S, VEC>(rr, v * E, H, ok), bv);
        typename S::store_t tmp[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
            tmp[e] = S::narrow(av[e] + bv[e]);
            sv[e] = S::widen(tmp[e]);
        }
        if (ok) store_chunk<S, VEC>(xor_, v * E, H, sv);
        return __builtin_bit_cast(uint4, tmp);
    }
}

// CACHED: the row's chunks stay in registers between the two phases
// (H <= 64 * kNormCached * E); otherwise the second phase re-reads the row
// (with ADD, the sums this lane stored in the first phase).
// ADD: the row is RNE(x + r), written to xo (which may alias x), and then
// normalized -- the residual add of a pre-norm block fused with its norm.
// GATHER (cached, no ADD): row t is row ids[t] of the table x of V rows (a
// zero row for an id outside [0, V)), written to xo as bi_embed writes it,
// then normalized -- the embedding lookup fused with the first norm.
template <typename S, bool VEC, bool CACHED, bool ADD, bool GATHER = false>
__global__ __launch_bounds__(kNormRowsPerBlock * kWave)
void rmsnorm_kernel(const typename S::store_t *x, const typename S::store_t *__restrict__ r,
                    typename S::store_t *xo, const typename S::store_t *__restrict__ w,
                    typename S::store_t *__restrict__ y, int64_t rows, int64_t H, float eps,
                    const int32_t *__restrict__ ids, int64_t V)
{
    static_assert(!GATHER || (VEC && CACHED && !ADD), "the gather form is the cached plain norm, 16-byte rows");
    constexpr int E = S::kElemsPer16B;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kNormRowsPerBlock + wave_id();
    if (row >= rows) return;
    int32_t id = 0;
    bool idok = true;
    if constexpr (GATHER) {
        id = ids[row];
        idok = id >= 0 && id < V;
    }
    const typename S::store_t *xr = GATHER ? x + (int64_t)(idok ? id : 0) * H : x + row * H;
    const typename S::store_t *rr = ADD ? r + row * H : nullptr;
    typename S::store_t *xor_ = ADD ? xo + row * H : nullptr;
    typename S::store_t *yr = y + row * H;
    const int64_t nch = cdiv(H, E);

    if (CACHED) {
        uint4 cache[kNormCached], wc[kNormCached];
        float ss = 0.0f;
        // the weight chunks are requested with the row, ahead of the sum
#pragma unroll
        for (int i = 0; i < kNormCached; ++i) {
            const int64_t v = lane + (int64_t)i * kWave;
            wc[i] = load_chunk<S, VEC>(w, v * E, H, v < nch);
        }
        if constexpr (ADD) {
            // every load of x and r is issued before the first store to xo: xo
            // may alias x, so a store would otherwise hold back the loads after it
            uint4 ra[kNormCached];
#pragma unroll
            for (int i = 0; i < kNormCached; ++i) {
                const int64_t v = lane + (int64_t)i * kWave;
                cache[i] = load_chunk<S, VEC>(xr, v * E, H, v < nch);
                ra[i] = load_chunk<S, VEC>(rr, v * E, H, v < nch);
            }
#pragma unroll
            for (int i = 0; i < kNormCached; ++i) {
                const int64_t v = lane + (int64_t)i * kWave;
                float av[E], bv[E], sv[E];
                chunk_vals<S>(cache[i], av);
                chunk_vals<S>(ra[i], bv);
                typename S::store_t tmp[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    tmp[e] = S::narrow(av[e] + bv[e]);
                    sv[e] = S::widen(tmp[e]);
                }
                if (v < nch) store_chunk<S, VEC>(xor_, v * E, H, sv);
                cache[i] = __builtin_bit_cast(uint4, tmp);
#pragma unroll
                for (int e = 0; e < E; ++e) ss = __builtin_fmaf(sv[e], sv[e], ss);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kNormCached; ++i) {
                const int64_t v = lane + (int64_t)i * kWave;
                cache[i] = row_chunk<S, VEC, ADD>(xr, rr, xor_, v, H, v < nch && idok);
                float xv[E];
                chunk_vals<S>(cache[i], xv);
#pragma unroll
                for (int e = 0; e < E; ++e) ss = __builtin_fmaf(xv[e], xv[e], ss);
            }
            if constexpr (GATHER) {
#pragma unroll
                for (int i = 0; i < kNormCached; ++i) {
                    const int64_t v = lane + (int64_t)i * kWave;
                    if (v < nch) *reinterpret_cast<uint4 *>(xo + row * H + v * E) = cache[i];
                }
            }
        }
        ss = wave_sum_butterfly(ss);
        const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
        for (int i = 0; i < kNormCached; ++i) {
            const int64_t v = lane + (int64_t)i * kWave;
            if (v >= nch) break;
            float xv[E], wv[E], yv[E];
            chunk_vals<S>(cache[i], xv);
            chunk_vals<S>(wc[i], wv);
#pragma unroll
            for (int e = 0; e < E; ++e) yv[e] = (xv[e] * inv) * wv[e];
            store_chunk<S, VEC>(yr, v * E, H, yv);
        }
    } else {
        float ss = 0.0f;
        for (int64_t v = lane; v < nch; v += kWave) {
            float xv[E];
            chunk_vals<S>(row_chunk<S, VEC, ADD>(xr, rr, xor_, v, H, true), xv);
#pragma unroll
            for (int e = 0; e < E; ++e) ss = __builtin_fmaf(xv[e], xv[e], ss);
        }
        ss = wave_sum_butterfly(ss);
        const float inv = 1.0f / sqrtf(ss / (float)H + eps);
        normalize_chunks<S, VEC>(ADD ? xor_ : xr, w, yr, H, 0, nch, lane, inv);
    }
}

// ---- comparison variant: one row split across `splits` workgroups -------------
template <typename S, bool VEC>
__global__ __launch_bounds__(kWave)
void rmsnorm_split_partial(const typename S::store_t *__restrict__ x, float *__restrict__ part,
                           int64_t rows, int64_t H, int splits)
{
    constexpr int E = S::kElemsPer16B;
    const int64_t row = blockIdx.x;
    const int s = blockIdx.y;
    const int64_t nch = cdiv(H, E);
    const int64_t c0 = (int64_t)s * nch / splits, c1 = (int64_t)(s + 1) * nch / splits;
    float ss = wave_sum_butterfly(lane_sumsq<S, VEC>(x + row * H, H, c0, c1, threadIdx.x));
    if (threadIdx.x == 0) part[row * splits + s] = ss;
}

template <typename S, bool VEC>
__global__ __launch_bounds__(kNormRowsPerBlock * kWave)
void rmsnorm_split_finish(const typename S::store_t *__restrict__ x, const typename S::store_t *__restrict__ w,
                          typename S::store_t *__restrict__ y, const float *__restrict__ part,
                          int64_t rows, int64_t H, float eps, int splits)
{
    constexpr int E = S::kElemsPer16B;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kNormRowsPerBlock + wave_id();
    if (row >= rows) return;
    float ss = part[row * splits];
    for (int s = 1; s < splits; ++s) ss = ss + part[row * splits + s];
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
    normalize_chunks<S, VEC>(x + row * H, w, y + row * H, H, 0, cdiv(H, E), lane, inv);
}

template <typename S, bool ADD>
static void launch_rmsnorm(const void *x, const void *r, void *xo, const void *w, void *y, int64_t rows, int64_t H,
                           float eps, hipStream_t st)
{
    using T = typename S::store_t;
    constexpr int E = S::kElemsPer16B;
    const bool vec = (H % E) == 0 && host_aligned16(x) && host_aligned16(w) && host_aligned16(y) &&
                     (!ADD || (host_aligned16(r) && host_aligned16(xo)));
    const bool cached = cdiv(cdiv(H, E), kWave) <= kNormCached;
    dim3 grid((unsigned)cdiv(rows, kNormRowsPerBlock)), block(kNormRowsPerBlock * kWave);
    const T *xt = (const T *)x, *rt = (const T *)r, *wt = (const T *)w;
    T *xot = (T *)xo, *yt = (T *)y;
    const int32_t *noids = nullptr;                  // no gather
    if (vec && cached)
        launch_kernel((rmsnorm_kernel<S, true, true, ADD>), grid, block, 0, st, xt, rt, xot, wt, yt, rows, H, eps, noids,
                      (int64_t)0);
    else if (vec)
        launch_kernel((rmsnorm_kernel<S, true, false, ADD>), grid, block, 0, st, xt, rt, xot, wt, yt, rows, H, eps, noids,
                      (int64_t)0);
    else if (cached)
        launch_kernel((rmsnorm_kernel<S, false, true, ADD>), grid, block, 0, st, xt, rt, xot, wt, yt, rows, H, eps, noids,
                      (int64_t)0);
    else
        launch_kernel((rmsnorm_kernel<S, false, false, ADD>), grid, block, 0, st, xt, rt, xot, wt, yt, rows, H, eps,
                      noids, (int64_t)0);
}

template <typename S>
static void launch_rmsnorm_split(const void *x, const void *w, void *y, float *part, int64_t rows, int64_t H,
                                 float eps, int splits, hipStream_t st)
{
    using T = typename S::store_t;
    constexpr int E = S::kElemsPer16B;
    if ((H % E) == 0 && host_aligned16(x) && host_aligned16(w) && host_aligned16(y)) {
        launch_kernel((rmsnorm_split_partial<S, true>), dim3((unsigned)rows, (unsigned)splits), dim3(kWave), 0, st, (const T *)x, part, rows, H, splits);
        launch_kernel((rmsnorm_split_finish<S, true>), dim3((unsigned)cdiv(rows, kNormRowsPerBlock)), dim3(kNormRowsPerBlock * kWave), 0, st, (const T *)x, (const T *)w, (T *)y, part, rows, H, eps, splits);
    } else {
        launch_kernel((rmsnorm_split_partial<S, false>), dim3((unsigned)rows, (unsigned)splits), dim3(kWave), 0, st, (const T *)x, part, rows, H, splits);
        launch_kernel((rmsnorm_split_finish<S, false>), dim3((unsigned)cdiv(rows, kNormRowsPerBlock)), dim3(kNormRowsPerBlock * kWave), 0, st, (const T *)x, (const T *)w, (T *)y, part, rows, H, eps, splits);
    }
}

static bi_status check_norm(const void *x, const void *w, const void *y, int64_t rows, int64_t H, float eps,
                            int32_t dtype)
{
    if (!x || !w || !y) return BI_ERR_NULL;
    if (rows < 1 || H < 1 || rows > (1ll << 31) - 1 || H > (1ll << 31) || !(eps >= 0.0f)) return BI_ERR_SHAPE;
    if (dtype != BI_BF16 && dtype != BI_F16 && dtype != BI_F32) return BI_ERR_DTYPE;
    const size_t esz = dtype == BI_F32 ? 4 : 2;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & (esz - 1)) return BI_ERR_ALIGN;
    return BI_OK;
}

}  // namespace bi

using namespace bi;

extern "C" bi_status bi_rmsnorm(const void *x, const void *w, void *y, int64_t rows, int64_t H, float eps,
                                int32_t dtype, hipStream_t stream)
{
    bi_status s = check_norm(x, w, y, rows, H, eps, dtype);
    if (s != BI_OK) return s;
    (void)hipGetLastError();
    if (dtype == BI_BF16) launch_rmsnorm<BF16, false>(x, nullptr, nullptr, w, y, rows, H, eps, stream);
    else if (dtype == BI_F16) launch_rmsnorm<F16, false>(x, nullptr, nullptr, w, y, rows, H, eps, stream);
    else launch_rmsnorm<F32, false>(x, nullptr, nullptr, w, y, rows, H, eps, stream);
    return launch_status();
}

extern "C" bi_status bi_add_rmsnorm(const void *x, const void *r, void *x_out, const void *w, void *y,
                                    int64_t rows, int64_t H, float eps, int32_t dtype, hipStream_t stream)
{
    bi_status s = check_norm(x, w, y, rows, H, eps, dtype);
    if (s != BI_OK) return s;
    if (!r || !x_out) return BI_ERR_NULL;
    const size_t esz = dtype == BI_F32 ? 4 : 2;
    if (((uintptr_t)r | (uintptr_t)x_out) & (esz - 1)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (dtype == BI_BF16) launch_rmsnorm<BF16, true>(x, r, x_out, w, y, rows, H, eps, stream);
    else if (dtype == BI_F16) launch_rmsnorm<F16, true>(x, r, x_out, w, y, rows, H, eps, stream);
    else launch_rmsnorm<F32, true>(x, r, x_out, w, y, rows, H, eps, stream);
    return launch_status();
}

extern "C" bi_status bi_embed_rmsnorm(const int32_t *ids, const void *table, void *x_out, const void *w, void *y,
                                      int64_t T, int64_t V, int64_t H, float eps, int32_t dtype, hipStream_t stream)
{
    bi_status s = check_norm(table, w, y, T, H, eps, dtype);
    if (s != BI_OK) return s;
    if (!ids || !x_out) return BI_ERR_NULL;
    if (dtype == BI_F32) return BI_ERR_DTYPE;             // the embedding is a 16-bit table
    if (V < 1 || V > (1ll << 31) - 1) return BI_ERR_SHAPE;
    if (((uintptr_t)x_out & 1u) || ((uintptr_t)ids & 3u)) return BI_ERR_ALIGN;
    const bool fused = H % 8 == 0 && cdiv(H / 8, kWave) <= kNormCached && host_aligned16(table) &&
                       host_aligned16(w) && host_aligned16(y) && host_aligned16(x_out);
    (void)hipGetLastError();
    if (fused) {
        const dim3 grid((unsigned)cdiv(T, kNormRowsPerBlock)), block(kNormRowsPerBlock * kWave);
        if (dtype == BI_BF16)
            launch_kernel((rmsnorm_kernel<BF16, true, true, false, true>), grid, block, 0, stream,
                          (const uint16_t *)table, (const uint16_t *)nullptr, (uint16_t *)x_out, (const uint16_t *)w,
                          (uint16_t *)y, T, H, eps, ids, V);
        else
            launch_kernel((rmsnorm_kernel<F16, true, true, false, true>), grid, block, 0, stream,
                          (const uint16_t *)table, (const uint16_t *)nullptr, (uint16_t *)x_out, (const uint16_t *)w,
                          (uint16_t *)y, T, H, eps, ids, V);
        return launch_status();
    }
    // other shapes: the lookup, then the norm (the same bits; bi_embed's own
    // requirements apply)
    s = bi_embed(ids, table, x_out, T, V, H, stream);
    if (s != BI_OK) return s;
    return bi_rmsnorm(x_out, w, y, T, H, eps, dtype, stream);
}

extern "C" size_t bi_rmsnorm_split_workspace_bytes(int64_t rows, int32_t splits)
{
    if (rows < 1 || splits < 1) return 0;
    return (size_t)rows * (size_t)splits * sizeof(float);
}

extern "C" bi_status bi_rmsnorm_split(const void *x, const void *w, void *y, int64_t rows, int64_t H, float eps,
                                      int32_t dtype, int32_t splits, void *ws, size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_norm(x, w, y, rows, H, eps, dtype);
    if (s != BI_OK) return s;
    if (splits < 1 || splits > 65535) return BI_ERR_SHAPE;
    if (!ws) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    if (ws_bytes < bi_rmsnorm_split_workspace_bytes(rows, splits)) return BI_ERR_WORKSPACE;
    (void)hipGetLastError();
    float *part = (float *)ws;
    if (dtype == BI_BF16) launch_rmsnorm_split<BF16>(x, w, y, part, rows, H, eps, splits, stream);
    else if (dtype == BI_F16) launch_rmsnorm_split<F16>(x, w, y, part, rows, H, eps, splits, stream);
    else launch_rmsnorm_split<F32>(x, w, y, part, rows, H, eps, splits, stream);
    return launch_status();
}
