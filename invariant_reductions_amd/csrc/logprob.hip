// logprob.hip -- batch-invariant row log-softmax, token log-probabilities and
// row mean on gfx950.
//
// Sources: "Batch-invariant kernels: why temperature-0 decoding is still
// nondeterministic" (The boring rule, item 1: one reduction strategy at every
// batch size; The trap: a sampler's and a trainer's log-probabilities must
// agree bit for bit for on-policy RL; Sources: the companion library's mean
// and log-softmax overrides).
//
// Reduction tree of one row (frozen; depends on cols only):
//   chunk k = elements [8k, 8k + 8) of the row (the last may be short); thread
//   t of the row's 1024-thread workgroup owns chunks t, t + 1024, ... in
//   ascending order, elements ascending inside a chunk.
//   max : exact (order-free).
//   sum : per thread a sequential fp32 fold over its elements of
//         expf(x - max) (log-softmax) or of x (mean); then in each wave a xor
//         butterfly (32, 16, 8, 4, 2, 1); then the 16 wave sums in wave order.
//   log-softmax y = (x - max) - logf(sum); a token's log-probability is the
//   same expression at its column; mean = sum / cols.
// A row is one workgroup and no other row enters it, so the number of rows
// and a row's place among them leave its bits unchanged.  Whether a chunk is
// read as one 16-byte load or element by element, once or once per pass,
// changes no sum.
#include "common.hpp"

#include <cmath>

namespace bi {

constexpr int kLsThreads = 1024;
constexpr int kLsWaves = kLsThreads / kWave;
enum RowOp { ROW_LOG_SOFTMAX = 0, ROW_TOKEN_LOGPROB = 1, ROW_MEAN = 2 };

template <typename S>
__device__ inline int row_chunk8(const typename S::store_t *xr, int64_t k, int64_t cols, bool vec, float (&v)[8])
{
    const int64_t c0 = k * 8;
    const int n = cols - c0 < 8 ? (int)(cols - c0) : 8;
    if constexpr (sizeof(typename S::store_t) == 2) {
        if (vec && n == 8) {
            const uint4 u = *reinterpret_cast<const uint4 *>(xr + c0);
            const uint16_t *h = reinterpret_cast<const uint16_t *>(&u);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = S::widen(h[e]);
            return 8;
        }
    } else {
        if (vec && n == 8) {
            const float4 a = *reinterpret_cast<const float4 *>(xr + c0), b = *reinterpret_cast<const float4 *>(xr + c0 + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            return 8;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < n ? S::widen(xr[c0 + e]) : 0.0f;
    return n;
}

// NC > 0: the row fits in NC chunks per thread (cols <= 8 * 1024 * NC) and is
// read from memory once, kept in registers for the later passes; NC == 0:
// every pass re-reads the row.  Either way each value enters the same fold in
// the same place.
template <typename S, int OP, int NC>
__global__ __launch_bounds__(kLsThreads)
void row_reduce_kernel(const typename S::store_t *__restrict__ x, float *__restrict__ y,
                       const int32_t *__restrict__ ids, int64_t cols, int vec)
{
    __shared__ float part[kLsWaves];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t r = blockIdx.x;
    const typename S::store_t *xr = x + r * cols;
    const int64_t nch = (cols + 7) / 8;
    float cache[NC > 0 ? NC : 1][8];
    int ncache[NC > 0 ? NC : 1];
    if constexpr (NC > 0) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int64_t k = t + (int64_t)i * kLsThreads;
            ncache[i] = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) cache[i][e] = 0.0f;
            if (k < nch) ncache[i] = row_chunk8<S>(xr, k, cols, vec != 0, cache[i]);
        }
    }
    // f(k, n, v) for this thread's chunks k = t, t + 1024, ... in ascending order
    auto visit = [&](auto &&f) {
        if constexpr (NC > 0) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int64_t k = t + (int64_t)i * kLsThreads;
                if (k < nch) f(k, ncache[i], cache[i]);
            }
        } else {
            for (int64_t k = t; k < nch; k += kLsThreads) {
                float v[8];
                const int n = row_chunk8<S>(xr, k, cols, vec != 0, v);
                f(k, n, v);
            }
        }
    };

    float m = -INFINITY;
    if constexpr (OP != ROW_MEAN) {
        visit([&](int64_t, int n, const float (&v)[8]) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < n) m = fmaxf(m, v[e]);
        });
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
        if (lane == 0) part[wave] = m;
        __syncthreads();
        m = part[0];
#pragma unroll
        for (int w = 1; w < kLsWaves; ++w) m = fmaxf(m, part[w]);
        __syncthreads();                            // part is reused for the sums
    }

    float s = 0.0f;
    visit([&](int64_t, int n, const float (&v)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e < n) s = s + (OP == ROW_MEAN ? v[e] : expf(v[e] - m));
    });
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s = s + __shfl_xor(s, off, kWave);
    if (lane == 0) part[wave] = s;
    __syncthreads();
    s = part[0];
#pragma unroll
    for (int w = 1; w < kLsWaves; ++w) s = s + part[w];

    if constexpr (OP == ROW_MEAN) {
        if (t == 0) y[r] = s / (float)cols;
        return;
    }
    const float ls = logf(s);
    if constexpr (OP == ROW_TOKEN_LOGPROB) {
        if (t == 0) {
            const int64_t id = ids[r];
            y[r] = (id >= 0 && id < cols) ? (S::widen(xr[id]) - m) - ls : __uint_as_float(0x7fc00000u);
        }
        return;
    }
    float *yr = y + r * cols;
    visit([&](int64_t k, int n, const float (&v)[8]) {
        if (vec && n == 8) {
            *reinterpret_cast<float4 *>(yr + k * 8) = make_float4((v[0] - m) - ls, (v[1] - m) - ls, (v[2] - m) - ls, (v[3] - m) - ls);
            *reinterpret_cast<float4 *>(yr + k * 8 + 4) = make_float4((v[4] - m) - ls, (v[5] - m) - ls, (v[6] - m) - ls, (v[7] - m) - ls);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e < n) yr[k * 8 + e] = (v[e] - m) - ls;
        }
    });
}

template <typename S, int OP>
static void launch_row(const void *x, float *y, const int32_t *ids, int64_t rows, int64_t cols, hipStream_t st)
{
    // 16-byte loads (and stores) need every row to start on a 16-byte boundary
    const int vec = (cols % 8 == 0) && host_aligned16(x) && (OP != ROW_LOG_SOFTMAX || host_aligned16(y));
    const int64_t nch = (cols + 7) / 8;
    if (nch <= (int64_t)kLsThreads * 4)
        launch_kernel((row_reduce_kernel<S, OP, 4>), dim3((unsigned)rows), dim3(kLsThreads), 0, st,
                      (const typename S::store_t *)x, y, ids, cols, vec);
    else if (nch <= (int64_t)kLsThreads * 8)
        launch_kernel((row_reduce_kernel<S, OP, 8>), dim3((unsigned)rows), dim3(kLsThreads), 0, st,
                      (const typename S::store_t *)x, y, ids, cols, vec);
    else
        launch_kernel((row_reduce_kernel<S, OP, 0>), dim3((unsigned)rows), dim3(kLsThreads), 0, st,
                      (const typename S::store_t *)x, y, ids, cols, vec);
}

template <int OP>
static bi_status run_row(const void *x, float *y, const int32_t *ids, int64_t rows, int64_t cols, int32_t dtype,
                         hipStream_t st)
{
    if (!x || !y || (OP == ROW_TOKEN_LOGPROB && !ids)) return BI_ERR_NULL;
    if (rows < 1 || cols < 1 || rows > (1ll << 31) - 1 || cols > (1ll << 40)) return BI_ERR_SHAPE;
    if (dtype != BI_BF16 && dtype != BI_F16 && dtype != BI_F32) return BI_ERR_DTYPE;
    const size_t esz = dtype == BI_F32 ? 4 : 2;
    if (((uintptr_t)x & (esz - 1)) || ((uintptr_t)y & 3u) || ((uintptr_t)ids & 3u)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (dtype == BI_BF16) launch_row<BF16, OP>(x, y, ids, rows, cols, st);
    else if (dtype == BI_F16) launch_row<F16, OP>(x, y, ids, rows, cols, st);
    else launch_row<F32, OP>(x, y, ids, rows, cols, st);
    return launch_status();
}

}  // namespace bi

using namespace bi;

extern "C" bi_status bi_log_softmax(const void *x, float *y, int64_t rows, int64_t cols, int32_t dtype,
                                    hipStream_t stream)
{
    return run_row<ROW_LOG_SOFTMAX>(x, y, nullptr, rows, cols, dtype, stream);
}

extern "C" bi_status bi_token_logprob(const void *x, const int32_t *ids, float *out, int64_t rows, int64_t cols,
                                      int32_t dtype, hipStream_t stream)
{
    return run_row<ROW_TOKEN_LOGPROB>(x, out, ids, rows, cols, dtype, stream);
}

extern "C" bi_status bi_row_mean(const void *x, float *y, int64_t rows, int64_t cols, int32_t dtype,
                                 hipStream_t stream)
{
    return run_row<ROW_MEAN>(x, y, nullptr, rows, cols, dtype, stream);
}
