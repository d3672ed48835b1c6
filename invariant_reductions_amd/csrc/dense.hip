// dense.hip -- batch-invariant dense matmul y = x . W^T on gfx950 MFMA.
//
// Sources: "Fix/speculative shape invariance" (Problem: a single row and a
// short matrix selected GEMV / gemv_wide / GEMM and reduced differently;
// Changes: every row reduced by one canonical kernel and order, for both
// weight orientations); "Batch-invariant kernels: why temperature-0 decoding
// is still nondeterministic" (Case 3: the K tiling must not follow the batch;
// Case 6: one compiled configuration for every shape, no split-K, and no
// smaller instruction at small M).
//
// Reduction tree of one output y[m,n] (frozen; depends on K only):
//   * K is cut into blocks of KB elements (128 for bf16/f16, 16 for f32);
//     block b is reduced by wave (b mod P) of the workgroup, P = kDenseWaves.
//   * Inside a block, four MFMA steps (v_mfma_f32_16x16x32_{bf16,f16} or
//     v_mfma_f32_16x16x4_f32) consume the block; lane group g (lanes 16g..16g+15)
//     supplies the contiguous elements [g*KB/4, (g+1)*KB/4) of the block, step s
//     the s-th quarter of them.  A wave accumulates its blocks in ascending
//     order in the MFMA accumulator.
//   * The P wave partials are added in wave order 0..P-1 in fp32, then rounded
//     to the output type (RNE).
// Row m of the output only ever meets row m of x inside an MFMA, so the M-tile
// it falls in, the other rows of that tile, the number of M-tiles and the
// N-tile width (all chosen from the shape) leave its bits unchanged.  M = 1 is
// the same MFMA with fifteen zero rows.
#include "common.hpp"

namespace bi {

constexpr int kDenseWaves = 8;   // P: K-block owners per output tile (frozen)

template <typename S> struct DenseMfma;

template <> struct DenseMfma<BF16> {
    static constexpr int CPB = 4;                 // 16-byte chunks per lane per block
    __device__ static f32x4 step(const uint4 *a, const uint4 *b, int s, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                       __builtin_bit_cast(bf16x8, b[s]), c, 0, 0, 0);
    }
};
template <> struct DenseMfma<F16> {
    static constexpr int CPB = 4;
    __device__ static f32x4 step(const uint4 *a, const uint4 *b, int s, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[s]),
                                                      __builtin_bit_cast(f16x8, b[s]), c, 0, 0, 0);
    }
};
template <> struct DenseMfma<F32> {
    static constexpr int CPB = 1;
    __device__ static f32x4 step(const uint4 *a, const uint4 *b, int s, f32x4 c) {
        const float av = __uint_as_float(s == 0 ? a[0].x : s == 1 ? a[0].y : s == 2 ? a[0].z : a[0].w);
        const float bv = __uint_as_float(s == 0 ? b[0].x : s == 1 ? b[0].y : s == 2 ? b[0].z : b[0].w);
        return __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, c, 0, 0, 0);
    }
};

template <typename S>
struct DenseGeom {
    static constexpr int E = S::kElemsPer16B;            // elements per 16-byte chunk
    static constexpr int CPB = DenseMfma<S>::CPB;
    static constexpr int KB = 4 * CPB * E;               // elements per block
};

// Loads the chunks lane (g, c) contributes to block b for one operand row.
// Transposed operand: `row` points at the start of the K-contiguous row.
template <typename S, bool VEC>
__device__ inline void load_row_chunks(uint4 *dst, const typename S::store_t *row, int64_t kbase,
                                       int64_t K, bool ok)
{
    using G = DenseGeom<S>;
#pragma unroll
    for (int ci = 0; ci < G::CPB; ++ci) dst[ci] = load_chunk<S, VEC>(row, kbase + ci * G::E, K, ok);
}

// Natural-layout weight [K, N]: gathers column `col` at the same k positions.
template <typename S>
__device__ inline void load_col_chunks(uint4 *dst, const typename S::store_t *w, int64_t kbase,
                                       int64_t K, int64_t N, int64_t col, bool ok)
{
    using G = DenseGeom<S>;
    using T = typename S::store_t;
#pragma unroll
    for (int ci = 0; ci < G::CPB; ++ci) {
        T tmp[G::E];
#pragma unroll
        for (int e = 0; e < G::E; ++e) {
            const int64_t k = kbase + ci * G::E + e;
            tmp[e] = (ok && k < K) ? w[k * N + col] : (T)0;
        }
        dst[ci] = __builtin_bit_cast(uint4, tmp);
    }
}

// One workgroup: output tile of MT*16 rows x NS*16 columns, kDenseWaves waves.
// blockIdx.z selects a K range for the split comparison variant (splits > 1,
// partials written to `part` as fp32 [splits, M, N]); the invariant path runs
// with splits == 1 and part == nullptr.
template <typename S, bool TRANS, bool VEC, int MT, int NS>
__global__ __launch_bounds__(kDenseWaves * kWave)
void dense_kernel(const typename S::store_t *__restrict__ x, const typename S::store_t *__restrict__ w,
                  typename S::store_t *__restrict__ y, float *__restrict__ part,
                  int64_t M, int64_t N, int64_t K, int64_t nblocks, int splits)
{
    using G = DenseGeom<S>;
    constexpr int P = kDenseWaves;
    constexpr int TR = MT * 16, TC = NS * 16;
    __shared__ float red[P][TR][TC + 1];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, c = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * TC;
    const int64_t m0 = (int64_t)blockIdx.y * TR;
    const int64_t zb0 = (int64_t)blockIdx.z * nblocks / splits;
    const int64_t zb1 = (int64_t)(blockIdx.z + 1) * nblocks / splits;

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const typename S::store_t *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t r = m0 + i * 16 + c;
        xok[i] = r < M;
        xrow[i] = x + (xok[i] ? r : 0) * K;
    }
    int64_t wcol[NS];
    bool wok[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int64_t n = n0 + j * 16 + c;
        wok[j] = n < N;
        wcol[j] = wok[j] ? n : 0;
    }

    uint4 A0[MT][G::CPB], B0[NS][G::CPB], A1[MT][G::CPB], B1[NS][G::CPB];

    auto load = [&](uint4 (&A)[MT][G::CPB], uint4 (&B)[NS][G::CPB], int64_t b) {
        const int64_t kbase = b * G::KB + (int64_t)g * G::CPB * G::E;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (TRANS) load_row_chunks<S, VEC>(B[j], w + wcol[j] * K, kbase, K, wok[j]);
            else load_col_chunks<S>(B[j], w, kbase, K, N, wcol[j], wok[j]);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) load_row_chunks<S, VEC>(A[i], xrow[i], kbase, K, xok[i]);
    };
    auto compute = [&](const uint4 (&A)[MT][G::CPB], const uint4 (&B)[NS][G::CPB]) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NS; ++j) acc[i][j] = DenseMfma<S>::step(A[i], B[j], s, acc[i][j]);
    };

    int64_t b = zb0 + wave;
    if (b < zb1) load(A0, B0, b);
    while (b < zb1) {
        const int64_t b1 = b + P;
        if (b1 < zb1) load(A1, B1, b1);
        compute(A0, B0);
        if (b1 >= zb1) break;
        const int64_t b2 = b1 + P;
        if (b2 < zb1) load(A0, B0, b2);
        compute(A1, B1);
        b = b2;
    }

    // MFMA 16x16 accumulator layout: lane (g, c), register r holds row 4g + r, column c.
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][i * 16 + g * 4 + r][j * 16 + c] = acc[i][j][r];
    __syncthreads();

    for (int o = threadIdx.x; o < TR * TC; o += P * kWave) {
        const int r = o / TC, cc = o % TC;
        const int64_t row = m0 + r, col = n0 + cc;
        if (row >= M || col >= N) continue;
        float v = red[0][r][cc];
#pragma unroll
        for (int p = 1; p < P; ++p) v = v + red[p][r][cc];
        if (part) part[((int64_t)blockIdx.z * M + row) * N + col] = v;
        else y[row * N + col] = S::narrow(v);
    }
}

// Cleanup reduction of the split comparison variant: y = sum_z part[z] in z order.
template <typename S>
__global__ void split_reduce_kernel(const float *__restrict__ part, typename S::store_t *__restrict__ y,
                                    int64_t MN, int splits)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += (int64_t)gridDim.x * blockDim.x) {
        float v = part[i];
        for (int z = 1; z < splits; ++z) v = v + part[(int64_t)z * MN + i];
        y[i] = S::narrow(v);
    }
}

template <typename S, bool TRANS, bool VEC, int MT, int NS>
static void launch_dense_t(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                           int64_t K, int splits, hipStream_t st)
{
    using G = DenseGeom<S>;
    using T = typename S::store_t;
    const int64_t nblocks = cdiv(K, G::KB);
    dim3 grid((unsigned)cdiv(N, NS * 16), (unsigned)cdiv(M, MT * 16), (unsigned)splits);
    hipLaunchKernelGGL((dense_kernel<S, TRANS, VEC, MT, NS>), grid, dim3(kDenseWaves * kWave), 0, st,
                       (const T *)x, (const T *)w, (T *)y, part, M, N, K, nblocks, splits);
}

template <typename S, bool TRANS, bool VEC>
static void launch_dense_mt(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                            int64_t K, int splits, hipStream_t st)
{
    // Tile shape is free: it never changes a row's reduction.
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_dense_t<S, TRANS, VEC, 1, 1>(x, w, y, part, M, N, K, splits, st);
    else if (mt <= 2) launch_dense_t<S, TRANS, VEC, 2, 1>(x, w, y, part, M, N, K, splits, st);
    else if (N >= 4096 && M > 64) launch_dense_t<S, TRANS, VEC, 4, 2>(x, w, y, part, M, N, K, splits, st);
    else launch_dense_t<S, TRANS, VEC, 4, 1>(x, w, y, part, M, N, K, splits, st);
}

template <typename S>
static void launch_dense(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                         int64_t K, bool trans, int splits, hipStream_t st)
{
    // 16-byte chunk loads when K is a multiple of the chunk length (chunks then
    // never straddle K) and both operands start on 16-byte boundaries; the
    // element-wise path fills the same slots, so the tree is the same.
    const bool vec = (K % S::kElemsPer16B) == 0 && host_aligned16(x) && (host_aligned16(w) || !trans);
    if (trans) {
        if (vec) launch_dense_mt<S, true, true>(x, w, y, part, M, N, K, splits, st);
        else launch_dense_mt<S, true, false>(x, w, y, part, M, N, K, splits, st);
    } else {
        if (vec) launch_dense_mt<S, false, true>(x, w, y, part, M, N, K, splits, st);
        else launch_dense_mt<S, false, false>(x, w, y, part, M, N, K, splits, st);
    }
}

static bi_status check_dense(const void *x, const void *w, const void *y, int64_t M, int64_t N, int64_t K,
                             int32_t dtype)
{
    if (!x || !w || !y) return BI_ERR_NULL;
    if (M < 1 || N < 1 || K < 1 || M > (1ll << 31) || N > (1ll << 31) || K > (1ll << 31)) return BI_ERR_SHAPE;
    if (dtype != BI_BF16 && dtype != BI_F16 && dtype != BI_F32) return BI_ERR_DTYPE;
    const size_t esz = dtype == BI_F32 ? 4 : 2;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & (esz - 1)) return BI_ERR_ALIGN;
    return BI_OK;
}

static void dispatch_dense(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                           int64_t K, int32_t dtype, bool trans, int splits, hipStream_t st)
{
    if (dtype == BI_BF16) launch_dense<BF16>(x, w, y, part, M, N, K, trans, splits, st);
    else if (dtype == BI_F16) launch_dense<F16>(x, w, y, part, M, N, K, trans, splits, st);
    else launch_dense<F32>(x, w, y, part, M, N, K, trans, splits, st);
}

}  // namespace bi

using namespace bi;

extern "C" bi_status bi_matmul(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                               int32_t dtype, int32_t w_transposed, hipStream_t stream)
{
    bi_status s = check_dense(x, w, y, M, N, K, dtype);
    if (s != BI_OK) return s;
    (void)hipGetLastError();
    dispatch_dense(x, w, y, nullptr, M, N, K, dtype, w_transposed != 0, 1, stream);
    return launch_status();
}

extern "C" size_t bi_matmul_split_workspace_bytes(int64_t M, int64_t N, int32_t splits)
{
    if (M < 1 || N < 1 || splits < 1) return 0;
    return (size_t)M * (size_t)N * (size_t)splits * sizeof(float);
}

extern "C" bi_status bi_matmul_split(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                                     int32_t dtype, int32_t w_transposed, int32_t splits, void *ws,
                                     size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_dense(x, w, y, M, N, K, dtype);
    if (s != BI_OK) return s;
    if (splits < 1 || splits > 1024) return BI_ERR_SHAPE;
    if (splits == 1) return bi_matmul(x, w, y, M, N, K, dtype, w_transposed, stream);
    if (!ws) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    if (ws_bytes < bi_matmul_split_workspace_bytes(M, N, splits)) return BI_ERR_WORKSPACE;
    (void)hipGetLastError();
    float *part = (float *)ws;
    dispatch_dense(x, w, y, part, M, N, K, dtype, w_transposed != 0, splits, stream);
    const int64_t MN = M * N;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(MN, 256), 65536);
    if (dtype == BI_BF16) hipLaunchKernelGGL(split_reduce_kernel<BF16>, dim3(blocks), dim3(256), 0, stream, part, (uint16_t *)y, MN, splits);
    else if (dtype == BI_F16) hipLaunchKernelGGL(split_reduce_kernel<F16>, dim3(blocks), dim3(256), 0, stream, part, (uint16_t *)y, MN, splits);
    else hipLaunchKernelGGL(split_reduce_kernel<F32>, dim3(blocks), dim3(256), 0, stream, part, (float *)y, MN, splits);
    return launch_status();
}
