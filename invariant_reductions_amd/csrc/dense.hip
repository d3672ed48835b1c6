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
//     v_mfma_f32_16x16x4_f32) consume the block.  16-bit types: step s takes
//     elements [32s, 32s + 32) of the block, lane group g (lanes 16g..16g+15)
//     the 8 at 32s + 8g, so every load instruction reads 64 contiguous bytes
//     of each row.  f32: lane group g holds the 4 elements at 4g and step s
//     takes the s-th of them.  A wave accumulates its blocks in ascending order
//     in the MFMA accumulator.
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
    // element offset, within a block, of chunk ci of lane group g
    __device__ static constexpr int chunk_off(int g, int ci) { return CPB == 4 ? ci * 32 + g * 8 : g * 4; }
};

// Loads the chunks lane (g, c) contributes to block b for one operand row.
// Transposed operand: `row` points at the start of the K-contiguous row.
template <typename S, bool VEC>
__device__ inline void load_row_chunks(uint4 *dst, const typename S::store_t *row, int64_t kblk, int g,
                                       int64_t K, bool ok)
{
    using G = DenseGeom<S>;
#pragma unroll
    for (int ci = 0; ci < G::CPB; ++ci) dst[ci] = load_chunk<S, VEC>(row, kblk + G::chunk_off(g, ci), K, ok);
}

// Natural-layout weight [K, N]: gathers column `col` at the same k positions.
template <typename S>
__device__ inline void load_col_chunks(uint4 *dst, const typename S::store_t *w, int64_t kblk, int g,
                                       int64_t K, int64_t N, int64_t col, bool ok)
{
    using G = DenseGeom<S>;
    using T = typename S::store_t;
#pragma unroll
    for (int ci = 0; ci < G::CPB; ++ci) {
        T tmp[G::E];
#pragma unroll
        for (int e = 0; e < G::E; ++e) {
            const int64_t k = kblk + G::chunk_off(g, ci) + e;
            tmp[e] = (ok && k < K) ? w[k * N + col] : (T)0;
        }
        dst[ci] = __builtin_bit_cast(uint4, tmp);
    }
}

// One workgroup: output tile of MT*16 rows x NS*16 columns, kDenseWaves waves.
// blockIdx.z selects a K range for the split comparison variant (splits > 1,
// partials written to `part` as fp32 [splits, M, N]); the invariant path runs
// with splits == 1 and part == nullptr.
template <typename S, bool TRANS, bool VEC, int MT, int NS, bool PART>
__global__ __launch_bounds__(kDenseWaves * kWave, (TRANS && VEC && !(MT >= 4 && NS >= 2)) ? 4 : 2)
void dense_kernel(const typename S::store_t *__restrict__ x, const typename S::store_t *__restrict__ w,
                  typename S::store_t *__restrict__ y, float *__restrict__ part,
                  int64_t M, int64_t N, int64_t K, int64_t nblocks, int splits)
{
    using G = DenseGeom<S>;
    constexpr int P = kDenseWaves;
    constexpr int TR = MT * 16, TC = NS * 16;
    __shared__ float red[P][TR][TC + 1];

    const int lane = threadIdx.x & 63, wave = wave_id();
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

    // Row pointers are clamped to valid rows: a padding row of the M tile or
    // a padding column of the N tile then reads real, in-bounds data, and the
    // outputs it feeds are never stored (an MFMA keeps rows and columns
    // independent), so full blocks need no per-load bounds test.
    const typename S::store_t *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t r = m0 + i * 16 + c;
        xok[i] = r < M;
        xrow[i] = x + (xok[i] ? r : M - 1) * K;
    }
    int64_t wcol[NS];
    bool wok[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int64_t n = n0 + j * 16 + c;
        wok[j] = n < N;
        wcol[j] = wok[j] ? n : N - 1;
    }

    // Register ring of DEPTH block buffers: the wave keeps DEPTH - 1 blocks
    // of loads in flight while it multiplies the oldest one.
    constexpr int DEPTH = MT == 1 ? 3 : (MT == 2 ? 2 : 1);
    uint4 Ab[DEPTH][MT][G::CPB], Bb[DEPTH][NS][G::CPB];

    // Masked loads: elements at k >= K and padding rows/columns read as zero.
    auto load_masked = [&](uint4 (&A)[MT][G::CPB], uint4 (&B)[NS][G::CPB], int64_t b) {
        const int64_t kblk = b * G::KB;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (TRANS) load_row_chunks<S, VEC>(B[j], w + wcol[j] * K, kblk, g, K, wok[j]);
            else load_col_chunks<S>(B[j], w, kblk, g, K, N, wcol[j], wok[j]);
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) load_row_chunks<S, VEC>(A[i], xrow[i], kblk, g, K, xok[i]);
    };
    // Full blocks (VEC only): unconditional 16-byte loads.
    auto load_full = [&](uint4 (&A)[MT][G::CPB], uint4 (&B)[NS][G::CPB], int64_t b) {
        const int64_t kblk = b * G::KB;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (TRANS) {
                const typename S::store_t *wr = w + wcol[j] * K + kblk;
#pragma unroll
                for (int ci = 0; ci < G::CPB; ++ci)
                    B[j][ci] = *reinterpret_cast<const uint4 *>(wr + G::chunk_off(g, ci));
            } else {
                load_col_chunks<S>(B[j], w, kblk, g, K, N, wcol[j], true);
            }
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const typename S::store_t *xr = xrow[i] + kblk;
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci) A[i][ci] = *reinterpret_cast<const uint4 *>(xr + G::chunk_off(g, ci));
        }
    };
    auto compute = [&](const uint4 (&A)[MT][G::CPB], const uint4 (&B)[NS][G::CPB]) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NS; ++j) acc[i][j] = DenseMfma<S>::step(A[i], B[j], s, acc[i][j]);
    };

    // This wave's blocks: zb0 + wave, zb0 + wave + P, ... (< zb1), ascending.
    // Full blocks stream through the ring; the body is straight-line code (the
    // last prefetches re-read the final block instead of branching, so every
    // wait on a load is exact) and scheduling fences keep the loads ahead of
    // the multiplies.  The one partial block at the end of K (if any) is
    // loaded with masks, last.
    const int64_t nfull = VEC ? K / G::KB : 0;
    const int64_t bend = zb1 < nfull ? zb1 : nfull;
    const int64_t first = zb0 + wave;
    const int64_t nmine = first < bend ? (bend - first + P - 1) / P : 0;     // full blocks of this wave
    if (nmine > 0) {
        const int64_t lastb = nmine - 1;
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_full(Ab[d], Bb[d], first + (d < lastb ? d : lastb) * P);
        for (int64_t i = 0; i < nmine; i += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int64_t li = i + d + DEPTH - 1;
                load_full(Ab[(d + DEPTH - 1) % DEPTH], Bb[(d + DEPTH - 1) % DEPTH], first + (li < lastb ? li : lastb) * P);
                __builtin_amdgcn_sched_barrier(0);
                if (i + d < nmine) compute(Ab[d], Bb[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    for (int64_t b = first + nmine * P; b < zb1; b += P) {
        load_masked(Ab[0], Bb[0], b);
        compute(Ab[0], Bb[0]);
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
        if (PART) part[((int64_t)blockIdx.z * M + row) * N + col] = v;
        else y[row * N + col] = S::narrow(v);
    }
}

// Persistent streaming form of the same reduction (transposed weights, 16-byte
// aligned rows, K a multiple of the block): a fixed grid of workgroups walks
// the output tiles t = blockIdx.x, blockIdx.x + gridDim.x, ...  Each wave
// streams the sequence (tile, block) of its blocks through a register ring
// that runs across tile boundaries, so the loads of the next tile are in
// flight while the current tile's eight partials are combined.  Per output
// the tree is exactly that of dense_kernel: block b of K belongs to wave
// b mod P, accumulated in ascending order, partials added in wave order.
template <typename S, int MT, int NS>
__global__ __launch_bounds__(kDenseWaves * kWave, (MT >= 4 && NS >= 2) ? 2 : 4)
void dense_stream_kernel(const typename S::store_t *__restrict__ x, const typename S::store_t *__restrict__ w,
                         typename S::store_t *__restrict__ y, int64_t M, int64_t N, int64_t K,
                         int64_t ntm, int64_t ntn)
{
    using G = DenseGeom<S>;
    using T = typename S::store_t;
    constexpr int P = kDenseWaves;
    constexpr int TR = MT * 16, TC = NS * 16;
    constexpr int DEPTH = MT == 1 ? 3 : (MT == 2 ? 2 : 1);
    __shared__ float red[P][TR][TC + 1];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int64_t nb = K / G::KB;                                  // every block is full here
    const int64_t nmine = wave < nb ? (nb - wave + P - 1) / P : 0; // blocks of this wave per tile
    const int64_t ntiles = ntm * ntn;
    const int64_t mytiles = blockIdx.x < ntiles ? (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
    const int64_t items = mytiles * nmine;

    // tile u of this workgroup -> (row tile, column tile).  Tiles are walked in
    // groups of up to 64 row tiles, row tile fastest, so the workgroups in
    // flight at any time share a few column tiles of W and a group's rows of x
    // stay cache-resident while W streams past (only matters for large M).
    auto tile_of = [&](int64_t u, int64_t &tm, int64_t &tn) {
        constexpr int64_t GM = 64;
        const int64_t t = blockIdx.x + u * gridDim.x;
        const int64_t grp = t / (GM * ntn), r = t % (GM * ntn);
        const int64_t gm = ntm - grp * GM < GM ? ntm - grp * GM : GM;
        tm = grp * GM + r % gm;
        tn = r / gm;
    };

    uint4 Ab[DEPTH][MT][G::CPB], Bb[DEPTH][NS][G::CPB];
    auto load_item = [&](uint4 (&A)[MT][G::CPB], uint4 (&B)[NS][G::CPB], int64_t it) {
        int64_t tm, tn;
        tile_of(it / nmine, tm, tn);
        const int64_t kblk = (wave + (it % nmine) * P) * G::KB;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            int64_t n = tn * TC + j * 16 + c;
            n = n < N ? n : N - 1;                                // padding columns read a real row
            const T *wr = w + n * K + kblk;
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci) B[j][ci] = *reinterpret_cast<const uint4 *>(wr + G::chunk_off(g, ci));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            int64_t r = tm * TR + i * 16 + c;
            r = r < M ? r : M - 1;
            const T *xr = x + r * K + kblk;
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci) A[i][ci] = *reinterpret_cast<const uint4 *>(xr + G::chunk_off(g, ci));
        }
    };

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto finish_tile = [&](int64_t u) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wave][i * 16 + g * 4 + r][j * 16 + c] = acc[i][j][r];
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        __syncthreads();
        int64_t tm, tn;
        tile_of(u, tm, tn);
        for (int o = threadIdx.x; o < TR * TC; o += P * kWave) {
            const int r = o / TC, cc = o % TC;
            const int64_t row = tm * TR + r, col = tn * TC + cc;
            if (row >= M || col >= N) continue;
            float v = red[0][r][cc];
#pragma unroll
            for (int p = 1; p < P; ++p) v = v + red[p][r][cc];
            y[row * N + col] = S::narrow(v);
        }
        __syncthreads();
    };

    if (items > 0) {
        const int64_t last = items - 1;
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_item(Ab[d], Bb[d], d < last ? d : last);
        for (int64_t i = 0; i < items; i += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                const int64_t li = i + d + DEPTH - 1;
                load_item(Ab[(d + DEPTH - 1) % DEPTH], Bb[(d + DEPTH - 1) % DEPTH], li < last ? li : last);
                __builtin_amdgcn_sched_barrier(0);
                if (i + d < items) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int a = 0; a < MT; ++a)
#pragma unroll
                            for (int b2 = 0; b2 < NS; ++b2)
                                acc[a][b2] = DenseMfma<S>::step(Ab[d][a], Bb[d][b2], s, acc[a][b2]);
                    if ((i + d) % nmine == nmine - 1) finish_tile((i + d) / nmine);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // a wave that owns no block of K still takes part in every combine
        for (int64_t u = 0; u < mytiles; ++u) finish_tile(u);
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
    // The split comparison variant is its own instantiation, so profiles of the
    // invariant kernel never mix in its launches.
    if (part)
        hipLaunchKernelGGL((dense_kernel<S, TRANS, VEC, MT, NS, true>), grid, dim3(kDenseWaves * kWave), 0, st,
                           (const T *)x, (const T *)w, (T *)y, part, M, N, K, nblocks, splits);
    else
        hipLaunchKernelGGL((dense_kernel<S, TRANS, VEC, MT, NS, false>), grid, dim3(kDenseWaves * kWave), 0, st,
                           (const T *)x, (const T *)w, (T *)y, part, M, N, K, nblocks, splits);
}

template <typename S, bool TRANS, bool VEC>
static void launch_dense_mt(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                            int64_t K, int splits, hipStream_t st)
{
    // Tile shape is free: it never changes a row's reduction.
    // Wider N tiles once there are enough of them: every workgroup re-reads its
    // rows of x, so a tile of 2x16 columns halves that traffic.
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_dense_t<S, TRANS, VEC, 1, 1>(x, w, y, part, M, N, K, splits, st);
    else if (mt <= 2) launch_dense_t<S, TRANS, VEC, 2, 1>(x, w, y, part, M, N, K, splits, st);
    else if (N >= 8192) launch_dense_t<S, TRANS, VEC, 4, 2>(x, w, y, part, M, N, K, splits, st);
    else launch_dense_t<S, TRANS, VEC, 4, 1>(x, w, y, part, M, N, K, splits, st);
}

static int device_cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
        cached[dev] = cu;                       // benign race: every writer stores the same value
    }
    return cached[dev];
}

template <typename S, int MT, int NS>
static void launch_stream_t(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, hipStream_t st)
{
    using T = typename S::store_t;
    const int64_t ntm = cdiv(M, MT * 16), ntn = cdiv(N, NS * 16);
    const int per_cu = (MT >= 4 && NS >= 2) ? 1 : 2;             // resident workgroups per CU at the register cap
    const int64_t grid = std::min<int64_t>(ntm * ntn, (int64_t)device_cu_count() * per_cu);
    hipLaunchKernelGGL((dense_stream_kernel<S, MT, NS>), dim3((unsigned)grid), dim3(kDenseWaves * kWave), 0, st,
                       (const T *)x, (const T *)w, (T *)y, M, N, K, ntm, ntn);
}

template <typename S>
static bool try_launch_stream(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                              hipStream_t st)
{
    using G = DenseGeom<S>;
    if (K % G::KB != 0 || !host_aligned16(x) || !host_aligned16(w)) return false;
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_stream_t<S, 1, 1>(x, w, y, M, N, K, st);
    else if (mt <= 2) launch_stream_t<S, 2, 1>(x, w, y, M, N, K, st);
    else if (N >= 16384) launch_stream_t<S, 4, 4>(x, w, y, M, N, K, st);
    else if (N >= 6144) launch_stream_t<S, 4, 2>(x, w, y, M, N, K, st);
    else launch_stream_t<S, 4, 1>(x, w, y, M, N, K, st);
    return true;
}

template <typename S>
static void launch_dense(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                         int64_t K, bool trans, int splits, hipStream_t st)
{
    if (trans && splits == 1 && part == nullptr && try_launch_stream<S>(x, w, y, M, N, K, st)) return;
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
