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
//     block b belongs to slot (b mod P), P = kDenseWaves = 8.
//   * Inside a block, four MFMA steps (v_mfma_f32_16x16x32_{bf16,f16} or
//     v_mfma_f32_16x16x4_f32) consume the block.  16-bit types: step s takes
//     elements [32s, 32s + 32) of the block, lane group g (lanes 16g..16g+15)
//     the 8 at 32s + 8g, so every load instruction reads 64 contiguous bytes
//     of each row.  f32: lane group g holds the 4 elements at 4g and step s
//     takes the s-th of them.  A slot's blocks are accumulated in ascending
//     order in one MFMA accumulator (one wave owns the slot).
//   * The P slot partials are added pairwise in fp32,
//     ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)), then rounded to the
//     output type (RNE).
// Row m of the output only ever meets row m of x inside an MFMA, so the M-tile
// it falls in, the other rows of that tile, the number of M-tiles and the
// N-tile width (all chosen from the shape) leave its bits unchanged.  M = 1 is
// the same MFMA with fifteen padding rows.  Which workgroup owns a slot (all
// eight in one workgroup, or spread over several with the partials of each
// aligned slot group combined through a workspace) is a launch choice that
// the tree does not see.
#include "common.hpp"

namespace bi {

constexpr int kDenseWaves = 8;   // P: K-block slots per output (frozen)

// The frozen combine of the P = 8 slot partials, pairwise:
//   ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)).
// Every aligned group of 1, 2, 4 or 8 consecutive slots is a subtree of it, so
// a workgroup that owns such a group may add its own slots first.
template <typename F>
__device__ inline float slot_tree(F p)
{
    return ((p(0) + p(1)) + (p(2) + p(3))) + ((p(4) + p(5)) + (p(6) + p(7)));
}

template <typename S> struct DenseMfma;

template <> struct DenseMfma<BF16> {
    static constexpr int CPB = 4;                 // 16-byte chunks per lane per block
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static f32x4 step(const uint4 *a, const uint4 *b, int s, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                       __builtin_bit_cast(bf16x8, b[s]), c, 0, 0, 0);
    }
};
template <> struct DenseMfma<F16> {
    static constexpr int CPB = 4;
    __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
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
        const float v = slot_tree([&](int p) { return red[p][r][cc]; });
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
// b mod P, accumulated in ascending order, partials added by slot_tree.
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
    constexpr int DEPTH = MT <= 2 ? 2 : 1;
    __shared__ float red[P][TR][TC + 1];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int nb = (int)(K / G::KB);                               // every block is full here
    const int nmine = wave < nb ? (nb - wave + P - 1) / P : 0;     // blocks of this wave per tile
    const int ntiles = (int)(ntm * ntn);
    const int mytiles = (int)blockIdx.x < ntiles ? (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    const int items = mytiles * nmine;

    // tile u of this workgroup -> (row tile, column tile).  Tiles are walked in
    // groups of up to 64 row tiles, row tile fastest, so the workgroups in
    // flight at any time share a few column tiles of W and a group's rows of x
    // stay cache-resident while W streams past (only matters for large M).
    // 32-bit arithmetic, evaluated once per tile.
    auto tile_of = [&](int u, int &tm, int &tn) {
        constexpr int GM = 64;
        const int t = (int)blockIdx.x + u * (int)gridDim.x;
        const int gsz = GM * (int)ntn;
        const int grp = t / gsz, r = t - grp * gsz;
        const int gm = (int)ntm - grp * GM < GM ? (int)ntm - grp * GM : GM;
        tn = r / gm;
        tm = grp * GM + (r - tn * gm);
    };

    uint4 Ab[DEPTH][MT][G::CPB], Bb[DEPTH][NS][G::CPB];
    // Prefetch cursor: item (pu, pj) = block wave + pj*P of tile pu; it walks the
    // items in order and holds at the last one (the ring's final re-reads).
    int pu = 0, pj = 0, ptm = 0, ptn = 0;
    if (items > 0) tile_of(0, ptm, ptn);
    auto load_next = [&](uint4 (&A)[MT][G::CPB], uint4 (&B)[NS][G::CPB]) {
        const int64_t kblk = (int64_t)(wave + pj * P) * G::KB;
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            int64_t n = (int64_t)ptn * TC + j * 16 + c;
            n = n < N ? n : N - 1;                                // padding columns read a real row
            const T *wr = w + n * K + kblk;
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci) B[j][ci] = *reinterpret_cast<const uint4 *>(wr + G::chunk_off(g, ci));
        }
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            int64_t r = (int64_t)ptm * TR + i * 16 + c;
            r = r < M ? r : M - 1;
            const T *xr = x + r * K + kblk;
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci) A[i][ci] = *reinterpret_cast<const uint4 *>(xr + G::chunk_off(g, ci));
        }
        // advance (wave-uniform scalars)
        if (pj + 1 < nmine) {
            ++pj;
        } else if (pu + 1 < mytiles) {
            pj = 0;
            ++pu;
            tile_of(pu, ptm, ptn);
        }
    };

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto finish_tile = [&](int u) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NS; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wave][i * 16 + g * 4 + r][j * 16 + c] = acc[i][j][r];
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        __syncthreads();
        int tm, tn;
        tile_of(u, tm, tn);
        for (int o = threadIdx.x; o < TR * TC; o += P * kWave) {
            const int r = o / TC, cc = o % TC;
            const int64_t row = (int64_t)tm * TR + r, col = (int64_t)tn * TC + cc;
            if (row >= M || col >= N) continue;
            const float v = slot_tree([&](int p) { return red[p][r][cc]; });
            y[row * N + col] = S::narrow(v);
        }
        __syncthreads();
    };

    if (items > 0) {
        // compute cursor: tile cu, block cj within it
        int cu = 0, cj = 0;
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_next(Ab[d], Bb[d]);
        for (int i = 0; i < items; i += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                load_next(Ab[(d + DEPTH - 1) % DEPTH], Bb[(d + DEPTH - 1) % DEPTH]);
                __builtin_amdgcn_sched_barrier(0);
                if (i + d < items) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int a = 0; a < MT; ++a)
#pragma unroll
                            for (int b2 = 0; b2 < NS; ++b2)
                                acc[a][b2] = DenseMfma<S>::step(Ab[d][a], Bb[d][b2], s, acc[a][b2]);
                    if (++cj == nmine) {
                        finish_tile(cu);
                        cj = 0;
                        ++cu;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // a wave that owns no block of K still takes part in every combine
        for (int u = 0; u < mytiles; ++u) finish_tile(u);
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
        launch_kernel((dense_kernel<S, TRANS, VEC, MT, NS, true>), grid, dim3(kDenseWaves * kWave), 0, st,
                           (const T *)x, (const T *)w, (T *)y, part, M, N, K, nblocks, splits);
    else
        launch_kernel((dense_kernel<S, TRANS, VEC, MT, NS, false>), grid, dim3(kDenseWaves * kWave), 0, st,
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

template <typename S, int MT, int NS>
static void launch_stream_t(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, hipStream_t st)
{
    using T = typename S::store_t;
    const int64_t ntm = cdiv(M, MT * 16), ntn = cdiv(N, NS * 16);
    const int per_cu = (MT >= 4 && NS >= 2) ? 1 : 2;             // resident workgroups per CU at the register cap
    const int64_t grid = std::min<int64_t>(ntm * ntn, (int64_t)device_cu_count() * per_cu);
    launch_kernel((dense_stream_kernel<S, MT, NS>), dim3((unsigned)grid), dim3(kDenseWaves * kWave), 0, st,
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

// ---------------------------------------------------------------------------
// Slot-group form for short M (at most 64 rows): transposed W, 16-bit types,
// K a multiple of the block, x and W 16-byte aligned.
//
// Workgroup (ct, grp) owns the 128 output columns of tile ct (wave v: columns
// 16v .. 16v + 15) and the Q consecutive slots grp*Q .. grp*Q + Q - 1.  It
// walks its blocks as items u -> (step j = u / Q, slot grp*Q + u % Q), i.e.
// block 8j + grp*Q + u % Q.  Each block of x (all rows of the M tile) is
// staged once in LDS and read by all eight waves; each wave streams its 16
// rows of W through a register ring.  Slot i of the group accumulates in its
// own MFMA accumulator, block by block in ascending order, exactly as a wave
// of the kernels above does, and the Q slot partials are added by their
// subtree of slot_tree.  With 8/Q > 1 groups per tile, each group writes that
// sum to the workspace; the last workgroup of the tile to arrive (counted with
// a device-scope atomic) reads all group sums, adds them by the rest of
// slot_tree and stores y.  Arrival order decides only who adds, never how.
constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// What the slot kernel does with a finished tile: store y (EPI_Y), or the
// SwiGLU activation of an interleaved gate/up tile (EPI_SWIGLU: the 128
// columns of tile ct are gate columns 64ct .. 64ct + 63 followed by the up
// columns of the same indices; a[m, 64ct + j] = silu_mul1(y[m, 128ct + j],
// y[m, 128ct + 64 + j]), from the bf16-rounded y exactly as bi_silu_mul
// would read it).
enum SlotEpilogue { EPI_Y = 0, EPI_SWIGLU = 1 };

template <typename S, int MT, int Q, int DW, int OCC, int EPI>
__global__ __launch_bounds__(kDenseWaves * kWave, OCC)
void dense_slots_kernel(const typename S::store_t *__restrict__ x, const typename S::store_t *__restrict__ w,
                        typename S::store_t *__restrict__ y, float *__restrict__ part,
                        unsigned *__restrict__ counters, int64_t M, int64_t N, int64_t K)
{
    using G = DenseGeom<S>;
    using T = typename S::store_t;
    constexpr int P = kDenseWaves, NT = P * kWave;
    constexpr int GRP = P / Q;                     // slot groups per column tile
    constexpr int TR = MT * 16, KB = G::KB;
    constexpr int XS = KB + 8;                     // LDS row stride: 272 bytes, 16-byte aligned, 4-bank shift per row
    constexpr int XCH = TR * (KB / 8);             // 16-byte chunks in one block of x
    constexpr int XPT = XCH > NT ? XCH / NT : 1;   // chunks staged per thread
    constexpr int DX = 3;                          // x register ring depth (DW: W ring depth)
    constexpr int U = lcm_c(lcm_c(3, DW), Q);       // unroll: a multiple of the LDS ring (3 = DX), DW and Q
    static_assert(G::CPB == 4 && XPT <= 2 && (XCH % NT == 0 || XPT == 1), "slot kernel geometry");
    __shared__ __attribute__((aligned(16))) T xs[3][TR][XS];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int ct = blockIdx.x, grp = blockIdx.y;
    const int nb = (int)(K / KB);
    const int slot0 = grp * Q;
    const int nsteps = slot0 < nb ? (nb - slot0 + P - 1) / P : 0;
    const int nitems = nsteps * Q;
    // Block of item u.  Items past the last block re-read block slot0 (valid
    // whenever nitems > 0) and are never multiplied.
    auto block_of = [&](int u) {
        const int b = (u / Q) * P + slot0 + (u % Q);
        return b < nb ? b : slot0;
    };

    const int64_t n = (int64_t)ct * (P * 16) + wave * 16 + c;
    const bool nok = n < N;
    const T *wr = w + (nok ? n : N - 1) * K;     // padding columns read a real row, never stored
    const int t = threadIdx.x, xc = t & 15;

    struct XChunks { uint4 v0, v1; };
    XChunks xr0, xr1, xr2;
    auto xreg = [&](auto sc) -> XChunks & {
        constexpr int sl = decltype(sc)::value % DX;
        if constexpr (sl == 0) return xr0;
        else if constexpr (sl == 1) return xr1;
        else return xr2;
    };
    // thread t stages chunk (t + h*NT) mod XCH of the block: row / 16, 16 bytes at (chunk % 16) * 16
    auto load_x = [&](XChunks &r, int u) {
        const int64_t kb = (int64_t)block_of(u) * KB + xc * 8;
        static_for<0, XPT>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const int row = ((t + h * NT) % XCH) >> 4;
            const uint4 v = *reinterpret_cast<const uint4 *>(x + (int64_t)(row < M ? row : M - 1) * K + kb);
            if constexpr (h == 0) r.v0 = v;
            else r.v1 = v;
        });
    };
    auto store_x = [&](const XChunks &r, int buf) {
        static_for<0, XPT>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const int row = ((t + h * NT) % XCH) >> 4;
            *reinterpret_cast<uint4 *>(&xs[buf][row][xc * 8]) = h == 0 ? r.v0 : r.v1;
        });
    };
    uint4 wb[DW][G::CPB];
    auto load_w = [&](uint4 (&B)[G::CPB], int u) {
        const T *p = wr + (int64_t)block_of(u) * KB;
#pragma unroll
        for (int ci = 0; ci < G::CPB; ++ci) B[ci] = *reinterpret_cast<const uint4 *>(p + G::chunk_off(g, ci));
    };

    f32x4 acc[Q][MT];
#pragma unroll
    for (int i = 0; i < Q; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nitems > 0) {
        // Pipeline: x of item u + 1 goes to LDS slot (u + 1) % 3 at item u (its
        // register slot is refilled with item u + 1 + DX); W runs DW - 1 items
        // ahead.  Three LDS slots let one barrier per item separate the writers
        // of slot (u + 1) % 3 from the last readers of that slot (item u - 2).
        static_for<0, DX>([&](auto dc) { load_x(xreg(dc), decltype(dc)::value); });
        store_x(xr0, 0);
        load_x(xr0, DX);
        static_for<0, DW - 1>([&](auto dc) { load_w(wb[decltype(dc)::value], decltype(dc)::value); });
        // One item: stage x of item u + 1, refill the rings, wait for the
        // workgroup, multiply item u (unless it lies past the last block).
        auto item = [&](auto dc, int u) {
            constexpr int d = decltype(dc)::value;
            XChunks &nx = xreg(std::integral_constant<int, d + 1>{});
            store_x(nx, (d + 1) % 3);
            load_x(nx, u + 1 + DX);
            load_w(wb[(d + DW - 1) % DW], u + DW - 1);
            __syncthreads();
            if ((u / Q) * P + slot0 + (d % Q) < nb) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    uint4 a[MT];
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        a[m] = *reinterpret_cast<const uint4 *>(&xs[d % 3][m * 16 + c][G::chunk_off(g, st)]);
#pragma unroll
                    for (int m = 0; m < MT; ++m) acc[d % Q][m] = DenseMfma<S>::mma(a[m], wb[d % DW][st], acc[d % Q][m]);
                }
            }
        };
        // Whole unrolled rounds run without item guards (exact load waits);
        // the last partial round is guarded.
        int u0 = 0;
        for (; u0 + U <= nitems; u0 += U) static_for<0, U>([&](auto dc) { item(dc, u0 + decltype(dc)::value); });
        if (u0 < nitems)
            static_for<0, U>([&](auto dc) {
                if (u0 + decltype(dc)::value < nitems) item(dc, u0 + decltype(dc)::value);
            });
    }

    // the group's subtree of slot_tree
    f32x4 h[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        if constexpr (Q == 1) h[m] = acc[0][m];
        else if constexpr (Q == 2) h[m] = acc[0][m] + acc[1][m];
        else if constexpr (Q == 4) h[m] = (acc[0][m] + acc[1][m]) + (acc[2][m] + acc[3][m]);
        else h[m] = ((acc[0][m] + acc[1][m]) + (acc[2][m] + acc[3][m])) + ((acc[4][m] + acc[5][m]) + (acc[6][m] + acc[7][m]));
    }
    // MFMA accumulator layout: lane (g, c), register r holds row 4g + r, column c.
    auto store_y = [&](const f32x4 (&v)[MT]) {
        if constexpr (EPI == EPI_Y) {
            if (!nok) return;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = m * 16 + g * 4 + r;
                    if (row < M) y[row * N + n] = S::narrow(v[m][r]);
                }
        } else {
            // the tile's rounded y into LDS (the x ring is free by now), then
            // each thread forms 8 consecutive activations of one row
            T (*tile)[XS] = xs[0];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) tile[m * 16 + g * 4 + r][wave * 16 + c] = S::narrow(v[m][r]);
            __syncthreads();
            const int F = (int)(N / 2);
            for (int it = threadIdx.x; it < TR * 8; it += NT) {
                const int row = it >> 3, jg = (it & 7) * 8;
                if (row >= M) continue;
                const uint4 gv = *reinterpret_cast<const uint4 *>(&tile[row][jg]);
                const uint4 uv = *reinterpret_cast<const uint4 *>(&tile[row][64 + jg]);
                const uint16_t *g8 = reinterpret_cast<const uint16_t *>(&gv), *u8 = reinterpret_cast<const uint16_t *>(&uv);
                uint16_t o8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o8[e] = silu_mul1(g8[e], u8[e]);
                *reinterpret_cast<uint4 *>(y + (int64_t)row * F + (int64_t)ct * 64 + jg) = __builtin_bit_cast(uint4, o8);
            }
        }
    };
    if constexpr (GRP == 1) {
        if constexpr (EPI != EPI_Y) __syncthreads();   // every wave is done reading the x ring
        store_y(h);
    } else {
        // Group sums go to the workspace as 16-byte records, m-major: record
        // (tile, group, wave, m) holds lane l's four values at byte 16 l.
        // Stores and loads are device scope (sc1: through to the level every
        // CU sees), so no cache-wide write-back or invalidate is needed: the
        // wait below and the barrier order this workgroup's stores before
        // thread 0 bumps the tile's counter, and the last workgroup reads the
        // sums only after it has seen the count.
        constexpr int CPOL_DEVICE = 16;            // sc1
        constexpr int REC = MT * kWave * 16;       // bytes per (group, wave)
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(part + (int64_t)ct * GRP * P * (REC / 4), (short)0, GRP * P * REC, 0x00020000);
#pragma unroll
        for (int m = 0; m < MT; ++m)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, h[m]), rsrc,
                                                   (grp * P + wave) * REC + m * kWave * 16 + lane * 16, 0, CPOL_DEVICE);
        __builtin_amdgcn_s_waitcnt(0);             // every store of this wave acknowledged
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(&counters[ct], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (unsigned)(GRP - 1);
        }
        __syncthreads();
        if (!s_last) return;
        if (threadIdx.x == 0) __hip_atomic_store(&counters[ct], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f32x4 out[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f32x4 v[GRP];
#pragma unroll
            for (int q = 0; q < GRP; ++q)
                v[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rsrc, (q * P + wave) * REC + m * kWave * 16 + lane * 16, 0, CPOL_DEVICE));
            if constexpr (GRP == 2) out[m] = v[0] + v[1];
            else if constexpr (GRP == 4) out[m] = (v[0] + v[1]) + (v[2] + v[3]);
            else out[m] = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
        }
        store_y(out);
    }
}

// Workspace of the slot-group form: a fixed counter area (one counter per
// column tile, room for kSlotMaxTiles tiles, left zero by every call) followed
// by the group sums.  The counter area has the same place and size for every
// shape, so the group sums of one call never land on the counters of another
// call that shares the workspace.
constexpr int64_t kSlotTileCols = kDenseWaves * 16;
constexpr int64_t kSlotMaxTiles = 16384;                    // N up to 2^21 columns
constexpr size_t kSlotCounterBytes = kSlotMaxTiles * sizeof(unsigned);

static int slot_mt(int64_t M) { return M <= 32 ? 2 : 4; }

static size_t slot_ws_bytes(int64_t M, int64_t N, int groups)
{
    const int64_t rec = (int64_t)slot_mt(M) * 4 * kWave * (int64_t)sizeof(float);
    return kSlotCounterBytes + (size_t)(cdiv(N, kSlotTileCols) * groups * kDenseWaves * rec);
}

template <typename S, int MT, int Q, int EPI>
static void launch_slots_t(const void *x, const void *w, void *y, void *ws, int64_t M, int64_t N, int64_t K,
                           hipStream_t st)
{
    using T = typename S::store_t;
    const int64_t ntc = cdiv(N, kSlotTileCols);
    unsigned *counters = (unsigned *)ws;
    float *part = (float *)((char *)ws + kSlotCounterBytes);
    // W ring depth and waves per SIMD: two workgroups per CU (at most 128
    // VGPRs) wherever the accumulators allow it.
    constexpr int DW = MT == 4 ? 2 : 4;
    constexpr int OCC = Q * MT <= 4 ? 4 : 2;
    launch_kernel((dense_slots_kernel<S, MT, Q, DW, OCC, EPI>), dim3((unsigned)ntc, (unsigned)(kDenseWaves / Q)),
                       dim3(kDenseWaves * kWave), 0, st, (const T *)x, (const T *)w, (T *)y, part, counters, M, N, K);
}

// Slots per workgroup: the largest group that still gives at least one
// workgroup per CU (MT = 4 keeps at most four slots in registers).
template <typename S, int MT, int EPI>
static void launch_slots_mt(const void *x, const void *w, void *y, void *ws, int64_t M, int64_t N, int64_t K,
                            hipStream_t st)
{
    const int64_t ntc = cdiv(N, kSlotTileCols), cu = device_cu_count();
    // All eight slots in one workgroup (no exchange) once the column tiles
    // alone come close to one per CU.
    if (ntc * 4 >= cu * 3) {
        launch_slots_t<S, MT, 8, EPI>(x, w, y, ws, M, N, K, st);
        return;
    }
    if (ntc * 2 >= cu) launch_slots_t<S, MT, 4, EPI>(x, w, y, ws, M, N, K, st);
    else if (ntc * 4 >= cu) launch_slots_t<S, MT, 2, EPI>(x, w, y, ws, M, N, K, st);
    else launch_slots_t<S, MT, 1, EPI>(x, w, y, ws, M, N, K, st);
}

template <typename S, int EPI = EPI_Y>
static bool try_launch_slots(const void *x, const void *w, void *y, void *ws, size_t ws_bytes, int64_t M,
                             int64_t N, int64_t K, hipStream_t st)
{
    using G = DenseGeom<S>;
    // M <= 16: x is small, and bi_matmul's one-workgroup-per-tile kernel,
    // which needs no exchange of partial sums, streams W faster.
    if (!ws || M <= 16 || M > 64 || K % G::KB != 0 || !host_aligned16(x) || !host_aligned16(w) ||
        !host_aligned16(ws))
        return false;
    if (ws_bytes < slot_ws_bytes(M, N, kDenseWaves)) return false;
    if (slot_mt(M) == 2) launch_slots_mt<S, 2, EPI>(x, w, y, ws, M, N, K, st);
    else launch_slots_mt<S, 4, EPI>(x, w, y, ws, M, N, K, st);
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

// SwiGLU activation of an interleaved gate/up product (the fallback of
// bi_matmul_swiglu): in each row, columns 128 i + j and 128 i + 64 + j are
// gate and up of activation 64 i + j.  Thread = 8 consecutive activations.
__global__ void swiglu_il_kernel(const uint16_t *__restrict__ gu, uint16_t *__restrict__ a, int64_t rows, int64_t F)
{
    const int64_t fc = F / 8, n = rows * fc;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = c / fc, i = (c - r * fc) * 8;
        const uint16_t *gp = gu + r * 2 * F + (i / 64) * 128 + (i % 64);
        const uint4 gv = *reinterpret_cast<const uint4 *>(gp), uv = *reinterpret_cast<const uint4 *>(gp + 64);
        const uint16_t *g8 = reinterpret_cast<const uint16_t *>(&gv), *u8 = reinterpret_cast<const uint16_t *>(&uv);
        uint16_t o8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = silu_mul1(g8[e], u8[e]);
        *reinterpret_cast<uint4 *>(a + r * F + i) = __builtin_bit_cast(uint4, o8);
    }
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

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

extern "C" size_t bi_matmul_ws_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t w_transposed)
{
    if (M <= 16 || N < 1 || K < 1 || M > 64 || !w_transposed || (dtype != BI_BF16 && dtype != BI_F16) ||
        cdiv(N, kSlotTileCols) > kSlotMaxTiles)
        return 0;
    return slot_ws_bytes(M, N, kDenseWaves);
}

extern "C" bi_status bi_matmul_ws(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                                  int32_t dtype, int32_t w_transposed, void *ws, size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_dense(x, w, y, M, N, K, dtype);
    if (s != BI_OK) return s;
    const size_t need = bi_matmul_ws_workspace_bytes(M, N, K, dtype, w_transposed);
    if (need > 0 && (!ws || ws_bytes < need)) return BI_ERR_WORKSPACE;
    if (need > 0 && !host_aligned16(ws)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    bool done = false;
    if (need > 0) {
        if (dtype == BI_BF16) done = try_launch_slots<BF16>(x, w, y, ws, ws_bytes, M, N, K, stream);
        else done = try_launch_slots<F16>(x, w, y, ws, ws_bytes, M, N, K, stream);
    }
    if (!done) dispatch_dense(x, w, y, nullptr, M, N, K, dtype, w_transposed != 0, 1, stream);
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
    if (dtype == BI_BF16) launch_kernel(split_reduce_kernel<BF16>, dim3(blocks), dim3(256), 0, stream, part, (uint16_t *)y, MN, splits);
    else if (dtype == BI_F16) launch_kernel(split_reduce_kernel<F16>, dim3(blocks), dim3(256), 0, stream, part, (uint16_t *)y, MN, splits);
    else launch_kernel(split_reduce_kernel<F32>, dim3(blocks), dim3(256), 0, stream, part, (float *)y, MN, splits);
    return launch_status();
}

extern "C" bi_status bi_time_next_launch(hipEvent_t start, hipEvent_t stop)
{
    bi::launch_timing() = bi::LaunchTiming{start, stop};
    return BI_OK;
}

extern "C" size_t bi_matmul_swiglu_workspace_bytes(int64_t M, int64_t F, int64_t K, int32_t dtype)
{
    if (M < 1 || F < 1 || K < 1 || dtype != BI_BF16 || F % 64 || M > (1ll << 31) || F > (1ll << 30)) return 0;
    // the slot form's counter area, then its group sums or (any other shape)
    // the scratch product: never both in one call
    const size_t slot = bi_matmul_ws_workspace_bytes(M, 2 * F, K, dtype, 1);
    const size_t prod = align256((size_t)M * (size_t)(2 * F) * sizeof(uint16_t));
    return kSlotCounterBytes + std::max(slot > 0 ? slot - kSlotCounterBytes : 0, prod);
}

extern "C" bi_status bi_matmul_swiglu(const void *x, const void *w_il, void *a, int64_t M, int64_t F, int64_t K,
                                      int32_t dtype, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (F < 1 || F > (1ll << 30)) return BI_ERR_SHAPE;
    bi_status s = check_dense(x, w_il, a, M, 2 * F, K, dtype);
    if (s != BI_OK) return s;
    if (dtype != BI_BF16) return BI_ERR_DTYPE;
    if (F % 64) return BI_ERR_SHAPE;
    if (!host_aligned16(a)) return BI_ERR_ALIGN;
    const size_t need = bi_matmul_swiglu_workspace_bytes(M, F, K, dtype);
    if (!ws || ws_bytes < need) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    const size_t slot = bi_matmul_ws_workspace_bytes(M, 2 * F, K, dtype, 1);
    (void)hipGetLastError();
    if (slot > 0 && try_launch_slots<BF16, EPI_SWIGLU>(x, w_il, a, ws, slot, M, 2 * F, K, stream)) return launch_status();
    // any other shape: the product into the scratch after the counter area
    // (which stays zero for later slot-form calls on this workspace), then
    // the activation
    uint16_t *gu = (uint16_t *)((char *)ws + kSlotCounterBytes);
    dispatch_dense(x, w_il, gu, nullptr, M, 2 * F, K, dtype, true, 1, stream);
    const int64_t n = M * F / 8;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(n, 256), 65536);
    hipLaunchKernelGGL(swiglu_il_kernel, dim3(blocks), dim3(256), 0, stream, (const uint16_t *)gu, (uint16_t *)a, M, F);
    return launch_status();
}
