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
#include "dense_common.hpp"

#include <algorithm>

namespace bi {

// One workgroup: output tile of MT*16 rows x NS*16 columns, kDenseWaves waves.
// blockIdx.z selects a K range for the split comparison variant (splits > 1,
// partials written to `part` as fp32 [splits, M, N]); the invariant path runs
// with splits == 1 and part == nullptr.
template <typename S, bool TRANS, bool VEC, int MT, int NS, bool PART, bool PK>
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
    int64_t wcol[NS], wrg[NS];
    bool wok[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int64_t n = n0 + j * 16 + c;
        wok[j] = n < N;
        wcol[j] = wok[j] ? n : N - 1;
        const int64_t rg = n0 / 16 + j, nrg = (N + 15) / 16;
        wrg[j] = rg < nrg ? rg : nrg - 1;              // packed: row group (a whole padding group reads the last one)
    }
    const int64_t nbk = K / G::KB;

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
            if constexpr (PK) {
#pragma unroll
                for (int ci = 0; ci < G::CPB; ++ci)
                    B[j][ci] = *reinterpret_cast<const uint4 *>(w + packed_off(wrg[j], nbk, b, ci, lane));
            } else if (TRANS) {
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
template <typename S, int MT, int NS, bool PK>
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
            if constexpr (PK) {
                int64_t rg = (int64_t)ptn * NS + j;
                rg = rg < (N + 15) / 16 ? rg : (N + 15) / 16 - 1;   // a padding row group reads a real one
#pragma unroll
                for (int ci = 0; ci < G::CPB; ++ci)
                    B[j][ci] = *reinterpret_cast<const uint4 *>(w + packed_off(rg, nb, wave + pj * P, ci, lane));
            } else {
                int64_t n = (int64_t)ptn * TC + j * 16 + c;
                n = n < N ? n : N - 1;                            // padding columns read a real row
                const T *wr = w + n * K + kblk;
#pragma unroll
                for (int ci = 0; ci < G::CPB; ++ci) B[j][ci] = *reinterpret_cast<const uint4 *>(wr + G::chunk_off(g, ci));
            }
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

template <typename S, bool TRANS, bool VEC, int MT, int NS, bool PK>
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
        launch_kernel((dense_kernel<S, TRANS, VEC, MT, NS, true, PK>), grid, dim3(kDenseWaves * kWave), 0, st,
                           (const T *)x, (const T *)w, (T *)y, part, M, N, K, nblocks, splits);
    else
        launch_kernel((dense_kernel<S, TRANS, VEC, MT, NS, false, PK>), grid, dim3(kDenseWaves * kWave), 0, st,
                           (const T *)x, (const T *)w, (T *)y, part, M, N, K, nblocks, splits);
}

template <typename S, bool TRANS, bool VEC, bool PK = false>
static void launch_dense_mt(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                            int64_t K, int splits, hipStream_t st)
{
    // Tile shape is free: it never changes a row's reduction.
    // Wider N tiles once there are enough of them: every workgroup re-reads its
    // rows of x, so a tile of 2x16 columns halves that traffic.
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_dense_t<S, TRANS, VEC, 1, 1, PK>(x, w, y, part, M, N, K, splits, st);
    else if (mt <= 2) launch_dense_t<S, TRANS, VEC, 2, 1, PK>(x, w, y, part, M, N, K, splits, st);
    else if (N >= 8192) launch_dense_t<S, TRANS, VEC, 4, 2, PK>(x, w, y, part, M, N, K, splits, st);
    else launch_dense_t<S, TRANS, VEC, 4, 1, PK>(x, w, y, part, M, N, K, splits, st);
}

template <typename S, int MT, int NS, bool PK>
static void launch_stream_t(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, hipStream_t st)
{
    using T = typename S::store_t;
    const int64_t ntm = cdiv(M, MT * 16), ntn = cdiv(N, NS * 16);
    const int per_cu = (MT >= 4 && NS >= 2) ? 1 : 2;             // resident workgroups per CU at the register cap
    const int64_t grid = std::min<int64_t>(ntm * ntn, (int64_t)device_cu_count() * per_cu);
    launch_kernel((dense_stream_kernel<S, MT, NS, PK>), dim3((unsigned)grid), dim3(kDenseWaves * kWave), 0, st,
                       (const T *)x, (const T *)w, (T *)y, M, N, K, ntm, ntn);
}

template <typename S, bool PK>
static bool try_launch_stream(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                              hipStream_t st)
{
    using G = DenseGeom<S>;
    if (K % G::KB != 0 || !host_aligned16(x) || !host_aligned16(w)) return false;
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_stream_t<S, 1, 1, PK>(x, w, y, M, N, K, st);
    else if (mt <= 2) launch_stream_t<S, 2, 1, PK>(x, w, y, M, N, K, st);
    else if (N >= 16384) launch_stream_t<S, 4, 4, PK>(x, w, y, M, N, K, st);
    else if (N >= 6144) launch_stream_t<S, 4, 2, PK>(x, w, y, M, N, K, st);
    else launch_stream_t<S, 4, 1, PK>(x, w, y, M, N, K, st);
    return true;
}

template <typename S>
static void launch_dense(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N,
                         int64_t K, int32_t layout, int splits, hipStream_t st)
{
    const bool plain = splits == 1 && part == nullptr;
    if constexpr (!std::is_same_v<S, F32>) {
        // long M: the LDS-tiled form (operands shared by the workgroup's
        // waves) once it has tiles for most CUs -- more than one 128-row tile,
        // or at least 192 column tiles; a single row tile of a narrow matrix
        // (a verify block of 16 sequences on a 4096-column projection) stays
        // on the streaming kernel, which spreads it over every CU
        // Up to 512 rows where the 128 x 128 tiles would fill under 5/8 of
        // the CUs (a verify block on a 4096- or 6144-column projection: 96 or
        // 144 tiles; with 224 tiles and more the tiled kernel is ahead): the
        // slot form, one workgroup per (64-column tile, 64-row chunk), all
        // eight slots in it
        if (plain && M > 64 && M <= kSlotRowsMax && cdiv(M, 128) * cdiv(N, 128) * 8 < 5 * (int64_t)device_cu_count() &&
            layout != W_NATURAL && K % 128 == 0 && host_aligned16(x) && host_aligned16(w) && N < (1ll << 30) &&
            K < (1ll << 30)) {
            launch_dense_slot_rows<S>(x, w, y, M, N, K, layout == W_PACKED, st);
            return;
        }
        if (plain && M > 64 && (M > 128 || cdiv(N, 128) >= 192) && layout != W_NATURAL && K % 128 == 0 &&
            K >= 1024 && host_aligned16(x) && host_aligned16(w) && M < (1ll << 31) && N < (1ll << 31) &&
            K < (1ll << 31)) {
            launch_dense_tile<S>(x, w, y, M, N, K, layout == W_PACKED, st);
            return;
        }
        if (layout == W_PACKED) {                  // K % 128 == 0 and 16-byte aligned operands (checked)
            if (plain && try_launch_stream<S, true>(x, w, y, M, N, K, st)) return;
            launch_dense_mt<S, true, true, true>(x, w, y, part, M, N, K, splits, st);
            return;
        }
    }
    const bool trans = layout != W_NATURAL;
    if (trans && plain && try_launch_stream<S, false>(x, w, y, M, N, K, st)) return;
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

void dispatch_dense(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N, int64_t K,
                    int32_t dtype, int32_t layout, int splits, hipStream_t st)
{
    if (dtype == BI_BF16) launch_dense<BF16>(x, w, y, part, M, N, K, layout, splits, st);
    else if (dtype == BI_F16) launch_dense<F16>(x, w, y, part, M, N, K, layout, splits, st);
    else launch_dense<F32>(x, w, y, part, M, N, K, layout, splits, st);
}

// [N, K] -> tile-packed (W_PACKED): thread = one 16-byte chunk of the packed
// buffer; rows past N are written as zeros.
__global__ void pack_weights_kernel(const uint16_t *__restrict__ w, uint16_t *__restrict__ wp, int64_t N, int64_t K)
{
    const int64_t nb = K / 128, nrg = (N + 15) / 16, n = nrg * nb * 256;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int lane = (int)(i & 63), s = (int)((i >> 6) & 3);
        const int64_t rest = i >> 8, b = rest % nb, rg = rest / nb;
        const int64_t row = rg * 16 + (lane & 15), k = b * 128 + s * 32 + (lane >> 4) * 8;
        const uint4 v = row < N ? *reinterpret_cast<const uint4 *>(w + row * K + k) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(wp + packed_off(rg, nb, b, s, lane)) = v;
    }
}

}  // namespace bi

using namespace bi;

extern "C" size_t bi_packed_weight_bytes(int64_t N, int64_t K, int32_t dtype)
{
    if (N < 1 || K < 1 || K % 128 || N > (1ll << 31) || K > (1ll << 31) || (dtype != BI_BF16 && dtype != BI_F16))
        return 0;
    return (size_t)cdiv(N, 16) * 16 * (size_t)K * 2;
}

extern "C" bi_status bi_pack_weights(const void *w, void *wp, int64_t N, int64_t K, int32_t dtype, hipStream_t stream)
{
    if (!w || !wp) return BI_ERR_NULL;
    if (dtype != BI_BF16 && dtype != BI_F16) return BI_ERR_DTYPE;
    if (bi_packed_weight_bytes(N, K, dtype) == 0) return BI_ERR_SHAPE;
    if (!host_aligned16(w) || !host_aligned16(wp)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    const int64_t chunks = cdiv(N, 16) * (K / 128) * 256;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(chunks, 256), 65536);
    launch_kernel(pack_weights_kernel, dim3(blocks), dim3(256), 0, stream, (const uint16_t *)w, (uint16_t *)wp, N, K);
    return launch_status();
}

extern "C" bi_status bi_matmul(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                               int32_t dtype, int32_t w_layout, hipStream_t stream)
{
    bi_status s = check_dense(x, w, y, M, N, K, dtype, w_layout);
    if (s != BI_OK) return s;
    (void)hipGetLastError();
    dispatch_dense(x, w, y, nullptr, M, N, K, dtype, w_layout, 1, stream);
    return launch_status();
}

extern "C" size_t bi_matmul_split_workspace_bytes(int64_t M, int64_t N, int32_t splits)
{
    if (M < 1 || N < 1 || splits < 1) return 0;
    return (size_t)M * (size_t)N * (size_t)splits * sizeof(float);
}

extern "C" bi_status bi_matmul_split(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                                     int32_t dtype, int32_t w_layout, int32_t splits, void *ws,
                                     size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_dense(x, w, y, M, N, K, dtype, w_layout);
    if (s != BI_OK) return s;
    if (splits < 1 || splits > 1024) return BI_ERR_SHAPE;
    if (splits == 1) return bi_matmul(x, w, y, M, N, K, dtype, w_layout, stream);
    if (!ws) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    if (ws_bytes < bi_matmul_split_workspace_bytes(M, N, splits)) return BI_ERR_WORKSPACE;
    (void)hipGetLastError();
    float *part = (float *)ws;
    dispatch_dense(x, w, y, part, M, N, K, dtype, w_layout, splits, stream);
    const int64_t MN = M * N;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(MN, 256), 65536);
    if (dtype == BI_BF16) launch_kernel(split_reduce_kernel<BF16>, dim3(blocks), dim3(256), 0, stream, part, (uint16_t *)y, MN, splits);
    else if (dtype == BI_F16) launch_kernel(split_reduce_kernel<F16>, dim3(blocks), dim3(256), 0, stream, part, (uint16_t *)y, MN, splits);
    else launch_kernel(split_reduce_kernel<F32>, dim3(blocks), dim3(256), 0, stream, part, (float *)y, MN, splits);
    return launch_status();
}

extern "C" bi_status bi_time_next_launch(hipEvent_t start, hipEvent_t stop)
{
    bi::launch_timing() = bi::LaunchTiming{start, stop, (start || stop) ? 1 : 0};
    return BI_OK;
}

extern "C" bi_status bi_time_next_launches(hipEvent_t start, hipEvent_t stop, int32_t count)
{
    if (count < 0) return BI_ERR_SHAPE;
    bi::launch_timing() = bi::LaunchTiming{start, stop, count};
    return BI_OK;
}

