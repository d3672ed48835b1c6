// dense_common.hpp -- the frozen reduction tree and operand layout shared by
// the dense matmul kernels (dense.hip, dense_slots.hip) on gfx950 MFMA.
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
#pragma once
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

// Weight layouts (the w_layout argument of the dense entry points).
enum WLayout { W_NATURAL = 0, W_TRANS = 1, W_PACKED = 2 };

// Tile-packed weight (W_PACKED; 16-bit types, K a multiple of 128).  The
// fragment one wave multiplies for one block -- rows 16r .. 16r + 15 (row
// group r; rows >= N are zero) by k in [128b, 128b + 128) -- is 4 KiB of
// contiguous memory, in the order the MFMA consumes it: step s, then lane
// l = 16g + c, then the 8 elements W[16r + c][128b + 32s + 8g + e].  A load
// instruction of a wave then reads 1 KiB in one piece and the four of a block
// read one 4 KiB piece, where the [N, K] layout gives 16 pieces of 256 bytes
// 2 K bytes apart (far fewer DRAM pages touched per byte streamed).  The lane
// that loads an element is the lane that multiplies it, as in [N, K], so the
// tree is the same.
__host__ __device__ constexpr int64_t packed_off(int64_t rg, int64_t nb, int64_t b, int s, int lane)
{
    return (((rg * nb + b) * 4 + s) * 64 + lane) * 8;
}

inline bi_status check_dense(const void *x, const void *w, const void *y, int64_t M, int64_t N, int64_t K,
                             int32_t dtype, int32_t layout)
{
    if (!x || !w || !y) return BI_ERR_NULL;
    if (M < 1 || N < 1 || K < 1 || M > (1ll << 31) || N > (1ll << 31) || K > (1ll << 31)) return BI_ERR_SHAPE;
    if (dtype != BI_BF16 && dtype != BI_F16 && dtype != BI_F32) return BI_ERR_DTYPE;
    if (layout != W_NATURAL && layout != W_TRANS && layout != W_PACKED) return BI_ERR_SHAPE;
    const size_t esz = dtype == BI_F32 ? 4 : 2;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & (esz - 1)) return BI_ERR_ALIGN;
    if (layout == W_PACKED) {
        if (dtype == BI_F32) return BI_ERR_DTYPE;
        if (K % 128) return BI_ERR_SHAPE;
        if (((uintptr_t)w & 15) || ((uintptr_t)x & 15)) return BI_ERR_ALIGN;
    }
    return BI_OK;
}

// Plain dense launch (dense.hip): every shape and layout, bi_matmul's kernels.
void dispatch_dense(const void *x, const void *w, void *y, float *part, int64_t M, int64_t N, int64_t K,
                    int32_t dtype, int32_t layout, int splits, hipStream_t st);

// The LDS-tiled form for M > 64 (dense_tile.hip): 16-bit types, transposed or
// packed W, K % 128 == 0 and K >= 1024, x and W 16-byte aligned, M, N, K < 2^31.
template <typename S>
void launch_dense_tile(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, bool packed,
                       hipStream_t st);

// The slot form over 64-row chunks for 64 < M <= kSlotRowsMax
// (dense_slots.hip): 16-bit types, transposed or packed W, K % 128 == 0, x
// and W 16-byte aligned, N, K < 2^30.
constexpr int64_t kSlotRowsMax = 512;
template <typename S>
void launch_dense_slot_rows(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, bool packed,
                            hipStream_t st);

}  // namespace bi
