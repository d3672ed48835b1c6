// qmatmul_common.hpp -- pieces shared by the group-quantized matmul kernels
// (qmatmul.hip: the 4-bit formats; qmatmul_wide.hip: affine codes of 2 to 8
// bits and mxfp8).  Both run one reduction tree over K: blocks of 128, block b
// owned by wave b mod 8 of an 8-wave workgroup, lane group g of a wave
// supplying elements [32g, 32g + 32) of a block as four
// v_mfma_f32_16x16x32_f16 steps of 8, wave partials added in wave order.
#pragma once

#include "common.hpp"

namespace bi {

constexpr int kQWaves = 8;          // frozen: same K slicing as the dense kernel
constexpr int kQBlock = 128;

__device__ inline f32x4 qmfma(uint4 a, uint4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// e4m3fn byte -> fp32 (exact); S.1111.111 -> NaN.  Selects, no branches.
__device__ inline float e4m3_to_f32(uint32_t s)
{
    const uint32_t sign = (s & 0x80u) << 24, e = (s >> 3) & 0xfu, m = s & 7u;
    const uint32_t normal = sign | ((e + 120u) << 23) | (m << 20);
    const uint32_t sub = __float_as_uint((float)m * 0x1p-9f) | sign;      // subnormal m/8 * 2^-6 (exact)
    const uint32_t v = e == 0 ? sub : normal;
    return __uint_as_float((s & 0x7fu) == 0x7fu ? 0x7fc00000u : v);
}

// OCP MX e8m0 scale byte -> fp32 (exact): 2^(e - 127), 0xFF -> NaN.
__device__ inline float e8m0_to_f32(uint32_t e)
{
    const uint32_t v = e == 0 ? 0x00400000u : (e << 23);                     // 2^-127 is subnormal
    return __uint_as_float(e == 0xffu ? 0x7fc00000u : v);
}

// Bytes of one (16-row group, K block) constants chunk of the tile-packed
// layout: 16 rows x (128 / gs) entries of scale | bias << 16 (affine, 4 bytes)
// or one scale byte (the fp formats).
__host__ __device__ constexpr int qconst_chunk_bytes(int qm, int gs) { return 16 * (128 / gs) * (qm == BI_AFFINE ? 4 : 1); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

}  // namespace bi

// The wide-code entries (qmatmul_wide.hip); arguments already validated by
// bi_qmatmul / bi_pack_qweights: qmode affine with bits in 2..8 other than 4,
// or mxfp8; layout 0 (natural), 1 (transposed) or 2 (packed, K % 128 == 0).
bi_status bi_qmatmul_wide(const void *x, const uint32_t *wq, const void *scales, const void *biases, void *y,
                          int64_t M, int64_t N, int64_t K, int32_t qmode, int32_t bits, int32_t group_size,
                          int32_t w_layout, hipStream_t stream);
bi_status bi_pack_qweights_wide(const uint32_t *wq, const void *scales, const void *biases, void *wqp, int64_t N,
                                int64_t K, int32_t qmode, int32_t bits, int32_t group_size, hipStream_t stream);
bi_status bi_gather_qmatmul_wide(const void *x, const int32_t *lhs, const int32_t *rhs, const uint32_t *wq,
                                 const void *scales, const void *biases, void *y, int64_t M, int64_t x_rows,
                                 int64_t N, int64_t K, int64_t E, int32_t qmode, int32_t bits, int32_t group_size,
                                 int32_t w_layout, hipStream_t stream);
