// qmatmul_wide.hip -- batch-invariant group-quantized matmul on gfx950 for the
// code widths beyond the 4-bit formats: affine codes of 2 to 8 bits (other
// than 4) and mxfp8 (OCP e4m3 codes, one e8m0 scale per 32).
//
// Sources: "Fix fp quantized matmul corruption when the quantized dim is not a
// multiple of 32" (Validation: the differential campaign over affine codes of
// 2 to 8 bits at group sizes 32/64/128 and the mx and nv fp formats; Fix:
// mxfp8's group size is 32, a multiple of the K tile, so no group is cut by a
// K remainder); "Fix/speculative shape invariance" (Problem: the quantized
// matmul must not pick its reduction by M).
//
// What is computed: W is dequantized in registers to binary16 --
//   affine: w = RNE16(fma(s, q, b)) with binary16 s, b (s*q is exact in fp32,
//           at most 11 + 8 significant bits, so the fma rounds once, exactly
//           like mul-then-add);
//   mxfp8 : w = RNE16(e4m3(q) * 2^(e - 127)), the exact product rounded once
//           (the e4m3 decode is the hardware's OCP conversion, checked for
//           every code at every scale against the oracle) --
// and multiplied against binary16 x by the K tree of the 4-bit kernels: blocks
// of 128 owned by wave b mod 8, lane group g supplying [32g, 32g + 32) of a
// block as four v_mfma_f32_16x16x32_f16 steps, wave partials added in wave
// order, RNE to binary16.  Group sizes are at least 32, so a lane's 32 codes
// of a block share one group.  M, the M tile and the column tiling are free.
//
// Codes: every stored row is a little-endian bit stream of BITS-bit codes in
// 32-bit words, so in the transposed layout a lane's 32 codes are exactly
// BITS consecutive words.  In the natural layout column n's code in row k
// starts at stream bit n * BITS of row k and may straddle two words.
//
// Packed layout (bi_pack_qweights, K % 128 == 0): the 4-bit layout with BITS
// words per lane -- for row group r and K block b, 64 lanes x BITS words in
// MFMA lane order at word ((r * nb + b) * 64 + lane) * BITS (lane 16g + c:
// row 16r + c, k in [128b + 32g, +32)), then after all code chunks one
// constants chunk per (r, b) as in the 4-bit layout.
//
// Bounds: transposed K is a multiple of the group size (>= 32), so a lane's 32
// codes lie wholly below K or wholly at/after it; natural K is arbitrary and a
// code at k >= K is not read; columns n >= N read nothing and store nothing.
#include <algorithm>

#include "qmatmul_common.hpp"

namespace bi {

// Code e (0..31; a compile-time constant once unrolled) of a lane's words.
template <int BITS>
__device__ inline uint32_t wcode(const uint32_t (&w)[BITS], int e)
{
    const int o = e * BITS, i = o >> 5, sh = o & 31;
    uint32_t v = w[i] >> sh;
    if (sh + BITS > 32) v |= w[i + 1] << (32 - sh);
    return v & ((1u << BITS) - 1u);
}

// The BITS words of a lane: 16-byte loads when BITS % 4 == 0, 8-byte ones when
// BITS is even (the offsets are multiples of those sizes whenever wq is
// 16-byte aligned and K % 32 == 0), else single words.
template <int BITS>
__device__ inline void load_words(uint32_t (&w)[BITS], const uint32_t *src, bool vec)
{
    if (vec && BITS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 4; ++i) {
            const uint4 v = reinterpret_cast<const uint4 *>(src)[i];
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    } else if (vec && BITS % 2 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) {
            const uint2 v = reinterpret_cast<const uint2 *>(src)[i];
            w[2 * i] = v.x; w[2 * i + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[i] = src[i];
    }
}

// Group constants from the raw scale (and bias) a lane loaded.
template <int QM>
__device__ inline void wgroup(uint32_t sc, uint32_t bs, float &s, float &b)
{
    if constexpr (QM == BI_MXFP8) {
        s = e8m0_to_f32(sc);
        b = 0.0f;
    } else {
        s = F16::widen((uint16_t)sc);
        b = F16::widen((uint16_t)bs);
    }
}

template <int QM>
__device__ inline void load_raw_group(const void *scales, const uint16_t *biases, int64_t gi, uint32_t &sc,
                                      uint32_t &bs)
{
    if constexpr (QM == BI_MXFP8) {
        sc = ((const uint8_t *)scales)[gi];
        bs = 0;
    } else {
        sc = ((const uint16_t *)scales)[gi];
        bs = biases[gi];
    }
}

// Lane (g, c)'s words and raw group constants of row group rg, block b in the
// packed layout (gshift = log2 gs).
template <int QM, int BITS>
__device__ inline void load_packed(const uint32_t *wqp, int64_t nrg, int64_t nb, int64_t rg, int64_t b, int lane,
                                   int gshift, uint32_t (&w)[BITS], uint32_t &sc, uint32_t &bs)
{
    const int g = lane >> 4, c = lane & 15, gpb = 128 >> gshift;
    load_words<BITS>(w, wqp + ((rg * nb + b) * 64 + lane) * BITS, true);
    const uint8_t *cb = reinterpret_cast<const uint8_t *>(wqp) + nrg * nb * 256 * BITS +
                        (rg * nb + b) * (int64_t)(16 * gpb * (QM == BI_MXFP8 ? 1 : 4));
    const int ei = c * gpb + ((32 * g) >> gshift);
    if constexpr (QM == BI_MXFP8) {
        sc = cb[ei];
        bs = 0;
    } else {
        const uint32_t v = reinterpret_cast<const uint32_t *>(cb)[ei];
        sc = v & 0xffffu;
        bs = v >> 16;
    }
}

// Codes 8s .. 8s + 7 of a lane's 32 -> one 16-byte MFMA operand chunk.
//   affine: code -> fp32 (exact), fma(s, q, b), pairs rounded to binary16 by
//           one packed conversion;
//   mxfp8 : two codes at a time to fp32 by the OCP e4m3 conversion
//           (v_cvt_pk_f32_fp8: exact, NaN codes give NaN), times the scale
//           2^(e - 127) -- exact in fp32, or +-inf where binary16 overflows
//           anyway, and where fp32 is subnormal binary16 rounds to zero
//           anyway -- then rounded once to binary16.
template <int QM, int BITS>
__device__ inline uint4 wdeq8(const uint32_t (&w)[BITS], int s, float gsv, float gbv)
{
    uint32_t out[4];
    if constexpr (QM == BI_MXFP8) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int word = (int)w[2 * s + (p >> 1)];
            const f32x2 e = (p & 1) ? __builtin_amdgcn_cvt_pk_f32_fp8(word, true)      // codes 2p, 2p + 1
                                    : __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            const f32x2 v = e * gsv;
            out[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float q0 = (float)wcode<BITS>(w, 8 * s + 2 * p), q1 = (float)wcode<BITS>(w, 8 * s + 2 * p + 1);
            const f32x2 v = f32x2{__builtin_fmaf(gsv, q0, gbv), __builtin_fmaf(gsv, q1, gbv)};
            out[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
        }
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// One code of the natural layout -> binary16 bits (the same value wdeq8 gives).
template <int QM>
__device__ inline uint16_t wdeq1(uint32_t q, uint32_t sc, uint32_t bs)
{
    if constexpr (QM == BI_MXFP8) {
        return F16::narrow(e4m3_to_f32(q) * e8m0_to_f32(sc));
    } else {
        return F16::narrow(__builtin_fmaf(F16::widen((uint16_t)sc), (float)q, F16::widen((uint16_t)bs)));
    }
}

// General form: any M (tiles of 16*MT rows), 16 columns per workgroup, either
// layout.  gshift = log2(group size).
template <int QM, int BITS, bool TRANS, int MT, bool PK>
__global__ __launch_bounds__(kQWaves * kWave)
void qwide_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ wq, const void *__restrict__ scales,
                  const uint16_t *__restrict__ biases, uint16_t *__restrict__ y, int64_t M, int64_t N, int64_t K,
                  int gshift, int wvec)
{
    constexpr int P = kQWaves, TR = MT * 16, TC = 16;
    __shared__ float red[P][TR][TC + 1];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * TC, m0 = (int64_t)blockIdx.y * TR;
    const int64_t nblocks = cdiv(K, kQBlock);
    const bool xvec = (K % 8) == 0 && aligned16(x);
    const int64_t n = n0 + c;
    const bool nok = n < N;

    f32x4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t r = m0 + i * 16 + c;
        xok[i] = r < M;
        xrow[i] = x + (xok[i] ? r : 0) * K;
    }

    for (int64_t b = wave; b < nblocks; b += P) {
        const int64_t kbase = b * kQBlock + (int64_t)g * 32;
        uint4 Bf[4];
        if constexpr (PK) {
            // K % 128 == 0: every block is whole; padding rows of the group are zeros
            uint32_t w[BITS], sc, bs;
            load_packed<QM, BITS>(wq, cdiv(N, 16), nblocks, (int64_t)blockIdx.x, b, lane, gshift, w, sc, bs);
            float gsv, gbv;
            wgroup<QM>(sc, bs, gsv, gbv);
#pragma unroll
            for (int s = 0; s < 4; ++s) Bf[s] = wdeq8<QM, BITS>(w, s, gsv, gbv);
        } else if constexpr (TRANS) {
            if (nok && kbase < K) {
                const int64_t wpr = K / 32 * BITS;
                uint32_t w[BITS];
                load_words<BITS>(w, wq + n * wpr + (kbase / 32) * BITS, wvec != 0);
                uint32_t sc, bs;
                load_raw_group<QM>(scales, biases, n * (K >> gshift) + (kbase >> gshift), sc, bs);
                float gsv, gbv;
                wgroup<QM>(sc, bs, gsv, gbv);
#pragma unroll
                for (int s = 0; s < 4; ++s) Bf[s] = wdeq8<QM, BITS>(w, s, gsv, gbv);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) Bf[s] = make_uint4(0, 0, 0, 0);
            }
        } else {
            const int64_t wpr = N / 32 * BITS, groups = N >> gshift;
            const int64_t bit = n * BITS, wi = bit >> 5;
            const int sh = (int)(bit & 31);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                uint16_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int64_t k = kbase + s * 8 + e;
                    h[e] = 0;
                    if (nok && k < K) {
                        const uint32_t *row = wq + k * wpr;
                        uint32_t v = row[wi] >> sh;
                        if (sh + BITS > 32) v |= row[wi + 1] << (32 - sh);   // the code ends inside the row
                        uint32_t sc, bs;
                        load_raw_group<QM>(scales, biases, k * groups + (n >> gshift), sc, bs);
                        h[e] = wdeq1<QM>(v & ((1u << BITS) - 1u), sc, bs);
                    }
                }
                Bf[s] = __builtin_bit_cast(uint4, h);
            }
        }
        uint4 A[MT][4];
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                A[i][s] = xvec ? load_chunk<F16, true>(xrow[i], kbase + s * 8, K, xok[i])
                               : load_chunk<F16, false>(xrow[i], kbase + s * 8, K, xok[i]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] = qmfma(A[i][s], Bf[s], acc[i]);
    }

#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][i * 16 + g * 4 + r][c] = acc[i][r];
    __syncthreads();
    for (int o = threadIdx.x; o < TR * TC; o += P * kWave) {
        const int r = o / TC, cc = o % TC;
        const int64_t row = m0 + r, col = n0 + cc;
        if (row >= M || col >= N) continue;
        float v = red[0][r][cc];
#pragma unroll
        for (int p = 1; p < P; ++p) v = v + red[p][r][cc];
        y[row * N + col] = F16::narrow(v);
    }
}

// Persistent streaming form for short M (at most 16 rows), transposed
// weights, K % 128 == 0 and 16-byte aligned x: a fixed grid walks the output
// tiles (16 rows x NS*16 columns) t = blockIdx.x, blockIdx.x + gridDim.x, ...;
// each wave streams its (tile, block) items -- a lane's code words, group
// constants and x chunks -- through a D-deep register ring that runs across
// tile boundaries.  Per output the tree is qwide_kernel's.
template <int QM, int BITS, int NS, int D, bool PK>
__global__ __launch_bounds__(kQWaves * kWave, 2)
void qwide_stream_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ wq,
                         const void *__restrict__ scales, const uint16_t *__restrict__ biases,
                         uint16_t *__restrict__ y, int64_t M, int64_t N, int64_t K, int ntn, int gshift, int wvec)
{
    constexpr int P = kQWaves, TC = NS * 16;
    __shared__ float red[P][16][TC + 1];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int nb = (int)(K / kQBlock);
    const int nmine = wave < nb ? (nb - wave + P - 1) / P : 0;        // blocks of this wave per tile
    const int mytiles = (int)blockIdx.x < ntn ? (ntn - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    const int items = mytiles * nmine;
    const int64_t wpr = K / 32 * BITS, groups = K >> gshift;
    // x row of A-operand row c; rows >= M are not loaded and never stored
    const uint16_t *xr = x + (int64_t)(c < M ? c : M - 1) * K;

    uint32_t Wr[D][NS][BITS];
    uint4 Xr[D][4];
    uint32_t Sr[D][NS], Br[D][NS];
    // prefetch cursor: item (pu, pj) = block wave + pj*P of tile pu; holds at the last item
    int pu = 0, pj = 0;
    auto load_next = [&](uint32_t (&Wd)[NS][BITS], uint32_t (&Sd)[NS], uint32_t (&Bd)[NS], uint4 (&Xd)[4]) {
        const int64_t t = (int64_t)blockIdx.x + (int64_t)pu * gridDim.x;
        const int64_t kb = (int64_t)(wave + pj * P) * kQBlock + g * 32;     // this lane's first code
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if constexpr (PK) {
                const int64_t nrg = (N + 15) / 16, rg = t * NS + j;
                load_packed<QM, BITS>(wq, nrg, nb, rg < nrg ? rg : nrg - 1, wave + pj * P, lane, gshift, Wd[j], Sd[j],
                                      Bd[j]);
            } else {
                int64_t n = t * TC + j * 16 + c;
                n = n < N ? n : N - 1;                                      // padding columns read a real row
                load_words<BITS>(Wd[j], wq + n * wpr + (kb / 32) * BITS, wvec != 0);
                load_raw_group<QM>(scales, biases, n * groups + (kb >> gshift), Sd[j], Bd[j]);
            }
        }
        if (c < M) {
#pragma unroll
            for (int s = 0; s < 4; ++s) Xd[s] = *reinterpret_cast<const uint4 *>(xr + kb + s * 8);
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) Xd[s] = make_uint4(0, 0, 0, 0);
        }
        if (pj + 1 < nmine) {
            ++pj;
        } else if (pu + 1 < mytiles) {
            pj = 0;
            ++pu;
        }
    };
    f32x4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto finish_tile = [&](int u) {
#pragma unroll
        for (int j = 0; j < NS; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][g * 4 + r][j * 16 + c] = acc[j][r];
            acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();
        const int64_t n0 = ((int64_t)blockIdx.x + (int64_t)u * gridDim.x) * TC;
        for (int o = threadIdx.x; o < 16 * TC; o += P * kWave) {
            const int r = o / TC, cc = o % TC;
            const int64_t col = n0 + cc;
            if (r >= M || col >= N) continue;
            float v = red[0][r][cc];
#pragma unroll
            for (int p = 1; p < P; ++p) v = v + red[p][r][cc];
            y[(int64_t)r * N + col] = F16::narrow(v);
        }
        __syncthreads();
    };

    if (items > 0) {
        int cu = 0, cj = 0;
        static_for<0, D - 1>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            load_next(Wr[d], Sr[d], Br[d], Xr[d]);
        });
        for (int i = 0; i < items; i += D) {
            static_for<0, D>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                constexpr int dn = (d + D - 1) % D;
                load_next(Wr[dn], Sr[dn], Br[dn], Xr[dn]);
                __builtin_amdgcn_sched_barrier(0);
                if (i + d < items) {
                    float gsv[NS], gbv[NS];
#pragma unroll
                    for (int j = 0; j < NS; ++j) wgroup<QM>(Sr[d][j], Br[d][j], gsv[j], gbv[j]);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
#pragma unroll
                        for (int j = 0; j < NS; ++j)
                            acc[j] = qmfma(Xr[d][s], wdeq8<QM, BITS>(Wr[d][j], s, gsv[j], gbv[j]), acc[j]);
                    if (++cj == nmine) {
                        finish_tile(cu);
                        cj = 0;
                        ++cu;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    } else {
        // a wave that owns no block of K still takes part in every combine
        for (int u = 0; u < mytiles; ++u) finish_tile(u);
    }
}

template <int QM, int BITS, bool TRANS, int MT, bool PK = false>
static void launch_qw_t(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                        int64_t N, int64_t K, int gshift, int wvec, hipStream_t st)
{
    dim3 grid((unsigned)cdiv(N, 16), (unsigned)cdiv(M, MT * 16));
    launch_kernel((qwide_kernel<QM, BITS, TRANS, MT, PK>), grid, dim3(kQWaves * kWave), 0, st, (const uint16_t *)x, wq,
                  s, (const uint16_t *)b, (uint16_t *)y, M, N, K, gshift, wvec);
}

template <int QM, int BITS, int NS, bool PK>
static void launch_qw_stream(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                             int64_t N, int64_t K, int gshift, int wvec, hipStream_t st)
{
    constexpr int D = BITS >= 6 ? 2 : 3;                 // register ring depth: wide codes hold more words
    const int64_t ntn = cdiv(N, NS * 16);
    const int64_t grid = std::min<int64_t>(ntn, (int64_t)device_cu_count() * 2);
    launch_kernel((qwide_stream_kernel<QM, BITS, NS, D, PK>), dim3((unsigned)grid), dim3(kQWaves * kWave), 0, st,
                  (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)y, M, N, K, (int)ntn, gshift, wvec);
}

template <int QM, int BITS, bool TRANS, bool PK>
static void launch_qw_mt(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                         int64_t N, int64_t K, int gshift, int wvec, hipStream_t st)
{
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_qw_t<QM, BITS, TRANS, 1, PK>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
    else if (mt <= 2) launch_qw_t<QM, BITS, TRANS, 2, PK>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
    else launch_qw_t<QM, BITS, TRANS, 4, PK>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
}

template <int QM, int BITS>
static void launch_qw(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M, int64_t N,
                      int64_t K, int gs, int layout, hipStream_t st)
{
    const int gshift = gs == 32 ? 5 : (gs == 64 ? 6 : 7);
    const int wvec = host_aligned16(wq) ? 1 : 0;         // row and lane offsets are then multiples of the load size
    const bool stream = layout >= 1 && M <= 16 && K % kQBlock == 0 && host_aligned16(x) && cdiv(N, 16) <= (1ll << 30);
    if (stream) {
        if (layout == 2) {                               // packed: 16-byte aligned (checked)
            if (N >= 8192) launch_qw_stream<QM, BITS, 2, true>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
            else launch_qw_stream<QM, BITS, 1, true>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
        } else {
            if (N >= 8192) launch_qw_stream<QM, BITS, 2, false>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
            else launch_qw_stream<QM, BITS, 1, false>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
        }
        return;
    }
    if (layout == 2) launch_qw_mt<QM, BITS, true, true>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
    else if (layout == 1) launch_qw_mt<QM, BITS, true, false>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
    else launch_qw_mt<QM, BITS, false, false>(x, wq, s, b, y, M, N, K, gshift, wvec, st);
}

// [N, K*bits/32] codes + [N, K/gs] constants -> the packed layout; one thread
// per lane chunk of `bits` words, then one per constant entry.
template <int QM>
__global__ void pack_qwide_kernel(const uint32_t *__restrict__ wq, const void *__restrict__ scales,
                                  const uint16_t *__restrict__ biases, uint32_t *__restrict__ wqp, int64_t N,
                                  int64_t K, int bits, int gshift)
{
    const int64_t nb = K / kQBlock, nrg = (N + 15) / 16, wpr = K / 32 * bits, groups = K >> gshift;
    const int gpb = 128 >> gshift;                               // constant entries per row per block
    const int64_t ncode = nrg * nb * 64, nconst = nrg * nb * 16 * gpb;
    uint8_t *cbase = reinterpret_cast<uint8_t *>(wqp) + nrg * nb * 256 * bits;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ncode + nconst;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < ncode) {
            const int lane = (int)(i & 63);
            const int64_t rb = i >> 6, b = rb % nb, rg = rb / nb;
            const int64_t row = rg * 16 + (lane & 15);
            const uint32_t *src = wq + row * wpr + (4 * b + (lane >> 4)) * bits;
            for (int w = 0; w < bits; ++w) wqp[i * bits + w] = row < N ? src[w] : 0u;
        } else {
            const int64_t e = i - ncode, q = e % gpb, cr = e / gpb, c = cr % 16, rb = cr / 16;
            const int64_t b = rb % nb, rg = rb / nb, row = rg * 16 + c;
            const int64_t gi = row * groups + b * gpb + q;
            if constexpr (QM == BI_AFFINE) {
                const uint32_t v = row < N ? (uint32_t)((const uint16_t *)scales)[gi] | ((uint32_t)biases[gi] << 16) : 0u;
                *reinterpret_cast<uint32_t *>(cbase + e * 4) = v;
            } else {
                cbase[e] = row < N ? ((const uint8_t *)scales)[gi] : (uint8_t)0;
            }
        }
    }
}

// Expert ("gather") matmul at these widths: workgroup (t, e) owns the 16
// columns of tile t for expert e, compacts the rows routed to e (ascending, a
// slab of up to kWideGatherSlab rows at a time) into LDS and runs them 16 at a
// time through qwide_kernel's reduction, so each row has the bits of the
// plain quantized matmul of its token with its expert.  The workgroups of
// e = E write NaN to the rows whose token or expert index is out of range.
// Per expert: codes [N, K*BITS/32] (or [K, N*BITS/32]) and constants, or one
// packed buffer (PK).
constexpr int kWideGatherSlab = 4096;

template <int QM, int BITS, bool TRANS, bool PK>
__global__ __launch_bounds__(kQWaves * kWave)
void qwide_gather_kernel(const uint16_t *__restrict__ x, const int32_t *__restrict__ lhs,
                         const int32_t *__restrict__ rhs, const uint32_t *__restrict__ wq,
                         const void *__restrict__ scales, const uint16_t *__restrict__ biases,
                         uint16_t *__restrict__ y, int64_t M, int64_t x_rows, int64_t N, int64_t K, int E, int gshift)
{
    constexpr int P = kQWaves, NT = kQWaves * kWave;
    constexpr int SB = QM == BI_AFFINE ? 2 : 1;
    __shared__ float red[P][16][17];
    __shared__ int perm[kWideGatherSlab];
    __shared__ int wcnt[P];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int e = (int)blockIdx.y;
    const int64_t n0 = (int64_t)blockIdx.x * 16, n = n0 + c;
    const bool nok = n < N;
    const int64_t nblocks = cdiv(K, kQBlock), nrg = cdiv(N, 16);
    const bool xvec = (K % 8) == 0 && aligned16(x);
    const int gpb = 128 >> gshift;
    const int64_t words_e = PK ? nrg * nblocks * (64 * BITS + 4 * gpb * (QM == BI_MXFP8 ? 1 : 4))
                               : N * K / 32 * BITS;
    const int64_t groups_e = N * K >> gshift;
    const int ee = e < E ? e : 0;
    const uint32_t *we = wq + (int64_t)ee * words_e;
    const void *se = (const uint8_t *)scales + (int64_t)ee * groups_e * SB;
    const uint16_t *be = biases ? biases + (int64_t)ee * groups_e : nullptr;

    auto bucket = [&](int64_t m) -> int {
        const int64_t r = rhs[m], xr = lhs ? (int64_t)lhs[m] : m;
        return (r >= 0 && r < E && xr >= 0 && xr < x_rows) ? (int)r : E;
    };

    for (int64_t s0 = 0; s0 < M; s0 += kWideGatherSlab) {
        const int ns = (int)(M - s0 < kWideGatherSlab ? M - s0 : kWideGatherSlab);
        int found = 0;
        for (int i0 = 0; i0 < ns; i0 += NT) {
            const int i = i0 + tid;
            const bool hit = i < ns && bucket(s0 + i) == e;
            const uint64_t mask = __ballot(hit);
            if (lane == 0) wcnt[wave] = __popcll(mask);
            __syncthreads();
            int off = found, tot = 0;
#pragma unroll
            for (int w = 0; w < P; ++w) {
                const int cw = wcnt[w];
                off += w < wave ? cw : 0;
                tot += cw;
            }
            if (hit) perm[off + __popcll(mask & ((1ull << lane) - 1ull))] = i;
            found += tot;
            __syncthreads();
        }
        if (e == E) {
            for (int i = tid; i < found * 16; i += NT) {
                const int64_t col = n0 + (i & 15);
                if (col < N) y[(s0 + perm[i >> 4]) * N + col] = 0x7e00u;
            }
            __syncthreads();
            continue;
        }
        for (int r0 = 0; r0 < found; r0 += 16) {
            const int nr = found - r0 < 16 ? found - r0 : 16;
            const bool rok = c < nr;
            const int64_t m = s0 + perm[r0 + (rok ? c : 0)];
            const uint16_t *xrow = x + (lhs ? (int64_t)lhs[m] : m) * K;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int64_t b = wave; b < nblocks; b += P) {
                const int64_t kbase = b * kQBlock + (int64_t)g * 32;
                if constexpr (PK || TRANS) {
                    uint4 Bf[4];
                    uint32_t w[BITS], sc = 0, bs = 0;
                    bool have = true;
                    if constexpr (PK) {
                        load_packed<QM, BITS>(we, nrg, nblocks, (int64_t)blockIdx.x, b, lane, gshift, w, sc, bs);
                    } else {
                        have = nok && kbase < K;
                        if (have) {
                            load_words<BITS>(w, we + n * (K / 32 * BITS) + (kbase / 32) * BITS, false);
                            load_raw_group<QM>(se, be, n * (K >> gshift) + (kbase >> gshift), sc, bs);
                        }
                    }
                    if (have) {
                        float gsv, gbv;
                        wgroup<QM>(sc, bs, gsv, gbv);
#pragma unroll
                        for (int s = 0; s < 4; ++s) Bf[s] = wdeq8<QM, BITS>(w, s, gsv, gbv);
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s) Bf[s] = make_uint4(0, 0, 0, 0);
                    }
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const uint4 As = xvec ? load_chunk<F16, true>(xrow, kbase + s * 8, K, rok)
                                              : load_chunk<F16, false>(xrow, kbase + s * 8, K, rok);
                        acc = qmfma(As, Bf[s], acc);
                    }
                } else {
                    const int64_t wpr = N / 32 * BITS, groups = N >> gshift;
                    const int64_t bit = n * BITS, wi = bit >> 5;
                    const int sh = (int)(bit & 31);
#pragma unroll 1
                    for (int s = 0; s < 4; ++s) {
                        uint16_t h[8];
#pragma unroll
                        for (int ei = 0; ei < 8; ++ei) {
                            const int64_t k = kbase + s * 8 + ei;
                            h[ei] = 0;
                            if (nok && k < K) {
                                const uint32_t *row = we + k * wpr;
                                uint32_t v = row[wi] >> sh;
                                if (sh + BITS > 32) v |= row[wi + 1] << (32 - sh);
                                uint32_t sc, bs;
                                load_raw_group<QM>(se, be, k * groups + (n >> gshift), sc, bs);
                                h[ei] = wdeq1<QM>(v & ((1u << BITS) - 1u), sc, bs);
                            }
                        }
                        const uint4 As = xvec ? load_chunk<F16, true>(xrow, kbase + s * 8, K, rok)
                                              : load_chunk<F16, false>(xrow, kbase + s * 8, K, rok);
                        acc = qmfma(As, __builtin_bit_cast(uint4, h), acc);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][g * 4 + r][c] = acc[r];
            __syncthreads();
            if (tid < 256) {
                const int r = tid >> 4, cc = tid & 15;
                if (r < nr && n0 + cc < N) {
                    float v = red[0][r][cc];
#pragma unroll
                    for (int p = 1; p < P; ++p) v = v + red[p][r][cc];
                    y[(s0 + perm[r0 + r]) * N + n0 + cc] = F16::narrow(v);
                }
            }
            __syncthreads();
        }
    }
}

template <int QM, int BITS>
static void launch_qw_gather(const void *x, const int32_t *lhs, const int32_t *rhs, const uint32_t *wq, const void *s,
                             const void *b, void *y, int64_t M, int64_t x_rows, int64_t N, int64_t K, int E, int gs,
                             int layout, hipStream_t st)
{
    const int gshift = gs == 32 ? 5 : (gs == 64 ? 6 : 7);
    const dim3 grid((unsigned)cdiv(N, 16), (unsigned)(E + 1)), block(kQWaves * kWave);
    const uint16_t *xx = (const uint16_t *)x, *bz = (const uint16_t *)b;
    uint16_t *yy = (uint16_t *)y;
    if (layout == 2)
        launch_kernel((qwide_gather_kernel<QM, BITS, true, true>), grid, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                      x_rows, N, K, E, gshift);
    else if (layout == 1)
        launch_kernel((qwide_gather_kernel<QM, BITS, true, false>), grid, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                      x_rows, N, K, E, gshift);
    else
        launch_kernel((qwide_gather_kernel<QM, BITS, false, false>), grid, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                      x_rows, N, K, E, gshift);
}

}  // namespace bi

using namespace bi;

bi_status bi_qmatmul_wide(const void *x, const uint32_t *wq, const void *scales, const void *biases, void *y,
                          int64_t M, int64_t N, int64_t K, int32_t qmode, int32_t bits, int32_t group_size,
                          int32_t w_layout, hipStream_t st)
{
    if (qmode == BI_MXFP8) {
        launch_qw<BI_MXFP8, 8>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st);
    } else {
        switch (bits) {
        case 2: launch_qw<BI_AFFINE, 2>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st); break;
        case 3: launch_qw<BI_AFFINE, 3>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st); break;
        case 5: launch_qw<BI_AFFINE, 5>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st); break;
        case 6: launch_qw<BI_AFFINE, 6>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st); break;
        case 7: launch_qw<BI_AFFINE, 7>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st); break;
        case 8: launch_qw<BI_AFFINE, 8>(x, wq, scales, biases, y, M, N, K, group_size, w_layout, st); break;
        default: return BI_ERR_GROUP;
        }
    }
    return launch_status();
}

bi_status bi_pack_qweights_wide(const uint32_t *wq, const void *scales, const void *biases, void *wqp, int64_t N,
                                int64_t K, int32_t qmode, int32_t bits, int32_t group_size, hipStream_t st)
{
    const int gshift = group_size == 32 ? 5 : (group_size == 64 ? 6 : 7);
    const int64_t nrg = cdiv(N, 16), nb = K / kQBlock;
    const int64_t n = nrg * nb * 64 + nrg * nb * 16 * (128 / group_size);
    const dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), block(256);
    if (qmode == BI_MXFP8)
        launch_kernel((pack_qwide_kernel<BI_MXFP8>), grid, block, 0, st, wq, scales, (const uint16_t *)biases,
                      (uint32_t *)wqp, N, K, (int)bits, gshift);
    else
        launch_kernel((pack_qwide_kernel<BI_AFFINE>), grid, block, 0, st, wq, scales, (const uint16_t *)biases,
                      (uint32_t *)wqp, N, K, (int)bits, gshift);
    return launch_status();
}

bi_status bi_gather_qmatmul_wide(const void *x, const int32_t *lhs, const int32_t *rhs, const uint32_t *wq,
                                 const void *scales, const void *biases, void *y, int64_t M, int64_t x_rows,
                                 int64_t N, int64_t K, int64_t E, int32_t qmode, int32_t bits, int32_t group_size,
                                 int32_t w_layout, hipStream_t st)
{
    const int e = (int)E;
    if (qmode == BI_MXFP8) {
        launch_qw_gather<BI_MXFP8, 8>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st);
    } else {
        switch (bits) {
        case 2: launch_qw_gather<BI_AFFINE, 2>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st); break;
        case 3: launch_qw_gather<BI_AFFINE, 3>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st); break;
        case 5: launch_qw_gather<BI_AFFINE, 5>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st); break;
        case 6: launch_qw_gather<BI_AFFINE, 6>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st); break;
        case 7: launch_qw_gather<BI_AFFINE, 7>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st); break;
        case 8: launch_qw_gather<BI_AFFINE, 8>(x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, e, group_size, w_layout, st); break;
        default: return BI_ERR_GROUP;
        }
    }
    return launch_status();
}
