// qmatmul.hip -- batch-invariant 4-bit group-quantized matmul on gfx950.
//
// Sources: "Fix fp quantized matmul corruption when the quantized dim is not a
// multiple of 32" (Problem: the reference is x @ dequantize(w).T and nvfp4's
// group size 16 makes K % 32 == 16 legal; The three defects and Fix: the K loop
// must stop at K, the N tail must be bounded on loads and stores, and masks
// must test rows against rows and columns against columns); "Fix/speculative
// shape invariance" (Problem: quantized matmul picked its path from M).
//
// What is computed: W is dequantized in registers to binary16 --
//   affine: w = RNE16(fma(s, q, b)) with binary16 s, b (the product s*q is
//           exact in fp32, so the fma rounds once, exactly like mul-then-add);
//   nvfp4 : w = e2m1(q) * e4m3(s), exact in fp32 and in binary16;
//   mxfp4 : w = RNE16(e2m1(q) * 2^(e - 127)), the exact product rounded once
//           (in registers by gfx950's OCP scaled fp4 conversion, checked for
//           every code at every scale byte against the oracle) --
// and multiplied against binary16 x by the same MFMA tree as the dense
// kernel: K blocks of 128, block b owned by wave b mod 8, lane group g
// supplying elements [32g, 32g + 32) of a block as four v_mfma_f32_16x16x32_f16
// steps, wave partials added in order 0..7, RNE to binary16.  The tree depends
// on K only; M, the M-tile a row falls in and the N-tile width are free.
//
// Bounds: a block that runs past K reads no packed word, scale or bias at or
// beyond K and feeds exact zeros to the MFMA; a column n >= N reads nothing and
// stores nothing.  The K % 32 == 16 shape (nvfp4) takes the word-granular path.
#include <algorithm>

#include "qmatmul_common.hpp"

namespace bi {

// e2m1 nibble -> fp32 (exact): magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6, sign in bit 3.
__device__ inline float e2m1_to_f32(uint32_t c)
{
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u);
    return __uint_as_float(((c & 8u) << 28) | mag);
}

template <int QM>
struct QGroup {                      // per-group dequantization constants
    float s, b;
};


// mxfp4 group of scale byte e: s = 2^(e - 127) in fp32 (NaN for 0xFF).
__device__ inline QGroup<BI_MXFP4> mx_group(uint32_t e)
{
    QGroup<BI_MXFP4> g;
    g.s = e8m0_to_f32(e);
    g.b = 0.0f;
    return g;
}

template <int QM>
__device__ inline QGroup<QM> load_group(const void *scales, const uint16_t *biases, int64_t gi)
{
    QGroup<QM> g;
    if constexpr (QM == BI_AFFINE) {
        g.s = F16::widen(((const uint16_t *)scales)[gi]);
        g.b = F16::widen(biases[gi]);
    } else if constexpr (QM == BI_NVFP4) {
        g.s = e4m3_to_f32(((const uint8_t *)scales)[gi]);
        g.b = 0.0f;
    } else {
        g = mx_group(((const uint8_t *)scales)[gi]);
    }
    return g;
}

// Constants of word s (of a lane's four) from the raw scale/bias a lane
// loaded: affine binary16 scale and bias; nvfp4 the two e4m3 bytes of the
// lane's two groups (words 0-1, 2-3); mxfp4 the one e8m0 byte.
template <int QM>
__device__ inline QGroup<QM> group_from_raw(uint32_t sc, uint32_t bs, int s)
{
    QGroup<QM> g;
    if constexpr (QM == BI_AFFINE) {
        g.s = F16::widen((uint16_t)sc);
        g.b = F16::widen((uint16_t)bs);
    } else if constexpr (QM == BI_NVFP4) {
        g.s = e4m3_to_f32((sc >> (s < 2 ? 0 : 8)) & 0xffu);
        g.b = 0.0f;
    } else {
        g = mx_group(sc & 0xffu);
    }
    return g;
}

// Tile-packed quantized weight (w_layout 2; transposed source, K % 128 == 0).
// Codes: for row group r (rows 16r .. 16r + 15; rows >= N zero) and K block b,
// 1 KiB in MFMA lane order -- lane l = 16g + c holds the four words of row
// 16r + c covering k in [128b + 32g, +32) -- at byte ((r * nb + b) * 64 + l) * 16.
// Group constants follow all code chunks, one chunk of qconst_chunk_bytes per
// (r, b) in the same order: 16 rows x (128 / gs) groups of, for affine,
// (scale16 | bias16 << 16), for nvfp4 and mxfp4 one scale byte.  A wave's codes
// for one block are one 1 KiB piece and its constants one piece of at most
// 256 bytes, where [N, K/8] + [N, K/gs] spread them over 16 rows each.  The
// lane that reads a code is the lane that multiplies it, as before.

// Lane (g, c)'s words and group constants of row group rg, block b (packed).
template <int QM, int GS>
__device__ inline void qload_packed_raw(const uint32_t *wqp, int64_t nrg, int64_t nb, int64_t rg, int64_t b, int lane,
                                        uint4 &words, uint32_t &sc, uint32_t &bs)
{
    const int g = lane >> 4, c = lane & 15;
    words = *reinterpret_cast<const uint4 *>(wqp + ((rg * nb + b) * 64 + lane) * 4);
    const uint8_t *cb = reinterpret_cast<const uint8_t *>(wqp) + nrg * nb * 1024 + (rg * nb + b) * qconst_chunk_bytes(QM, GS);
    if constexpr (QM == BI_AFFINE) {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(cb + (c * (128 / GS) + (32 * g) / GS) * 4);
        sc = v & 0xffffu;
        bs = v >> 16;
    } else if constexpr (QM == BI_NVFP4) {
        sc = *reinterpret_cast<const uint16_t *>(cb + c * 8 + 2 * g);   // groups 2g (low byte) and 2g + 1
        bs = 0;
    } else {
        sc = cb[c * 4 + g];                                             // the lane's one group
        bs = 0;
    }
}

template <int QM>
__device__ inline uint16_t deq1(uint32_t q, const QGroup<QM> &g)
{
    float v;
    if (QM == BI_AFFINE) v = __builtin_fmaf(g.s, (float)q, g.b);
    else v = e2m1_to_f32(q) * g.s;                 // exact in fp32 for both fp modes
    return F16::narrow(v);
}

// Eight codes of one word -> one 16-byte MFMA operand chunk (element e =
// nibble e), the same values deq1 gives:
//   affine: the nibbles are split into bytes (codes 0,2,4,6 and 1,3,5,7),
//           converted exactly to fp32, w = fma(s, q, b) in fp32, and each
//           pair rounded to binary16 (RNE) by one packed conversion;
//   nvfp4 : the e4m3 scale split as 2^E * f (f = +-1.mmm); e2m1 * 2^E by
//           the OCP scaled fp4 conversion, two codes per instruction, then one
//           packed binary16 multiply by f; both steps exact (at most 6
//           significant bits, |w| <= 2688, smallest magnitude 2^-10), so the
//           result is e2m1 * scale exactly.
// Byte p of v as fp32 (exact): one v_cvt_f32_ubyte<p>, which reads the byte in
// place (the compiler would otherwise extract each byte first).
__device__ inline float cvt_f32_ubyte(uint32_t v, int p)
{
    float f;
    switch (p) {
    case 0: asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(f) : "v"(v)); break;
    case 1: asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(f) : "v"(v)); break;
    case 2: asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(f) : "v"(v)); break;
    default: asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(f) : "v"(v)); break;
    }
    return f;
}

template <int QM>
__device__ inline uint4 deq_word(uint32_t w, const QGroup<QM> &g)
{
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    uint32_t out[4];
    if constexpr (QM == BI_AFFINE) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float q0 = cvt_f32_ubyte(lo, p), q1 = cvt_f32_ubyte(hi, p);
            const f32x2 v = f32x2{__builtin_fmaf(g.s, q0, g.b), __builtin_fmaf(g.s, q1, g.b)};
            out[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
        }
    } else if constexpr (QM == BI_MXFP4) {
        // two codes (one byte, low nibble first) at a time through the OCP
        // scaled fp4 conversion with the e8m0 scale 2^k: e2m1 * 2^k rounded
        // once to binary16
        out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, g.s, 0));
        out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, g.s, 1));
        out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, g.s, 2));
        out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, g.s, 3));
    } else {
        // scale = 2^E * f with f = +-1.mmm: e2m1 * 2^E by the OCP scaled fp4
        // conversion (exact: |e2m1 * 2^E| in [2^-10, 1536] or zero), then one
        // packed binary16 multiply by f (exact: at most 6 significant bits);
        // a NaN scale makes f NaN
        const uint32_t vb = __float_as_uint(g.s);
        const float s2 = __uint_as_float(vb & 0x7f800000u);
        const bool nan = (vb & 0x7fffffffu) > 0x7f800000u;
        const _Float16 fh = nan ? (_Float16)__uint_as_float(0x7fc00000u)
                                : (_Float16)__uint_as_float((vb & 0x807fffffu) | 0x3f800000u);
        const f16x2 fv = f16x2{fh, fh};
        out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s2, 0) * fv);
        out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s2, 1) * fv);
        out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s2, 2) * fv);
        out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s2, 3) * fv);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
}

// Transposed weights [N, K/8]: lane (g, c) of block b supplies the 32 codes of
// row n at k in [b*128 + 32g, +32) -- four consecutive words.
template <int QM, int GS, bool WVEC>
__device__ inline void qload_trans(uint4 *dst, const uint32_t *wq, const void *scales, const uint16_t *biases,
                                   int64_t n, bool nok, int64_t K, int64_t kbase)
{
    const int64_t words = K / 8, groups = K / GS;
    uint32_t w[4];
    if (WVEC) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (nok && kbase < K) v = *reinterpret_cast<const uint4 *>(wq + n * words + kbase / 8);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t k = kbase + s * 8;
            w[s] = (nok && k < K) ? wq[n * words + k / 8] : 0u;
        }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int64_t k = kbase + s * 8;
        if (nok && k < K) {
            const QGroup<QM> gr = load_group<QM>(scales, biases, n * groups + k / GS);
            dst[s] = deq_word<QM>(w[s], gr);
        } else {
            dst[s] = make_uint4(0, 0, 0, 0);
        }
    }
}

// Natural weights [K, N/8] quantized along N: column n's code at row k sits in
// word (k, n/8), nibble n % 8.  Eight consecutive k from k0 -> one operand chunk.
template <int QM, int GS>
__device__ inline uint4 qload_nat8(const uint32_t *wq, const void *scales, const uint16_t *biases, int64_t n,
                                   bool nok, int64_t N, int64_t K, int64_t k0)
{
    const int64_t words = N / 8, groups = N / GS;
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t k = k0 + e;
        if (nok && k < K) {
            const uint32_t q = (wq[k * words + n / 8] >> (4 * (n % 8))) & 15u;
            const QGroup<QM> gr = load_group<QM>(scales, biases, k * groups + n / GS);
            h[e] = deq1<QM>(q, gr);
        } else {
            h[e] = 0;
        }
    }
    return __builtin_bit_cast(uint4, h);
}

template <int QM, int GS>
__device__ inline void qload_nat(uint4 *dst, const uint32_t *wq, const void *scales, const uint16_t *biases,
                                 int64_t n, bool nok, int64_t N, int64_t K, int64_t kbase)
{
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = qload_nat8<QM, GS>(wq, scales, biases, n, nok, N, K, kbase + s * 8);
}

template <int QM, int GS, bool TRANS, bool WVEC, int MT, int NS, bool PK>
__global__ __launch_bounds__(kQWaves * kWave)
void qmatmul_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ wq, const void *__restrict__ scales,
                    const uint16_t *__restrict__ biases, uint16_t *__restrict__ y, int64_t M, int64_t N, int64_t K)
{
    constexpr int P = kQWaves;
    constexpr int TR = MT * 16, TC = NS * 16;
    __shared__ float red[P][TR][TC + 1];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * TC;
    const int64_t m0 = (int64_t)blockIdx.y * TR;
    const int64_t nblocks = cdiv(K, kQBlock);
    const bool xvec = (K % 8) == 0 && aligned16(x); // x rows 16-byte aligned: chunks never straddle K

    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t *xrow[MT];
    bool xok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t r = m0 + i * 16 + c;
        xok[i] = r < M;
        xrow[i] = x + (xok[i] ? r : 0) * K;
    }
    int64_t wn[NS];
    bool wok[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int64_t n = n0 + j * 16 + c;
        wok[j] = n < N;
        wn[j] = wok[j] ? n : 0;
    }

    for (int64_t b = wave; b < nblocks; b += P) {
        const int64_t kbase = b * kQBlock + (int64_t)g * 32;
        uint4 A[MT][4], Bf[NS][4];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if constexpr (PK) {
                // K % 128 == 0: every block is whole; padding columns multiply zeros
                const int64_t nrg = (N + 15) / 16, rg0 = n0 / 16 + j;
                uint4 wv;
                uint32_t sc, bs;
                qload_packed_raw<QM, GS>(wq, nrg, nblocks, rg0 < nrg ? rg0 : nrg - 1, b, lane, wv, sc, bs);
                const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int s = 0; s < 4; ++s) Bf[j][s] = deq_word<QM>(wa[s], group_from_raw<QM>(sc, bs, s));
            } else if (TRANS) {
                qload_trans<QM, GS, WVEC>(Bf[j], wq, scales, biases, wn[j], wok[j], K, kbase);
            } else {
                qload_nat<QM, GS>(Bf[j], wq, scales, biases, wn[j], wok[j], N, K, kbase);
            }
        }
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                A[i][s] = xvec ? load_chunk<F16, true>(xrow[i], kbase + s * 8, K, xok[i])
                               : load_chunk<F16, false>(xrow[i], kbase + s * 8, K, xok[i]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NS; ++j) acc[i][j] = qmfma(A[i][s], Bf[j][s], acc[i][j]);
    }

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
        y[row * N + col] = F16::narrow(v);
    }
}

// Streaming form for short M (at most 16 rows), the decode path, for the
// tile-packed (PK) and the [N, K/8] layouts, K a multiple of the block: one
// workgroup owns a contiguous run of output tiles (16 rows x NS*16 columns,
// the same count for every workgroup) and each wave streams its (tile, block)
// items -- NS code chunks and their group constants -- through a register
// ring.  When a wave owns at most
// kQXRes blocks of K, its x chunks are loaded once and kept in registers for
// every tile (x does not depend on the tile).  Rows >= M multiply row M - 1's
// x and are never stored (rows are independent inside an MFMA), so no load
// is predicated.  The tree is qmatmul_kernel's: block b of K belongs to wave b
// mod 8, lane group g supplies [32g, 32g + 32) of the block as four steps,
// wave partials are added in wave order.
constexpr int kQXRes = 4;

// MT > 1 (up to 64 rows): each dequantized weight word feeds MT MFMAs, one
// per row tile; one workgroup per CU (up to 256 VGPRs).  With resident x
// (XR, MT = 2) the workgroup walks its tiles once per 32 rows, with those
// rows' x chunks loaded once per pass (128 VGPRs); without, every item's x
// chunks of the MT row tiles go through the ring with the weights.
template <int QM, int GS, int NS, int D, bool XR, bool PK, bool SPL = false, int MT = 1>
__global__ __launch_bounds__(kQWaves * kWave, MT > 1 ? 1 : 2)
void qmatmul_stream_kernel(const uint16_t *__restrict__ x, const uint32_t *__restrict__ wqp,
                       const void *__restrict__ scales, const uint16_t *__restrict__ biases, uint16_t *__restrict__ y,
                       int M, int N, int K, int ntn, int per, float *__restrict__ part, int splits)
{
    static_assert(MT == 1 || !SPL, "the split variant: one row tile");
    static_assert(!XR || MT <= 2, "resident x: at most two row tiles");
    constexpr int P = kQWaves, TC = NS * 16, CB = qconst_chunk_bytes(QM, GS);
    __shared__ float red[P][16 * MT][TC + 1];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int nb = K / kQBlock, nrg = (N + 15) / 16;
    // The split comparison variant (SPL) reduces only the contiguous blocks
    // [kb0, kb1) of split blockIdx.y and writes fp32 partials; the invariant
    // kernel always covers every block.
    const int kb0 = SPL ? (int)((int64_t)blockIdx.y * nb / splits) : 0;
    const int nbl = SPL ? (int)((int64_t)(blockIdx.y + 1) * nb / splits) - kb0 : nb;
    const int nmine = wave < nbl ? (nbl - wave + P - 1) / P : 0;        // blocks of this wave per tile
    const int t0 = (int)blockIdx.x * per;
    const int ntile = max(0, min(ntn, t0 + per) - t0);
    const int items = ntile * nmine;
    // per-lane constants offset inside a (row group, block) chunk
    int coff;
    if constexpr (QM == BI_AFFINE) coff = (c * (128 / GS) + (32 * g) / GS) * 4;
    else if constexpr (QM == BI_NVFP4) coff = c * 8 + 2 * g;
    else coff = c * 4 + g;
    const uint8_t *cbase = reinterpret_cast<const uint8_t *>(wqp) + (int64_t)nrg * nb * 1024;
    int64_t xoff[MT];                                    // row tile i: row 16 i + c (padding rows read row M - 1)
#pragma unroll
    for (int i = 0; i < MT; ++i) xoff[i] = (int64_t)(16 * i + c < M ? 16 * i + c : M - 1) * K + g * 32;

    constexpr int NR = XR ? kQXRes : D;                  // ring slots
    uint4 W[NR][NS];
    uint32_t S[NR][NS];
    uint4 X[XR ? kQXRes : D][MT][4];
    // resident x of rows [rb, rb + 16 MT) (rows >= M read row M - 1)
    auto load_x_res = [&](int rb) {
#pragma unroll
        for (int j = 0; j < kQXRes; ++j)
            if (j < nmine) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int row = min(rb + 16 * i + c, M - 1);
                    const uint16_t *xp = x + (int64_t)row * K + g * 32 + (int64_t)(kb0 + wave + j * P) * kQBlock;
#pragma unroll
                    for (int s = 0; s < 4; ++s) X[j][i][s] = *reinterpret_cast<const uint4 *>(xp + s * 8);
                }
            }
    };
    int lu = 0, lj = 0;                                     // load cursor: tile t0 + lu, block wave + lj*P
    auto load_item = [&](auto dc_) {
        constexpr int d = decltype(dc_)::value;
        const int b = kb0 + wave + lj * P;
#pragma unroll
        for (int jj = 0; jj < NS; ++jj) {
            const int rg = min((t0 + lu) * NS + jj, nrg - 1);
            if constexpr (PK) {
                const int64_t chunk = (int64_t)rg * nb + b;
                W[d][jj] = *reinterpret_cast<const uint4 *>(wqp + (chunk * 64 + lane) * 4);
                const uint8_t *cp = cbase + chunk * CB + coff;
                if constexpr (QM == BI_AFFINE) S[d][jj] = *reinterpret_cast<const uint32_t *>(cp);
                else if constexpr (QM == BI_NVFP4) S[d][jj] = *reinterpret_cast<const uint16_t *>(cp);
                else S[d][jj] = *cp;
            } else {
                // [N, K/8] codes, [N, K/gs] constants; a padding row reads row N - 1
                const int64_t n = min(rg * 16 + c, N - 1);
                const int64_t kb = (int64_t)b * kQBlock + g * 32;         // this lane's first code
                W[d][jj] = *reinterpret_cast<const uint4 *>(wqp + n * (K / 8) + kb / 8);
                const int64_t gi = n * (K / GS) + kb / GS;
                if constexpr (QM == BI_AFFINE)
                    S[d][jj] = (uint32_t)((const uint16_t *)scales)[gi] | ((uint32_t)biases[gi] << 16);
                else if constexpr (QM == BI_NVFP4) S[d][jj] = ((const uint16_t *)scales)[gi / 2];   // the two group bytes
                else S[d][jj] = ((const uint8_t *)scales)[gi];
            }
        }
        if constexpr (!XR) {
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int s = 0; s < 4; ++s) X[d][i][s] = *reinterpret_cast<const uint4 *>(x + xoff[i] + b * kQBlock + s * 8);
        }
        if (++lj == nmine) {
            lj = 0;
            ++lu;
        }
    };
    f32x4 acc[MT][NS];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int jj = 0; jj < NS; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    // tile u of rows [rb, rb + 16 MT): wave partials added in wave order
    auto finish_tile = [&](int u, int rb) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int jj = 0; jj < NS; ++jj) {
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wave][16 * i + g * 4 + r][jj * 16 + c] = acc[i][jj][r];
                acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        __syncthreads();
        const int n0 = (t0 + u) * TC;
        for (int o = threadIdx.x; o < 16 * MT * TC; o += P * kWave) {
            const int r = o / TC, cc = o % TC;
            if (rb + r >= M || n0 + cc >= N) continue;
            float v = red[0][r][cc];
#pragma unroll
            for (int p = 1; p < P; ++p) v = v + red[p][r][cc];
            if constexpr (SPL) part[((int64_t)blockIdx.y * M + rb + r) * N + n0 + cc] = v;
            else y[(int64_t)(rb + r) * N + n0 + cc] = F16::narrow(v);
        }
        __syncthreads();
    };
    auto compute_item = [&](auto dc_, auto jc_) {
        constexpr int d = decltype(dc_)::value, j = decltype(jc_)::value;
        QGroup<QM> g01[NS], g23[NS];
#pragma unroll
        for (int jj = 0; jj < NS; ++jj) {
            g01[jj] = group_from_raw<QM>(S[d][jj], S[d][jj] >> 16, 0);
            g23[jj] = QM == BI_NVFP4 ? group_from_raw<QM>(S[d][jj], 0, 2) : g01[jj];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int jj = 0; jj < NS; ++jj) {
                const uint32_t wv = s == 0 ? W[d][jj].x : s == 1 ? W[d][jj].y : s == 2 ? W[d][jj].z : W[d][jj].w;
                const uint4 wd = deq_word<QM>(wv, s < 2 ? g01[jj] : g23[jj]);   // once for every row tile
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[i][jj] = qmfma(X[XR ? j : d][i][s], wd, acc[i][jj]);   // compile-time indices
            }
        }
    };

    if (nmine > 0 && XR) {
        // ring slot j holds block j of the tile in flight: a tile's items are
        // requested while the previous tile's are multiplied; one pass over
        // the tiles per 16 MT rows
        const int npass = MT == 1 ? 1 : (M + 16 * MT - 1) / (16 * MT);       // M <= 16 with one row tile
        for (int ps = 0; ps < npass; ++ps) {
            const int rb = ps * 16 * MT;
            load_x_res(rb);
            lu = 0;
            lj = 0;
            static_for<0, kQXRes>([&](auto jc) {
                if (decltype(jc)::value < nmine) load_item(jc);
            });
            for (int u = 0; u < ntile; ++u) {
                static_for<0, kQXRes>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if (j < nmine) {
                        compute_item(jc, jc);
                        if (u + 1 < ntile) load_item(jc);
                    }
                });
                finish_tile(u, rb);
            }
        }
    } else if (nmine > 0) {
        static_for<0, D - 1>([&](auto dc) {
            if (decltype(dc)::value < items) load_item(dc);
        });
        int cu = 0, cj = 0;
        for (int i = 0; i < items; i += D) {
            static_for<0, D>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                if (i + d + D - 1 < items) load_item(std::integral_constant<int, (d + D - 1) % D>{});
                if (i + d < items) {
                    compute_item(dc, std::integral_constant<int, 0>{});
                    if (++cj == nmine) {
                        finish_tile(cu, 0);
                        cj = 0;
                        ++cu;
                    }
                }
            });
        }
    } else {
        // a wave that owns no block of K still takes part in every combine
        const int npass = XR && MT > 1 ? (M + 16 * MT - 1) / (16 * MT) : 1;
        for (int ps = 0; ps < npass; ++ps)
            for (int u = 0; u < ntile; ++u) finish_tile(u, ps * 16 * MT);
    }
}

template <int QM, int GS, int NS, bool PK>
static void launch_q_stream_t(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                          int64_t N, int64_t K, hipStream_t st)
{
    const int64_t ntn = cdiv(N, NS * 16);
    const int64_t slots = (int64_t)device_cu_count() * 2;
    const int64_t per = cdiv(ntn, slots), grid = cdiv(ntn, per);
    const bool xres = cdiv(K / kQBlock, kQWaves) <= kQXRes;
    if (xres)
        launch_kernel((qmatmul_stream_kernel<QM, GS, NS, 3, true, PK>), dim3((unsigned)grid), dim3(kQWaves * kWave), 0, st,
                      (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)y, (int)M, (int)N, (int)K, (int)ntn,
                      (int)per, (float *)nullptr, 1);
    else
        launch_kernel((qmatmul_stream_kernel<QM, GS, NS, 3, false, PK>), dim3((unsigned)grid), dim3(kQWaves * kWave), 0,
                      st, (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)y, (int)M, (int)N, (int)K,
                      (int)ntn, (int)per, (float *)nullptr, 1);
}

// 17..64 rows with at most kQXRes blocks of K per wave: two row tiles with
// resident x, one pass over the workgroup's tiles per 32 rows, one
// workgroup per CU
template <int QM, int GS, bool PK>
static void launch_q_stream_xr2(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                                int64_t N, int64_t K, hipStream_t st)
{
    const int64_t ntn = cdiv(N, 16);
    const int64_t per = cdiv(ntn, (int64_t)device_cu_count()), grid = cdiv(ntn, per);
    launch_kernel((qmatmul_stream_kernel<QM, GS, 1, 3, true, PK, false, 2>), dim3((unsigned)grid),
                  dim3(kQWaves * kWave), 0, st, (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)y, (int)M,
                  (int)N, (int)K, (int)ntn, (int)per, (float *)nullptr, 1);
}

// 17..64 rows, longer K: MT row tiles, x through a 2-deep ring, one
// workgroup per CU
template <int QM, int GS, int MT, bool PK>
static void launch_q_stream_mt(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                               int64_t N, int64_t K, hipStream_t st)
{
    const int64_t ntn = cdiv(N, 16);
    const int64_t per = cdiv(ntn, (int64_t)device_cu_count()), grid = cdiv(ntn, per);
    launch_kernel((qmatmul_stream_kernel<QM, GS, 1, 2, false, PK, false, MT>), dim3((unsigned)grid),
                  dim3(kQWaves * kWave), 0, st, (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)y, (int)M,
                  (int)N, (int)K, (int)ntn, (int)per, (float *)nullptr, 1);
}

template <int QM, int GS, bool PK>
static bool try_launch_q_stream(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                                int64_t N, int64_t K, hipStream_t st)
{
    if (M > 64 || K % kQBlock != 0 || !host_aligned16(x) || !host_aligned16(wq) || N >= (1ll << 30) ||
        K >= (1ll << 30))
        return false;
    if (M <= 16) launch_q_stream_t<QM, GS, 1, PK>(x, wq, s, b, y, M, N, K, st);
    else if (cdiv(K / kQBlock, kQWaves) <= kQXRes) launch_q_stream_xr2<QM, GS, PK>(x, wq, s, b, y, M, N, K, st);
    else if (M <= 32) launch_q_stream_mt<QM, GS, 2, PK>(x, wq, s, b, y, M, N, K, st);
    else launch_q_stream_mt<QM, GS, 4, PK>(x, wq, s, b, y, M, N, K, st);
    return true;
}

// Split-K comparison variant of the streaming kernel: split z reduces the
// contiguous blocks [z nb / splits, (z + 1) nb / splits) into fp32 partials
// [splits, M, N], which q_split_reduce_kernel adds in z order.  The tree then
// depends on `splits` -- the batch-dependent split-K the invariant kernel
// exists to avoid -- so it serves only to price invariance.
template <int QM, int GS, bool PK>
static void launch_q_split(const void *x, const uint32_t *wq, const void *s, const void *b, float *part, int64_t M,
                           int64_t N, int64_t K, int splits, hipStream_t st)
{
    const int64_t ntn = cdiv(N, 16), slots = (int64_t)device_cu_count() * 2;
    const int64_t per = cdiv(ntn * splits, slots), grid = cdiv(ntn, per);
    const bool xres = cdiv(cdiv(K / kQBlock, splits), kQWaves) <= kQXRes;
    const dim3 g((unsigned)grid, (unsigned)splits);
    if (xres)
        launch_kernel((qmatmul_stream_kernel<QM, GS, 1, 3, true, PK, true>), g, dim3(kQWaves * kWave), 0, st,
                      (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)nullptr, (int)M, (int)N, (int)K,
                      (int)ntn, (int)per, part, splits);
    else
        launch_kernel((qmatmul_stream_kernel<QM, GS, 1, 3, false, PK, true>), g, dim3(kQWaves * kWave), 0, st,
                      (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)nullptr, (int)M, (int)N, (int)K,
                      (int)ntn, (int)per, part, splits);
}

__global__ void q_split_reduce_kernel(const float *__restrict__ part, uint16_t *__restrict__ y, int64_t MN, int splits)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < MN; i += (int64_t)gridDim.x * blockDim.x) {
        float v = part[i];
        for (int z = 1; z < splits; ++z) v = v + part[(int64_t)z * MN + i];
        y[i] = F16::narrow(v);
    }
}

template <int QM, int GS, bool TRANS, bool WVEC, int MT, bool PK>
static void launch_q_t(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                       int64_t N, int64_t K, hipStream_t st)
{
    dim3 grid((unsigned)cdiv(N, 16), (unsigned)cdiv(M, MT * 16));
    launch_kernel((qmatmul_kernel<QM, GS, TRANS, WVEC, MT, 1, PK>), grid, dim3(kQWaves * kWave), 0, st,
                       (const uint16_t *)x, wq, s, (const uint16_t *)b, (uint16_t *)y, M, N, K);
}

template <int QM, int GS, bool TRANS, bool WVEC, bool PK = false>
static void launch_q_mt(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M,
                        int64_t N, int64_t K, hipStream_t st)
{
    const int64_t mt = cdiv(M, 16);
    if (mt <= 1) launch_q_t<QM, GS, TRANS, WVEC, 1, PK>(x, wq, s, b, y, M, N, K, st);
    else if (mt <= 2) launch_q_t<QM, GS, TRANS, WVEC, 2, PK>(x, wq, s, b, y, M, N, K, st);
    else launch_q_t<QM, GS, TRANS, WVEC, 4, PK>(x, wq, s, b, y, M, N, K, st);
}

template <int QM, int GS>
static void launch_q(const void *x, const uint32_t *wq, const void *s, const void *b, void *y, int64_t M, int64_t N,
                     int64_t K, int layout, hipStream_t st)
{
    if (layout == 2) {                              // packed: K % 128 == 0, wq 16-byte aligned (checked)
        if (!try_launch_q_stream<QM, GS, true>(x, wq, s, b, y, M, N, K, st))
            launch_q_mt<QM, GS, true, true, true>(x, wq, s, b, y, M, N, K, st);
    } else if (layout == 0) {
        launch_q_mt<QM, GS, false, false>(x, wq, s, b, y, M, N, K, st);
    } else if (try_launch_q_stream<QM, GS, false>(x, wq, s, b, y, M, N, K, st)) {
        return;
    } else if (K % 32 == 0 && host_aligned16(wq)) {
        launch_q_mt<QM, GS, true, true>(x, wq, s, b, y, M, N, K, st);
    } else {
        launch_q_mt<QM, GS, true, false>(x, wq, s, b, y, M, N, K, st);
    }
}

// [N, K/8] codes + [N, K/gs] constants -> the packed layout; one thread per
// 16-byte code chunk, then one per constant entry.
template <int QM, int GS>
__global__ void pack_q_kernel(const uint32_t *__restrict__ wq, const void *__restrict__ scales,
                              const uint16_t *__restrict__ biases, uint32_t *__restrict__ wqp, int64_t N, int64_t K)
{
    const int64_t nb = K / kQBlock, nrg = (N + 15) / 16, words = K / 8, groups = K / GS;
    constexpr int GPB = 128 / GS;                                // constant entries per row per block
    const int64_t ncode = nrg * nb * 64, nconst = nrg * nb * 16 * GPB;
    uint8_t *cbase = reinterpret_cast<uint8_t *>(wqp) + nrg * nb * 1024;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ncode + nconst;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < ncode) {
            const int lane = (int)(i & 63);
            const int64_t rb = i >> 6, b = rb % nb, rg = rb / nb;
            const int64_t row = rg * 16 + (lane & 15);
            const uint4 v = row < N ? *reinterpret_cast<const uint4 *>(wq + row * words + b * 16 + (lane >> 4) * 4)
                                    : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(wqp + i * 4) = v;
        } else {
            const int64_t e = i - ncode, q = e % GPB, cr = e / GPB, c = cr % 16, rb = cr / 16;
            const int64_t b = rb % nb, rg = rb / nb, row = rg * 16 + c;
            const int64_t gi = row * groups + b * GPB + q;
            if constexpr (QM == BI_AFFINE) {
                const uint32_t v = row < N ? (uint32_t)((const uint16_t *)scales)[gi] | ((uint32_t)biases[gi] << 16) : 0u;
                *reinterpret_cast<uint32_t *>(cbase + e * 4) = v;
            } else {
                cbase[e] = row < N ? ((const uint8_t *)scales)[gi] : (uint8_t)0;
            }
        }
    }
}

// Expert ("gather") matmul of a mixture-of-experts layer: row m of y is
// x[lhs[m]] @ dequantize(W[rhs[m]])^T (or the natural-layout product).
// Workgroup (t, e) owns the 16 columns of tile t for expert e: it compacts the
// rows routed to e (in ascending row order, a slab of up to kGatherSlab rows
// at a time) into LDS and runs them 16 at a time, so the rows of one MFMA
// tile share the weight fragment, each used expert's columns stream once per
// slab, and the experts proceed in parallel.  A chunk reduces exactly as
// qmatmul_kernel does (block b of K to wave b mod 8, lane group g supplying
// [32g, 32g + 32) of the block, wave partials added in order), so a row gets
// the bits of the plain quantized matmul of its token with its expert --
// whatever the other rows, their experts, their order or which chunk it lands
// in.  The workgroups of e = E write NaN to the rows whose token or expert
// index is out of range.
constexpr int kGatherSlab = 4096;
constexpr int kGatherMaxExperts = 1023;

template <int QM, int GS, bool TRANS, bool WVEC, bool PK>
__global__ __launch_bounds__(kQWaves * kWave)
void gather_q_kernel(const uint16_t *__restrict__ x, const int32_t *__restrict__ lhs, const int32_t *__restrict__ rhs,
                     const uint32_t *__restrict__ wq, const void *__restrict__ scales,
                     const uint16_t *__restrict__ biases, uint16_t *__restrict__ y, int64_t M, int64_t x_rows,
                     int64_t N, int64_t K, int E)
{
    constexpr int P = kQWaves, NT = kQWaves * kWave;
    constexpr int SB = QM == BI_AFFINE ? 2 : 1;                 // bytes per scale entry
    __shared__ float red[P][16][17];
    __shared__ int perm[kGatherSlab];
    __shared__ int wcnt[P];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int e = (int)blockIdx.y;
    const int64_t n0 = (int64_t)blockIdx.x * 16, n = n0 + c;
    const bool nok = n < N;
    const int64_t nblocks = cdiv(K, kQBlock);
    const bool xvec = (K % 8) == 0 && aligned16(x);
    const int64_t nrg = (N + 15) / 16;
    // per expert: codes [N, K/8] and constants [N, K/gs], or one packed buffer
    const int64_t words_e = PK ? nrg * nblocks * (256 + qconst_chunk_bytes(QM, GS) / 4) : N * K / 8;
    const int64_t groups_e = N * K / GS;
    const uint32_t *we = wq + (int64_t)(e < E ? e : 0) * words_e;
    const void *se = (const uint8_t *)scales + (int64_t)(e < E ? e : 0) * groups_e * SB;
    const uint16_t *be = biases ? biases + (int64_t)(e < E ? e : 0) * groups_e : nullptr;

    auto bucket = [&](int64_t m) -> int {
        const int64_t r = rhs[m], xr = lhs ? (int64_t)lhs[m] : m;
        return (r >= 0 && r < E && xr >= 0 && xr < x_rows) ? (int)r : E;
    };

    for (int64_t s0 = 0; s0 < M; s0 += kGatherSlab) {
        const int ns = (int)(M - s0 < kGatherSlab ? M - s0 : kGatherSlab);
        // compact the slab's rows of bucket e into perm, in ascending order
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
            __syncthreads();                                    // wcnt is rewritten next round
        }
        if (e == E) {                                           // rows with a bad index: NaN
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
                if constexpr (PK) {
                    // K % 128 == 0: every block is whole; padding rows of the group are zeros
                    uint4 A[4], wv;
                    uint32_t sc, bs;
                    qload_packed_raw<QM, GS>(we, nrg, nblocks, (int64_t)blockIdx.x, b, lane, wv, sc, bs);
                    const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        A[s] = xvec ? load_chunk<F16, true>(xrow, kbase + s * 8, K, rok)
                                    : load_chunk<F16, false>(xrow, kbase + s * 8, K, rok);
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = qmfma(A[s], deq_word<QM>(wa[s], group_from_raw<QM>(sc, bs, s)), acc);
                } else if constexpr (TRANS) {
                    uint4 A[4], Bf[4];
                    qload_trans<QM, GS, WVEC>(Bf, we, se, be, nok ? n : 0, nok, K, kbase);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        A[s] = xvec ? load_chunk<F16, true>(xrow, kbase + s * 8, K, rok)
                                    : load_chunk<F16, false>(xrow, kbase + s * 8, K, rok);
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = qmfma(A[s], Bf[s], acc);
                } else {
                    // element-wise gathers: one step of 8 at a time keeps the registers bounded
#pragma unroll 1
                    for (int s = 0; s < 4; ++s) {
                        const uint4 Bs = qload_nat8<QM, GS>(we, se, be, nok ? n : 0, nok, N, K, kbase + s * 8);
                        const uint4 As = xvec ? load_chunk<F16, true>(xrow, kbase + s * 8, K, rok)
                                              : load_chunk<F16, false>(xrow, kbase + s * 8, K, rok);
                        acc = qmfma(As, Bs, acc);
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

// Streaming form of the expert matmul for at most 16 rows (a decode step),
// transposed weights, K % 128 == 0, 16-byte aligned x and wq.  The workgroup
// lists the distinct experts of the rows (ascending) and walks the tiles
// (expert, 16*NS columns) of that list as qmatmul_stream_kernel walks its
// column tiles: each wave streams its (tile, block) items -- packed words,
// group constants and x chunks -- through a D-deep register ring.  A-operand
// row c is row c of the call, its x chunk zero unless the row is routed to
// the tile's expert; only such rows are stored.  Per row the tree is
// qmatmul_stream_kernel's, hence the plain quantized matmul's bits.
template <int QM, int GS, int NS, int D, bool PK>
__global__ __launch_bounds__(kQWaves * kWave, 2)
void gather_q_stream_kernel(const uint16_t *__restrict__ x, const int32_t *__restrict__ lhs,
                            const int32_t *__restrict__ rhs, const uint32_t *__restrict__ wq,
                            const void *__restrict__ scales, const uint16_t *__restrict__ biases,
                            uint16_t *__restrict__ y, int64_t M, int64_t x_rows, int64_t N, int64_t K, int E, int ntn)
{
    constexpr int P = kQWaves, TC = NS * 16, NT = kQWaves * kWave;
    constexpr int SB = QM == BI_AFFINE ? 2 : 1;                 // bytes per scale entry
    __shared__ float red[P][16][TC + 1];
    __shared__ int s_bucket[16], s_active[16], s_nact;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    if (tid < 16) {
        int bk = -1;                                            // -1: no such row; E: a bad index
        if (tid < M) {
            const int64_t r = rhs[tid], xi = lhs ? (int64_t)lhs[tid] : tid;
            bk = (r >= 0 && r < E && xi >= 0 && xi < x_rows) ? (int)r : E;
        }
        s_bucket[tid] = bk;
    }
    __syncthreads();
    if (tid == 0) {                                             // distinct experts, ascending
        int na = 0, last = -1;
        for (;;) {
            int best = E;
            for (int r = 0; r < 16; ++r) {
                const int b = s_bucket[r];
                if (b > last && b < best) best = b;
            }
            if (best == E) break;
            s_active[na++] = best;
            last = best;
        }
        s_nact = na;
    }
    __syncthreads();
    const int ntiles = s_nact * ntn;
    const int nb = (int)(K / kQBlock);
    const int nmine = wave < nb ? (nb - wave + P - 1) / P : 0;        // blocks of this wave per tile
    const int mytiles = (int)blockIdx.x < ntiles ? (ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    const int items = mytiles * nmine;
    const int64_t nrg = (N + 15) / 16;
    const int64_t words = K / 8, groups = K / GS, groups_e = N * K / GS;
    const int64_t words_e = PK ? nrg * nb * (256 + qconst_chunk_bytes(QM, GS) / 4) : N * K / 8;
    const int mybk = s_bucket[c];
    const bool myok = mybk >= 0 && mybk < E;
    // x row of A-operand row c (rows without a valid expert read row 0 and are never stored)
    const uint16_t *xr = x + (myok ? (lhs ? (int64_t)lhs[c] : (int64_t)c) : 0) * K + g * 32;

    uint4 Wr[D][NS], Xr[D][4];
    uint32_t Sr[D][NS], Br[D][NS];
    int pu = 0, pj = 0;
    auto load_next = [&](uint4 (&Wd)[NS], uint32_t (&Sd)[NS], uint32_t (&Bd)[NS], uint4 (&Xd)[4]) {
        const int t = (int)blockIdx.x + pu * (int)gridDim.x;
        const int e = s_active[t / ntn], ct = t % ntn;
        const uint32_t *we = wq + (int64_t)e * words_e;
        const uint8_t *se = (const uint8_t *)scales + (int64_t)e * groups_e * SB;
        const int64_t kb = (int64_t)(wave + pj * P) * kQBlock + g * 32;     // this lane's first code
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if constexpr (PK) {
                const int64_t rg = (int64_t)ct * NS + j;
                qload_packed_raw<QM, GS>(we, nrg, nb, rg < nrg ? rg : nrg - 1, wave + pj * P, lane, Wd[j], Sd[j], Bd[j]);
                continue;
            }
            int64_t n = (int64_t)ct * TC + j * 16 + c;
            n = n < N ? n : N - 1;                                      // padding columns read a real row
            Wd[j] = *reinterpret_cast<const uint4 *>(we + n * words + kb / 8);
            const int64_t gi = n * groups + kb / GS;
            if (QM == BI_AFFINE) {
                Sd[j] = ((const uint16_t *)se)[gi];
                Bd[j] = (biases + (int64_t)e * groups_e)[gi];
            } else if (QM == BI_NVFP4) {
                Sd[j] = ((const uint16_t *)se)[gi / 2];                 // the lane's two group bytes
                Bd[j] = 0;
            } else {
                Sd[j] = se[gi];                                         // the lane's one group byte
                Bd[j] = 0;
            }
        }
        if (mybk == e) {
#pragma unroll
            for (int s = 0; s < 4; ++s) Xd[s] = *reinterpret_cast<const uint4 *>(xr + (kb - g * 32) + s * 8);
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
        const int t = (int)blockIdx.x + u * (int)gridDim.x;
        const int e = s_active[t / ntn];
        const int64_t n0 = (int64_t)(t % ntn) * TC;
        for (int o = tid; o < 16 * TC; o += NT) {
            const int r = o / TC, cc = o % TC;
            const int64_t col = n0 + cc;
            if (s_bucket[r] != e || col >= N) continue;
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
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
#pragma unroll
                        for (int j = 0; j < NS; ++j) {
                            const QGroup<QM> gr = group_from_raw<QM>(Sr[d][j], Br[d][j], s);
                            const uint32_t wv = s == 0 ? Wr[d][j].x : s == 1 ? Wr[d][j].y : s == 2 ? Wr[d][j].z : Wr[d][j].w;
                            acc[j] = qmfma(Xr[d][s], deq_word<QM>(wv, gr), acc[j]);
                        }
                    }
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
        for (int u = 0; u < mytiles; ++u) finish_tile(u);
    }
    // rows with a bad index: NaN
    for (int64_t i = (int64_t)blockIdx.x * NT + tid; i < M * N; i += (int64_t)gridDim.x * NT)
        if (s_bucket[i / N] == E) y[i] = 0x7e00u;
}

template <int QM, int GS>
static void launch_gather(const void *x, const int32_t *lhs, const int32_t *rhs, const uint32_t *wq, const void *s,
                          const void *b, void *y, int64_t M, int64_t x_rows, int64_t N, int64_t K, int E, int layout,
                          hipStream_t st)
{
    // one workgroup per (16-column tile, expert), plus one per tile for the rows with a bad index
    const dim3 grid((unsigned)cdiv(N, 16), (unsigned)(E + 1)), block(kQWaves * kWave);
    const uint16_t *bz = (const uint16_t *)b;
    const bool packed = layout == 2;                     // K % 128 == 0 and 16-byte aligned (checked)
    if (layout >= 1 && M <= 16 && K % kQBlock == 0 && host_aligned16(x) && host_aligned16(wq) &&
        cdiv(N, 16) <= (1ll << 24)) {
        const int ns = N >= 8192 ? 2 : 1;
        const int64_t ntn = cdiv(N, 16 * ns);
        const int64_t tiles = std::min<int64_t>(M, E) * ntn;            // at most this many (expert, tile) pairs
        const dim3 g((unsigned)std::min<int64_t>(tiles, (int64_t)device_cu_count() * 2));
        const uint16_t *xx = (const uint16_t *)x;
        uint16_t *yy = (uint16_t *)y;
        if (ns == 2 && packed)
            launch_kernel((gather_q_stream_kernel<QM, GS, 2, 3, true>), g, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                          x_rows, N, K, E, (int)ntn);
        else if (ns == 2)
            launch_kernel((gather_q_stream_kernel<QM, GS, 2, 3, false>), g, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                          x_rows, N, K, E, (int)ntn);
        else if (packed)
            launch_kernel((gather_q_stream_kernel<QM, GS, 1, 3, true>), g, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                          x_rows, N, K, E, (int)ntn);
        else
            launch_kernel((gather_q_stream_kernel<QM, GS, 1, 3, false>), g, block, 0, st, xx, lhs, rhs, wq, s, bz, yy, M,
                          x_rows, N, K, E, (int)ntn);
        return;
    }
    if (packed)
        launch_kernel((gather_q_kernel<QM, GS, true, true, true>), grid, block, 0, st, (const uint16_t *)x, lhs, rhs, wq,
                      s, bz, (uint16_t *)y, M, x_rows, N, K, E);
    else if (layout == 0)
        launch_kernel((gather_q_kernel<QM, GS, false, false, false>), grid, block, 0, st, (const uint16_t *)x, lhs, rhs,
                      wq, s, bz, (uint16_t *)y, M, x_rows, N, K, E);
    else if (K % 32 == 0 && host_aligned16(wq))     // then every expert's matrix starts 16-byte aligned too
        launch_kernel((gather_q_kernel<QM, GS, true, true, false>), grid, block, 0, st, (const uint16_t *)x, lhs, rhs,
                      wq, s, bz, (uint16_t *)y, M, x_rows, N, K, E);
    else
        launch_kernel((gather_q_kernel<QM, GS, true, false, false>), grid, block, 0, st, (const uint16_t *)x, lhs, rhs,
                      wq, s, bz, (uint16_t *)y, M, x_rows, N, K, E);
}

}  // namespace bi

using namespace bi;

static bi_status check_qmode(int32_t qmode, int32_t bits, int32_t group_size)
{
    if (qmode == BI_AFFINE)
        return (bits >= 2 && bits <= 8 && (group_size == 32 || group_size == 64 || group_size == 128)) ? BI_OK
                                                                                                      : BI_ERR_GROUP;
    if (qmode == BI_NVFP4) return (bits == 4 && group_size == 16) ? BI_OK : BI_ERR_GROUP;
    if (qmode == BI_MXFP4) return (bits == 4 && group_size == 32) ? BI_OK : BI_ERR_GROUP;
    if (qmode == BI_MXFP8) return (bits == 8 && group_size == 32) ? BI_OK : BI_ERR_GROUP;
    return BI_ERR_GROUP;
}

// The formats this file's kernels (and the packed layout) serve; the rest go
// to qmatmul_wide.hip.
static bool four_bit_mode(int32_t qmode, int32_t bits) { return bits == 4 && qmode != BI_MXFP8; }

extern "C" bi_status bi_qmatmul(const void *x, const uint32_t *wq, const void *scales, const void *biases, void *y,
                                int64_t M, int64_t N, int64_t K, int32_t qmode, int32_t bits, int32_t group_size,
                                int32_t w_layout, hipStream_t stream)
{
    const bool packed = w_layout == 2;
    if (!x || !wq || !y || (!scales && !packed)) return BI_ERR_NULL;
    if (M < 1 || N < 1 || K < 1 || M > (1ll << 31) || N > (1ll << 31) || K > (1ll << 31)) return BI_ERR_SHAPE;
    if (w_layout < 0 || w_layout > 2) return BI_ERR_SHAPE;
    const bi_status qs = check_qmode(qmode, bits, group_size);
    if (qs != BI_OK) return qs;
    if (!packed) {
        if (qmode == BI_AFFINE && !biases) return BI_ERR_NULL;
        if (qmode != BI_AFFINE && biases) return BI_ERR_GROUP;
    }
    const int64_t qdim = w_layout ? K : N;
    if (qdim % group_size) return BI_ERR_GROUP;
    if (packed && K % kQBlock) return BI_ERR_SHAPE;
    if ((((uintptr_t)x | (uintptr_t)y) & 1u) || ((uintptr_t)wq & (packed ? 15u : 3u)) ||
        (!packed && (((uintptr_t)scales & 1u) || ((uintptr_t)biases & 1u))))
        return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (!four_bit_mode(qmode, bits))
        return bi_qmatmul_wide(x, wq, scales, biases, y, M, N, K, qmode, bits, group_size, w_layout, stream);
    if (qmode == BI_NVFP4) launch_q<BI_NVFP4, 16>(x, wq, scales, biases, y, M, N, K, w_layout, stream);
    else if (qmode == BI_MXFP4) launch_q<BI_MXFP4, 32>(x, wq, scales, biases, y, M, N, K, w_layout, stream);
    else if (group_size == 32) launch_q<BI_AFFINE, 32>(x, wq, scales, biases, y, M, N, K, w_layout, stream);
    else if (group_size == 64) launch_q<BI_AFFINE, 64>(x, wq, scales, biases, y, M, N, K, w_layout, stream);
    else launch_q<BI_AFFINE, 128>(x, wq, scales, biases, y, M, N, K, w_layout, stream);
    return launch_status();
}

extern "C" size_t bi_qmatmul_split_workspace_bytes(int64_t M, int64_t N, int32_t splits)
{
    if (M < 1 || N < 1 || splits < 1 || M > (1ll << 31) || N > (1ll << 31)) return 0;
    return (size_t)splits * (size_t)M * (size_t)N * sizeof(float);
}

extern "C" bi_status bi_qmatmul_split(const void *x, const uint32_t *wq, const void *scales, const void *biases,
                                      void *y, int64_t M, int64_t N, int64_t K, int32_t qmode, int32_t bits,
                                      int32_t group_size, int32_t w_layout, int32_t splits, void *ws, size_t ws_bytes,
                                      hipStream_t stream)
{
    if (splits < 1 || splits > 1024) return BI_ERR_SHAPE;
    if (splits == 1)
        return bi_qmatmul(x, wq, scales, biases, y, M, N, K, qmode, bits, group_size, w_layout, stream);
    // validation of the operands first (the invariant entry point's rules)
    const bool packed = w_layout == 2;
    if (!x || !wq || !y || (!scales && !packed)) return BI_ERR_NULL;
    if (M < 1 || N < 1 || K < 1 || M > (1ll << 31) || N > (1ll << 31) || K > (1ll << 31)) return BI_ERR_SHAPE;
    if (w_layout < 0 || w_layout > 2) return BI_ERR_SHAPE;
    const bi_status qs = check_qmode(qmode, bits, group_size);
    if (qs != BI_OK) return qs;
    if (!packed) {
        if (qmode == BI_AFFINE && !biases) return BI_ERR_NULL;
        if (qmode != BI_AFFINE && biases) return BI_ERR_GROUP;
    }
    if ((w_layout ? K : N) % group_size) return BI_ERR_GROUP;
    // the split form exists for the streaming decode kernel's shapes only
    if (!four_bit_mode(qmode, bits) || w_layout == 0 || M > 16 || K % kQBlock || N >= (1ll << 30) ||
        K >= (1ll << 30))
        return BI_ERR_UNSUPPORTED;
    if (splits > K / kQBlock) return BI_ERR_SHAPE;
    if ((((uintptr_t)x | (uintptr_t)y) & 1u) || !host_aligned16(x) || !host_aligned16(wq) ||
        (!packed && (((uintptr_t)scales & 1u) || ((uintptr_t)biases & 1u))))
        return BI_ERR_ALIGN;
    if (!ws || ws_bytes < bi_qmatmul_split_workspace_bytes(M, N, splits)) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    float *part = (float *)ws;
    const void *s = scales, *b = biases;
#define BI_QSPLIT(QM_, GS_)                                                                            \
    do {                                                                                              \
        if (packed) launch_q_split<QM_, GS_, true>(x, wq, s, b, part, M, N, K, splits, stream);       \
        else launch_q_split<QM_, GS_, false>(x, wq, s, b, part, M, N, K, splits, stream);             \
    } while (0)
    if (qmode == BI_NVFP4) BI_QSPLIT(BI_NVFP4, 16);
    else if (qmode == BI_MXFP4) BI_QSPLIT(BI_MXFP4, 32);
    else if (group_size == 32) BI_QSPLIT(BI_AFFINE, 32);
    else if (group_size == 64) BI_QSPLIT(BI_AFFINE, 64);
    else BI_QSPLIT(BI_AFFINE, 128);
#undef BI_QSPLIT
    const int64_t MN = M * N;
    launch_kernel(q_split_reduce_kernel, dim3((unsigned)std::min<int64_t>(cdiv(MN, 256), 65536)), dim3(256), 0, stream,
                  (const float *)part, (uint16_t *)y, MN, (int)splits);
    return launch_status();
}

extern "C" size_t bi_packed_qweight_bytes(int64_t N, int64_t K, int32_t qmode, int32_t bits, int32_t group_size)
{
    if (N < 1 || K < 1 || K % kQBlock || N > (1ll << 31) || K > (1ll << 31) || check_qmode(qmode, bits, group_size) != BI_OK)
        return 0;
    const size_t chunks = (size_t)cdiv(N, 16) * (size_t)(K / kQBlock);
    return chunks * ((size_t)256 * bits + (size_t)qconst_chunk_bytes(qmode, group_size));   // 64 lanes x bits words
}

extern "C" bi_status bi_pack_qweights(const uint32_t *wq, const void *scales, const void *biases, void *wqp, int64_t N,
                                      int64_t K, int32_t qmode, int32_t bits, int32_t group_size, hipStream_t stream)
{
    if (!wq || !scales || !wqp) return BI_ERR_NULL;
    const bi_status qs = check_qmode(qmode, bits, group_size);
    if (qs != BI_OK) return qs;
    if (qmode == BI_AFFINE && !biases) return BI_ERR_NULL;
    if (qmode != BI_AFFINE && biases) return BI_ERR_GROUP;
    if (bi_packed_qweight_bytes(N, K, qmode, bits, group_size) == 0) return BI_ERR_SHAPE;
    if (!host_aligned16(wq) || !host_aligned16(wqp) || ((uintptr_t)scales & 1u) || ((uintptr_t)biases & 1u))
        return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (!four_bit_mode(qmode, bits)) return bi_pack_qweights_wide(wq, scales, biases, wqp, N, K, qmode, bits, group_size, stream);
    const int64_t nrg = cdiv(N, 16), nb = K / kQBlock;
    const int64_t n = nrg * nb * 64 + nrg * nb * 16 * (128 / group_size);
    const dim3 grid((unsigned)std::min<int64_t>(cdiv(n, 256), 65536)), block(256);
    const uint32_t *w = wq;
    const uint16_t *bz = (const uint16_t *)biases;
    uint32_t *o = (uint32_t *)wqp;
    if (qmode == BI_NVFP4) launch_kernel((pack_q_kernel<BI_NVFP4, 16>), grid, block, 0, stream, w, scales, bz, o, N, K);
    else if (qmode == BI_MXFP4) launch_kernel((pack_q_kernel<BI_MXFP4, 32>), grid, block, 0, stream, w, scales, bz, o, N, K);
    else if (group_size == 32) launch_kernel((pack_q_kernel<BI_AFFINE, 32>), grid, block, 0, stream, w, scales, bz, o, N, K);
    else if (group_size == 64) launch_kernel((pack_q_kernel<BI_AFFINE, 64>), grid, block, 0, stream, w, scales, bz, o, N, K);
    else launch_kernel((pack_q_kernel<BI_AFFINE, 128>), grid, block, 0, stream, w, scales, bz, o, N, K);
    return launch_status();
}

extern "C" bi_status bi_gather_qmatmul(const void *x, const int32_t *lhs_idx, const int32_t *rhs_idx,
                                       const uint32_t *wq, const void *scales, const void *biases, void *y,
                                       int64_t M, int64_t x_rows, int64_t N, int64_t K, int64_t E, int32_t qmode,
                                       int32_t bits, int32_t group_size, int32_t w_layout, hipStream_t stream)
{
    const bool packed = w_layout == 2;
    if (!x || !rhs_idx || !wq || (!scales && !packed) || !y) return BI_ERR_NULL;
    if (M < 1 || x_rows < 1 || N < 1 || K < 1 || E < 1 || M > (1ll << 31) || x_rows > (1ll << 31) ||
        N > (1ll << 31) || K > (1ll << 31) || E > kGatherMaxExperts || (!lhs_idx && x_rows < M))
        return BI_ERR_SHAPE;
    if (w_layout < 0 || w_layout > 2) return BI_ERR_SHAPE;
    const bi_status qs = check_qmode(qmode, bits, group_size);
    if (qs != BI_OK) return qs;
    if (!packed) {
        if (qmode == BI_AFFINE && !biases) return BI_ERR_NULL;
        if (qmode != BI_AFFINE && biases) return BI_ERR_GROUP;
    }
    if ((w_layout ? K : N) % group_size) return BI_ERR_GROUP;
    if (packed && K % kQBlock) return BI_ERR_SHAPE;
    if ((((uintptr_t)x | (uintptr_t)y) & 1u) || ((uintptr_t)wq & (packed ? 15u : 3u)) ||
        (!packed && (((uintptr_t)scales | (uintptr_t)biases) & 1u)) ||
        (((uintptr_t)lhs_idx | (uintptr_t)rhs_idx) & 3u))
        return BI_ERR_ALIGN;
    (void)hipGetLastError();
    if (!four_bit_mode(qmode, bits))
        return bi_gather_qmatmul_wide(x, lhs_idx, rhs_idx, wq, scales, biases, y, M, x_rows, N, K, E, qmode, bits,
                                      group_size, w_layout, stream);
    const int e = (int)E;
    if (qmode == BI_NVFP4)
        launch_gather<BI_NVFP4, 16>(x, lhs_idx, rhs_idx, wq, scales, biases, y, M, x_rows, N, K, e, w_layout, stream);
    else if (qmode == BI_MXFP4)
        launch_gather<BI_MXFP4, 32>(x, lhs_idx, rhs_idx, wq, scales, biases, y, M, x_rows, N, K, e, w_layout, stream);
    else if (group_size == 32)
        launch_gather<BI_AFFINE, 32>(x, lhs_idx, rhs_idx, wq, scales, biases, y, M, x_rows, N, K, e, w_layout, stream);
    else if (group_size == 64)
        launch_gather<BI_AFFINE, 64>(x, lhs_idx, rhs_idx, wq, scales, biases, y, M, x_rows, N, K, e, w_layout, stream);
    else
        launch_gather<BI_AFFINE, 128>(x, lhs_idx, rhs_idx, wq, scales, biases, y, M, x_rows, N, K, e, w_layout, stream);
    return launch_status();
}
