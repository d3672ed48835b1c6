// sdpa.hip -- batch-invariant decode / verify attention on gfx950.
//
// Sources: "Fix/speculative shape invariance" (Problem: two-pass SDPA derived
// its split count from the query length; Changes: the single-query split
// configuration for a query alone or inside a short causal block);
// "Batch-invariant kernels: why temperature-0 decoding is still
// nondeterministic" (Case 6: a fixed split SIZE with a varying number of
// splits, KV cache updated before the kernel; Try this, item 5).
//
// Reduction tree of one query row r at position p (frozen; depends on p only):
//   Pass 1 -- keys are cut into chunks of kChunk = 256 positions; chunk c holds
//   keys [256c, 256c + 256) and is handled by its own workgroup for all query
//   rows of one (sequence, KV head).  Inside the chunk, wave w owns keys
//   [64w, 64w + 64):
//     s_t   = scale * (q . k_t)      one 16x16x32 bf16 MFMA chain over d
//                                    (4 steps; lane group g supplies d in
//                                    [32g, 32g + 32), step s the s-th 8 of them)
//     m_c   = max of s_t over the chunk's keys t <= p (exact, order-free)
//     p_t   = exp(s_t - m_c); keys t > p contribute exactly +0
//     l_c   = sum p_t: per lane over its 4 key tiles in order, then a xor
//             butterfly over the 16 lanes of a row (1, 2, 4, 8), then waves in
//             order 0..3
//     o_c   = sum bf16(p_t) * v_t: MFMA over the wave's 64 keys (2 steps of 32),
//             then the four wave partials added in order 0..3
//   Pass 2 -- for the chunks 0..floor(p/256):
//     M = max_c m_c (exact);  w_c = exp(m_c - M)
//     o = sum_c o_c * w_c and l = sum_c l_c * w_c, both in ascending c
//     out = RNE(o / l)
// A query row never meets another row except inside an MFMA (rows are
// independent there), so the number of queries Q, the GQA group, the batch and
// where the row sits in its tile leave its bits unchanged; a query of a causal
// verify block and a lone query at the same position reduce identically.
#include "common.hpp"

namespace bi {

constexpr int kChunk = 256;          // keys per chunk (frozen)
constexpr int kHeadDim = 128;        // D supported by this build
constexpr int kAttnWaves = 4;        // waves per chunk workgroup (frozen: 64 keys each)
constexpr int kKeysPerWave = kChunk / kAttnWaves;
constexpr int kPartStride = kHeadDim + 4;   // floats per (row, chunk) partial: o[D], m, l, pad
constexpr int kVStride = kHeadDim + 2;      // LDS row stride (elements) of the staged V tile
constexpr int64_t kMaxKv = 1ll << 20;     // keeps pass 2's per-chunk weights within 32 KiB of LDS

__device__ inline f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ inline f32x4 mfma_f16(uint4 a, uint4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <typename S>
__device__ inline f32x4 mfma16(uint4 a, uint4 b, f32x4 c);
template <> __device__ inline f32x4 mfma16<BF16>(uint4 a, uint4 b, f32x4 c) { return mfma_bf16(a, b, c); }
template <> __device__ inline f32x4 mfma16<F16>(uint4 a, uint4 b, f32x4 c) { return mfma_f16(a, b, c); }

struct AttnShape {
    int64_t B, Q, Lcap, nchunks, max_kv;
    int Hq, Hkv, G;
    float scale;
    int causal;
};

__device__ inline int64_t row_last_key(int64_t kvlen, int64_t Q, int64_t j, int causal)
{
    return causal ? kvlen - Q + j : kvlen - 1;
}

// Pass 1: one workgroup of kAttnWaves waves per (sequence b, chunk c, KV head
// hk), on a 1-D grid ordered so that the workgroups of all KV heads of one
// (b, c) are dispatched together onto one XCD: id L -> XCD L % 8 (the
// hardware's round-robin), heads hk = (L / 8) % Hkv, item (b, c) =
// (L / (8 Hkv)) * 8 + L % 8.  Their key rows [b][pos][0..Hkv)[0..D) are
// contiguous, so each cache line of K and V is wanted by one XCD at one time.
template <typename S>
__global__ __launch_bounds__(kAttnWaves * kWave)
void attn_chunk_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                       const uint16_t *__restrict__ v, const int32_t *__restrict__ kv_len,
                       float *__restrict__ part, AttnShape sh)
{
    // The staged V tiles are dead once each wave holds its V fragments; the P
    // tiles and the wave partials of o then reuse the same bytes.
    typedef uint16_t VTile[kKeysPerWave][kVStride];
    typedef uint16_t PTile[16][kKeysPerWave + 8];
    typedef float OTile[16][kHeadDim + 1];
    constexpr size_t kVBytes = sizeof(VTile) * kAttnWaves;
    constexpr size_t kPOBytes = (sizeof(PTile) + sizeof(OTile)) * kAttnWaves;
    static_assert(kPOBytes <= kVBytes, "P/O tiles must fit in the V staging buffer");
    __shared__ __attribute__((aligned(16))) unsigned char lds[kVBytes];
    __shared__ float xm[kAttnWaves][16], xl[kAttnWaves][16];           // wave partials of max / sum
    VTile *vl = reinterpret_cast<VTile *>(lds);
    PTile *pl = reinterpret_cast<PTile *>(lds);
    OTile *ol = reinterpret_cast<OTile *>(lds + sizeof(PTile) * kAttnWaves);

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g4 = lane >> 4, c16 = lane & 15;
    const int64_t L = blockIdx.x;
    const int hk = (int)((L >> 3) % sh.Hkv);
    const int64_t item = (L >> 3) / sh.Hkv * 8 + (L & 7);
    if (item >= sh.B * sh.nchunks) return;
    const int64_t b = item / sh.nchunks, c = item - b * sh.nchunks;
    // kv_len is device data the host cannot validate; clamping it keeps every
    // access inside the cache and the workspace even for a bad value.
    const int64_t kvlen = min((int64_t)kv_len[b], sh.max_kv);
    const int64_t key0 = c * kChunk;
    const int R = (int)sh.Q * sh.G;                                      // query rows of this KV head

    // Largest position any row of this (b, hk) attends to; chunks past it have no work.
    const int64_t pmax = row_last_key(kvlen, sh.Q, sh.Q - 1, sh.causal);
    if (key0 > pmax) return;

    // --- K fragments for this wave's 64 keys: 4 key tiles x 4 d-chunks -------
    const int64_t wkey0 = key0 + wave * kKeysPerWave;
    uint4 kf[4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
        const int64_t key = wkey0 + kt * 16 + c16;
        const bool ok = key < kvlen;
        const uint16_t *kr = k + (((b * sh.Lcap + (ok ? key : 0)) * sh.Hkv + hk) * kHeadDim) + g4 * 32;
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[kt][s] = ok ? *reinterpret_cast<const uint4 *>(kr + s * 8) : make_uint4(0, 0, 0, 0);
    }
    // --- stage this wave's V tile [64 keys][128 d] in LDS ------------------------
    // lane covers 16 bytes of a key row per step: 16 chunks per row, 4 rows per step.
#pragma unroll
    for (int it = 0; it < kKeysPerWave * (kHeadDim / 8) / kWave; ++it) {
        const int flat = it * kWave + lane;
        const int kr = flat >> 4, dc = (flat & 15) * 8;
        const int64_t key = wkey0 + kr;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (key < kvlen) val = *reinterpret_cast<const uint4 *>(v + ((b * sh.Lcap + key) * sh.Hkv + hk) * kHeadDim + dc);
        uint32_t *dst = reinterpret_cast<uint32_t *>(&vl[wave][kr][dc]);
        dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
    }
    __syncthreads();
    // V as the B operand: lane (g4, c16), d tile dt, step s2 holds keys s2*32 + 8*g4 + e (e < 8), column dt*16 + c16.
    uint4 vf[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            uint16_t tmp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) tmp[e] = vl[wave][s2 * 32 + g4 * 8 + e][dt * 16 + c16];
            vf[dt][s2] = __builtin_bit_cast(uint4, tmp);
        }
    __syncthreads();                                                   // V staging bytes are reused below

    const int ntiles = (R + 15) / 16;
    for (int mt = 0; mt < ntiles; ++mt) {
        // Query row handled as A-operand row c16 of this tile.
        const int ra = mt * 16 + c16;
        const bool ra_ok = ra < R;
        const int ja = ra_ok ? ra / sh.G : 0, ia = ra_ok ? ra - ja * sh.G : 0;
        // Rows of the accumulator layout held by this lane: 4*g4 + i.
        int64_t lastk[4];
        bool rowok[4];
        bool any = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + g4 * 4 + i;
            rowok[i] = r < R;
            lastk[i] = rowok[i] ? row_last_key(kvlen, sh.Q, r / sh.G, sh.causal) : -1;
            rowok[i] = rowok[i] && lastk[i] >= key0;
        }
        // Tile-uniform skip: no row of this tile reaches this chunk.
        {
            const int rlast = mt * 16 + 15 < R ? mt * 16 + 15 : R - 1;
            any = row_last_key(kvlen, sh.Q, rlast / sh.G, sh.causal) >= key0;
        }
        if (!any) continue;

        uint4 qf[4];
        {
            const int64_t h = (int64_t)hk * sh.G + ia;
            const uint16_t *qr = q + ((b * sh.Q + ja) * sh.Hq + h) * kHeadDim + g4 * 32;
#pragma unroll
            for (int s = 0; s < 4; ++s) qf[s] = ra_ok ? *reinterpret_cast<const uint4 *>(qr + s * 8) : make_uint4(0, 0, 0, 0);
        }
        // scores: tile kt -> lane (g4, c16) reg i = row 4*g4 + i, key wkey0 + kt*16 + c16
        float sc[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma16<S>(qf[s], kf[kt][s], acc);
            const int64_t key = wkey0 + kt * 16 + c16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vis = rowok[i] && key <= lastk[i];
                sc[kt][i] = vis ? acc[i] * sh.scale : -INFINITY;
            }
        }
        // chunk max per row
        float mx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
            mx[i] = m;
        }
        if (c16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xm[wave][g4 * 4 + i] = mx[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = g4 * 4 + i;
            mx[i] = fmaxf(fmaxf(xm[0][rr], xm[1][rr]), fmaxf(xm[2][rr], xm[3][rr]));
        }
        // probabilities, row sums, and the bf16 P tile
        float ls[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ls[i] = 0.0f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool vis = sc[kt][i] != -INFINITY;
                const float pv = vis ? expf(sc[kt][i] - mx[i]) : 0.0f;
                ls[i] = ls[i] + pv;
                pl[wave][g4 * 4 + i][kt * 16 + c16] = S::narrow(pv);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float l = ls[i];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) l = l + __shfl_xor(l, off, kWave);
            ls[i] = l;
        }
        if (c16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) xl[wave][g4 * 4 + i] = ls[i];
        }
        __syncthreads();
        // o partial of this wave: P (16 x 64) . V (64 x 128)
        uint4 pf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) pf[s2] = *reinterpret_cast<const uint4 *>(&pl[wave][c16][s2 * 32 + g4 * 8]);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) acc = mfma16<S>(pf[s2], vf[dt][s2], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) ol[wave][g4 * 4 + i][dt * 16 + c16] = acc[i];
        }
        __syncthreads();
        // combine the four wave partials in order and write this chunk's partial
        for (int e = threadIdx.x; e < 16 * kHeadDim; e += kAttnWaves * kWave) {
            const int rr = e / kHeadDim, d = e % kHeadDim;
            const int r = mt * 16 + rr;
            if (r >= R) continue;
            const int j = r / sh.G;
            if (row_last_key(kvlen, sh.Q, j, sh.causal) < key0) continue;
            const int64_t h = (int64_t)hk * sh.G + (r - j * sh.G);
            float* dst = part + (((b * sh.Q + j) * sh.Hq + h) * sh.nchunks + c) * kPartStride;
            const float o = ((ol[0][rr][d] + ol[1][rr][d]) + ol[2][rr][d]) + ol[3][rr][d];
            dst[d] = o;
            if (d == 0) {
                dst[kHeadDim] = fmaxf(fmaxf(xm[0][rr], xm[1][rr]), fmaxf(xm[2][rr], xm[3][rr]));
                dst[kHeadDim + 1] = ((xl[0][rr] + xl[1][rr]) + xl[2][rr]) + xl[3][rr];
            }
        }
        __syncthreads();
    }
}

// Pass 2: one workgroup of kHeadDim threads per query row (b, j, h).
template <typename S>
__global__ __launch_bounds__(kHeadDim)
void attn_merge_kernel(const float *__restrict__ part, const int32_t *__restrict__ kv_len,
                       uint16_t *__restrict__ out, AttnShape sh, int64_t chunk_size)
{
    extern __shared__ float smem[];
    const int64_t row = blockIdx.x;                       // (b * Q + j) * Hq + h
    const int64_t j = (row / sh.Hq) % sh.Q, b = row / (sh.Hq * sh.Q);
    const int d = threadIdx.x;
    const int64_t kvlen = min((int64_t)kv_len[b], sh.max_kv);
    const int64_t lastkey = row_last_key(kvlen, sh.Q, j, sh.causal);
    const int64_t last = lastkey < 0 ? 0 : lastkey / chunk_size;     // a bad kv_len gives garbage, never an out-of-range read
    const float *pr = part + row * sh.nchunks * kPartStride;
    float *wts = smem;                                    // [nchunks]
    float *lws = smem + sh.nchunks;                       // [nchunks]
    __shared__ float red[kHeadDim / kWave];

    float m = -INFINITY;
    for (int64_t cc = d; cc <= last; cc += kHeadDim) m = fmaxf(m, pr[cc * kPartStride + kHeadDim]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    if ((d & 63) == 0) red[d >> 6] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int i = 1; i < kHeadDim / kWave; ++i) m = fmaxf(m, red[i]);
    for (int64_t cc = d; cc <= last; cc += kHeadDim) {
        const float wv = expf(pr[cc * kPartStride + kHeadDim] - m);
        wts[cc] = wv;
        lws[cc] = pr[cc * kPartStride + kHeadDim + 1] * wv;
    }
    __syncthreads();
    float o = 0.0f, l = 0.0f;
#pragma unroll 8
    for (int64_t cc = 0; cc <= last; ++cc) {
        o = o + pr[cc * kPartStride + d] * wts[cc];
        l = l + lws[cc];
    }
    out[row * kHeadDim + d] = S::narrow(o / l);
}

static bi_status check_attn(const void *q, const void *k, const void *v, const void *o, const int32_t *kv_len,
                            int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t dtype)
{
    if (!q || !k || !v || !o || !kv_len) return BI_ERR_NULL;
    if (B < 1 || Q < 1 || Lcap < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
    if (max_kv_len < Q || max_kv_len > Lcap || max_kv_len > kMaxKv) return BI_ERR_SHAPE;
    if (Hkv > 65535 || B * Q * Hq > (1ll << 31) - 1 || Q * (Hq / Hkv) > (1ll << 30) ||
        cdiv(B * cdiv(max_kv_len, kChunk), 8) * 8 * Hkv > (1ll << 31) - 1)
        return BI_ERR_SHAPE;
    if (D != kHeadDim) return BI_ERR_UNSUPPORTED;
    if (dtype != BI_BF16 && dtype != BI_F16) return BI_ERR_DTYPE;
    if (!host_aligned16(q) || !host_aligned16(k) || !host_aligned16(v) || !host_aligned16(o) ||
        ((uintptr_t)kv_len & 3u))
        return BI_ERR_ALIGN;
    return BI_OK;
}

template <typename S>
static void launch_attn(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len, float *part,
                        const AttnShape &sh, int64_t chunk, hipStream_t st)
{
    const int64_t groups = cdiv(sh.B * sh.nchunks, 8);
    hipLaunchKernelGGL((attn_chunk_kernel<S>), dim3((unsigned)(groups * 8 * sh.Hkv)),
                       dim3(kAttnWaves * kWave), 0, st, (const uint16_t *)q, (const uint16_t *)k,
                       (const uint16_t *)v, kv_len, part, sh);
    const size_t smem = (size_t)sh.nchunks * 2 * sizeof(float);
    hipLaunchKernelGGL((attn_merge_kernel<S>), dim3((unsigned)(sh.B * sh.Q * sh.Hq)), dim3(kHeadDim), smem, st,
                       (const float *)part, kv_len, (uint16_t *)o, sh, chunk);
}

}  // namespace bi

using namespace bi;

extern "C" size_t bi_sdpa_workspace_bytes(int64_t B, int64_t Q, int64_t max_kv_len, int32_t Hq, int32_t D)
{
    if (B < 1 || Q < 1 || max_kv_len < 1 || Hq < 1 || D != kHeadDim) return 0;
    return (size_t)B * Q * Hq * cdiv(max_kv_len, kChunk) * kPartStride * sizeof(float);
}

extern "C" bi_status bi_sdpa(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                             int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                             int32_t D, float scale, int32_t causal, int32_t dtype, void *ws, size_t ws_bytes,
                             hipStream_t stream)
{
    bi_status s = check_attn(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, dtype);
    if (s != BI_OK) return s;
    if (!ws) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    if (ws_bytes < bi_sdpa_workspace_bytes(B, Q, max_kv_len, Hq, D)) return BI_ERR_WORKSPACE;
    AttnShape sh{B, Q, Lcap, cdiv(max_kv_len, kChunk), max_kv_len, Hq, Hkv, Hq / Hkv, scale, causal ? 1 : 0};
    (void)hipGetLastError();
    if (dtype == BI_BF16) launch_attn<BF16>(q, k, v, o, kv_len, (float *)ws, sh, kChunk, stream);
    else launch_attn<F16>(q, k, v, o, kv_len, (float *)ws, sh, kChunk, stream);
    return launch_status();
}
