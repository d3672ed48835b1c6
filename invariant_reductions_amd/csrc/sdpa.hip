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
#include <algorithm>

#include "common.hpp"

namespace bi {

constexpr int kChunk = 256;          // keys per chunk (frozen)
constexpr int kHeadDim = 128;        // D supported by this build
constexpr int kAttnWaves = 4;        // waves per chunk workgroup (frozen: 64 keys each)
constexpr int kKeysPerWave = kChunk / kAttnWaves;
constexpr int kPartStride = kHeadDim + 4;   // floats per (row, chunk) partial: o[D], m, l, pad
constexpr int64_t kMaxKv = 1ll << 20;     // keeps pass 2's per-chunk weights within 32 KiB of LDS
constexpr int kAttnMinTiles = 4;     // fewest query-row tiles (of 16) per work item when a prompt is split

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
    int64_t B, Q, Lcap, nchunks, max_kv, nmg;     // nmg: row groups of mgt 16-row tiles per (b, c, hk)
    int Hq, Hkv, G, mgt;
    float scale;
    int causal;
    int64_t ks, hs;       // cache strides (elements) between consecutive keys and between KV heads
};

__device__ inline int64_t row_last_key(int64_t kvlen, int64_t Q, int64_t j, int causal)
{
    return causal ? kvlen - Q + j : kvlen - 1;
}

// In-place 8 x 8 transpose of 16-bit elements held by one lane: row e is
// m[e] (elements j = 0..7); afterwards m[j] holds column j.  Pairs of rows
// are interleaved at 16-bit granularity with v_perm_b32; the rest is
// register selection.  Every input is read before any output is written.
__device__ inline void transpose8x8_b16(uint4 (&m)[8])
{
    const uint4 (&in)[8] = m;
    uint32_t t0[4][4], t1[4][4];        // t0[p][w]: (row 2p, row 2p+1) of column 2w; t1: column 2w+1
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t a[4] = {in[2 * p].x, in[2 * p].y, in[2 * p].z, in[2 * p].w};
        const uint32_t b[4] = {in[2 * p + 1].x, in[2 * p + 1].y, in[2 * p + 1].z, in[2 * p + 1].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            t0[p][w] = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);   // lo16(a), lo16(b)
            t1[p][w] = __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);   // hi16(a), hi16(b)
        }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        m[2 * w] = make_uint4(t0[0][w], t0[1][w], t0[2][w], t0[3][w]);
        m[2 * w + 1] = make_uint4(t1[0][w], t1[1][w], t1[2][w], t1[3][w]);
    }
}

// Pass 1 as a persistent, software-pipelined kernel.  Work item = (sequence
// b, chunk c, KV head hk, row group mg) -- mg picks sh.mgt of the 16-row query
// tiles, so a long prompt with few sequences spreads over many workgroups (at
// decode and verify sizes there is one group); a fixed grid of workgroups
// walks the item ids
// t = blockIdx.x, blockIdx.x + gridDim.x, ...  With u = t / nmg and mg = t %
// nmg, the ids are ordered so that the items of all KV heads of one (b, c)
// are processed together on one XCD at decode sizes (nmg = 1): id u -> XCD u
// % 8 (the hardware's round-robin when gridDim.x % 8 == 0), hk = (u / 8) %
// Hkv, (b, c) = (u / (8 Hkv)) * 8 + u % 8; their key rows
// [b][pos][0..Hkv)[0..D) are contiguous in the cache.  Inside an item, wave w
// owns keys [64w, 64w + 64) of the chunk (the frozen tree above).  The
// resident workgroups drift out of step, so the cache streams without the
// idle gaps of a grid that starts and finishes its workgroups in rounds.
//
// Register layouts (lane = 16 g4 + c16):
//   K  : kf[kt][s] = key 16kt + c16, d in [32 g4 + 8 s, +8)   (MFMA B of q . k)
//   V  : rows loaded as vr[s2][e] = key 32 s2 + 8 g4 + e, d in [8 c16, +8),
//        transposed in place to vr[s2][j] = those 8 keys at d = 8 c16 + j,
//        the MFMA B operand of P . V (k slot 8 g4 + e of step s2 = key
//        32 s2 + 8 g4 + e, column c16 = d 8 c16 + j of output tile j).
template <typename S, bool MG>
__global__ __launch_bounds__(kAttnWaves * kWave, 2)
void attn_chunk_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                       const uint16_t *__restrict__ v, const int32_t *__restrict__ kv_len,
                       float *__restrict__ part, AttnShape sh, int64_t nid)
{
    typedef uint16_t PTile[16][kKeysPerWave + 8];
    typedef float OTile[16][kHeadDim + 4];
    __shared__ __attribute__((aligned(16))) PTile pl[kAttnWaves];
    __shared__ __attribute__((aligned(16))) OTile ol[kAttnWaves];
    __shared__ float xm[kAttnWaves][16], xl[kAttnWaves][16];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g4 = lane >> 4, c16 = lane & 15;
    const int R = (int)sh.Q * sh.G;                                      // query rows per KV head
    const int ntm = (R + 15) / 16;
    const int64_t nitems = sh.B * sh.nchunks;

    // b, c, hk and the clamped length of one item; kv_len is device data the
    // host cannot validate, so it is clamped to max_kv, which keeps every
    // access inside the cache and the workspace even for a bad value.
    struct Item {
        int b, c, hk, kvlen, mg;
    };
    auto decode = [&](int64_t t0) {
        Item it;
        const int64_t t = MG ? t0 / sh.nmg : t0;
        it.mg = MG ? (int)(t0 - t * sh.nmg) : 0;
        it.hk = (int)((t >> 3) % sh.Hkv);
        const int64_t bc = (t >> 3) / sh.Hkv * 8 + (t & 7);
        const bool exists = bc < nitems;
        it.b = exists ? (int)(bc / sh.nchunks) : 0;
        it.c = exists ? (int)(bc - (int64_t)it.b * sh.nchunks) : -1;
        it.kvlen = (int)min((int64_t)kv_len[it.b], sh.max_kv);
        return it;
    };
    const int Qi = (int)sh.Q;
    auto last_key = [&](int kvlen, int j) { return sh.causal ? kvlen - Qi + j : kvlen - 1; };
    // an item has work when it exists and its first key is visible to the last row of its group
    auto has_work = [&](const Item &it) {
        if (!MG) return it.c >= 0 && it.c * kChunk <= last_key(it.kvlen, Qi - 1);
        const int rl = min(R, (it.mg + 1) * sh.mgt * 16) - 1;
        return it.c >= 0 && it.c * kChunk <= last_key(it.kvlen, rl / sh.G);
    };
    auto next_id = [&](int64_t t) {
        for (; t < nid; t += gridDim.x)
            if (has_work(decode(t))) break;
        return t;
    };
    // Loads are unconditional: a missing key (position >= kv_len) reads the
    // item's first key, which always exists (the item has work), and the
    // value is then replaced by zero.  Bases are wave-uniform; per-lane
    // offsets are 32-bit.
    const int rs = (int)sh.ks;                                           // elements between keys
    auto item_base = [&](const uint16_t *p, const Item &it) {
        return p + (int64_t)it.b * sh.Lcap * sh.Hkv * kHeadDim + (int64_t)it.c * kChunk * rs + (int64_t)it.hk * sh.hs;
    };
    // keys of this wave that exist
    auto wave_valid = [&](const Item &it) { return min(max(it.kvlen - (it.c * kChunk + wave * kKeysPerWave), 0), kKeysPerWave); };
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    auto load_k = [&](const Item &it, uint4 (&kf)[4][4]) {
        const uint16_t *kb = item_base(k, it);
        const int nv = wave_valid(it);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int kk = kt * 16 + c16;
            const bool ok = kk < nv;
            const uint16_t *kr = kb + (ok ? wave * kKeysPerWave + kk : 0) * rs + g4 * 32;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 x = *reinterpret_cast<const uint4 *>(kr + s * 8);
                kf[kt][s] = ok ? x : zero4;
            }
        }
    };
    auto load_v = [&](const Item &it, uint4 (&vr)[2][8]) {
        const uint16_t *vb = item_base(v, it);
        const int nv = wave_valid(it);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = s2 * 32 + g4 * 8 + e;
                const bool ok = kk < nv;
                const uint4 x = *reinterpret_cast<const uint4 *>(vb + (ok ? wave * kKeysPerWave + kk : 0) * rs + c16 * 8);
                vr[s2][e] = ok ? x : zero4;
            }
    };
    // q rows of M tile mt as the MFMA A operand: row c16 of the tile, d in [32 g4 + 8 s, +8)
    auto load_q = [&](const Item &it, int mt, uint4 (&qf)[4]) {
        const int ra = mt * 16 + c16;
        const bool ok = ra < R;
        const int ja = ok ? ra / sh.G : 0, ia = ok ? ra - ja * sh.G : 0;
        const uint16_t *qb = q + ((int64_t)it.b * sh.Q * sh.Hq + (int64_t)it.hk * sh.G) * kHeadDim;
        const uint16_t *qr = qb + (ja * sh.Hq + ia) * kHeadDim + g4 * 32;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 x = *reinterpret_cast<const uint4 *>(qr + s * 8);
            qf[s] = ok ? x : zero4;
        }
    };

    uint4 kf[4][4], vr[2][8], qf[4];
    for (int64_t t = next_id(blockIdx.x); t < nid; t = next_id(t + gridDim.x)) {
        const Item it = decode(t);
        const int key0 = it.c * kChunk;
        const int wkey0 = key0 + wave * kKeysPerWave;
        const int mt0 = MG ? it.mg * sh.mgt : 0, mt1 = MG ? min(ntm, mt0 + sh.mgt) : ntm;
        load_q(it, mt0, qf);
        load_k(it, kf);
        load_v(it, vr);
        transpose8x8_b16(vr[0]);                       // this item's V as the P . V B operand
        transpose8x8_b16(vr[1]);

        for (int mt = mt0; mt < mt1; ++mt) {
            // Rows of the accumulator layout held by this lane: 4 g4 + i.
            int lastk[4];
            bool rowok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = mt * 16 + g4 * 4 + i;
                rowok[i] = r < R;
                lastk[i] = rowok[i] ? last_key(it.kvlen, r / sh.G) : -1;
                rowok[i] = rowok[i] && lastk[i] >= key0;
            }
            // Tile-uniform skip: no row of this tile reaches this chunk.
            const int rlast = mt * 16 + 15 < R ? mt * 16 + 15 : R - 1;
            const bool any = last_key(it.kvlen, rlast / sh.G) >= key0;
            if (mt > mt0) load_q(it, mt, qf);

            // scores: tile kt -> lane (g4, c16) reg i = row 4 g4 + i, key wkey0 + 16 kt + c16
            float sc[4][4];
            if (any) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc = mfma16<S>(qf[s], kf[kt][s], acc);
                    const int key = wkey0 + kt * 16 + c16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool vis = rowok[i] && key <= lastk[i];
                        sc[kt][i] = vis ? acc[i] * sh.scale : -INFINITY;
                    }
                }
            }
            if (!any) continue;

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
            for (int j = 0; j < 8; ++j) {
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) acc = mfma16<S>(pf[s2], vr[s2][j], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) ol[wave][g4 * 4 + i][c16 * 8 + j] = acc[i];
            }
            __syncthreads();
            // combine the four wave partials in order and write this chunk's
            // partial: thread -> row t / 16 of the tile, d in [8 (t % 16), +8)
            {
                const int rr = threadIdx.x >> 4, dg = threadIdx.x & 15;
                const int r = mt * 16 + rr;
                if (r < R) {
                    const int j = r / sh.G;
                    if (last_key(it.kvlen, j) >= key0) {
                        const int64_t h = (int64_t)it.hk * sh.G + (r - j * sh.G);
                        float *dst = part + ((((int64_t)it.b * sh.Q + j) * sh.Hq + h) * sh.nchunks + it.c) * kPartStride;
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int d = dg * 8 + half * 4;
                            const float4 o0 = *reinterpret_cast<const float4 *>(&ol[0][rr][d]);
                            const float4 o1 = *reinterpret_cast<const float4 *>(&ol[1][rr][d]);
                            const float4 o2 = *reinterpret_cast<const float4 *>(&ol[2][rr][d]);
                            const float4 o3 = *reinterpret_cast<const float4 *>(&ol[3][rr][d]);
                            float4 o;
                            o.x = ((o0.x + o1.x) + o2.x) + o3.x;
                            o.y = ((o0.y + o1.y) + o2.y) + o3.y;
                            o.z = ((o0.z + o1.z) + o2.z) + o3.z;
                            o.w = ((o0.w + o1.w) + o2.w) + o3.w;
                            *reinterpret_cast<float4 *>(dst + d) = o;
                        }
                        if (dg == 0) {
                            dst[kHeadDim] = fmaxf(fmaxf(xm[0][rr], xm[1][rr]), fmaxf(xm[2][rr], xm[3][rr]));
                            dst[kHeadDim + 1] = ((xl[0][rr] + xl[1][rr]) + xl[2][rr]) + xl[3][rr];
                        }
                    }
                }
            }
            __syncthreads();
        }
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
    // the first kMergeEarly chunks' o values do not depend on the max: request
    // them now, with the m values, rather than after the weights are known
    constexpr int kMergeEarly = 8;
    float oe[kMergeEarly];
#pragma unroll
    for (int cc = 0; cc < kMergeEarly; ++cc) oe[cc] = cc <= last ? pr[cc * kPartStride + d] : 0.0f;

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
#pragma unroll
    for (int cc = 0; cc < kMergeEarly; ++cc) {
        if (cc <= last) {
            o = o + oe[cc] * wts[cc];
            l = l + lws[cc];
        }
    }
#pragma unroll 8
    for (int64_t cc = kMergeEarly; cc <= last; ++cc) {
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
    // item ids (padded to whole groups of 8); a persistent grid of two
    // workgroups per CU, a multiple of 8 so that a workgroup stays on one XCD
    const int64_t nid = cdiv(sh.B * sh.nchunks, 8) * 8 * sh.Hkv * sh.nmg;
    const int64_t grid = std::min<int64_t>(nid, (int64_t)device_cu_count() * 2 / 8 * 8);
    if (sh.nmg > 1)
        launch_kernel((attn_chunk_kernel<S, true>), dim3((unsigned)grid), dim3(kAttnWaves * kWave), 0, st,
                      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, kv_len, part, sh, nid);
    else
        launch_kernel((attn_chunk_kernel<S, false>), dim3((unsigned)grid), dim3(kAttnWaves * kWave), 0, st,
                      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, kv_len, part, sh, nid);
    const size_t smem = (size_t)sh.nchunks * 2 * sizeof(float);
    launch_kernel((attn_merge_kernel<S>), dim3((unsigned)(sh.B * sh.Q * sh.Hq)), dim3(kHeadDim), smem, st,
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
                             int32_t D, float scale, int32_t causal, int32_t dtype, int32_t kv_layout, void *ws,
                             size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_attn(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, dtype);
    if (s != BI_OK) return s;
    if (kv_layout != 0 && kv_layout != 1) return BI_ERR_SHAPE;
    if (!ws) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    if (ws_bytes < bi_sdpa_workspace_bytes(B, Q, max_kv_len, Hq, D)) return BI_ERR_WORKSPACE;
    // kv_layout 0: [B, Lcap, Hkv, D]; 1: [B, Hkv, Lcap, D] (head-major)
    const int64_t ks = kv_layout ? (int64_t)D : (int64_t)Hkv * D, hs = kv_layout ? Lcap * D : (int64_t)D;
    // query-row groups: when the (sequence, chunk, head) items alone give fewer
    // than two per workgroup slot, split the rows so that about 4096 ids exist
    // (half of a causal prompt's (chunk, rows) pairs being empty), never under
    // kAttnMinTiles tiles each; otherwise one group
    const int64_t ntm = cdiv(Q * (Hq / Hkv), 16), nbase = cdiv(B * cdiv(max_kv_len, kChunk), 8) * 8 * Hkv;
    const int64_t ngroups = nbase >= 1024 ? 1 : std::max<int64_t>(1, cdiv(4096, nbase));
    const int64_t mgt = std::max<int64_t>(kAttnMinTiles, cdiv(ntm, ngroups));
    AttnShape sh{B, Q, Lcap, cdiv(max_kv_len, kChunk), max_kv_len, cdiv(ntm, mgt), Hq, Hkv, Hq / Hkv, (int)std::min<int64_t>(mgt, ntm),
                 scale, causal ? 1 : 0, ks, hs};
    (void)hipGetLastError();
    if (dtype == BI_BF16) launch_attn<BF16>(q, k, v, o, kv_len, (float *)ws, sh, kChunk, stream);
    else launch_attn<F16>(q, k, v, o, kv_len, (float *)ws, sh, kChunk, stream);
    return launch_status();
}
