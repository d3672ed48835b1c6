// sdpa.hip -- batch-invariant decode / verify / prefill attention on gfx950.
//
// Sources: "Fix/speculative shape invariance" (Problem: two-pass SDPA derived
// its split count from the query length; Changes: the single-query split
// configuration for a query alone or inside a short causal block);
// "Batch-invariant kernels: why temperature-0 decoding is still
// nondeterministic" (Case 6: a fixed split SIZE with a varying number of
// splits, KV cache updated before the kernel; Try this, item 5).
//
// Reduction tree of one query row r at position p (frozen; depends on p only):
//   Chunks -- keys are cut into chunks of kChunk = 256 positions; chunk c holds
//   keys [256c, 256c + 256) and is handled by one workgroup for all query rows
//   of one (sequence, KV head).  Inside the chunk, wave w owns keys
//   [64w, 64w + 64):
//     s_t   = (scale log2 e) * (q . k_t)   the score in base-2 units (the
//                                    constant rounded once); q . k_t is one
//                                    16x16x32 MFMA chain over d (4 steps;
//                                    step s takes d in [32s, 32s + 32), lane
//                                    group g supplies the 8 at 32s + 8g)
//     m_c   = max of s_t over the chunk's keys t <= p (exact, order-free)
//     p_t   = 2^(s_t - m_c) (= exp of the natural-unit difference; the
//             hardware's base-2 exponential); keys t > p contribute exactly +0
//     l_c   = sum p_t: per lane over its 4 key tiles in order, then a xor
//             butterfly over the 16 lanes of a row (1, 2, 4, 8), then waves in
//             order 0..3
//     o_c   = sum p_t * v_t with p_t carried as two 16-bit parts, hi =
//             RNE(p_t) and lo = RNE(p_t - hi): MFMA over the wave's 64 keys,
//             the lo products (2 steps of 32 keys) before the hi products,
//             then the four wave partials added in order 0..3
//   Ranges -- chunks are grouped in ranges of kRange = 16 (4096 keys); for the
//   chunks 16r .. min(16r + 15, floor(p / 256)) of range r:
//     M_r = max m_c (exact);  w_c = 2^(m_c - M_r)
//     o_r = sum o_c * w_c and l_r = sum l_c * w_c in ascending c
//   Row -- over the ranges 0 .. floor(p / 4096):
//     M = max M_r (exact);  u_r = 2^(M_r - M)
//     o = sum o_r * u_r and l = sum l_r * u_r in ascending r;  out = RNE(o / l)
// A query row never meets another row except inside an MFMA (rows are
// independent there), so the number of queries Q, the GQA group, the batch and
// where the row sits in its tile leave its bits unchanged; a query of a causal
// verify block and a lone query at the same position reduce identically.
//
// The chunk level is one launch (attn_kernel); the range and row levels are a
// second (attn_merge_kernel), one workgroup per query row -- or, for many
// short (sequence, KV head) groups, the same workgroup that wrote a group's
// chunk partials (attn_kernel's WHOLE form, one launch); prompts take
// attn_prefill_kernel, one launch without partials.
#include <algorithm>
#include <mutex>

#include "common.hpp"

namespace bi {

constexpr int kChunk = 256;          // keys per chunk (frozen)
constexpr int kRange = 16;           // chunks per merge range (frozen: 4096 keys)
constexpr int kHeadDim = 128;        // D supported by this build
constexpr int kAttnWaves = 4;        // waves per chunk workgroup (frozen: 64 keys each)
constexpr int kKeysPerWave = kChunk / kAttnWaves;
constexpr int kPartStride = kHeadDim + 4;   // floats per (row, chunk) partial: o[D], m, l, pad
typedef int i32x2 __attribute__((ext_vector_type(2)));
// The whole-group form (attn_kernel's WHOLE): at most kWholeMaxChunks chunks
// per group with its chunk partials in the workspace, or with at most
// kWholeLdsParts (query row, chunk) partials per group (4 rows over 12
// chunks, 8 over 6) in the workgroup's LDS.  Up to kWholeMaxChunks chunks an
// instantiation with room for kWholeLdsSmall partials keeps them at a fixed
// stride of kWholeMaxChunks per row (groups of at most 8 rows), which leaves
// its registers as they were without LDS partials.
constexpr int64_t kWholeMaxChunks = 4;
constexpr int kWholeLdsParts = 48, kWholeLdsSmall = 32;
constexpr int64_t kMaxKv = 1ll << 20;
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
    int64_t B, Q, Lcap, nchunks, nranges, max_kv, nmg;  // nmg: row groups of mgt 16-row tiles per (b, c, hk)
    int Hq, Hkv, G, mgt;
    float scale;          // the base-2 score scale: the caller's scale x log2(e)
    int causal;
    int64_t ks, hs;       // cache strides (elements) between consecutive keys and between KV heads
    int cps;              // chunks per work item: 1; the split variant's run; WHOLE: all of them
    int64_t nsplit;       // work items per (sequence, KV head): nchunks; the split count; WHOLE: 1
};

struct AttnBufs {
    const uint16_t *q, *k, *v;
    const int32_t *kv_len;
    uint16_t *o;
    float *part;          // chunk partials [B][Hkv][nchunks][Q G][kPartStride] (see attn_part_block)
};

// The workspace holds the chunk partials group-major: for (sequence b, KV
// head hk, chunk or split c) one block of the group's Q G query rows (row r
// = query j G + head i), kPartStride floats each; a row's partials of
// consecutive chunks are Q G kPartStride floats apart.  First float of the
// block:
__device__ inline int64_t attn_part_block(const AttnShape &sh, int64_t b, int64_t hk, int64_t c)
{
    return ((b * sh.Hkv + hk) * sh.nchunks + c) * (sh.Q * sh.G) * kPartStride;
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

__device__ inline int attn_last_key(int kvlen, int Q, int j, int causal) { return causal ? kvlen - Q + j : kvlen - 1; }

__device__ inline int64_t attn_row(const AttnShape &sh, int b, int hk, int rl)
{
    const int j = rl / sh.G;
    return ((int64_t)b * sh.Q + j) * sh.Hq + (int64_t)hk * sh.G + (rl - j * sh.G);
}

// Scores are kept in base-2 units: s = (q . k) x scale log2(e), the constant
// rounded once on the host (AttnShape::scale), so that every exponential of
// the softmax -- exp(s_nat - m_nat) = 2^(s - m) -- is the hardware's base-2
// exponential of a difference.  Every attention kernel here takes its
// exponentials from this one function and its scores from that one
// constant, so their trees stay bit-compatible with each other.
constexpr float kLog2e = 1.44269504088896341f;
__device__ inline float attn_exp(float x) { return __builtin_amdgcn_exp2f(x); }

// A DPP lane move inside rows of 16 lanes (every lane active).
template <int CTRL>
__device__ inline float dpp_move(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E;          // quad permutes [1,0,3,2] and [2,3,0,1]
constexpr int kDppHalfMirror = 0x141, kDppMirror = 0x140;

// The xor butterfly over the 16 lanes of a row (partners at distance 1, 2, 4,
// 8; each lane adds its own value and its partner's).  Distances 1 and 2 are
// quad permutes; once a quad holds one value, the half-row mirror reaches the
// partner quad's value, and once a half-row holds one value the row mirror
// reaches the other half's -- the operands of the xor butterfly, without a
// trip through the LDS unit.
__device__ inline float row16_sum(float l)
{
    l = l + dpp_move<kDppXor1>(l);
    l = l + dpp_move<kDppXor2>(l);
    l = l + dpp_move<kDppHalfMirror>(l);
    return l + dpp_move<kDppMirror>(l);
}
__device__ inline float row16_max(float m)
{
    m = fmaxf(m, dpp_move<kDppXor1>(m));
    m = fmaxf(m, dpp_move<kDppXor2>(m));
    m = fmaxf(m, dpp_move<kDppHalfMirror>(m));
    return fmaxf(m, dpp_move<kDppMirror>(m));
}

// RNE of two floats to the 16-bit type, packed (a in the low half), by one
// packed conversion.
template <typename S>
__device__ inline uint32_t narrow2(float a, float b)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    if constexpr (std::is_same_v<S, BF16>) {
        typedef __bf16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
    } else {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, h2));
    }
}

// Writes out = RNE(o / l) for the four d values of one quad.
template <typename S>
__device__ inline void attn_store_out(uint16_t *dst, float4 o, float l)
{
    uint2 pk;
    pk.x = (uint32_t)S::narrow(o.x / l) | ((uint32_t)S::narrow(o.y / l) << 16);
    pk.y = (uint32_t)S::narrow(o.z / l) | ((uint32_t)S::narrow(o.w / l) << 16);
    *reinterpret_cast<uint2 *>(dst) = pk;
}

// The range and row levels of attn_merge_kernel for the query rows of one
// (sequence b, KV head hk) group (at most 16 rows), by one workgroup of
// kAttnWaves waves: thread -> (row tid / 32 + 8 k, d in [4 (tid % 32), +4)),
// ranges walked one after another with the same arithmetic in the same
// order: M = max of the row's chunk maxima; per range r, M_r, o_r and l_r
// over its chunks ascending; o and l as the sum of o_r exp(M_r - M) over the
// ranges ascending (the first term assigned, not added to 0); out = RNE(o/l).
// The partials were written by this workgroup: plain loads see them.  lds:
// the group's partials in LDS (row rr's chunk c at (rr lcs + c)
// kPartStride), or null for the workspace.
template <typename S>
__device__ inline void attn_merge_rows(const AttnBufs &bf, const AttnShape &sh, int b, int hk, int kvlen,
                                       const float *lds, int lcs)
{
    const int R = (int)sh.Q * sh.G;
    const int quad = threadIdx.x & 31;
    for (int rr = threadIdx.x >> 5; rr < R; rr += kAttnWaves * kWave / 32) {
        const int j = rr / sh.G;
        const int lk = attn_last_key(kvlen, (int)sh.Q, j, sh.causal);
        if (lk < 0) continue;
        const int64_t row = ((int64_t)b * sh.Q + j) * sh.Hq + (int64_t)hk * sh.G + (rr - j * sh.G);
        // row rr's partial of chunk c at pr + c cs
        const float *pr = lds ? lds + (int64_t)rr * lcs * kPartStride
                              : bf.part + attn_part_block(sh, b, hk, 0) + (int64_t)rr * kPartStride;
        const int64_t cs = lds ? kPartStride : R * (int64_t)kPartStride;
        const int nch = lk / kChunk + 1, nr = (nch + kRange - 1) / kRange;
        float M = -INFINITY;
        for (int c = 0; c < nch; ++c) M = fmaxf(M, pr[c * cs + kHeadDim]);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float l = 0.0f;
        for (int r = 0; r < nr; ++r) {
            const int c0 = r * kRange, n = min(nch - c0, kRange);
            float Mr = pr[c0 * cs + kHeadDim];
            for (int i = 1; i < n; ++i) Mr = fmaxf(Mr, pr[(c0 + i) * cs + kHeadDim]);
            float w = attn_exp(pr[c0 * cs + kHeadDim] - Mr);
            float4 ov = *reinterpret_cast<const float4 *>(pr + c0 * cs + quad * 4);
            float4 orr = make_float4(ov.x * w, ov.y * w, ov.z * w, ov.w * w);
            float lr = pr[c0 * cs + kHeadDim + 1] * w;
            for (int i = 1; i < n; ++i) {
                const float *pc = pr + (c0 + i) * cs;
                w = attn_exp(pc[kHeadDim] - Mr);
                ov = *reinterpret_cast<const float4 *>(pc + quad * 4);
                orr.x = orr.x + ov.x * w;
                orr.y = orr.y + ov.y * w;
                orr.z = orr.z + ov.z * w;
                orr.w = orr.w + ov.w * w;
                lr = lr + pc[kHeadDim + 1] * w;
            }
            const float u = attn_exp(Mr - M);
            const float4 tv = make_float4(orr.x * u, orr.y * u, orr.z * u, orr.w * u);
            const float tl = lr * u;
            if (r == 0) {
                o = tv;
                l = tl;
            } else {
                o.x = o.x + tv.x;
                o.y = o.y + tv.y;
                o.z = o.z + tv.z;
                o.w = o.w + tv.w;
                l = l + tl;
            }
        }
        attn_store_out<S>(bf.o + row * kHeadDim + quad * 4, o, l);
    }
}

// The kernel: a persistent, software-pipelined walk over work items.  Work
// item = (sequence b, chunk c, KV head hk, row group mg) -- mg picks sh.mgt of
// the 16-row query tiles, so a long prompt with few sequences spreads over
// many workgroups (at decode and verify sizes there is one group); a fixed
// grid of workgroups walks the item ids t = blockIdx.x, blockIdx.x +
// gridDim.x, ...  With u = t / nmg and mg = t % nmg, the ids are ordered so
// that the items of all KV heads of one (b, c) are processed together on one
// XCD at decode sizes (nmg = 1): id u -> XCD u % 8 (the hardware's
// round-robin when gridDim.x % 8 == 0), hk = (u / 8) % Hkv, (b, c) = (u / (8
// Hkv)) * 8 + u % 8.  Inside an item, wave w owns keys [64w, 64w + 64) of the
// chunk (the frozen tree above).  The next item's K and q are requested as
// soon as the current item's last scores have read them (in flight during the
// softmax, P . V, the arrival handshake and any merge), its V once the
// current item is done (in flight during the next scores).
//
// Register layouts (lane = 16 g4 + c16):
//   K  : kf[kt][s] = key 16kt + c16, d in [32 s + 8 g4, +8)   (MFMA B of q . k)
//   V  : rows loaded as vr[s2][e] = key 32 s2 + 8 g4 + e, d in [8 c16, +8),
//        transposed in place to vr[s2][j] = those 8 keys at d = 8 c16 + j,
//        the MFMA B operand of P . V (k slot 8 g4 + e of step s2 = key
//        32 s2 + 8 g4 + e, column c16 = d 8 c16 + j of output tile j).
//
// SPL: the split comparison variant (one 16-row tile per item, nmg == 1).
// Its item is a run of sh.cps consecutive chunks -- a split whose length
// follows the caller's split count -- walked in order by one workgroup with
// the softmax state carried across chunks (o and l rescaled to the running
// max); the split's (o, m, l) is the partial, or with a single split the
// output itself.  The tree then depends on the split count; it exists only
// to price the invariant tree.
//
// WHOLE: the invariant tree for many (sequence, KV head) groups of at most
// 32 query rows (nmg == 1): the item is a group with all its chunks, walked
// by one workgroup; every chunk's partial is formed exactly as above -- in
// the workgroup's LDS for groups of at most kWholeLdsRows rows, else in the
// workspace -- and after the last one the same workgroup reads them back and
// runs attn_merge_kernel's range and row levels for the group's rows: one
// launch, and the partials never leave the workgroup's own view.  The walk
// takes the group's last chunk first, then the others in order: that chunk
// is the one a decoding context fills gradually, and its few rows, requested
// at the start, come back ahead of the full chunks' traffic instead of
// behind all of it at the end.  Each partial lands at its own chunk index,
// so the order of the walk never reaches the merge.
// WLP: the (query row, chunk) partials the WHOLE form's LDS holds.
template <typename S, bool MG, bool SPL = false, bool WHOLE = false, int WLP = 0>
__global__ __launch_bounds__(kAttnWaves * kWave, 2)
void attn_kernel(AttnBufs bf, const int32_t *__restrict__ kv_len, AttnShape sh, int64_t nid)
{
    constexpr bool RUNS = SPL || WHOLE;                                  // an item walks a run of chunks
    static_assert(!(WHOLE && (MG || SPL)), "the whole-group form has one row group and no splits");
    typedef uint16_t PTile[16][kKeysPerWave + 8];
    typedef float OTile[16][kHeadDim + 4];
    __shared__ __attribute__((aligned(16))) PTile phi[kAttnWaves], plo[kAttnWaves];
    __shared__ __attribute__((aligned(16))) OTile ol[kAttnWaves];
    __shared__ float xm[kAttnWaves][16], xl[kAttnWaves][16];
    static_assert(WHOLE == (WLP > 0), "LDS partials belong to the whole-group form");
    __shared__ __attribute__((aligned(16))) float wpart[WHOLE ? WLP * kPartStride : 4];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g4 = lane >> 4, c16 = lane & 15;
    const int R = (int)sh.Q * sh.G;                                      // query rows per KV head
    const int ntm = (R + 15) / 16;
    const int64_t nitems = sh.B * sh.nsplit;
    const int Qi = (int)sh.Q;
    // WHOLE with few (row, chunk) partials: those in LDS
    constexpr bool WBIG = WLP > kWholeLdsSmall;                       // launched for > kWholeMaxChunks chunks only
    const bool lds_parts = WHOLE && (WBIG || R * (int)kWholeMaxChunks <= WLP);
    const int lcs = WBIG ? (int)sh.nchunks : (int)kWholeMaxChunks;   // LDS partials per row

    // The sequence lengths, clamped to max_kv (device data the host cannot
    // validate: the clamp keeps every access inside the cache and the
    // workspace even for a bad value), are read with scalar loads (a
    // wave-uniform index into a read-only argument): a vector-memory read
    // inside the walk would make the wave wait for every load in flight, one
    // counter covering them all.
    auto seq_len = [&](int b) {
        return (int)min((int64_t)kv_len[__builtin_amdgcn_readfirstlane(b)], sh.max_kv);
    };
    // b, c, hk and the clamped length of one item
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
        it.b = exists ? (int)(bc / sh.nsplit) : 0;
        it.c = exists ? (int)(bc - (int64_t)it.b * sh.nsplit) * (RUNS ? sh.cps : 1) : -1;
        it.kvlen = seq_len(it.b);
        // WHOLE: the walk starts at the group's last chunk (see below)
        if (WHOLE && exists) it.c = max(attn_last_key(it.kvlen, Qi, (R - 1) / sh.G, sh.causal), 0) / kChunk;
        return it;
    };
    auto last_key = [&](int kvlen, int j) { return attn_last_key(kvlen, Qi, j, sh.causal); };
    // rows [r0, r1) of an item's row group
    auto group_rows = [&](const Item &it, int &r0, int &r1) {
        r0 = MG ? it.mg * sh.mgt * 16 : 0;
        r1 = MG ? min(R, r0 + sh.mgt * 16) : R;
    };
    // last key any row of the item's group sees
    auto group_last_key = [&](const Item &it) {
        int r0, r1;
        group_rows(it, r0, r1);
        return last_key(it.kvlen, (r1 - 1) / sh.G);
    };
    // an item has work when it exists and its first key is visible to the last row of its group
    auto has_work = [&](const Item &it) { return it.c >= 0 && it.c * kChunk <= group_last_key(it); };
    auto next_id = [&](int64_t t) {
        for (; t < nid; t += gridDim.x)
            if (has_work(decode(t))) break;
        return t;
    };
    // Keys at or past kv_len are not read: a lane whose key is missing reads
    // the item's first key (which always exists) instead.  Nothing is
    // selected on the loaded values here -- a select would make the wave wait
    // for each load as it is issued; the scores of missing keys (and padding
    // rows of q) are masked after the product, and missing V rows are zeroed
    // just before P . V reads them.  Bases are wave-uniform; per-lane offsets
    // are 32-bit.
    const int rs = (int)sh.ks;                                           // elements between keys
    auto item_base = [&](const uint16_t *p, const Item &it) {
        return p + (int64_t)it.b * sh.Lcap * sh.Hkv * kHeadDim + (int64_t)it.c * kChunk * rs + (int64_t)it.hk * sh.hs;
    };
    auto wave_valid = [&](const Item &it) { return min(max(it.kvlen - (it.c * kChunk + wave * kKeysPerWave), 0), kKeysPerWave); };
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    auto load_k = [&](const Item &it, uint4 (&kf)[4][4]) {
        const uint16_t *kb = item_base(bf.k, it);
        const int nv = wave_valid(it);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int kk = kt * 16 + c16;
            const uint16_t *kr = kb + (kk < nv ? wave * kKeysPerWave + kk : 0) * rs + g4 * 8;
#pragma unroll
            for (int s = 0; s < 4; ++s) kf[kt][s] = *reinterpret_cast<const uint4 *>(kr + s * 32);
        }
    };
    auto load_v = [&](const Item &it, uint4 (&vr)[2][8]) {
        const uint16_t *vb = item_base(bf.v, it);
        const int nv = wave_valid(it);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int kk = s2 * 32 + g4 * 8 + e;
                vr[s2][e] = *reinterpret_cast<const uint4 *>(vb + (kk < nv ? wave * kKeysPerWave + kk : 0) * rs + c16 * 8);
            }
    };
    // q rows of M tile mt as the MFMA A operand: row c16 of the tile, d in [32 s + 8 g4, +8)
    auto load_q = [&](const Item &it, int mt, uint4 (&qf)[4]) {
        const int ra = mt * 16 + c16;
        const bool ok = ra < R;                                          // padding rows read row 0
        const int ja = ok ? ra / sh.G : 0, ia = ok ? ra - ja * sh.G : 0;
        const uint16_t *qb = bf.q + ((int64_t)it.b * sh.Q * sh.Hq + (int64_t)it.hk * sh.G) * kHeadDim;
        const uint16_t *qr = qb + (ja * sh.Hq + ia) * kHeadDim + g4 * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const uint4 *>(qr + s * 32);
    };

    uint4 kf[4][4], vr[2][8], qf[4];
    int64_t t = next_id(blockIdx.x);
    if (t < nid) {
        const Item it = decode(t);
        load_q(it, MG ? it.mg * sh.mgt : 0, qf);
        load_k(it, kf);
        load_v(it, vr);
    }
    while (t < nid) {
        Item it = decode(t);
        int r0, r1;
        group_rows(it, r0, r1);
        const int mt0 = r0 / 16, mt1 = (r1 + 15) / 16;
        const int64_t tn = next_id(t + gridDim.x);
        // SPL: the split's chunks it.c .. clast in order, with the running
        // softmax state of row threadIdx.x / 16, d in [8 (threadIdx.x % 16), +8)
        const int split = SPL ? it.c / sh.cps : 0;
        const int clast = WHOLE ? it.c : RUNS ? min(it.c + sh.cps - 1, group_last_key(it) / kChunk) : it.c;
        float rM = -INFINITY, rl = 0.0f, ro[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ro[e] = 0.0f;
        // one chunk of the item; `more`: another chunk of this split follows
        auto chunk = [&](const bool more) {
            const bool has_next = more || tn < nid;
            auto next_item = [&]() {
                if (RUNS && more) {
                    Item nx = it;
                    nx.c = WHOLE && it.c == clast ? 0 : it.c + 1;
                    return nx;
                }
                return decode(tn);
            };
            const int key0 = it.c * kChunk;
            const int wkey0 = key0 + wave * kKeysPerWave;
            bool prefetched = false;                       // the next item's K and q are requested
            bool vready = false;                           // this item's V is in P . V operand form

            // One 16-row query tile against this chunk.  The first tile runs on
            // the q rows requested with the item; later tiles (verify blocks and
            // prompts of more than 16 rows per head) request theirs first.  The
            // first call is separate from the loop so that the waits of the
            // common one-tile case count only the loads that precede its q.
            auto run_tile = [&](const int mt) {
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
                if (!any) return;

                // scores: tile kt -> lane (g4, c16) reg i = row 4 g4 + i, key wkey0 + 16 kt + c16
                float sc[4][4];
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
                // the next item's K and first q tile: requested once the last tile
                // has read this item's
                if (mt == mt1 - 1 && has_next) {
                    const Item nx = next_item();
                    load_k(nx, kf);
                    load_q(nx, MG ? nx.mg * sh.mgt : 0, qf);
                    prefetched = true;
                }

                // chunk max per row
                float mx[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float m = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
                    m = row16_max(m);
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
                // probabilities, row sums, and the P tile as hi and lo 16-bit parts
                float ls[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) ls[i] = 0.0f;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const bool vis = sc[kt][i] != -INFINITY;
                        const float pv = vis ? attn_exp(sc[kt][i] - mx[i]) : 0.0f;
                        ls[i] = ls[i] + pv;
                        const uint16_t hi = S::narrow(pv);
                        phi[wave][g4 * 4 + i][kt * 16 + c16] = hi;
                        plo[wave][g4 * 4 + i][kt * 16 + c16] = S::narrow(pv - S::widen(hi));
                    }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float l = ls[i];
                    l = row16_sum(l);
                    ls[i] = l;
                }
                if (c16 == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xl[wave][g4 * 4 + i] = ls[i];
                }
                __syncthreads();
                // this item's V as the P . V B operand (its loads had the scores
                // and the softmax to arrive)
                if (!vready) {
                    const int nv = wave_valid(it);
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (s2 * 32 + g4 * 8 + e >= nv) vr[s2][e] = zero4;   // p is 0 there; keep 0 * v exact
                    transpose8x8_b16(vr[0]);
                    transpose8x8_b16(vr[1]);
                    vready = true;
                }
                // o partial of this wave: P (16 x 64) . V (64 x 128), lo parts first
                uint4 ph[2], pq[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    ph[s2] = *reinterpret_cast<const uint4 *>(&phi[wave][c16][s2 * 32 + g4 * 8]);
                    pq[s2] = *reinterpret_cast<const uint4 *>(&plo[wave][c16][s2 * 32 + g4 * 8]);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) acc = mfma16<S>(pq[s2], vr[s2][j], acc);
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) acc = mfma16<S>(ph[s2], vr[s2][j], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) ol[wave][g4 * 4 + i][c16 * 8 + j] = acc[i];
                }
                __syncthreads();
                // combine the four wave partials in order and write this chunk's
                // partial: thread -> row t / 16 of the tile, d in [8 (t % 16), +8)
                if constexpr (SPL) {
                    // fold the chunk into the split's running state instead
                    const int rr = threadIdx.x >> 4, dg = threadIdx.x & 15;
                    const int r = mt * 16 + rr;
                    if (r < R && last_key(it.kvlen, r / sh.G) >= key0) {
                        float oc[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int d = dg * 8 + e;
                            oc[e] = ((ol[0][rr][d] + ol[1][rr][d]) + ol[2][rr][d]) + ol[3][rr][d];
                        }
                        const float mc = fmaxf(fmaxf(xm[0][rr], xm[1][rr]), fmaxf(xm[2][rr], xm[3][rr]));
                        const float lc = ((xl[0][rr] + xl[1][rr]) + xl[2][rr]) + xl[3][rr];
                        if (rM == -INFINITY) {
                            rM = mc;
                            rl = lc;
#pragma unroll
                            for (int e = 0; e < 8; ++e) ro[e] = oc[e];
                        } else {
                            const float mn = fmaxf(rM, mc), a = attn_exp(rM - mn), bw = attn_exp(mc - mn);
                            rl = rl * a + lc * bw;
#pragma unroll
                            for (int e = 0; e < 8; ++e) ro[e] = ro[e] * a + oc[e] * bw;
                            rM = mn;
                        }
                    }
                } else {
                    const int rr = threadIdx.x >> 4, dg = threadIdx.x & 15;
                    const int r = mt * 16 + rr;
                    if (r < R) {
                        const int j = r / sh.G;
                        if (last_key(it.kvlen, j) >= key0) {
                            float4 o[2];
#pragma unroll
                            for (int half = 0; half < 2; ++half) {
                                const int d = dg * 8 + half * 4;
                                const float4 o0 = *reinterpret_cast<const float4 *>(&ol[0][rr][d]);
                                const float4 o1 = *reinterpret_cast<const float4 *>(&ol[1][rr][d]);
                                const float4 o2 = *reinterpret_cast<const float4 *>(&ol[2][rr][d]);
                                const float4 o3 = *reinterpret_cast<const float4 *>(&ol[3][rr][d]);
                                o[half].x = ((o0.x + o1.x) + o2.x) + o3.x;
                                o[half].y = ((o0.y + o1.y) + o2.y) + o3.y;
                                o[half].z = ((o0.z + o1.z) + o2.z) + o3.z;
                                o[half].w = ((o0.w + o1.w) + o2.w) + o3.w;
                            }
                            const float mc = fmaxf(fmaxf(xm[0][rr], xm[1][rr]), fmaxf(xm[2][rr], xm[3][rr]));
                            const float lc = ((xl[0][rr] + xl[1][rr]) + xl[2][rr]) + xl[3][rr];
                            if (lds_parts) {
                                float *dst = &wpart[(r * lcs + it.c) * kPartStride];
#pragma unroll
                                for (int half = 0; half < 2; ++half)
                                    *reinterpret_cast<float4 *>(dst + dg * 8 + half * 4) = o[half];
                                if (dg == 0) {
                                    dst[kHeadDim] = mc;
                                    dst[kHeadDim + 1] = lc;
                                }
                            } else {
                                // the (sequence, KV head, chunk) block of R row partials: a
                                // wave-uniform base and a 32-bit row offset (no per-lane
                                // 64-bit address to keep alive across the walk)
                                const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
                                    bf.part + attn_part_block(sh, it.b, it.hk, it.c), (short)0, 0x7fffffff, 0x00020000);
                                const int voff = r * (kPartStride * 4) + dg * 32;
#pragma unroll
                                for (int half = 0; half < 2; ++half)
                                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o[half]), prs,
                                                                           voff + half * 16, 0, 0);
                                if (dg == 0)                   // voff is the row's first byte here
                                    __builtin_amdgcn_raw_buffer_store_b64(
                                        i32x2{__builtin_bit_cast(int, mc), __builtin_bit_cast(int, lc)}, prs,
                                        voff + kHeadDim * 4, 0, 0);
                            }
                        }
                    }
                }
                __syncthreads();
            };
            run_tile(mt0);
            for (int mt = mt0 + 1; mt < mt1; ++mt) {
                load_q(it, mt, qf);
                run_tile(mt);
            }
            // The group's last row, in the last tile, sees key0 (the item has
            // work), so the last tile is never skipped and the next item's K and q
            // are already in flight; this is the fallback should it ever be.
            if (!prefetched && has_next) {
                const Item nx = next_item();
                load_k(nx, kf);
                load_q(nx, MG ? nx.mg * sh.mgt : 0, qf);
            }
            // the next item's V (its K and q are in flight since this item's scores)
            if (has_next) load_v(next_item(), vr);
        };
        if constexpr (RUNS) {
            for (;;) {
                const bool more = WHOLE ? (it.c == clast ? clast > 0 : it.c + 1 < clast) : it.c < clast;
                chunk(more);
                if (!more) break;
                it.c = WHOLE && it.c == clast ? 0 : it.c + 1;
            }
        } else {
            chunk(false);
        }
        if constexpr (WHOLE) {
            // the group's range and row levels, from the partials this
            // workgroup just wrote (every store of every wave done first)
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            attn_merge_rows<S>(bf, sh, it.b, it.hk, it.kvlen, lds_parts ? wpart : nullptr, lcs);
            __syncthreads();
        }
        if constexpr (SPL) {
            // the split's partial (o, m, l), or with one split the output
            const int rr = threadIdx.x >> 4, dg = threadIdx.x & 15;
            const int r = mt0 * 16 + rr;
            if (r < R && rM != -INFINITY) {
                const int j = r / sh.G;
                const int64_t row = ((int64_t)it.b * sh.Q + j) * sh.Hq + (int64_t)it.hk * sh.G + (r - j * sh.G);
                if (sh.nchunks == 1) {
                    attn_store_out<S>(bf.o + row * kHeadDim + dg * 8, make_float4(ro[0], ro[1], ro[2], ro[3]), rl);
                    attn_store_out<S>(bf.o + row * kHeadDim + dg * 8 + 4, make_float4(ro[4], ro[5], ro[6], ro[7]), rl);
                } else {
                    float *dst = bf.part + attn_part_block(sh, it.b, it.hk, split) + (int64_t)r * kPartStride;
                    *reinterpret_cast<float4 *>(dst + dg * 8) = make_float4(ro[0], ro[1], ro[2], ro[3]);
                    *reinterpret_cast<float4 *>(dst + dg * 8 + 4) = make_float4(ro[4], ro[5], ro[6], ro[7]);
                    if (dg == 0) {
                        dst[kHeadDim] = rM;
                        dst[kHeadDim + 1] = rl;
                    }
                }
            }
        }
        t = tn;
    }
}

// Prompts (many query rows per KV head, at most 8192 keys: one or two
// ranges).  One workgroup of 8 waves per (sequence, KV head, block of 128
// query rows), heaviest blocks of all sequences and heads first; wave w owns
// the block's 16-row tile w and plays all four key quarters of every chunk
// itself -- the "waves" of the chunk tree are the quarters [64q, 64q + 64)
// of a chunk, whoever computes them -- so a chunk's max, l and o are
// combined in registers in the tree's order and no partial leaves the
// workgroup.  The range weights need the maxima of the row's chunks before
// any o_c is weighted, so the walk runs twice: pass 1 computes every chunk
// max m_c (kept in LDS) and M = max m_c; pass 2 recomputes the scores and
// forms, per chunk and in ascending order, o_r = sum o_c 2^(m_c - M_r) and
// l_r within each range, then o = sum o_r 2^(M_r - M) and l over the ranges,
// exactly as attn_merge_kernel does with the partials.  Each quarter's K (as
// the score MFMA's B operand) and V (transposed into the P . V operand, as
// attn_kernel does in registers) are staged once in LDS for all eight
// waves, two buffers deep.
constexpr int kPreWaves = 8, kPreRows = 16 * kPreWaves;
constexpr int kPreMaxRanges = 2;             // max_kv <= 8192

// NR: the ranges the launch's keys span (1 or 2); one range keeps the row
// sums out of the registers (its range weight 2^(M_r - M) is 1).
template <typename S, int NR>
__global__ __launch_bounds__(kPreWaves * kWave, 1)
void attn_prefill_kernel(AttnBufs bf, const int32_t *__restrict__ kv_len, AttnShape sh, int nrb)
{
    typedef uint4 KStage[4][4][kWave];         // [key tile][d step][lane]: score B operands
    typedef uint4 VStage[2][8][kWave];         // [32-key step][output tile j][lane]: P . V B operands
    typedef uint4 VRows[kKeysPerWave][kHeadDim / 8];   // V rows of a quarter as stored
    __shared__ __attribute__((aligned(16))) KStage k0, k1;
    __shared__ __attribute__((aligned(16))) VStage v0, v1;
    __shared__ __attribute__((aligned(16))) VRows w0, w1;
    typedef uint16_t PTile[16][kKeysPerWave + 8];
    __shared__ __attribute__((aligned(16))) PTile phi[kPreWaves], plo[kPreWaves];
    __shared__ float mstore[kPreWaves][16][NR * kRange];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g4 = lane >> 4, c16 = lane & 15;
    const int R = (int)sh.Q * sh.G, Qi = (int)sh.Q;
    // block id -> (row block, b, hk): the row blocks of the latest positions
    // (the most keys) of every (sequence, KV head) first, so the dispatcher
    // hands out the heaviest workgroups first and the lightest fill in last
    const int ng = (int)sh.B * sh.Hkv;
    const int rbi = (int)blockIdx.x / ng, gi = (int)blockIdx.x - rbi * ng;
    const int rb = nrb - 1 - rbi, b = gi / sh.Hkv, hk = gi - b * sh.Hkv;
    const int kvlen = (int)min((int64_t)kv_len[b], sh.max_kv);
    const int rt0 = rb * kPreRows + wave * 16;                  // this wave's tile
    const int rlast = min(rb * kPreRows + kPreRows, R) - 1;     // the block's last row
    const int lastkey = attn_last_key(kvlen, Qi, rlast / sh.G, sh.causal);
    if (kvlen < 1 || lastkey < 0) return;                       // a bad kv_len: nothing this block may read
    const int lastc = lastkey / kChunk;
    const int nunits = (lastc + 1) * 4;                         // (chunk, quarter) units

    // rows of the accumulator layout held by this lane: rt0 + 4 g4 + i
    int lk[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = rt0 + g4 * 4 + i;
        ok[i] = r < R;
        lk[i] = ok[i] ? attn_last_key(kvlen, Qi, r / sh.G, sh.causal) : -1;
    }
    const bool wave_rows = rt0 < R;
    // q of row rt0 + c16 as the MFMA A operand (padding rows read row 0)
    uint4 qf[4];
    {
        const int ra = rt0 + c16 < R ? rt0 + c16 : 0;
        const int ja = ra / sh.G, ia = ra - ja * sh.G;
        const uint16_t *qr = bf.q + (((int64_t)b * sh.Q + ja) * sh.Hq + (int64_t)hk * sh.G + ia) * kHeadDim + g4 * 8;
#pragma unroll
        for (int st = 0; st < 4; ++st) qf[st] = *reinterpret_cast<const uint4 *>(qr + st * 32);
    }

    const int rs = (int)sh.ks;
    const uint16_t *kbase = bf.k + (int64_t)b * sh.Lcap * sh.Hkv * kHeadDim + (int64_t)hk * sh.hs;
    const uint16_t *vbase = bf.v + (int64_t)b * sh.Lcap * sh.Hkv * kHeadDim + (int64_t)hk * sh.hs;
    // K of unit u: 16 one-KiB chunks [kt][st], two per wave, straight into LDS
    auto stage_k = [&](KStage &dst, int u) __attribute__((always_inline)) {
        const int key0 = (u >> 2) * kChunk + (u & 3) * kKeysPerWave;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int idx = wave * 2 + h, kt = idx >> 2, st = idx & 3;
            const int key = min(key0 + kt * 16 + c16, kvlen - 1);   // keys past kv_len read a real key, masked
            __builtin_amdgcn_global_load_lds(kbase + (int64_t)key * rs + st * 32 + g4 * 8, &dst[kt][st][0], 16, 0, 0);
        }
    };
    // V of unit u: waves 6 and 7 bring the 32-key steps 0 and 1 into LDS as
    // stored (4 keys per 1 KiB load), then read 8 key rows per lane back,
    // zero keys past kv_len, transpose and store the P . V operands.  A V
    // load never stays in flight in registers across other work.
    auto stage_v = [&](VRows &dst, int u) __attribute__((always_inline)) {
        const int key0 = (u >> 2) * kChunk + (u & 3) * kKeysPerWave + (wave - 6) * 32;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int key = min(key0 + t * 4 + (lane >> 4), kvlen - 1);
            __builtin_amdgcn_global_load_lds(vbase + (int64_t)key * rs + c16 * 8, &dst[(wave - 6) * 32 + t * 4][0], 16, 0,
                                             0);
        }
    };
    auto transpose_v = [&](const VRows &src, VStage &dst, int u) __attribute__((always_inline)) {
        const int s2 = wave - 6;
        const int key0 = (u >> 2) * kChunk + (u & 3) * kKeysPerWave + s2 * 32 + g4 * 8;
        uint4 vr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // keys past kv_len become zeros (p is 0 there; keep 0 * v exact), by a mask, not a select
            const uint32_t keep = key0 + e < kvlen ? 0xffffffffu : 0u;
            const uint4 t = src[s2 * 32 + g4 * 8 + e][c16];
            vr[e] = make_uint4(t.x & keep, t.y & keep, t.z & keep, t.w & keep);
        }
        transpose8x8_b16(vr);
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[s2][j][lane] = vr[j];
    };
    // A row's last key grows with its position, so the first row of a tile
    // with no padding rows sees the fewest keys: a unit that row sees in full
    // is seen in full by the whole tile and needs no mask.
    const int lkfull = rt0 + 15 < R ? attn_last_key(kvlen, Qi, rt0 / sh.G, sh.causal) : -1;
    auto unit_full = [&](int u) { return (u >> 2) * kChunk + (u & 3) * kKeysPerWave + kKeysPerWave - 1 <= lkfull; };
    // scores of unit u for this wave's rows, masked (-inf outside a row's keys)
    auto scores = [&](const KStage &ks_, int u, bool full, float (&sc)[4][4]) __attribute__((always_inline)) {
        const int keyq = (u >> 2) * kChunk + (u & 3) * kKeysPerWave;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) acc = mfma16<S>(qf[st], ks_[kt][st][lane], acc);
            const int key = keyq + kt * 16 + c16;
            if (full) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[kt][i] = acc[i] * sh.scale;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool vis = ok[i] && key >= 0 && key <= lk[i];
                    sc[kt][i] = vis ? acc[i] * sh.scale : -INFINITY;
                }
            }
        }
    };

    // ---- pass 1: chunk maxima
    float mc[4], M[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mc[i] = M[i] = -INFINITY;
    auto pass1_unit = [&](const KStage &cur, KStage &nxt, int u) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (u + 1 < nunits) stage_k(nxt, u + 1);
        if (wave_rows) {
            float sc[4][4];
            scores(cur, u, unit_full(u), sc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float m = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
                m = row16_max(m);
                mc[i] = fmaxf(mc[i], m);
            }
            if ((u & 3) == 3) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (c16 == 0) mstore[wave][g4 * 4 + i][u >> 2] = mc[i];
                    M[i] = fmaxf(M[i], mc[i]);
                    mc[i] = -INFINITY;
                }
            }
        }
    };
    stage_k(k0, 0);
    for (int u = 0; u < nunits; u += 2) {
        pass1_unit(k0, k1, u);
        if (u + 1 < nunits) pass1_unit(k1, k0, u + 1);
    }

    // ---- pass 2: the chunk tree and the range combine
    // oc, lc: the chunk's sums; orr, lr: the range's; ow, lw: the row's
    f32x4 oc[8], orr[8], ow[8];
    float lc[4], lr[4], lw[4], mrow[4], Mr[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) oc[j] = orr[j] = ow[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) lc[i] = lr[i] = lw[i] = mrow[i] = Mr[i] = 0.0f;
    // unit u: its V (loaded during unit u - 1) goes into vbuf, free since
    // everyone passed the barrier after multiplying unit u - 2 with it
    // the compute of unit u (pass 2)
    auto compute2 = [&](const VStage &vbuf, const KStage &kcur, int u) __attribute__((always_inline)) {
        if (!wave_rows) return;
        const int c = u >> 2, qq = u & 3;
        if (qq == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) mrow[i] = mstore[wave][g4 * 4 + i][c];
        }
        float sc[4][4];
        const bool full = unit_full(u);
        scores(kcur, u, full, sc);
        // probabilities, this quarter's row sums (0 + p = p: the first term
        // is taken as it is, p being never -0), P as hi and lo parts -- rows
        // 4 g4 + i and 4 g4 + i + 1 converted together; the unmasked form for
        // units the whole tile sees
        float ls[4];
        auto probs = [&](auto full_) __attribute__((always_inline)) {
            constexpr bool FULL = decltype(full_)::value;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    float pv[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float x = sc[kt][i + h];
                        pv[h] = FULL || x != -INFINITY ? attn_exp(x - mrow[i + h]) : 0.0f;
                        ls[i + h] = kt == 0 ? pv[h] : ls[i + h] + pv[h];
                    }
                    const uint32_t hp = narrow2<S>(pv[0], pv[1]);
                    const uint32_t lp = narrow2<S>(pv[0] - S::widen((uint16_t)hp), pv[1] - S::widen((uint16_t)(hp >> 16)));
                    phi[wave][g4 * 4 + i][kt * 16 + c16] = (uint16_t)hp;
                    phi[wave][g4 * 4 + i + 1][kt * 16 + c16] = (uint16_t)(hp >> 16);
                    plo[wave][g4 * 4 + i][kt * 16 + c16] = (uint16_t)lp;
                    plo[wave][g4 * 4 + i + 1][kt * 16 + c16] = (uint16_t)(lp >> 16);
                }
        };
        if (full) probs(std::true_type{});
        else probs(std::false_type{});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float l = ls[i];
            l = row16_sum(l);
            lc[i] = qq == 0 ? l : lc[i] + l;
        }
        // this quarter's o: P (16 x 64) . V (64 x 128), lo parts first
        uint4 ph[2], pq[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            ph[s2] = *reinterpret_cast<const uint4 *>(&phi[wave][c16][s2 * 32 + g4 * 8]);
            pq[s2] = *reinterpret_cast<const uint4 *>(&plo[wave][c16][s2 * 32 + g4 * 8]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) acc = mfma16<S>(pq[s2], vbuf[s2][j][lane], acc);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) acc = mfma16<S>(ph[s2], vbuf[s2][j][lane], acc);
            oc[j] = qq == 0 ? acc : oc[j] + acc;
        }
        if (qq == 3) {
            // chunk c done: weight it into the range sums of the rows that see
            // it (range maximum M_r over the row's chunks of the range, taken
            // from pass 1's chunk maxima as the range starts), and once a
            // row's range is complete -- its last chunk of the range or its
            // last chunk -- weight the range into the row sums: the range and
            // row levels of attn_merge_kernel, in its order and arithmetic
            const int rg = c / kRange, c0 = rg * kRange;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (!(ok[i] && lk[i] >= c * kChunk)) continue;
                if constexpr (NR == 1) {
                    // one range: M_r = M, and the row level is the range level
                    // times 2^(M - M) = 1, taken at the output
                    const float w = attn_exp(mrow[i] - M[i]);
                    if (c == 0) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) orr[j][i] = oc[j][i] * w;
                        lr[i] = lc[i] * w;
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) orr[j][i] = orr[j][i] + oc[j][i] * w;
                        lr[i] = lr[i] + lc[i] * w;
                    }
                    continue;
                }
                const int clast = min(c0 + kRange - 1, lk[i] / kChunk);
                if (c == c0) {
                    float m = mstore[wave][g4 * 4 + i][c0];
                    for (int cc = c0 + 1; cc <= clast; ++cc) m = fmaxf(m, mstore[wave][g4 * 4 + i][cc]);
                    Mr[i] = m;
                }
                const float w = attn_exp(mrow[i] - Mr[i]);
                if (c == c0) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) orr[j][i] = oc[j][i] * w;
                    lr[i] = lc[i] * w;
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) orr[j][i] = orr[j][i] + oc[j][i] * w;
                    lr[i] = lr[i] + lc[i] * w;
                }
                if (c == clast) {
                    const float u = attn_exp(Mr[i] - M[i]);
                    if (rg == 0) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) ow[j][i] = orr[j][i] * u;
                        lw[i] = lr[i] * u;
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) ow[j][i] = ow[j][i] + orr[j][i] * u;
                        lw[i] = lw[i] + lr[i] * u;
                    }
                }
            }
        }
    };
    // VW: this wave stages V (waves 6 and 7); the two roles run separate
    // copies of the walk.  Unit u: everyone's loads of unit u have landed and
    // unit u's V operands are in vcur (staged by waves 6 and 7 at the end of
    // unit u - 1); start unit u + 1's loads, multiply, and (waves 6, 7) turn
    // unit u + 1's V rows into vnxt -- free, since everyone passed this
    // unit's barrier after multiplying unit u - 1 with it.
    auto pass2_unit = [&](auto vw_, const KStage &kcur, KStage &knxt, const VStage &vcur, VStage &vnxt,
                          VRows &wnxt, int u) __attribute__((always_inline)) {
        constexpr bool VW = decltype(vw_)::value;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (u + 1 < nunits) {
            stage_k(knxt, u + 1);
            if constexpr (VW) stage_v(wnxt, u + 1);
        }
        compute2(vcur, kcur, u);
        if constexpr (VW) {
            if (u + 1 < nunits) {
                __builtin_amdgcn_s_waitcnt(0);             // this wave's V rows of unit u + 1
                transpose_v(wnxt, vnxt, u + 1);
            }
        }
    };
    auto pass2 = [&](auto vw_) __attribute__((always_inline)) {
        constexpr bool VW = decltype(vw_)::value;
        stage_k(k0, 0);
        if constexpr (VW) {
            stage_v(w0, 0);
            __builtin_amdgcn_s_waitcnt(0);
            transpose_v(w0, v0, 0);
        }
        for (int u = 0; u < nunits; u += 2) {
            pass2_unit(vw_, k0, k1, v0, v1, w1, u);
            if (u + 1 < nunits) pass2_unit(vw_, k1, k0, v1, v0, w0, u + 1);
        }
    };
    if (wave >= 6) pass2(std::true_type{});
    else pass2(std::false_type{});
    if (!wave_rows) return;
    // out = RNE(o / l) from the row sums (one range: o = o_r 2^(M - M))
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!ok[i] || lk[i] < 0) continue;
        const int r = rt0 + g4 * 4 + i, j = r / sh.G;
        const int64_t row = ((int64_t)b * sh.Q + j) * sh.Hq + (int64_t)hk * sh.G + (r - j * sh.G);
        if constexpr (NR == 1) {
            const float u = attn_exp(M[i] - M[i]);
            const float l = lr[i] * u;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                ow[jj][i] = orr[jj][i] * u;
                lw[i] = l;
            }
        }
        uint16_t o8[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) o8[jj] = S::narrow(ow[jj][i] / lw[i]);
        *reinterpret_cast<uint4 *>(bf.o + row * kHeadDim + c16 * 8) = __builtin_bit_cast(uint4, o8);
    }
}

// Range and row levels for one query row (b, j, h) per workgroup of
// 32 * kMergeRanges threads: thread (r', quad) handles range r' of the current
// batch of kMergeRanges ranges and d in [4 quad, +4).
//   1. Range r: M_r = max m_c, o_r = sum o_c exp(m_c - M_r), l_r likewise, c
//      ascending within the range.
//   2. M = max over the row's chunk maxima (exact, any order: from the M_r
//      when the ranges fit one batch, else read beforehand); range r's term
//      o_r exp(M_r - M) goes to LDS.
//   3. The 32 threads of range slot 0 add the batch's terms in ascending r to
//      the running sums; batches follow in ascending order.
// All of a range's chunk partials are requested at once, so a row costs about
// two memory round trips whatever its length.
constexpr int kMergeRanges = 32;     // ranges per batch (threads = 32 per range): 131072 keys

template <typename S>
__global__ __launch_bounds__(32 * kMergeRanges)
void attn_merge_kernel(const float *__restrict__ part, const int32_t *__restrict__ kv_len,
                       uint16_t *__restrict__ out, AttnShape sh)
{
    __shared__ __attribute__((aligned(16))) float term[kMergeRanges][kHeadDim + 4];
    __shared__ float red[32 * kMergeRanges / kWave], rmax[kMergeRanges];
    const int64_t row = blockIdx.x;                       // (b * Q + j) * Hq + h
    const int j = (int)((row / sh.Hq) % sh.Q), h = (int)(row % sh.Hq);
    const int64_t b = row / (sh.Hq * sh.Q);
    const int hk = h / sh.G;
    const int kvlen = (int)min((int64_t)kv_len[b], sh.max_kv);
    const int lk = attn_last_key(kvlen, (int)sh.Q, j, sh.causal);
    const int nthr = blockDim.x, slots = nthr / 32;
    const int quad = threadIdx.x & 31, slot = threadIdx.x >> 5;
    if (lk < 0) return;                                   // a bad kv_len: nothing this row may read
    const int nch = lk / (kChunk * sh.cps) + 1, nr = (nch + kRange - 1) / kRange;
    // this row's partial of chunk (or split) c at pr + c cs
    const float *pr = part + attn_part_block(sh, b, hk, 0) + ((int64_t)j * sh.G + (h - hk * sh.G)) * kPartStride;
    const int64_t cs = sh.Q * sh.G * (int64_t)kPartStride;

    // M = max over the chunk maxima: read first when the row's ranges take
    // several batches, else taken from the range maxima below (the same value:
    // a max is exact)
    const bool one_batch = nr <= slots;
    float M = -INFINITY;
    if (!one_batch) {
        for (int c = threadIdx.x; c < nch; c += nthr) M = fmaxf(M, pr[c * cs + kHeadDim]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = M;
        __syncthreads();
        M = red[0];
        for (int w = 1; w < nthr / kWave; ++w) M = fmaxf(M, red[w]);
    }

    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.0f;
    for (int r0 = 0; r0 < nr; r0 += slots) {
        const int r = r0 + slot;
        float Mr = -INFINITY, lr = 0.0f;
        float4 orr = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < nr) {
            const int c0 = r * kRange, n = min(nch - c0, kRange);
            float mv[kRange], lv[kRange];
            float4 ov[kRange];
#pragma unroll
            for (int i = 0; i < kRange; ++i) {
                const float *pc = pr + (c0 + min(i, n - 1)) * cs;   // stays on written partials
                mv[i] = pc[kHeadDim];
                lv[i] = pc[kHeadDim + 1];
                ov[i] = *reinterpret_cast<const float4 *>(pc + quad * 4);
            }
            Mr = mv[0];
#pragma unroll
            for (int i = 1; i < kRange; ++i)
                if (i < n) Mr = fmaxf(Mr, mv[i]);
            float w = attn_exp(mv[0] - Mr);
            orr = make_float4(ov[0].x * w, ov[0].y * w, ov[0].z * w, ov[0].w * w);
            lr = lv[0] * w;
#pragma unroll
            for (int i = 1; i < kRange; ++i) {
                if (i < n) {
                    w = attn_exp(mv[i] - Mr);
                    orr.x = orr.x + ov[i].x * w;
                    orr.y = orr.y + ov[i].y * w;
                    orr.z = orr.z + ov[i].z * w;
                    orr.w = orr.w + ov[i].w * w;
                    lr = lr + lv[i] * w;
                }
            }
        }
        if (one_batch) {
            if (quad == 0) rmax[slot] = Mr;
            __syncthreads();
            M = rmax[0];
            for (int i = 1; i < nr; ++i) M = fmaxf(M, rmax[i]);
        }
        if (r < nr) {
            const float u = attn_exp(Mr - M);
            *reinterpret_cast<float4 *>(&term[slot][quad * 4]) =
                make_float4(orr.x * u, orr.y * u, orr.z * u, orr.w * u);
            if (quad == 0) term[slot][kHeadDim] = lr * u;
        }
        __syncthreads();
        if (slot == 0) {
            const int nb = min(slots, nr - r0);
            for (int i = 0; i < nb; ++i) {
                const float4 tv = *reinterpret_cast<const float4 *>(&term[i][quad * 4]);
                const float tl = term[i][kHeadDim];
                if (r0 + i == 0) {
                    o = tv;
                    l = tl;
                } else {
                    o.x = o.x + tv.x;
                    o.y = o.y + tv.y;
                    o.z = o.z + tv.z;
                    o.w = o.w + tv.w;
                    l = l + tl;
                }
            }
        }
        __syncthreads();
    }
    if (slot == 0) {
        uint2 pk;
        pk.x = (uint32_t)S::narrow(o.x / l) | ((uint32_t)S::narrow(o.y / l) << 16);
        pk.y = (uint32_t)S::narrow(o.z / l) | ((uint32_t)S::narrow(o.w / l) << 16);
        *reinterpret_cast<uint2 *>(out + row * kHeadDim + quad * 4) = pk;
    }
}

static bi_status check_attn(const void *q, const void *k, const void *v, const void *o, const int32_t *kv_len,
                            int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t dtype)
{
    if (!q || !k || !v || !o || !kv_len) return BI_ERR_NULL;
    if (B < 1 || Q < 1 || Lcap < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv) return BI_ERR_SHAPE;
    if (max_kv_len < Q || max_kv_len > Lcap || max_kv_len > kMaxKv) return BI_ERR_SHAPE;
    if (Hkv > 65535 || B * Q * Hq > (1ll << 31) - 1 || Q * (Hq / Hkv) > (1ll << 30) ||
        cdiv(B * cdiv(max_kv_len, kChunk), 8) * 8 * Hkv > (1ll << 31) - 1 || B * Lcap * Hkv * (int64_t)D > (1ll << 40))
        return BI_ERR_SHAPE;
    if (D != kHeadDim) return BI_ERR_UNSUPPORTED;
    if (dtype != BI_BF16 && dtype != BI_F16) return BI_ERR_DTYPE;
    if (!host_aligned16(q) || !host_aligned16(k) || !host_aligned16(v) || !host_aligned16(o) ||
        ((uintptr_t)kv_len & 3u))
        return BI_ERR_ALIGN;
    return BI_OK;
}

// Workspace: the chunk partials, fp32 [B][Hkv][nchunks][Q Hq / Hkv][kPartStride].
static size_t attn_partial_bytes(int64_t B, int64_t Q, int64_t max_kv_len, int64_t Hq)
{
    return (size_t)(B * Q * Hq) * (size_t)cdiv(max_kv_len, kChunk) * kPartStride * sizeof(float);
}

struct AttnPlan {
    AttnShape sh;
    int64_t nid, grid, merge_threads;
    size_t parts;
};

// cps: chunks per partial -- 1 for the invariant tree; the split variant's
// run length (its partials are then per split).
static AttnPlan attn_plan(int64_t B, int64_t Q, int64_t max_kv_len, int64_t Lcap, int32_t Hq, int32_t Hkv,
                          float scale, int32_t causal, int32_t kv_layout, int cps = 1)
{
    const int64_t D = kHeadDim;
    // kv_layout 0: [B, Lcap, Hkv, D]; 1: [B, Hkv, Lcap, D] (head-major)
    const int64_t ks = kv_layout ? D : (int64_t)Hkv * D, hs = kv_layout ? Lcap * D : D;
    // query-row groups: when the (sequence, chunk, head) items alone give fewer
    // than two per workgroup slot, split the rows so that about 4096 ids exist
    // (half of a causal prompt's (chunk, rows) pairs being empty), never under
    // kAttnMinTiles tiles each; otherwise one group
    const int64_t G = Hq / Hkv;
    const int64_t ntm = cdiv(Q * G, 16), nbase = cdiv(B * cdiv(max_kv_len, kChunk), 8) * 8 * Hkv;
    const int64_t ngroups = nbase >= 1024 ? 1 : std::max<int64_t>(1, cdiv(4096, nbase));
    const int64_t mgt = std::min<int64_t>(std::max<int64_t>(kAttnMinTiles, cdiv(ntm, ngroups)), ntm);
    const int64_t nch = cdiv(cdiv(max_kv_len, kChunk), cps);            // partials per row
    AttnPlan p;
    p.sh = AttnShape{B, Q, Lcap, nch, cdiv(nch, kRange), max_kv_len, cdiv(ntm, mgt), Hq, Hkv, (int)G, (int)mgt,
                     scale * kLog2e, causal ? 1 : 0, ks, hs, cps, nch};
    // item ids (padded to whole groups of 8); a persistent grid of two
    // workgroups per CU, a multiple of 8 so that a workgroup stays on one XCD
    p.nid = cdiv(B * nch, 8) * 8 * Hkv * p.sh.nmg;
    p.grid = std::min<int64_t>(p.nid, (int64_t)device_cu_count() * 2 / 8 * 8);
    // merge: 32 threads per range of the longest row, whole waves, at most kMergeRanges ranges at once
    p.merge_threads = cdiv(32 * std::min<int64_t>(p.sh.nranges, kMergeRanges), kWave) * kWave;
    p.parts = (size_t)(B * Q * Hq) * (size_t)nch * kPartStride * sizeof(float);
    return p;
}

// Short contexts (at most kWholeMaxChunks chunks, or at most kWholeLdsParts
// (query row, chunk) partials per group) with at least one (sequence, KV
// head) group of at most 32 query rows for each of the persistent grid's
// workgroups (two per CU): one work item per group with all its chunks,
// merged in the workgroup (attn_kernel's WHOLE form) -- every workgroup is
// busy without cutting the groups into chunks, and the merge launch is gone.
// Fewer groups keep the chunk items, which spread a context over the whole
// chip; so do longer contexts whose partials would go to the workspace,
// where a workgroup streaming one group's whole cache region (every group
// at once, far apart) read HBM more slowly than the chunk items do: 8196 keys
// at 64 sequences x 8 KV heads took 473 us whole against 437 us as chunks
// plus merge.  With the partials in LDS the whole form is ahead: at 64 x 8
// groups of one query, 43 against 50 us at 768 keys, 101 against 113 us at
// 2048 and 145 against 164 us at 3072.
static bool attn_whole(const AttnPlan &p)
{
    return p.sh.nmg == 1 && p.sh.Q * p.sh.G <= 32 &&
           (p.sh.nchunks <= kWholeMaxChunks || p.sh.Q * p.sh.G * p.sh.nchunks <= kWholeLdsParts) &&
           p.sh.B * p.sh.Hkv >= 2 * (int64_t)device_cu_count() && p.sh.cps == 1;
}

template <typename S>
static void launch_attn(const AttnBufs &bf, const AttnPlan &p, hipStream_t st)
{
    if (attn_whole(p)) {
        AttnShape sh = p.sh;
        sh.cps = (int)sh.nchunks;                  // one item: every chunk of the group
        sh.nsplit = 1;
        const int64_t nid = cdiv(sh.B, 8) * 8 * sh.Hkv;
        const int64_t grid = std::min<int64_t>(nid, (int64_t)device_cu_count() * 2 / 8 * 8);
        if (sh.nchunks <= kWholeMaxChunks)
            launch_kernel((attn_kernel<S, false, false, true, kWholeLdsSmall>), dim3((unsigned)grid),
                          dim3(kAttnWaves * kWave), 0, st, bf, bf.kv_len, sh, nid);
        else
            launch_kernel((attn_kernel<S, false, false, true, kWholeLdsParts>), dim3((unsigned)grid),
                          dim3(kAttnWaves * kWave), 0, st, bf, bf.kv_len, sh, nid);
        return;
    }
    if (p.sh.nmg > 1)
        launch_kernel((attn_kernel<S, true>), dim3((unsigned)p.grid), dim3(kAttnWaves * kWave), 0, st, bf, bf.kv_len,
                      p.sh, p.nid);
    else
        launch_kernel((attn_kernel<S, false>), dim3((unsigned)p.grid), dim3(kAttnWaves * kWave), 0, st, bf, bf.kv_len,
                      p.sh, p.nid);
    launch_kernel((attn_merge_kernel<S>), dim3((unsigned)(p.sh.B * p.sh.Q * p.sh.Hq)), dim3((unsigned)p.merge_threads),
                  0, st, (const float *)bf.part, bf.kv_len, bf.o, p.sh);
}

// The split comparison variant: the chunk kernel in its SPL form, then the
// merge over the splits (none with a single split: the kernel wrote out).
template <typename S>
static void launch_attn_split(const AttnBufs &bf, const AttnPlan &p, hipStream_t st)
{
    launch_kernel((attn_kernel<S, false, true>), dim3((unsigned)p.grid), dim3(kAttnWaves * kWave), 0, st, bf, bf.kv_len,
                  p.sh, p.nid);
    if (p.sh.nchunks > 1)
        launch_kernel((attn_merge_kernel<S>), dim3((unsigned)(p.sh.B * p.sh.Q * p.sh.Hq)),
                      dim3((unsigned)p.merge_threads), 0, st, (const float *)bf.part, bf.kv_len, bf.o, p.sh);
}

// Shared by the entry points: validation, the launch plan, the launches.
static bi_status attn_run(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                          int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv, int32_t D,
                          float scale, int32_t causal, int32_t dtype, int32_t kv_layout, void *ws, size_t ws_bytes,
                          hipStream_t stream)
{
    bi_status s = check_attn(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, dtype);
    if (s != BI_OK) return s;
    if (kv_layout != 0 && kv_layout != 1) return BI_ERR_SHAPE;
    if (!ws) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    const AttnPlan p = attn_plan(B, Q, max_kv_len, Lcap, Hq, Hkv, scale, causal, kv_layout);
    if (ws_bytes < p.parts) return BI_ERR_WORKSPACE;
    AttnBufs bf{(const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, kv_len, (uint16_t *)o, (float *)ws};
    (void)hipGetLastError();
    // prompts: at least one block of 128 query rows per KV head, at most
    // two ranges of keys
    const int64_t R = Q * (Hq / Hkv), nrb = cdiv(R, kPreRows);
    if (R >= kPreRows && max_kv_len <= (int64_t)kPreMaxRanges * kRange * kChunk && B * Hkv * nrb < (1ll << 31)) {
        const dim3 grid((unsigned)(B * Hkv * nrb)), block(kPreWaves * kWave);
        const bool one = max_kv_len <= (int64_t)kRange * kChunk;
        if (dtype == BI_BF16) {
            if (one) launch_kernel((attn_prefill_kernel<BF16, 1>), grid, block, 0, stream, bf, kv_len, p.sh, (int)nrb);
            else launch_kernel((attn_prefill_kernel<BF16, 2>), grid, block, 0, stream, bf, kv_len, p.sh, (int)nrb);
        } else {
            if (one) launch_kernel((attn_prefill_kernel<F16, 1>), grid, block, 0, stream, bf, kv_len, p.sh, (int)nrb);
            else launch_kernel((attn_prefill_kernel<F16, 2>), grid, block, 0, stream, bf, kv_len, p.sh, (int)nrb);
        }
        return launch_status();
    }
    if (dtype == BI_BF16) launch_attn<BF16>(bf, p, stream);
    else launch_attn<F16>(bf, p, stream);
    return launch_status();
}

// ---------------------------------------------------------------------------
// Fixed scratch for callers that cannot allocate (bi_sdpa_noalloc): the chunk
// partials live in this file-scope device array, one copy per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the symbol); it passes the device
// address hipGetSymbolAddress returned for the current device.
constexpr size_t kAttnScratchBytes = 64ull << 20;
__device__ __align__(256) char attn_scratch[kAttnScratchBytes];

constexpr int kMaxDevices = 64;
static void *g_attn_scratch[kMaxDevices];
static std::mutex g_attn_scratch_mu;

// The current device's scratch address, looked up once per device.
static bi_status attn_scratch_ptr(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BI_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_attn_scratch_mu);
    if (!g_attn_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(attn_scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return BI_ERR_LAUNCH;
        }
        g_attn_scratch[dev] = p;
    }
    *out = g_attn_scratch[dev];
    return BI_OK;
}

}  // namespace bi

using namespace bi;

extern "C" size_t bi_sdpa_workspace_bytes(int64_t B, int64_t Q, int64_t max_kv_len, int32_t Hq, int32_t D)
{
    if (B < 1 || Q < 1 || max_kv_len < 1 || Hq < 1 || D != kHeadDim) return 0;
    return attn_partial_bytes(B, Q, max_kv_len, Hq);
}

extern "C" bi_status bi_sdpa(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                             int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                             int32_t D, float scale, int32_t causal, int32_t dtype, int32_t kv_layout, void *ws,
                             size_t ws_bytes, hipStream_t stream)
{
    return attn_run(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, scale, causal, dtype, kv_layout, ws,
                    ws_bytes, stream);
}

// chunks per split for `splits` splits of max_kv_len keys, and the resulting split count
static void split_geometry(int64_t max_kv_len, int32_t splits, int &cps, int64_t &nsplit)
{
    const int64_t nch = cdiv(max_kv_len, kChunk);
    cps = (int)cdiv(nch, std::min<int64_t>(splits, nch));
    nsplit = cdiv(nch, cps);
}

extern "C" size_t bi_sdpa_split_workspace_bytes(int64_t B, int64_t Q, int64_t max_kv_len, int32_t Hq, int32_t D,
                                                int32_t splits)
{
    if (B < 1 || Q < 1 || max_kv_len < 1 || max_kv_len > kMaxKv || Hq < 1 || D != kHeadDim || splits < 1) return 0;
    int cps;
    int64_t nsplit;
    split_geometry(max_kv_len, splits, cps, nsplit);
    return nsplit == 1 ? 0 : (size_t)(B * Q * Hq) * (size_t)nsplit * kPartStride * sizeof(float);
}

extern "C" bi_status bi_sdpa_split(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                                   int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                                   int32_t D, float scale, int32_t causal, int32_t dtype, int32_t kv_layout,
                                   int32_t splits, void *ws, size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_attn(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, dtype);
    if (s != BI_OK) return s;
    if (kv_layout != 0 && kv_layout != 1) return BI_ERR_SHAPE;
    if (splits < 1) return BI_ERR_SHAPE;
    if (Q * (Hq / Hkv) > 16) return BI_ERR_UNSUPPORTED;        // one 16-row query tile per (sequence, KV head)
    int cps;
    int64_t nsplit;
    split_geometry(max_kv_len, splits, cps, nsplit);
    const size_t need = bi_sdpa_split_workspace_bytes(B, Q, max_kv_len, Hq, D, splits);
    if (need > 0 && (!ws || ws_bytes < need)) return BI_ERR_WORKSPACE;
    if (need > 0 && !host_aligned16(ws)) return BI_ERR_ALIGN;
    const AttnPlan p = attn_plan(B, Q, max_kv_len, Lcap, Hq, Hkv, scale, causal, kv_layout, cps);
    AttnBufs bf{(const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, kv_len, (uint16_t *)o, (float *)ws};
    (void)hipGetLastError();
    if (dtype == BI_BF16) launch_attn_split<BF16>(bf, p, stream);
    else launch_attn_split<F16>(bf, p, stream);
    return launch_status();
}

extern "C" size_t bi_sdpa_noalloc_max_bytes(void) { return kAttnScratchBytes; }

extern "C" bi_status bi_sdpa_noalloc(const void *q, const void *k, const void *v, void *o, const int32_t *kv_len,
                                     int64_t max_kv_len, int64_t B, int64_t Q, int64_t Lcap, int32_t Hq, int32_t Hkv,
                                     int32_t D, float scale, int32_t causal, int32_t dtype, int32_t kv_layout,
                                     hipStream_t stream)
{
    bi_status s = check_attn(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, dtype);
    if (s != BI_OK) return s;
    if (bi_sdpa_workspace_bytes(B, Q, max_kv_len, Hq, D) > kAttnScratchBytes) return BI_ERR_WORKSPACE;
    void *ws = nullptr;
    s = attn_scratch_ptr(&ws);
    if (s != BI_OK) return s;
    return attn_run(q, k, v, o, kv_len, max_kv_len, B, Q, Lcap, Hq, Hkv, D, scale, causal, dtype, kv_layout, ws,
                    kAttnScratchBytes, stream);
}
