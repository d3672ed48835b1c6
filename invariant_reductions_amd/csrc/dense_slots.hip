// dense_slots.hip -- the slot-group form of the batch-invariant dense matmul
// for short M (bi_matmul_ws) and its SwiGLU-fused variant (bi_matmul_swiglu).
// Same tree as every dense kernel (dense_common.hpp); sources as there, and
// "Batch-invariant kernels ..." (Mental model: pointwise ops are invariant, so
// the activation may be fused into the producing reduction).
#include "dense_common.hpp"

#include <algorithm>

namespace bi {

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
// SwiGLU activation of a gate/up product interleaved in blocks of 8 columns
// (EPI_SWIGLU: the 16 columns of every wave are gate columns 8j .. 8j + 7
// followed by the up columns of the same indices, j = the wave's global
// 16-column index; a[m, 8j + i] = silu_mul1(y[m, 16j + i], y[m, 16j + 8 + i])
// from the bf16-rounded y exactly as bi_silu_mul would read it).  The pair
// sits in lanes c and c + 8 of one row of the accumulator layout, so the
// epilogue stays inside the wave.
enum SlotEpilogue { EPI_Y = 0, EPI_SWIGLU = 1 };

template <typename S, int MT, int Q, int DW, int OCC, int EPI, int NW, bool PK>
__global__ __launch_bounds__(NW * kWave, OCC)
void dense_slots_kernel(const typename S::store_t *__restrict__ x, const typename S::store_t *__restrict__ w,
                        typename S::store_t *__restrict__ y, float *__restrict__ part,
                        unsigned *__restrict__ counters, int64_t M, int64_t N, int64_t K)
{
    using G = DenseGeom<S>;
    using T = typename S::store_t;
    constexpr int P = kDenseWaves;                 // K slots (the tree)
    constexpr int NT = NW * kWave;                 // NW waves: 16 NW columns per tile
    constexpr int GRP = P / Q;                     // slot groups per column tile
    constexpr int TR = MT * 16, KB = G::KB;
    constexpr int XS = KB + 8;                     // LDS row stride: 272 bytes, 16-byte aligned, 4-bank shift per row
    constexpr int XCH = TR * (KB / 8);             // 16-byte chunks in one block of x
    constexpr int XPT = (XCH + NT - 1) / NT;       // chunks staged per thread (the last round may be partial)
    constexpr int DX = 3;                          // x register ring depth (DW: W ring depth)
    constexpr int U = lcm_c(lcm_c(3, DW), Q);       // unroll: a multiple of the LDS ring (3 = DX), DW and Q
    static_assert(G::CPB == 4 && XPT <= 4, "slot kernel geometry");
    __shared__ __attribute__((aligned(16))) T xs[3][TR][XS];
    __shared__ int s_last;

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int ct = blockIdx.x, grp = blockIdx.y;
    // Row chunk blockIdx.z: rows [TR z, TR z + TR) of a call with more rows
    // than one tile; with an exchange, each (column tile, row chunk) has its
    // own counter and group sums
    {
        const int64_t r0 = (int64_t)blockIdx.z * TR;
        x += r0 * K;
        y += r0 * (EPI == EPI_Y ? N : N / 2);
        M -= r0;
    }
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

    const int64_t n = (int64_t)ct * (NW * 16) + wave * 16 + c;
    const bool nok = n < N;
    const T *wr = w + (nok ? n : N - 1) * K;     // padding columns read a real row, never stored
    const int64_t nrg = (N + 15) / 16;
    const int64_t wrg = (int64_t)ct * NW + wave < nrg ? (int64_t)ct * NW + wave : nrg - 1;   // packed row group
    const int t = threadIdx.x, xc = t & 15;

    struct XChunks { uint4 v0, v1, v2, v3; };
    XChunks xr0, xr1, xr2;
    auto xreg = [&](auto sc) -> XChunks & {
        constexpr int sl = decltype(sc)::value % DX;
        if constexpr (sl == 0) return xr0;
        else if constexpr (sl == 1) return xr1;
        else return xr2;
    };
    // thread t stages chunks t + h NT (< XCH) of the block: row / 16, 16 bytes
    // at (chunk % 16) * 16.  A chunk index past the block (partial last round)
    // loads the block's last chunk and is not staged.
    auto load_x = [&](XChunks &r, int u) {
        const int64_t kb = (int64_t)block_of(u) * KB + xc * 8;
        static_for<0, XPT>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            const int ch = t + h * NT < XCH ? t + h * NT : XCH - 1;
            const int row = ch >> 4;
            const uint4 v = *reinterpret_cast<const uint4 *>(x + (int64_t)(row < M ? row : M - 1) * K + kb);
            if constexpr (h == 0) r.v0 = v;
            else if constexpr (h == 1) r.v1 = v;
            else if constexpr (h == 2) r.v2 = v;
            else r.v3 = v;
        });
    };
    auto store_x = [&](const XChunks &r, int buf) {
        static_for<0, XPT>([&](auto hc) {
            constexpr int h = decltype(hc)::value;
            if (XCH % NT == 0 || h + 1 < XPT || t + h * NT < XCH) {
                const int row = (t + h * NT) >> 4;
                *reinterpret_cast<uint4 *>(&xs[buf][row][xc * 8]) = h == 0 ? r.v0 : h == 1 ? r.v1 : h == 2 ? r.v2 : r.v3;
            }
        });
    };
    uint4 wb[DW][G::CPB];
    auto load_w = [&](uint4 (&B)[G::CPB], int u) {
        if constexpr (PK) {
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci)
                B[ci] = *reinterpret_cast<const uint4 *>(w + packed_off(wrg, nb, block_of(u), ci, lane));
        } else {
            const T *p = wr + (int64_t)block_of(u) * KB;
#pragma unroll
            for (int ci = 0; ci < G::CPB; ++ci) B[ci] = *reinterpret_cast<const uint4 *>(p + G::chunk_off(g, ci));
        }
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
        if (!nok) return;                          // EPI_SWIGLU: N % 16 == 0, so a whole wave is in or out
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m * 16 + g * 4 + r;
                const T b = S::narrow(v[m][r]);
                if constexpr (EPI == EPI_Y) {
                    if (row < M) y[row * N + n] = b;
                } else {
                    const T u = (T)__shfl_xor((int)b, 8, kWave);   // the up value of this lane's gate column
                    if (c < 8 && row < M)
                        y[row * (N / 2) + ((int64_t)ct * NW + wave) * 8 + c] = silu_mul1(b, u);
                }
            }
    };
    if constexpr (GRP == 1) {
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
        const int64_t tile = (int64_t)blockIdx.z * gridDim.x + ct;           // (row chunk, column tile)
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc(part + tile * GRP * NW * (REC / 4), (short)0, GRP * NW * REC, 0x00020000);
#pragma unroll
        for (int m = 0; m < MT; ++m)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, h[m]), rsrc,
                                                   (grp * NW + wave) * REC + m * kWave * 16 + lane * 16, 0, CPOL_DEVICE);
        __builtin_amdgcn_s_waitcnt(0);             // every store of this wave acknowledged
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (unsigned)(GRP - 1);
        }
        __syncthreads();
        if (!s_last) return;
        if (threadIdx.x == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        f32x4 out[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f32x4 v[GRP];
#pragma unroll
            for (int q = 0; q < GRP; ++q)
                v[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rsrc, (q * NW + wave) * REC + m * kWave * 16 + lane * 16, 0, CPOL_DEVICE));
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
constexpr int64_t kSlotExchRowsMax = 128;                   // rows of the form with an exchange
constexpr size_t kSlotCounterBytes = kSlotMaxTiles * sizeof(unsigned);

// Row tiles of the slot form: four (padding rows read row M - 1 and are
// never stored), or one up to 16 rows on a weight with enough column tiles
// for a workgroup per CU with half the slots.  Two tiles at 17..32 rows ran
// slower than four on every decoder projection (18.9 against 14.8 us on 6144
// x 4096 at 32 rows; 16.3 against 14.8 at 16 rows): the four-tile
// instantiations get the slot pairs over 64- or 96-column tiles and their
// register budget; on the wide weights one tile stays ~2% ahead.
static int slot_mt(int64_t M, int64_t N)
{
    return M <= 16 && cdiv(N, kSlotTileCols) * 2 >= (int64_t)device_cu_count() ? 1 : 4;
}

// Row counts the slot form takes: 16 < M <= 64, and down to M = 9 or 13 when
// the weight is large -- there the one-workgroup-per-tile kernel reads each
// tile's x rows once per column tile from L2 and falls behind the LDS-shared
// x of the slot form (measured on the decoder's projections; at M <= 8 and
// on 4096 x 4096 the streaming kernel stays ahead).
static bool slot_takes(int64_t M, int64_t N, int64_t K)
{
    if (M > kSlotExchRowsMax || M < 1) return false;
    // two 64-row chunks, each meeting its own group sums, where the tiled
    // kernel's 128 x 128 tiles would fill under 5/8 of the CUs (the narrow
    // projections of a 16-sequence verify block: 80 x 4096 x 14336 40 us,
    // 62 us with all eight slots per workgroup); from 129 rows the chunks
    // with all eight slots per workgroup and no exchange are ahead (320 x
    // 4096 x 14336: 85 against 104 us), bi_matmul's form
    if (M > 64) return cdiv(N, 128) * 8 < 5 * (int64_t)device_cu_count();
    if (M > 16) return true;
    if (N >= 16384) return M > 8;
    return M > 12 && N * K > 4096ll * 4096ll;
}

static size_t slot_ws_bytes(int64_t M, int64_t N, int groups)
{
    const int64_t rec = (int64_t)slot_mt(M, N) * 4 * kWave * (int64_t)sizeof(float);
    const int64_t nrc = cdiv(M, slot_mt(M, N) * 16);                    // row chunks, each with its own sums
    return kSlotCounterBytes + (size_t)(nrc * cdiv(N, kSlotTileCols) * groups * kDenseWaves * rec);
}

template <typename S, int MT, int Q, int EPI, bool PK, int NW = kDenseWaves>
static void launch_slots_t(const void *x, const void *w, void *y, void *ws, int64_t M, int64_t N, int64_t K,
                           hipStream_t st)
{
    using T = typename S::store_t;
    // group-sum records: (N / 16 NW tiles) x (8 / Q groups) x NW waves fit in
    // slot_ws_bytes's (N / 128) x 8 x 8 whenever NW Q >= 8 or there is no exchange
    static_assert(NW == kDenseWaves || Q == kDenseWaves || NW * Q >= kDenseWaves, "group sums exceed the workspace");
    const int64_t ntc = cdiv(N, NW * 16), nrc = cdiv(M, MT * 16);      // column tiles, row chunks
    unsigned *counters = (unsigned *)ws;
    float *part = (float *)((char *)ws + kSlotCounterBytes);
    // W ring depth and waves per SIMD: two workgroups per CU (at most 128
    // VGPRs) wherever the accumulators allow it.
    constexpr int DW = MT == 4 ? 2 : 4;
    constexpr int OCC = Q * MT <= 4 ? 4 : 2;
    launch_kernel((dense_slots_kernel<S, MT, Q, DW, OCC, EPI, NW, PK>),
                  dim3((unsigned)ntc, (unsigned)(kDenseWaves / Q), (unsigned)nrc), dim3(NW * kWave), 0, st,
                  (const T *)x, (const T *)w, (T *)y, part, counters, M, N, K);
}

// More than 64 rows, few column tiles (bi_matmul's path, dense.hip): one
// workgroup of 4 waves per (64-column tile, 64-row chunk) with all eight
// slots -- no exchange, no workspace -- the row chunks of a column tile
// reading the same W strip.  16-bit types, transposed or packed W, K a
// multiple of the block, x and W 16-byte aligned, M <= kSlotRowsMax.
template <typename S>
void launch_dense_slot_rows(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, bool packed,
                            hipStream_t st)
{
    using T = typename S::store_t;
    constexpr int NW = 4;
    const int64_t ntc = cdiv(N, NW * 16), nrc = cdiv(M, 64);
    const dim3 grid((unsigned)ntc, 1u, (unsigned)nrc);
    if (packed)
        launch_kernel((dense_slots_kernel<S, 4, 8, 2, 2, EPI_Y, NW, true>), grid, dim3(NW * kWave), 0, st,
                      (const T *)x, (const T *)w, (T *)y, (float *)nullptr, (unsigned *)nullptr, M, N, K);
    else
        launch_kernel((dense_slots_kernel<S, 4, 8, 2, 2, EPI_Y, NW, false>), grid, dim3(NW * kWave), 0, st,
                      (const T *)x, (const T *)w, (T *)y, (float *)nullptr, (unsigned *)nullptr, M, N, K);
}
template void launch_dense_slot_rows<BF16>(const void *, const void *, void *, int64_t, int64_t, int64_t, bool,
                                           hipStream_t);
template void launch_dense_slot_rows<F16>(const void *, const void *, void *, int64_t, int64_t, int64_t, bool,
                                          hipStream_t);

// Share of the CUs busy over the rounds of a grid of `tiles` one-per-CU workgroups.
static double cu_balance(int64_t tiles, int64_t cu) { return (double)tiles / (double)(cdiv(tiles, cu) * cu); }

// Slots per workgroup: the largest group that still gives at least one
// workgroup per CU (MT = 4 keeps at most four slots in registers).
template <typename S, int MT, int EPI, bool PK>
static void launch_slots_mt(const void *x, const void *w, void *y, void *ws, int64_t M, int64_t N, int64_t K,
                            hipStream_t st)
{
    // (tiles counted over all row chunks of a call past one chunk)
    const int64_t nrc = cdiv(M, MT * 16), ntc = cdiv(N, kSlotTileCols) * nrc, cu = device_cu_count();
    // All eight slots in one workgroup (no exchange) once the column tiles
    // alone come close to one per CU; with 7-wave (112-column) tiles when
    // those fill the CUs more evenly (one such workgroup runs per CU).
    if (ntc * 4 >= cu * 3) {
        if (cu_balance(cdiv(N, 7 * 16) * nrc, cu) > cu_balance(ntc, cu) + 0.02)
            launch_slots_t<S, MT, 8, EPI, PK, 7>(x, w, y, ws, M, N, K, st);
        else
            launch_slots_t<S, MT, 8, EPI, PK>(x, w, y, ws, M, N, K, st);
        return;
    }
    if (ntc * 2 >= cu) {
        launch_slots_t<S, MT, 4, EPI, PK>(x, w, y, ws, M, N, K, st);
    } else if constexpr (MT == 4) {
        // Few column tiles: 64-column tiles with pairs of slots (four groups)
        // give as many workgroups as 128-column tiles with single slots, but
        // half the group sums to exchange and a quarter for the last arriver
        // to read; 96-column tiles where those fill the CUs more evenly
        // (6144 columns: 256 workgroups instead of 384).
        if (cu_balance(cdiv(N, 6 * 16) * 4 * nrc, cu) > cu_balance(cdiv(N, 4 * 16) * 4 * nrc, cu) + 0.02)
            launch_slots_t<S, MT, 2, EPI, PK, 6>(x, w, y, ws, M, N, K, st);
        else
            launch_slots_t<S, MT, 2, EPI, PK, 4>(x, w, y, ws, M, N, K, st);
    } else {
        if (ntc * 4 >= cu) launch_slots_t<S, MT, 2, EPI, PK>(x, w, y, ws, M, N, K, st);
        else launch_slots_t<S, MT, 1, EPI, PK>(x, w, y, ws, M, N, K, st);
    }
}

template <typename S, int EPI = EPI_Y>
static bool try_launch_slots(const void *x, const void *w, void *y, void *ws, size_t ws_bytes, int64_t M,
                             int64_t N, int64_t K, bool packed, hipStream_t st)
{
    using G = DenseGeom<S>;
    if (!ws || !slot_takes(M, N, K) || K % G::KB != 0 || !host_aligned16(x) || !host_aligned16(w) ||
        !host_aligned16(ws))
        return false;
    if (ws_bytes < slot_ws_bytes(M, N, kDenseWaves)) return false;
    if (packed) {
        if (slot_mt(M, N) == 1) launch_slots_mt<S, 1, EPI, true>(x, w, y, ws, M, N, K, st);
        else launch_slots_mt<S, 4, EPI, true>(x, w, y, ws, M, N, K, st);
    } else {
        if (slot_mt(M, N) == 1) launch_slots_mt<S, 1, EPI, false>(x, w, y, ws, M, N, K, st);
        else launch_slots_mt<S, 4, EPI, false>(x, w, y, ws, M, N, K, st);
    }
    return true;
}

// SwiGLU activation of an interleaved gate/up product (the fallback of
// bi_matmul_swiglu): in each row, columns 16 i + j and 16 i + 8 + j are gate
// and up of activation 8 i + j.  Thread = the 8 activations of one block.
__global__ void swiglu_il_kernel(const uint16_t *__restrict__ gu, uint16_t *__restrict__ a, int64_t rows, int64_t F)
{
    const int64_t fc = F / 8, n = rows * fc;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = c / fc, i = c - r * fc;
        const uint16_t *gp = gu + r * 2 * F + i * 16;
        const uint4 gv = *reinterpret_cast<const uint4 *>(gp), uv = *reinterpret_cast<const uint4 *>(gp + 8);
        const uint16_t *g8 = reinterpret_cast<const uint16_t *>(&gv), *u8 = reinterpret_cast<const uint16_t *>(&uv);
        uint16_t o8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o8[e] = silu_mul1(g8[e], u8[e]);
        *reinterpret_cast<uint4 *>(a + r * F + i * 8) = __builtin_bit_cast(uint4, o8);
    }
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace bi

using namespace bi;

extern "C" size_t bi_matmul_ws_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t w_layout)
{
    if (N < 1 || K < 1 || !slot_takes(M, N, K) || (w_layout != W_TRANS && w_layout != W_PACKED) || (dtype != BI_BF16 && dtype != BI_F16) ||
        cdiv(N, kSlotTileCols) > kSlotMaxTiles || (M > 64 && cdiv(M, 64) * cdiv(N, 64) > kSlotMaxTiles))
        return 0;
    return slot_ws_bytes(M, N, kDenseWaves);
}

extern "C" bi_status bi_matmul_ws(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K,
                                  int32_t dtype, int32_t w_layout, void *ws, size_t ws_bytes, hipStream_t stream)
{
    bi_status s = check_dense(x, w, y, M, N, K, dtype, w_layout);
    if (s != BI_OK) return s;
    const size_t need = bi_matmul_ws_workspace_bytes(M, N, K, dtype, w_layout);
    if (need > 0 && (!ws || ws_bytes < need)) return BI_ERR_WORKSPACE;
    if (need > 0 && !host_aligned16(ws)) return BI_ERR_ALIGN;
    (void)hipGetLastError();
    bool done = false;
    if (need > 0) {
        const bool pk = w_layout == W_PACKED;
        if (dtype == BI_BF16) done = try_launch_slots<BF16>(x, w, y, ws, ws_bytes, M, N, K, pk, stream);
        else done = try_launch_slots<F16>(x, w, y, ws, ws_bytes, M, N, K, pk, stream);
    }
    if (!done) dispatch_dense(x, w, y, nullptr, M, N, K, dtype, w_layout, 1, stream);
    return launch_status();
}

extern "C" size_t bi_matmul_swiglu_workspace_bytes(int64_t M, int64_t F, int64_t K, int32_t dtype)
{
    if (M < 1 || F < 1 || K < 1 || dtype != BI_BF16 || F % 8 || M > (1ll << 31) || F > (1ll << 30)) return 0;
    // the slot form's counter area, then its group sums or (any other shape)
    // the scratch product: never both in one call
    const size_t slot = bi_matmul_ws_workspace_bytes(M, 2 * F, K, dtype, 1);
    const size_t prod = align256((size_t)M * (size_t)(2 * F) * sizeof(uint16_t));
    return kSlotCounterBytes + std::max(slot > 0 ? slot - kSlotCounterBytes : 0, prod);
}

extern "C" bi_status bi_matmul_swiglu(const void *x, const void *w_il, void *a, int64_t M, int64_t F, int64_t K,
                                      int32_t dtype, int32_t w_layout, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (F < 1 || F > (1ll << 30)) return BI_ERR_SHAPE;
    bi_status s = check_dense(x, w_il, a, M, 2 * F, K, dtype, w_layout);
    if (s != BI_OK) return s;
    if (w_layout == W_NATURAL) return BI_ERR_UNSUPPORTED;
    if (dtype != BI_BF16) return BI_ERR_DTYPE;
    if (F % 8) return BI_ERR_SHAPE;
    if (!host_aligned16(a)) return BI_ERR_ALIGN;
    const size_t need = bi_matmul_swiglu_workspace_bytes(M, F, K, dtype);
    if (!ws || ws_bytes < need) return BI_ERR_WORKSPACE;
    if (!host_aligned16(ws)) return BI_ERR_ALIGN;
    const size_t slot = bi_matmul_ws_workspace_bytes(M, 2 * F, K, dtype, 1);
    (void)hipGetLastError();
    if (slot > 0 &&
        try_launch_slots<BF16, EPI_SWIGLU>(x, w_il, a, ws, slot, M, 2 * F, K, w_layout == W_PACKED, stream))
        return launch_status();
    // any other shape: the product into the scratch after the counter area
    // (which stays zero for later slot-form calls on this workspace), then
    // the activation
    uint16_t *gu = (uint16_t *)((char *)ws + kSlotCounterBytes);
    dispatch_dense(x, w_il, gu, nullptr, M, 2 * F, K, dtype, w_layout, 1, stream);
    const int64_t n = M * F / 8;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(n, 256), 65536);
    launch_kernel(swiglu_il_kernel, dim3(blocks), dim3(256), 0, stream, (const uint16_t *)gu, (uint16_t *)a, M, F);
    return launch_status();
}
