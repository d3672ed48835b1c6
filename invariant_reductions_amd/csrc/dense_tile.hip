// dense_tile.hip -- LDS-tiled form of the batch-invariant dense matmul for
// long M (verify blocks of many sequences, prompts): 16-bit types, weights
// transposed [N, K] or tile-packed, K a multiple of the 128-element block.
//
// Same tree as every dense kernel (dense_common.hpp; sources as there): K
// block b belongs to slot b mod 8, a slot's blocks are accumulated in
// ascending order by v_mfma_f32_16x16x32_{bf16,f16} in four steps of 32 (lane
// group g supplying the 8 elements at 32 s + 8 g), and the eight slot
// partials are added as ((p0 + p1) + (p2 + p3)) + ((p4 + p5) + (p6 + p7)).
//
// The other kernels give each wave its own slot, so no two waves ever read
// the same operand and nothing is shared through LDS; past 64 rows that
// leaves the MFMA units mostly idle.  Here all eight waves of a workgroup
// work on the same block at once, on different parts of a 128 x 128 output
// tile (wave = 64 rows x 32 columns), with the block's x and W tiles staged
// once in LDS.  The workgroup walks the slots one after another -- slot 0's
// blocks 0, 8, 16, ..., then slot 1's, ... -- and folds each finished slot
// partial into the pairwise sum right away, so only three partial sums are
// live besides the running accumulator:
//   after slot 0: S0 = p0          after slot 4: S1 = p4
//   after slot 1: S0 = S0 + p1     after slot 5: S1 = S1 + p5
//   after slot 2: S1 = p2          after slot 6: S2 = p6
//   after slot 3: S1 = S1 + p3,    after slot 7: S2 = S2 + p7, S1 = S1 + S2,
//                 S0 = S0 + S1                   S0 = S0 + S1
// which is the tree above, term for term.
//
// Operand staging: the block's x tile (8 row tiles of 16) and W tile (8
// column tiles of 16) are stored in LDS in the MFMA operand order -- 1 KiB
// per (tile, step), lane l's 16 bytes at 16 l -- so each operand read is one
// conflict-free ds_read_b128.  They are written by direct global-to-LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at 16 l of the 1 KiB the
// instruction addresses), in stages of half a block, four buffers deep: the
// three stages after the one being multiplied are in flight.
#include "dense_common.hpp"

#include <algorithm>

namespace bi {

constexpr int kTileRows = 128, kTileCols = 128;
constexpr int kTileWaves = 8;                     // 2 (rows) x 4 (columns) waves of 64 x 32
constexpr int kTileGroupM = 8;                    // row tiles per launch-order group

template <typename S, bool PK>
__global__ __launch_bounds__(kTileWaves * kWave, 1)
void dense_tile_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, uint16_t *__restrict__ y,
                       int M, int N, int K, int ntm, int ntn, int per_xcd)
{
    // four stage buffers, each half a block: [0: x, 1: W][tile][step of the
    // half][lane] (32 KiB); separate arrays, so that the compiler can tell the
    // loads streaming into one from the reads of another (a read of a buffer
    // being filled would otherwise wait for every load in flight)
    typedef uint4 Stage[2][8][2][kWave];
    __shared__ __attribute__((aligned(16))) Stage lds0, lds1, lds2, lds3;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, c = lane & 15;
    const int wm = wave & 1, wn = wave >> 1;      // rows 64 wm .. +64, columns 32 wn .. +32 of the tile

    // Launch order: workgroup id -> (XCD = id % 8, k = id / 8); XCD x takes
    // the tiles x * per_xcd .. + per_xcd - 1 of a list that walks groups of
    // kTileGroupM row tiles column tile by column tile, so the workgroups one
    // XCD runs together share W and x tiles in its L2.
    const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
    if (k8 >= per_xcd) return;
    const int t = xcd * per_xcd + k8;
    if (t >= ntm * ntn) return;
    const int grp = t / (kTileGroupM * ntn), idx = t - grp * kTileGroupM * ntn;
    const int gm = min(kTileGroupM, ntm - grp * kTileGroupM);
    const int tn = idx / gm, tm = grp * kTileGroupM + (idx - (idx / gm) * gm);

    const int nb = K / 128, nrg = (N + 15) / 16;
    const int q = nb >> 3, r = nb & 7;            // slot s holds q + (s < r) blocks
    // block of the i-th item in slot-major order
    auto block_of = [&](int i) {
        int s, j;
        if (i < r * (q + 1)) {
            s = i / (q + 1);
            j = i - s * (q + 1);
        } else {
            const int i2 = i - r * (q + 1);
            s = r + i2 / q;
            j = i2 - (s - r) * q;
        }
        return s + 8 * j;
    };

    // Staging: waves 0-3 load x, waves 4-7 load W; wave v takes tiles
    // 2 (v mod 4) and 2 (v mod 4) + 1 of its operand, all four steps of each
    // (eight 1 KiB chunks per block).  Per-lane source rows are fixed for the
    // whole walk.
    const bool isw = wave >= 4;
    const int tl0 = 2 * (wave & 3);
    const uint16_t *src[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int tl = tl0 + h;
        if (!isw) {
            const int row = min(tm * kTileRows + tl * 16 + c, M - 1);          // padding rows read a real row
            src[h] = x + (int64_t)row * K + g * 8;
        } else if constexpr (PK) {
            const int rg = min(tn * (kTileCols / 16) + tl, nrg - 1);
            src[h] = w + packed_off(rg, nb, 0, 0, lane);
        } else {
            const int n = min(tn * kTileCols + tl * 16 + c, N - 1);            // padding columns read a real row
            src[h] = w + (int64_t)n * K + g * 8;
        }
    }
    // element offsets of (block b, step st) from src: packed chunks are 512
    // elements per step and 2048 per block; row-major ones 32 and 128
    const int sstep = (isw && PK) ? 4 * 8 * 16 : 32, sblk = (isw && PK) ? 4 * kWave * 8 : 128;
    // stage u = (item u / 2, half u % 2): steps 2 (u % 2) and 2 (u % 2) + 1
    // of block block_of(u / 2); four loads per wave
    auto stage = [&](Stage &buf, int u) {
        const int64_t base = (int64_t)block_of(u >> 1) * sblk + (u & 1) * 2 * sstep;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int st = 0; st < 2; ++st)
                __builtin_amdgcn_global_load_lds(src[h] + base + st * sstep, &buf[isw ? 1 : 0][tl0 + h][st][0], 16,
                                                 0, 0);
    };

    f32x4 acc[4][2], S0[4][2], S1[4][2], S2[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = S0[i][j] = S1[i][j] = S2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // One half block: two steps.  A step's six operands (four x tiles, two W
    // tiles) are read by one asm block that also waits for them: the compiler
    // cannot tell a plain LDS read of this buffer from the direct loads still
    // streaming into the other three, and would make every read wait for all
    // of them.  The second step's reads are issued before the first step
    // multiplies.
    const uint32_t xoff = (uint32_t)(((wm * 4) * 2 * kWave + lane) * 16);              // x tile 4 wm, step 0
    const uint32_t woff = (uint32_t)(((8 + wn * 2) * 2 * kWave + lane) * 16);          // W tile 2 wn, step 0
    auto multiply = [&](const Stage &buf) {
        const uint32_t base = (uint32_t)(uintptr_t)&buf[0][0][0][0];
        i32x4 a[2][4], bb[2][2];
        auto fetch = [&](int st, i32x4 (&ar)[4], i32x4 (&br)[2]) {
            const uint32_t xa = base + xoff + st * kWave * 16, wa = base + woff + st * kWave * 16;
            asm volatile(
                "ds_read_b128 %0, %6\n\t"
                "ds_read_b128 %1, %6 offset:2048\n\t"
                "ds_read_b128 %2, %6 offset:4096\n\t"
                "ds_read_b128 %3, %6 offset:6144\n\t"
                "ds_read_b128 %4, %7\n\t"
                "ds_read_b128 %5, %7 offset:2048\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(ar[0]), "=&v"(ar[1]), "=&v"(ar[2]), "=&v"(ar[3]), "=&v"(br[0]), "=&v"(br[1])
                : "v"(xa), "v"(wa)
                : "memory");
        };
        fetch(0, a[0], bb[0]);
        fetch(1, a[1], bb[1]);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = DenseMfma<S>::mma(__builtin_bit_cast(uint4, a[st][i]), __builtin_bit_cast(uint4, bb[st][j]),
                                                  acc[i][j]);
    };

    // fold slot sl's partial into the pairwise sum (uniform branches)
    auto fold = [&](int sl) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x4 p = acc[i][j];
                if (sl == 0) {
                    S0[i][j] = p;
                } else if (sl == 1) {
                    S0[i][j] = S0[i][j] + p;
                } else if (sl == 2 || sl == 4) {
                    S1[i][j] = p;
                } else if (sl == 3) {
                    S1[i][j] = S1[i][j] + p;
                    S0[i][j] = S0[i][j] + S1[i][j];
                } else if (sl == 5) {
                    S1[i][j] = S1[i][j] + p;
                } else if (sl == 6) {
                    S2[i][j] = p;
                } else {
                    S2[i][j] = S2[i][j] + p;
                    S1[i][j] = S1[i][j] + S2[i][j];
                    S0[i][j] = S0[i][j] + S1[i][j];
                }
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
    };
    // Stage u of the slot-major walk (every slot has a block: nb >= 8): wait
    // for its operands (the two stages after it stay in flight), start stage
    // u + 3 in the buffer stage u - 1 used, multiply, and after the second
    // half of a slot's last block fold the slot.
    const int split_i = r * (q + 1);               // items of the slots with q + 1 blocks
    const int nst = 2 * nb;
    auto step = [&](const Stage &cur, Stage &nxt, int u) {
        if (u + 2 < nst) __builtin_amdgcn_s_waitcnt(0x0F78);        // vmcnt(8): stages u + 1, u + 2 in flight
        else if (u + 1 < nst) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
        else __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0)
        // Everyone's loads of stage u have landed (each wave waited for its
        // own above: a direct-to-LDS load counts as done once its data is in
        // LDS) and nobody reads nxt any more.  A bare barrier: a fenced one
        // (__syncthreads) would also wait for the stages still streaming in;
        // the memory clobber keeps every LDS access on its side of it.
        asm volatile("s_barrier" ::: "memory");
        if (u + 3 < nst) stage(nxt, u + 3);
        multiply(cur);
        if (u & 1) {
            const int e = (u >> 1) + 1;            // slot boundaries: multiples of q + 1, then of q
            const bool last = e <= split_i ? e % (q + 1) == 0 : (e - split_i) % q == 0;
            if (last) fold(e <= split_i ? e / (q + 1) - 1 : r + (e - split_i) / q - 1);
        }
    };
    stage(lds0, 0);
    stage(lds1, 1);
    stage(lds2, 2);
    for (int u = 0; u < nst; u += 4) {
        step(lds0, lds3, u);
        step(lds1, lds0, u + 1);
        if (u + 2 < nst) step(lds2, lds1, u + 2);
        if (u + 3 < nst) step(lds3, lds2, u + 3);
    }

    // MFMA accumulator layout: lane (g, c), register e holds row 4 g + e, column c.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = tn * kTileCols + wn * 32 + j * 16 + c;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = tm * kTileRows + wm * 64 + i * 16 + g * 4 + e;
                if (row < M) y[(int64_t)row * N + col] = S::narrow(S0[i][j][e]);
            }
        }
}

// Launch for M > 64 (the caller checks dtype, K % 128 == 0, 16-byte
// alignment of x and W, and M, N, K < 2^31).
template <typename S>
void launch_dense_tile(const void *x, const void *w, void *y, int64_t M, int64_t N, int64_t K, bool packed,
                       hipStream_t st)
{
    const int ntm = (int)cdiv(M, kTileRows), ntn = (int)cdiv(N, kTileCols);
    const int per_xcd = (int)cdiv((int64_t)ntm * ntn, 8);
    const dim3 grid((unsigned)(8 * per_xcd)), block(kTileWaves * kWave);
    if (packed)
        launch_kernel((dense_tile_kernel<S, true>), grid, block, 0, st, (const uint16_t *)x, (const uint16_t *)w,
                      (uint16_t *)y, (int)M, (int)N, (int)K, ntm, ntn, per_xcd);
    else
        launch_kernel((dense_tile_kernel<S, false>), grid, block, 0, st, (const uint16_t *)x, (const uint16_t *)w,
                      (uint16_t *)y, (int)M, (int)N, (int)K, ntm, ntn, per_xcd);
}

template void launch_dense_tile<BF16>(const void *, const void *, void *, int64_t, int64_t, int64_t, bool,
                                      hipStream_t);
template void launch_dense_tile<F16>(const void *, const void *, void *, int64_t, int64_t, int64_t, bool,
                                     hipStream_t);

}  // namespace bi
