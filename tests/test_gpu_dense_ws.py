"""Dense matmul with a workspace (bi_matmul_ws): the same bits as bi_matmul.

bi_matmul_ws spreads the eight K slots of a short-M product over several
workgroups and meets their partial sums in a workspace; the tree of every
output is bi_matmul's, so the two must agree bit for bit on every shape,
including those where the slot groups, the column tiles or the rows are
ragged, where some slot groups own no block of K at all (K < 8 blocks), and
where the call falls back to bi_matmul's kernels.  Workload shapes: the
decoder's projections at decode batch sizes (hidden 4096, SwiGLU 14336,
vocab 32000) -- "Fix/speculative shape invariance" (Problem: one row and a
short block must reduce alike) and "Batch-invariant kernels ..." (Case 6)."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f16": torch.float16}


def rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(TD[dtype]).to(dev())


def same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [
    (1, 96, 128),          # M <= 16: bi_matmul's kernels
    (9, 28672, 512),       # 8 < M <= 16 on a wide weight: the slot form with one 16-row tile
    (13, 6144, 4096),      # ... on a narrow one: four row tiles (padding rows never stored)
    (12, 6144, 4096),      # ... but not here: bi_matmul's kernels
    (17, 96, 128),         # one block: slots 1..7 own nothing
    (23, 1000, 896),       # 7 blocks, ragged column tile
    (16, 4096, 4096),
    (17, 6144, 4096),      # four row tiles, 17 rows
    (33, 4096, 14336),     # the down projection, 112 blocks
    (64, 4096, 4096),
    (64, 1000, 4224),      # 33 blocks: uneven slots
    (64, 6144, 4096),      # 96-column tiles: 256 workgroups instead of 384
    (64, 6000, 4096),      # ... the last tile ragged (48 columns)
    (40, 5008, 1024),      # ... the last tile one wave wide
    (32, 32768, 1024),     # enough column tiles for all eight slots in one workgroup
    (64, 32768, 1024),
    (64, 28656, 256),      # 7-wave (112-column) tiles fill 256 CUs; last tile ragged
    (20, 28656, 384),
    (65, 512, 4096),       # past 64 rows: 64-row chunks, each with its own group sums
    (80, 6144, 4096),      # a verify block of 16 sequences on the QKV projection
    (80, 4096, 14336),     # ... on the down projection
    (128, 4096, 4096),     # the most rows the form with an exchange takes
    (100, 1000, 896),      # ragged chunk, ragged column tile
    (129, 4096, 4096),     # past that: bi_matmul's kernels
    (320, 6144, 4096),     # a verify block of 64 sequences
    (64, 512, 4100),       # K not a multiple of 128: bi_matmul's kernels
])
def test_bits_equal_plain_matmul(dtype, M, N, K):
    x = rand((M, K), dtype, seed=M * 7 + K)
    w = rand((N, K), dtype, seed=N * 3 + K, scale=0.02)
    ws = bi.matmul_workspace(M, N, K, TD[dtype], device=dev())
    y = bi.matmul_ws(x, w, ws)
    assert same(y, bi.matmul(x, w)), f"{M}x{N}x{K}"


def test_decoder_shapes_and_every_m():
    """Every M in 1..64 at the decoder's projection shapes: rows equal the
    plain kernel's and the M = 1 result."""
    K = 4096
    for N in (6144, 4096, 28672, 32000):
        w = rand((N, K), "bf16", seed=N, scale=0.02)
        x = rand((64, K), "bf16", seed=N + 1)
        ws = bi.matmul_workspace(64, N, K, device=dev())
        full = bi.matmul(x, w)
        for M in (1, 2, 5, 9, 12, 13, 16, 17, 31, 32, 33, 48, 63, 64):
            assert same(bi.matmul_ws(x[:M].contiguous(), w, ws), full[:M]), f"N={N} M={M}"
        assert same(bi.matmul_ws(x[40:41].contiguous(), w, ws), full[40:41])
    w = rand((4096, 14336), "bf16", seed=5, scale=0.02)
    x = rand((64, 14336), "bf16", seed=6)
    ws = bi.matmul_workspace(64, 4096, 14336, device=dev())
    full = bi.matmul(x, w)
    for M in (1, 8, 64):
        assert same(bi.matmul_ws(x[:M].contiguous(), w, ws), full[:M]), f"down M={M}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,N,K", [(64, 1000, 4224), (25, 300, 1024), (64, 128, 256)])
def test_oracle_parity(dtype, M, N, K):
    x, wt, _ = inputs.dense_case(M, N, K, dtype, seed=M + N + K)
    ws = bi.matmul_workspace(M, N, K, TD[dtype], device=dev())
    y = to_np(bi.matmul_ws(to_dev(x, dtype), to_dev(wt, dtype), ws))
    assert_parity(y, oracle.matmul(x, wt, dtype, True), dtype, f"{M}x{N}x{K}")


def test_workspace_reuse_leaves_counters_zero():
    """One workspace across calls of different shapes in stream order: every
    result is right and the counter area is zero after each call."""
    L = bi.lib()
    need = max(L.bi_matmul_ws_workspace_bytes(*sh, 0, 1) for sh in ((64, 32000, 4096), (128, 6144, 4096)))
    big = torch.zeros(need, dtype=torch.uint8, device=dev())
    for (M, N, K) in ((64, 32000, 4096), (64, 4096, 4096), (7, 4096, 14336), (64, 1000, 4224), (1, 96, 128),
                      (128, 6144, 4096), (80, 4096, 14336), (64, 32000, 4096), (64, 4096, 4096), (100, 4096, 4096),
                      (64, 28672, 4096), (1, 32000, 4096)):
        x = rand((M, K), "bf16", seed=M + N)
        w = rand((N, K), "bf16", seed=N + K, scale=0.02)
        y = bi.matmul_ws(x, w, big)
        assert same(y, bi.matmul(x, w)), f"{M}x{N}x{K}"
        assert int(big[:65536].count_nonzero()) == 0
    assert L.bi_matmul_ws_workspace_bytes(64, 4096, 4096, 0, 1) <= big.numel()


def test_bounded_stores():
    """Output surrounded by canaries at a ragged column count."""
    M, N, K = 37, 1000, 1152
    x, wt, _ = inputs.dense_case(M, N, K, "bf16", seed=11)
    ws = bi.matmul_workspace(M, N, K, device=dev())
    yg = Guarded((M, N), torch.bfloat16, poison=0xA5)
    bi.matmul_ws(to_dev(x, "bf16"), to_dev(wt, "bf16"), ws, out=yg.view)
    torch.cuda.synchronize()
    assert yg.canaries_intact()
    assert_parity(to_np(yg.view), oracle.matmul(x, wt, "bf16", True), "bf16")


def test_run_to_run_determinism():
    x = rand((64, 4096), "bf16", seed=1)
    w = rand((4096, 4096), "bf16", seed=2, scale=0.02)
    ws = bi.matmul_workspace(64, 4096, 4096, device=dev())
    first = bi.matmul_ws(x, w, ws)
    for _ in range(50):
        assert same(bi.matmul_ws(x, w, ws), first)


@pytest.mark.parametrize("M,F,K", [
    (1, 14336, 4096),      # decode rows on the one-workgroup-per-tile kernel: fallback (product + activation)
    (16, 64, 128),
    (17, 14336, 4096),     # the fused slot kernel, 32-row form
    (40, 192, 896),        # few column tiles: slot groups exchange partial sums
    (64, 14336, 4096),     # the decoder's MLP at batch 64
    (64, 3072, 4096),      # 96-column tiles
    (40, 2504, 1024),      # 96-column tiles, the last one wave wide
    (64, 640, 4224),
    (17, 14328, 256),      # 7-wave tiles, last tile ragged
    (33, 200, 512),        # F not a multiple of 64: 8-row interleave blocks across tiles
    (65, 14336, 4096),     # long M: fallback
    (64, 128, 4100),       # K not a multiple of 128: fallback
])
def test_swiglu_bits_equal_matmul_then_silu(M, F, K):
    """Fused gate/up + SwiGLU equals bi_matmul followed by bi_silu_mul bit
    for bit, whichever form the call takes."""
    x = rand((M, K), "bf16", seed=M + F)
    wg = rand((F, K), "bf16", seed=F + K, scale=0.02)
    wu = rand((F, K), "bf16", seed=F + K + 1, scale=0.02)
    ref = bi.silu_mul(bi.matmul(x, torch.cat([wg, wu], 0).contiguous()))
    ws = bi.matmul_swiglu_workspace(M, F, K, device=dev())
    a = bi.matmul_swiglu(x, bi.interleave_gate_up(wg, wu), ws)
    assert same(a, ref), f"{M}x{F}x{K}"
    assert int(ws[:65536].count_nonzero()) == 0          # counters left zero by either form


def test_swiglu_rows_independent_and_canaries():
    """Every prefix of the rows gives the full call's rows, with one workspace
    shared by both forms of the call in stream order; stores stay in the
    output."""
    F, K = 1024, 4096
    x = rand((64, K), "bf16", seed=3)
    wil = bi.interleave_gate_up(rand((F, K), "bf16", seed=4, scale=0.02), rand((F, K), "bf16", seed=5, scale=0.02))
    ws = bi.matmul_swiglu_workspace(64, F, K, device=dev())
    full = bi.matmul_swiglu(x, wil, ws)
    for M in (1, 9, 16, 17, 33, 63, 2, 40):
        assert same(bi.matmul_swiglu(x[:M].contiguous(), wil, ws), full[:M]), f"M={M}"
    ag = Guarded((37, F), torch.bfloat16, poison=0x5A)
    bi.matmul_swiglu(x[:37].contiguous(), wil, ws, out=ag.view)
    torch.cuda.synchronize()
    assert ag.canaries_intact()
    assert same(ag.view, full[:37])


def test_swiglu_oracle_parity():
    """Against the oracle's matmul (rounded to bf16, as the decoder stores
    it) then SiLU*mul, to the bf16 parity tolerance."""
    M, F, K = 48, 320, 1024
    x, wt, _ = inputs.dense_case(M, 2 * F, K, "bf16", seed=21)
    gu = oracle.round_to(oracle.matmul(x, wt, "bf16", True), "bf16")
    ref = oracle.silu_mul(gu[:, :F].copy(), gu[:, F:].copy(), "bf16")
    w = to_dev(wt, "bf16")
    ws = bi.matmul_swiglu_workspace(M, F, K, device=dev())
    a = to_np(bi.matmul_swiglu(to_dev(x, "bf16"), bi.interleave_gate_up(w[:F], w[F:]), ws))
    assert_parity(a, ref, "bf16", "swiglu")


# ---------------------------------------------------------------------------
# tile-packed weights: same bits as [N, K] in every dense path
# ---------------------------------------------------------------------------

def test_pack_layout_matches_definition():
    """Every element lands where the header's formula puts it; rows past N
    are zero."""
    N, K = 37, 384
    w = torch.arange(N * K, dtype=torch.int32).remainder(30011).to(torch.int16).view(N, K)
    wp = bi.pack_weights(w.view(torch.bfloat16).to(dev())).data.view(torch.int16).cpu().numpy()
    nb, nrg = K // 128, (N + 15) // 16
    assert wp.size == nrg * 16 * K
    ref = np.zeros(nrg * 16 * K, np.int16)
    wn = w.numpy()
    for r in range(nrg):
        for b in range(nb):
            for s in range(4):
                for lane in range(64):
                    g, c = lane >> 4, lane & 15
                    row = 16 * r + c
                    off = (((r * nb + b) * 4 + s) * 64 + lane) * 8
                    if row < N:
                        ref[off:off + 8] = wn[row, 128 * b + 32 * s + 8 * g:128 * b + 32 * s + 8 * g + 8]
    assert np.array_equal(wp, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,K", [(96, 128), (1000, 896), (4096, 4096), (28656, 256), (6144, 4096)])
def test_packed_bits_equal(dtype, N, K):
    """bi_matmul and bi_matmul_ws on the packed weight give the [N, K]
    weight's bits for every M form: the streaming kernel (M <= 16), the slot
    form (16 < M <= 64) and the tiled kernel (M > 64)."""
    w = rand((N, K), dtype, seed=N + K, scale=0.02)
    wp = bi.pack_weights(w)
    x = rand((96, K), dtype, seed=K + 1)
    ws = bi.matmul_workspace(64, N, K, TD[dtype], device=dev())
    full = bi.matmul(x, w)
    assert same(bi.matmul(x, wp), full), "M=96 tiled"
    for M in (1, 5, 16, 17, 40, 64):
        xm = x[:M].contiguous()
        assert same(bi.matmul(xm, wp), full[:M]), f"matmul M={M}"
        assert same(bi.matmul_ws(xm, wp, ws), full[:M]), f"matmul_ws M={M}"
    assert int(ws[:65536].count_nonzero()) == 0


def test_packed_swiglu_and_split_variant():
    F, K = 1024, 512
    wg = rand((F, K), "bf16", seed=7, scale=0.02)
    wu = rand((F, K), "bf16", seed=8, scale=0.02)
    wil = bi.interleave_gate_up(wg, wu)
    wilp = bi.pack_weights(wil)
    ws = bi.matmul_swiglu_workspace(70, F, K, device=dev())       # sized for the most rows of the calls below
    for M in (1, 17, 64, 70):
        x = rand((M, K), "bf16", seed=M)
        assert same(bi.matmul_swiglu(x, wilp, ws), bi.matmul_swiglu(x, wil, ws)), f"M={M}"
    # the comparison variant reads packed weights too (same bits as on [N, K])
    x = rand((8, K), "bf16", seed=3)
    for s in (1, 2, 4):
        assert same(bi.matmul_split(x, wilp, s), bi.matmul_split(x, wil, s)), f"splits={s}"
