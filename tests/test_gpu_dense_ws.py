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
    (17, 96, 128),         # one block: slots 1..7 own nothing
    (23, 1000, 896),       # 7 blocks, ragged column tile
    (16, 4096, 4096),
    (17, 6144, 4096),      # two row tiles of the 32-row form
    (33, 4096, 14336),     # the down projection, 112 blocks
    (64, 4096, 4096),
    (64, 1000, 4224),      # 33 blocks: uneven slots
    (64, 6144, 4096),
    (32, 32768, 1024),     # enough column tiles for all eight slots in one workgroup
    (64, 32768, 1024),
    (65, 512, 4096),       # long M: bi_matmul's kernels
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
        for M in (1, 2, 5, 16, 17, 31, 32, 33, 48, 63, 64):
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
    big = bi.matmul_workspace(64, 32000, 4096, device=dev())
    L = bi.lib()
    for (M, N, K) in ((64, 32000, 4096), (64, 4096, 4096), (7, 4096, 14336), (64, 1000, 4224), (1, 96, 128),
                      (64, 32000, 4096), (64, 4096, 4096), (64, 28672, 4096), (1, 32000, 4096)):
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
