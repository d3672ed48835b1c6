"""Expert ("gather") quantized matmul of a mixture-of-experts layer on the GPU:
parity with the oracle, and invariance under routing -- every row has the bits
of the plain quantized matmul of its token with its expert, whatever the
other rows, their order (sorted or not) or their number.

Workload: E expert matrices W_e ~ N(0,1) quantized per group (affine gs 32/64
with fp16 scale and bias, nvfp4, mxfp4), x [T, K] ~ N(0,1) fp16, each token
routed to top-k distinct experts drawn uniformly; rows ordered by token
(unsorted) or by expert (sorted).  Shapes: the pages' sorted gather (T = 64
rows, K = 1040, nvfp4) and unsorted gather (M = 50, K = 1040) from "Fix fp
quantized matmul corruption when the quantized dim is not a multiple of 32"
(Validation), a decode-sized MoE step (8 tokens, top-2 of 8 experts, K =
4096) and a natural-layout case."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

QM = {"affine": bi.AFFINE, "nvfp4": bi.NVFP4, "mxfp4": bi.MXFP4}
OQM = {"affine": oracle.AFFINE, "nvfp4": oracle.NVFP4, "mxfp4": oracle.MXFP4}


def dev_w(wq, s, b):
    wqd = torch.from_numpy(np.ascontiguousarray(wq).view(np.int32)).to(dev())
    sd = torch.from_numpy(np.ascontiguousarray(s) if s.dtype == np.uint8
                          else np.ascontiguousarray(s).view(np.int16)).to(dev())
    bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev())
    return wqd, sd, bd


def idx(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def gather(x, lhs, rhs, w, N, K, mode, gs, transposed):
    wqd, sd, bd = w
    return to_np(bi.gather_qmatmul(to_dev(x, "f16") if isinstance(x, np.ndarray) else x, idx(lhs), idx(rhs), wqd, sd,
                                   bd, N, K, QM[mode], gs, transposed))


CASES = [
    # mode, gs, T, topk, E, K, N, transposed, sorted
    ("nvfp4", 16, 32, 2, 8, 1040, 128, True, True),       # sorted gather, 64 rows, K % 32 == 16
    ("nvfp4", 16, 25, 2, 8, 1040, 128, True, False),      # unsorted gather, 50 rows
    ("affine", 64, 8, 2, 8, 4096, 512, True, False),      # decode-sized MoE step (streaming form, M <= 16)
    ("nvfp4", 16, 6, 2, 8, 2048, 8192, True, True),       # streaming form, two column groups per tile
    ("mxfp4", 32, 16, 4, 16, 2048, 256, True, True),
    ("affine", 32, 12, 2, 4, 512, 96, False, False),      # natural layout
    ("nvfp4", 16, 10, 2, 4, 1040, 64, False, True),
]


@pytest.mark.parametrize("mode,gs,T,topk,E,K,N,transposed,sort_rows", CASES)
def test_gather_matches_oracle_and_plain_rows(mode, gs, T, topk, E, K, N, transposed, sort_rows):
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, transposed, sort_rows, seed=T + K)
    w = dev_w(wq, s, b)
    y = gather(x, lhs, rhs, w, N, K, mode, gs, transposed)
    assert_parity(y, oracle.gather_qmatmul(x, lhs, rhs, wq, s, b, N, K, OQM[mode], gs, transposed), "f16")
    # each row: the plain quantized matmul of its token with its expert (M = 1), bit for bit
    xd = to_dev(x, "f16")
    for m in range(0, rhs.size, max(1, rhs.size // 9)):
        e = int(rhs[m])
        wqe, se, be = w[0][e], w[1][e], None if w[2] is None else w[2][e]
        one = to_np(bi.qmatmul(xd[lhs[m]:lhs[m] + 1].contiguous(), wqe, se, be, N, K, QM[mode], gs, transposed))
        assert bits_equal(y[m:m + 1], one), f"row {m} (expert {e})"


@pytest.mark.parametrize("transposed", [True, False])
def test_gather_invariant_under_order_and_batch(transposed):
    """Sorting the rows, shuffling them or taking a subset changes no row's
    bits; lhs = NULL reads x[m]."""
    mode, gs, T, topk, E, K, N = "affine", 64, 20, 2, 6, 1024, 128
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, transposed, False, seed=7)
    w = dev_w(wq, s, b)
    y = gather(x, lhs, rhs, w, N, K, mode, gs, transposed)
    order = np.argsort(rhs, kind="stable")
    assert bits_equal(gather(x, lhs[order], rhs[order], w, N, K, mode, gs, transposed), y[order])
    perm = np.random.default_rng(1).permutation(rhs.size)
    assert bits_equal(gather(x, lhs[perm], rhs[perm], w, N, K, mode, gs, transposed), y[perm])
    sub = np.arange(3, 17)
    assert bits_equal(gather(x, lhs[sub], rhs[sub], w, N, K, mode, gs, transposed), y[sub])
    xr = x[lhs]                                                    # materialised rows: lhs = NULL
    assert bits_equal(gather(xr, None, rhs, w, N, K, mode, gs, transposed), y)


def test_gather_more_rows_than_one_slab():
    """M = 5000 rows (two slabs of the in-workgroup bucketing) over 3
    experts: parity, and rows equal to the same rows gathered alone."""
    mode, gs, T, topk, E, K, N = "mxfp4", 32, 2500, 2, 3, 256, 48
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, True, False, seed=9)
    w = dev_w(wq, s, b)
    y = gather(x, lhs, rhs, w, N, K, mode, gs, True)
    assert_parity(y, oracle.gather_qmatmul(x, lhs, rhs, wq, s, b, N, K, OQM[mode], gs, True), "f16")
    pick = np.array([0, 1, 4095, 4096, 4999])
    assert bits_equal(gather(x, lhs[pick], rhs[pick], w, N, K, mode, gs, True), y[pick])


@pytest.mark.parametrize("K", [1040, 1024])
def test_gather_out_of_range_rows_are_nan_and_fenced(K):
    """Rows with a bad expert or token index are NaN; the others keep their
    bits; nothing is written outside y (K = 1024: the streaming form)."""
    mode, gs, T, topk, E, N = "nvfp4", 16, 6, 2, 4, 80
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, True, False, seed=3)
    w = dev_w(wq, s, b)
    y = gather(x, lhs, rhs, w, N, K, mode, gs, True)
    bad_r, bad_l = rhs.copy(), lhs.copy()
    bad_r[2], bad_r[5], bad_l[7] = E, -1, T
    M = rhs.size
    yg = Guarded((M, N), torch.float16, poison=0x99)
    wqd, sd, bd = w
    bi.gather_qmatmul(to_dev(x, "f16"), idx(bad_l), idx(bad_r), wqd, sd, bd, N, K, QM[mode], gs, True, out=yg.view)
    torch.cuda.synchronize()
    assert yg.canaries_intact()
    g = inputs.from_storage(to_np(yg.view), "f16")
    bad = np.zeros(M, bool)
    bad[[2, 5, 7]] = True
    assert np.all(np.isnan(g[bad]))
    assert bits_equal(to_np(yg.view)[~bad], y[~bad])


def test_gather_every_row_bad_is_all_nan():
    mode, gs, T, topk, E, K, N = "affine", 32, 4, 2, 3, 512, 64
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, True, False, seed=8)
    w = dev_w(wq, s, b)
    y = gather(x, lhs, np.full_like(rhs, E), w, N, K, mode, gs, True)
    assert np.all(np.isnan(inputs.from_storage(y, "f16")))


def test_gather_200_runs_one_result():
    mode, gs, T, topk, E, K, N = "nvfp4", 16, 25, 2, 8, 1040, 128
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, True, False, seed=5)
    wqd, sd, bd = dev_w(wq, s, b)
    xd, ld, rd = to_dev(x, "f16"), idx(lhs), idx(rhs)
    first = bi.gather_qmatmul(xd, ld, rd, wqd, sd, bd, N, K, QM[mode], gs, True)
    outs = [bi.gather_qmatmul(xd, ld, rd, wqd, sd, bd, N, K, QM[mode], gs, True) for _ in range(200)]
    assert all(torch.equal(o.view(torch.int16), first.view(torch.int16)) for o in outs)


@pytest.mark.parametrize("mode,gs,T,topk,E,K,N", [
    ("affine", 64, 8, 2, 8, 1024, 512),       # streaming form (16 rows)
    ("nvfp4", 16, 6, 2, 8, 1024, 8192),       # streaming form, two column groups per tile
    ("mxfp4", 32, 20, 2, 4, 512, 200),        # tiled form (40 rows), padded last row group
])
def test_gather_packed_bits_equal_transposed(mode, gs, T, topk, E, K, N):
    """Experts packed one by one with pack_qweights and stacked give the
    transposed gather's bits."""
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, True, False, seed=T + N)
    wqd, sd, bd = dev_w(wq, s, b)
    wp = torch.stack([bi.pack_qweights(wqd[e], sd[e], None if bd is None else bd[e], N, K, QM[mode], gs)
                      for e in range(E)])
    y = gather(x, lhs, rhs, (wqd, sd, bd), N, K, mode, gs, True)
    yp = to_np(bi.gather_qmatmul(to_dev(x, "f16"), idx(lhs), idx(rhs), wp, None, None, N, K, QM[mode], gs,
                                 packed=True))
    assert bits_equal(yp, y)


@pytest.mark.parametrize("mode,gs,bits", [("affine", 64, 3), ("affine", 32, 8), ("mxfp8", 32, 8), ("affine", 128, 6)])
@pytest.mark.parametrize("layout", ["transposed", "natural", "packed"])
def test_gather_other_widths(mode, gs, bits, layout):
    """Affine codes of 2 to 8 bits and mxfp8: parity with the oracle, and
    every row the plain quantized matmul of its token with its expert (the
    packed experts: the transposed call's bits)."""
    T, topk, E, K, N = 10, 2, 4, 512 if layout != "natural" else 520, 128
    transposed = layout != "natural"
    qm = {"affine": bi.AFFINE, "mxfp8": bi.MXFP8}[mode]
    oqm = {"affine": oracle.AFFINE, "mxfp8": oracle.MXFP8}[mode]
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, transposed, False, seed=bits, bits=bits)
    wqd, sd, bd = dev_w(wq, s, b)
    xd = to_dev(x, "f16")
    if layout == "packed":
        wp = torch.stack([bi.pack_qweights(wqd[e], sd[e], None if bd is None else bd[e], N, K, qm, gs, bits=bits)
                          for e in range(E)])
        y = to_np(bi.gather_qmatmul(xd, idx(lhs), idx(rhs), wp, None, None, N, K, qm, gs, packed=True, bits=bits))
    else:
        y = to_np(bi.gather_qmatmul(xd, idx(lhs), idx(rhs), wqd, sd, bd, N, K, qm, gs, transposed, bits=bits))
    assert_parity(y, oracle.gather_qmatmul(x, lhs, rhs, wq, s, b, N, K, oqm, gs, transposed, bits=bits), "f16")
    for m in (0, 7, 19):
        e = int(rhs[m])
        one = to_np(bi.qmatmul(xd[lhs[m]:lhs[m] + 1].contiguous(), wqd[e], sd[e], None if bd is None else bd[e], N, K,
                               qm, gs, transposed, bits=bits))
        assert bits_equal(y[m:m + 1], one), f"row {m} (expert {e})"
