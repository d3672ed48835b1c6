"""A seeded random campaign over the quantized matmul's legal space, in the
spirit of the randomized differential campaign of "Fix fp quantized matmul
corruption when the quantized dim is not a multiple of 32" (Validation:
affine 2 to 8 bits at gs 32/64/128, mxfp4, mxfp8, nvfp4, both transposes,
plain and gather): every case is checked against the oracle, and one row of
each against the same row computed alone (bitwise).

Workload: per case, mode / width / group size / layout / M / K / N drawn from
a fixed-seed generator (the quantized dimension a multiple of the group size,
the packed layout only where K % 128 == 0); W ~ N(0,1) quantized host-side,
x ~ N(0,1) binary16; gather cases draw E experts and top-k routing."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

QM = {"affine": bi.AFFINE, "nvfp4": bi.NVFP4, "mxfp4": bi.MXFP4, "mxfp8": bi.MXFP8}
OQM = {"affine": oracle.AFFINE, "nvfp4": oracle.NVFP4, "mxfp4": oracle.MXFP4, "mxfp8": oracle.MXFP8}


def draw_case(rng):
    mode = ["affine", "affine", "affine", "nvfp4", "mxfp4", "mxfp8"][rng.integers(6)]
    if mode == "affine":
        bits, gs = int(rng.integers(2, 9)), int(rng.choice([32, 64, 128]))
    else:
        bits, gs = (8, 32) if mode == "mxfp8" else (4, 16 if mode == "nvfp4" else 32)
    layout = ["transposed", "natural", "packed"][rng.integers(3)]
    M = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 17, 33, 64, 70]))
    if layout == "packed":
        K = 128 * int(rng.integers(1, 10))
        N = int(rng.integers(1, 300))
    elif layout == "transposed":
        K = gs * int(rng.integers(1, 1200 // gs + 1))
        N = int(rng.integers(1, 300))
    else:
        K = int(rng.integers(1, 1200))
        N = gs * int(rng.integers(1, 300 // gs + 1))
    return mode, bits, gs, layout, M, K, N


CASES = [draw_case(np.random.default_rng(1000 + i)) for i in range(200)]


def dev_q(wq, s, b):
    wqd = torch.from_numpy(np.ascontiguousarray(wq).view(np.int32)).to(dev())
    sd = torch.from_numpy(np.ascontiguousarray(s) if s.dtype == np.uint8
                          else np.ascontiguousarray(s).view(np.int16)).to(dev())
    bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev())
    return wqd, sd, bd


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_random_qmatmul_case(case):
    mode, bits, gs, layout, M, K, N = case
    transposed = layout != "natural"
    x, wq, s, b = inputs.qmatmul_case(M, K, N, mode, gs, transposed, seed=M * 7 + K + N, bits=bits)
    wqd, sd, bd = dev_q(wq, s, b)
    if layout == "packed":
        wqd = bi.pack_qweights(wqd, sd, bd, N, K, QM[mode], gs, bits=bits)
        sd = bd = None
    xd = to_dev(x, "f16")
    call = lambda xm: to_np(bi.qmatmul(xm, wqd, sd, bd, N, K, QM[mode], gs, transposed, packed=layout == "packed",
                                       bits=bits))
    y = call(xd)
    assert_parity(y, oracle.qmatmul(x, wq, s, b, M, N, K, OQM[mode], gs, transposed, bits=bits), "f16")
    i = M - 1
    assert bits_equal(call(xd[i:i + 1].contiguous()), y[i:i + 1])


GATHER_CASES = []
for i in range(60):
    rng = np.random.default_rng(5000 + i)
    mode, bits, gs, layout, _, K, N = draw_case(rng)
    T, E = int(rng.integers(1, 20)), int(rng.integers(1, 9))
    topk = int(rng.integers(1, E + 1))
    GATHER_CASES.append((mode, bits, gs, layout, T, topk, E, K, N, bool(rng.integers(2))))


@pytest.mark.parametrize("case", GATHER_CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_random_gather_case(case):
    mode, bits, gs, layout, T, topk, E, K, N, sort_rows = case
    transposed = layout != "natural"
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, mode, gs, transposed, sort_rows, seed=T + K + N,
                                               bits=bits)
    wqd, sd, bd = dev_q(wq, s, b)
    packed = layout == "packed"
    if packed:
        wqd = torch.stack([bi.pack_qweights(wqd[e], sd[e], None if bd is None else bd[e], N, K, QM[mode], gs, bits=bits)
                           for e in range(E)])
        sd = bd = None
    xd = to_dev(x, "f16")
    li = torch.from_numpy(lhs).to(dev())
    ri = torch.from_numpy(rhs).to(dev())
    y = to_np(bi.gather_qmatmul(xd, li, ri, wqd, sd, bd, N, K, QM[mode], gs, transposed, packed=packed, bits=bits))
    assert_parity(y, oracle.gather_qmatmul(x, lhs, rhs, wq, s, b, N, K, OQM[mode], gs, transposed, bits=bits), "f16")
    m = rhs.size - 1
    one = to_np(bi.gather_qmatmul(xd, li[m:m + 1].contiguous(), ri[m:m + 1].contiguous(), wqd, sd, bd, N, K,
                                  QM[mode], gs, transposed, packed=packed, bits=bits))
    assert bits_equal(one, y[m:m + 1])
