"""RMSNorm on the GPU: parity with the oracle and bitwise invariance over B.

Workload: x [B, 4096] bf16 ~ N(0,1)*3, w = 1 + 0.1*N(0,1), B in
{1, 8, 64, 512, 4096}, eps 1e-6 -- the reduction of "Batch-invariant kernels:
why temperature-0 decoding is still nondeterministic", Case 4 and Case 6."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu


def test_config_rows_identical_across_batch_sizes():
    x, w = inputs.rmsnorm_case(4096, 4096, seed=0)
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    full = to_np(bi.rmsnorm(xd, wd, 1e-6))
    assert_parity(full, oracle.rmsnorm(x, w, "bf16", 1e-6), "bf16", "B=4096")
    for B in (1, 8, 64, 512):
        y = to_np(bi.rmsnorm(xd[:B].contiguous(), wd, 1e-6))
        assert bits_equal(y, full[:B]), f"B={B}"
    for off in (1, 3, 1000):
        y = to_np(bi.rmsnorm(xd[off:off + 64].contiguous(), wd, 1e-6))
        assert bits_equal(y, full[off:off + 64])


def test_case4_row_on_the_gpu():
    """The chapter's Case 4 row (2^-(i//64), weight 1) in f32: the GPU's tree
    gives a sum of squares within the fp32 bound of the exact 85.333..., and the
    output is within the f32 tolerance of the oracle."""
    H = 4096
    row = np.array([2.0 ** -(i // 64) for i in range(H)], np.float32)
    x = np.stack([row, row[::-1].copy()])
    w = np.ones(H, np.float32)
    y = to_np(bi.rmsnorm(to_dev(x, "f32"), to_dev(w, "f32"), 1e-6))
    assert_parity(y, oracle.rmsnorm(x, w, "f32", 1e-6), "f32")


def test_integer_rows_bit_exact_vs_oracle():
    """Small integers: the sum of squares is exact in any order, so the GPU and
    the oracle apply the same IEEE ops to the same value -> same bits."""
    rng = np.random.default_rng(1)
    for dtype in ("bf16", "f16", "f32"):
        x = inputs.integer_values(rng, (64, 4096), -3, 3, dtype)
        w = inputs.normal(rng, (4096,), 0.1, loc=1.0, dtype=dtype)
        ref = oracle.round_to(oracle.rmsnorm(x, w, dtype, 1e-6), dtype)
        assert bits_equal(to_np(bi.rmsnorm(to_dev(x, dtype), to_dev(w, dtype), 1e-6)), ref), dtype


@pytest.mark.parametrize("dtype", inputs.DTYPES)
@pytest.mark.parametrize("rows,H", [(1, 1), (3, 7), (5, 100), (9, 4100), (2, 8192), (3, 16384), (2, 20000),
                                    (7, 4095)])
def test_ragged_shapes(dtype, rows, H):
    x, w = inputs.rmsnorm_case(rows, H, seed=H, dtype=dtype)
    xd, wd = to_dev(x, dtype), to_dev(w, dtype)
    y = to_np(bi.rmsnorm(xd, wd, 1e-6))
    assert_parity(y, oracle.rmsnorm(x, w, dtype, 1e-6), dtype, f"{rows}x{H}")
    assert bits_equal(to_np(bi.rmsnorm(xd[-1:].contiguous(), wd, 1e-6)), y[-1:])


def test_bounded_loads_and_stores():
    rows, H = 13, 4100
    x, w = inputs.rmsnorm_case(rows, H, seed=3)
    xg = Guarded((rows, H), torch.bfloat16, init=to_dev(x, "bf16"))
    wg = Guarded((H,), torch.bfloat16, init=to_dev(w, "bf16"))
    yg = Guarded((rows, H), torch.bfloat16, poison=0x5A)
    bi.rmsnorm(xg.view, wg.view, 1e-6, out=yg.view)
    torch.cuda.synchronize()
    assert yg.canaries_intact()
    assert_parity(to_np(yg.view), oracle.rmsnorm(x, w, "bf16", 1e-6), "bf16")


def test_split_variant_is_correct_but_not_invariant():
    x, w = inputs.rmsnorm_case(64, 4096, seed=0, dtype="f32")
    xd, wd = to_dev(x, "f32"), to_dev(w, "f32")
    inv = to_np(bi.rmsnorm(xd, wd, 1e-6))
    ref = oracle.rmsnorm(x, w, "f32", 1e-6)
    differs = 0
    for s in (2, 3, 8, 32):
        y = to_np(bi.rmsnorm_split(xd, wd, s, 1e-6))
        assert_parity(y, ref, "f32", f"splits={s}")
        differs += int(not bits_equal(y, inv))
    assert differs > 0
