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


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,H", [(64, 4096), (3, 4100), (5, 8192), (7, 5000), (1, 1)])
def test_add_rmsnorm_equals_add_then_norm(dtype, rows, H):
    """The fused residual add + RMSNorm gives the bits of bi_add (for bf16)
    followed by bi_rmsnorm, in place (x_out = x) and out of place, on the
    cached / streamed and vector / element-wise paths; the norm is within
    the tolerance of the oracle's norm of the rounded sum."""
    rng = np.random.default_rng(rows * 7 + H)
    x = inputs.normal(rng, (rows, H), 3.0, dtype=dtype)
    r = inputs.normal(rng, (rows, H), 0.5, dtype=dtype)
    w = inputs.normal(rng, (H,), 0.1, loc=1.0, dtype=dtype)
    xd, rd, wd = to_dev(x, dtype), to_dev(r, dtype), to_dev(w, dtype)
    s_ref = oracle.round_to(inputs.from_storage(x, dtype) + inputs.from_storage(r, dtype), dtype)
    xo, y = bi.add_rmsnorm(xd, rd, wd, 1e-6)
    assert bits_equal(to_np(xo), s_ref)
    assert bits_equal(to_np(y), to_np(bi.rmsnorm(xo, wd, 1e-6)))
    assert_parity(to_np(y), oracle.rmsnorm(s_ref, w, dtype, 1e-6), dtype)
    xi = xd.clone()
    yi = torch.empty_like(xi)
    bi.add_rmsnorm(xi, rd, wd, 1e-6, x_out=xi, out=yi)
    assert bits_equal(to_np(xi), s_ref) and bits_equal(to_np(yi), to_np(y))
    if dtype == "bf16":
        assert bits_equal(to_np(bi.add(xd, rd)), s_ref)


def test_add_rmsnorm_rows_invariant_and_bounded():
    """Rows of the fused op at B = 64 equal those at B = 1, 7; the outputs are
    fenced by canaries."""
    rng = np.random.default_rng(9)
    x = inputs.normal(rng, (64, 4096), 3.0)
    r = inputs.normal(rng, (64, 4096), 0.5)
    w = inputs.normal(rng, (4096,), 0.1, loc=1.0)
    xd, rd, wd = to_dev(x, "bf16"), to_dev(r, "bf16"), to_dev(w, "bf16")
    _, full = bi.add_rmsnorm(xd, rd, wd, 1e-6)
    for B in (1, 7):
        _, y = bi.add_rmsnorm(xd[:B].contiguous(), rd[:B].contiguous(), wd, 1e-6)
        assert bits_equal(to_np(y), to_np(full[:B]))
    xg = Guarded((64, 4096), torch.bfloat16, poison=0xA5)
    yg = Guarded((64, 4096), torch.bfloat16, poison=0x5A)
    bi.add_rmsnorm(xd, rd, wd, 1e-6, x_out=xg.view, out=yg.view)
    torch.cuda.synchronize()
    assert xg.canaries_intact() and yg.canaries_intact()
    assert bits_equal(to_np(yg.view), to_np(full))


@pytest.mark.parametrize("rows", [2048, 2049, 4096, 5000])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_many_rows_form_equals_row_alone(rows, dtype):
    """Thousands of rows (more rows than the GPU holds waves at once): rows,
    fused and plain, in and out of place, equal the same rows normalized
    alone or in a small batch, and the outputs are fenced by canaries."""
    H = 4096
    rng = np.random.default_rng(rows)
    x = inputs.normal(rng, (rows, H), 3.0, dtype=dtype)
    r = inputs.normal(rng, (rows, H), 0.5, dtype=dtype)
    w = inputs.normal(rng, (H,), 0.1, loc=1.0, dtype=dtype)
    xd, rd, wd = to_dev(x, dtype), to_dev(r, dtype), to_dev(w, dtype)
    yg = Guarded((rows, H), xd.dtype, poison=0x5A)
    bi.rmsnorm(xd, wd, 1e-6, out=yg.view)
    xog, yag = Guarded((rows, H), xd.dtype, poison=0xA5), Guarded((rows, H), xd.dtype, poison=0x3C)
    bi.add_rmsnorm(xd, rd, wd, 1e-6, x_out=xog.view, out=yag.view)
    torch.cuda.synchronize()
    assert yg.canaries_intact() and xog.canaries_intact() and yag.canaries_intact()
    y, xo, ya = to_np(yg.view), to_np(xog.view), to_np(yag.view)
    pick = [0, 1, rows // 2, rows - 2, rows - 1]
    for i in pick:
        assert bits_equal(to_np(bi.rmsnorm(xd[i:i + 1].contiguous(), wd, 1e-6)), y[i:i + 1]), i
        xo1, ya1 = bi.add_rmsnorm(xd[i:i + 1].contiguous(), rd[i:i + 1].contiguous(), wd, 1e-6)
        assert bits_equal(to_np(xo1), xo[i:i + 1]) and bits_equal(to_np(ya1), ya[i:i + 1]), i
    small = to_np(bi.rmsnorm(xd[:512].contiguous(), wd, 1e-6))
    assert bits_equal(small, y[:512])
    assert_parity(y[pick], oracle.rmsnorm(np.ascontiguousarray(x[pick]), w, dtype, 1e-6), dtype)
    xi = xd.clone()
    yi = torch.empty_like(xi)
    bi.add_rmsnorm(xi, rd, wd, 1e-6, x_out=xi, out=yi)
    assert bits_equal(to_np(xi), xo) and bits_equal(to_np(yi), ya)
