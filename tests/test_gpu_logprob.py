"""Row log-softmax, token log-probabilities and row mean on the GPU: parity
with the oracle, closed forms, and bitwise identity of a row alone and inside
any batch.

Workload: logits of the decoder's LM head shape (rows up to 64, vocab 32000)
~ N(0, 4) in bf16, plus f16 / f32 and ragged column counts -- the
log-probabilities a sampler and a trainer compare ("Batch-invariant kernels
...", The trap; The boring rule, item 2: f(x[None]) against f(batch)[0] across
batch sizes)."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, dev, to_dev
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def logits(rows, cols, dtype, seed):
    rng = np.random.default_rng(seed)
    return inputs.to_storage((rng.standard_normal((rows, cols)) * 4).astype(np.float32), dtype)


def rel(g, r):
    g = g.astype(np.float64); r = r.astype(np.float64)
    return float(np.abs(g - r).max() / max(np.abs(r).max(), 1e-30))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,cols", [(64, 32000), (3, 1001), (5, 8), (2, 1), (2, 50000), (1, 70000)])
def test_log_softmax_parity_and_logprob(dtype, rows, cols):
    x = logits(rows, cols, dtype, seed=rows + cols)
    xd = to_dev(x, dtype)
    y = bi.log_softmax(xd).cpu().numpy()
    assert rel(y, oracle.log_softmax(x, dtype)) <= 1e-5
    ids = torch.tensor(np.random.default_rng(cols).integers(0, cols, size=rows).astype(np.int32), device=dev())
    lp = bi.token_logprob(xd, ids).cpu().numpy()
    assert np.array_equal(lp.view(np.uint32), y[np.arange(rows), ids.cpu().numpy()].view(np.uint32))
    m = bi.row_mean(xd).cpu().numpy()
    assert rel(m, oracle.row_mean(x, dtype)) <= 1e-5


@pytest.mark.parametrize("cols", [32000, 4099])
def test_rows_independent_of_batch(cols):
    """Every prefix and every single row give the full call's bits (log-softmax,
    token log-prob, mean)."""
    x = to_dev(logits(64, cols, "bf16", seed=7), "bf16")
    ids = torch.randint(0, cols, (64,), dtype=torch.int32, device=dev())
    full, lpf, mf = bi.log_softmax(x), bi.token_logprob(x, ids), bi.row_mean(x)
    for B in (1, 2, 8, 33, 64):
        assert torch.equal(bi.log_softmax(x[:B].contiguous()).view(torch.int32), full[:B].view(torch.int32))
        assert torch.equal(bi.token_logprob(x[:B].contiguous(), ids[:B].contiguous()).view(torch.int32),
                           lpf[:B].view(torch.int32))
        assert torch.equal(bi.row_mean(x[:B].contiguous()).view(torch.int32), mf[:B].view(torch.int32))
    for r in (0, 17, 63):
        assert torch.equal(bi.log_softmax(x[r:r + 1].contiguous()).view(torch.int32), full[r:r + 1].view(torch.int32))


def test_closed_forms_and_bounded_stores():
    """Constant rows: every entry equal, -ln(cols) to fp32 accuracy; a dominant
    logit: exactly 0 there and exactly -100 elsewhere; integer rows of length
    4096: exact means; out-of-range ids give NaN; stores stay in bounds."""
    cols = 32000
    x = torch.full((3, cols), 2.5, dtype=torch.bfloat16, device=dev())
    y = bi.log_softmax(x).cpu().numpy()
    assert np.all(y == y[0, 0]) and abs(float(y[0, 0]) + np.log(cols)) <= 4e-7 * np.log(cols)
    z = torch.zeros((1, 1000), dtype=torch.float32, device=dev())
    z[0, 417] = 100.0
    yz = bi.log_softmax(z).cpu().numpy()[0]
    assert yz[417] == 0.0 and np.all(np.delete(yz, 417) == -100.0)
    xi = torch.randint(-100, 100, (4, 4096), device=dev()).to(torch.bfloat16)
    assert np.array_equal(bi.row_mean(xi).cpu().numpy().astype(np.float64),
                          xi.double().cpu().numpy().mean(axis=1))
    bad = torch.tensor([-1, cols, 5], dtype=torch.int32, device=dev())
    lp = bi.token_logprob(x, bad).cpu().numpy()
    assert np.isnan(lp[0]) and np.isnan(lp[1]) and np.isfinite(lp[2])
    yg = Guarded((5, 1001), torch.float32, poison=0x7F)
    bi.log_softmax(to_dev(logits(5, 1001, "bf16", seed=3), "bf16"), out=yg.view)
    torch.cuda.synchronize()
    assert yg.canaries_intact()


def test_run_to_run_determinism():
    x = to_dev(logits(64, 32000, "bf16", seed=9), "bf16")
    first = bi.log_softmax(x)
    for _ in range(20):
        assert torch.equal(bi.log_softmax(x).view(torch.int32), first.view(torch.int32))
