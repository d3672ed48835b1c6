"""A seeded random campaign over the row reductions: RMSNorm (plain and fused
with the residual add), row log-softmax and row mean, at random row counts,
row lengths (ragged, not multiples of the 16-byte chunk) and dtypes.  Each
case is checked against the oracle, and one row against the same row alone
(bitwise) -- "Batch-invariant kernels" (Case 4: the sum-of-squares order must
not follow the batch; The boring rule, item 1; The trap).

Workload: x ~ N(0,1)*3, r ~ N(0,1), w = 1 + 0.1 N(0,1), logits ~ N(0,1)*4,
drawn from a fixed-seed generator and rounded to the case's dtype."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import assert_parity, bits_equal, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu


def draw_case(rng):
    op = ["rmsnorm", "add_rmsnorm", "log_softmax", "row_mean"][rng.integers(4)]
    dtype = ["bf16", "f16", "f32"][rng.integers(3)]
    rows = int(rng.integers(1, 300))
    H = int(rng.choice([int(rng.integers(1, 9000)), 4096, 4099, 32000, 70001]))
    return op, dtype, rows, H


CASES = [draw_case(np.random.default_rng(4000 + i)) for i in range(60)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c))
def test_random_row_case(case):
    op, dtype, rows, H = case
    rng = np.random.default_rng(rows + H)
    x = inputs.normal(rng, (rows, H), 3.0 if op != "log_softmax" else 4.0, dtype=dtype)
    xd = to_dev(x, dtype)
    i = rows // 2
    if op in ("rmsnorm", "add_rmsnorm"):
        w = inputs.normal(rng, (H,), 0.1, 1.0, dtype=dtype)
        wd = to_dev(w, dtype)
        if op == "rmsnorm":
            y = to_np(bi.rmsnorm(xd, wd))
            assert_parity(y, oracle.rmsnorm(x, w, dtype), dtype)
            assert bits_equal(to_np(bi.rmsnorm(xd[i:i + 1].contiguous(), wd)), y[i:i + 1])
        else:
            r = inputs.normal(rng, (rows, H), 1.0, dtype=dtype)
            rd = to_dev(r, dtype)
            xs = torch.empty_like(xd)
            y = to_np(bi.add_rmsnorm(xd, rd, wd, x_out=xs)[1])
            # the residual sum, rounded once to the dtype, from the oracle side
            s_ref = oracle.round_to(inputs.from_storage(x, dtype) + inputs.from_storage(r, dtype), dtype)
            assert bits_equal(to_np(xs), s_ref)
            if dtype == "bf16":
                assert bits_equal(to_np(bi.add(xd, rd)), s_ref)
            ref = oracle.rmsnorm(s_ref, w, dtype)
            assert_parity(y, ref, dtype)
            xs1 = torch.empty_like(xd[i:i + 1])
            y1 = to_np(bi.add_rmsnorm(xd[i:i + 1].contiguous(), rd[i:i + 1].contiguous(), wd, x_out=xs1)[1])
            assert bits_equal(y1, y[i:i + 1])
    elif op == "log_softmax":
        y = to_np(bi.log_softmax(xd))
        ref = oracle.log_softmax(x, dtype)
        assert np.abs(y - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
        assert bits_equal(to_np(bi.log_softmax(xd[i:i + 1].contiguous())), y[i:i + 1])
    else:
        y = to_np(bi.row_mean(xd))
        ref = oracle.row_mean(x, dtype)
        assert np.abs(y - ref).max() <= 1e-5 * max(1.0, np.abs(ref).max())
        assert bits_equal(to_np(bi.row_mean(xd[i:i + 1].contiguous())), y[i:i + 1])
