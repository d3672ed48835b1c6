"""A seeded random campaign over decode / verify / prefill attention: batch,
query block width, per-sequence KV lengths (chunk boundaries and ragged
tails), head grouping, cache layout, causal or not, bf16 or f16.  Each case is
checked against the oracle, and one query row against the same query issued
alone at its position (bitwise) -- "Fix/speculative shape invariance"
(Problem, Changes) and "Batch-invariant kernels" (Case 6: a fixed split size).

Workload: K, V ~ N(0,1) then q ~ N(0,1), D = 128, drawn from a fixed-seed
generator; kv_len per sequence uniform in [Q, Lcap]."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu


def draw_case(rng):
    dtype = ["bf16", "bf16", "f16"][rng.integers(3)]
    Hq, Hkv = [(32, 8), (8, 8), (16, 4), (8, 1)][rng.integers(4)]
    B = int(rng.integers(1, 5))
    Q = int(rng.choice([1, 1, 2, 5, 8, 33, 130]))
    Lcap = int(rng.integers(Q, 1400))
    causal = bool(rng.integers(4) != 0)
    head_major = bool(rng.integers(2))
    kv = rng.integers(Q, Lcap + 1, size=B).astype(np.int32)
    return dtype, Hq, Hkv, B, Q, Lcap, causal, head_major, tuple(int(v) for v in kv)


CASES = [draw_case(np.random.default_rng(3000 + i)) for i in range(60)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(v) for v in c[:8]))
def test_random_sdpa_case(case):
    dtype, Hq, Hkv, B, Q, Lcap, causal, head_major, kv = case
    q, k, v = inputs.sdpa_case(B, Q, Lcap, Hq, Hkv, 128, seed=B + Q + Lcap, dtype=dtype)
    kvl = np.array(kv, np.int32)
    sc = 1.0 / np.sqrt(128.0)
    kd, vd = to_dev(k, dtype), to_dev(v, dtype)
    if head_major:
        kd, vd = kd.permute(0, 2, 1, 3).contiguous(), vd.permute(0, 2, 1, 3).contiguous()
    max_kv = int(kvl.max())
    kvd = torch.from_numpy(kvl).to(dev())
    o = to_np(bi.sdpa(to_dev(q, dtype), kd, vd, kvd, max_kv, sc, causal, head_major=head_major))
    assert_parity(o, oracle.sdpa(q, k, v, kvl, sc, causal, dtype), dtype)
    # the last sequence's last query row, issued alone at its position (it sees
    # keys [0, kv_len) in both modes)
    b, j = B - 1, Q - 1
    alone_len = np.array([kvl[b]], np.int32)
    qa = to_dev(np.ascontiguousarray(q[b:b + 1, j:j + 1]), dtype)
    ka, va = kd[b:b + 1].contiguous(), vd[b:b + 1].contiguous()
    oa = to_np(bi.sdpa(qa, ka, va, torch.from_numpy(alone_len).to(dev()), int(alone_len[0]), sc, True,
                       head_major=head_major))
    assert bits_equal(oa[0, 0], o[b, j])
