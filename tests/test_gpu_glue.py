"""Decoder glue kernels on the GPU against the oracle's pointwise pieces."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu


def test_embed_gathers_rows():
    rng = np.random.default_rng(0)
    table = inputs.normal(rng, (1000, 256), 1.0)
    ids = rng.integers(0, 1000, size=37).astype(np.int32)
    out = to_np(bi.embed(torch.from_numpy(ids).to(dev()), to_dev(table, "bf16")))
    assert bits_equal(out, table[ids])


def test_rope_and_kv_write_bit_exact():
    """Rotation uses separately rounded products and sums on both sides, so the
    GPU equals the oracle bit for bit; k and v land at positions kv_len-Q+j."""
    rng = np.random.default_rng(1)
    B, Q, Hq, Hkv, D, Lcap = 3, 5, 8, 2, 128, 64
    qkv = inputs.normal(rng, (B * Q, (Hq + 2 * Hkv) * D), 2.0)
    kv_len = np.array([5, 17, 64], np.int32)
    cos_t, sin_t = inputs.rope_tables(128, D)
    qo = torch.empty((B * Q, Hq * D), dtype=torch.bfloat16, device=dev())
    kc = torch.zeros((B, Lcap, Hkv, D), dtype=torch.bfloat16, device=dev())
    vc = torch.zeros((B, Lcap, Hkv, D), dtype=torch.bfloat16, device=dev())
    bi.rope_kv_write(to_dev(qkv, "bf16"), qo, kc, vc, torch.from_numpy(kv_len).to(dev()),
                     torch.from_numpy(cos_t).to(dev()), torch.from_numpy(sin_t).to(dev()), B, Q, Hq, Hkv, D)
    pos = (kv_len[:, None] - Q + np.arange(Q)[None, :]).reshape(-1).astype(np.int32)
    q_ref = oracle.round_to(oracle.rope(np.ascontiguousarray(qkv[:, :Hq * D].reshape(B * Q, Hq, D)), pos,
                                        cos_t, sin_t, "bf16"), "bf16")
    k_ref = oracle.round_to(oracle.rope(np.ascontiguousarray(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(B * Q, Hkv, D)),
                                        pos, cos_t, sin_t, "bf16"), "bf16")
    assert bits_equal(to_np(qo).reshape(B * Q, Hq, D), q_ref)
    kcn, vcn = to_np(kc), to_np(vc)
    v_src = qkv[:, (Hq + Hkv) * D:].reshape(B, Q, Hkv, D)
    for b in range(B):
        for j in range(Q):
            p = kv_len[b] - Q + j
            assert bits_equal(kcn[b, p], k_ref[b * Q + j])
            assert bits_equal(vcn[b, p], v_src[b, j])
    untouched = np.ones((B, Lcap), bool)
    for b in range(B):
        untouched[b, kv_len[b] - Q:kv_len[b]] = False
    assert np.all(kcn[untouched] == 0) and np.all(vcn[untouched] == 0)


def test_silu_mul_within_one_ulp():
    rng = np.random.default_rng(2)
    g = inputs.normal(rng, (64, 1000), 4.0)
    u = inputs.normal(rng, (64, 1000), 1.0)
    gu = np.concatenate([g, u], axis=1)
    out = to_np(bi.silu_mul(to_dev(gu, "bf16")))
    r = oracle.round_to(oracle.silu_mul(g, u, "bf16"), "bf16")
    # exp may differ by an ulp between libraries; after bf16 rounding at most one bf16 ulp apart
    d = np.abs(out.astype(np.int32) - r.astype(np.int32))
    assert d.max() <= 1 and np.mean(d == 0) > 0.99


def test_add_bit_exact():
    rng = np.random.default_rng(3)
    a = inputs.normal(rng, (4097,), 3.0)
    b = inputs.normal(rng, (4097,), 0.01)
    out = to_np(bi.add(to_dev(a, "bf16"), to_dev(b, "bf16")))
    r = oracle.round_to(inputs.from_storage(a, "bf16") + inputs.from_storage(b, "bf16"), "bf16")
    assert bits_equal(out, r)


def test_argmax_matches_oracle_and_breaks_ties_low():
    rng = np.random.default_rng(4)
    x = inputs.normal(rng, (33, 32000), 1.0)
    x[5, 100] = x[5, 31000] = inputs.to_storage(np.array([50.0], np.float32), "bf16")[0]
    x[6, :] = x[6, 0]
    got = to_np(bi.argmax(to_dev(x, "bf16")))
    assert np.array_equal(got, oracle.argmax(x, "bf16"))
    assert got[5] == 100 and got[6] == 0
