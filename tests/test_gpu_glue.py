"""Decoder glue kernels on the GPU against the oracle's pointwise pieces."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu


def test_embed_gathers_rows():
    rng = np.random.default_rng(0)
    table = inputs.normal(rng, (1000, 256), 1.0)
    ids = rng.integers(0, 1000, size=37).astype(np.int32)
    out = to_np(bi.embed(torch.from_numpy(ids).to(dev()), to_dev(table, "bf16")))
    assert bits_equal(out, table[ids])


@pytest.mark.parametrize("dtype,H,T", [("bf16", 4096, 64), ("f16", 4096, 7), ("bf16", 8192, 5), ("bf16", 1000, 3)])
def test_embed_rmsnorm_equals_lookup_then_norm(dtype, H, T):
    """The lookup fused with the first norm gives bi_embed's rows (zero rows for
    ids outside [0, V)) and bi_rmsnorm's bits on them; 8192 columns (past the
    one-launch form) and 1000 (not 16-byte rows) take the two-launch path and
    must agree too.  The norm of the gathered rows is within the gate of the
    oracle's."""
    V = 1000
    rng = np.random.default_rng(H + T)
    table = inputs.normal(rng, (V, H), 3.0, dtype=dtype)
    w = inputs.to_storage(1.0 + 0.1 * rng.standard_normal(H).astype(np.float32), dtype)
    ids = rng.integers(0, V, size=T).astype(np.int32)
    if T >= 3:
        ids[1], ids[2] = -1, V                            # outside the table: zero rows
    idd = torch.from_numpy(ids).to(dev())
    td, wd = to_dev(table, dtype), to_dev(w, dtype)
    if H % 8:
        with pytest.raises(bi.BIError):                   # bi_embed's 16-byte rows
            bi.embed_rmsnorm(idd, td, wd)
        return
    xo, y = bi.embed_rmsnorm(idd, td, wd)
    x_ref = bi.embed(idd, td)
    y_ref = bi.rmsnorm(x_ref, wd)
    assert bits_equal(to_np(xo), to_np(x_ref))
    assert bits_equal(to_np(y), to_np(y_ref))
    rows = np.where(((ids >= 0) & (ids < V))[:, None], table[np.clip(ids, 0, V - 1)], 0).astype(table.dtype)
    assert bits_equal(to_np(xo), rows)
    assert_parity(to_np(y), oracle.rmsnorm(rows, w, dtype, 1e-6), dtype, f"{T}x{H}")


@pytest.mark.parametrize("D", [128, 24])
def test_rope_and_kv_write_bit_exact(D):
    """Rotation uses separately rounded products and sums on both sides, so the
    GPU equals the oracle bit for bit; k and v land at positions kv_len-Q+j.
    D = 128 takes the 8-pair vector path, D = 24 the pair-at-a-time one."""
    rng = np.random.default_rng(1)
    B, Q, Hq, Hkv, Lcap = 3, 5, 8, 2, 64
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
    # the head-major cache holds the same rows at [b, h, p]
    kh = torch.zeros((B, Hkv, Lcap, D), dtype=torch.bfloat16, device=dev())
    vh = torch.zeros((B, Hkv, Lcap, D), dtype=torch.bfloat16, device=dev())
    bi.rope_kv_write(to_dev(qkv, "bf16"), qo, kh, vh, torch.from_numpy(kv_len).to(dev()),
                     torch.from_numpy(cos_t).to(dev()), torch.from_numpy(sin_t).to(dev()), B, Q, Hq, Hkv, D,
                     head_major=True)
    assert bits_equal(to_np(kh.transpose(1, 2).contiguous()), kcn)
    assert bits_equal(to_np(vh.transpose(1, 2).contiguous()), vcn)


@pytest.mark.parametrize("F", [1000, 1001, 14336])
def test_silu_mul_within_one_ulp(F):
    """F % 8 == 0 takes the 16-byte path, F = 1001 the element-wise one."""
    rng = np.random.default_rng(2)
    g = inputs.normal(rng, (64 if F < 14336 else 8, F), 4.0)
    u = inputs.normal(rng, g.shape, 1.0)
    gu = np.concatenate([g, u], axis=1)
    out = to_np(bi.silu_mul(to_dev(gu, "bf16")))
    r = oracle.round_to(oracle.silu_mul(g, u, "bf16"), "bf16")
    # exp may differ by an ulp between libraries; after bf16 rounding at most one bf16 ulp apart
    d = np.abs(out.astype(np.int32) - r.astype(np.int32))
    assert d.max() <= 1 and np.mean(d == 0) > 0.99


@pytest.mark.parametrize("n", [4097, 4096 * 64])
def test_add_bit_exact(n):
    rng = np.random.default_rng(3)
    a = inputs.normal(rng, (n,), 3.0)
    b = inputs.normal(rng, (n,), 0.01)
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


@pytest.mark.parametrize("rows,cols", [(64, 32000), (5, 32001), (3, 8), (2, 1), (4, 65536 + 24)])
def test_argmax_ties_across_threads_and_ragged_rows(rows, cols):
    """Equal maxima placed in different threads' chunks and in the last
    chunk: the lowest index wins on the 16-byte path (cols % 8 == 0) and the
    element-wise path alike."""
    rng = np.random.default_rng(rows + cols)
    x = inputs.normal(rng, (rows, cols), 1.0)
    big = inputs.to_storage(np.array([60.0], np.float32), "bf16")[0]
    if cols > 9000:
        x[0, [8 * 1024 + 7, 7, cols - 1]] = big          # three threads hold the maximum
        x[1, [cols - 1, cols - 2]] = big                 # ties in the final chunk
    x[-1, :] = x[-1, 0]                                  # every element equal: index 0
    got = to_np(bi.argmax(to_dev(x, "bf16")))
    assert np.array_equal(got, oracle.argmax(x, "bf16"))
    assert got[-1] == 0
    if cols > 9000:
        assert got[0] == 7 and got[1] == cols - 2
