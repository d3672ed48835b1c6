"""Decode / verify attention on the GPU: parity with the oracle and bitwise
identity between a lone query and the same query inside a causal verify block.

Workload: GQA with 32 query heads, 8 KV heads, head_dim 128; K, V, q ~ N(0,1)
bf16; key lengths Lk in {1028, 8196, 16388, 65540}; scale 1/sqrt(128); a query
block of 1 token or a causal block of 8 tokens at the end of the context --
the SDPA check of "Fix/speculative shape invariance" (Changes; the reviewer's
SDPA scenario)."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128
SCALE = 1.0 / np.sqrt(128.0)


def run(q, k, v, kv_len, causal=True, dtype="bf16", max_kv=None):
    kvd = torch.tensor(np.asarray(kv_len, np.int32), device=dev())
    mk = int(max(kv_len)) if max_kv is None else max_kv
    return to_np(bi.sdpa(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), kvd, mk, SCALE, causal))


@pytest.mark.parametrize("Lk", [1028, 8196, 16388, 65540])
def test_config_lone_query_equals_verify_block(Lk):
    q8, k, v = inputs.sdpa_case(1, 8, Lk, HQ, HKV, D, seed=0)
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    blk = to_np(bi.sdpa(to_dev(q8, "bf16"), kd, vd, torch.tensor([Lk], dtype=torch.int32, device=dev()),
                        Lk, SCALE, True))
    ref = oracle.sdpa(q8, k, v, np.array([Lk], np.int32), SCALE, True, "bf16")
    assert_parity(blk, ref, "bf16", f"Lk={Lk} Q=8")
    for j in range(8):
        L = Lk - 8 + j + 1
        one = to_np(bi.sdpa(to_dev(np.ascontiguousarray(q8[:, j:j + 1]), "bf16"), kd, vd,
                            torch.tensor([L], dtype=torch.int32, device=dev()), L, SCALE, True))
        assert bits_equal(one[0, 0], blk[0, j]), f"Lk={Lk} query {j}"


def test_q1_at_full_length_equals_last_block_row():
    Lk = 8196
    q8, k, v = inputs.sdpa_case(1, 8, Lk, HQ, HKV, D, seed=1)
    blk = run(q8, k, v, [Lk])
    one = run(np.ascontiguousarray(q8[:, 7:8]), k, v, [Lk])
    assert bits_equal(one[0, 0], blk[0, 7])


@pytest.mark.parametrize("Q", [1, 2, 5, 8, 13])
def test_every_block_width(Q):
    """Any verify width: query j of a causal block of Q equals the lone query."""
    Lk = 700
    qq, k, v = inputs.sdpa_case(1, Q, Lk, HQ, HKV, D, seed=Q)
    blk = run(qq, k, v, [Lk])
    assert_parity(blk, oracle.sdpa(qq, k, v, np.array([Lk], np.int32), SCALE, True, "bf16"), "bf16")
    for j in range(Q):
        one = run(np.ascontiguousarray(qq[:, j:j + 1]), k, v, [Lk - Q + j + 1])
        assert bits_equal(one[0, 0], blk[0, j]), f"Q={Q} j={j}"


def test_ragged_batch_and_batch_invariance():
    """Sequences of different lengths in one call; each sequence's output equals
    the output of the same sequence run alone, and matches the oracle."""
    B, Q, Lcap = 4, 5, 1300
    qq, k, v = inputs.sdpa_case(B, Q, Lcap, HQ, HKV, D, seed=2)
    kv_len = [1300, 5, 257, 1024]
    full = run(qq, k, v, kv_len, max_kv=1300)
    assert_parity(full, oracle.sdpa(qq, k, v, np.array(kv_len, np.int32), SCALE, True, "bf16"), "bf16")
    for b in range(B):
        one = run(np.ascontiguousarray(qq[b:b + 1]), np.ascontiguousarray(k[b:b + 1]),
                  np.ascontiguousarray(v[b:b + 1]), [kv_len[b]])
        assert bits_equal(one, full[b:b + 1]), f"sequence {b}"


@pytest.mark.parametrize("Lk", [1, 8, 255, 256, 257, 511, 512, 513])
def test_chunk_edges(Lk):
    Q = min(8, Lk)
    qq, k, v = inputs.sdpa_case(1, Q, Lk, HQ, HKV, D, seed=Lk)
    out = run(qq, k, v, [Lk])
    assert_parity(out, oracle.sdpa(qq, k, v, np.array([Lk], np.int32), SCALE, True, "bf16"), "bf16", f"Lk={Lk}")


def test_non_causal_and_f16():
    qq, k, v = inputs.sdpa_case(2, 3, 900, HQ, HKV, D, seed=5, dtype="f16")
    kv = [900, 600]
    for causal in (False, True):
        out = run(qq, k, v, kv, causal=causal, dtype="f16")
        ref = oracle.sdpa(qq, k, v, np.array(kv, np.int32), SCALE, causal, "f16")
        assert_parity(out, ref, "f16", f"causal={causal}")


def test_other_gqa_groupings():
    for hq, hkv in ((8, 8), (16, 2), (4, 1)):
        qq, k, v = inputs.sdpa_case(1, 4, 600, hq, hkv, D, seed=hq + hkv)
        kvd = torch.tensor([600], dtype=torch.int32, device=dev())
        out = to_np(bi.sdpa(to_dev(qq, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), kvd, 600, SCALE, True))
        assert_parity(out, oracle.sdpa(qq, k, v, np.array([600], np.int32), SCALE, True, "bf16"), "bf16")


def test_single_key_and_constant_values():
    qq, k, v = inputs.sdpa_case(1, 1, 64, HQ, HKV, D, seed=9)
    out = run(qq, k, v, [1])
    vf = v[0, 0]                                           # [Hkv, D]
    for h in range(HQ):
        assert bits_equal(out[0, 0, h], vf[h // 4])
    vc = inputs.to_storage(np.full(v.shape, -0.5, np.float32), "bf16")
    out = run(qq, k, vc, [37])
    assert np.all(out == vc.flat[0])


def test_cache_beyond_kv_len_is_never_read():
    """Positions at and past kv_len hold NaN: the output must not change."""
    Lcap, L = 1024, 700
    qq, k, v = inputs.sdpa_case(1, 8, Lcap, HQ, HKV, D, seed=11)
    base = run(qq, k, v, [L], max_kv=L)
    k2, v2 = k.copy(), v.copy()
    k2[:, L:] = 0x7FC1
    v2[:, L:] = 0xFFC1
    assert bits_equal(run(qq, k2, v2, [L], max_kv=L), base)


def test_bounded_stores():
    B, Q, L = 2, 8, 300
    qq, k, v = inputs.sdpa_case(B, Q, L, HQ, HKV, D, seed=12)
    og = Guarded((B, Q, HQ, D), torch.bfloat16, poison=0x3C)
    kvd = torch.tensor([L, 100], dtype=torch.int32, device=dev())
    need = bi.sdpa_workspace_bytes(B, Q, L, HQ, D)
    wsg = Guarded((need,), torch.uint8, poison=0x77)
    bi.sdpa(to_dev(qq, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), kvd, L, SCALE, True, out=og.view, ws=wsg.view)
    torch.cuda.synchronize()
    assert og.canaries_intact() and wsg.canaries_intact()
    assert_parity(to_np(og.view), oracle.sdpa(qq, k, v, np.array([L, 100], np.int32), SCALE, True, "bf16"), "bf16")


def test_run_to_run_determinism():
    qq, k, v = inputs.sdpa_case(1, 8, 4100, HQ, HKV, D, seed=13)
    qd, kd, vd = to_dev(qq, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    kvd = torch.tensor([4100], dtype=torch.int32, device=dev())
    first = bi.sdpa(qd, kd, vd, kvd, 4100, SCALE, True)
    for _ in range(30):
        assert torch.equal(bi.sdpa(qd, kd, vd, kvd, 4100, SCALE, True).view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("B,Q,Lk", [(1, 8, 1028), (3, 1, 783), (2, 5, 300), (4, 1, 4100)])
def test_head_major_cache_same_bits(B, Q, Lk):
    """The head-major cache [B, Hkv, Lcap, D] gives the [B, Lcap, Hkv, D]
    cache's bits (only the strides change), ragged lengths included."""
    q, k, v = inputs.sdpa_case(B, Q, Lk, HQ, HKV, D, seed=B + Q)
    kv_len = np.array([Lk - 3 * b for b in range(B)], np.int32)
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    kvd = torch.tensor(kv_len, device=dev())
    qd = to_dev(q, "bf16")
    std = to_np(bi.sdpa(qd, kd, vd, kvd, Lk, SCALE, True))
    hm = to_np(bi.sdpa(qd, kd.transpose(1, 2).contiguous(), vd.transpose(1, 2).contiguous(), kvd, Lk, SCALE, True,
                       head_major=True))
    assert bits_equal(hm, std)


@pytest.mark.parametrize("L,chunk", [(1100, 256), (777, 100), (520, 1)])
def test_prefill_chunking_invariance(L, chunk):
    """A prompt prefilled in one causal call and the same prompt prefilled in
    chunks over the growing cache give every token the same bits: a token's
    tree depends on its position only, not on the prefill chunking or on how
    much of the prefix was cached (the invariant-prefill property of chunked
    prefill)."""
    q, k, v = inputs.sdpa_case(1, L, L, HQ, HKV, D, seed=L)
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    qd = to_dev(q, "bf16")
    one = bi.sdpa(qd, kd, vd, torch.tensor([L], dtype=torch.int32, device=dev()), L, SCALE, True)
    parts = []
    for s0 in range(0, L, chunk):
        s1 = min(s0 + chunk, L)
        parts.append(bi.sdpa(qd[:, s0:s1].contiguous(), kd, vd, torch.tensor([s1], dtype=torch.int32, device=dev()),
                             s1, SCALE, True))
    assert torch.equal(torch.cat(parts, dim=1).view(torch.int16), one.view(torch.int16))


@pytest.mark.parametrize("B,Q,Lk,causal", [(1, 1, 16388, True), (3, 1, 2000, True), (2, 4, 1300, True),
                                           (2, 2, 700, False)])
def test_split_variant_parity(B, Q, Lk, causal):
    """The split-KV comparison variant (bi_sdpa_split: the chunk kernel
    carrying its softmax state across a run of chunks, the run length set by
    the caller's split count) is within the parity gate of the oracle at every
    split count, and runs of one chunk are bi_sdpa's own tree.  Ragged lengths
    (B = 3: Lk, Lk - 300, Lk - 855) and causal blocks included."""
    q, k, v = inputs.sdpa_case(B, Q, Lk, HQ, HKV, D, seed=11)
    kv = np.array([Lk - 300 * i - (255 if i > 1 else 0) for i in range(B)], np.int32)
    ref = oracle.sdpa(q, k, v, kv, SCALE, causal, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    kvd = torch.tensor(kv, device=dev())
    inv = to_np(bi.sdpa(qd, kd, vd, kvd, Lk, SCALE, causal))
    nch = -(-Lk // 256)
    for sp in (1, 2, 3, 7):
        assert_parity(to_np(bi.sdpa_split(qd, kd, vd, kvd, Lk, SCALE, sp, causal)), ref, "bf16", f"splits={sp}")
    assert bits_equal(to_np(bi.sdpa_split(qd, kd, vd, kvd, Lk, SCALE, nch, causal)), inv)
    assert bits_equal(to_np(bi.sdpa_split(qd, kd, vd, kvd, Lk, SCALE, 10 * nch, causal)), inv)


def test_split_variant_bits_follow_the_split_count():
    """Negative control: the split count changes output bits, so the
    invariance tests can tell a split tree from the fixed one.  The two trees
    differ by a few fp32 ulps, which a 16-bit rounding hides for most values
    (in bf16 almost all: at 4096 outputs no split count changed a bit), so
    the check runs in f16 over 131072 outputs (B 8, a causal block of 4)."""
    B, Q, Lk = 8, 4, 3000
    q, k, v = inputs.sdpa_case(B, Q, Lk, HQ, HKV, D, seed=12, dtype="f16")
    kvd = torch.full((B,), Lk, dtype=torch.int32, device=dev())
    qd, kd, vd = to_dev(q, "f16"), to_dev(k, "f16"), to_dev(v, "f16")
    inv = to_np(bi.sdpa(qd, kd, vd, kvd, Lk, SCALE, True))
    ref = oracle.sdpa(q, k, v, np.full(B, Lk, np.int32), SCALE, True, "f16")
    changed = 0
    for sp in (2, 3, 5):
        y = to_np(bi.sdpa_split(qd, kd, vd, kvd, Lk, SCALE, sp, True))
        assert_parity(y, ref, "f16", f"splits={sp}")
        changed += int(np.count_nonzero(y.view(np.uint16) != inv.view(np.uint16)))
    assert changed > 0


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("head_major", [False, True])
def test_prompt_kernel_rows_equal_lone_queries(causal, head_major):
    """Prompts (at least 128 query rows per KV head, up to 4096 keys) take
    the prompt-shaped kernel (a wave plays all four key quarters of a chunk;
    two passes over the chunks).  Every row must equal the same query run
    alone through the decode kernel at its position, with ragged lengths, a
    partial last block of rows and both cache layouts; sampled rows are within
    the parity gate of the oracle."""
    B, Q, Lcap = 2, 1000, 2600
    q, k, v = inputs.sdpa_case(B, Q, Lcap, HQ, HKV, D, seed=21)
    kv = np.array([2600, 1900], np.int32)
    qd = to_dev(q, "bf16")
    kd, vd = to_dev(k, "bf16"), to_dev(v, "bf16")
    if head_major:
        kd, vd = kd.transpose(1, 2).contiguous(), vd.transpose(1, 2).contiguous()
    kvd = torch.tensor(kv, device=dev())
    full = to_np(bi.sdpa(qd, kd, vd, kvd, int(kv.max()), SCALE, causal, head_major=head_major))
    for bb in range(B):
        for j in (0, 1, 37, Q // 2, Q - 2, Q - 1):
            L = int(kv[bb]) - Q + j + 1 if causal else int(kv[bb])
            qj = qd[bb:bb + 1, j:j + 1].contiguous()
            one = to_np(bi.sdpa(qj, kd[bb:bb + 1].contiguous(), vd[bb:bb + 1].contiguous(),
                                torch.tensor([L], dtype=torch.int32, device=dev()), L, SCALE, True,
                                head_major=head_major))
            assert bits_equal(one[0, 0], full[bb, j]), (bb, j)
    # parity: a few rows through the oracle, each as a lone query at its position
    for j in (0, 499, 999):
        lens = kv - Q + j + 1 if causal else kv
        ref = oracle.sdpa(np.ascontiguousarray(q[:, j:j + 1]), k, v, lens.astype(np.int32), SCALE, True, "bf16")
        assert_parity(full[:, j:j + 1], ref, "bf16", f"row {j}")


@pytest.mark.parametrize("Q,head_major,Lcap", [(1, False, 1024), (1, True, 1024), (4, False, 1024), (5, False, 1024),
                                               (8, True, 1024), (1, True, 3072), (2, False, 1536)])
def test_whole_group_form_equals_lone_sequences(Q, head_major, Lcap):
    """At least two (sequence, KV head) groups of at most 32 query rows per
    CU over at most 1024 keys, or with at most 48 (query row, chunk) partials
    (one query over 3072 keys, two over 1536): one workgroup walks all of a
    group's chunks and merges them itself, with no merge launch (the
    partials in LDS when they fit, else in the workspace).  Each sequence
    must equal the same sequence run alone (chunk items, then the merge
    launch), with ragged lengths on both sides of the chunk edges (256 keys),
    both cache layouts and causal blocks of 2, 4, 5 (a verify block: two row
    tiles) and 8; sampled sequences are within the parity gate of the
    oracle.  K, V, q ~ N(0,1) bf16 drawn on the device (seeded)."""
    cus = torch.cuda.get_device_properties(dev()).multi_processor_count
    B = -(-2 * cus // HKV)
    g = torch.Generator(device=dev()).manual_seed(40 + Q + 2 * head_major + Lcap)
    shape = (B, HKV, Lcap, D) if head_major else (B, Lcap, HKV, D)
    kd = torch.randn(shape, generator=g, device=dev()).to(torch.bfloat16)
    vd = torch.randn(shape, generator=g, device=dev()).to(torch.bfloat16)
    qd = torch.randn((B, Q, HQ, D), generator=g, device=dev()).to(torch.bfloat16)
    edges = [Q, Q + 1] + [e + d for e in range(256, Lcap, 256 if Lcap <= 1024 else 512) for d in (-1, 0, 1)] + [Lcap - 1, Lcap]
    rng = np.random.default_rng(Q)
    kv = np.array(edges + list(rng.integers(Q, Lcap + 1, B - len(edges))), np.int32)
    kvd = torch.tensor(kv, device=dev())
    full = to_np(bi.sdpa(qd, kd, vd, kvd, Lcap, SCALE, True, head_major=head_major))
    for b in range(B):
        L = int(kv[b])
        one = to_np(bi.sdpa(qd[b:b + 1].contiguous(), kd[b:b + 1].contiguous(), vd[b:b + 1].contiguous(),
                            kvd[b:b + 1].contiguous(), L, SCALE, True, head_major=head_major))
        assert bits_equal(one, full[b:b + 1]), f"sequence {b} (kv_len {L})"
    for b in (2, 9, 12):
        kb, vb = kd[b:b + 1], vd[b:b + 1]
        if head_major:
            kb, vb = kb.transpose(1, 2), vb.transpose(1, 2)
        ref = oracle.sdpa(to_np(qd[b:b + 1]), to_np(kb), to_np(vb), kv[b:b + 1], SCALE, True, "bf16")
        assert_parity(full[b:b + 1], ref, "bf16", f"sequence {b}")


@pytest.mark.parametrize("causal", [True, False])
def test_prompt_kernel_two_ranges_rows_equal_lone_queries(causal):
    """Prompts over more than 4096 keys (at most 8192) take the prompt kernel
    with two ranges of 16 chunks: per row, the range maximum from the first
    pass's chunk maxima, the range sums, and the row sums weighted range by
    range as the merge does.  Every row equals the same query run alone
    through the decode kernels (chunk partials, then the merge launch's range
    and row levels), with ragged lengths on both sides of the range edge;
    sampled rows are within the parity gate of the oracle."""
    B, Q, Lcap = 2, 300, 6100
    q, k, v = inputs.sdpa_case(B, Q, Lcap, HQ, HKV, D, seed=23)
    kv = np.array([6100, 4250], np.int32)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    kvd = torch.tensor(kv, device=dev())
    full = to_np(bi.sdpa(qd, kd, vd, kvd, int(kv.max()), SCALE, causal))
    for bb in range(B):
        for j in (0, 1, 150, Q - 1):
            L = int(kv[bb]) - Q + j + 1 if causal else int(kv[bb])
            one = to_np(bi.sdpa(qd[bb:bb + 1, j:j + 1].contiguous(), kd[bb:bb + 1].contiguous(),
                                vd[bb:bb + 1].contiguous(), torch.tensor([L], dtype=torch.int32, device=dev()), L,
                                SCALE, True))
            assert bits_equal(one[0, 0], full[bb, j]), (bb, j)
    for j in (0, Q - 1):
        lens = kv - Q + j + 1 if causal else kv
        ref = oracle.sdpa(np.ascontiguousarray(q[:, j:j + 1]), k, v, lens.astype(np.int32), SCALE, True, "bf16")
        assert_parity(full[:, j:j + 1], ref, "bf16", f"row {j}")


@pytest.mark.parametrize("kv_pair", [(8192, 4097), (4097, 8192)])
def test_prompt_kernel_two_ranges_f16_head_major_at_the_edges(kv_pair):
    """The two-range prompt kernel in f16 on a head-major cache, with key
    lengths at the limit of the one-launch form (8192) and one past the first
    range (4097, whose last chunk holds a single key), and 40 query positions
    (160 rows per KV head: one full block of 128 and a partial one): rows
    equal lone queries (decode kernels) and sampled rows are within the f16
    parity gate of the oracle."""
    B, Q, Lcap = 2, 40, 8192
    q, k, v = inputs.sdpa_case(B, Q, Lcap, HQ, HKV, D, seed=29, dtype="f16")
    kv = np.array(kv_pair, np.int32)
    kh, vh = (np.ascontiguousarray(a.transpose(0, 2, 1, 3)) for a in (k, v))
    qd, kd, vd = to_dev(q, "f16"), to_dev(kh, "f16"), to_dev(vh, "f16")
    full = to_np(bi.sdpa(qd, kd, vd, torch.tensor(kv, device=dev()), int(kv.max()), SCALE, True, head_major=True))
    for bb in range(B):
        for j in (0, 1, Q - 1):
            L = int(kv[bb]) - Q + j + 1
            one = to_np(bi.sdpa(qd[bb:bb + 1, j:j + 1].contiguous(), kd[bb:bb + 1].contiguous(),
                                vd[bb:bb + 1].contiguous(), torch.tensor([L], dtype=torch.int32, device=dev()), L,
                                SCALE, True, head_major=True))
            assert bits_equal(one[0, 0], full[bb, j]), (bb, j)
    for j in (0, Q - 1):
        ref = oracle.sdpa(np.ascontiguousarray(q[:, j:j + 1]), k, v, (kv - Q + j + 1).astype(np.int32), SCALE, True,
                          "f16")
        assert_parity(full[:, j:j + 1], ref, "f16", f"row {j}")
