"""The 4-layer Llama-style decoder on the GPU: greedy tokens and logits are
bit-identical across batch sizes and between plain and speculative decoding,
and the logits agree with the oracle's teacher-forced forward.

Workload: hidden 4096, 32 query / 8 KV heads, head_dim 128, SwiGLU 14336,
vocab 32000, RMSNorm, RoPE, bf16, random init N(0, 0.02); 512-token random
prompts, 256 greedy steps at B in {1, 4, 16, 64}; speculative verification
with 4-token drafts.  This is the serving scenario of "Batch-invariant
kernels: why temperature-0 decoding is still nondeterministic" (Thesis, Case 5)
and the speculative-decoding motivation of "Fix/speculative shape invariance"
(Problem)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import dev
from invariant_reductions_amd import inputs
from invariant_reductions_amd.decoder import Decoder

pytestmark = pytest.mark.gpu

CFG = inputs.LLAMA_4L
P, STEPS, BMAX = 512, 256, 64


@pytest.fixture(scope="module")
def weights():
    return inputs.decoder_weights(CFG, seed=0)


@pytest.fixture(scope="module")
def model(weights):
    return Decoder(CFG, weights, max_batch=BMAX, max_q=P, max_len=P + STEPS + 8, device=dev())


@pytest.fixture(scope="module")
def prompts():
    return inputs.prompts(BMAX, P, CFG["vocab"], seed=1)


class Checksums:
    """Two weighted sums of each logits row's 16-bit patterns: any change of
    the row's bits changes them (barring a collision of both)."""

    def __init__(self, B, steps, V):
        self.cs = torch.zeros((B, steps, 2), dtype=torch.int64, device=dev())
        self.w1 = torch.arange(1, V + 1, dtype=torch.int64, device=dev())
        g = torch.Generator().manual_seed(7)
        self.w2 = torch.randint(1, 1 << 20, (V,), generator=g, dtype=torch.int64).to(dev())

    def row(self, lg):
        v = lg.view(torch.int16).to(torch.int64)
        return torch.stack([(v * self.w1).sum(-1), (v * self.w2).sum(-1)], dim=-1)

    def plain(self, i, lg):
        self.cs[:, i] = self.row(lg)

    def spec(self, b, i, lg):
        self.cs[b, i] = self.row(lg)


@pytest.fixture(scope="module")
def plain64(model, prompts):
    cs = Checksums(BMAX, STEPS, CFG["vocab"])
    toks = model.generate(torch.from_numpy(prompts).to(dev()), STEPS, on_logits=cs.plain)
    return toks, cs.cs.cpu().numpy()


@pytest.mark.parametrize("B", [1, 4, 16])
def test_tokens_and_logits_identical_across_batch_sizes(model, prompts, plain64, B):
    toks64, cs64 = plain64
    cs = Checksums(B, STEPS, CFG["vocab"])
    toks = model.generate(torch.from_numpy(prompts[:B]).to(dev()), STEPS, on_logits=cs.plain)
    assert np.array_equal(toks, toks64[:B])
    assert np.array_equal(cs.cs.cpu().numpy(), cs64[:B])


def test_replayed_advancing_plan_equals_generate(model, prompts, plain64):
    """The one-token plan with the argmax's own bookkeeping (next ids and kv
    lengths written by the kernel), replayed step after step, produces the
    plain decoding's tokens."""
    B, n = 16, 24
    first, _ = model.prefill(torch.from_numpy(prompts[:B]).to(dev()))
    model.ids[:B].copy_(torch.from_numpy(first).to(dev()))
    model.kv_len[:B].fill_(P + 1)
    plan = model.plan(B, 1, P + STEPS, advance=True)
    got = [first]
    for _ in range(1, n):
        model.run_plan(plan)
        got.append(model.next_ids[:B].cpu().numpy())
    assert np.array_equal(np.stack(got, axis=1), plain64[0][:B, :n])
    assert np.array_equal(model.kv_len[:B].cpu().numpy(), np.full(B, P + n, np.int32))
    assert np.array_equal(model.ids[:B].cpu().numpy(), got[-1])


def test_tokens_vary_between_sequences(plain64):
    toks64, _ = plain64
    assert len({tuple(r) for r in toks64}) > 1


@pytest.mark.parametrize("B,mode", [(64, "replay"), (16, "corrupt"), (4, "corrupt"), (1, "corrupt")])
def test_speculative_equals_plain(model, prompts, plain64, B, mode):
    toks64, cs64 = plain64

    def draft(b, i, n):
        idx = np.arange(i, i + n)
        prop = np.where(idx < STEPS, toks64[b, np.minimum(idx, STEPS - 1)], 0).astype(np.int32)
        if mode == "corrupt":
            bad = (idx * 7 + b * 3) % 5 == 0
            prop = np.where(bad, (prop + 1) % CFG["vocab"], prop).astype(np.int32)
        return prop

    cs = Checksums(B, STEPS, CFG["vocab"])
    toks = model.generate_speculative(torch.from_numpy(prompts[:B]).to(dev()), STEPS, draft, 4, on_logits=cs.spec)
    assert np.array_equal(toks, toks64[:B])
    assert np.array_equal(cs.cs.cpu().numpy(), cs64[:B])
    if mode == "replay":
        assert model.rounds <= (STEPS + 3) // 5 + 1          # every draft accepted: 5 tokens per round


def test_logits_match_oracle_teacher_forced(weights, prompts):
    """Config 5's 768 positions at B = 1 against the oracle: the 512-token
    prompt, then 256 more tokens fed one per step through the decode path (a
    seeded continuation, so no oracle input comes from the GPU; the decode
    steps run exactly as in greedy decoding).

    Gate.  The 2e-2 bf16 tolerance bounds one op's output and every op is held
    to it by its own tests.  The logits here sit ~47 bf16-rounded ops deep,
    where the oracle itself is only defined up to the choice of fixed order:
    the same oracle with every reduction folded descending instead of
    ascending (tests/golden/decoder_tree_spread.json, written by
    tests/golden/make_decoder_spread.py from oracle/ alone) differs from the
    ascending one by up to 1.85e-2 per position (median 1.33e-2) on these
    very inputs, and picks a different greedy token at 24 of the 768
    positions ("Batch-invariant kernels", Case 5 and The trap: close is not
    identical -- identity is checked GPU-vs-GPU above).  The GPU, a third
    fixed order, must sit no further from the oracle than that spread allows:
    every position within 1.25x the spread's maximum, the median within 1.25x
    its median (1.25: the sampling noise of a maximum over 768 positions),
    and at least 99% of positions within the per-op 2e-2.  Where the
    oracle's top-2 margin exceeds 5e-2 of max |logit| (more than twice the
    gate), the GPU's greedy token (its own argmax kernel on its own logits)
    must be the oracle's: an error within the gate cannot reorder that pair."""
    import json
    import os
    S = STEPS
    with open(os.path.join(os.path.dirname(__file__), "golden", "decoder_tree_spread.json")) as f:
        spread = json.load(f)
    m = Decoder(CFG, weights, max_batch=1, max_q=P, max_len=P + S + 8, device=dev())
    pr = prompts[:1]
    cont = inputs.prompts(1, S, CFG["vocab"], seed=5)
    got = np.zeros((P + S, CFG["vocab"]), np.float32)
    gtok = np.zeros(P + S, np.int64)

    def keep(p, lg):
        got[p] = lg[0].float().cpu().numpy()
        if p == 0:                                   # the prefill's argmax of every prompt position
            gtok[:P] = m.next_ids[:P].cpu().numpy()
        elif p >= P:
            gtok[p] = int(m.next_ids[0].item())

    m.teacher_forced(torch.from_numpy(pr).to(dev()), cont, keep)
    seq = np.concatenate([pr[0], cont[0]])
    cos_t, sin_t = inputs.rope_tables(P + S + 8, CFG["head_dim"])
    from oracle import decoder as odec
    ref32, _, ref_tok = odec.forward(weights, CFG, seq, cos_t, sin_t)
    r = ref32.astype(np.float64)
    scale = np.abs(r).max(1)
    rel = np.abs(got - r).max(1) / scale
    top = np.sort(r, 1)[:, -2:]
    decisive = (top[:, 1] - top[:, 0]) > 0.05 * scale
    within = float(np.mean(rel <= 2e-2))
    print(f"decoder logits vs oracle over {P + S} positions: worst {rel.max():.4e} at {int(rel.argmax())}, "
          f"median {np.median(rel):.4e}, p99 {np.quantile(rel, 0.99):.4e}, within 2e-2 {within:.4f}; "
          f"oracle tree spread max {spread['max']:.4e} median {spread['median']:.4e}; "
          f"decisive positions {int(decisive.sum())}")
    assert spread["positions"] == P + S
    assert rel.max() <= 1.25 * spread["max"], (int(rel.argmax()), float(rel.max()))
    assert np.median(rel) <= 1.25 * spread["median"], float(np.median(rel))
    assert within >= 0.99, within
    bad = np.nonzero(decisive & (gtok != ref_tok))[0]
    assert bad.size == 0, bad[:10]


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336), (32000, 4096)])
def test_projection_shapes_per_op_parity(N, K):
    """Each projection of the decoder at its decode shape (M = 64) is within
    the per-op bf16 gate of the oracle, and row 5 equals its M = 1 result."""
    import invariant_reductions_amd as bi
    import oracle
    from gpu_util import assert_parity, bits_equal, to_dev, to_np
    x, w, _ = inputs.dense_case(64, N, K, "bf16", seed=N + K)
    xd, wd = to_dev(x, "bf16"), to_dev(w, "bf16")
    y = to_np(bi.matmul(xd, wd))
    rows = [0, 5, 63]
    assert_parity(y[rows], oracle.matmul(np.ascontiguousarray(x[rows]), w, "bf16", True), "bf16")
    assert bits_equal(to_np(bi.matmul(xd[5:6].contiguous(), wd)), y[5:6])
