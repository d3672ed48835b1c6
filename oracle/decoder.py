"""Oracle forward pass of the 4-layer Llama-style decoder (teacher forced).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The model is the composition the chapter "Batch-invariant kernels: why
temperature-0 decoding is still nondeterministic" names in its Mental model
and Case 6: pointwise ops plus the three reductions (RMSNorm, matmul,
attention), with the KV cache holding exactly the keys/values the attention of
later tokens reads.  Every op's output is rounded to bf16 (the model's storage
type) before the next op reads it; accumulation inside each op is the
oracle's fixed-order fp32.

Layer (pre-norm, no biases):
    h   = rmsnorm(x, attn_norm)
    qkv = h @ Wqkv^T           (q: Hq*D, k: Hkv*D, v: Hkv*D columns)
    q,k = rope(q, pos), rope(k, pos)
    o   = causal attention of q over k, v at positions 0..pos
    x   = x + o @ Wo^T
    h   = rmsnorm(x, mlp_norm)
    g,u = h @ Wgu^T            (gate: F columns, up: F columns)
    x   = x + (silu(g) * u) @ Wdown^T
logits = rmsnorm(x, final_norm) @ Wlm^T
"""
from __future__ import annotations

import numpy as np

from . import BF16, argmax, matmul, rmsnorm, rope, round_to, sdpa, silu_mul, widen
from . import matmul as _matmul
from . import rmsnorm as _rmsnorm
from . import sdpa as _sdpa


def _bf(a32: np.ndarray) -> np.ndarray:
    return round_to(a32, BF16)


def _add(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """bf16 + bf16 -> fp32 add -> bf16."""
    return _bf(widen(a, BF16) + widen(b, BF16))


def forward(weights: dict, cfg: dict, tokens: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray,
            descending: bool = False):
    """Teacher-forced forward of one sequence `tokens` [T] at positions 0..T-1.
    Returns (logits fp32 [T, V], logits bf16 bits [T, V], greedy ids [T]).
    descending=True folds every reduction -- matmul over k, the RMSNorm sum of
    squares, attention's dot products and its sums over keys -- in descending
    order: a second valid fixed-order model, whose distance from the ascending
    one measures how far two correct trees drift apart through the composed
    layers."""
    H, Hq, Hkv, D, F = cfg["hidden"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"]
    eps = cfg["eps"]

    def matmul(a, w, dt, tr):
        return _matmul(a, w, dt, tr, descending=descending)

    def rmsnorm(a, w, dt, e):
        return _rmsnorm(a, w, dt, e, descending=descending)

    def sdpa(q, k, v, kv, sc, causal, dt):
        return _sdpa(q, k, v, kv, sc, causal, dt, descending=descending)

    tokens = np.asarray(tokens, np.int64)
    T = tokens.shape[0]
    pos = np.arange(T, dtype=np.int32)
    x = np.ascontiguousarray(weights["embed"][tokens])                      # [T, H] bf16
    qn, kn = Hq * D, Hkv * D
    for L in weights["layers"]:
        h = _bf(rmsnorm(x, L["attn_norm"], BF16, eps))
        qkv = _bf(matmul(h, L["wqkv"], BF16, True))                       # [T, qn + 2 kn]
        q = _bf(rope(np.ascontiguousarray(qkv[:, :qn].reshape(T, Hq, D)), pos, cos_t, sin_t, BF16))
        k = _bf(rope(np.ascontiguousarray(qkv[:, qn:qn + kn].reshape(T, Hkv, D)), pos, cos_t, sin_t, BF16))
        v = np.ascontiguousarray(qkv[:, qn + kn:].reshape(T, Hkv, D))
        o = _bf(sdpa(q[None], k[None], v[None], np.array([T], np.int32), 1.0 / np.sqrt(D), True, BF16))
        x = _add(x, _bf(matmul(np.ascontiguousarray(o.reshape(T, qn)), L["wo"], BF16, True)))
        h = _bf(rmsnorm(x, L["mlp_norm"], BF16, eps))
        gu = _bf(matmul(h, L["wgu"], BF16, True))                          # [T, 2F]
        a = _bf(silu_mul(np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]), BF16))
        x = _add(x, _bf(matmul(a, L["wdown"], BF16, True)))
    h = _bf(rmsnorm(x, weights["final_norm"], BF16, eps))
    logits = matmul(h, weights["lm_head"], BF16, True)
    lb = _bf(logits)
    return logits, lb, argmax(lb, BF16)


def decode_step(weights: dict, cfg: dict, ids: np.ndarray, kcache: list, vcache: list, kv_len: np.ndarray,
                cos_t: np.ndarray, sin_t: np.ndarray):
    """One greedy decode step for B sequences, one new token each: token b sits
    at position kv_len[b] - 1; its rotated key and its value are written into
    the per-layer caches kcache[l], vcache[l] ([B, Lcap, Hkv, D] bf16 bits)
    before attention reads them.  Returns (logits fp32 [B, V], greedy ids [B])."""
    H, Hq, Hkv, D, F = cfg["hidden"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"]
    eps = cfg["eps"]
    B = ids.shape[0]
    pos = (np.asarray(kv_len, np.int32) - 1).astype(np.int32)
    qn, kn = Hq * D, Hkv * D
    x = np.ascontiguousarray(weights["embed"][np.asarray(ids, np.int64)])
    for li, L in enumerate(weights["layers"]):
        h = _bf(rmsnorm(x, L["attn_norm"], BF16, eps))
        qkv = _bf(matmul(h, L["wqkv"], BF16, True))
        q = _bf(rope(np.ascontiguousarray(qkv[:, :qn].reshape(B, Hq, D)), pos, cos_t, sin_t, BF16))
        k = _bf(rope(np.ascontiguousarray(qkv[:, qn:qn + kn].reshape(B, Hkv, D)), pos, cos_t, sin_t, BF16))
        v = qkv[:, qn + kn:].reshape(B, Hkv, D)
        for b in range(B):
            kcache[li][b, pos[b]] = k[b]
            vcache[li][b, pos[b]] = v[b]
        o = _bf(sdpa(q[:, None], kcache[li], vcache[li], kv_len, 1.0 / np.sqrt(D), True, BF16))
        x = _add(x, _bf(matmul(np.ascontiguousarray(o.reshape(B, qn)), L["wo"], BF16, True)))
        h = _bf(rmsnorm(x, L["mlp_norm"], BF16, eps))
        gu = _bf(matmul(h, L["wgu"], BF16, True))
        a = _bf(silu_mul(np.ascontiguousarray(gu[:, :F]), np.ascontiguousarray(gu[:, F:]), BF16))
        x = _add(x, _bf(matmul(a, L["wdown"], BF16, True)))
    h = _bf(rmsnorm(x, weights["final_norm"], BF16, eps))
    logits = matmul(h, weights["lm_head"], BF16, True)
    return logits, argmax(_bf(logits), BF16)
