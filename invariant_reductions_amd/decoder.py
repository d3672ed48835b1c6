"""Llama-style decoder built from the batch-invariant ops: greedy decoding,
plain and speculative.

Sources: "Batch-invariant kernels: why temperature-0 decoding is still
nondeterministic" (Thesis and Mental model: make RMSNorm, matmul and attention
batch-invariant and greedy decoding stops depending on the batch; Case 5: the
load-dependent greedy token; Case 6: KV cache written before attention) and
"Fix/speculative shape invariance" (Problem: a token evaluated alone and the
same token inside a verification block must produce identical results).

Model (pre-norm, no biases, bf16 storage between ops):
    h   = rmsnorm(x, attn_norm);  qkv = h @ Wqkv^T
    q,k = rope(q, k at their positions); k, v written to the cache
    o   = causal attention over the cache;  x = x + o @ Wo^T
    h   = rmsnorm(x, mlp_norm);   g|u = h @ Wgu^T
    x   = x + (silu(g) * u) @ Wdown^T
logits = rmsnorm(x, final_norm) @ Wlm^T; next token = argmax (lowest index on ties)

Every op is one or two launches of the C ABI on torch's current stream; all
buffers are allocated once, so a decode step allocates nothing.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (W_PACKED, add_rmsnorm, argmax, embed_rmsnorm, interleave_gate_up, lib, matmul_swiglu, matmul_ws,
               pack_weights, rope_kv_write, sdpa, sdpa_workspace_bytes)
from .inputs import rope_tables


def _dev16(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


class Decoder:
    def __init__(self, cfg: dict, weights: dict, max_batch: int, max_q: int, max_len: int, device="cuda:0"):
        self.cfg = cfg
        self.dev = torch.device(device)
        c = cfg
        self.H, self.Hq, self.Hkv, self.D = c["hidden"], c["n_heads"], c["n_kv_heads"], c["head_dim"]
        self.F, self.V, self.L = c["ffn"], c["vocab"], c["n_layers"]
        self.eps = float(c["eps"])
        self.qn = self.Hq * self.D
        self.qkvn = (self.Hq + 2 * self.Hkv) * self.D
        d = self.dev
        W = weights
        self.embed_w = _dev16(W["embed"], d)
        self.layers = [{k: _dev16(v, d) for k, v in lw.items()} for lw in W["layers"]]
        # Projection weights are kept tile-packed (pack_weights: same bits,
        # fewer DRAM pages per byte streamed); the gate/up weight [Wg; Wu] is
        # first interleaved in blocks of 8 rows, the layout the fused
        # projection + SwiGLU kernel reads.
        for lw in self.layers:
            wgu = lw.pop("wgu")
            lw["wgu_il"] = pack_weights(interleave_gate_up(wgu[:self.F], wgu[self.F:]))
            del wgu
            for k in ("wqkv", "wo", "wdown"):
                lw[k] = pack_weights(lw[k])
        self.final_norm = _dev16(W["final_norm"], d)
        self.lm_head = pack_weights(_dev16(W["lm_head"], d))
        cos_t, sin_t = rope_tables(max_len, self.D, c.get("rope_theta", 10000.0))
        self.cos_t = torch.from_numpy(cos_t).to(d)
        self.sin_t = torch.from_numpy(sin_t).to(d)
        self.max_batch, self.max_q, self.max_len = max_batch, max_q, max_len
        T = max_batch * max_q
        bf = torch.bfloat16
        z = lambda *s: torch.zeros(*s, dtype=bf, device=d)
        # head-major KV caches [B, Hkv, Lcap, D]: each head's keys contiguous
        self.kc = [z(max_batch, self.Hkv, max_len, self.D) for _ in range(self.L)]
        self.vc = [z(max_batch, self.Hkv, max_len, self.D) for _ in range(self.L)]
        self.x, self.h, self.t1 = z(T, self.H), z(T, self.H), z(T, self.H)
        self.qkv, self.q, self.o = z(T, self.qkvn), z(T, self.qn), z(T, self.qn)
        self.a = z(T, self.F)
        self.logits = z(T, self.V)
        self.ids = torch.zeros(T, dtype=torch.int32, device=d)
        self.next_ids = torch.zeros(T, dtype=torch.int32, device=d)
        self.kv_len = torch.zeros(max_batch, dtype=torch.int32, device=d)
        ws = sdpa_workspace_bytes(max_batch, max_q, max_len, self.Hq, self.D)
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=d)
        # one zero-filled matmul workspace for every projection (calls are stream-ordered)
        mshapes = [(self.qkvn, self.H), (self.H, self.qn), (2 * self.F, self.H), (self.H, self.F), (self.V, self.H)]
        # (the slot form takes up to 128 rows on the narrow projections, every
        # 64-row chunk with its own group sums: size for the most rows a call has)
        need = max(lib().bi_matmul_ws_workspace_bytes(m, n, k, 0, 1) for n, k in mshapes for m in {min(T, 64), min(T, 128)})
        self.mws = torch.zeros(max(int(need), 16), dtype=torch.uint8, device=d)
        # the fused gate/up + SwiGLU call has its own (its size covers the
        # scratch product of the shapes the fused kernel does not take)
        sneed = max(lib().bi_matmul_swiglu_workspace_bytes(m, self.F, self.H, 0) for m in {min(T, 64), T})
        self.sws = torch.zeros(max(int(sneed), 16), dtype=torch.uint8, device=d)

    # -- one forward over Q new tokens of each of B sequences -----------------
    def forward(self, B: int, Q: int, max_kv: int):
        """Reads self.ids[:B*Q] and self.kv_len[:B] (lengths after the new
        tokens), fills self.logits[:B*Q] and self.next_ids[:B*Q]."""
        T = B * Q
        H, qn = self.H, self.qn
        x, h, t1 = self.x[:T], self.h[:T], self.t1[:T]
        qkv, q, o = self.qkv[:T], self.q[:T], self.o[:T]
        a = self.a[:T]
        kv = self.kv_len[:B]
        scale = 1.0 / float(np.sqrt(self.D))
        # The embedding lookup is fused with the first RMSNorm, and every
        # residual add with the RMSNorm that reads its result (the next
        # block's norm, or the final norm after the last layer).
        embed_rmsnorm(self.ids[:T], self.embed_w, self.layers[0]["attn_norm"], self.eps, x_out=x, out=h)
        for li, Lw in enumerate(self.layers):
            matmul_ws(h, Lw["wqkv"], self.mws, out=qkv)
            kc, vc = self.kc[li][:B], self.vc[li][:B]
            rope_kv_write(qkv, q, kc, vc, kv, self.cos_t, self.sin_t, B, Q, self.Hq, self.Hkv, self.D, head_major=True)
            sdpa(q.view(B, Q, self.Hq, self.D), kc, vc, kv, max_kv, scale, True, head_major=True,
                 out=o.view(B, Q, self.Hq, self.D), ws=self.ws)
            matmul_ws(o, Lw["wo"], self.mws, out=t1)
            add_rmsnorm(x, t1, Lw["mlp_norm"], self.eps, x_out=x, out=h)
            matmul_swiglu(h, Lw["wgu_il"], self.sws, out=a)
            matmul_ws(a, Lw["wdown"], self.mws, out=t1)
            nxt = self.layers[li + 1]["attn_norm"] if li + 1 < self.L else self.final_norm
            add_rmsnorm(x, t1, nxt, self.eps, x_out=x, out=h)
        matmul_ws(h, self.lm_head, self.mws, out=self.logits[:T])
        argmax(self.logits[:T], out=self.next_ids[:T])
        return self.logits[:T]

    # -- launch plans -----------------------------------------------------------------
    def plan(self, B: int, Q: int, max_kv: int, stream=None, advance: bool = False):
        """The forward as a list of (name, C entry point, argument tuple) over the
        fixed buffers, for callers that replay the same step many times (a
        serving loop, the benchmark) without re-marshalling arguments.  The
        device-side ids / kv_len buffers are read at run time, so one plan
        serves every step whose lengths stay within max_kv.  advance (greedy
        decode, Q = 1): the final argmax also writes each token into ids and
        grows kv_len by one, so the plan can be replayed step after step."""
        import ctypes
        from . import lib
        L = lib()
        st = ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        T = B * Q
        H, qn = self.H, self.qn
        x, h, t1 = self.x[:T], self.h[:T], self.t1[:T]
        qkv, q, o = self.qkv[:T], self.q[:T], self.o[:T]
        a = self.a[:T]
        kv = self.kv_len[:B]
        scale = ctypes.c_float(1.0 / float(np.sqrt(self.D)))
        eps = ctypes.c_float(self.eps)
        steps = [("embed_rmsnorm", L.bi_embed_rmsnorm, (p(self.ids), p(self.embed_w), p(x),
                                                         p(self.layers[0]["attn_norm"]), p(h), T, self.V, H, eps, 0,
                                                         st))]
        mws, mwsb = p(self.mws), self.mws.numel()
        mm = lambda xin, w, out, N, K: ("matmul", L.bi_matmul_ws, (p(xin), p(w.data), p(out), T, N, K, 0, W_PACKED, mws,
                                                                    mwsb, st))
        for li, Lw in enumerate(self.layers):
            kc, vc = self.kc[li], self.vc[li]
            Lcap = kc.shape[2]
            nxt = self.layers[li + 1]["attn_norm"] if li + 1 < self.L else self.final_norm
            steps += [
                mm(h, Lw["wqkv"], qkv, self.qkvn, H),
                ("rope_kv", L.bi_rope_kv_write, (p(qkv), p(q), p(kc), p(vc), p(kv), p(self.cos_t), p(self.sin_t),
                                                 B, Q, Lcap, self.Hq, self.Hkv, self.D, self.cos_t.shape[0], 1, st)),
                ("sdpa", L.bi_sdpa, (p(q), p(kc), p(vc), p(o), p(kv), max_kv, B, Q, Lcap, self.Hq, self.Hkv,
                                     self.D, scale, 1, 0, 1, p(self.ws), self.ws.numel(), st)),
                mm(o, Lw["wo"], t1, H, qn),
                ("add_rmsnorm", L.bi_add_rmsnorm, (p(x), p(t1), p(x), p(Lw["mlp_norm"]), p(h), T, H, eps, 0, st)),
                ("matmul_swiglu", L.bi_matmul_swiglu, (p(h), p(Lw["wgu_il"].data), p(a), T, self.F, H, 0, W_PACKED,
                                                       p(self.sws), self.sws.numel(), st)),
                mm(a, Lw["wdown"], t1, H, self.F),
                ("add_rmsnorm", L.bi_add_rmsnorm, (p(x), p(t1), p(x), p(nxt), p(h), T, H, eps, 0, st)),
            ]
        steps += [mm(h, self.lm_head, self.logits, self.V, H),
                  ("argmax", L.bi_argmax, (p(self.logits), p(self.next_ids), T, self.V, st)) if not advance else
                  ("argmax", L.bi_argmax_advance, (p(self.logits), p(self.next_ids), p(self.ids), p(kv), T, self.V, st))]
        if advance and Q != 1:
            raise ValueError("plan(advance=True) is the one-token greedy step (Q = 1)")
        return steps

    @staticmethod
    def run_plan(plan):
        for name, fn, args in plan:
            rc = fn(*args)
            if rc != 0:
                from . import BIError
                raise BIError(rc, name)

    # -- greedy decoding ----------------------------------------------------------
    def prefill(self, prompts: torch.Tensor):
        """prompts int32 [B, P] on the device; returns the first generated ids [B] (host)."""
        B, P = prompts.shape
        assert B <= self.max_batch and P <= self.max_q and P < self.max_len
        self.ids[:B * P].copy_(prompts.reshape(-1))
        self.kv_len[:B].fill_(P)
        self.forward(B, P, P)
        return self.next_ids[:B * P].view(B, P)[:, -1].cpu().numpy().copy(), \
            self.logits[:B * P].view(B, P, self.V)[:, -1]

    def generate(self, prompts: torch.Tensor, steps: int, on_logits=None):
        """Plain greedy decoding: one token per sequence per step.
        on_logits(i, logits [B, V]) sees the logits that chose generated token i.
        Returns the generated ids [B, steps] (host int32)."""
        B, P = prompts.shape
        assert P + steps <= self.max_len
        first, lg = self.prefill(prompts)
        if on_logits:
            on_logits(0, lg)
        out = np.zeros((B, steps), np.int32)
        out[:, 0] = first
        self.ids[:B].copy_(torch.from_numpy(first).to(self.dev))
        for t in range(1, steps):
            self.kv_len[:B].fill_(P + t)
            lg = self.forward(B, 1, P + t)
            if on_logits:
                on_logits(t, lg)
            self.ids[:B].copy_(self.next_ids[:B])
            out[:, t] = self.next_ids[:B].cpu().numpy()
        return out

    def teacher_forced(self, prompts: torch.Tensor, cont: np.ndarray, on_logits):
        """Score a fixed continuation: prefill the prompts [B, P], then feed
        cont [B, S] one token per step through the decode path (Q = 1, reading
        the growing cache), as greedy decoding would feed its own tokens.
        on_logits(p, logits [B, V]) sees the logits at every position p =
        0 .. P + S - 1 (the prefill's rows first)."""
        B, P = prompts.shape
        S = cont.shape[1]
        assert P + S <= self.max_len
        self.prefill(prompts)
        lg = self.logits[:B * P].view(B, P, self.V)
        for p in range(P):
            on_logits(p, lg[:, p])
        for t in range(S):
            self.ids[:B].copy_(torch.from_numpy(np.ascontiguousarray(cont[:, t], np.int32)).to(self.dev))
            self.kv_len[:B].fill_(P + t + 1)
            on_logits(P + t, self.forward(B, 1, P + t + 1))

    def generate_speculative(self, prompts: torch.Tensor, steps: int, draft, draft_len: int = 4, on_logits=None):
        """Greedy speculative decoding: each round verifies the last committed
        token plus `draft_len` drafted tokens in one causal block (Q =
        draft_len + 1), accepts the longest prefix of drafts the model agrees
        with, and takes the model's own token after it.  Sequences advance at
        their own pace; each keeps its own KV length, and the cache slots of
        rejected drafts are overwritten by the next round.
        draft(b, i, n) -> n proposed ids for generated positions i, i+1, ...
        on_logits(b, i, logits [V]) sees the logits that chose generated token i
        of sequence b."""
        B, P = prompts.shape
        Q = draft_len + 1
        assert Q <= self.max_q and P + steps + Q <= self.max_len
        first, lg = self.prefill(prompts)
        out = np.zeros((B, steps), np.int32)
        out[:, 0] = first
        if on_logits:
            for b in range(B):
                on_logits(b, 0, lg[b])
        done = np.ones(B, np.int64)                  # generated tokens committed per sequence
        rounds = 0
        while (done < steps).any():
            ids = np.zeros((B, Q), np.int32)
            kvl = np.zeros(B, np.int32)
            for b in range(B):
                n = int(min(done[b], steps))         # finished sequences re-verify their last block
                ids[b, 0] = out[b, n - 1]
                ids[b, 1:] = draft(b, n, draft_len)
                kvl[b] = P + n - 1 + Q                # block occupies positions P+n-1 .. P+n-1+draft_len
            self.ids[:B * Q].copy_(torch.from_numpy(ids.reshape(-1)).to(self.dev))
            self.kv_len[:B].copy_(torch.from_numpy(kvl).to(self.dev))
            lgs = self.forward(B, Q, int(kvl.max())).view(B, Q, self.V)
            tgt = self.next_ids[:B * Q].view(B, Q).cpu().numpy()
            for b in range(B):
                n = int(done[b])
                if n >= steps:
                    continue
                a = 0
                while a < draft_len and ids[b, 1 + a] == tgt[b, a]:
                    a += 1
                new = list(ids[b, 1:1 + a]) + [tgt[b, a]]
                for j, tok in enumerate(new):
                    if n + j >= steps:
                        break
                    out[b, n + j] = tok
                    if on_logits:
                        on_logits(b, n + j, lgs[b, j])
                done[b] = n + len(new)
            rounds += 1
        self.rounds = rounds
        return out
