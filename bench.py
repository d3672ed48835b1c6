"""Benchmark of the batch-invariant hot path on one MI355X.

One step = one greedy decode step of the 4-layer Llama-style decoder (hidden
4096, 32 query / 8 KV heads, head_dim 128, SwiGLU 14336, vocab 32000, bf16,
random init) for B sequences at a context of `--ctx` tokens: embedding,
4 x (RMSNorm, QKV matmul, RoPE + KV-cache write, two-pass attention, O
matmul, residual add, RMSNorm, gate/up matmul with the SiLU*mul activation,
down matmul, residual add), final RMSNorm, LM-head matmul, argmax -- every reduction
through the invariant kernels.  Inputs (weights, KV cache, token ids) are
seeded synthetic data resident in HBM before timing starts.

Printed (one JSON line): whole-step algorithmic throughput in GB/s, the
roofline of the dominant kernel (the dense matmul) timed live with HIP events
on the launch stream, and the CPU oracle timed on a bounded sample of the
same step.  Extra fields: per-op breakdown, the quantized matmul at a decode
shape, and the cost of invariance against split-K comparison variants.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "invariant matmul/SDPA/RMSNorm GB/s & TFLOP/s, % roofline, M=1..64"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_TFLOPS = 2500.0        # dense bf16 MFMA, published


def step_traffic(cfg, B, ctx):
    """Algorithmic bytes and flops of one decode step (each tensor read or
    written once, at its storage size)."""
    H, Hq, Hkv, D, F, V, L = (cfg[k] for k in ("hidden", "n_heads", "n_kv_heads", "head_dim", "ffn", "vocab", "n_layers"))
    qkvn = (Hq + 2 * Hkv) * D
    # (M, N, K, columns stored) of every matmul launch; the gate/up product
    # stores only its SwiGLU activation (F columns), fused into the matmul
    mm = []
    for _ in range(L):
        mm += [(B, qkvn, H, qkvn), (B, H, Hq * D, H), (B, 2 * F, H, F), (B, H, F, H)]
    mm.append((B, V, H, V))
    mm_bytes = sum(2 * (N * K + M * K + M * O) for M, N, K, O in mm)
    swiglu_bytes = L * 2 * (2 * F * H + B * H + B * F)
    mm_flops = sum(2 * M * N * K for M, N, K, _ in mm)
    # one plain RMSNorm (x -> h), then 2L residual adds fused with the norm that
    # follows them (x, r -> x, h)
    norm_bytes = (4 * B * H + 2 * H) + 2 * L * (8 * B * H + 2 * H)
    attn_bytes = L * (4 * B * ctx * Hkv * D + 4 * B * Hq * D)
    attn_flops = L * 4 * B * Hq * D * ctx
    glue_bytes = (2 * B * H * 2                              # embed
                  + L * (2 * B * qkvn + 2 * B * Hq * D + 4 * B * Hkv * D)   # rope + cache write
                  + 2 * B * V)                               # argmax
    return dict(mm=mm, mm_bytes=mm_bytes, swiglu_bytes=swiglu_bytes, mm_flops=mm_flops, norm_bytes=norm_bytes,
                attn_bytes=attn_bytes, attn_flops=attn_flops, glue_bytes=glue_bytes,
                total_bytes=mm_bytes + norm_bytes + attn_bytes + glue_bytes, total_flops=mm_flops + attn_flops)


def measured_traffic():
    """HBM bytes per matmul launch from the committed counter runs
    (profiles/dense_slots_kernel_decode_b64_traffic.json), or None when the
    dense kernel sources it lists have changed since those counters were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "dense_slots_kernel_decode_b64_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for src in rec["sources"]:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest()[:16] != rec["source_sha256_16"]:
            return None
        return float(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(W, cfg, B, ctx, kc_host, vc_host, ids, budget_s):
    """The oracle's decode step on the host, repeated until `budget_s` seconds
    have passed (at least one step, at most sixteen)."""
    import oracle
    from oracle import decoder as odec
    from invariant_reductions_amd.inputs import rope_tables
    cos_t, sin_t = rope_tables(ctx + 8, cfg["head_dim"])
    kv = np.full(B, ctx, np.int32)
    t0 = time.perf_counter()
    n = 0
    while n < 16:
        odec.decode_step(W, cfg, ids, kc_host, vc_host, kv, cos_t, sin_t)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return n, time.perf_counter() - t0, oracle.num_threads()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=768)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the batch-invariant hot path is a single-GPU kernel set "
              "(multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_reductions_amd as bi
    from invariant_reductions_amd import inputs
    from invariant_reductions_amd.decoder import Decoder

    cfg = inputs.LLAMA_4L
    B, ctx, K, Wm = args.batch, args.ctx, args.steps, args.warmup
    dev = torch.device("cuda:0")
    bi.lib()
    t_setup = time.perf_counter()
    W = inputs.decoder_weights(cfg, seed=0)
    cap = ctx + 2 * K + Wm + 8
    model = Decoder(cfg, W, max_batch=B, max_q=1, max_len=cap, device=dev)
    rng = np.random.default_rng(1)
    Hkv, D = cfg["n_kv_heads"], cfg["head_dim"]
    kc_host, vc_host = [], []
    for li in range(cfg["n_layers"]):
        kh = inputs.normal(rng, (B, cap, Hkv, D))
        vh = inputs.normal(rng, (B, cap, Hkv, D))
        # the decoder keeps its caches head-major [B, Hkv, cap, D]
        model.kc[li].copy_(torch.from_numpy(kh.view(np.int16)).view(torch.bfloat16).transpose(1, 2))
        model.vc[li].copy_(torch.from_numpy(vh.view(np.int16)).view(torch.bfloat16).transpose(1, 2))
        kc_host.append(kh)
        vc_host.append(vh)
    ids0 = rng.integers(0, cfg["vocab"], size=B).astype(np.int32)
    model.ids[:B].copy_(torch.from_numpy(ids0))
    model.kv_len[:B].fill_(ctx)
    stream = torch.cuda.current_stream()
    # A plain 256 MiB device-to-device copy: counter runs of this command
    # (FETCH_SIZE, WRITE_SIZE) read it to scale the counters to bytes.
    calib = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    calib.fill_(1.0)
    calib2 = torch.empty_like(calib)
    calib2.copy_(calib)
    del calib, calib2
    # the step's last launch (argmax) also feeds its tokens back as the next
    # step's ids and grows kv_len: the plan is replayed as is, step after step
    plan = model.plan(B, 1, cap, stream, advance=True)
    MM_OPS = ("matmul", "matmul_swiglu")
    mm_idx = [i for i, s in enumerate(plan) if s[0] in MM_OPS]
    # (N, K) of each matmul launch (the fused gate/up call passes F = N / 2)
    mm_shape = [(plan[i][2][4] * (2 if plan[i][0] == "matmul_swiglu" else 1), plan[i][2][5]) for i in mm_idx]
    mm_out = {(plan[i][2][4] * 2, plan[i][2][5]) if plan[i][0] == "matmul_swiglu" else (plan[i][2][4], plan[i][2][5]):
              plan[i][2][4] for i in mm_idx}                                  # columns stored per shape
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    for _ in range(Wm):
        model.run_plan(plan)
    # Timed region: K whole steps, nothing but the step's own launches (a HIP
    # event record costs several microseconds of idle GPU time, so none is
    # placed between the kernels here).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        model.run_plan(plan)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K

    # Roofline pass, right after: the same K steps again (the cache keeps
    # growing as in the timed region).  Every matmul launch carries a pair of
    # HIP events on its stream that the launch itself records as the kernel
    # starts and ends (bi_time_next_launch -> hipExtLaunchKernel), i.e. the
    # kernel's own duration, as a kernel trace reports it.
    L = bi.lib()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K * len(mm_idx))]
    for s_, t_ in ev:                          # create the event handles
        s_.record(stream)
        t_.record(stream)
    torch.cuda.synchronize()
    e = 0
    for _ in range(K):
        for i, (name, fn, a) in enumerate(plan):
            if name in MM_OPS:
                L.bi_time_next_launch(ctypes.c_void_p(ev[e][0].cuda_event), ctypes.c_void_p(ev[e][1].cuda_event))
                rc = fn(*a)
                e += 1
            else:
                rc = fn(*a)
            if rc != 0:
                raise bi.BIError(rc, name)
    torch.cuda.synchronize()
    durs = [s.elapsed_time(t) for s, t in ev]
    mm_ms = sum(durs)
    per_shape = {}
    for j, d in enumerate(durs):
        per_shape.setdefault(mm_shape[j % len(mm_idx)], []).append(d)

    ctx_mean = ctx + Wm + (K - 1) / 2.0                     # mean context over the timed steps
    tr = step_traffic(cfg, B, ctx_mean)
    value = tr["total_bytes"] / (ms_step * 1e-3) / 1e9
    mm_gbs = tr["mm_bytes"] * K / (mm_ms * 1e-3) / 1e9
    mm_avg_us = mm_ms * 1e3 / (K * len(mm_idx))

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: random-init weights N(0,0.02), KV cache and token ids N(0,1)/uniform, seeded",
        "config": {"workload": f"greedy decode step, 4-layer Llama-style decoder (hidden 4096, 32q/8kv heads, "
                               f"d128, SwiGLU 14336, vocab 32000), batch {B}, context {ctx}",
                   "batch": B, "context": ctx, "layers": cfg["n_layers"]},
        "tflops": round(tr["total_flops"] / (ms_step * 1e-3) / 1e12, 3),
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "roofline": {"kernel": "bi_matmul_ws / bi_matmul_swiglu -> dense_slots_kernel<bf16, MT, Q, EPI> (every "
                               "instantiation the step launches; achieved = all matmul algorithmic bytes / all "
                               "matmul launch time)",
                     "bound": "hbm",
                     "achieved": round(mm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(mm_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "traffic_unit": "bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE, B=64 ctx 768 step mix)",
                     "algorithmic_bytes_per_launch": round(tr["mm_bytes"] / len(mm_idx)),
                     "launches_per_step": len(mm_idx), "avg_launch_us": round(mm_avg_us, 2),
                     "share_of_step": round(mm_ms / K / ms_step, 3),
                     "per_shape": {f"{B}x{N}x{Kk}": {"us": round(1e3 * np.mean(v), 1),
                                                     "gbs": round(2 * (N * Kk + B * Kk + B * mm_out[(N, Kk)])
                                                                  / (np.mean(v) * 1e-3) / 1e9, 1)}
                                   for (N, Kk), v in per_shape.items()}},
        "setup_s": round(setup_s, 1),
    }

    if not args.no_extras:
        out["ops"] = op_breakdown(model, plan, stream, B, ctx_mean, cfg, torch)
        out["invariance_overhead"] = split_overhead(torch, bi, model, B, per_shape)
        out["qmatmul"] = qmatmul_decode(torch, bi, dev)
        out["row_ops"] = row_ops(torch, bi, model, B)
        out["sweep"] = op_sweep(torch, bi, dev)

    if not args.no_cpu_baseline:
        n, secs, cores = cpu_baseline(W, cfg, B, ctx, kc_host, vc_host, ids0, args.cpu_budget)
        trc = step_traffic(cfg, B, ctx)
        out["cpu_baseline"] = {"value": round(trc["total_bytes"] * n / secs / 1e9, 3), "unit": "GB/s",
                               "cores": cores, "kind": "oracle",
                               "sample": f"{n} decode step(s) of the same workload (batch {B}, context {ctx}) "
                                         f"through the oracle's fixed-order fp32 ops, {secs:.1f} s"}
    print(json.dumps(out), flush=True)


def op_breakdown(model, plan, stream, B, ctx_mean, cfg, torch):
    """Per-op device time of one step (HIP events around every launch, 5 steps)."""
    reps = 5
    evs = []
    for _ in range(reps):
        row = []
        for name, fn, a in plan:
            s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn(*a)
            t.record(stream)
            row.append((name, s, t))
        evs.append(row)
    torch.cuda.synchronize()
    tot = {}
    for row in evs:
        for name, s, t in row:
            tot[name] = tot.get(name, 0.0) + s.elapsed_time(t) / reps
    tr = step_traffic(cfg, B, ctx_mean)
    H, L = cfg["hidden"], cfg["n_layers"]
    bytes_of = {"matmul": tr["mm_bytes"] - tr["swiglu_bytes"], "matmul_swiglu": tr["swiglu_bytes"],
                "sdpa": tr["attn_bytes"], "rmsnorm": 4 * B * H + 2 * H,
                "add_rmsnorm": 2 * L * (8 * B * H + 2 * H)}
    res = {}
    for name, ms in tot.items():
        r = {"us_per_step": round(ms * 1e3, 1)}
        if name in bytes_of:
            gbs = bytes_of[name] / (ms * 1e-3) / 1e9
            r.update(gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
        res[name] = r
    return res


def _time(torch, fn, reps=20):
    s, t = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    t.record()
    torch.cuda.synchronize()
    return s.elapsed_time(t) / reps


def split_overhead(torch, bi, model, B, per_shape):
    """Invariant dense matmul (its launches inside the timed decode steps) vs the
    fastest split-K comparison variant at the same shapes, on the decoder's own
    weights, rotating over the layers so the weights are as cold as in a step."""
    dev = model.dev
    res = {}
    mats = {(model.qkvn, model.H): [L["wqkv"] for L in model.layers], (model.H, model.qn): [L["wo"] for L in model.layers],
            (2 * model.F, model.H): [L["wgu_il"] for L in model.layers], (model.H, model.F): [L["wdown"] for L in model.layers],
            (model.V, model.H): [model.lm_head]}
    for (N, K), ws_list in mats.items():
        x = torch.randn(B, K, device=dev).to(torch.bfloat16)
        y = torch.empty(B, N, dtype=torch.bfloat16, device=dev)
        t_inv = float(np.mean(per_shape[(N, K)]))
        best = None
        for s in (2, 4, 8, 16):
            ws = torch.empty(B * N * s * 4, dtype=torch.uint8, device=dev)
            it = iter(range(1 << 30))
            t = _time(torch, lambda: bi.matmul_split(x, ws_list[next(it) % len(ws_list)], s, True, out=y, ws=ws))
            if best is None or t < best[1]:
                best = (s, t)
        res[f"{B}x{N}x{K}"] = {"invariant_us": round(t_inv * 1e3, 1), "best_split": best[0],
                               "split_us": round(best[1] * 1e3, 1), "overhead": round(t_inv / best[1] - 1, 3)}
    return res


def _time_kernel(torch, bi, fn, reps, launches=1):
    """Mean execution time (ms) of the `launches` bi kernels `fn` launches: a
    start/stop event pair recorded by the launches themselves
    (bi_time_next_launches), so host-side launch overhead is not counted."""
    L = bi.lib()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s_, t_ in ev:
        s_.record()
        t_.record()
    fn(0)
    torch.cuda.synchronize()
    for i, (s_, t_) in enumerate(ev):
        L.bi_time_next_launches(ctypes.c_void_p(s_.cuda_event), ctypes.c_void_p(t_.cuda_event), launches)
        fn(i)
    torch.cuda.synchronize()
    return float(np.mean([s_.elapsed_time(t_) for s_, t_ in ev]))


def op_sweep(torch, bi, dev):
    """The four reductions at the measurement shapes, cold (rotated copies of
    the streamed operand, at least 512 MiB in all), kernel time:
      dense (packed weights): the pages' 4096 x 4096 and the decoder's
        projections at M in 1..64;
      RMSNorm: H = 4096 at B in {1, 8, 64, 512, 4096};
      SDPA (two launches: chunks and merge): B = 1, Q in {1, 8} at
        Lk in {1028, 8196, 16388, 65540}, and B in {4, 16, 64} at Q = 1,
        Lk = 8196."""
    res = {"matmul": {}, "rmsnorm": {}, "sdpa": {}}
    bf = torch.bfloat16
    for (N, K) in ((4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336), (32000, 4096)):
        copies = max(2, -(-(512 << 20) // (N * K * 2)))
        wps = [bi.pack_weights((torch.randn(N, K, device=dev) * 0.02).to(bf)) for _ in range(copies)]
        ws = bi.matmul_workspace(64, N, K, device=dev)
        for M in (1, 2, 4, 8, 16, 32, 64):
            x = torch.randn(M, K, device=dev).to(bf)
            y = torch.empty(M, N, dtype=bf, device=dev)
            t = _time_kernel(torch, bi, lambda i: bi.matmul_ws(x, wps[i % copies], ws, out=y), reps=3 * copies)
            gbs = 2 * (N * K + M * K + M * N) / (t * 1e-3) / 1e9
            res["matmul"][f"{M}x{N}x{K}"] = {"us": round(t * 1e3, 2), "gbs": round(gbs, 1),
                                             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del wps
    H = 4096
    w = torch.ones(H, dtype=bf, device=dev)
    for Bn in (1, 8, 64, 512, 4096):
        copies = max(2, min(64, -(-(512 << 20) // (Bn * H * 2))))
        xs = [torch.randn(Bn, H, device=dev).to(bf) for _ in range(copies)]
        y = torch.empty(Bn, H, dtype=bf, device=dev)
        t = _time_kernel(torch, bi, lambda i: bi.rmsnorm(xs[i % copies], w, out=y), reps=3 * copies)
        gbs = (4 * Bn * H + 2 * H) / (t * 1e-3) / 1e9
        res["rmsnorm"][f"{Bn}x{H}"] = {"us": round(t * 1e3, 2), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del xs
    Hq, Hkv, D = 32, 8, 128
    cases = [(1, Q, Lk) for Lk in (1028, 8196, 16388, 65540) for Q in (1, 8)] + [(Bn, 1, 8196) for Bn in (4, 16, 64)]
    for Bn, Q, Lk in cases:
        kvb = 4 * Bn * Lk * Hkv * D
        copies = max(2, min(16, -(-(512 << 20) // kvb)))
        ks = [torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf) for _ in range(copies)]
        vs = [torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf) for _ in range(copies)]
        q = torch.randn(Bn, Q, Hq, D, device=dev).to(bf)
        kv = torch.full((Bn,), Lk, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        wsd = torch.empty(bi.sdpa_workspace_bytes(Bn, Q, Lk, Hq, D), dtype=torch.uint8, device=dev)
        t = _time_kernel(torch, bi, lambda i: bi.sdpa(q, ks[i % copies], vs[i % copies], kv, Lk, 0.088, True, out=o,
                                                      ws=wsd, head_major=True), reps=3 * copies, launches=2)
        gbs = (kvb + 4 * Bn * Q * Hq * D) / (t * 1e-3) / 1e9
        res["sdpa"][f"B{Bn} Q{Q} Lk{Lk}"] = {"us": round(t * 1e3, 2), "gbs": round(gbs, 1),
                                              "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del ks, vs
    # causal prefill: Q = Lk (a whole prompt in one call), flops over the visible (query, key) pairs
    res["prefill"] = {}
    for Bn, Q in ((1, 512), (1, 2048), (8, 512), (64, 512)):
        Lk = Q
        ks = torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf)
        vs = torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf)
        q = torch.randn(Bn, Q, Hq, D, device=dev).to(bf)
        kv = torch.full((Bn,), Lk, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        wsd = torch.empty(bi.sdpa_workspace_bytes(Bn, Q, Lk, Hq, D), dtype=torch.uint8, device=dev)
        t = _time_kernel(torch, bi, lambda i: bi.sdpa(q, ks, vs, kv, Lk, 0.088, True, out=o, ws=wsd, head_major=True),
                         reps=5, launches=2)
        pairs = Q * (Q + 1) // 2
        tf = 4 * Bn * Hq * D * pairs / (t * 1e-3) / 1e12
        res["prefill"][f"B{Bn} Q{Q} Lk{Lk} causal"] = {"us": round(t * 1e3, 2), "tflops": round(tf, 2),
                                                       "frac_mfma": round(tf / 2500.0, 4)}
        del ks, vs, wsd
    torch.cuda.empty_cache()
    return res


def row_ops(torch, bi, model, B):
    """Log-softmax, token log-probabilities and row mean over the step's own
    logits [B, vocab] bf16 (kernel time, launch-recorded events)."""
    x = model.logits[:B]
    ids = model.next_ids[:B]
    y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    lp = torch.empty(B, dtype=torch.float32, device=x.device)
    res = {}
    V = x.shape[1]
    for name, fn, nbytes in (("log_softmax", lambda i: bi.log_softmax(x, out=y), 2 * B * V + 4 * B * V),
                             ("token_logprob", lambda i: bi.token_logprob(x, ids, out=lp), 2 * B * V + 8 * B),
                             ("row_mean", lambda i: bi.row_mean(x, out=lp), 2 * B * V + 4 * B)):
        t = _time_kernel(torch, bi, fn, reps=50)
        gbs = nbytes / (t * 1e-3) / 1e9
        res[f"{name} {B}x{V}"] = {"us": round(t * 1e3, 2), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def qmatmul_decode(torch, bi, dev):
    """Quantized matmul at decode shapes (M = 8; K = N = 4096 and the MLP
    shape 28672 x 4096), cold: the seeded quantized weight plus bit-permuted
    copies (distinct bytes, same sizes) rotated so no launch finds its weight
    in a cache.  Transposed [N, K*bits/32] weights and the tile-packed
    layout; kernel execution time (launch-recorded events)."""
    from invariant_reductions_amd import inputs
    res = {}
    for mode, gs, bits in (("affine", 64, 4), ("nvfp4", 16, 4), ("mxfp4", 32, 4),
                           ("affine", 64, 3), ("affine", 64, 8), ("mxfp8", 32, 8)):
        for (N, K) in ((4096, 4096), (28672, 4096)):
            M = 8
            x, wq, s, b = inputs.qmatmul_case(M, K, N, mode, gs, True, seed=0, bits=bits)
            xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.float16)
            wq0 = torch.from_numpy(wq.view(np.int32)).to(dev)
            sd = torch.from_numpy(s if s.dtype == np.uint8 else s.view(np.int16)).to(dev)
            bd = None if b is None else torch.from_numpy(b.view(np.int16)).to(dev)
            copies = max(2, int(0.8e9 // (N * K * bits // 8)))
            wqs = [wq0] + [torch.bitwise_xor(wq0, (0x01010101 * r) & 0x7fffffff) for r in range(1, copies)]
            qm = {"affine": bi.AFFINE, "nvfp4": bi.NVFP4, "mxfp4": bi.MXFP4, "mxfp8": bi.MXFP8}[mode]
            y = torch.empty(M, N, dtype=torch.float16, device=dev)
            wbytes = N * K * bits // 8 + N * (K // gs) * (4 if mode == "affine" else 1)
            tot = wbytes + 2 * M * K + 2 * M * N
            runs = [("transposed", lambda r: bi.qmatmul(xd, wqs[r], sd, bd, N, K, qm, gs, True, out=y, bits=bits))]
            wps = [bi.pack_qweights(w, sd, bd, N, K, qm, gs, bits=bits) for w in wqs]
            runs.append(("packed", lambda r: bi.qmatmul(xd, wps[r], None, None, N, K, qm, gs, out=y, packed=True,
                                                        bits=bits)))
            name = f"{mode}-gs{gs}" + (f"-b{bits}" if mode == "affine" and bits != 4 else "")
            for tag, fn in runs:
                t = _time_kernel(torch, bi, lambda i: fn(i % copies), reps=4 * copies)
                gbs = tot / (t * 1e-3) / 1e9
                res[f"{name} {M}x{N}x{K} {tag}"] = {"us": round(t * 1e3, 1), "gbs": round(gbs, 1),
                                                   "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
            del wqs, wps
    # a mixture-of-experts decode step: 8 tokens, top-2 of 8 experts, each
    # expert 14336 x 4096 affine gs64; algorithmic bytes = the experts used
    T, topk, E, N, K, gs = 8, 2, 8, 14336, 4096, 64
    x, lhs, rhs, wq, s, b = inputs.gather_case(T, topk, K, N, E, "affine", gs, True, False, seed=0)
    xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.float16)
    ld, rd = torch.from_numpy(lhs).to(dev), torch.from_numpy(rhs).to(dev)
    w0 = torch.from_numpy(wq.view(np.int32)).to(dev)
    sd, bd = torch.from_numpy(s.view(np.int16)).to(dev), torch.from_numpy(b.view(np.int16)).to(dev)
    copies = 3
    ws = [w0] + [torch.bitwise_xor(w0, (0x01010101 * r) & 0x7fffffff) for r in range(1, copies)]
    y = torch.empty(rhs.size, N, dtype=torch.float16, device=dev)
    used = len(set(rhs.tolist()))
    tot = used * (N * K // 2 + N * (K // gs) * 4) + 2 * T * K + 2 * rhs.size * N
    t = _time_kernel(torch, bi, lambda i: bi.gather_qmatmul(xd, ld, rd, ws[i % copies], sd, bd, N, K, bi.AFFINE, gs,
                                                            True, out=y), reps=4 * copies)
    gbs = tot / (t * 1e-3) / 1e9
    res[f"gather affine-gs64 T{T} top{topk} of E{E} ({used} used) {N}x{K} transposed"] = {
        "us": round(t * 1e3, 1), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    wps = [torch.stack([bi.pack_qweights(w[e], sd[e], bd[e], N, K, bi.AFFINE, gs) for e in range(E)]) for w in ws]
    t = _time_kernel(torch, bi, lambda i: bi.gather_qmatmul(xd, ld, rd, wps[i % copies], None, None, N, K, bi.AFFINE,
                                                            gs, out=y, packed=True), reps=4 * copies)
    gbs = tot / (t * 1e-3) / 1e9
    res[f"gather affine-gs64 T{T} top{topk} of E{E} ({used} used) {N}x{K} packed"] = {
        "us": round(t * 1e3, 1), "gbs": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return res


if __name__ == "__main__":
    main()
