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
    # the first RMSNorm fused with the embedding lookup (h written, w read; the
    # row itself is counted under embed), then 2L residual adds fused with the
    # norm that follows them (x, r -> x, h)
    norm_bytes = (2 * B * H + 2 * H) + 2 * L * (8 * B * H + 2 * H)
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, cfg, B, ctx, kc_host, vc_host, ids):
    """The oracle's decode step on the host: the bench's batch with every
    core (median of up to 5 steps, at most ~12 s), and batch 1 on one core
    (median of 3 steps).  The oracle splits only independent outputs across
    threads; each output's fold is the same at any thread count."""
    import oracle
    from oracle import decoder as odec
    from invariant_reductions_amd.inputs import rope_tables
    cos_t, sin_t = rope_tables(ctx + 8, cfg["head_dim"])
    nproc = os.cpu_count() or 1

    def run(Bn, reps, budget):
        kv = np.full(Bn, ctx, np.int32)
        ts = []
        t_all = time.perf_counter()
        for _ in range(reps):
            t0 = time.perf_counter()
            odec.decode_step(W, cfg, ids[:Bn], [k[:Bn] for k in kc_host], [v[:Bn] for v in vc_host], kv, cos_t, sin_t)
            ts.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all > budget:
                break
        return float(np.median(ts)), len(ts)

    oracle.set_num_threads(nproc)
    all_threads = oracle.num_threads()
    t_all, n_all = run(B, 5, 12.0)
    oracle.set_num_threads(1)
    t_one, n_one = run(1, 3, 12.0)
    oracle.set_num_threads(nproc)
    return dict(t_all=t_all, n_all=n_all, threads=all_threads, t_one=t_one, n_one=n_one, model=cpu_model(),
                nproc=nproc)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--op", choices=sorted(OP_WORKLOADS),
                    help="run only one op's profiling workload (for rocprofv3 kernel traces and counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the batch-invariant hot path is a single-GPU kernel set "
              "(multi-GPU sharding is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_reductions_amd as bi
    from invariant_reductions_amd import inputs
    from invariant_reductions_amd.decoder import Decoder
    if args.op:
        op_workload(torch, bi, args.op)
        return

    cfg = inputs.LLAMA_4L
    B, ctx, K, Wm = args.batch, args.ctx, args.steps, args.warmup
    dev = torch.device("cuda:0")
    bi.lib()
    t_setup = time.perf_counter()
    W = inputs.decoder_weights(cfg, seed=0)
    cap = ctx + 2 * K + Wm + 8
    model = Decoder(cfg, W, max_batch=B, max_q=5, max_len=cap, device=dev)      # max_q 5: the verify sweep
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

    progress(f"timed {K} steps: {ms_step:.4f} ms/step")
    if not args.no_extras:
        out["ops"] = op_breakdown(model, plan, stream, B, ctx_mean, cfg, torch)
        progress("per-op breakdown done")
        out["decode_sweep"] = decode_sweep(torch, model, stream, cap, ctx)
        progress("decode sweep done")
        out["measured_peaks"] = measured_peaks(torch, bi, dev)
        out["roofline"]["frac_of_measured_read"] = round(mm_gbs / out["measured_peaks"]["hbm_read_gbs"], 4)
        progress("measured peaks done")
        out["invariance_overhead"] = invariance_overhead(torch, bi, dev, B)
        progress("invariance overhead done")
        out["qmatmul"] = qmatmul_decode(torch, bi, dev)
        out["row_ops"] = row_ops(torch, bi, model, B)
        progress("quantized and row ops done")
        out["sweep"] = op_sweep(torch, bi, dev)
        progress("sweep done")

    if not args.no_cpu_baseline:
        progress("CPU oracle baseline: starting")
        cb = cpu_baseline(W, cfg, B, ctx, kc_host, vc_host, ids0)
        progress("CPU oracle baseline done")
        trc, tr1 = step_traffic(cfg, B, ctx), step_traffic(cfg, 1, ctx)
        out["cpu_baseline"] = {
            "value": round(trc["total_bytes"] / cb["t_all"] / 1e9, 3), "unit": "GB/s", "cores": cb["threads"],
            "kind": "oracle", "cpu": cb["model"], "nproc": cb["nproc"],
            "sample": f"median of {cb['n_all']} decode step(s) of the same workload (batch {B}, context {ctx}) "
                      f"through the oracle's fixed-order fp32 ops on {cb['threads']} threads: "
                      f"{cb['t_all']:.2f} s per step",
            "single_thread": {"value": round(tr1["total_bytes"] / cb["t_one"] / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "sample": f"median of {cb['n_one']} decode step(s) at batch 1, context {ctx}: "
                                        f"{cb['t_one']:.2f} s per step"}}
    print(json.dumps(out), flush=True)


def _op_matmul(torch, bi, dev):
    """Dense projections: the decoder's at M = 64 (slot kernel), the verify
    block of 64 sequences x 5 tokens (M = 320) and a 4096-row prompt."""
    bf = torch.bfloat16
    # reference point for MFMA counters: the bf16 MFMA probe (back-to-back
    # v_mfma_f32_16x16x32_bf16, 8 waves per CU)
    sink = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    L = bi.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    yield "probe mfma 2048 workgroups x 4096 rounds", lambda i: L.bi_probe_mfma(ctypes.c_void_p(sink.data_ptr()), 2048,
                                                                               4096, st), 5
    for M, N, K in ((64, 4096, 4096), (64, 6144, 4096), (64, 28672, 4096), (320, 28672, 4096),
                    (320, 4096, 4096), (4096, 4096, 4096), (4096, 14336, 4096)):
        copies = max(2, -(-(512 << 20) // (N * K * 2)))
        ws_ = [bi.pack_weights((torch.randn(N, K, device=dev) * 0.02).to(bf)) for _ in range(copies)]
        x = torch.randn(M, K, device=dev).to(bf)
        y = torch.empty(M, N, dtype=bf, device=dev)
        mws = bi.matmul_workspace(M, N, K, device=dev)
        yield f"matmul {M}x{N}x{K} packed", lambda i: bi.matmul_ws(x, ws_[i % copies], mws, out=y), 2 * copies
        del ws_


def _op_qmatmul(torch, bi, dev):
    """4-bit decode projections 28672 x 4096 at M = 1, 4, 8, 32, 64 in the
    transposed and tile-packed layouts, three formats."""
    from invariant_reductions_amd import inputs
    N, K = 28672, 4096
    for mode, gs, qm in (("affine", 64, bi.AFFINE), ("nvfp4", 16, bi.NVFP4), ("mxfp4", 32, bi.MXFP4)):
        x, wq, s, b = inputs.qmatmul_case(64, K, N, mode, gs, True, seed=0)
        xd = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.float16)
        wq0 = torch.from_numpy(wq.view(np.int32)).to(dev)
        sd = torch.from_numpy(s if s.dtype == np.uint8 else s.view(np.int16)).to(dev)
        bd = None if b is None else torch.from_numpy(b.view(np.int16)).to(dev)
        copies = 12
        wqs = [wq0] + [torch.bitwise_xor(wq0, (0x01010101 * r) & 0x7fffffff) for r in range(1, copies)]
        wps = [bi.pack_qweights(w, sd, bd, N, K, qm, gs) for w in wqs]
        for M in (1, 4, 8, 32, 64):
            y = torch.empty(M, N, dtype=torch.float16, device=dev)
            xm = xd[:M].contiguous()
            yield (f"qmatmul {mode} gs{gs} {M}x{N}x{K} transposed",
                   lambda i: bi.qmatmul(xm, wqs[i % copies], sd, bd, N, K, qm, gs, True, out=y), 2 * copies)
            yield (f"qmatmul {mode} gs{gs} {M}x{N}x{K} packed",
                   lambda i: bi.qmatmul(xm, wps[i % copies], None, None, N, K, qm, gs, out=y, packed=True), 2 * copies)
        del wqs, wps


def _op_sdpa(torch, bi, dev):
    """Decode attention (32 query / 8 KV heads, d 128, head-major bf16
    cache): one sequence at 16388 and 65540 keys, 64 sequences at 768 and
    8196 keys, a verify block of 8 at 65540 keys; and causal prompts
    (prefill) of 2048 tokens (one range of chunks) and 8192 tokens (two)."""
    Hq, Hkv, D = 32, 8, 128
    for B, Q, Lk in ((1, 1, 16388), (1, 1, 65540), (1, 8, 65540), (64, 1, 768), (64, 1, 8196), (1, 2048, 2048),
                     (1, 8192, 8192)):
        copies = max(2, min(8, -(-(512 << 20) // (4 * B * Lk * Hkv * D))))
        ks = [torch.randn(B, Hkv, Lk, D, device=dev).to(torch.bfloat16) for _ in range(copies)]
        vs = [torch.randn(B, Hkv, Lk, D, device=dev).to(torch.bfloat16) for _ in range(copies)]
        q = torch.randn(B, Q, Hq, D, device=dev).to(torch.bfloat16)
        kv = torch.full((B,), Lk, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        ws = torch.empty(bi.sdpa_workspace_bytes(B, Q, Lk, Hq, D), dtype=torch.uint8, device=dev)
        yield (f"sdpa B{B} Q{Q} Lk{Lk}",
               lambda i: bi.sdpa(q, ks[i % copies], vs[i % copies], kv, Lk, 0.088, True, out=o, ws=ws,
                                 head_major=True), 10, sdpa_launches(B, Q, Hq, Hkv, Lk, _cus(torch, dev)))
        del ks, vs


def _op_rmsnorm(torch, bi, dev):
    """RMSNorm and fused add + RMSNorm over 4096-wide bf16 rows: 64 rows
    (decode) and 4096 rows."""
    H = 4096
    w = torch.ones(H, dtype=torch.bfloat16, device=dev)
    for Bn in (64, 4096):
        copies = max(2, min(64, -(-(512 << 20) // (Bn * H * 2))))
        xs = [torch.randn(Bn, H, device=dev).to(torch.bfloat16) for _ in range(copies)]
        r = torch.randn(Bn, H, device=dev).to(torch.bfloat16)
        y = torch.empty(Bn, H, dtype=torch.bfloat16, device=dev)
        xo = torch.empty_like(y)
        yield f"rmsnorm {Bn}x{H}", lambda i: bi.rmsnorm(xs[i % copies], w, out=y), 2 * copies
        yield f"add_rmsnorm {Bn}x{H}", lambda i: bi.add_rmsnorm(xs[i % copies], r, w, x_out=xo, out=y), 2 * copies
        del xs


OP_WORKLOADS = {"matmul": _op_matmul, "qmatmul": _op_qmatmul, "sdpa": _op_sdpa, "rmsnorm": _op_rmsnorm}


def op_workload(torch, bi, name):
    """One op's profiling workload: a plain 256 MiB device copy first (counter
    runs scale FETCH_SIZE / WRITE_SIZE by what it reads), then every case of
    the op, each called repeatedly on operands rotated over copies of at least
    512 MiB (no case finds its operands in a cache).  Prints one line per case
    with the library kernels one call launches and the median event-timed
    call (host launch overhead included)."""
    dev = torch.device("cuda:0")
    bi.lib()
    calib = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    calib2 = torch.empty_like(calib)
    calib2.copy_(calib)
    torch.cuda.synchronize()
    del calib, calib2
    for label, fn, reps, *kpc in OP_WORKLOADS[name](torch, bi, dev):
        fn(0)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record()
            fn(i)
            b.record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[reps // 2]
        print(f"case {label}: {reps} calls of {kpc[0] if kpc else 1} kernels, median {us:.1f} us", flush=True)
        torch.cuda.empty_cache()


def progress(msg):
    """One line on stderr per finished section (the JSON result is stdout's only line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


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
                "sdpa": tr["attn_bytes"], "embed_rmsnorm": 6 * B * H + 2 * H,
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


def _cus(torch, dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def sdpa_launches(B, Q, Hq, Hkv, Lk, cus):
    """Kernels one bi_sdpa call launches on a GPU of `cus` compute units: one
    for a prompt (at least 128 query rows per KV head, at most 8192 keys: the
    prompt-shaped kernel) and for at least 2 * cus (sequence, KV head) groups
    of at most 32 query rows over at most 1024 keys, or of at most 48 (query
    row, 256-key chunk) pairs (one workgroup walks a group's chunks and
    merges them), else two (chunk partials, then the merge)."""
    R = Q * (Hq // Hkv)
    if R >= 128 and Lk <= 8192:
        return 1
    nch = -(-Lk // 256)
    return 1 if R <= 32 and (nch <= 4 or R * nch <= 48) and B * Hkv >= 2 * cus else 2


def op_sweep(torch, bi, dev):
    """The four reductions at the measurement shapes, cold (rotated copies of
    the streamed operand, at least 512 MiB in all), kernel time:
      dense (packed weights): the pages' 4096 x 4096 and the decoder's
        projections at M in 1..64;
      RMSNorm: H = 4096 at B in {1, 8, 64, 512, 4096};
      SDPA: B = 1, Q in {1, 8} at Lk in {1028, 8196, 16388, 65540}, and
        B in {4, 16, 64} at Q = 1, Lk = 8196;
      4-bit quantized matmul (packed): K = N = 4096 and the decoder's
        projections at M in 1..64, affine group sizes 32/64/128, nvfp4, mxfp4;
      causal prefill attention at prompts of 512, 2048 and 8192 tokens."""
    res = {"target": "decode shapes with >= 32 MiB of weights or KV, and RMSNorm at B = 4096: frac_hbm >= 0.70",
           "matmul": {}, "rmsnorm": {}, "sdpa": {}}
    bf = torch.bfloat16
    for (N, K) in ((4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336), (32000, 4096)):
        copies = max(2, -(-(512 << 20) // (N * K * 2)))
        wps = [bi.pack_weights((torch.randn(N, K, device=dev) * 0.02).to(bf)) for _ in range(copies)]
        ws = bi.matmul_workspace(64, N, K, device=dev)
        for M in (1, 2, 3, 4, 8, 16, 32, 64):
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
                                                      ws=wsd, head_major=True), reps=3 * copies,
                         launches=sdpa_launches(Bn, Q, Hq, Hkv, Lk, _cus(torch, dev)))
        gbs = (kvb + 4 * Bn * Q * Hq * D) / (t * 1e-3) / 1e9
        res["sdpa"][f"B{Bn} Q{Q} Lk{Lk}"] = {"us": round(t * 1e3, 2), "gbs": round(gbs, 1),
                                              "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        del ks, vs
    # 4-bit quantized matmul (tile-packed, cold) at K = N = 4096 and the decoder's projections over M.  The
    # kernel time depends on the shapes alone, so codes and scales are drawn on the device: random 4-bit
    # words, fp16 scales and biases (affine), scale bytes of moderate exponent (nvfp4: e4m3, mxfp4: e8m0).
    res["qmatmul"] = {}
    gq = torch.Generator(device=dev).manual_seed(0)
    for (N, K) in ((4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336), (32000, 4096)):
        xd = torch.randn(64, K, device=dev, generator=gq).to(torch.float16)
        for mode, gs, qm in (("affine", 32, bi.AFFINE), ("affine", 64, bi.AFFINE), ("affine", 128, bi.AFFINE),
                             ("nvfp4", 16, bi.NVFP4), ("mxfp4", 32, bi.MXFP4)):
            copies = max(2, -(-(512 << 20) // (N * K // 2)))

            def packed_copy():
                wq = torch.randint(-(1 << 31), (1 << 31) - 1, (N, K // 8), dtype=torch.int32, device=dev, generator=gq)
                if mode == "affine":
                    sc = (torch.rand(N, K // gs, device=dev, generator=gq) * 0.01 + 0.001).to(torch.float16)
                    bs = (torch.randn(N, K // gs, device=dev, generator=gq) * 0.01).to(torch.float16)
                else:
                    lo, hi = (0x28, 0x48) if mode == "nvfp4" else (120, 131)
                    sc = torch.randint(lo, hi, (N, K // gs), dtype=torch.uint8, device=dev, generator=gq)
                    bs = None
                return bi.pack_qweights(wq, sc, bs, N, K, qm, gs)

            wps = [packed_copy() for _ in range(copies)]
            alg = N * K // 2 + N * (K // gs) * (4 if mode == "affine" else 1)
            for M in (1, 2, 4, 8, 16, 32, 64):
                xm = xd[:M].contiguous()
                y = torch.empty(M, N, dtype=torch.float16, device=dev)
                t = _time_kernel(torch, bi, lambda i: bi.qmatmul(xm, wps[i % copies], None, None, N, K, qm, gs,
                                                                 out=y, packed=True), reps=3 * copies)
                gbs = (alg + 2 * M * K + 2 * M * N) / (t * 1e-3) / 1e9
                res["qmatmul"][f"{mode}-gs{gs} {M}x{N}x{K}"] = {"us": round(t * 1e3, 2), "gbs": round(gbs, 1),
                                                                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
            del wps
    # causal prefill: Q = Lk (a whole prompt in one call), flops over the visible (query, key) pairs
    res["prefill"] = {}
    for Bn, Q in ((1, 512), (1, 2048), (1, 8192), (8, 512), (64, 512)):
        Lk = Q
        ks = torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf)
        vs = torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf)
        q = torch.randn(Bn, Q, Hq, D, device=dev).to(bf)
        kv = torch.full((Bn,), Lk, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        wsd = torch.empty(bi.sdpa_workspace_bytes(Bn, Q, Lk, Hq, D), dtype=torch.uint8, device=dev)
        t = _time_kernel(torch, bi, lambda i: bi.sdpa(q, ks, vs, kv, Lk, 0.088, True, out=o, ws=wsd, head_major=True),
                         reps=5, launches=sdpa_launches(Bn, Q, Hq, Hkv, Lk, _cus(torch, dev)))
        pairs = Q * (Q + 1) // 2
        tf = 4 * Bn * Hq * D * pairs / (t * 1e-3) / 1e12
        res["prefill"][f"B{Bn} Q{Q} Lk{Lk} causal"] = {"us": round(t * 1e3, 2), "tflops": round(tf, 2),
                                                       "frac_mfma": round(tf / 2500.0, 4)}
        del ks, vs, wsd
    torch.cuda.empty_cache()
    return res


def measured_peaks(torch, bi, dev):
    """What this GPU sustains, by the library's probes (kernel time,
    launch-recorded events, median of 5): a streaming read and a copy of
    1 GiB (best of three grid sizes) and back-to-back bf16 MFMA."""
    L = bi.lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    sink = torch.empty(1 << 22, dtype=torch.uint8, device=dev)

    def ktime(fn, reps=5):
        ts = []
        for _ in range(reps):
            s_, t_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()                                   # creates the event handles
            t_.record()
            L.bi_time_next_launch(ctypes.c_void_p(s_.cuda_event), ctypes.c_void_p(t_.cuda_event))
            rc = fn()
            assert rc == 0, rc
            torch.cuda.synchronize()
            ts.append(s_.elapsed_time(t_))
        return float(np.median(ts)) * 1e-3

    read = max(n / ktime(lambda: L.bi_probe_read(ctypes.c_void_p(a.data_ptr()), n, ctypes.c_void_p(sink.data_ptr()),
                                                 wg, st)) / 1e9 for wg in (512, 2048, 8192))
    copy = max(2 * n / ktime(lambda: L.bi_probe_copy(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()), n,
                                                     wg, st)) / 1e9 for wg in (1024, 4096))
    wg, iters = 2048, 20000
    mf = wg * 4 * iters * 8 * 16384 / ktime(lambda: L.bi_probe_mfma(ctypes.c_void_p(sink.data_ptr()), wg, iters, st),
                                           reps=3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round(read, 1), "hbm_copy_gbs": round(copy, 1), "mfma_bf16_tflops": round(mf, 1),
            "method": "bi_probe_read / bi_probe_copy over 1 GiB (best of 3 grid sizes), bi_probe_mfma "
                      "(v_mfma_f32_16x16x32_bf16, 8 independent chains per wave); kernel time, median of 5"}


def _ab(torch, fns, reps=11, inner=10):
    """Median ms per call of each callable, timed in alternating order (A, B,
    C, A, B, C, ...): every sample is one event pair around `inner` calls."""
    ev = {k: [] for k in fns}
    for k, f in fns.items():                      # warm every side once
        for i in range(inner):
            f(i)
    torch.cuda.synchronize()
    for r in range(reps):
        for k, f in fns.items():
            s_, t_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()
            for i in range(inner):
                f(r * inner + i)
            t_.record()
            ev[k].append((s_, t_))
    torch.cuda.synchronize()
    return {k: float(np.median([s_.elapsed_time(t_) / inner for s_, t_ in v])) for k, v in ev.items()}


def _raw(fn, per_call):
    """A callable i -> fn(*per_call[i % len]) with every argument already a
    ctypes value: the library's entry point without the Python binding's
    checks, so a small kernel's time is not the binding's host overhead."""
    def call(i):
        rc = fn(*per_call[i % len(per_call)])
        if rc != 0:
            raise RuntimeError(f"bench call failed: {rc}")
    return call


def invariance_overhead(torch, bi, dev, B):
    """Cost of invariance per op: the invariant kernel against the fastest
    non-invariant way to compute the same thing on this GPU -- the vendor
    libraries torch dispatches to (hipBLASLt for the matmuls, torch's RMSNorm
    and scaled-dot-product attention, which choose their kernels and splits by
    shape) and this library's split comparison variants (split-K matmul and
    quantized matmul with a cleanup reduction, split-row RMSNorm, split-KV
    attention with the split count as a free parameter; best split count per
    shape).  Both
    sides on the same stream, same operands (weights rotated over copies of
    at least 512 MiB so that neither side finds them in a cache), median of
    11 alternating samples of 10 calls.  overhead = t_invariant / t_best - 1
    (negative: the invariant kernel is the faster)."""
    import torch.nn.functional as F
    bf, f16 = torch.bfloat16, torch.float16
    res = {"method": "median of 11 alternating A/B samples, 10 calls each, events around the calls (same for every "
                     "side); cold operands; this library's entry points called through ctypes with prepared "
                     "arguments, torch's through torch", "matmul": {}, "qmatmul": {}, "rmsnorm": {}, "sdpa": {}}
    L = bi.lib()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def overhead_entry(t_inv, alts):
        best = min(alts, key=alts.get)
        return {"invariant_us": round(t_inv * 1e3, 2), **{f"{k}_us": round(v * 1e3, 2) for k, v in alts.items()},
                "best_non_invariant": best, "overhead": round(t_inv / alts[best] - 1, 3),
                "faster": "invariant" if t_inv <= alts[best] else best}

    shapes = [(M, 4096, 4096) for M in (1, 2, 4, 8)] + [(B, N, K) for (N, K) in
                                                         ((6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336),
                                                          (32000, 4096))]
    for M, N, K in shapes:
        copies = max(2, -(-(512 << 20) // (N * K * 2)))
        ws_ = [(torch.randn(N, K, device=dev) * 0.02).to(bf) for _ in range(copies)]
        wp = [bi.pack_weights(w) for w in ws_]
        x = torch.randn(M, K, device=dev).to(bf)
        y = torch.empty(M, N, dtype=bf, device=dev)
        mws = bi.matmul_workspace(M, N, K, device=dev)
        fns = {"inv": _raw(L.bi_matmul_ws, [(vp(x), vp(w.data), vp(y), M, N, K, 0, 2, vp(mws), mws.numel(), st)
                                            for w in wp]),
               "hipblaslt": lambda i: torch.mm(x, ws_[i % copies].t(), out=y)}
        for sp in (2, 4, 8):
            sws = torch.empty(M * N * sp * 4, dtype=torch.uint8, device=dev)
            fns[f"split{sp}"] = _raw(L.bi_matmul_split, [(vp(x), vp(w.data), vp(y), M, N, K, 0, 2, sp, vp(sws),
                                                          sws.numel(), st) for w in wp])
        t = _ab(torch, fns)
        alts = {k: v for k, v in t.items() if k != "inv"}
        best_split = min((k for k in alts if k.startswith("split")), key=alts.get)
        alts = {"hipblaslt": alts["hipblaslt"], best_split: alts[best_split]}
        res["matmul"][f"{M}x{N}x{K}"] = overhead_entry(t["inv"], alts)
        del ws_, wp
    # quantized: the invariant 4-bit kernel (tile-packed) against its own
    # split-K variant (best of 2, 4, 8 splits) and hipBLASLt on the same
    # matrix already dequantized to binary16 (the path without a quantized
    # kernel)
    from invariant_reductions_amd import inputs
    gs = 32
    for N, K, Ms in ((4096, 4096, (1, 2, 4, 8)), (28672, 4096, (1, 4, 8))):
        _, wq, sc, _ = inputs.qmatmul_case(1, K, N, "mxfp4", gs, True, seed=0)
        wq0 = torch.from_numpy(wq.view(np.int32)).to(dev)
        sd = torch.from_numpy(sc).to(dev)
        copies = max(2, -(-(512 << 20) // (N * K // 2)))
        wqp = [bi.pack_qweights(torch.bitwise_xor(wq0, (0x01010101 * r) & 0x7fffffff), sd, None, N, K, bi.MXFP4,
                                gs) for r in range(copies)]
        ndd = max(2, -(-(512 << 20) // (N * K * 2)))
        wd = [torch.randn(N, K, device=dev).to(f16) for _ in range(ndd)]
        for M in Ms:
            x = torch.randn(M, K, device=dev).to(f16)
            y = torch.empty(M, N, dtype=f16, device=dev)
            fns = {"inv": _raw(L.bi_qmatmul, [(vp(x), vp(w), None, None, vp(y), M, N, K, bi.MXFP4, 4, gs, 2, st)
                                              for w in wqp]),
                   "hipblaslt_f16": lambda i: torch.mm(x, wd[i % ndd].t(), out=y)}
            for sp in (2, 4, 8):
                qws = torch.empty(L.bi_qmatmul_split_workspace_bytes(M, N, sp), dtype=torch.uint8, device=dev)
                fns[f"split{sp}"] = _raw(L.bi_qmatmul_split, [(vp(x), vp(w), None, None, vp(y), M, N, K, bi.MXFP4, 4,
                                                               gs, 2, sp, vp(qws), qws.numel(), st) for w in wqp])
            t = _ab(torch, fns)
            alts = {k: v for k, v in t.items() if k != "inv"}
            best_split = min((k for k in alts if k.startswith("split")), key=alts.get)
            res["qmatmul"][f"mxfp4 {M}x{N}x{K}"] = overhead_entry(t["inv"], {"hipblaslt_f16": alts["hipblaslt_f16"],
                                                                      best_split: alts[best_split]})
        del wqp, wd
    H = 4096
    w = torch.ones(H, dtype=bf, device=dev)
    for Bn in (1, 64, 4096):
        copies = max(2, min(64, -(-(512 << 20) // (Bn * H * 2))))
        xs = [torch.randn(Bn, H, device=dev).to(bf) for _ in range(copies)]
        y = torch.empty(Bn, H, dtype=bf, device=dev)
        eps = ctypes.c_float(1e-6)
        fns = {"inv": _raw(L.bi_rmsnorm, [(vp(xx), vp(w), vp(y), Bn, H, eps, 0, st) for xx in xs]),
               "torch": lambda i: F.rms_norm(xs[i % copies], (H,), w, 1e-6)}
        for sp in (2, 4, 8):
            sws = torch.empty(max(16, L.bi_rmsnorm_split_workspace_bytes(Bn, sp)), dtype=torch.uint8, device=dev)
            fns[f"split{sp}"] = _raw(L.bi_rmsnorm_split, [(vp(xx), vp(w), vp(y), Bn, H, eps, 0, sp, vp(sws),
                                                           sws.numel(), st) for xx in xs])
        t = _ab(torch, fns)
        alts = {k: v for k, v in t.items() if k != "inv"}
        best_split = min((k for k in alts if k.startswith("split")), key=alts.get)
        res["rmsnorm"][f"{Bn}x{H}"] = overhead_entry(t["inv"], {"torch": alts["torch"], best_split: alts[best_split]})
        del xs
    Hq, Hkv, D = 32, 8, 128
    for Bn, Lk in ((1, 16388), (1, 65540), (B, 768)):
        copies = max(2, min(8, -(-(512 << 20) // (4 * Bn * Lk * Hkv * D))))
        ks = [torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf) for _ in range(copies)]
        vs = [torch.randn(Bn, Hkv, Lk, D, device=dev).to(bf) for _ in range(copies)]
        q = torch.randn(Bn, 1, Hq, D, device=dev).to(bf)
        qt = q.transpose(1, 2).contiguous()                      # [B, Hq, 1, D] for torch
        kv = torch.full((Bn,), Lk, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        wsd = torch.empty(bi.sdpa_workspace_bytes(Bn, 1, Lk, Hq, D), dtype=torch.uint8, device=dev)
        fns = {"inv": _raw(L.bi_sdpa, [(vp(q), vp(kk), vp(vv), vp(o), vp(kv), Lk, Bn, 1, Lk, Hq, Hkv, D,
                                        ctypes.c_float(0.088), 1, 0, 1, vp(wsd), wsd.numel(), st)
                                       for kk, vv in zip(ks, vs)]),
               "torch_sdpa": lambda i: F.scaled_dot_product_attention(qt, ks[i % copies], vs[i % copies], scale=0.088,
                                                                      enable_gqa=True)}
        # the split-KV variant at split counts from one run per (sequence, KV
        # head) up to runs of 4 chunks
        nch = -(-Lk // 256)
        for sp in sorted({1, 2, 4, 8, 16, 32, 64, 128, max(1, nch // 4)}):
            if sp > nch:
                continue
            nb = L.bi_sdpa_split_workspace_bytes(Bn, 1, Lk, Hq, D, sp)
            sws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
            fns[f"split{sp}"] = _raw(L.bi_sdpa_split, [(vp(q), vp(kk), vp(vv), vp(o), vp(kv), Lk, Bn, 1, Lk, Hq, Hkv,
                                                        D, ctypes.c_float(0.088), 1, 0, 1, sp, vp(sws), sws.numel(),
                                                        st) for kk, vv in zip(ks, vs)])
        t = _ab(torch, fns)
        alts = {k: v for k, v in t.items() if k != "inv"}
        best_split = min((k for k in alts if k.startswith("split")), key=alts.get)
        res["sdpa"][f"B{Bn} Q1 Lk{Lk}"] = overhead_entry(t["inv"], {"torch_sdpa": alts["torch_sdpa"],
                                                             best_split: alts[best_split]})
        del ks, vs
    torch.cuda.empty_cache()
    return res


def decode_sweep(torch, model, stream, cap, ctx, steps=10):
    """Config-5 step time at B in {1, 4, 16, 64}: plain greedy decoding (the
    self-advancing one-token plan, replayed) and speculative verification
    (one causal block of 5 tokens per sequence: the last committed token and
    4 drafts).  Tokens/s for verification assume every draft is accepted
    (5 tokens per sequence per step); with rejections it scales with the
    accepted count plus one."""
    res = {}
    for Bs in (1, 4, 16, 64):
        if Bs > model.max_batch:
            continue
        r = {}
        model.kv_len[:Bs].fill_(ctx)
        plan = model.plan(Bs, 1, cap, stream, advance=True)
        for _ in range(2):
            model.run_plan(plan)
        model.kv_len[:Bs].fill_(ctx)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            model.run_plan(plan)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        r["plain"] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(Bs / (ms * 1e-3), 1)}
        if model.max_q >= 5:
            model.kv_len[:Bs].fill_(ctx + 5)
            vplan = model.plan(Bs, 5, cap, stream)
            model.run_plan(vplan)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                model.run_plan(vplan)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            r["verify_q5"] = {"ms_per_step": round(ms, 4), "tokens_per_s_all_accepted": round(5 * Bs / (ms * 1e-3), 1)}
        res[f"B{Bs}"] = r
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
