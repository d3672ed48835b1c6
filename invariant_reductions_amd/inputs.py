"""Seeded synthetic inputs for the batch-invariant reductions.

This module only *makes* inputs: random draws, conversion of those draws to
the storage types, packing of group-quantized weights and the rotary tables a
decoder carries as buffers.  It holds none of the reductions' arithmetic and
is the only module that both the HIP path's callers and the CPU oracle's
callers share.

Storage conventions (what every entry point consumes):
  * bf16 and f16 tensors are numpy ``uint16`` arrays of bit patterns; f32 is
    ``float32``.  Conversion from the fp32 draw uses round to nearest even
    (torch's CPU cast for bf16, numpy's for f16).
  * Draws are made at the largest batch a workload uses and sliced, so row i
    is the same row for every batch size.
"""
from __future__ import annotations

import numpy as np
import torch

DTYPES = ("bf16", "f16", "f32")


# --------------------------------------------------------------------------
# storage-type conversion of draws
# --------------------------------------------------------------------------

def to_storage(a, dtype: str) -> np.ndarray:
    """fp32 (or fp64) values -> storage array of `dtype` (RNE)."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        t = torch.from_numpy(a).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def from_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> fp32 values (exact widening)."""
    if dtype == "f32":
        return np.asarray(a, np.float32)
    if dtype == "f16":
        return np.asarray(a, np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def normal(rng: np.random.Generator, shape, scale: float = 1.0, loc: float = 0.0,
           dtype: str = "bf16") -> np.ndarray:
    """loc + scale * N(0,1), drawn in fp64, cast to fp32, stored as `dtype`."""
    v = rng.standard_normal(shape) * scale + loc
    return to_storage(v.astype(np.float32), dtype)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def dense_case(M: int, N: int = 512, K: int = 4096, dtype: str = "bf16", seed: int = 0,
               w_scale: float = 0.02):
    """W [N,K] ~ N(0,1)*w_scale drawn first, then x [M,K] ~ N(0,1).
    Returns (x, W_transposed [N,K], W_natural [K,N]) as storage arrays; the
    natural copy holds the same values transposed."""
    rng = np.random.default_rng(seed)
    w = normal(rng, (N, K), w_scale, dtype=dtype)
    x = normal(rng, (M, K), 1.0, dtype=dtype)
    return x, w, np.ascontiguousarray(w.T)


def rmsnorm_case(B: int, H: int = 4096, seed: int = 0, dtype: str = "bf16"):
    """x [B,H] ~ N(0,1)*3 drawn first, then w [H] = 1 + 0.1*N(0,1)."""
    rng = np.random.default_rng(seed)
    x = normal(rng, (B, H), 3.0, dtype=dtype)
    w = normal(rng, (H,), 0.1, loc=1.0, dtype=dtype)
    return x, w


def sdpa_case(B: int, Q: int, Lcap: int, Hq: int = 32, Hkv: int = 8, D: int = 128,
              seed: int = 0, dtype: str = "bf16"):
    """K, V [B,Lcap,Hkv,D] ~ N(0,1) drawn first (K then V), then q [B,Q,Hq,D]."""
    rng = np.random.default_rng(seed)
    k = normal(rng, (B, Lcap, Hkv, D), dtype=dtype)
    v = normal(rng, (B, Lcap, Hkv, D), dtype=dtype)
    q = normal(rng, (B, Q, Hq, D), dtype=dtype)
    return q, k, v


def integer_values(rng: np.random.Generator, shape, lo: int, hi: int, dtype: str) -> np.ndarray:
    """Uniform integers in [lo, hi] stored exactly as `dtype`."""
    return to_storage(rng.integers(lo, hi + 1, size=shape).astype(np.float32), dtype)


# --------------------------------------------------------------------------
# group quantization (host data preparation, the analogue of a quantize op)
# --------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, cols] codes 0..15 -> [rows, cols/8] uint32, the element with the
    lowest column index in bits 0..3."""
    codes = np.asarray(codes, dtype=np.uint32)
    rows, cols = codes.shape
    assert cols % 8 == 0
    c = codes.reshape(rows, cols // 8, 8)
    out = np.zeros((rows, cols // 8), np.uint32)
    for i in range(8):
        out |= c[:, :, i] << np.uint32(4 * i)
    return out


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """[rows, cols] codes 0..2^bits-1 -> [rows, cols*bits/32] uint32: each row
    a little-endian bit stream, code j in bits [j*bits, (j+1)*bits), stream bit
    i in bit i % 32 of word i / 32.  At bits = 4 this equals pack_nibbles."""
    codes = np.asarray(codes, dtype=np.uint64)
    rows, cols = codes.shape
    assert (cols * bits) % 32 == 0 and 1 <= bits <= 8
    assert int(codes.max(initial=0)) < (1 << bits)
    # 32 codes of `bits` bits fill exactly `bits` words
    c = codes.reshape(rows, cols // 32, 32)
    out = np.zeros((rows, cols // 32, bits), np.uint32)
    for j in range(32):
        o = j * bits
        w, sh = o // 32, o % 32
        v = c[:, :, j]
        out[:, :, w] |= ((v << np.uint64(sh)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
        if sh + bits > 32:
            out[:, :, w + 1] |= (v >> np.uint64(32 - sh)).astype(np.uint32)
    return out.reshape(rows, cols * bits // 32)


def quantize_affine(w: np.ndarray, group_size: int, bits: int = 4):
    """Min-max affine quantization to `bits` bits along the last axis of fp32
    `w` [rows, cols]: with L = 2^bits - 1, per group s = (max-min)/L and b =
    min, both rounded to binary16; q = clamp(rint((w - b)/s), 0, L), q = 0
    where s == 0.  Returns (wq uint32 [rows, cols*bits/32], scales f16 bits,
    biases f16 bits)."""
    w = np.asarray(w, np.float32)
    rows, cols = w.shape
    assert cols % group_size == 0
    L = (1 << bits) - 1
    g = w.reshape(rows, cols // group_size, group_size).astype(np.float64)
    lo, hi = g.min(axis=2), g.max(axis=2)
    s16 = ((hi - lo) / L).astype(np.float16)
    b16 = lo.astype(np.float16)
    s = s16.astype(np.float64)[:, :, None]
    b = b16.astype(np.float64)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint((g - b) / np.where(s > 0, s, 1.0)), 0.0)
    q = np.clip(q, 0, L).astype(np.uint32).reshape(rows, cols)
    return pack_bits(q, bits), s16.view(np.uint16), b16.view(np.uint16)


_E2M1_GRID = None


def _e2m1_grid():
    """All 16 e2m1 codes with their values, built from the bit fields
    (sign | 2-bit exponent, bias 1 | 1-bit mantissa)."""
    global _E2M1_GRID
    if _E2M1_GRID is None:
        vals = []
        for c in range(16):
            s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
            mag = (m * 0.5) if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
            vals.append(-mag if s else mag)
        _E2M1_GRID = np.array(vals, np.float64)
    return _E2M1_GRID


def encode_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest e2m1 code (ties to the code with an even mantissa bit),
    saturating at +-6."""
    grid = _e2m1_grid()
    v = np.clip(np.asarray(v, np.float64), -6.0, 6.0)
    pos = grid[:8]                                   # codes 0..7 are the non-negative values
    a = np.abs(v)[..., None]
    d = np.abs(a - pos)
    best = d.min(axis=-1, keepdims=True)
    cand = (d == best)
    # prefer an even mantissa bit (code & 1 == 0) among equidistant codes
    even = cand & ((np.arange(8) & 1) == 0)
    pick = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    code = pick.astype(np.uint32)
    neg = (v < 0) & (code != 0)
    return np.where(neg, code | 8, code).astype(np.uint32)


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """fp32 -> OCP e4m3fn byte, round to nearest even, saturating at 448."""
    v = np.clip(np.asarray(v, np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def quantize_nvfp4(w: np.ndarray):
    """nvfp4-style quantization along the last axis of fp32 `w` [rows, cols]:
    per 16 elements one e4m3 scale s = e4m3(amax / 6); codes = e2m1(w / s),
    all codes 0 where s == 0.  Returns (wq uint32 [rows, cols/8], scale bytes
    uint8 [rows, cols/16])."""
    w = np.asarray(w, np.float32)
    rows, cols = w.shape
    assert cols % 16 == 0
    g = w.reshape(rows, cols // 16, 16)
    amax = np.abs(g).max(axis=2)
    sb = encode_e4m3((amax / 6.0).astype(np.float32))
    sv = torch.from_numpy(sb).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sv[:, :, None] > 0, g / np.where(sv > 0, sv, 1.0)[:, :, None], 0.0)
    codes = encode_e2m1(r).reshape(rows, cols)
    return pack_nibbles(codes), sb


def quantize_mxfp4(w: np.ndarray):
    """mxfp4-style quantization along the last axis of fp32 `w` [rows, cols]:
    per 32 elements one e8m0 scale 2^(e - 127) with e = floor(log2(amax)) - 2
    + 127 (the largest e2m1 magnitude is 6 = 1.5 * 2^2), clamped to [0, 254];
    codes = e2m1(w / scale), saturating; a zero group gets e = 0 and zero
    codes.  Returns (wq uint32 [rows, cols/8], scale bytes uint8 [rows, cols/32])."""
    w = np.asarray(w, np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    g = w.reshape(rows, cols // 32, 32).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2 + 127, 0)
    e = np.clip(e, 0, 254).astype(np.int64)
    scale = np.ldexp(1.0, (e - 127).astype(np.int32))
    r = np.where(amax[:, :, None] > 0, g / scale[:, :, None], 0.0)
    codes = encode_e2m1(r).reshape(rows, cols)
    return pack_nibbles(codes), e.astype(np.uint8)


def quantize_mxfp8(w: np.ndarray):
    """mxfp8-style quantization along the last axis of fp32 `w` [rows, cols]:
    per 32 elements one e8m0 scale 2^(e - 127) with e = floor(log2(amax)) - 8
    + 127 (the largest e4m3 magnitude is 448 = 1.75 * 2^8), clamped to [0,
    254]; codes = e4m3(w / scale), round to nearest even, saturating; a zero
    group gets e = 0 and zero codes.  Returns (wq uint32 [rows, cols/4], the
    codes as the row's bytes in order, and scale bytes uint8 [rows, cols/32])."""
    w = np.asarray(w, np.float32)
    rows, cols = w.shape
    assert cols % 32 == 0
    g = w.reshape(rows, cols // 32, 32).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8 + 127, 0)
    e = np.clip(e, 0, 254).astype(np.int64)
    scale = np.ldexp(1.0, (e - 127).astype(np.int32))
    r = np.where(amax[:, :, None] > 0, g / scale[:, :, None], 0.0)
    codes = encode_e4m3(r.astype(np.float32)).reshape(rows, cols)
    return pack_bits(codes.astype(np.uint32), 8), e.astype(np.uint8)


def qmatmul_case(M: int, K: int, N: int, qmode: str, group_size: int, transposed: bool = True,
                 seed: int = 0, bits: int = 4):
    """W ~ N(0,1) drawn first, quantized along the matrix's stored minor axis
    ([N,K] along K when transposed, [K,N] along N when natural), then
    x [M,K] ~ N(0,1) as binary16 bits.  `bits` is the affine code width (2 to
    8); the fp modes have fixed widths (nvfp4 and mxfp4 4, mxfp8 8).  Returns
    (x, wq, scales, biases)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((N, K) if transposed else (K, N)).astype(np.float32)
    if qmode == "affine":
        wq, s, b = quantize_affine(w, group_size, bits)
    elif qmode == "nvfp4":
        assert group_size == 16
        wq, s = quantize_nvfp4(w)
        b = None
    elif qmode == "mxfp4":
        assert group_size == 32
        wq, s = quantize_mxfp4(w)
        b = None
    elif qmode == "mxfp8":
        assert group_size == 32
        wq, s = quantize_mxfp8(w)
        b = None
    else:
        raise ValueError(qmode)
    x = normal(rng, (M, K), dtype="f16")
    return x, wq, s, b


def gather_case(T: int, topk: int, K: int, N: int, E: int, qmode: str, group_size: int, transposed: bool = True,
                sort_rows: bool = False, seed: int = 0, bits: int = 4):
    """A mixture-of-experts expert matmul: E weight matrices W_e ~ N(0,1)
    ([N,K] when transposed, else [K,N]), each quantized as qmatmul_case does,
    then x [T,K] ~ N(0,1) binary16, then per token `topk` distinct experts
    drawn uniformly.  Row m = t*topk + j reads token t and its j-th expert;
    sort_rows orders the rows by expert (stable), as a sorted-index caller
    would.  Returns (x, lhs int32 [M], rhs int32 [M], wq [E, ...], scales
    [E, ...], biases [E, ...] or None)."""
    rng = np.random.default_rng(seed)
    parts = []
    for _ in range(E):
        w = rng.standard_normal((N, K) if transposed else (K, N)).astype(np.float32)
        if qmode == "affine":
            parts.append(quantize_affine(w, group_size, bits))
        elif qmode == "nvfp4":
            parts.append(quantize_nvfp4(w) + (None,))
        elif qmode == "mxfp4":
            parts.append(quantize_mxfp4(w) + (None,))
        elif qmode == "mxfp8":
            parts.append(quantize_mxfp8(w) + (None,))
        else:
            raise ValueError(qmode)
    wq = np.stack([p[0] for p in parts])
    sc = np.stack([p[1] for p in parts])
    bs = None if parts[0][2] is None else np.stack([p[2] for p in parts])
    x = normal(rng, (T, K), dtype="f16")
    rhs = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).reshape(-1).astype(np.int32)
    lhs = np.repeat(np.arange(T, dtype=np.int32), topk)
    if sort_rows:
        order = np.argsort(rhs, kind="stable")
        lhs, rhs = lhs[order], rhs[order]
    return x, lhs, rhs, wq, sc, bs


def rope_tables(max_pos: int, head_dim: int, theta: float = 10000.0):
    """cos/sin [max_pos, head_dim/2] of pos * theta^(-2i/head_dim), computed in
    fp64 and stored as fp32 (model buffers, like the weights)."""
    half = head_dim // 2
    inv = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / head_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def prompts(B: int, L: int = 512, vocab: int = 32000, seed: int = 1, max_batch: int = 64):
    """Random token ids, drawn as [max_batch, L] and sliced to B rows."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=(max(B, max_batch), L)).astype(np.int32)[:B]


LLAMA_4L = dict(hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=14336, vocab=32000,
                n_layers=4, eps=1e-6, rope_theta=10000.0)


def decoder_weights(cfg: dict = LLAMA_4L, seed: int = 0, std: float = 0.02):
    """Random-init weights of a Llama-style decoder as bf16 storage arrays:
    every projection and the embedding ~ N(0, std), drawn in a fixed order
    (embedding, then per layer qkv, o, gate|up, down, then lm_head); RMSNorm
    weights are ones.  Projections are stored [out_features, in_features]."""
    H, F, V = cfg["hidden"], cfg["ffn"], cfg["vocab"]
    qkv = (cfg["n_heads"] + 2 * cfg["n_kv_heads"]) * cfg["head_dim"]
    rng = np.random.default_rng(seed)

    def draw(shape):
        return to_storage(rng.standard_normal(shape, dtype=np.float32) * np.float32(std), "bf16")

    ones = to_storage(np.ones(H, np.float32), "bf16")
    W = {"embed": draw((V, H)), "layers": []}
    for _ in range(cfg["n_layers"]):
        W["layers"].append(dict(attn_norm=ones.copy(), wqkv=draw((qkv, H)),
                                wo=draw((H, cfg["n_heads"] * cfg["head_dim"])), mlp_norm=ones.copy(),
                                wgu=draw((2 * F, H)), wdown=draw((H, F))))
    W["final_norm"] = ones.copy()
    W["lm_head"] = draw((V, H))
    return W
