"""CPU oracle for the batch-invariant reductions.

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the library's product
path never does.  It shares no code with the HIP kernels.

Every function returns the raw fp32 result of a fixed-order fp32 computation
(see ``bi_oracle.c``) and, where asked, the value rounded to the output type
with the oracle's own round-to-nearest-even routine.

Sources followed (cited by page title and section):
  * "Batch-invariant kernels: why temperature-0 decoding is still
    nondeterministic" -- Case 1 (non-associativity), Case 2 (sequential,
    pairwise and split reductions), Case 4 (RMSNorm sum of squares), Case 6
    (the three reductions and their batch-invariant strategies).
  * "Fix fp quantized matmul corruption when the quantized dim is not a
    multiple of 32" -- Problem (the reference is x @ dequantize(W).T) and Fix
    (group sizes; nvfp4 = e2m1 codes with one e4m3 scale per 16; mxfp4 has
    group size 32 -- its e2m1 codes and power-of-two e8m0 scale follow the
    OCP microscaling format, which the pages name but do not define).
  * "Fix/speculative shape invariance" -- Problem and Changes (dense matmul,
    quantized matmul and two-pass SDPA must reduce a token the same way alone
    or inside a verification block).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bi_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16, F16, F32 = 0, 1, 2
AFFINE, NVFP4, MXFP4, MXFP8 = 0, 1, 2, 3
_DT = {"bf16": BF16, "f16": F16, "f32": F32}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc.  -ffp-contract=off keeps every multiply and
    add separately rounded, as the oracle's definition states."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.bo_bf16_to_f32.argtypes = [ctypes.c_uint16]; L.bo_bf16_to_f32.restype = ctypes.c_float
        L.bo_f16_to_f32.argtypes = [ctypes.c_uint16]; L.bo_f16_to_f32.restype = ctypes.c_float
        L.bo_f32_to_bf16.argtypes = [ctypes.c_float]; L.bo_f32_to_bf16.restype = ctypes.c_uint16
        L.bo_f32_to_f16.argtypes = [ctypes.c_float]; L.bo_f32_to_f16.restype = ctypes.c_uint16
        L.bo_e2m1_to_f32.argtypes = [ctypes.c_uint8]; L.bo_e2m1_to_f32.restype = ctypes.c_float
        L.bo_e4m3_to_f32.argtypes = [ctypes.c_uint8]; L.bo_e4m3_to_f32.restype = ctypes.c_float
        L.bo_e8m0_to_f32.argtypes = [ctypes.c_uint8]; L.bo_e8m0_to_f32.restype = ctypes.c_float
        L.bo_round.argtypes = [P, P, I64, I32]
        L.bo_widen.argtypes = [P, P, I64, I32]
        L.bo_fold_seq_f32.argtypes = [P, I64]; L.bo_fold_seq_f32.restype = ctypes.c_float
        L.bo_fold_seq_f64.argtypes = [P, I64]; L.bo_fold_seq_f64.restype = ctypes.c_double
        L.bo_fold_pairwise_f32.argtypes = [P, I64]; L.bo_fold_pairwise_f32.restype = ctypes.c_float
        L.bo_fold_split_f32.argtypes = [P, I64, I64]; L.bo_fold_split_f32.restype = ctypes.c_float
        L.bo_matmul.argtypes = [P, P, P, I64, I64, I64, I32, I32]
        L.bo_matmul_desc.argtypes = [P, P, P, I64, I64, I64, I32, I32]
        L.bo_dequantize.argtypes = [P, P, P, P, I64, I64, I32, I32, I32]
        L.bo_qmatmul.argtypes = [P, P, P, P, P, I64, I64, I64, I32, I32, I32, I32]
        L.bo_gather_qmatmul.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I32, I32, I32, I32]
        L.bo_rmsnorm.argtypes = [P, P, P, P, I64, I64, ctypes.c_float, I32]
        L.bo_rmsnorm_desc.argtypes = [P, P, P, P, I64, I64, ctypes.c_float, I32]
        L.bo_sdpa.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_float, I32, I32]
        L.bo_sdpa_desc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_float, I32, I32]
        L.bo_rope.argtypes = [P, P, P, P, P, I64, I64, I64, I32]
        L.bo_silu_mul.argtypes = [P, P, P, I64, I32]
        L.bo_argmax.argtypes = [P, P, I64, I64, I32]
        L.bo_log_softmax.argtypes = [P, P, I64, I64, I32]
        L.bo_row_mean.argtypes = [P, P, I64, I64, I32]
        L.bo_num_threads.argtypes = []; L.bo_num_threads.restype = ctypes.c_int
        L.bo_set_num_threads.argtypes = [ctypes.c_int]; L.bo_set_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def _dt(dtype) -> int:
    return _DT[dtype] if isinstance(dtype, str) else int(dtype)


def num_threads() -> int:
    return lib().bo_num_threads()


def set_num_threads(n: int) -> int:
    """Threads of the oracle's parallel loops (over independent outputs only)."""
    return lib().bo_set_num_threads(int(n))


# --- number formats --------------------------------------------------------

def widen(bits: np.ndarray, dtype) -> np.ndarray:
    """bf16/f16 bit patterns (uint16) or fp32 values -> fp32 values."""
    a = np.ascontiguousarray(bits)
    out = np.empty(a.shape, np.float32)
    _check(lib().bo_widen(_p(a), _p(out), a.size, _dt(dtype)), "widen")
    return out


def round_to(values: np.ndarray, dtype) -> np.ndarray:
    """fp32 -> storage type with the oracle's RNE routine (uint16 bits for
    bf16/f16, float32 for f32)."""
    a = np.ascontiguousarray(values, dtype=np.float32)
    d = _dt(dtype)
    out = np.empty(a.shape, np.float32 if d == F32 else np.uint16)
    _check(lib().bo_round(_p(a), _p(out), a.size, d), "round")
    return out


def e2m1_value(code: int) -> float:
    return lib().bo_e2m1_to_f32(code)


def e4m3_value(code: int) -> float:
    return lib().bo_e4m3_to_f32(code)


def e8m0_value(code: int) -> float:
    return lib().bo_e8m0_to_f32(code)


# --- folds (Case 1 / Case 2) -------------------------------------------------

def fold_seq_f32(a) -> float:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return lib().bo_fold_seq_f32(_p(a), a.size)


def fold_seq_f64(a) -> float:
    a = np.ascontiguousarray(a, dtype=np.float64)
    return lib().bo_fold_seq_f64(_p(a), a.size)


def fold_pairwise_f32(a) -> float:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return lib().bo_fold_pairwise_f32(_p(a), a.size)


def fold_split_f32(a, splits: int) -> float:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return lib().bo_fold_split_f32(_p(a), a.size, splits)


# --- the four reductions -------------------------------------------------------

def matmul(x: np.ndarray, w: np.ndarray, dtype, w_transposed: bool = True, descending: bool = False) -> np.ndarray:
    """y = x @ W^T (W [N,K]) or x @ W (W [K,N]); fp32 [M,N].  Each output is a
    sequential fp32 fold over k ascending, or with descending=True over k
    descending -- a second valid fixed tree (the "reverse" order of the
    chapter's Case 4), used to measure how far two valid trees drift apart
    through a composed model."""
    x = np.ascontiguousarray(x); w = np.ascontiguousarray(w)
    M, K = x.shape
    N = w.shape[0] if w_transposed else w.shape[1]
    assert (w.shape[1] if w_transposed else w.shape[0]) == K
    y = np.empty((M, N), np.float32)
    fn = lib().bo_matmul_desc if descending else lib().bo_matmul
    _check(fn(_p(x), _p(w), _p(y), M, N, K, _dt(dtype), int(w_transposed)), "matmul")
    return y


def dequantize(wq, scales, biases, rows: int, cols: int, qmode: int, group_size: int, bits: int = 4) -> np.ndarray:
    """Packed `bits`-bit weights (each row a little-endian bit stream of codes
    in 32-bit words) -> binary16 bits [rows, cols]."""
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    scales = np.ascontiguousarray(scales)
    b = None if biases is None else np.ascontiguousarray(biases, dtype=np.uint16)
    out = np.empty((rows, cols), np.uint16)
    _check(lib().bo_dequantize(_p(wq), _p(scales), None if b is None else _p(b), _p(out),
                               rows, cols, qmode, bits, group_size), "dequantize")
    return out


def qmatmul(x, wq, scales, biases, M: int, N: int, K: int, qmode: int, group_size: int,
            w_transposed: bool = True, bits: int = 4) -> np.ndarray:
    """y = x @ dequantize(W)^T with x binary16 bits [M,K]; fp32 [M,N]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    scales = np.ascontiguousarray(scales)
    b = None if biases is None else np.ascontiguousarray(biases, dtype=np.uint16)
    y = np.empty((M, N), np.float32)
    _check(lib().bo_qmatmul(_p(x), _p(wq), _p(scales), None if b is None else _p(b), _p(y),
                            M, N, K, qmode, bits, group_size, int(w_transposed)), "qmatmul")
    return y


def gather_qmatmul(x, lhs, rhs, wq, scales, biases, N: int, K: int, qmode: int, group_size: int,
                   w_transposed: bool = True, bits: int = 4) -> np.ndarray:
    """Expert matmul: y[m] = x[lhs[m]] @ dequantize(W[rhs[m]])^T (lhs None:
    x[m]); wq, scales, biases stacked over the E experts on axis 0; fp32 [M,N]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    rhs = np.ascontiguousarray(rhs, dtype=np.int32)
    lh = None if lhs is None else np.ascontiguousarray(lhs, dtype=np.int32)
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    scales = np.ascontiguousarray(scales)
    b = None if biases is None else np.ascontiguousarray(biases, dtype=np.uint16)
    M, E = rhs.shape[0], wq.shape[0]
    y = np.empty((M, N), np.float32)
    _check(lib().bo_gather_qmatmul(_p(x), None if lh is None else _p(lh), _p(rhs), _p(wq), _p(scales),
                                   None if b is None else _p(b), _p(y), M, x.shape[0], N, K, E, qmode, bits,
                                   group_size, int(w_transposed)), "gather_qmatmul")
    return y


def rmsnorm(x: np.ndarray, w: np.ndarray, dtype, eps: float = 1e-6, return_ss: bool = False,
            descending: bool = False):
    """Sum of squares folded over i ascending (descending=True: the second
    valid tree, Case 4's reverse order)."""
    x = np.ascontiguousarray(x); w = np.ascontiguousarray(w)
    rows, H = x.shape
    y = np.empty((rows, H), np.float32)
    ss = np.empty(rows, np.float32)
    fn = lib().bo_rmsnorm_desc if descending else lib().bo_rmsnorm
    _check(fn(_p(x), _p(w), _p(y), _p(ss), rows, H, eps, _dt(dtype)), "rmsnorm")
    return (y, ss) if return_ss else y


def sdpa(q, k, v, kv_len, scale: float, causal: bool, dtype, descending: bool = False) -> np.ndarray:
    """q [B,Q,Hq,D]; k,v [B,Lcap,Hkv,D]; kv_len int32 [B] -> fp32 [B,Q,Hq,D].
    Every sum ascending (descending=True: over d and over keys descending)."""
    q = np.ascontiguousarray(q); k = np.ascontiguousarray(k); v = np.ascontiguousarray(v)
    kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
    B, Q, Hq, D = q.shape
    _, Lcap, Hkv, _ = k.shape
    o = np.empty((B, Q, Hq, D), np.float32)
    fn = lib().bo_sdpa_desc if descending else lib().bo_sdpa
    _check(fn(_p(q), _p(k), _p(v), _p(o), _p(kv_len), B, Q, Lcap, Hq, Hkv, D,
              scale, int(causal), _dt(dtype)), "sdpa")
    return o


def rope(x, pos, cos_t, sin_t, dtype) -> np.ndarray:
    """x [T, nh, D]; pos int32 [T]; cos/sin fp32 [P, D/2] -> fp32 [T, nh, D]."""
    x = np.ascontiguousarray(x)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    cos_t = np.ascontiguousarray(cos_t, dtype=np.float32)
    sin_t = np.ascontiguousarray(sin_t, dtype=np.float32)
    T, nh, D = x.shape
    out = np.empty((T, nh, D), np.float32)
    _check(lib().bo_rope(_p(x), _p(out), _p(pos), _p(cos_t), _p(sin_t), T, nh, D, _dt(dtype)), "rope")
    return out


def silu_mul(g, u, dtype) -> np.ndarray:
    g = np.ascontiguousarray(g); u = np.ascontiguousarray(u)
    out = np.empty(g.shape, np.float32)
    _check(lib().bo_silu_mul(_p(g), _p(u), _p(out), g.size, _dt(dtype)), "silu_mul")
    return out


def argmax(x, dtype) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    idx = np.empty(rows, np.int32)
    _check(lib().bo_argmax(_p(x), _p(idx), rows, cols, _dt(dtype)), "argmax")
    return idx


def log_softmax(x, dtype) -> np.ndarray:
    """fp32 [rows, cols]: (x - max) - log(sum exp(x - max)), the sum in
    ascending column order ("Batch-invariant kernels ...", The trap and
    Sources: the log-softmax / logprob outputs an RL trainer compares with its
    sampler)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float32)
    _check(lib().bo_log_softmax(_p(x), _p(y), rows, cols, _dt(dtype)), "log_softmax")
    return y


def row_mean(x, dtype) -> np.ndarray:
    """fp32 [rows]: the ascending fp32 sum of each row divided by cols."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    y = np.empty(rows, np.float32)
    _check(lib().bo_row_mean(_p(x), _p(y), rows, cols, _dt(dtype)), "row_mean")
    return y
