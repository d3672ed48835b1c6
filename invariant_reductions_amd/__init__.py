"""invariant_reductions_amd -- batch-invariant reductions for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/bi.h`` (``libbi.so``, built
in-tree by ``invariant_reductions_amd.build``).  The binding only marshals
arguments: it checks devices, dtypes and contiguity, passes raw device
pointers and torch's current HIP stream, and raises :class:`BIError` on a
non-OK status.  Every step of the computation runs in the HIP kernels; there
is no CPU path.  If the library has not been built, every op raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "BIError", "library_path", "lib", "build_info",
    "matmul", "matmul_ws", "matmul_workspace", "matmul_swiglu", "matmul_swiglu_workspace", "interleave_gate_up",
    "PackedWeight", "pack_weights", "pack_qweights", "log_softmax", "token_logprob", "row_mean",
    "qmatmul", "rmsnorm", "add_rmsnorm", "sdpa", "sdpa_workspace_bytes", "sdpa_noalloc",
    "matmul_split", "rmsnorm_split", "qmatmul_split", "sdpa_split",
    "embed", "rope_kv_write", "silu_mul", "add", "argmax",
    "BF16", "F16", "F32", "AFFINE", "NVFP4",
]

BF16, F16, F32 = 0, 1, 2
AFFINE, NVFP4, MXFP4, MXFP8 = 0, 1, 2, 3
_TORCH_DT = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libbi.so")


class BIError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib_handle.bi_status_str(status).decode() if _lib_handle is not None else str(status)
        super().__init__(f"{where}: {msg}")


_lib_handle = None


def lib():
    """The loaded libbi.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libbi.so not found at {path}; build it with "
                               "`python -m invariant_reductions_amd.build`")
        L = ctypes.CDLL(path)
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        SZ = ctypes.c_size_t
        sig = {
            "bi_matmul": [P, P, P, I64, I64, I64, I32, I32, P],
            "bi_qmatmul": [P, P, P, P, P, I64, I64, I64, I32, I32, I32, I32, P],
            "bi_gather_qmatmul": [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I32, I32, I32, I32, P],
            "bi_rmsnorm": [P, P, P, I64, I64, F, I32, P],
            "bi_add_rmsnorm": [P, P, P, P, P, I64, I64, F, I32, P],
            "bi_sdpa": [P, P, P, P, P, I64, I64, I64, I64, I32, I32, I32, F, I32, I32, I32, P, SZ, P],
            "bi_sdpa_noalloc": [P, P, P, P, P, I64, I64, I64, I64, I32, I32, I32, F, I32, I32, I32, P],
            "bi_embed": [P, P, P, I64, I64, I64, P],
            "bi_embed_rmsnorm": [P, P, P, P, P, I64, I64, I64, F, I32, P],
            "bi_rope_kv_write": [P, P, P, P, P, P, P, I64, I64, I64, I32, I32, I32, I64, I32, P],
            "bi_silu_mul": [P, P, I64, I64, P],
            "bi_add": [P, P, P, I64, P],
            "bi_argmax": [P, P, I64, I64, P],
            "bi_matmul_split": [P, P, P, I64, I64, I64, I32, I32, I32, P, SZ, P],
            "bi_matmul_ws": [P, P, P, I64, I64, I64, I32, I32, P, SZ, P],
            "bi_matmul_swiglu": [P, P, P, I64, I64, I64, I32, I32, P, SZ, P],
            "bi_pack_weights": [P, P, I64, I64, I32, P],
            "bi_pack_qweights": [P, P, P, P, I64, I64, I32, I32, I32, P],
            "bi_log_softmax": [P, P, I64, I64, I32, P],
            "bi_argmax_advance": [P, P, P, P, I64, I64, P],
            "bi_token_logprob": [P, P, P, I64, I64, I32, P],
            "bi_row_mean": [P, P, I64, I64, I32, P],
            "bi_rmsnorm_split": [P, P, P, I64, I64, F, I32, I32, P, SZ, P],
            "bi_qmatmul_split": [P, P, P, P, P, I64, I64, I64, I32, I32, I32, I32, I32, P, SZ, P],
            "bi_sdpa_split": [P, P, P, P, P, I64, I64, I64, I64, I32, I32, I32, F, I32, I32, I32, I32, P, SZ, P],
            "bi_probe_read": [P, SZ, P, I32, P],
            "bi_probe_copy": [P, P, SZ, I32, P],
            "bi_probe_mfma": [P, I32, I64, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        L.bi_sdpa_workspace_bytes.argtypes = [I64, I64, I64, I32, I32]
        L.bi_sdpa_workspace_bytes.restype = SZ
        L.bi_sdpa_noalloc_max_bytes.argtypes = []
        L.bi_sdpa_noalloc_max_bytes.restype = SZ
        L.bi_packed_qweight_bytes.argtypes = [I64, I64, I32, I32, I32]
        L.bi_packed_qweight_bytes.restype = SZ
        L.bi_packed_weight_bytes.argtypes = [I64, I64, I32]
        L.bi_packed_weight_bytes.restype = SZ
        L.bi_matmul_swiglu_workspace_bytes.argtypes = [I64, I64, I64, I32]
        L.bi_matmul_swiglu_workspace_bytes.restype = SZ
        L.bi_matmul_ws_workspace_bytes.argtypes = [I64, I64, I64, I32, I32]
        L.bi_matmul_ws_workspace_bytes.restype = SZ
        L.bi_matmul_split_workspace_bytes.argtypes = [I64, I64, I32]
        L.bi_matmul_split_workspace_bytes.restype = SZ
        L.bi_rmsnorm_split_workspace_bytes.argtypes = [I64, I32]
        L.bi_rmsnorm_split_workspace_bytes.restype = SZ
        L.bi_qmatmul_split_workspace_bytes.argtypes = [I64, I64, I32]
        L.bi_qmatmul_split_workspace_bytes.restype = SZ
        L.bi_sdpa_split_workspace_bytes.argtypes = [I64, I64, I64, I32, I32, I32]
        L.bi_sdpa_split_workspace_bytes.restype = SZ
        L.bi_time_next_launch.argtypes = [P, P]
        L.bi_time_next_launch.restype = ctypes.c_int32
        L.bi_time_next_launches.argtypes = [P, P, I32]
        L.bi_time_next_launches.restype = ctypes.c_int32
        L.bi_status_str.argtypes = [I32]
        L.bi_status_str.restype = ctypes.c_char_p
        L.bi_build_info.argtypes = []
        L.bi_build_info.restype = ctypes.c_char_p
        _lib_handle = L
    return _lib_handle


def build_info() -> str:
    return lib().bi_build_info().decode()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("invariant_reductions_amd ops take GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _dt(t) -> int:
    if t.dtype not in _TORCH_DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _TORCH_DT[t.dtype]


def _check(rc: int, where: str):
    if rc != 0:
        raise BIError(rc, where)


# ---------------------------------------------------------------------------
# the four reductions
# ---------------------------------------------------------------------------

W_NATURAL, W_TRANSPOSED, W_PACKED = 0, 1, 2


class PackedWeight:
    """A [N, K] weight in the tile-packed layout (bi_pack_weights): `data` is
    the packed buffer (ceil(N/16)*16 x K elements of the weight's dtype)."""

    def __init__(self, data: torch.Tensor, N: int, K: int):
        self.data, self.N, self.K = data, N, K
        self.dtype, self.device = data.dtype, data.device


def pack_weights(w: torch.Tensor, stream=None) -> PackedWeight:
    """[N, K] bf16/f16 (K % 128 == 0) -> PackedWeight (same bits in every
    dense entry point, fewer DRAM pages per byte streamed)."""
    _dev(w)
    N, K = w.shape
    nbytes = lib().bi_packed_weight_bytes(N, K, _dt(w))
    if nbytes == 0:
        raise ValueError("pack_weights: needs a bf16/f16 [N, K] weight with K % 128 == 0")
    wp = torch.empty(nbytes // w.element_size(), dtype=w.dtype, device=w.device)
    _check(lib().bi_pack_weights(_ptr(w), _ptr(wp), N, K, _dt(w), _stream(stream)), "bi_pack_weights")
    return PackedWeight(wp, N, K)


def _wargs(w, transposed: bool, K: int, dtype, where: str):
    """(tensor, N, layout) of a weight argument: a PackedWeight, or a tensor
    [N, K] (transposed) / [K, N]."""
    if isinstance(w, PackedWeight):
        if w.K != K or w.dtype != dtype:
            raise ValueError(f"{where}: shape/dtype mismatch")
        return w.data, w.N, W_PACKED
    N = w.shape[0] if transposed else w.shape[1]
    if (w.shape[1] if transposed else w.shape[0]) != K or w.dtype != dtype:
        raise ValueError(f"{where}: shape/dtype mismatch")
    return w, N, W_TRANSPOSED if transposed else W_NATURAL


def matmul(x: torch.Tensor, w, transposed: bool = True, out=None, stream=None):
    """y = x @ w.T (w [N,K], transposed=True), x @ w (w [K,N]), or with a
    PackedWeight of [N,K]."""
    M, K = x.shape
    wt, N, layout = _wargs(w, transposed, K, x.dtype, "matmul")
    _dev(x, wt, out)
    y = out if out is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(lib().bi_matmul(_ptr(x), _ptr(wt), _ptr(y), M, N, K, _dt(x), layout, _stream(stream)), "bi_matmul")
    return y


def matmul_workspace(M: int, N: int, K: int, dtype=torch.bfloat16, transposed: bool = True, device=None):
    """A zero-filled workspace for `matmul_ws` at this shape (a 16-byte
    placeholder when the shape needs none)."""
    need = lib().bi_matmul_ws_workspace_bytes(M, N, K, _TORCH_DT[dtype], int(transposed))
    return torch.zeros(max(int(need), 16), dtype=torch.uint8, device=device)


def matmul_ws(x: torch.Tensor, w, ws: torch.Tensor, transposed: bool = True, out=None, stream=None):
    """Same bits as `matmul`; `ws` from `matmul_workspace` (or any zero-filled
    buffer of at least the workspace size), reused across calls in stream
    order.  `w` as in `matmul`."""
    M, K = x.shape
    wt, N, layout = _wargs(w, transposed, K, x.dtype, "matmul_ws")
    _dev(x, wt, out, ws)
    y = out if out is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(lib().bi_matmul_ws(_ptr(x), _ptr(wt), _ptr(y), M, N, K, _dt(x), layout, _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(stream)), "bi_matmul_ws")
    return y


def interleave_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """[2F, K] weight for matmul_swiglu: gate and up rows interleaved in
    blocks of 8 (a layout change done once, on any device)."""
    F, K = w_gate.shape
    if w_up.shape != (F, K) or F % 8:
        raise ValueError("interleave_gate_up: gate/up must be [F, K] with F % 8 == 0")
    return torch.stack([w_gate.view(F // 8, 8, K), w_up.view(F // 8, 8, K)], dim=1).reshape(2 * F, K).contiguous()


def matmul_swiglu_workspace(M: int, F: int, K: int, device=None):
    """A zero-filled workspace for matmul_swiglu at this shape."""
    need = lib().bi_matmul_swiglu_workspace_bytes(M, F, K, BF16)
    return torch.zeros(max(int(need), 16), dtype=torch.uint8, device=device)


def matmul_swiglu(x: torch.Tensor, w_il, ws: torch.Tensor, out=None, stream=None):
    """a = silu(x @ Wg^T) * (x @ Wu^T), bitwise matmul + silu_mul; w_il from
    interleave_gate_up, as a [2F, K] tensor or packed by pack_weights."""
    M, K = x.shape
    if x.dtype != torch.bfloat16:
        raise ValueError("matmul_swiglu: bf16 only")
    wt, N2, layout = _wargs(w_il, True, K, x.dtype, "matmul_swiglu")
    _dev(x, wt, out, ws)
    if N2 % 16:
        raise ValueError("matmul_swiglu: 2F must be a multiple of 16")
    F = N2 // 2
    a = out if out is not None else torch.empty((M, F), dtype=x.dtype, device=x.device)
    _check(lib().bi_matmul_swiglu(_ptr(x), _ptr(wt), _ptr(a), M, F, K, BF16, layout, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "bi_matmul_swiglu")
    return a


def matmul_split(x, w, splits: int, transposed: bool = True, out=None, ws=None, stream=None):
    """Non-invariant split-K comparison variant (see include/bi.h)."""
    M, K = x.shape
    wt, N, layout = _wargs(w, transposed, K, x.dtype, "matmul_split")
    _dev(x, wt, out, ws)
    y = out if out is not None else torch.empty((M, N), dtype=x.dtype, device=x.device)
    need = lib().bi_matmul_split_workspace_bytes(M, N, splits)
    if ws is None and splits > 1:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().bi_matmul_split(_ptr(x), _ptr(wt), _ptr(y), M, N, K, _dt(x), layout, splits,
                                 _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "bi_matmul_split")
    return y


def qmatmul(x, wq, scales, biases, N: int, K: int, qmode: int, group_size: int, transposed: bool = True,
            out=None, stream=None, packed: bool = False, bits: int = 4):
    """y = x @ dequantize(W)^T; x float16 [M,K]; wq int32 (uint32 bit patterns:
    each stored row a little-endian stream of `bits`-bit codes), or
    (packed=True, 4-bit modes) the buffer of pack_qweights, with scales/biases
    None.  bits: 2..8 for AFFINE, 4 for NVFP4 and MXFP4, 8 for MXFP8."""
    _dev(x, wq, scales, biases, out)
    if x.dtype != torch.float16:
        raise ValueError("qmatmul: x must be float16")
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("qmatmul: x shape")
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    layout = W_PACKED if packed else (W_TRANSPOSED if transposed else W_NATURAL)
    _check(lib().bi_qmatmul(_ptr(x), _ptr(wq), _ptr(scales), _ptr(biases), _ptr(y), M, N, K, qmode, bits,
                            group_size, layout, _stream(stream)), "bi_qmatmul")
    return y


def qmatmul_split(x, wq, scales, biases, N: int, K: int, qmode: int, group_size: int, splits: int,
                  transposed: bool = True, out=None, ws=None, stream=None, packed: bool = False, bits: int = 4):
    """Non-invariant split-K comparison variant of qmatmul (see include/bi.h)."""
    _dev(x, wq, scales, biases, out, ws)
    M = x.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    need = lib().bi_qmatmul_split_workspace_bytes(M, N, splits)
    if ws is None and splits > 1:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    layout = W_PACKED if packed else (W_TRANSPOSED if transposed else W_NATURAL)
    _check(lib().bi_qmatmul_split(_ptr(x), _ptr(wq), _ptr(scales), _ptr(biases), _ptr(y), M, N, K, qmode, bits,
                                  group_size, layout, splits, _ptr(ws),
                                  0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "bi_qmatmul_split")
    return y


def gather_qmatmul(x, lhs, rhs, wq, scales, biases, N: int, K: int, qmode: int, group_size: int,
                   transposed: bool = True, out=None, stream=None, bits: int = 4, packed: bool = False):
    """Expert matmul: y[m] = x[lhs[m]] @ dequantize(W[rhs[m]])^T; x float16
    [x_rows, K]; lhs (or None: row m) and rhs int32 [M] on the device; wq,
    scales, biases stacked over the experts on dim 0 -- or (packed=True) wq
    the experts' pack_qweights buffers stacked on dim 0, scales/biases None."""
    _dev(x, lhs, rhs, wq, scales, biases, out)
    if x.dtype != torch.float16 or rhs.dtype != torch.int32 or (lhs is not None and lhs.dtype != torch.int32):
        raise ValueError("gather_qmatmul: x float16, indices int32")
    if x.shape[1] != K:
        raise ValueError("gather_qmatmul: x shape")
    M, E = rhs.shape[0], wq.shape[0]
    y = out if out is not None else torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check(lib().bi_gather_qmatmul(_ptr(x), _ptr(lhs), _ptr(rhs), _ptr(wq), _ptr(scales), _ptr(biases), _ptr(y),
                                   M, x.shape[0], N, K, E, qmode, bits, group_size,
                                   W_PACKED if packed else (W_TRANSPOSED if transposed else W_NATURAL),
                                   _stream(stream)), "bi_gather_qmatmul")
    return y


def pack_qweights(wq, scales, biases, N: int, K: int, qmode: int, group_size: int, stream=None,
                  bits: int = 4) -> torch.Tensor:
    """Transposed quantized weights -> the packed buffer qmatmul(packed=True) reads."""
    _dev(wq, scales, biases)
    nbytes = lib().bi_packed_qweight_bytes(N, K, qmode, bits, group_size)
    if nbytes == 0:
        raise ValueError("pack_qweights: needs K % 128 == 0 and a legal mode / group size")
    wqp = torch.empty(nbytes // 4, dtype=torch.int32, device=wq.device)
    _check(lib().bi_pack_qweights(_ptr(wq), _ptr(scales), _ptr(biases), _ptr(wqp), N, K, qmode, bits, group_size,
                                  _stream(stream)), "bi_pack_qweights")
    return wqp


def rmsnorm(x, w, eps: float = 1e-6, out=None, stream=None):
    _dev(x, w, out)
    rows, H = x.shape
    y = out if out is not None else torch.empty_like(x)
    _check(lib().bi_rmsnorm(_ptr(x), _ptr(w), _ptr(y), rows, H, eps, _dt(x), _stream(stream)), "bi_rmsnorm")
    return y


def add_rmsnorm(x, r, w, eps: float = 1e-6, x_out=None, out=None, stream=None):
    """x_out = x + r (rounded as `add`), out = rmsnorm(x_out); x_out may be x."""
    _dev(x, r, w, x_out, out)
    rows, H = x.shape
    xo = x_out if x_out is not None else torch.empty_like(x)
    y = out if out is not None else torch.empty_like(x)
    _check(lib().bi_add_rmsnorm(_ptr(x), _ptr(r), _ptr(xo), _ptr(w), _ptr(y), rows, H, eps, _dt(x), _stream(stream)),
           "bi_add_rmsnorm")
    return xo, y


def rmsnorm_split(x, w, splits: int, eps: float = 1e-6, out=None, ws=None, stream=None):
    _dev(x, w, out, ws)
    rows, H = x.shape
    y = out if out is not None else torch.empty_like(x)
    need = lib().bi_rmsnorm_split_workspace_bytes(rows, splits)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _check(lib().bi_rmsnorm_split(_ptr(x), _ptr(w), _ptr(y), rows, H, eps, _dt(x), splits, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "bi_rmsnorm_split")
    return y


def sdpa_workspace_bytes(B: int, Q: int, max_kv_len: int, Hq: int, D: int) -> int:
    return lib().bi_sdpa_workspace_bytes(B, Q, max_kv_len, Hq, D)


def sdpa(q, k, v, kv_len, max_kv_len: int, scale: float, causal: bool = True, out=None, ws=None, stream=None,
         head_major: bool = False):
    """q [B,Q,Hq,D]; k, v [B,Lcap,Hkv,D] (or [B,Hkv,Lcap,D] with head_major);
    kv_len int32 [B] on the device."""
    _dev(q, k, v, kv_len, out, ws)
    B, Q, Hq, D = q.shape
    if head_major:
        _, Hkv, Lcap, _ = k.shape
    else:
        _, Lcap, Hkv, _ = k.shape
    if kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32")
    o = out if out is not None else torch.empty_like(q)
    need = sdpa_workspace_bytes(B, Q, max_kv_len, Hq, D)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().bi_sdpa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv_len), max_kv_len, B, Q, Lcap, Hq, Hkv, D,
                         scale, int(causal), _dt(q), int(head_major), _ptr(ws), ws.numel() * ws.element_size(),
                         _stream(stream)), "bi_sdpa")
    return o


def sdpa_split(q, k, v, kv_len, max_kv_len: int, scale: float, splits: int, causal: bool = True, out=None,
               ws=None, stream=None, head_major: bool = False):
    """Non-invariant split-KV comparison variant of sdpa (see include/bi.h)."""
    _dev(q, k, v, kv_len, out, ws)
    B, Q, Hq, D = q.shape
    if head_major:
        _, Hkv, Lcap, _ = k.shape
    else:
        _, Lcap, Hkv, _ = k.shape
    if kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32")
    o = out if out is not None else torch.empty_like(q)
    need = lib().bi_sdpa_split_workspace_bytes(B, Q, max_kv_len, Hq, D, splits)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().bi_sdpa_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv_len), max_kv_len, B, Q, Lcap, Hq, Hkv, D,
                               scale, int(causal), _dt(q), int(head_major), splits, _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)), "bi_sdpa_split")
    return o


def sdpa_noalloc(q, k, v, kv_len, max_kv_len: int, scale: float, causal: bool = True, out=None, stream=None,
                 head_major: bool = False):
    """bi_sdpa on the library's fixed per-GPU scratch (no workspace, nothing
    allocated by the call itself except `out` when it is not given)."""
    _dev(q, k, v, kv_len, out)
    B, Q, Hq, D = q.shape
    if head_major:
        _, Hkv, Lcap, _ = k.shape
    else:
        _, Lcap, Hkv, _ = k.shape
    if kv_len.dtype != torch.int32:
        raise ValueError("kv_len must be int32")
    o = out if out is not None else torch.empty_like(q)
    _check(lib().bi_sdpa_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(kv_len), max_kv_len, B, Q, Lcap, Hq, Hkv,
                                 D, scale, int(causal), _dt(q), int(head_major), _stream(stream)), "bi_sdpa_noalloc")
    return o


# ---------------------------------------------------------------------------
# decoder glue
# ---------------------------------------------------------------------------

def embed(ids, table, out=None, stream=None):
    _dev(ids, table, out)
    T = ids.numel()
    V, H = table.shape
    y = out if out is not None else torch.empty((T, H), dtype=table.dtype, device=table.device)
    _check(lib().bi_embed(_ptr(ids), _ptr(table), _ptr(y), T, V, H, _stream(stream)), "bi_embed")
    return y


def embed_rmsnorm(ids, table, w, eps: float = 1e-6, x_out=None, out=None, stream=None):
    """x_out = embed(ids, table), out = rmsnorm(x_out, w) in one launch (same bits)."""
    _dev(ids, table, w, x_out, out)
    T = ids.numel()
    V, H = table.shape
    xo = x_out if x_out is not None else torch.empty((T, H), dtype=table.dtype, device=table.device)
    y = out if out is not None else torch.empty((T, H), dtype=table.dtype, device=table.device)
    _check(lib().bi_embed_rmsnorm(_ptr(ids), _ptr(table), _ptr(xo), _ptr(w), _ptr(y), T, V, H, eps, _dt(table),
                                  _stream(stream)), "bi_embed_rmsnorm")
    return xo, y


def rope_kv_write(qkv, q_out, kc, vc, kv_len, cos_t, sin_t, B: int, Q: int, Hq: int, Hkv: int, D: int, stream=None,
                  head_major: bool = False):
    """Caches [B,Lcap,Hkv,D], or [B,Hkv,Lcap,D] with head_major."""
    _dev(qkv, q_out, kc, vc, kv_len, cos_t, sin_t)
    Lcap = kc.shape[2] if head_major else kc.shape[1]
    _check(lib().bi_rope_kv_write(_ptr(qkv), _ptr(q_out), _ptr(kc), _ptr(vc), _ptr(kv_len), _ptr(cos_t),
                                  _ptr(sin_t), B, Q, Lcap, Hq, Hkv, D, cos_t.shape[0], int(head_major),
                                  _stream(stream)), "bi_rope_kv_write")


def silu_mul(gu, out=None, stream=None):
    _dev(gu, out)
    rows, F2 = gu.shape
    y = out if out is not None else torch.empty((rows, F2 // 2), dtype=gu.dtype, device=gu.device)
    _check(lib().bi_silu_mul(_ptr(gu), _ptr(y), rows, F2 // 2, _stream(stream)), "bi_silu_mul")
    return y


def add(a, b, out=None, stream=None):
    _dev(a, b, out)
    y = out if out is not None else torch.empty_like(a)
    _check(lib().bi_add(_ptr(a), _ptr(b), _ptr(y), a.numel(), _stream(stream)), "bi_add")
    return y


def argmax(x, out=None, stream=None):
    _dev(x, out)
    rows, cols = x.shape
    y = out if out is not None else torch.empty(rows, dtype=torch.int32, device=x.device)
    _check(lib().bi_argmax(_ptr(x), _ptr(y), rows, cols, _stream(stream)), "bi_argmax")
    return y


# ---------------------------------------------------------------------------
# log-probabilities and means
# ---------------------------------------------------------------------------

def log_softmax(x, out=None, stream=None):
    """fp32 [rows, cols] log-softmax of x [rows, cols] (bf16/f16/f32)."""
    _dev(x, out)
    rows, cols = x.shape
    y = out if out is not None else torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    _check(lib().bi_log_softmax(_ptr(x), _ptr(y), rows, cols, _dt(x), _stream(stream)), "bi_log_softmax")
    return y


def token_logprob(x, ids, out=None, stream=None):
    """fp32 [rows]: log_softmax(x)[r, ids[r]], bit for bit; ids int32 [rows] on the device."""
    _dev(x, ids, out)
    rows, cols = x.shape
    if ids.dtype != torch.int32 or ids.numel() != rows:
        raise ValueError("token_logprob: ids must be int32 [rows]")
    y = out if out is not None else torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib().bi_token_logprob(_ptr(x), _ptr(ids), _ptr(y), rows, cols, _dt(x), _stream(stream)),
           "bi_token_logprob")
    return y


def row_mean(x, out=None, stream=None):
    """fp32 [rows] mean of each row of x [rows, cols]."""
    _dev(x, out)
    rows, cols = x.shape
    y = out if out is not None else torch.empty(rows, dtype=torch.float32, device=x.device)
    _check(lib().bi_row_mean(_ptr(x), _ptr(y), rows, cols, _dt(x), _stream(stream)), "bi_row_mean")
    return y
