"""Helpers for the GPU tests: moving storage arrays to and from the device,
the tolerance metric, and guarded (canary / poison) allocations."""
from __future__ import annotations

import numpy as np
import torch

import invariant_reductions_amd as bi

TOL = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-5}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bi.lib()                                  # fail loudly if the HIP library is missing
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array (uint16 bits or float32) -> CUDA tensor of `dtype`."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(dev())
    return torch.from_numpy(a.view(np.int16)).to(dev()).view(TORCH[dtype])


def to_np(t: torch.Tensor) -> np.ndarray:
    """CUDA tensor -> storage array (uint16 bits for 16-bit types)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    from invariant_reductions_amd.inputs import from_storage
    return from_storage(bits, dtype)


def rel_err(gpu_bits: np.ndarray, ref32: np.ndarray, dtype: str) -> float:
    """Norm-wise relative error max|g - o| / max|o| (fp64)."""
    g = widen(gpu_bits, dtype).astype(np.float64)
    o = ref32.astype(np.float64)
    assert g.shape == o.shape
    assert np.array_equal(np.isnan(g), np.isnan(o)), "NaN positions differ"
    fin = ~np.isnan(o)
    den = np.abs(o[fin]).max() if fin.any() else 1.0
    return float(np.abs(g[fin] - o[fin]).max() / (den if den > 0 else 1.0))


def assert_parity(gpu_bits, ref32, dtype, what=""):
    e = rel_err(gpu_bits, ref32, dtype)
    assert e <= TOL[dtype], f"{what}: relative error {e:.3e} > {TOL[dtype]:.0e}"
    return e


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


class Guarded:
    """A device buffer whose logical extent is surrounded by `pad` bytes of a
    poison byte pattern on both sides; `view` is the logical tensor."""

    def __init__(self, shape, dtype: torch.dtype, pad_bytes: int = 4096, poison: int = 0xFF, init=None):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        assert pad_bytes % 16 == 0
        self.pad = pad_bytes
        self.nbytes = n * esz
        self.raw = torch.full((pad_bytes * 2 + self.nbytes,), poison, dtype=torch.uint8, device=dev())
        self.view = self.raw[pad_bytes:pad_bytes + self.nbytes].view(dtype).view(shape)
        if init is not None:
            self.view.copy_(init)
        self.poison = poison

    def canaries_intact(self) -> bool:
        r = self.raw.cpu().numpy()
        return bool(np.all(r[:self.pad] == self.poison) and np.all(r[self.pad + self.nbytes:] == self.poison))


def guarded_from(a: np.ndarray, dtype: str, poison: int = 0xFF, pad_bytes: int = 4096) -> Guarded:
    t = to_dev(a, dtype) if dtype in TORCH else torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return Guarded(tuple(t.shape), t.dtype, pad_bytes, poison, init=t)
