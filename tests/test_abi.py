"""The C-ABI library loads on the host, exports every entry point its header
declares, and rejects bad arguments with the documented status codes before
touching the GPU (no test here launches anything)."""
import ctypes
import os
import re

import pytest

import invariant_reductions_amd as bi
from conftest import ROOT

HDR = os.path.join(ROOT, "include", "bi.h")

P = ctypes.c_void_p
A = P(0x10000)          # 16-byte aligned, never dereferenced: every call below fails validation first
ODD = P(0x10001)        # misaligned for every element size: always rejected

OK, NULL, SHAPE, DTYPE, GROUP, ALIGN, WORKSPACE, LAUNCH, UNSUP = range(9)


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", text)))


def test_library_builds_into_the_package():
    assert os.path.exists(bi.library_path()), "run `python -m invariant_reductions_amd.build` first"


def test_every_declared_symbol_is_exported():
    L = bi.lib()
    names = declared_functions()
    assert "bi_matmul" in names and "bi_qmatmul" in names and "bi_rmsnorm" in names and "bi_sdpa" in names
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_status_strings_and_build_info():
    L = bi.lib()
    for s in range(9):
        assert L.bi_status_str(s)
    assert b"unknown" in L.bi_status_str(99)
    info = bi.build_info()
    assert "gfx950" in info and "256 keys" in info


@pytest.mark.parametrize("args,code", [
    ((None, A, A, 4, 512, 4096, 0, 1), NULL),
    ((A, None, A, 4, 512, 4096, 0, 1), NULL),
    ((A, A, A, 0, 512, 4096, 0, 1), SHAPE),
    ((A, A, A, 4, -1, 4096, 0, 1), SHAPE),
    ((A, A, A, 4, 512, 0, 0, 1), SHAPE),
    ((A, A, A, 4, 512, 4096, 7, 1), DTYPE),
    ((ODD, A, A, 4, 512, 4096, 0, 1), ALIGN),
    ((A, A, ODD, 4, 512, 4096, 0, 1), ALIGN),
])
def test_matmul_validation(args, code):
    assert bi.lib().bi_matmul(*args, None) == code


@pytest.mark.parametrize("M,N,K,qmode,bits,gs,trans,biases,code", [
    (1, 512, 4096, 0, 1, 32, 1, A, GROUP),          # affine bits 2..8
    (1, 512, 4096, 0, 9, 32, 1, A, GROUP),
    (1, 512, 4096, 1, 8, 16, 1, None, GROUP),       # nvfp4 is 4-bit
    (1, 512, 4096, 2, 8, 32, 1, None, GROUP),       # mxfp4 is 4-bit
    (1, 512, 4096, 3, 4, 32, 1, None, GROUP),       # mxfp8 is 8-bit
    (1, 512, 4096, 3, 8, 16, 1, None, GROUP),       # mxfp8 needs gs 32
    (1, 512, 4096, 3, 8, 32, 1, A, GROUP),          # mxfp8 takes no biases
    (1, 512, 4096, 0, 3, 32, 1, None, NULL),        # affine needs biases at any width
    (50, 128, 1040, 0, 8, 32, 1, A, GROUP),         # K % gs != 0 at 8 bits
    (64, 100, 32768, 3, 8, 32, 0, None, GROUP),     # natural mxfp8: 100 % 32 != 0
    (1, 512, 4096, 0, 4, 48, 1, A, GROUP),          # illegal affine group size
    (1, 512, 4096, 0, 4, 16, 1, A, GROUP),          # 16 is nvfp4 only
    (1, 512, 4096, 1, 4, 32, 1, None, GROUP),       # nvfp4 needs gs 16
    (1, 512, 4096, 1, 4, 16, 1, A, GROUP),          # nvfp4 takes no biases
    (1, 512, 4096, 0, 4, 32, 1, None, NULL),        # affine needs biases
    (50, 128, 1040, 0, 4, 32, 1, A, GROUP),         # affine K % gs != 0 (transposed)
    (64, 100, 32768, 0, 4, 32, 0, A, GROUP),        # natural layout quantizes N: 100 % 32 != 0
    (1, 512, 4096, 2, 4, 16, 1, None, GROUP),       # mxfp4 needs gs 32
    (1, 512, 4096, 2, 4, 32, 1, A, GROUP),          # mxfp4 takes no biases
    (1, 512, 4096, 4, 4, 32, 1, None, GROUP),       # unknown mode
    (0, 512, 4096, 0, 4, 32, 1, A, SHAPE),
])
def test_qmatmul_validation(M, N, K, qmode, bits, gs, trans, biases, code):
    assert bi.lib().bi_qmatmul(A, A, A, biases, A, M, N, K, qmode, bits, gs, trans, None) == code


def test_rmsnorm_validation():
    L = bi.lib()
    assert L.bi_rmsnorm(None, A, A, 4, 4096, 1e-6, 0, None) == NULL
    assert L.bi_rmsnorm(A, A, A, 0, 4096, 1e-6, 0, None) == SHAPE
    assert L.bi_rmsnorm(A, A, A, 4, 0, 1e-6, 0, None) == SHAPE
    assert L.bi_rmsnorm(A, A, A, 4, 4096, -1.0, 0, None) == SHAPE
    assert L.bi_rmsnorm(A, A, A, 4, 4096, float("nan"), 0, None) == SHAPE
    assert L.bi_rmsnorm(A, A, A, 4, 4096, 1e-6, 5, None) == DTYPE
    assert L.bi_rmsnorm(A, ODD, A, 4, 4096, 1e-6, 0, None) == ALIGN


def test_sdpa_validation_and_workspace_size():
    L = bi.lib()
    ws_need = L.bi_sdpa_workspace_bytes(1, 8, 65540, 32, 128)
    assert ws_need == 1 * 8 * 32 * 257 * 132 * 4           # one fp32 partial per (query row, chunk)
    assert L.bi_sdpa_workspace_bytes(1, 8, 65540, 32, 64) == 0
    def call(**kw):
        a = dict(q=A, k=A, v=A, o=A, kv=A, maxkv=1028, B=1, Q=8, Lcap=2048, Hq=32, Hkv=8, D=128,
                 scale=0.088, causal=1, dt=0, ws=A, wsb=10 ** 9)
        a.update(kw)
        return L.bi_sdpa(a["q"], a["k"], a["v"], a["o"], a["kv"], a["maxkv"], a["B"], a["Q"], a["Lcap"],
                         a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["dt"], a.get("lay", 0), a["ws"],
                         a["wsb"], None)
    assert call(kv=None) == NULL
    assert call(lay=2) == SHAPE                     # no such cache layout
    assert call(Hkv=5) == SHAPE
    assert call(maxkv=4) == SHAPE                   # max_kv_len < Q
    assert call(maxkv=4096) == SHAPE                # max_kv_len > Lcap
    assert call(D=64) == UNSUP
    assert call(dt=2) == DTYPE
    assert call(ws=None) == WORKSPACE
    assert call(wsb=100) == WORKSPACE
    assert call(q=ODD) == ALIGN


def test_split_variant_validation():
    L = bi.lib()
    assert L.bi_matmul_split(A, A, A, 4, 512, 4096, 0, 1, 0, A, 10 ** 9, None) == SHAPE
    assert L.bi_matmul_split(A, A, A, 4, 512, 4096, 0, 1, 4, None, 0, None) == WORKSPACE
    assert L.bi_matmul_split(A, A, A, 4, 512, 4096, 0, 1, 4, A, 16, None) == WORKSPACE
    assert L.bi_rmsnorm_split(A, A, A, 4, 4096, 1e-6, 0, 4, None, 0, None) == WORKSPACE
    assert L.bi_matmul_split_workspace_bytes(4, 512, 8) == 4 * 512 * 8 * 4


def test_quantized_and_attention_split_validation():
    L = bi.lib()
    MX = bi.MXFP4
    # qmatmul_split(x, wq, scales, biases, y, M, N, K, qmode, bits, gs, layout, splits, ws, ws_bytes, stream)
    assert L.bi_qmatmul_split(A, A, A, None, A, 4, 512, 4096, MX, 4, 32, 1, 0, A, 10 ** 9, None) == SHAPE
    assert L.bi_qmatmul_split(A, A, A, None, A, 4, 512, 4096, MX, 4, 32, 1, 33, A, 10 ** 9, None) == SHAPE
    assert L.bi_qmatmul_split(A, A, A, None, A, 32, 512, 4096, MX, 4, 32, 1, 4, A, 10 ** 9, None) == UNSUP
    assert L.bi_qmatmul_split(A, A, A, None, A, 4, 512, 4096, MX, 4, 32, 0, 4, A, 10 ** 9, None) == UNSUP
    assert L.bi_qmatmul_split(A, A, A, None, A, 4, 512, 4096, MX, 4, 32, 1, 4, None, 0, None) == WORKSPACE
    assert L.bi_qmatmul_split(A, A, A, None, A, 4, 512, 4096, MX, 4, 32, 1, 4, A, 16, None) == WORKSPACE
    assert L.bi_qmatmul_split(A, A, A, None, A, 4, 512, 4096, MX, 4, 31, 1, 4, A, 10 ** 9, None) == GROUP
    assert L.bi_qmatmul_split_workspace_bytes(4, 512, 8) == 4 * 512 * 8 * 4
    f = ctypes.c_float(0.1)
    # sdpa_split(q, k, v, o, kv, max_kv, B, Q, Lcap, Hq, Hkv, D, scale, causal, dtype, layout, splits, ws, wsb, st)
    assert L.bi_sdpa_split(A, A, A, A, A, 1000, 2, 1, 1024, 32, 8, 128, f, 1, 0, 0, 0, A, 10 ** 9, None) == SHAPE
    assert L.bi_sdpa_split(A, A, A, A, A, 1000, 2, 5, 1024, 32, 8, 128, f, 1, 0, 0, 2, A, 10 ** 9, None) == UNSUP
    assert L.bi_sdpa_split(A, A, A, A, A, 1000, 2, 1, 1024, 32, 8, 128, f, 1, 0, 0, 2, None, 0, None) == WORKSPACE
    # 1000 keys = 4 chunks: 3 splits -> runs of 2 chunks -> 2 partials per row
    assert L.bi_sdpa_split_workspace_bytes(2, 1, 1000, 32, 128, 3) == 2 * 32 * 2 * 132 * 4
    assert L.bi_sdpa_split_workspace_bytes(2, 1, 1000, 32, 128, 1) == 0
    assert L.bi_sdpa_split_workspace_bytes(2, 1, 1000, 32, 128, 99) == 2 * 32 * 4 * 132 * 4


def test_matmul_ws_validation_and_workspace_size():
    """Workspace errors are reported before any launch; shapes that need no
    workspace report 0 bytes."""
    L = bi.lib()
    need = L.bi_matmul_ws_workspace_bytes(64, 4096, 4096, 0, 1)
    # fixed 64 KiB counter area + 32 column tiles x 8 groups x 8 waves x 4 KiB records
    assert need == 65536 + 32 * 8 * 8 * 4 * 4 * 64 * 4
    # from 17 rows the slot form takes four 16-row tiles (records of 4 KiB)
    assert L.bi_matmul_ws_workspace_bytes(17, 4096, 4096, 0, 1) == 65536 + 32 * 8 * 8 * 4 * 4 * 64 * 4
    assert L.bi_matmul_ws_workspace_bytes(16, 4096, 4096, 0, 1) == 0      # short M: bi_matmul's kernels
    assert L.bi_matmul_ws_workspace_bytes(8, 28672, 4096, 0, 1) == 0
    # 8 < M <= 16 on a large weight: the slot form, 16-row tiles (1 KiB records)
    assert L.bi_matmul_ws_workspace_bytes(9, 28672, 4096, 0, 1) == 65536 + 224 * 8 * 8 * 1 * 4 * 64 * 4
    assert L.bi_matmul_ws_workspace_bytes(64, 128 * 16385, 128, 0, 1) == 0   # beyond the counter area
    # past 64 rows on a narrow weight (256 CUs assumed without a GPU): every
    # 64-row chunk has its own group sums
    assert L.bi_matmul_ws_workspace_bytes(65, 4096, 4096, 0, 1) == 65536 + 2 * 32 * 8 * 8 * 4 * 4 * 64 * 4
    assert L.bi_matmul_ws_workspace_bytes(100, 28672, 4096, 0, 1) == 0    # wide: bi_matmul's tiled kernel
    assert L.bi_matmul_ws_workspace_bytes(129, 4096, 4096, 0, 1) == 0     # longer M: bi_matmul's kernels
    assert L.bi_matmul_ws_workspace_bytes(64, 4096, 4096, 2, 1) == 0      # f32
    assert L.bi_matmul_ws_workspace_bytes(64, 4096, 4096, 0, 0) == 0      # natural layout
    assert L.bi_matmul_ws(A, A, A, 64, 4096, 4096, 0, 1, None, 0, None) == WORKSPACE
    assert L.bi_matmul_ws(A, A, A, 64, 4096, 4096, 0, 1, A, need - 1, None) == WORKSPACE
    assert L.bi_matmul_ws(A, A, A, 64, 4096, 4096, 0, 1, P(0x10010 + 2), need, None) == ALIGN
    assert L.bi_matmul_ws(ODD, A, A, 64, 4096, 4096, 0, 1, A, need, None) == ALIGN
    assert L.bi_matmul_ws(A, A, A, 0, 4096, 4096, 0, 1, A, need, None) == SHAPE
    assert L.bi_matmul_ws(A, A, A, 64, 4096, 4096, 7, 1, A, need, None) == DTYPE


def test_matmul_swiglu_validation_and_workspace_size():
    """bf16 only, F a multiple of 64, a 16-byte aligned output and a workspace
    of the reported size; errors come before any launch."""
    L = bi.lib()
    need = L.bi_matmul_swiglu_workspace_bytes(64, 14336, 4096, 0)
    # the 64 KiB counter area, then the slot form's group sums or a scratch [M, 2F] bf16 product
    assert need == L.bi_matmul_ws_workspace_bytes(64, 2 * 14336, 4096, 0, 1)      # group sums are the larger
    assert L.bi_matmul_swiglu_workspace_bytes(1, 64, 128, 0) == 65536 + 256       # 1 x 128 bf16, 256-byte rounded
    assert L.bi_matmul_swiglu_workspace_bytes(1, 8, 128, 0) == 65536 + 256        # F = 8: one interleave block
    assert L.bi_matmul_swiglu_workspace_bytes(65, 14336, 4096, 0) == 65536 + 65 * 2 * 14336 * 2
    assert L.bi_matmul_swiglu_workspace_bytes(64, 14336, 4096, 1) == 0            # f16
    assert L.bi_matmul_swiglu_workspace_bytes(64, 100, 4096, 0) == 0              # F % 8
    assert L.bi_matmul_swiglu(A, A, A, 64, 14336, 4096, 0, 1, None, 0, None) == WORKSPACE
    assert L.bi_matmul_swiglu(A, A, A, 64, 14336, 4096, 0, 1, A, need - 1, None) == WORKSPACE
    assert L.bi_matmul_swiglu(A, A, A, 64, 14336, 4096, 1, 1, A, need, None) == DTYPE
    assert L.bi_matmul_swiglu(A, A, A, 64, 100, 4096, 0, 1, A, need, None) == SHAPE
    assert L.bi_matmul_swiglu(A, A, A, 0, 14336, 4096, 0, 1, A, need, None) == SHAPE
    assert L.bi_matmul_swiglu(A, A, P(0x10010 + 2), 64, 14336, 4096, 0, 1, A, need, None) == ALIGN
    assert L.bi_matmul_swiglu(A, A, A, 64, 14336, 4096, 0, 1, P(0x10010 + 2), need, None) == ALIGN
    assert L.bi_matmul_swiglu(None, A, A, 64, 14336, 4096, 0, 1, A, need, None) == NULL


def test_packed_weight_validation():
    """Packing needs a 16-bit [N, K] weight with K % 128 == 0 and 16-byte
    aligned buffers; the packed layout is refused where the kernels cannot
    read it, before any launch."""
    L = bi.lib()
    assert L.bi_packed_weight_bytes(37, 384, 0) == 48 * 384 * 2
    assert L.bi_packed_weight_bytes(16, 384, 1) == 16 * 384 * 2
    assert L.bi_packed_weight_bytes(16, 100, 0) == 0        # K % 128
    assert L.bi_packed_weight_bytes(16, 128, 2) == 0        # f32
    assert L.bi_pack_weights(None, A, 16, 128, 0, None) == NULL
    assert L.bi_pack_weights(A, A, 16, 100, 0, None) == SHAPE
    assert L.bi_pack_weights(A, A, 16, 128, 2, None) == DTYPE
    assert L.bi_pack_weights(A, P(0x10010 + 2), 16, 128, 0, None) == ALIGN
    assert L.bi_matmul(A, A, A, 4, 16, 100, 0, 2, None) == SHAPE       # packed needs K % 128 == 0
    assert L.bi_matmul(A, A, A, 4, 16, 128, 2, 2, None) == DTYPE       # packed f32
    assert L.bi_matmul(A, P(0x10010 + 2), A, 4, 16, 128, 0, 2, None) == ALIGN
    assert L.bi_matmul(A, A, A, 4, 16, 128, 0, 3, None) == SHAPE       # no such layout
    assert L.bi_matmul_swiglu(A, A, A, 64, 64, 128, 0, 0, A, 1 << 30, None) == UNSUP


@pytest.mark.parametrize("args,code", [
    # x, lhs, rhs, wq, scales, biases, y, M, x_rows, N, K, E, qmode, bits, gs, layout
    ((None, A, A, A, A, A, A, 4, 4, 64, 256, 8, 0, 4, 32, 1), NULL),
    ((A, A, None, A, A, A, A, 4, 4, 64, 256, 8, 0, 4, 32, 1), NULL),
    ((A, A, A, A, A, None, A, 4, 4, 64, 256, 8, 0, 4, 32, 1), NULL),       # affine needs biases
    ((A, None, A, A, A, A, A, 8, 4, 64, 256, 8, 0, 4, 32, 1), SHAPE),      # no lhs: x_rows >= M
    ((A, A, A, A, A, A, A, 4, 4, 64, 256, 0, 0, 4, 32, 1), SHAPE),         # no experts
    ((A, A, A, A, A, A, A, 4, 4, 64, 256, 1024, 0, 4, 32, 1), SHAPE),      # too many experts
    ((A, A, A, A, None, None, A, 4, 4, 64, 192, 8, 0, 4, 32, 2), SHAPE),   # packed: K % 128
    ((A, A, A, P(0x10014), None, None, A, 4, 4, 64, 256, 8, 0, 4, 32, 2), ALIGN),   # packed: 16-byte wq
    ((A, A, A, A, A, A, A, 4, 4, 64, 256, 8, 3, 8, 32, 1), GROUP),         # mxfp8 takes no biases
    ((A, A, A, A, A, A, A, 4, 4, 64, 1040, 8, 0, 8, 32, 1), GROUP),        # affine 8-bit: K % gs
    ((A, A, A, A, A, A, A, 4, 4, 64, 256, 8, 0, 9, 32, 1), GROUP),         # affine bits 2..8
    ((A, A, A, A, A, A, A, 4, 4, 64, 1040, 8, 0, 4, 32, 1), GROUP),        # K % gs
    ((A, A, A, A, A, A, A, 4, 4, 64, 256, 8, 1, 4, 16, 1), GROUP),         # nvfp4 takes no biases
    ((A, P(0x10002), A, A, A, A, A, 4, 4, 64, 256, 8, 0, 4, 32, 1), ALIGN),
])
def test_gather_qmatmul_validation(args, code):
    assert bi.lib().bi_gather_qmatmul(*args, None) == code


def test_packed_qweight_validation():
    L = bi.lib()
    assert L.bi_packed_qweight_bytes(20, 256, 0, 4, 64) == 2 * 2 * (1024 + 16 * 2 * 4)
    assert L.bi_packed_qweight_bytes(16, 128, 1, 4, 16) == 1024 + 128
    assert L.bi_packed_qweight_bytes(16, 192, 0, 4, 64) == 0           # K % 128
    assert L.bi_packed_qweight_bytes(16, 128, 0, 4, 16) == 0           # affine gs 16
    # other widths: 64 lanes x bits words per chunk, then the same constants
    assert L.bi_packed_qweight_bytes(16, 128, 0, 8, 32) == 64 * 8 * 4 + 16 * 4 * 4
    assert L.bi_packed_qweight_bytes(20, 256, 3, 8, 32) == 2 * 2 * (64 * 8 * 4 + 16 * 4)
    assert L.bi_packed_qweight_bytes(16, 128, 0, 3, 128) == 64 * 3 * 4 + 16 * 1 * 4
    assert L.bi_packed_qweight_bytes(16, 128, 0, 9, 32) == 0
    assert L.bi_pack_qweights(A, A, A, A, 16, 192, 0, 3, 32, None) == SHAPE       # K % 128
    assert L.bi_pack_qweights(A, A, None, P(0x10010 + 4), 16, 128, 3, 8, 32, None) == ALIGN
    assert L.bi_pack_qweights(A, A, A, A, 16, 128, 3, 8, 32, None) == GROUP       # mxfp8 takes no biases
    assert L.bi_qmatmul(A, A, None, None, A, 4, 16, 192, 3, 8, 32, 2, None) == SHAPE    # K % 128
    assert L.bi_qmatmul(A, P(0x10010 + 4), None, None, A, 4, 16, 128, 0, 6, 64, 2, None) == ALIGN
    assert L.bi_pack_qweights(A, A, None, A, 16, 128, 0, 4, 64, None) == NULL    # affine needs biases
    assert L.bi_pack_qweights(A, A, A, A, 16, 128, 1, 4, 16, None) == GROUP      # nvfp4 takes none
    assert L.bi_pack_qweights(A, A, A, A, 16, 192, 0, 4, 64, None) == SHAPE
    assert L.bi_pack_qweights(A, A, A, P(0x10010 + 4), 16, 128, 0, 4, 64, None) == ALIGN
    # packed qmatmul: constants are inside the buffer (scales/biases may be NULL)
    assert L.bi_qmatmul(A, A, None, None, A, 4, 16, 192, 0, 4, 64, 2, None) == SHAPE   # K % 128
    assert L.bi_qmatmul(A, P(0x10010 + 4), None, None, A, 4, 16, 128, 0, 4, 64, 2, None) == ALIGN
    assert L.bi_qmatmul(A, A, A, A, A, 4, 16, 128, 0, 4, 64, 3, None) == SHAPE         # no such layout
    assert L.bi_qmatmul(A, A, None, None, A, 4, 16, 128, 0, 4, 64, 1, None) == NULL    # transposed needs scales


def test_argmax_advance_validation():
    L = bi.lib()
    assert L.bi_argmax_advance(A, A, None, A, 4, 32000, None) == NULL
    assert L.bi_argmax_advance(A, A, A, None, 4, 32000, None) == NULL
    assert L.bi_argmax_advance(A, A, A, P(0x10002), 4, 32000, None) == ALIGN
    assert L.bi_argmax_advance(A, A, A, A, 0, 32000, None) == SHAPE


def test_row_reduction_validation():
    L = bi.lib()
    assert L.bi_log_softmax(None, A, 4, 32000, 0, None) == NULL
    assert L.bi_token_logprob(A, None, A, 4, 32000, 0, None) == NULL
    assert L.bi_row_mean(A, A, 0, 32000, 0, None) == SHAPE
    assert L.bi_log_softmax(A, A, 4, 0, 0, None) == SHAPE
    assert L.bi_log_softmax(A, A, 4, 32000, 9, None) == DTYPE
    assert L.bi_log_softmax(ODD, A, 4, 32000, 0, None) == ALIGN
    assert L.bi_row_mean(A, P(0x10002), 4, 32000, 0, None) == ALIGN


def test_embed_rmsnorm_validation():
    L = bi.lib()
    ids = P(0x10000)
    assert L.bi_embed_rmsnorm(None, A, A, A, A, 4, 1000, 4096, 1e-6, 0, None) == NULL
    assert L.bi_embed_rmsnorm(ids, A, None, A, A, 4, 1000, 4096, 1e-6, 0, None) == NULL
    assert L.bi_embed_rmsnorm(P(0x10002), A, A, A, A, 4, 1000, 4096, 1e-6, 0, None) == ALIGN
    assert L.bi_embed_rmsnorm(ids, A, ODD, A, A, 4, 1000, 4096, 1e-6, 0, None) == ALIGN
    assert L.bi_embed_rmsnorm(ids, A, A, A, A, 0, 1000, 4096, 1e-6, 0, None) == SHAPE
    assert L.bi_embed_rmsnorm(ids, A, A, A, A, 4, 0, 4096, 1e-6, 0, None) == SHAPE
    assert L.bi_embed_rmsnorm(ids, A, A, A, A, 4, 1000, 4096, -1.0, 0, None) == SHAPE
    assert L.bi_embed_rmsnorm(ids, A, A, A, A, 4, 1000, 4096, 1e-6, 2, None) == DTYPE   # f32: not a 16-bit table
    assert L.bi_embed_rmsnorm(ids, A, A, A, A, 4, 1000, 4096, 1e-6, 9, None) == DTYPE


def test_add_rmsnorm_validation():
    L = bi.lib()
    assert L.bi_add_rmsnorm(A, None, A, A, A, 4, 4096, 1e-6, 0, None) == NULL
    assert L.bi_add_rmsnorm(A, A, None, A, A, 4, 4096, 1e-6, 0, None) == NULL
    assert L.bi_add_rmsnorm(A, ODD, A, A, A, 4, 4096, 1e-6, 0, None) == ALIGN
    assert L.bi_add_rmsnorm(A, A, ODD, A, A, 4, 4096, 1e-6, 0, None) == ALIGN
    assert L.bi_add_rmsnorm(A, A, A, A, A, 0, 4096, 1e-6, 0, None) == SHAPE
    assert L.bi_add_rmsnorm(A, A, A, A, A, 4, 4096, -1.0, 0, None) == SHAPE
    assert L.bi_add_rmsnorm(A, A, A, A, A, 4, 4096, 1e-6, 9, None) == DTYPE


def test_time_next_launch_is_host_only():
    """Setting and clearing the one-shot timing hook touches no device."""
    L = bi.lib()
    assert L.bi_time_next_launch(None, None) == OK
    assert L.bi_time_next_launches(None, None, 0) == OK
    assert L.bi_time_next_launches(None, None, -1) == SHAPE


def test_glue_validation():
    L = bi.lib()
    assert L.bi_embed(None, A, A, 1, 10, 64, None) == NULL
    assert L.bi_embed(A, A, A, 1, 10, 12, None) == SHAPE
    assert L.bi_rope_kv_write(A, A, A, A, A, A, A, 1, 1, 16, 4, 2, 7, 16, 0, None) == SHAPE
    assert L.bi_rope_kv_write(A, A, A, A, A, A, A, 1, 1, 16, 4, 2, 8, 16, 2, None) == SHAPE   # no such layout
    assert L.bi_silu_mul(A, None, 4, 8, None) == NULL
    assert L.bi_add(A, A, ODD, 8, None) == ALIGN
    assert L.bi_argmax(A, A, 0, 8, None) == SHAPE
