"""Group-quantized matmul at the other code widths on the GPU: affine codes of
2 to 8 bits and mxfp8 -- parity with the dequantize-then-matmul oracle,
bitwise invariance over M and across the streaming and tiled kernels,
bounded tails, every mxfp8 code at every finite scale.

Workload: x fp16 ~ N(0,1); W ~ N(0,1) quantized per group (min-max affine
at 2..8 bits with fp16 scale and bias at group sizes 32/64/128; mxfp8: e4m3
codes with one e8m0 scale per 32), each stored row a little-endian bit
stream of codes.  The widths and modes are those of the differential
campaign in "Fix fp quantized matmul corruption when the quantized dim is not
a multiple of 32" (Validation); shapes are the decode shape (1..8, 4096,
512), tiled M (20, 50, 64), the page's tail shapes and an N tail."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, assert_parity, bits_equal, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

# (mode, group size, bits)
WIDE = [("affine", 32, 2), ("affine", 64, 3), ("affine", 128, 5), ("affine", 32, 6), ("affine", 64, 7),
        ("affine", 128, 8), ("affine", 32, 8), ("mxfp8", 32, 8)]
QM = {"affine": bi.AFFINE, "mxfp8": bi.MXFP8}
OQM = {"affine": oracle.AFFINE, "mxfp8": oracle.MXFP8}


def dev_q(wq, s, b, offset_words=0):
    """Device copies; offset_words > 0 places wq that many words past a
    16-byte boundary."""
    w = torch.from_numpy(np.ascontiguousarray(wq).view(np.int32)).to(dev())
    if offset_words:
        buf = torch.zeros(w.numel() + offset_words, dtype=torch.int32, device=dev())
        buf[offset_words:] = w.reshape(-1)
        w = buf[offset_words:].view(w.shape)
    if s.dtype == np.uint8:
        sd = torch.from_numpy(np.ascontiguousarray(s)).to(dev())
    else:
        sd = torch.from_numpy(np.ascontiguousarray(s).view(np.int16)).to(dev())
    bd = None if b is None else torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(dev())
    return w, sd, bd


def run(x, wq, s, b, N, K, mode, gs, bits, transposed, offset_words=0):
    wqd, sd, bd = dev_q(wq, s, b, offset_words)
    return to_np(bi.qmatmul(to_dev(x, "f16"), wqd, sd, bd, N, K, QM[mode], gs, transposed, bits=bits))


def ref(x, wq, s, b, M, N, K, mode, gs, bits, transposed):
    return oracle.qmatmul(x, wq, s, b, M, N, K, OQM[mode], gs, transposed, bits=bits)


@pytest.mark.parametrize("mode,gs,bits", WIDE)
@pytest.mark.parametrize("transposed", [True, False])
def test_decode_rows_match_alone_and_oracle(mode, gs, bits, transposed):
    """M = 1..8 at K = 4096, N = 512 (transposed: the streaming kernel;
    natural: the tiled one): every row equals the row computed alone, bit for
    bit, and the oracle within tolerance."""
    K, N = 4096, 512
    x, wq, s, b = inputs.qmatmul_case(8, K, N, mode, gs, transposed, seed=bits, bits=bits)
    r = ref(x, wq, s, b, 8, N, K, mode, gs, bits, transposed)
    wqd, sd, bd = dev_q(wq, s, b)
    xd = to_dev(x, "f16")
    call = lambda xm: to_np(bi.qmatmul(xm, wqd, sd, bd, N, K, QM[mode], gs, transposed, bits=bits))
    alone = [call(xd[i:i + 1].contiguous()) for i in range(8)]
    for M in (1, 3, 8):
        y = call(xd[:M].contiguous())
        assert_parity(y, r[:M], "f16", f"M={M}")
        for i in range(M):
            assert bits_equal(y[i:i + 1], alone[i]), f"row {i} of M={M}"


@pytest.mark.parametrize("mode,gs,bits", WIDE)
@pytest.mark.parametrize("transposed", [True, False])
def test_tiled_m_matches_streaming_rows(mode, gs, bits, transposed):
    """M = 20 and 50 (tiles of 32 and 64 rows) at K = 1024, N = 200 (an N
    tail): parity with the oracle, and each row bitwise equal to the same row
    at M = 1 (the streaming kernel where the layout allows it)."""
    K, N = 1024, 256 if not transposed else 200
    x, wq, s, b = inputs.qmatmul_case(50, K, N, mode, gs, transposed, seed=10 + bits, bits=bits)
    r = ref(x, wq, s, b, 50, N, K, mode, gs, bits, transposed)
    wqd, sd, bd = dev_q(wq, s, b)
    xd = to_dev(x, "f16")
    call = lambda xm: to_np(bi.qmatmul(xm, wqd, sd, bd, N, K, QM[mode], gs, transposed, bits=bits))
    y50 = call(xd)
    assert_parity(y50, r, "f16", "M=50")
    y20 = call(xd[:20].contiguous())
    assert bits_equal(y20, y50[:20])
    for i in (0, 17, 49):
        assert bits_equal(call(xd[i:i + 1].contiguous()), y50[i:i + 1]), f"row {i}"


@pytest.mark.parametrize("mode,gs,bits,M,K,N,transposed", [
    ("affine", 32, 3, 5, 1056, 128, True),       # K % 128 == 32: ragged last block, tiled kernel
    ("mxfp8", 32, 8, 7, 1056, 96, True),
    ("affine", 64, 6, 9, 1000, 128, False),      # natural: any K, x rows not 16-byte aligned
    ("mxfp8", 32, 8, 3, 1041, 64, False),
    ("affine", 128, 8, 8, 4096, 8192, True),     # N >= 8192: two column groups per streaming tile
    ("mxfp8", 32, 8, 16, 4096, 8192, True),
])
def test_tails_and_wide_tiles(mode, gs, bits, M, K, N, transposed):
    x, wq, s, b = inputs.qmatmul_case(M, K, N, mode, gs, transposed, seed=M + K, bits=bits)
    y = run(x, wq, s, b, N, K, mode, gs, bits, transposed)
    assert_parity(y, ref(x, wq, s, b, M, N, K, mode, gs, bits, transposed), "f16")


@pytest.mark.parametrize("mode,gs,bits", [("affine", 32, 3), ("affine", 64, 6), ("mxfp8", 32, 8)])
@pytest.mark.parametrize("M", [4, 40])
def test_unaligned_words_same_bits(mode, gs, bits, M):
    """wq one word past a 16-byte boundary takes single-word loads: same bits
    as the aligned call."""
    K, N = 2048, 256
    x, wq, s, b = inputs.qmatmul_case(M, K, N, mode, gs, True, seed=3, bits=bits)
    a = run(x, wq, s, b, N, K, mode, gs, bits, True)
    u = run(x, wq, s, b, N, K, mode, gs, bits, True, offset_words=1)
    assert bits_equal(a, u)
    assert_parity(a, ref(x, wq, s, b, M, N, K, mode, gs, bits, True), "f16")


@pytest.mark.parametrize("bits", [2, 3, 5, 6, 7, 8])
@pytest.mark.parametrize("transposed", [True, False])
def test_affine_unit_scale_integer_x_bit_exact(bits, transposed):
    """Scale 1, bias -2^(bits-1), integer x: every product and partial sum is
    an integer below 2^20, so the GPU equals the oracle bit for bit whatever
    the order of the sums -- a check of the code extraction itself."""
    M, K, N, gs = 6, 512, 64, 32
    rng = np.random.default_rng(bits)
    rows, cols = (N, K) if transposed else (K, N)
    codes = rng.integers(0, 1 << bits, size=(rows, cols)).astype(np.uint32)
    wq = inputs.pack_bits(codes, bits)
    s = np.full((rows, cols // gs), 0x3C00, np.uint16)
    b = np.full((rows, cols // gs), np.float16(-(1 << (bits - 1))).view(np.uint16), np.uint16)
    x = inputs.integer_values(rng, (M, K), -4, 4, "f16")
    r = oracle.round_to(ref(x, wq, s, b, M, N, K, "affine", gs, bits, transposed), "f16")
    assert bits_equal(run(x, wq, s, b, N, K, "affine", gs, bits, transposed), r)


def _e4m3_finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint32)


@pytest.mark.parametrize("M", [16, 254])
def test_mxfp8_every_code_and_finite_scale(M):
    """One-hot rows of x read single dequantized weights: every non-NaN e4m3
    code at every scale byte whose values stay finite in binary16 (e <= 134),
    through the streaming (M <= 16, several calls) and tiled kernels, equals
    the oracle's binary16 rounding bit for bit -- subnormal and zero results
    and both signs included."""
    es = np.arange(0, 135, dtype=np.uint8)
    codes1 = _e4m3_finite_codes()                         # 254 codes
    K = 256
    row = np.zeros(K, np.uint32)
    row[:codes1.size] = codes1
    N = es.size
    codes = np.tile(row, (N, 1))
    wq = inputs.pack_bits(codes, 8)
    s = np.repeat(es[:, None], K // 32, axis=1)
    wqd, sd, _ = dev_q(wq, s, None)
    for m0 in range(0, codes1.size, M):
        m = min(M, codes1.size - m0)
        x = np.zeros((m, K), np.float32)
        x[np.arange(m), m0 + np.arange(m)] = 1.0
        xb = inputs.to_storage(x, "f16")
        r = oracle.round_to(ref(xb, wq, s, None, m, N, K, "mxfp8", 32, 8, True), "f16")
        g = to_np(bi.qmatmul(to_dev(xb, "f16"), wqd, sd, None, N, K, bi.MXFP8, 32, True, bits=8))
        assert bits_equal(g, r), f"codes {m0}..{m0 + m}"


def test_mxfp8_every_code_and_finite_scale_natural():
    """The same check through the natural layout's element-wise decode: W
    [K, N] with row k holding code k in every column and column group j
    scaled by 2^(j - 127), j = 0..134."""
    es = np.arange(0, 135, dtype=np.uint8)
    codes1 = _e4m3_finite_codes()
    K, N = codes1.size, 32 * es.size
    codes = np.repeat(codes1[:, None], N, axis=1)
    wq = inputs.pack_bits(codes, 8)
    s = np.tile(es[None, :], (K, 1))
    x = inputs.to_storage(np.eye(K, dtype=np.float32), "f16")
    r = oracle.round_to(ref(x, wq, s, None, K, N, K, "mxfp8", 32, 8, False), "f16")
    assert bits_equal(run(x, wq, s, None, N, K, "mxfp8", 32, 8, False), r)


@pytest.mark.parametrize("transposed", [True, False])
def test_mxfp8_extreme_scales_and_nan_codes(transposed):
    """Scales far outside binary16 (e = 0, 1, 100, 150, 254), the NaN scale
    byte and the NaN codes: weights overflow to inf, flush to zero or are NaN
    exactly as the oracle rounds them.  Finite outputs sum small dyadic
    multiples exactly (scale-1 groups, integer x), so outputs agree value for
    value, inf for inf and NaN for NaN."""
    M, K = 2, 256
    N = 64 if transposed else 96          # natural: column groups 0 NaN, 1 inf, 2 finite
    rng = np.random.default_rng(5)
    fin = _e4m3_finite_codes()
    # moderate codes (|v| <= 4) so that scale-1 sums stay exact
    small = fin[np.abs(torch.from_numpy(fin.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()) <= 4]
    rows, cols = (N, K) if transposed else (K, N)
    codes = rng.choice(small, size=(rows, cols)).astype(np.uint32)
    s = np.full((rows, cols // 32), 127, np.uint8)
    if transposed:
        s[8:16, 2] = rng.choice(np.array([150, 254], np.uint8), size=8)            # overflow to +inf ...
        codes[8:16, 64:96] = rng.choice(small[(small > 0) & (small < 0x80)], size=(8, 32))   # ... from positive codes
        s[16:24, 5] = 255                                                           # NaN scale
        s[24:32, ::2] = rng.choice(np.array([0, 1, 100], np.uint8), size=(8, 4))    # flush to zero
        codes[40, 7] = 0x7F                                                         # NaN codes
        codes[41, 200] = 0xFF
    else:
        s[64:96, 1] = rng.choice(np.array([150, 254], np.uint8), size=32)
        codes[64:96, 32:64] = rng.choice(small[(small > 0) & (small < 0x80)], size=(32, 32))
        s[100:120, 0] = 255
        s[130:140, :] = rng.choice(np.array([0, 1, 100], np.uint8), size=(10, 3))
        codes[150, 70] = 0x7F
        codes[151, 40] = 0xFF
    wq = inputs.pack_bits(codes, 8)
    x = inputs.integer_values(rng, (M, K), 1, 2, "f16")                             # positive: no 0 * inf
    r = oracle.round_to(ref(x, wq, s, None, M, N, K, "mxfp8", 32, 8, transposed), "f16")
    g = run(x, wq, s, None, N, K, "mxfp8", 32, 8, transposed)
    rf, gf = inputs.from_storage(r, "f16"), inputs.from_storage(g, "f16")
    assert np.isnan(rf).any() and np.isinf(rf).any() and np.isfinite(rf).any()
    assert np.array_equal(rf, gf, equal_nan=True)


@pytest.mark.parametrize("mode,gs,bits,M,K,N,transposed", [
    ("affine", 32, 3, 9, 1056, 100, True), ("mxfp8", 32, 8, 4, 4096, 200, True),
    ("affine", 64, 5, 50, 1000, 128, False), ("mxfp8", 32, 8, 20, 1041, 96, False)])
def test_bounded_loads_and_stores(mode, gs, bits, M, K, N, transposed):
    """Code words followed by all-ones words, scales by NaN patterns, output
    fenced by canaries."""
    x, wq, s, b = inputs.qmatmul_case(M, K, N, mode, gs, transposed, seed=4, bits=bits)
    wqd, sd, bd = dev_q(wq, s, b)
    wg = Guarded(tuple(wqd.shape), torch.int32, poison=0xFF, init=wqd)
    sg = Guarded(tuple(sd.shape), sd.dtype, poison=0xFF, init=sd)
    bg = None if bd is None else Guarded(tuple(bd.shape), torch.int16, poison=0xFF, init=bd)
    xg = Guarded((M, K), torch.float16, poison=0xFF, init=to_dev(x, "f16"))
    yg = Guarded((M, N), torch.float16, poison=0x99)
    bi.qmatmul(xg.view, wg.view, sg.view, None if bg is None else bg.view, N, K, QM[mode], gs, transposed,
               out=yg.view, bits=bits)
    torch.cuda.synchronize()
    assert yg.canaries_intact()
    assert_parity(to_np(yg.view), ref(x, wq, s, b, M, N, K, mode, gs, bits, transposed), "f16")


@pytest.mark.parametrize("mode,gs,bits", WIDE)
@pytest.mark.parametrize("M,N", [(8, 512), (40, 200), (4, 8192)])
def test_packed_bits_equal_transposed(mode, gs, bits, M, N):
    """The tile-packed layout (streaming kernel at M <= 16, tiled above, a
    padded last row group at N = 200) gives the transposed call's bits."""
    K = 1024
    x, wq, s, b = inputs.qmatmul_case(M, K, N, mode, gs, True, seed=M + bits, bits=bits)
    wqd, sd, bd = dev_q(wq, s, b)
    wp = bi.pack_qweights(wqd, sd, bd, N, K, QM[mode], gs, bits=bits)
    xd = to_dev(x, "f16")
    a = to_np(bi.qmatmul(xd, wqd, sd, bd, N, K, QM[mode], gs, True, bits=bits))
    p = to_np(bi.qmatmul(xd, wp, None, None, N, K, QM[mode], gs, packed=True, bits=bits))
    assert bits_equal(a, p)


@pytest.mark.parametrize("mode,gs,bits", [("affine", 64, 3), ("mxfp8", 32, 8), ("affine", 128, 6)])
def test_packed_buffer_layout(mode, gs, bits):
    """The packed buffer is the documented layout: for row group r and K block
    b, lane 16g + c holds the `bits` words of row 16r + c for k in [128b + 32g,
    +32); then one constants chunk per (r, b): 16 rows x 128/gs entries."""
    N, K = 40, 256
    _, wq, s, b = inputs.qmatmul_case(1, K, N, mode, gs, True, seed=2, bits=bits)
    wqd, sd, bd = dev_q(wq, s, b)
    got = bi.pack_qweights(wqd, sd, bd, N, K, QM[mode], gs, bits=bits).cpu().numpy().view(np.uint32)
    nrg, nb, gpb = (N + 15) // 16, K // 128, 128 // gs
    rows = np.zeros((nrg * 16, wq.shape[1]), np.uint32)
    rows[:N] = wq
    codes = np.zeros((nrg, nb, 64, bits), np.uint32)
    for r in range(nrg):
        for blk in range(nb):
            for lane in range(64):
                g, c = lane >> 4, lane & 15
                codes[r, blk, lane] = rows[16 * r + c, (4 * blk + g) * bits:(4 * blk + g + 1) * bits]
    ncode = codes.size
    assert np.array_equal(got[:ncode], codes.reshape(-1))
    cbytes = got[ncode:].view(np.uint8)
    if mode == "affine":
        sv = np.zeros((nrg * 16, K // gs), np.uint32)
        sv[:N] = s.astype(np.uint32) | (b.astype(np.uint32) << 16)
        want = np.stack([sv[16 * r:16 * r + 16, blk * gpb:(blk + 1) * gpb] for r in range(nrg) for blk in range(nb)])
        assert np.array_equal(cbytes.view(np.uint32), want.reshape(-1))
    else:
        sv = np.zeros((nrg * 16, K // gs), np.uint8)
        sv[:N] = s
        want = np.stack([sv[16 * r:16 * r + 16, blk * gpb:(blk + 1) * gpb] for r in range(nrg) for blk in range(nb)])
        assert np.array_equal(cbytes, want.reshape(-1))
