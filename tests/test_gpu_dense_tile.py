"""The dense kernels for long M: the slot form over 64-row chunks (up to 512
rows where 128 x 128 tiles would fill under 5/8 of the CUs: one workgroup
per (64-column tile, 64-row chunk) with all eight slots), the LDS-tiled
kernel (M > 128, or M > 64 with at least 192 column tiles of 128; K at least
1024) and the streaming kernel they hand the other M > 64 shapes to (16-bit,
transposed or tile-packed weights, K a multiple of 128): every row equals the
same row computed alone (M = 1 takes the streaming kernel), across ragged M
and N, K with an uneven number of blocks per slot, both weight layouts and
both 16-bit types; the outputs stay inside their bounds; sampled rows are
within the parity gate of the oracle.  This is the invariance of
"Fix/speculative shape invariance" (Problem: the same row must not change
with the number of rows) and "Batch-invariant kernels" (Case 3) for verify
blocks and prompts.

Workload: W [N,K] ~ N(0,1)*0.02 then x [M,K] ~ N(0,1), rounded to the dtype."""
import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import Guarded, assert_parity, bits_equal, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,K", [
    (65, 100, 1024),        # slot form over row chunks: one chunk of 64 plus one row
    (128, 4096, 4096),      # ... two full chunks
    (80, 24577, 1024),      # LDS-tiled kernel: one row tile, 193 ragged column tiles
    (129, 6144, 4096),      # ... a last chunk of one row
    (320, 512, 1152),       # ... five chunks, 9 blocks of K
    (300, 1000, 14336),     # ... ragged chunk and column tile, 112 blocks of K
    (512, 640, 256),        # ... the most rows it takes, 2 blocks of K
    (200, 28672, 1024),     # LDS-tiled kernel: enough 128 x 128 tiles
    (1000, 2048, 4096),     # ... more rows than the slot form takes
    (4096, 256, 2048),
    (200, 28672, 512)])     # streaming kernel: enough tiles, K below 1024
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("packed", [False, True])
def test_long_m_rows_equal_row_alone(M, N, K, dtype, packed):
    x, w, _ = inputs.dense_case(M, N, K, dtype, seed=M + N + K)
    xd, wd = to_dev(x, dtype), to_dev(w, dtype)
    wt = bi.pack_weights(wd) if packed else wd
    yg = Guarded((M, N), xd.dtype, poison=0x5A)
    bi.matmul(xd, wt, out=yg.view)
    torch.cuda.synchronize()
    assert yg.canaries_intact()
    y = to_np(yg.view)
    rows = sorted({0, 1, 15, 16, 63, 64, M // 2, M - 2, M - 1})
    for i in rows:
        assert bits_equal(to_np(bi.matmul(xd[i:i + 1].contiguous(), wt)), y[i:i + 1]), f"row {i}"
    # the last 80 rows (other tile and chunk positions)
    lo = max(0, M - 80)
    assert bits_equal(to_np(bi.matmul(xd[lo:].contiguous(), wt)), y[lo:])
    assert_parity(y[rows], oracle.matmul(np.ascontiguousarray(x[rows]), w, dtype, True), dtype)


def test_verify_block_of_64_sequences_equals_decode_rows():
    """The decoder's verify shape (64 sequences x 5 tokens = 320 rows) on the
    fused QKV projection: each row equals the decode batch of 64 (the slot
    kernel) holding that row."""
    M, N, K = 320, 6144, 4096
    x, w, _ = inputs.dense_case(M, N, K, "bf16", seed=5)
    xd, wt = to_dev(x, "bf16"), bi.pack_weights(to_dev(w, "bf16"))
    y = to_np(bi.matmul(xd, wt))
    for b0 in (0, 64, 256):
        ws = bi.matmul_workspace(64, N, K, device=xd.device)
        assert bits_equal(to_np(bi.matmul_ws(xd[b0:b0 + 64].contiguous(), wt, ws)), y[b0:b0 + 64]), b0
