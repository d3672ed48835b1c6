"""The allocation-free attention entry point (bi_sdpa_noalloc, for callers
that cannot allocate device memory) gives bi_sdpa's bits through the C ABI,
on two calls in a row -- the second smaller than the first, so it runs on
scratch the first call left dirty -- and stays within the oracle's bf16 gate."""
import ctypes

import numpy as np
import pytest
import torch

import invariant_reductions_amd as bi
import oracle
from gpu_util import assert_parity, dev, to_dev, to_np
from invariant_reductions_amd import inputs

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128
SCALE = 1.0 / np.sqrt(128.0)


def _call_noalloc(q, k, v, kv, max_kv, Lcap, causal=True):
    B, Q = q.shape[0], q.shape[1]
    o = torch.empty_like(q)
    rc = bi.lib().bi_sdpa_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                  ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                                  ctypes.c_void_p(kv.data_ptr()), max_kv, B, Q, Lcap, HQ, HKV, D, SCALE, int(causal),
                                  0, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, bi.lib().bi_status_str(rc)
    return o


@pytest.mark.parametrize("big,small", [((4, 8, 9000, [9000, 4100, 300, 8999]), (1, 1, 1028, [1028])),
                                       ((2, 5, 20000, [20000, 12345]), (3, 2, 700, [700, 257, 2]))])
def test_noalloc_equals_workspace_call_twice(big, small):
    for B, Q, L, lens in (big, small):
        q, k, v = inputs.sdpa_case(B, Q, L, HQ, HKV, D, seed=B * 100 + Q)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        kv = torch.tensor(lens, dtype=torch.int32, device=dev())
        got = to_np(_call_noalloc(qd, kd, vd, kv, L, L))
        want = to_np(bi.sdpa(qd, kd, vd, kv, L, SCALE, True))
        assert np.array_equal(got, want), (B, Q, L)
        assert_parity(got, oracle.sdpa(q, k, v, np.array(lens, np.int32), SCALE, True, "bf16"), "bf16")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    L = bi.lib()
    cap = L.bi_sdpa_noalloc_max_bytes()
    assert cap == 64 << 20
    # B = 64, Q = 8, 32 heads, 2^16 keys: 64 * 8 * 32 * 256 * 528 bytes of partials > 64 MiB
    assert L.bi_sdpa_workspace_bytes(64, 8, 1 << 16, HQ, D) > cap
    q = torch.zeros((64, 8, HQ, D), dtype=torch.bfloat16, device=dev())
    kc = torch.zeros((16,), dtype=torch.bfloat16, device=dev())     # never read: rejected before any launch
    kv = torch.full((64,), 1 << 16, dtype=torch.int32, device=dev())
    rc = L.bi_sdpa_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
                           ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kv.data_ptr()), 1 << 16, 64, 8, 1 << 16, HQ,
                           HKV, D, SCALE, 1, 0, 0, None)
    assert rc == 6                                                  # BI_ERR_WORKSPACE
