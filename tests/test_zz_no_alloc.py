"""The allocation-free entry point (qgemm_run_static) against qgemm_run through
the C ABI: the same plan on the same streaming kernel, so the same bits, and
within the oracle's bar; two calls in a row on the library's fixed scratch, the
second with a smaller input (a stream-K plan with partial tiles and counters,
then a whole-tile plan), then the first again (counters re-used)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth
from tests import gpu_util as G
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def _run_static(packed, N, K, x_bits):
    import torch
    from weight_streaming_gemm_amd import qgemm as Q
    R = x_bits.shape[0]
    xd = G.to_dev(x_bits)
    y = torch.full((R, N), float("nan"), dtype=torch.float32, device=G.dev())
    rc = Q.lib().qgemm_run_static(ctypes.c_void_p(packed.data_ptr()), N, K, ctypes.c_void_p(xd.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), R,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == Q.QGEMM_OK, Q.status_string(rc)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_run_static_matches_run(orc):
    import weight_streaming_gemm_amd as wsg
    cases = [(5120, 8192, 12, 1), (256, 1024, 5, 2), (5120, 8192, 12, 1)]   # big, smaller, big again
    for N, K, R, seed in cases:
        print(f"run_static N={N} K={K} R={R}", flush=True)
        canon = synth.matrix_rows(seed, 3, N, K)
        packed = G.upload_packed(canon, N, K)
        g = wsg.QGemm(packed, N, K, max_R=R)
        info = g.query(R)
        x = synth.x_bf16(seed, 4, R, K, outlier_p=0.01)
        ref_run = G.run(g, x)
        got = _run_static(packed, N, K, x)
        assert np.array_equal(got.view(np.uint32), ref_run.view(np.uint32)), \
            f"N={N} K={K} R={R}: qgemm_run_static differs from qgemm_run (plan {info})"
        assert_parity(got, orc.gemm(canon, N, K, x), f"static N={N} K={K} R={R}")
        g.close()


def test_run_static_rejects_oversized_scratch():
    """A plan whose partial tiles exceed the fixed area returns QGEMM_ESCRATCH
    before anything is enqueued: N = 256, K = 65536 at 64 rows needs 8 wave
    columns of 4 row tiles over at least 256 ranges, 2 x 256 x 8 x 4 KiB = 16 MiB
    of partials plus counters.  The buffers are real (zeros) all the same."""
    import torch
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import qgemm as Q
    N, K, R = 256, 65536, 64
    packed = torch.zeros(wsg.packed_size(N, K), dtype=torch.uint8, device=G.dev())
    x = torch.zeros((R, K), dtype=torch.int16, device=G.dev())
    y = torch.zeros((R, N), dtype=torch.float32, device=G.dev())
    torch.cuda.synchronize()
    rc = Q.lib().qgemm_run_static(ctypes.c_void_p(packed.data_ptr()), N, K, ctypes.c_void_p(x.data_ptr()),
                                  ctypes.c_void_p(y.data_ptr()), R,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == Q.QGEMM_ESCRATCH, Q.status_string(rc)
