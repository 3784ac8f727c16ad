"""Prompt-chunk rows sharing the weight pass (the row-tiled kernel behind
qgemm_run_prefill) against the fp64 oracle: small shapes spanning several
128-row and 128-output tiles with ragged tails, edge blocks, row
independence and repeatability, agreement with the streaming kernel where
both serve the row count, and one full-size layer matrix at decode rows plus
a 512-row prompt chunk (every row on sampled outputs, sampled rows on every output)."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from synth import workloads as W
from tests import gpu_util as G
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def run_prefill(g, x_bits):
    import torch
    R = x_bits.shape[0]
    xd = G.to_dev(x_bits)
    y = torch.full((R, g.N), -7.0, dtype=torch.float32, device=G.dev())
    g.run_prefill(xd, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


# (N, K, R): one tile; ragged rows and outputs over several tiles; one row; a
# single output sub-tile; an odd number of blocks (the K loop's last pass is half)
SHAPES = [(128, 256, 128), (300, 1024, 76), (1000, 2048, 200), (4100, 512, 129), (40, 3072, 524),
          (256, 1280, 1), (16, 768, 300), (520, 256, 65),
          # few tiles and long K: K cut into chunks (4 of 8 blocks; 8 of 13 with a last of 9;
          # an odd R x N, so the chunks' partial slices are padded)
          (300, 8192, 76), (520, 25600, 20), (301, 8192, 75),
          # many row and output tiles: the 12-wave grid (192-output tiles) is taken
          (4100, 512, 2060),
          # few rows, many outputs: the 64-row grid (1 x 8 waves, 256-output tiles) is taken
          (40000, 256, 40)]


@pytest.mark.parametrize("N,K,R", SHAPES)
def test_prefill_matches_oracle(orc, N, K, R):
    _flush(f"prefill N={N} K={K} R={R}")
    canon, g = G.make(21, N + K, N, K, max_R=1)
    x = synth.x_bf16(21, 300 + R, R, K)
    y = run_prefill(g, x)
    assert_parity(y, orc.gemm(canon, N, K, x), f"prefill N={N} K={K} R={R}")
    g.close()


@pytest.mark.parametrize("edge_mode", [1, 2])
def test_prefill_edge_blocks(orc, edge_mode):
    """Blocks with dmin = 0, all quants 0 and all quants 15 (cycling, or a seeded few)."""
    N, K, R = 600, 1024, 150
    _flush(f"prefill edge_mode={edge_mode}")
    canon, g = G.make(22, 7, N, K, max_R=1, edge_mode=edge_mode)
    x = synth.x_bf16(22, 8, R, K, outlier_p=0.01)
    y = run_prefill(g, x)
    assert_parity(y, orc.gemm(canon, N, K, x), f"prefill edge {edge_mode}")
    g.close()


def test_prefill_rows_independent_and_repeatable():
    """A row's result depends only on its own activations and not on the row's
    place in the tile grid: rolling the rows by 37 rolls the output bit for bit;
    a second run repeats the first bit for bit."""
    N, K, R = 700, 1536, 300
    _flush("prefill row independence")
    _, g = G.make(23, 3, N, K, max_R=1)
    x = synth.x_bf16(23, 4, R, K)
    y1 = run_prefill(g, x)
    y2 = run_prefill(g, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    yr = run_prefill(g, np.roll(x, 37, axis=0))
    assert np.array_equal(np.roll(y1, 37, axis=0).view(np.uint32), yr.view(np.uint32))
    # the first 12 rows alone give the same bits as inside the 300-row run
    y12 = run_prefill(g, x[:12])
    assert np.array_equal(y12.view(np.uint32), y1[:12].view(np.uint32))
    g.close()


def test_prefill_agrees_with_streaming_kernel(orc):
    """Both kernels serve 1..64 rows: they agree within the parity bar (their
    summation orders differ)."""
    N, K = 1000, 2048
    canon, g = G.make(24, 5, N, K, max_R=48)
    for R in (1, 12, 48):
        _flush(f"prefill vs stream R={R}")
        x = synth.x_bf16(24, 6 + R, R, K)
        assert_parity(run_prefill(g, x), G.run(g, x), f"prefill vs stream R={R}")
    g.close()


def test_prefill_argument_errors():
    import ctypes
    import torch
    from weight_streaming_gemm_amd import qgemm as Q
    _, g = G.make(25, 1, 64, 8192, max_R=1)
    x = torch.zeros((4, 8192), dtype=torch.int16, device=G.dev())
    y = torch.zeros((4, 64), dtype=torch.float32, device=G.dev())
    L = Q.lib()
    st = torch.cuda.current_stream().cuda_stream
    need = g.prefill_workspace_size(4)
    assert need > 0                                      # one tile, 32 blocks: K in chunks
    ws = torch.zeros(need, dtype=torch.uint8, device=G.dev())
    run = lambda xp, R, wsp=ws.data_ptr(), nb=need: L.qgemm_run_prefill(  # noqa: E731
        g.h, xp, y.data_ptr(), R, wsp, nb, st)
    assert run(x.data_ptr(), 0) == Q.QGEMM_OK
    assert run(x.data_ptr(), -1) == Q.QGEMM_ERANGE_R
    assert run(x.data_ptr(), Q.MAX_PREFILL_R + 1) == Q.QGEMM_ERANGE_R
    assert run(x.data_ptr() + 2, 4) == Q.QGEMM_EALIGN
    assert run(None, 4) == Q.QGEMM_EINVAL
    assert run(x.data_ptr(), 4, None, 0) == Q.QGEMM_EINVAL          # workspace needed
    assert run(x.data_ptr(), 4, ws.data_ptr(), need - 16) == Q.QGEMM_EINVAL
    assert run(x.data_ptr(), 4, ws.data_ptr() + 8, need) == Q.QGEMM_EALIGN
    sz = ctypes.c_size_t()
    assert L.qgemm_prefill_workspace_size(g.h, Q.MAX_PREFILL_R + 1, ctypes.byref(sz)) == Q.QGEMM_ERANGE_R
    assert run(x.data_ptr(), 4) == Q.QGEMM_OK
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0                   # zero activations, zero outputs
    g.close()


def test_prefill_full_size_down_k_chunks(orc):
    """down of one layer (25600 -> 5120) at 12 decode rows + 64 prompt rows: 40
    output tiles, so K runs in chunks; every output of every row."""
    import weight_streaming_gemm_amd as wsg
    from tests.test_gpu_fullsize import fused_canon, sample_ns, sampled_rows
    seed = W.SEED_LAYER
    m = {mm.name: mm for mm in W.layer_mats(0)}["down"]
    R = 12 + 64
    _flush(f"prefill full size down N={m.N} K={m.K} R={R}")
    packed = G.upload_packed(fused_canon(seed, m), m.N, m.K)
    g = wsg.QGemm(packed, m.N, m.K, max_R=1)
    assert g.prefill_workspace_size(R) > 0
    x = synth.x_bf16(seed, W.X_STREAM[m.K], R, m.K)
    y = run_prefill(g, x)
    assert_parity(y, orc.gemm(fused_canon(seed, m), m.N, m.K, x), "prefill down")
    g.close()


def test_prefill_full_size_layer_matrix_sampled(orc):
    """gate|up of one layer (5120 -> 51200) at 12 decode rows + a 512-row prompt
    chunk, as the benchmark times it: every row on 256 sampled outputs, and every
    output of rows 0, 11, 12, 300 and the last."""
    import torch
    import weight_streaming_gemm_amd as wsg
    from tests.test_gpu_fullsize import fused_canon, sample_ns, sampled_rows
    seed = W.SEED_LAYER
    m = {mm.name: mm for mm in W.layer_mats(0)}["gate_up"]
    R = 12 + 512
    _flush(f"prefill full size gate_up N={m.N} K={m.K} R={R}")
    packed = G.upload_packed(fused_canon(seed, m), m.N, m.K)
    g = wsg.QGemm(packed, m.N, m.K, max_R=1)
    x = synth.x_bf16(seed, W.X_STREAM[m.K], R, m.K)
    y = run_prefill(g, x)
    assert np.isfinite(y).all()
    ns = sample_ns(m.N, 256, 5)
    ref = orc.gemm(sampled_rows(seed, m, ns), len(ns), m.K, x)
    assert_parity(y[:, ns], ref, "prefill gate_up, every row, sampled outputs")
    rows = np.array([0, 11, 12, 300, R - 1])
    ref_rows = orc.gemm(fused_canon(seed, m), m.N, m.K, x[rows])
    assert_parity(y[rows], ref_rows, "prefill gate_up, sampled rows, every output")
    del packed
    g.close()
    torch.cuda.synchronize()
