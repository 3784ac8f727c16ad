"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Bars: dequantised fp32 weights bit-exact; y within max_rel <= 2e-3 and
rel_l2 <= 1e-4 (tests/parity.py); argmax exact; integer/index work bit-exact.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

import synth
from tests import gpu_util as G
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def _flush(msg: str):
    print(msg, flush=True)


# ---- builtin layouts and rounding (in-bounds probes, one wave each) ----------

def test_probe_mfma_16x16x32_f16_layout():
    import torch
    from tests import probe
    rng = np.random.default_rng(0)
    A = rng.integers(-4, 5, size=(16, 32)).astype(np.float16)
    B = rng.integers(-4, 5, size=(32, 16)).astype(np.float16)
    a = np.zeros((64, 8), np.float16)
    b = np.zeros((64, 8), np.float16)
    for l in range(64):
        for e in range(8):
            a[l, e] = A[l % 16, 8 * (l // 16) + e]
            b[l, e] = B[8 * (l // 16) + e, l % 16]
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    d = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    assert probe.lib().probe_mfma_16x16x32_f16(ad.data_ptr(), bd.data_ptr(), d.data_ptr()) == 0
    torch.cuda.synchronize()
    D = A.astype(np.float64) @ B.astype(np.float64)
    got = d.cpu().numpy()
    for l in range(64):
        for v in range(4):
            assert got[l, v] == D[4 * (l // 16) + v, l % 16]


def test_probe_mfma_16x16x4_f32_layout():
    import torch
    from tests import probe
    rng = np.random.default_rng(1)
    A = rng.integers(-9, 10, size=(16, 4)).astype(np.float32)
    B = rng.integers(-9, 10, size=(4, 16)).astype(np.float32)
    a = np.array([A[l % 16, l // 16] for l in range(64)], np.float32)
    b = np.array([B[l // 16, l % 16] for l in range(64)], np.float32)
    d = torch.zeros((64, 4), dtype=torch.float32, device="cuda")
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    assert probe.lib().probe_mfma_16x16x4_f32(ad.data_ptr(), bd.data_ptr(), d.data_ptr()) == 0
    torch.cuda.synchronize()
    D = A.astype(np.float64) @ B.astype(np.float64)
    got = d.cpu().numpy()
    for l in range(64):
        for v in range(4):
            assert got[l, v] == D[4 * (l // 16) + v, l % 16]


def test_probe_pk_fma_f16_exact_operands():
    """(1024 + q) sc - 1024 sc and (1024 + 16 q) sc/16 - 64 sc must give sc q
    exactly for every 6-bit sc and 4-bit q (single rounding of an exact value)."""
    import torch
    from tests import probe
    sc, q = np.meshgrid(np.arange(64), np.arange(16), indexing="ij")
    sc, q = sc.ravel().astype(np.float64), q.ravel().astype(np.float64)
    a = np.stack([1024 + q, 1024 + 16 * q], 1).astype(np.float16)
    b = np.stack([sc, sc / 16], 1).astype(np.float16)
    c = np.stack([-1024 * sc, -64 * sc], 1).astype(np.float16)
    n = a.shape[0]
    out = torch.zeros((n, 2), dtype=torch.float16, device="cuda")
    ad, bd, cd = (torch.from_numpy(v).cuda() for v in (a, b, c))
    assert probe.lib().probe_pk_fma_f16(ad.data_ptr(), bd.data_ptr(), cd.data_ptr(), out.data_ptr(), n) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:, 0], sc * q)
    assert np.array_equal(got[:, 1], sc * q)


# ---- dequantisation: bit-exact ----------------------------------------------

@pytest.mark.parametrize("N,K,edge", [(256, 1024, 0), (40, 512, 1), (1000, 2048, 2), (19, 256, 0)])
def test_dequant_bit_exact(orc, N, K, edge):
    _flush(f"dequant N={N} K={K} edge={edge}")
    canon, g = G.make(4, 11, N, K, max_R=4, edge_mode=edge)
    w = G.dequant(g)
    ref = orc.dequant(canon, N, K, f32=True)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))
    g.close()


# ---- GEMM parity ---------------------------------------------------------------

@pytest.fixture(scope="module")
def small():
    canon, g = G.make(0, 0, 256, 1024, max_R=64)
    yield canon, g
    g.close()


@pytest.mark.parametrize("R", list(range(1, 17)) + [24, 48, 64])
def test_gemm_small_workload_all_R(orc, small, R):
    _flush(f"gemm small R={R}")
    canon, g = small
    x = synth.x_bf16(0, 1, R, 1024)
    y = G.run(g, x)
    assert_parity(y, orc.gemm(canon, 256, 1024, x), f"R={R}")


@pytest.mark.parametrize("N,K,R", [(40, 8192, 12), (1000, 25600, 3), (17, 5120, 7), (5120, 1024, 12),
                                   (33, 256, 1), (4000, 2048, 48), (4100, 512, 12), (8200, 256, 1),
                                   (600, 5120, 64), (1000, 8192, 24), (16390, 2048, 48), (16384, 2048, 64)])
def test_gemm_ragged_and_split(orc, N, K, R):
    from weight_streaming_gemm_amd import qgemm as Q
    _flush(f"gemm N={N} K={K} R={R}")
    canon, g = G.make(1, 5, N, K, max_R=R)
    info = g.query(R)
    x = synth.x_bf16(1, 6, R, K, outlier_p=0.01)
    ref = orc.gemm(canon, N, K, x)
    assert_parity(G.run(g, x), ref, f"N={N} K={K} R={R} path={info['path']} wgs={info['workgroups']}")
    if info["path"] != Q.PATH_MFMA:     # the automatic choice took the row-tiled kernel: the streaming one too
        assert_parity(G.run(g, x, path=Q.PATH_MFMA), ref, f"N={N} K={K} R={R} streaming")
    g.close()


def test_automatic_choice_of_the_row_tiled_kernel(orc):
    """Matrices of at least 32768 outputs take the row-tiled kernel from 24 rows
    on, matrices of at least 2^26 weights from 48 rows on, every matrix at 64
    rows; below, or on handles made for fewer rows, the streaming kernel; an
    explicit request needs max_R >= 24."""
    from weight_streaming_gemm_amd import qgemm as Q
    _, wide = G.make(1, 9, 32768, 512, max_R=24)           # 2^24 weights, 32768 outputs
    assert wide.query(16)["path"] == Q.PATH_MFMA
    assert wide.query(24)["path"] == Q.PATH_TILED
    wide.close()
    _, big = G.make(1, 9, 16384, 4096, max_R=48)          # 2^26 weights, 16384 outputs
    assert big.query(24)["path"] == Q.PATH_MFMA
    assert big.query(48)["path"] == Q.PATH_TILED
    assert big.query(48)["kernels"] in (2, 3)
    big.close()
    _, small = G.make(1, 9, 1000, 2048, max_R=64)
    assert small.query(48)["path"] == Q.PATH_MFMA
    assert small.query(64)["path"] == Q.PATH_TILED
    assert small.query(12, Q.PATH_TILED)["path"] == Q.PATH_TILED
    small.close()
    canon, few = G.make(1, 9, 1000, 2048, max_R=12)
    assert Q.lib().qgemm_query(few.h, 12, Q.PATH_TILED, ctypes.byref(Q.Info())) == Q.QGEMM_EPATH
    few.close()


def test_plan_kinds_are_exercised():
    """The shapes above reach every kind of plan: whole-tile ranges, stream-K
    ranges, and K in chunks (activations of a tile row larger than LDS)."""
    info = {}
    from weight_streaming_gemm_amd import qgemm as Q
    for N, K, R in [(4100, 512, 12), (40, 8192, 12), (16390, 2048, 48), (16384, 2048, 64)]:
        _, g = G.make(1, 5, N, K, max_R=R)
        info[(N, K, R)] = g.query(R, Q.PATH_MFMA)
        g.close()
    assert info[(4100, 512, 12)]["whole_tile_ranges"] == 1 and info[(4100, 512, 12)]["k_chunks"] == 1
    assert info[(40, 8192, 12)]["whole_tile_ranges"] == 0
    assert info[(16390, 2048, 48)]["k_chunks"] == 2
    assert info[(16384, 2048, 64)]["k_chunks"] == 4


def _bf16_bits(v: float) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


@pytest.mark.parametrize("N,K,R,path", [
    (32768, 1024, 12, "mfma"),    # streaming kernel, min term from the sub-block sums
    (4096, 1024, 12, "mfma"),     # streaming kernel, min term per step
    (4096, 1024, 3, "valu"),      # vector-unit kernel (always the sums)
    (4096, 1024, 40, "tiled"),    # row-tiled kernel (sums in its activation image)
])
def test_large_subblock_sums(orc, N, K, R, path):
    """Sub-blocks of 32 activations at 4096 and at 65280 (the largest bf16 below
    binary16's limit): their sums leave binary16's range; every kernel path
    must stay finite and match the oracle."""
    from weight_streaming_gemm_amd import qgemm as Q
    _flush(f"large sub-block sums N={N} K={K} R={R} path={path}")
    canon, g = G.make(3, 7, N, K, max_R=max(R, 24))
    pid = {"mfma": Q.PATH_MFMA, "valu": Q.PATH_VALU, "tiled": Q.PATH_TILED}[path]
    info = g.query(R, pid)
    if path == "mfma":
        assert info["min_term_sums"] == (1 if N == 32768 else 0), info
    x = synth.x_bf16(3, 8, R, K).copy()
    x[0, 32:64] = _bf16_bits(4096.0)
    x[R - 1, K - 32:] = _bf16_bits(65280.0)
    x[R // 2, 256 + 96:256 + 128] = _bf16_bits(-65280.0)
    y = G.run(g, x, path=pid)
    assert np.isfinite(y).all()
    assert_parity(y, orc.gemm(canon, N, K, x), f"N={N} K={K} R={R} path={path}")
    g.close()


@pytest.mark.parametrize("R", [12, 40])
def test_large_subblock_sums_persistent(orc, R):
    """The same sub-blocks at 4096 and 65280 in the pass kernel with the min term
    from the sub-block sums (two binary16 parts of X_s / 256 per sum): finite and
    matching the oracle at one and at three row tiles."""
    import torch
    import weight_streaming_gemm_amd as wsg
    N, K = 4096, 1024
    _flush(f"large sub-block sums, pass kernel R={R}")
    canon, g = G.make(3, 7, N, K, max_R=48)
    x = synth.x_bf16(3, 8, R, K).copy()
    x[0, 32:64] = _bf16_bits(4096.0)
    x[R - 1, K - 32:] = _bf16_bits(65280.0)
    x[R // 2, 256 + 96:256 + 128] = _bf16_bits(-65280.0)
    seq = wsg.Seq([g], persistent=True, sub_block_sums=True)
    y = torch.empty((R, N), dtype=torch.float32, device="cuda")
    seq.run([G.to_dev(x)], [y], R)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.isfinite(got).all()
    assert_parity(got, orc.gemm(canon, N, K, x), f"pass kernel N={N} K={K} R={R}")
    assert seq.errors() == 0
    seq.close()
    g.close()


def test_edge_blocks_large_R(orc):
    N, K = 512, 2048
    canon, g = G.make(4, 0, N, K, max_R=48, edge_mode=1)
    for R in (24, 48):
        x = synth.x_bf16(4, R, R, K)
        assert_parity(G.run(g, x), orc.gemm(canon, N, K, x), f"edge R={R}")
    g.close()


def test_one_hot_columns_pin_gemm_dequant(orc):
    """x = e_k gives y[:, n] = w[n, k]; with the factored algebra this is the
    fp32 dequantised weight up to the final rounding of two exact parts."""
    N, K = 64, 512
    canon, g = G.make(2, 3, N, K, max_R=16)
    ks = [0, 1, 31, 32, 100, 255, 256, 300, 511, 64, 65, 127, 128, 200, 400, 480]
    x = np.zeros((len(ks), K), np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80
    y = G.run(g, x)
    w = orc.dequant(canon, N, K)
    for i, k in enumerate(ks):
        np.testing.assert_allclose(y[i], w[:, k], rtol=1e-6, atol=1e-7)


def test_determinism_and_row_independence(small):
    canon, g = small
    R = 12
    x = synth.x_bf16(7, 1, R, 1024)
    y1 = G.run(g, x)
    y2 = G.run(g, x)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    x2 = x.copy()
    x2[5:] = synth.x_bf16(8, 1, R - 5, 1024)
    y3 = G.run(g, x2)
    assert np.array_equal(y3[:5].view(np.uint32), y1[:5].view(np.uint32))


def test_row_count_zero_and_errors(small):
    import torch
    from weight_streaming_gemm_amd import qgemm as Q
    canon, g = small
    x = torch.zeros((65, 1024), dtype=torch.int16, device="cuda")
    y = torch.zeros((65, 256), dtype=torch.float32, device="cuda")
    L = Q.lib()
    st = torch.cuda.current_stream().cuda_stream
    assert L.qgemm_run(g.h, x.data_ptr(), y.data_ptr(), 0, st) == Q.QGEMM_OK
    assert L.qgemm_run(g.h, x.data_ptr(), y.data_ptr(), 65, st) == Q.QGEMM_ERANGE_R
    assert L.qgemm_run(g.h, x.data_ptr(), y.data_ptr(), -1, st) == Q.QGEMM_ERANGE_R
    assert L.qgemm_run(g.h, x.data_ptr() + 2, y.data_ptr(), 1, st) == Q.QGEMM_EALIGN
    assert L.qgemm_run_path(g.h, x.data_ptr(), y.data_ptr(), 1, 9, st) == Q.QGEMM_EINVAL
    torch.cuda.synchronize()
    assert float(y.abs().sum()) == 0.0


# ---- vector-unit path (R <= 4) -------------------------------------------------

@pytest.mark.parametrize("N,K", [(256, 1024), (33, 256), (17, 5120), (40, 8192), (4100, 512), (8200, 256),
                                 (5120, 1024), (1000, 25600)])
def test_vector_unit_path(orc, N, K):
    from weight_streaming_gemm_amd import qgemm as Q
    canon, g = G.make(3, 7, N, K, max_R=4)
    for R in (1, 2, 3, 4):
        _flush(f"valu N={N} K={K} R={R}")
        info = g.query(R, Q.PATH_VALU)
        assert info["path"] == Q.PATH_VALU and info["row_tiles"] == 0
        x = synth.x_bf16(3, 10 + R, R, K, outlier_p=0.01)
        assert_parity(G.run(g, x, path=Q.PATH_VALU), orc.gemm(canon, N, K, x),
                      f"valu N={N} K={K} R={R} wgs={info['workgroups']}")
    g.close()


def test_vector_unit_path_edge_blocks_and_determinism(orc):
    from weight_streaming_gemm_amd import qgemm as Q
    N, K = 512, 2048
    canon, g = G.make(4, 0, N, K, max_R=4, edge_mode=1)
    for R in (1, 4):
        _flush(f"valu edge R={R}")
        x = synth.x_bf16(4, 50 + R, R, K)
        y1 = G.run(g, x, path=Q.PATH_VALU)
        assert_parity(y1, orc.gemm(canon, N, K, x), f"valu edge R={R}")
        y2 = G.run(g, x, path=Q.PATH_VALU)
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    g.close()


def test_vector_unit_path_plan_kinds_and_errors(small):
    """Whole-tile and stream-K ranges both reach the vector-unit kernel; it
    serves R <= 4 only."""
    import torch
    from weight_streaming_gemm_amd import qgemm as Q
    for N, K, aligned in [(4100, 512, 1), (40, 8192, 0)]:
        _, g = G.make(1, 5, N, K, max_R=4)
        assert g.query(4, Q.PATH_VALU)["whole_tile_ranges"] == aligned
        g.close()
    canon, g = small
    x = torch.zeros((5, 1024), dtype=torch.int16, device="cuda")
    y = torch.zeros((5, 256), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert Q.lib().qgemm_run_path(g.h, x.data_ptr(), y.data_ptr(), 5, Q.PATH_VALU, st) == Q.QGEMM_EPATH
    assert Q.lib().qgemm_query(g.h, 5, Q.PATH_VALU, ctypes.byref(Q.Info())) == Q.QGEMM_EPATH
    torch.cuda.synchronize()
    assert float(y.abs().sum()) == 0.0


def test_seq_graph_cache_bound(orc):
    """More (R, pointer set) combinations than a sequence caches graphs for: the
    cache is dropped and rebuilt, and every run still gives the oracle's result."""
    import torch
    import weight_streaming_gemm_amd as wsg
    shapes = [(64, 512), (40, 256)]
    mats = [G.make(12, i, N, K, max_R=4) for i, (N, K) in enumerate(shapes)]
    seq = wsg.Seq([g for _, g in mats])
    R = 2
    xs_np = [synth.x_bf16(12, 30 + i, R, K) for i, (N, K) in enumerate(shapes)]
    xs = [G.to_dev(x) for x in xs_np]
    refs = [orc.gemm(c, N, K, x) for (c, _), (N, K), x in zip(mats, shapes, xs_np)]
    outs = [[torch.empty((R, N), dtype=torch.float32, device="cuda") for N, K in shapes] for _ in range(70)]
    for rep in range(2):
        _flush(f"seq cache pass {rep}")
        for ys in outs:
            for y in ys:
                y.fill_(-3.0)
            seq.run(xs, ys, R)
        torch.cuda.synchronize()
        for ys in outs:
            for y, ref in zip(ys, refs):
                assert_parity(y.cpu().numpy(), ref, "seq cache")
    seq.close()
    for _, g in mats:
        g.close()


# ---- argmax -------------------------------------------------------------------

def test_argmax_ties_and_nan():
    import torch
    import weight_streaming_gemm_amd as wsg
    y = np.array([[1, 3, 3, 2], [-1, -1, -5, -1], [0, 0, 0, 0], [np.nan, 2, np.nan, 2],
                  [np.nan, np.nan, np.nan, np.nan]], np.float32)
    yd = torch.from_numpy(y).cuda()
    idx = torch.empty(5, dtype=torch.int32, device="cuda")
    wsg.argmax_rows(yd, idx)
    torch.cuda.synchronize()
    assert idx.cpu().tolist() == [1, 0, 0, 1, 0]
    rng = np.random.default_rng(3)
    big = rng.standard_normal((12, 151936)).astype(np.float32)
    big[3, 100] = big[3, 5000] = big[3].max() + 1       # tie: lowest index wins
    bd = torch.from_numpy(big).cuda()
    idx = torch.empty(12, dtype=torch.int32, device="cuda")
    wsg.argmax_rows(bd, idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), np.argmax(big, axis=1))


@pytest.mark.parametrize("N", [1, 3, 5, 1001, 4099, 65537])
def test_argmax_unaligned_rows_ties_and_nan(N):
    """Rows that start off 16-byte alignment (N not a multiple of 4): the scalar
    head, the vector body and the scalar tail all take part; ties are planted
    across them (lowest index wins), NaN never wins, an all-NaN row gives 0."""
    import torch
    import weight_streaming_gemm_amd as wsg
    rng = np.random.default_rng(N)
    R = 7
    y = rng.standard_normal((R, N)).astype(np.float32)
    top = np.float32(10.0)
    picks = [0, N - 1, N // 2, min(2, N - 1), max(0, N - 3)]
    for r, n in enumerate(picks):
        y[r, n] = top
    y[1, 0] = top                                  # tie with N - 1: index 0 wins
    y[5, :] = np.nan                               # all NaN
    y[6, ::2] = np.nan                             # NaN interleaved with values
    yd = torch.from_numpy(y).cuda()
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    wsg.argmax_rows(yd, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for r in range(R):
        row = y[r]
        if np.isnan(row).all():
            assert got[r] == 0
            continue
        v = np.where(np.isnan(row), -np.inf, row)
        assert got[r] == int(np.flatnonzero(v == v.max())[0]), (r, got[r])


@pytest.mark.parametrize("N", [1, 5, 1001, 8193, 65537, 151936])
def test_argmax_chunked_matches_rule_and_reuses_workspace(N):
    """The chunked argmax (workspace, last chunk of a row combines) gives the same
    index as the rule on rows with ties across chunks, NaN and an all-NaN row;
    three runs on one workspace (its counters must come back to zero)."""
    import torch
    import weight_streaming_gemm_amd as wsg
    rng = np.random.default_rng(N + 7)
    R = 9
    y = rng.standard_normal((R, N)).astype(np.float32)
    top = np.float32(10.0)
    for r, n in enumerate([0, N - 1, N // 2, min(8191, N - 1), min(8192, N - 1)]):
        y[r, n] = top
    y[1, 0] = top                                  # tie across the first and last chunk
    y[5, :] = np.nan
    y[6, ::3] = np.nan
    y[7, :] = -np.inf                              # all -inf: index 0
    yd = torch.from_numpy(y).cuda()
    ws = torch.zeros(wsg.argmax_workspace_size(R, N), dtype=torch.uint8, device="cuda")
    for rep in range(3):
        _flush(f"argmax ws N={N} rep {rep}")
        idx = torch.full((R,), -5, dtype=torch.int32, device="cuda")
        wsg.argmax_rows_ws(yd, idx, ws)
        torch.cuda.synchronize()
        got = idx.cpu().numpy()
        for r in range(R):
            row = y[r]
            if np.isnan(row).all():
                assert got[r] == 0
                continue
            v = np.where(np.isnan(row), -np.inf, row)
            assert got[r] == int(np.flatnonzero(v == v.max())[0]), (r, got[r])
    counters = ws.view(torch.int32)[(R * ((N + 8191) // 8192) * 8) // 4:][: R + 1].cpu().numpy()
    assert (counters == 0).all()


@pytest.mark.parametrize("D", [0, 1, 2, 3])
def test_verify_greedy_matches_oracle(orc, D):
    import torch
    import weight_streaming_gemm_amd as wsg
    rng = np.random.default_rng(D)
    A = 64 // (D + 1)
    R = A * (D + 1)
    am = rng.integers(0, 6, size=R).astype(np.int32)            # few values: many accidental matches
    drafts = rng.integers(0, 6, size=(A, max(D, 1))).astype(np.int32)[:, :D]
    for a in range(0, A, 3):                                   # every third agent: all drafts copy the argmax
        drafts[a] = am[a * (D + 1): a * (D + 1) + D]
    tok_ref, n_ref = orc.verify_greedy(am, drafts, D)
    tokens = torch.full((A, D + 1), 99, dtype=torch.int32, device="cuda")
    n_new = torch.full((A,), 99, dtype=torch.int32, device="cuda")
    dd = torch.from_numpy(np.ascontiguousarray(drafts)).cuda() if D > 0 else None
    wsg.verify_greedy(torch.from_numpy(am).cuda(), dd, D, tokens, n_new)
    torch.cuda.synchronize()
    assert np.array_equal(tokens.cpu().numpy(), tok_ref) and np.array_equal(n_new.cpu().numpy(), n_ref)


def test_seq_run_verify_matches_oracle(orc):
    """Weight pass, head argmax and draft check in one call: 4 agents x (token + 2
    drafts) = 12 rows; drafts planted against the oracle's argmax (all stand, the
    first stands, none stands, random); repeated runs give the same bits."""
    import torch
    import weight_streaming_gemm_amd as wsg
    shapes = [(300, 1024), (1000, 512)]
    R, D = 12, 2
    A = R // (D + 1)
    mats = [G.make(14, i, N, K, max_R=R) for i, (N, K) in enumerate(shapes)]
    xs_np = [synth.x_bf16(14, 40 + i, R, K) for i, (N, K) in enumerate(shapes)]
    ref_y = orc.gemm(mats[-1][0], shapes[-1][0], shapes[-1][1], xs_np[-1])
    ref_idx = orc.argmax_rows(ref_y)
    drafts = np.zeros((A, D), np.int32)
    drafts[0] = ref_idx[0:2]                           # both stand
    drafts[1] = [ref_idx[3], ref_idx[4] + 1]           # first stands
    drafts[2] = [ref_idx[6] + 1, ref_idx[7]]           # none (second match ignored)
    drafts[3] = [5, 7]
    tok_ref, n_ref = orc.verify_greedy(ref_idx, drafts, D)
    seq = wsg.Seq([g for _, g in mats])
    xs = [G.to_dev(x) for x in xs_np]
    ys = [torch.empty((R, N), dtype=torch.float32, device="cuda") for N, K in shapes]
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    tokens = torch.empty((A, D + 1), dtype=torch.int32, device="cuda")
    n_new = torch.empty(A, dtype=torch.int32, device="cuda")
    dd = torch.from_numpy(drafts).cuda()
    top2 = np.sort(ref_y, axis=1)[:, -2:]
    for rep in range(3):
        _flush(f"seq verify rep {rep}")
        tokens.fill_(77)
        seq.run_verify(xs, ys, R, idx, dd, D, tokens, n_new)
        torch.cuda.synchronize()
        got_y = ys[-1].cpu().numpy()
        assert_parity(got_y, ref_y, "seq verify head")
        margin = top2[:, 1] - top2[:, 0]
        assert (margin > 10 * np.abs(got_y - ref_y).max()).all(), "argmax ambiguous within the error bound"
        assert np.array_equal(idx.cpu().numpy(), ref_idx)
        assert np.array_equal(tokens.cpu().numpy(), tok_ref) and np.array_equal(n_new.cpu().numpy(), n_ref)
    assert n_ref.tolist()[:3] == [3, 2, 1]
    seq.close()
    for _, g in mats:
        g.close()


# ---- full weight pass machinery (one cooperative launch over several GEMMs) ----

@pytest.mark.parametrize("mode", ["graph", "persistent", "persistent_sums"])
def test_seq_matches_oracle_and_repeats_bitwise(orc, mode):
    """A six-GEMM sequence (ragged N, K of 2 to 12 blocks) at 12 rows: parity with
    the oracle, bitwise-equal repeats with other work between them, the head
    argmax; then 16, 7 and 1 rows through the same sequence (odd row counts
    convert a missing last row in the persistent kernel's staging)."""
    import torch
    import weight_streaming_gemm_amd as wsg
    persistent = mode != "graph"
    shapes = [(300, 1024), (64, 2048), (4100, 512), (1000, 1024), (40, 3072), (151, 512)]
    R, RM = 12, 16
    mats = [G.make(9, i, N, K, max_R=RM) for i, (N, K) in enumerate(shapes)]
    xs_np = [synth.x_bf16(9, 100 + i, RM, K) for i, (N, K) in enumerate(shapes)]
    xs = [G.to_dev(x) for x in xs_np]
    ys = [torch.empty((RM, N), dtype=torch.float32, device="cuda") for N, K in shapes]
    idx = torch.empty(RM, dtype=torch.int32, device="cuda")
    seq = wsg.Seq([g for _, g in mats], persistent=persistent, sub_block_sums=mode == "persistent_sums")
    first = None
    for rep in range(4):
        _flush(f"seq {mode} rep {rep}")
        for y in ys:
            y.fill_(-7.0)
        seq.run([x[:R] for x in xs], [y[:R] for y in ys], R, argmax_idx=idx)
        torch.cuda.synchronize()
        _ = (torch.ones(1000, device="cuda") * rep).sum().item()   # other work between launches
        got = [y[:R].cpu().numpy() for y in ys]
        if first is None:
            first = got
            for i, ((canon, _), (N, K)) in enumerate(zip(mats, shapes)):
                assert_parity(got[i], orc.gemm(canon, N, K, xs_np[i][:R]), f"seq gemm {i}")
        for i in range(len(shapes)):
            assert np.array_equal(got[i].view(np.uint32), first[i].view(np.uint32)), (rep, i)
        assert np.array_equal(idx[:R].cpu().numpy(), np.argmax(got[-1], axis=1))
    assert seq.errors() == 0
    # other row counts through the same sequence
    for r in (16, 7, 1):
        _flush(f"seq {mode} R={r}")
        seq.run([x[:r] for x in xs], [y[:r] for y in ys], r)
        torch.cuda.synchronize()
        for i, ((canon, _), (N, K)) in enumerate(zip(mats, shapes)):
            assert_parity(ys[i][:r].cpu().numpy(), orc.gemm(canon, N, K, xs_np[i][:r]), f"seq R={r} gemm {i}")
    assert seq.errors() == 0
    seq.close()
    for _, g in mats:
        g.close()


@pytest.mark.parametrize("msum", [False, True])
def test_seq_persistent_row_tiles_match_oracle_and_repeat_bitwise(orc, msum):
    """Rows beyond 16 in the pass kernel: two or three 16-row tiles per weight
    step, the min term from the sub-block sums whatever the flag says.  A five-GEMM sequence whose K = 25600 GEMM runs in 20 K chunks at 24 rows
    and 25 at 48 (the chunk partials of a sub-tile added in two batches), at 48,
    33, 24 and 17 rows: parity with the oracle and a bitwise-equal repeat."""
    import torch
    import weight_streaming_gemm_amd as wsg
    shapes = [(300, 1024), (64, 25600), (4100, 512), (40, 8192), (151, 5120)]
    RM = 48
    mats = [G.make(11, i, N, K, max_R=RM) for i, (N, K) in enumerate(shapes)]
    xs_np = [synth.x_bf16(11, 200 + i, RM, K) for i, (N, K) in enumerate(shapes)]
    xs = [G.to_dev(x) for x in xs_np]
    ys = [torch.empty((RM, N), dtype=torch.float32, device="cuda") for N, K in shapes]
    seq = wsg.Seq([g for _, g in mats], persistent=True, sub_block_sums=msum)
    for r in (48, 33, 24, 17):
        first = None
        for rep in range(2):
            _flush(f"seq row tiles msum={msum} R={r} rep {rep}")
            for y in ys:
                y.fill_(-7.0)
            seq.run([x[:r] for x in xs], [y[:r] for y in ys], r)
            torch.cuda.synchronize()
            got = [y[:r].cpu().numpy() for y in ys]
            if first is None:
                first = got
                for i, ((canon, _), (N, K)) in enumerate(zip(mats, shapes)):
                    assert_parity(got[i], orc.gemm(canon, N, K, xs_np[i][:r]), f"seq R={r} gemm {i}")
            for i in range(len(shapes)):
                assert np.array_equal(got[i].view(np.uint32), first[i].view(np.uint32)), (r, rep, i)
    assert seq.errors() == 0
    seq.close()
    for _, g in mats:
        g.close()


@pytest.mark.parametrize("R", [12, 16, 5])
def test_seq_gated_inputs_match_oracle_and_ungated_bitwise(orc, R):
    """Persistent sequences with gated inputs: GEMMs 2 (8192 inputs, two K chunks
    at 12 or 16 rows) and 5 follow a GEMM of twice their input width, so each of
    their chunks waits only for the workgroups holding the outputs it reads.
    Results match the oracle and, bit for bit, the same sequence without the
    flag; no wait gives up."""
    import torch
    import weight_streaming_gemm_amd as wsg
    shapes = [(300, 1024), (16384, 256), (80, 8192), (4100, 512), (512, 2048), (40, 256)]
    mats = [G.make(11, i, N, K, max_R=16) for i, (N, K) in enumerate(shapes)]
    xs_np = [synth.x_bf16(11, 200 + i, R, K) for i, (N, K) in enumerate(shapes)]
    xs = [G.to_dev(x) for x in xs_np]
    out = {}
    for gated in (False, True):
        _flush(f"seq gated={gated} R={R}")
        ys = [torch.full((R, N), -7.0, dtype=torch.float32, device="cuda") for N, K in shapes]
        seq = wsg.Seq([g for _, g in mats], persistent=True, gated_inputs=gated)
        for _ in range(3):
            seq.run(xs, ys, R)
        torch.cuda.synchronize()
        assert seq.errors() == 0
        out[gated] = [y.cpu().numpy() for y in ys]
        seq.close()
    for i, ((canon, _), (N, K)) in enumerate(zip(mats, shapes)):
        assert np.array_equal(out[True][i].view(np.uint32), out[False][i].view(np.uint32)), i
        assert_parity(out[True][i], orc.gemm(canon, N, K, xs_np[i]), f"gated seq gemm {i}")
    for _, g in mats:
        g.close()


def test_seq_with_row_tiled_gemms_matches_oracle(orc):
    """A graph-replayed sequence at 64 rows, where every GEMM takes the row-tiled
    kernel (activation image, product, K-chunk sums), and at 24 rows on the
    streaming kernel through the same handles; repeats are bitwise equal."""
    import torch
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import qgemm as Q
    shapes = [(300, 1024), (5120, 2048), (40, 8192)]
    mats = [G.make(11, i, N, K, max_R=64) for i, (N, K) in enumerate(shapes)]
    assert all(g.query(64)["path"] == Q.PATH_TILED for _, g in mats)
    assert all(g.query(24)["path"] == Q.PATH_MFMA for _, g in mats)
    seq = wsg.Seq([g for _, g in mats])
    for R in (64, 24):
        _flush(f"seq row-tiled R={R}")
        xs_np = [synth.x_bf16(11, 200 + i, R, K) for i, (N, K) in enumerate(shapes)]
        xs = [G.to_dev(x) for x in xs_np]
        ys = [torch.full((R, N), -7.0, dtype=torch.float32, device="cuda") for N, K in shapes]
        seq.run(xs, ys, R)
        torch.cuda.synchronize()
        first = [y.cpu().numpy() for y in ys]
        for i, ((canon, _), (N, K)) in enumerate(zip(mats, shapes)):
            assert_parity(first[i], orc.gemm(canon, N, K, xs_np[i]), f"seq R={R} gemm {i}")
        seq.run(xs, ys, R)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), first[i].view(np.uint32))
    seq.close()
    for _, g in mats:
        g.close()
