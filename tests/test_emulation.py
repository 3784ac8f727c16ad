"""CPU replay of the kernels' index mappings and operand arithmetic (layout.h,
operand.h compiled for the host) against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import emu
from tests.parity import assert_parity


@pytest.mark.parametrize("N,K,edge", [(256, 1024, 0), (40, 512, 1), (19, 768, 2)])
def test_dequant_bit_exact(orc, N, K, edge):
    canon = synth.matrix_rows(4, 1, N, K, edge_mode=edge)
    w = emu.dequant(canon, N, K)
    ref = orc.dequant(canon, N, K, f32=True)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


def test_packed_size_and_padding():
    N, K = 21, 512
    canon = synth.matrix_rows(1, 2, N, K)
    p = emu.pack(canon, N, K)
    assert p.size == 32 * 2 * 144
    assert p.size == 32 * (K // 256) * 144
    # a pure re-arrangement: the multiset of bytes of real rows plus zero padding
    assert np.count_nonzero(p) <= np.count_nonzero(canon)


@pytest.mark.parametrize("N,K,R,NT,NW,V", [
    (256, 1024, 12, 2, 8, 1),     # the small correctness workload, one range
    (40, 1024, 5, 2, 8, 3),       # ragged N, K split into uneven parts
    (33, 512, 1, 1, 8, 2),
    (48, 512, 20, 1, 8, 1),       # two row tiles
    (16, 256, 48, 1, 4, 1),       # three row tiles
    (20, 256, 64, 1, 4, 1),       # four row tiles
    (700, 2048, 12, 2, 8, 4),     # several tiles, ranges shorter than a tile row
    (16, 512, 5, 1, 8, 1),        # 2 steps for 8 waves: empty sub-ranges
    (48, 1024, 7, 1, 8, 5),       # ranges of 2-3 steps over 8 waves
])
@pytest.mark.parametrize("msum", [1, 0])
def test_gemm_data_flow_matches_oracle(orc, N, K, R, NT, NW, V, msum):
    """Both forms of the min term: from staged sub-block sums, or per step."""
    canon = synth.matrix_rows(0, 3, N, K)
    x = synth.x_bf16(0, 5, R, K, outlier_p=0.01)
    y = emu.stream(canon, N, K, x, NT=NT, NW=NW, V=V, msum=msum)
    ref = orc.gemm(canon, N, K, x)
    m = assert_parity(y, ref, f"emu N={N} K={K} R={R} msum={msum}")
    assert m["rel_l2"] < 2e-6


def _bf16_bits(v: float) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


@pytest.mark.parametrize("big", [4096.0, 65280.0])
@pytest.mark.parametrize("msum", [1, 0])
def test_large_subblock_sums(orc, big, msum):
    """Sub-blocks of 32 large activations: their sums (32 x 4096 = 131072, or
    32 x 65280, the largest bf16 below binary16's limit) are far beyond
    binary16's range.  The min term keeps them in fp32, so both forms of the
    min term stay finite and match the oracle."""
    N, K, R = 48, 1024, 12
    canon = synth.matrix_rows(0, 3, N, K)
    x = synth.x_bf16(0, 5, R, K).copy()
    x[0, 32:64] = _bf16_bits(big)                 # sub-block 1 of block 0, row 0
    x[5, 256 + 96:256 + 128] = _bf16_bits(-big)   # sub-block 3 of block 1, row 5
    x[11, 1024 - 32:] = _bf16_bits(big)           # the last sub-block, the last row
    y = emu.stream(canon, N, K, x, NT=1, NW=8, V=2, msum=msum)
    assert np.isfinite(y).all()
    assert_parity(y, orc.gemm(canon, N, K, x), f"big={big} msum={msum}")


def test_large_subblock_sums_row_tiled(orc):
    """The row-tiled kernel's activation image holds the same fp32 sums."""
    N, K, R = 80, 512, 40
    canon = synth.matrix_rows(0, 4, N, K)
    x = synth.x_bf16(0, 6, R, K).copy()
    x[3, 0:32] = _bf16_bits(65280.0)
    x[39, 480:512] = _bf16_bits(-4096.0)
    y = emu.prefill(canon, N, K, x)
    assert np.isfinite(y).all()
    assert_parity(y, orc.gemm(canon, N, K, x), "row-tiled sums")


def test_edge_blocks_emulated(orc):
    N, K, R = 64, 1024, 24
    canon = synth.matrix_rows(4, 0, N, K, edge_mode=1)
    x = synth.x_bf16(4, 1, R, K)
    assert_parity(emu.stream(canon, N, K, x, NT=1, NW=8, V=3), orc.gemm(canon, N, K, x), "edge blocks")


@pytest.mark.parametrize("N,K,R,NT,NW,V", [
    (256, 1024, 12, 2, 4, 7),      # 2 tiles x 4 blocks over 7 ranges: every tile shared
    (256, 1024, 12, 2, 4, 2),      # one range per tile (no partials)
    (300, 2048, 5, 1, 8, 13),      # ragged last tile, uneven ranges
    (40, 3072, 20, 2, 4, 6),       # one tile, 12 blocks, 2 row tiles
    (700, 512, 3, 2, 4, 11),
    (1000, 8192, 12, 1, 8, 50),    # ranges of a few blocks each (activation slots < K/256)
])
def test_stream_schedule_matches_oracle_any_order(orc, N, K, R, NT, NW, V):
    canon = synth.matrix_rows(2, 8, N, K)
    x = synth.x_bf16(2, 9, R, K, outlier_p=0.01)
    ref = orc.gemm(canon, N, K, x)
    ys = [emu.stream(canon, N, K, x, NT=NT, NW=NW, V=V, order_seed=s) for s in range(3)]
    for y in ys:
        m = assert_parity(y, ref, f"stream N={N} K={K} R={R} V={V}")
        assert m["rel_l2"] < 2e-6
    # the reduction order is fixed: any arrival order gives the same bits
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32))


@pytest.mark.parametrize("N,K,R,NW,nwn,V", [
    (256, 1024, 12, 8, 2, 3),      # 2 columns x 4 sub-ranges, tiles of 32 outputs
    (320, 6144, 12, 8, 2, 40),     # an attention-output-like K, ranges over tile edges
    (330, 4352, 12, 8, 4, 23),     # ragged N: the last tile has idle columns
    (128, 4352, 5, 8, 8, 17),      # every wave its own column (no K split)
    (50, 2048, 20, 8, 4, 3),       # two row tiles, a single ragged tile
    (700, 1024, 48, 4, 2, 9),      # three row tiles, 4 waves
    (64, 512, 1, 8, 8, 1),         # one step per column
])
def test_wave_grid_matches_oracle_any_order(orc, N, K, R, NW, nwn, V):
    """Waves side by side along N (nwn columns) and along K (NW / nwn rows)."""
    canon = synth.matrix_rows(3, 4, N, K)
    x = synth.x_bf16(3, 7, R, K, outlier_p=0.01)
    ref = orc.gemm(canon, N, K, x)
    ys = [emu.stream(canon, N, K, x, NT=1, NW=NW, V=V, order_seed=s, nwn=nwn) for s in range(2)]
    for y in ys:
        m = assert_parity(y, ref, f"grid N={N} K={K} R={R} nwn={nwn} V={V}")
        assert m["rel_l2"] < 2e-6
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))


@pytest.mark.parametrize("N,K,R,NW,V", [
    (640, 1024, 12, 8, 16),        # 40 tiles over 16 ranges: 2 or 3 whole tiles each
    (300, 2048, 5, 8, 7),          # ragged last tile
    (48, 5120, 1, 8, 3),           # one tile per range, 20 blocks each
    (1000, 512, 20, 8, 63),        # two row tiles, 63 tiles over 63 ranges
    (700, 256, 48, 4, 11),         # three row tiles, one block per tile
])
def test_whole_tile_ranges_match_oracle(orc, N, K, R, NW, V):
    """Ranges of whole tiles: no tile is shared between workgroups."""
    canon = synth.matrix_rows(5, 2, N, K)
    x = synth.x_bf16(5, 3, R, K, outlier_p=0.01)
    m = assert_parity(emu.stream(canon, N, K, x, NT=1, NW=NW, V=V, aligned=1), orc.gemm(canon, N, K, x),
                      f"tile ranges N={N} K={K} R={R} V={V}")
    assert m["rel_l2"] < 2e-6


@pytest.mark.parametrize("N,K,R,NW,chunks,V,msum", [
    (640, 5120, 48, 4, 4, 16, 0),     # K in 4 chunks of 5 blocks, 4 ranges per chunk
    (320, 8192, 48, 4, 8, 16, 1),     # 8 chunks of 4 blocks, 2 ranges per chunk
    (300, 2048, 24, 8, 2, 6, 0),      # ragged last tile
    (40, 1536, 33, 4, 3, 3, 1),       # one range per chunk, 3 tiles
])
def test_k_chunks_match_oracle_any_order(orc, N, K, R, NW, chunks, V, msum):
    """K in chunks: each chunk of a tile leaves a partial; the last chunk to
    arrive adds them in chunk order (same bits in any arrival order)."""
    canon = synth.matrix_rows(8, 1, N, K)
    x = synth.x_bf16(8, 2, R, K, outlier_p=0.01)
    ref = orc.gemm(canon, N, K, x)
    ys = [emu.stream(canon, N, K, x, NT=1, NW=NW, V=V, aligned=1, msum=msum, chunks=chunks, order_seed=s)
          for s in range(2)]
    for y in ys:
        m = assert_parity(y, ref, f"chunks N={N} K={K} R={R} S={chunks}")
        assert m["rel_l2"] < 2e-6
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))


def test_sequence_shares_workspace_across_gemms(orc):
    """Several GEMMs of different shapes in one launch reuse the partial slots and
    tile counters; each result still matches the oracle and no counter stays armed."""
    shapes = [(300, 1024), (64, 2048), (1000, 512), (40, 3072)]
    R = 12
    mats = [(synth.matrix_rows(6, i, N, K), N, K) for i, (N, K) in enumerate(shapes)]
    xs = [synth.x_bf16(6, 50 + i, R, K) for i, (N, K) in enumerate(shapes)]
    Vs = [5, 5, 5, 5]
    nwns = [1, 2, 4, 1]            # each GEMM its own wave grid
    aligned = [0, 0, 1, 0]         # and its own kind of range
    msums = [1, 0, 1, 0]           # and its own form of the min term
    ys = emu.stream_seq(mats, xs, NT=2, NW=4, Vs=Vs, order_seed=3, nwns=nwns, aligned=aligned, msums=msums)
    # a GEMM with K in chunks between two others, sharing the workspace
    chunked = emu.stream_seq([mats[0], (synth.matrix_rows(6, 9, 600, 2048), 600, 2048), mats[2]],
                             [xs[0], synth.x_bf16(6, 59, R, 2048), xs[2]], NT=1, NW=4, Vs=[5, 8, 5],
                             order_seed=4, nwns=[1, 1, 4], aligned=[0, 1, 1], msums=[1, 0, 1], chunks=[1, 4, 1])
    assert_parity(chunked[1], orc.gemm(synth.matrix_rows(6, 9, 600, 2048), 600, 2048, synth.x_bf16(6, 59, R, 2048)),
                  "seq chunked")
    for (canon, N, K), x, y, V, nwn, al, ms in zip(mats, xs, ys, Vs, nwns, aligned, msums):
        m = assert_parity(y, orc.gemm(canon, N, K, x), f"seq N={N} K={K}")
        assert m["rel_l2"] < 2e-6
        # the same GEMM alone in its own launch gives the same bits
        alone = emu.stream(canon, N, K, x, NT=2, NW=4, V=V, order_seed=11, nwn=nwn, aligned=al, msum=ms)
        assert np.array_equal(alone.view(np.uint32), y.view(np.uint32))


def test_stream_schedule_slots_unique():
    """Within one tile the partial slots of its workgroups are distinct, and a
    workgroup never uses the same slot for two partial segments."""
    import itertools
    for T, KB, P in itertools.product([1, 2, 5, 13], [1, 4, 20, 100], [1, 2, 3, 7, 64]):
        I = T * KB
        if P > I:
            continue
        used = {}
        for p in range(P):
            it0, it1 = p * I // P, (p + 1) * I // P
            assert it1 > it0
            it = it0
            while it < it1:
                t, j = divmod(it, KB)
                jb = min(KB, j + (it1 - it))
                partial = not (j == 0 and jb == KB)
                if partial:
                    slot = 2 * p if it0 > t * KB else 2 * p + 1
                    assert slot not in used, (T, KB, P, p, t)
                    used[slot] = t
                it += jb - j
        for t in range(T):
            q_lo = ((t * KB + 1) * P + I - 1) // I - 1
            q_hi = (((t + 1) * KB) * P + I - 1) // I - 1
            owners = [p for p in range(P) if p * I // P < (t + 1) * KB and (p + 1) * I // P > t * KB]
            assert owners == list(range(q_lo, q_hi + 1))
            slots = [s for s, tt in used.items() if tt == t]
            assert len(slots) == (len(owners) if len(owners) > 1 else 0)


# ---- the row-tiled path (prompt-chunk rows, and large R) ----------------------

@pytest.mark.parametrize("N,K", [(10240, 5120), (5120, 8192), (51200, 5120), (5120, 25600), (151936, 5120),
                                 (300, 1024), (16, 256)])
@pytest.mark.parametrize("R", [1, 12, 48, 64, 76, 524, 2060])
def test_prefill_plan_covers_the_problem(N, K, R):
    """Every row, output and block is in exactly one workgroup's share; K chunks
    hold at least 8 blocks (or there is one); the workspace holds the image and
    the chunks' partial slices."""
    p = emu.prefill_plan(N, K, R)
    KB, NS = K // 256, (N + 15) // 16
    rows, subtiles = 16 * p["rtw"] * p["wm"], 2 * p["wn"]
    assert (p["wm"], p["wn"], p["rtw"]) in ((2, 4, 4), (2, 6, 4), (1, 8, 4), (1, 8, 2))
    assert p["mt"] * rows >= R > (p["mt"] - 1) * rows
    assert p["nt"] * subtiles >= NS > (p["nt"] - 1) * subtiles
    assert p["S"] * p["kc"] >= KB > (p["S"] - 1) * p["kc"]
    assert p["S"] == 1 or p["kc"] >= 8
    img = p["mt"] * KB * 9 * p["rtw"] * p["wm"] * 1024
    assert p["img_bytes"] == img
    slice_ = (R * N + 3) // 4 * 4
    assert p["ws_bytes"] == img + (p["S"] * slice_ * 4 if p["S"] > 1 else 0)


def test_prefill_plan_choices_on_the_layer():
    """The choices the measurements rest on: gate|up at 48 rows on the 64-row
    grid (one round), down at 76 rows in K chunks (40 output tiles), and the
    12-wave grid at 2060 rows."""
    assert (emu.prefill_plan(51200, 5120, 48)["wm"], emu.prefill_plan(51200, 5120, 48)["wn"]) == (1, 8)
    assert emu.prefill_plan(5120, 25600, 76)["S"] > 1
    p = emu.prefill_plan(51200, 5120, 2060)
    assert (p["wm"], p["wn"]) == (2, 6)


# (N, K, R, CUs): each wave grid, K in chunks (4 of 8 blocks; 4 of 9 with a last of 6),
# ragged rows and outputs, one row
PREFILL_CASES = [(400, 512, 130, 4, (2, 4), 1), (400, 512, 200, 3, (2, 6), 1), (400, 512, 130, 2, (1, 8), 1),
                 (300, 8192, 76, 64, (2, 4), 4), (70, 8448, 5, 64, None, 4), (33, 256, 1, 256, None, 1)]


@pytest.mark.parametrize("N,K,R,cus,grid,S", PREFILL_CASES)
def test_prefill_replay_matches_oracle(orc, N, K, R, cus, grid, S):
    """The row-tiled kernel's data flow replayed on the CPU (plan, activation image,
    lane layouts, per-block scale update, K-chunk slices added in chunk order),
    with emulated matrix-core products, against the fp64 oracle."""
    p = emu.prefill_plan(N, K, R, cus)
    if grid is not None:
        assert (p["wm"], p["wn"]) == grid
    assert p["S"] == S
    canon = synth.matrix_rows(31, N, N, K)
    x = synth.x_bf16(31, R, R, K, outlier_p=0.01)
    assert_parity(emu.prefill(canon, N, K, x, cus), orc.gemm(canon, N, K, x), f"replay N={N} K={K} R={R}")


def test_prefill_replay_catches_a_wrong_image_chunk(orc):
    """A planted mistake: rows of the image shifted by one row tile must fail."""
    N, K, R = 64, 512, 40
    canon = synth.matrix_rows(32, 1, N, K)
    x = synth.x_bf16(32, 2, R, K)
    y = emu.prefill(canon, N, K, x)
    ref = orc.gemm(canon, N, K, x)
    assert_parity(y, ref, "replay")
    wrong = emu.prefill(canon, N, K, np.roll(x, 16, axis=0))
    with pytest.raises(AssertionError):
        assert_parity(wrong, ref, "shifted rows")
