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


@pytest.mark.parametrize("N,K,R,NT,S", [
    (256, 1024, 12, 2, 1),     # the small correctness workload
    (40, 1024, 5, 2, 3),       # ragged N, K split into uneven parts
    (33, 512, 1, 1, 2),
    (48, 512, 20, 1, 1),       # two row tiles
    (16, 256, 48, 1, 1),       # three row tiles
])
def test_gemm_data_flow_matches_oracle(orc, N, K, R, NT, S):
    canon = synth.matrix_rows(0, 3, N, K)
    x = synth.x_bf16(0, 5, R, K, outlier_p=0.01)
    y = emu.gemm(canon, N, K, x, NT=NT, S=S)
    ref = orc.gemm(canon, N, K, x)
    m = assert_parity(y, ref, f"emu N={N} K={K} R={R}")
    assert m["rel_l2"] < 2e-6


def test_edge_blocks_emulated(orc):
    N, K, R = 64, 1024, 24
    canon = synth.matrix_rows(4, 0, N, K, edge_mode=1)
    x = synth.x_bf16(4, 1, R, K)
    assert_parity(emu.gemm(canon, N, K, x), orc.gemm(canon, N, K, x), "edge blocks")


@pytest.mark.parametrize("N,K,R,NT,P", [
    (256, 1024, 12, 2, 7),      # 2 tiles x 4 blocks over 7 workgroups: every tile shared
    (256, 1024, 12, 2, 2),      # one workgroup per tile (no partials)
    (300, 2048, 5, 1, 13),      # ragged last tile, uneven ranges
    (40, 3072, 20, 2, 6),       # one tile, 12 blocks, 2 row tiles
    (700, 512, 3, 2, 11),
])
def test_stream_schedule_matches_oracle_any_order(orc, N, K, R, NT, P):
    canon = synth.matrix_rows(2, 8, N, K)
    x = synth.x_bf16(2, 9, R, K, outlier_p=0.01)
    ref = orc.gemm(canon, N, K, x)
    ys = [emu.stream(canon, N, K, x, NT=NT, P=P, order_seed=s) for s in range(3)]
    for y in ys:
        m = assert_parity(y, ref, f"stream N={N} K={K} R={R} P={P}")
        assert m["rel_l2"] < 2e-6
    # the reduction order is fixed: any arrival order gives the same bits
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32))


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
