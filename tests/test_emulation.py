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
