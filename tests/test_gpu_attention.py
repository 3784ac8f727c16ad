"""GPU parity of the decode attention against the fp64 oracle, through the C ABI.

Bars: max_rel <= 2e-3 and rel_l2 <= 1e-4 per agent (tests/parity.py).  The
weights and values enter the matrix cores as binary16 (relative step 2^-11);
the keys and queries as bf16 (exact)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import attention as at
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def _bf(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)


def _run(q, k, v, lengths, max_len):
    """q, k, v in the oracle's layout ([agent, position, head, dim] caches); the
    entry point takes head-major caches ([agent, head, position, dim])."""
    import torch
    import weight_streaming_gemm_amd as wsg
    A, rows, Hq, d = q.shape
    Hkv = k.shape[2]
    k, v = k.transpose(0, 2, 1, 3), v.transpose(0, 2, 1, 3)
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)  # noqa: E731
    out = torch.full((A, rows, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(wsg.attention_workspace_size(A, rows, Hkv, max_len), dtype=torch.uint8, device=dev)
    ln = torch.tensor(lengths, dtype=torch.int32, device=dev)
    wsg.decode_attention(t(q), t(k), t(v), ln, out, ws, max_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("rows", [1, 2, 3, 4])
def test_attention_small_ragged_lengths(rows):
    """Lengths around split boundaries (6 agents x 2 heads: splits of 128
    positions, 1024 a boundary) and the 32-position steps, an empty cache, two
    key/value heads."""
    rng = np.random.default_rng(rows)
    lengths = [0, 31, 1023, 1024, 1025, 2500]
    A, Hkv, d = len(lengths), 2, 128
    max_len = max(lengths)
    cap = max_len + rows + 5
    q, k, v = _bf(rng, (A, rows, 8 * Hkv, d)), _bf(rng, (A, cap, Hkv, d)), _bf(rng, (A, cap, Hkv, d))
    print(f"attention rows={rows} lengths={lengths}", flush=True)
    got = _run(q, k, v, lengths, max_len)
    ref = at.decode_attention(q, k, v, lengths)
    for a in range(A):
        assert_parity(got[a], ref[a], f"agent {a} L={lengths[a]}")


def test_attention_peaked_scores():
    """Queries aligned with one cached key (scores ~ 40 apart after scaling):
    softmax close to one-hot, the exponent range of the online rescaling."""
    rng = np.random.default_rng(9)
    A, rows, Hkv, d, L = 2, 3, 2, 128, 700
    cap = L + rows
    k = _bf(rng, (A, cap, Hkv, d))
    v = _bf(rng, (A, cap, Hkv, d))
    q = np.empty((A, rows, 8 * Hkv, d), np.uint16)
    for a in range(A):
        for hq in range(8 * Hkv):
            src = k[a, (37 * hq + 11 * a) % L, hq // 8].view(np.uint16)
            f = ((src.astype(np.uint32) << 16).view(np.float32) * 4.0).astype(np.float32)
            q[a, :, hq] = ((f.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    got = _run(q, k, v, [L, L], L)
    ref = at.decode_attention(q, k, v, [L, L])
    for a in range(A):
        assert_parity(got[a], ref[a], f"peaked agent {a}")


def test_attention_four_agents_23k_context():
    """The pages' setting: 4 agents of about 23K positions (a length mix), a step
    of 3 rows each, 64 query heads over 8 key/value heads of 128."""
    rng = np.random.default_rng(23)
    lengths = [23000, 21877, 23552 - 3, 20001]
    A, rows, Hkv, d = 4, 3, 8, 128
    max_len = 23552 - 3
    cap = 23552
    q, k, v = _bf(rng, (A, rows, 8 * Hkv, d)), _bf(rng, (A, cap, Hkv, d)), _bf(rng, (A, cap, Hkv, d))
    print("attention 4 x 23K", flush=True)
    got = _run(q, k, v, lengths, max_len)
    ref = at.decode_attention(q, k, v, lengths)
    for a in range(A):
        assert_parity(got[a], ref[a], f"23K agent {a}")
