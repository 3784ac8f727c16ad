"""Pins of the fp64 decode-attention oracle (CPU): closed forms, invariants and
planted mistakes.  Rows of an agent's step sit at positions L, L + 1, ... and
see positions 0 .. L + i; query head hq reads key/value head hq // (Hq / Hkv)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import attention as at


def bf(x) -> np.ndarray:
    """bf16 bit patterns of values that are exact in bf16 (the tests pick such values)."""
    f = np.asarray(x, dtype=np.float32)
    bits = f.view(np.uint32)
    assert not (bits & 0xFFFF).any(), "test value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def rand_bf(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # round to bf16


def test_first_row_with_empty_cache_returns_first_value():
    """L = 0: row 0 sees only position 0, so its output is v[0] exactly."""
    rng = np.random.default_rng(1)
    q, k, v = rand_bf(rng, (1, 3, 8, 16)), rand_bf(rng, (1, 5, 2, 16)), rand_bf(rng, (1, 5, 2, 16))
    o = at.decode_attention(q, k, v, [0])
    V = at.bf16_to_f64(v)
    for hq in range(8):
        assert np.array_equal(o[0, 0, hq], V[0, 0, hq // 4])


def test_equal_keys_average_the_visible_values():
    """All keys equal: uniform weights, the output is the mean of the values
    each row sees (L + i + 1 of them)."""
    rng = np.random.default_rng(2)
    L, rows, d = 6, 3, 32
    k1 = rand_bf(rng, (d,))
    k = np.broadcast_to(k1, (1, L + rows, 1, d)).copy()
    v = rand_bf(rng, (1, L + rows, 1, d))
    q = rand_bf(rng, (1, rows, 4, d))
    o = at.decode_attention(q, k, v, [L])
    V = at.bf16_to_f64(v)[0, :, 0]
    for i in range(rows):
        np.testing.assert_allclose(o[0, i], np.broadcast_to(V[:L + i + 1].mean(0), (4, d)), rtol=1e-13, atol=1e-14)


def test_two_key_closed_form():
    """Keys k0 = (a, 0, ...), k1 = (0, b, ...) and q = (1, 1, 0, ...): scores a/sqrt(d),
    b/sqrt(d); the output is the logistic mix of v0 and v1."""
    d = 4
    k = np.zeros((1, 2, 1, d), np.float32)
    k[0, 0, 0, 0], k[0, 1, 0, 1] = 3.0, -1.0
    q = np.zeros((1, 1, 1, d), np.float32)
    q[0, 0, 0, :2] = 1.0
    v = np.zeros((1, 2, 1, d), np.float32)
    v[0, 0, 0] = [1, 2, 4, 8]
    v[0, 1, 0] = [-1, 0.5, 0, 2]
    o = at.decode_attention(bf(q), bf(k), bf(v), [1])
    w0 = 1.0 / (1.0 + np.exp((-1.0 - 3.0) / np.sqrt(d)))
    np.testing.assert_allclose(o[0, 0, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], rtol=1e-14)


def test_causality_and_head_groups():
    """Row i ignores positions after L + i; positions up to L + i matter.  Query
    heads of one group see the same cache head; equal queries there give equal
    outputs."""
    rng = np.random.default_rng(3)
    A, rows, Hq, Hkv, d, L = 2, 3, 16, 2, 32, 9
    q = rand_bf(rng, (A, rows, Hq, d))
    q[:, :, 1] = q[:, :, 0]                          # heads 0 and 1: same group (size 8)
    q[:, :, 9] = q[:, :, 0]                          # head 9: the other group
    k, v = rand_bf(rng, (A, L + rows + 2, Hkv, d)), rand_bf(rng, (A, L + rows + 2, Hkv, d))
    o = at.decode_attention(q, k, v, [L, L])
    assert np.array_equal(o[:, :, 1], o[:, :, 0])
    assert not np.allclose(o[:, :, 9], o[:, :, 0])
    for i in range(rows):
        v2 = v.copy()
        v2[:, L + i + 1:] = rand_bf(rng, v2[:, L + i + 1:].shape)
        assert np.array_equal(at.decode_attention(q, k, v2, [L, L])[:, i], o[:, i])
        v3 = v.copy()
        v3[:, L + i] ^= 0x0080                       # flip a bit of a value row i sees
        assert not np.array_equal(at.decode_attention(q, k, v3, [L, L])[:, i], o[:, i])


def _pins_fail(mutant: int) -> bool:
    fns = [test_first_row_with_empty_cache_returns_first_value, test_equal_keys_average_the_visible_values,
           test_two_key_closed_form, test_causality_and_head_groups]
    real = at.decode_attention
    try:
        at.decode_attention = lambda *a, **kw: real(*a, mutant=mutant)
        for f in fns:
            try:
                f()
            except AssertionError:
                return True
        return False
    finally:
        at.decode_attention = real


@pytest.mark.parametrize("mutant", [1, 2, 3])
def test_planted_mistakes_are_caught(mutant):
    assert _pins_fail(mutant), f"attention mutant {mutant} slipped through the pins"


def test_clean_oracle_passes_the_pins():
    assert not _pins_fail(0)
