"""Exact-rational brute force for tiny shapes (pins the fp64 oracle).

TEST INFRASTRUCTURE ONLY.  Written independently of ``oracle.c``: it re-reads
the canonical 144-byte super-block with its own Python parser and evaluates

    w[n, k] = d * sc_s * q_k - dmin * m_s,     y[r, n] = sum_k w[n, k] * x[r, k]

in ``fractions.Fraction``.  Every binary16 / bfloat16 value is a dyadic
rational, so the result is the exact value of the definition.  Pure-Python
loops: only for N <= 4, K <= 512, R <= 3.
"""
from __future__ import annotations

from fractions import Fraction


def _half(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 31:
        raise ValueError("inf/nan binary16 not allowed here")
    if e == 0:
        return sign * Fraction(f, 2 ** 24)
    return sign * Fraction(1024 + f, 1024) * (Fraction(2) ** (e - 15))


def _bf16(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 255:
        raise ValueError("inf/nan bfloat16 not allowed here")
    if e == 0:
        return sign * Fraction(f, 128) * (Fraction(2) ** -126)
    return sign * Fraction(128 + f, 128) * (Fraction(2) ** (e - 127))


def block_weights(sb) -> list:
    sb = bytes(bytearray(int(v) for v in sb))
    assert len(sb) == 144
    d = _half(sb[0] | sb[1] << 8)
    dmin = _half(sb[2] | sb[3] << 8)
    stream = int.from_bytes(sb[4:16], "little")
    sc = [(stream >> (6 * s)) & 63 for s in range(8)]
    m = [(stream >> (48 + 6 * s)) & 63 for s in range(8)]
    q = []
    for byte in sb[16:144]:
        q.append(byte & 0xF)
        q.append(byte >> 4)
    return [d * sc[k // 32] * q[k] - dmin * m[k // 32] for k in range(256)]


def gemm_exact(canon, N: int, K: int, x_bits) -> list:
    """Exact y as a list of lists of Fractions, shape R x N."""
    if N > 4 or K > 512:
        raise ValueError("tiny shapes only")
    KB = K // 256
    W = []
    for n in range(N):
        row = []
        for j in range(KB):
            off = (n * KB + j) * 144
            row.extend(block_weights(canon[off:off + 144]))
        W.append(row)
    xs = [[_bf16(int(b)) for b in xr] for xr in x_bits]
    return [[sum((W[n][k] * xr[k] for k in range(K)), Fraction(0)) for n in range(N)]
            for xr in xs]
