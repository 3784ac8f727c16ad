"""Pins for the fp64 oracle: each check ties it to something other than itself.

- golden super-blocks with closed-form values (tests/golden/superblocks.txt);
- numpy's binary16 decoder and the bfloat16 = top-half-of-binary32 definition;
- an exact-rational brute force written separately (oracle/tiny_exact.py);
- the integer special case (d=1, dmin=0, sc=1: W is the quant matrix Q),
  where numpy's float64 matmul is exact and so must agree bit for bit;
- invariants: row independence, scaling by powers of two, one-hot columns;
- planted mistakes: mutant builds of the oracle must fail at least one pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import tiny_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "superblocks.txt")


def load_golden():
    recs, cur = [], {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            cur[key.strip()] = val.strip()
            if key.strip() == "expect":
                recs.append(cur)
                cur = {}
    return recs


def golden_bytes(rec):
    b = bytes.fromhex(rec["hex"].replace(" ", ""))
    assert len(b) == 144
    return np.frombuffer(b, dtype=np.uint8).copy()


def golden_expect(rec):
    return [Fraction(eval(rec["expect"], {"__builtins__": {}}, {"k": k, "F": Fraction}))
            for k in range(256)]


# --- a test-local encoder of the canonical layout (independent of synth.c) ---

def f16_bits(v: float) -> int:
    return int(np.float16(v).view(np.uint16))


def encode_block(d_bits, dmin_bits, sc, m, q):
    stream = 0
    for s in range(8):
        stream |= (int(sc[s]) & 63) << (6 * s)
        stream |= (int(m[s]) & 63) << (48 + 6 * s)
    q = [int(v) for v in q]
    b = bytes([d_bits & 0xFF, d_bits >> 8, dmin_bits & 0xFF, dmin_bits >> 8])
    b += stream.to_bytes(12, "little")
    b += bytes((q[2 * i] & 15) | ((q[2 * i + 1] & 15) << 4) for i in range(128))
    return np.frombuffer(b, dtype=np.uint8).copy()


def encode_matrix(blocks):
    return np.concatenate(blocks)


# ------------------------------------------------------------------------------

@pytest.mark.parametrize("rec", load_golden(), ids=lambda r: r["name"])
def test_golden_blocks(orc, rec):
    sb = golden_bytes(rec)
    exp = golden_expect(rec)
    w = orc.dequant_block(sb)
    assert [Fraction(float(v)) for v in w] == exp
    assert tiny_exact.block_weights(sb) == exp
    w32 = orc.dequant(sb, 1, 256, f32=True)[0]
    assert np.array_equal(w32, np.array([float(e) for e in exp], dtype=np.float32))


def test_f16_decoder_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([orc.bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_integer_special_case_matches_numpy_bitwise(orc):
    """d = 1, dmin = 0, sc = 1 makes W the quant matrix Q; y = Q x^T is then
    exact in float64 (12-bit products, partial sums far below 2^53), so numpy's
    matmul (any summation order) must agree bit for bit."""
    rng = np.random.default_rng(5)
    N, K, R = 48, 1024, 12
    Q = rng.integers(0, 16, size=(N, K))
    blocks = []
    for n in range(N):
        for j in range(K // 256):
            blocks.append(encode_block(0x3C00, 0, [1] * 8, [0] * 8, list(Q[n, 256 * j:256 * j + 256])))
    canon = encode_matrix(blocks)
    x = synth.x_bf16(11, 3, R, K)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    # exponent spread guard for the exactness argument
    nz = np.abs(xf[xf != 0])
    assert math.log2(nz.max() * 15 * K) - math.log2(nz.min()) < 52
    y = orc.gemm(canon, N, K, x)
    ref = xf @ Q.T.astype(np.float64)
    assert np.array_equal(y, ref)


def test_min_only_case_closed_form(orc):
    """q = 0 everywhere: y[r, n] = -sum_s dmin * m_s * X_s[r] with X_s the
    sub-block sums of x; with d = dmin = 1 and small integer x this is exact."""
    N, K, R = 3, 512, 2
    rng = np.random.default_rng(9)
    ms = rng.integers(0, 64, size=(N, K // 256, 8))
    blocks = [encode_block(0x3C00, 0x3C00, [5] * 8, list(ms[n, j]), [0] * 256)
              for n in range(N) for j in range(K // 256)]
    canon = encode_matrix(blocks)
    xi = rng.integers(-8, 9, size=(R, K)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)   # small integers are exact in bf16
    y = orc.gemm(canon, N, K, x)
    Xs = xi.astype(np.float64).reshape(R, K // 32, 32).sum(axis=2)
    exp = np.zeros((R, N))
    for r in range(R):
        for n in range(N):
            exp[r, n] = -sum(ms[n, j, s] * Xs[r, j * 8 + s] for j in range(K // 256) for s in range(8))
    assert np.array_equal(y, exp)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_bruteforce_tiny(orc, seed):
    N, K, R = 3, 512, 3
    canon = synth.matrix_rows(seed, 7, N, K)
    x = synth.x_bf16(seed, 9, R, K, outlier_p=0.05)
    y = orc.gemm(canon, N, K, x)
    exact = tiny_exact.gemm_exact(canon, N, K, x)
    W = [tiny_exact.block_weights(canon[(n * 2 + j) * 144:(n * 2 + j + 1) * 144]) for n in range(N) for j in range(2)]
    for r in range(R):
        for n in range(N):
            wrow = W[2 * n] + W[2 * n + 1]
            xs = [tiny_exact._bf16(int(b)) for b in x[r]]
            absum = sum(abs(float(wrow[k] * xs[k])) for k in range(K))
            bound = K * 2.0 ** -53 * absum      # recursive-summation error bound
            assert abs(Fraction(float(y[r, n])) - exact[r][n]) <= Fraction(bound)


def test_row_independence_bitwise(orc):
    N, K, R = 64, 1024, 12
    canon = synth.matrix_rows(0, 0, N, K)
    x = synth.x_bf16(0, 1, R, K)
    y = orc.gemm(canon, N, K, x)
    for r in range(R):
        yr = orc.gemm(canon, N, K, x[r:r + 1])
        assert np.array_equal(yr[0], y[r])


def test_power_of_two_scaling_bitwise(orc):
    N, K, R = 32, 1024, 4
    canon = synth.matrix_rows(3, 0, N, K)
    x = synth.x_bf16(3, 1, R, K)
    y = orc.gemm(canon, N, K, x)
    x4 = x.copy()
    nz = (x4 & 0x7FFF) != 0
    x4[nz] = x4[nz] + (2 << 7)          # exponent + 2 : x * 4 exactly
    y4 = orc.gemm(canon, N, K, x4)
    assert np.array_equal(y4, 4.0 * y)


def test_one_hot_columns(orc):
    N, K = 16, 512
    canon = synth.matrix_rows(4, 2, N, K)
    w = orc.dequant(canon, N, K)
    ks = [0, 1, 31, 32, 255, 256, 300, 511]
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80                 # bf16 1.0
    y = orc.gemm(canon, N, K, x)
    for i, k in enumerate(ks):
        assert np.array_equal(y[i], w[:, k])


def test_dequant_f32_is_single_rounding(orc):
    canon = synth.matrix_rows(1, 4, 8, 1024)
    w64 = orc.dequant(canon, 8, 1024)
    w32 = orc.dequant(canon, 8, 1024, f32=True)
    assert np.array_equal(w32, w64.astype(np.float32))
    # spot-check against exact rationals: fp32 value is the nearest to the exact w
    ex = tiny_exact.block_weights(canon[:144])
    for k in range(0, 256, 7):
        e = ex[k]
        f = float(w32[0, k])
        up = float(np.nextafter(np.float32(f), np.float32(np.inf)))
        dn = float(np.nextafter(np.float32(f), np.float32(-np.inf)))
        assert abs(Fraction(f) - e) <= abs(Fraction(up) - e)
        assert abs(Fraction(f) - e) <= abs(Fraction(dn) - e)


def test_argmax_lowest_index_on_ties(orc):
    y = np.array([[1.0, 3.0, 3.0, 2.0], [-1.0, -1.0, -5.0, -1.0], [0.0, 0.0, 0.0, 0.0]])
    assert list(orc.argmax_rows(y)) == [1, 0, 0]
    rng = np.random.default_rng(1)
    yr = rng.standard_normal((7, 1000))
    assert np.array_equal(orc.argmax_rows(yr), np.argmax(yr, axis=1))


def test_exactness_domain_guard(orc):
    sb = encode_block(0x7BFF, 0x0001, [63] * 8, [63] * 8, [15] * 256)  # d = 65504, dmin = 2^-24
    with pytest.raises(ArithmeticError):
        orc.dequant_block(sb)


def test_page_pins():
    from synth import workloads
    from weight_streaming_gemm_amd import roofline
    # a full read of 16.7 GB at the card's nominal 936 GB/s takes about 18 ms
    ms = roofline.ideal_seconds(16.7e9, 936e9) * 1e3
    assert abs(ms - 17.84) < 0.01 and round(ms) == 18
    # four agents x (one next token + two drafts) = twelve rows
    assert workloads.R_DEFAULT == 12 == 4 * (1 + 2)
    assert workloads.pass_bytes() == 17_990_737_920
    assert workloads.pass_weights() == 31_983_534_080


# --- planted mistakes --------------------------------------------------------

# ---- greedy draft verification ------------------------------------------------
# Hand-derived cases of the rule: row i's argmax p_i stands for the position after
# row i's input; draft i (row i + 1's input) is accepted iff it equals p_i, in
# order, stopping at the first rejection; the agent emits p_0 and then p_{i+1} for
# each accepted draft.  Two drafts per agent (three rows) unless stated.
VERIFY_CASES = [
    # argmax rows,            drafts,            D, tokens,                          n_new
    ([10, 20, 30],            [[10, 20]],        2, [[10, 20, 30]],                  [3]),   # both drafts stand
    ([5, 6, 7],               [[9, 6]],          2, [[5, -1, -1]],                   [1]),   # first draft wrong: later match ignored
    ([4, 8, 1],               [[4, 2]],          2, [[4, 8, -1]],                    [2]),   # second draft wrong
    ([3, 3, 3],               [[3, 3]],          2, [[3, 3, 3]],                     [3]),   # repeated token
    ([7, 1, 2, 9, 9, 9],      [[7, 1], [8, 9]],  2, [[7, 1, 2], [9, -1, -1]],        [3, 1]),
    ([11, 12, 13, 14],        [],                0, [[11], [12], [13], [14]],        [1, 1, 1, 1]),  # no drafts
    ([2, 5, 6, 2, 5],         [[2, 5, 7, 9]],    4, [[2, 5, 6, -1, -1]],             [3]),   # four drafts, third wrong
    ([2, 5, 6, 2, 5],         [[2, 5, 6, 9]],    4, [[2, 5, 6, 2, -1]],              [4]),   # four drafts, fourth wrong
]


@pytest.mark.parametrize("case", range(len(VERIFY_CASES)))
def test_verify_greedy_hand_cases(orc, case):
    am, dr, D, tok, n = VERIFY_CASES[case]
    t, nn = orc.verify_greedy(am, dr, D)
    assert t.tolist() == tok and nn.tolist() == n


def test_verify_greedy_invariants(orc):
    """Drafts that copy the argmax of the row before them all stand; one changed
    draft cuts the agent's tokens right there; n_new is always in 1 .. D + 1 and
    the emitted tokens are the argmax rows in order."""
    rng = np.random.default_rng(5)
    for D in (1, 2, 3, 5):
        A = 7
        am = rng.integers(0, 50, size=A * (D + 1)).astype(np.int32)
        good = np.stack([am[a * (D + 1): a * (D + 1) + D] for a in range(A)])
        t, n = orc.verify_greedy(am, good, D)
        assert (n == D + 1).all()
        assert np.array_equal(t.ravel(), am)
        for cut in range(D):
            bad = good.copy()
            bad[:, cut] += 1
            t, n = orc.verify_greedy(am, bad, D)
            assert (n == cut + 1).all()
            for a in range(A):
                assert t[a, :cut + 1].tolist() == am[a * (D + 1): a * (D + 1) + cut + 1].tolist()
                assert (t[a, cut + 1:] == -1).all()


def _pins_fail(o: oracle.Oracle) -> bool:
    """Run a subset of the pins against an oracle; True when any pin fails."""
    try:
        for am, dr, D, tok, n in VERIFY_CASES:
            t, nn = o.verify_greedy(am, dr, D)
            if t.tolist() != tok or nn.tolist() != n:
                return True
        for rec in load_golden():
            w = o.dequant_block(golden_bytes(rec))
            if [Fraction(float(v)) for v in w] != golden_expect(rec):
                return True
        N, K, R = 3, 512, 2
        canon = synth.matrix_rows(0, 7, N, K)
        x = synth.x_bf16(0, 9, R, K)
        y = o.gemm(canon, N, K, x)
        exact = tiny_exact.gemm_exact(canon, N, K, x)
        for r in range(R):
            for n in range(N):
                if abs(float(exact[r][n]) - y[r, n]) > 1e-9 * (1 + abs(float(exact[r][n]))):
                    return True
    except (ArithmeticError, ValueError):
        return True
    return False


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6, 7])
def test_planted_mistakes_are_caught(tmp_path, mutant):
    path = str(tmp_path / f"liboracle_m{mutant}.so")
    oracle.build(force=True, mutant=mutant, path=path)
    assert _pins_fail(oracle.Oracle(path)), f"mutant {mutant} slipped through the pins"


def test_clean_oracle_passes_pin_subset(orc):
    assert not _pins_fail(orc)
