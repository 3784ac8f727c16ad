"""The persistent pass kernel's schedule (pass_sched.h) and data flow, replayed
on the CPU: every weight step of every GEMM is taken exactly once, the chunking
of the pass's shapes is what the LDS area allows, and the replayed pass (cursor
walk, pieces added in wave order, chunk partials added in chunk order) matches
the fp64 oracle."""
from __future__ import annotations

import os
import re

import numpy as np
import pytest

import synth
from synth import workloads as W
from tests import emu
from tests.parity import assert_parity

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "weight_streaming_gemm_amd", "csrc")


def test_replay_constants_match_the_kernel():
    text = open(os.path.join(CSRC, "qgemm_internal.h")).read()
    nc = int(re.search(r"constexpr int PASS_NC = (\d+);", text).group(1))
    pieces = int(re.search(r"constexpr int PASS_PIECES = (\d+);", text).group(1))
    chunks = int(re.search(r"constexpr int PASS_MAX_CHUNKS = (\d+);", text).group(1))
    rts = int(re.search(r"constexpr int PASS_MAX_RT = (\d+);", text).group(1))
    assert "return 160 * 1024 - PASS_NC * pass_pieces(RT) * RT * 1024 - 256;" in text
    assert "pass_pieces(int RT) { return RT == 1 ? PASS_PIECES : 1; }" in text
    assert "PASS_MAX_R = 16 * PASS_MAX_RT;" in text
    assert "pass_max_chunks(int RT) { return RT == 1 ? 16 : PASS_MAX_CHUNKS; }" in text
    assert emu.pass_max_chunks(16) == 16 and emu.pass_max_chunks(17) == chunks
    assert nc == emu.PASS_NC and pieces == emu.PASS_PIECES and chunks == emu.PASS_MAX_CHUNKS
    assert emu.PASS_MAX_R == 16 * rts
    for R in (1, 16, 17, 32, 33, 48):
        rt = (R + 15) // 16
        assert emu.pass_x_area(R) == 160 * 1024 - nc * (pieces if rt == 1 else 1) * rt * 1024 - 256


PASS_SHAPES = [(m.N, m.K) for m in W.layer_mats(0)] + [(W.lm_head().N, W.lm_head().K)]


@pytest.mark.parametrize("R", [1, 3, 12, 16, 24, 33, 48])
def test_pass_shapes_take_every_step_once(R):
    counts, chunks = emu.pass_coverage(PASS_SHAPES, R, P=256)
    for (N, K), c in zip(PASS_SHAPES, counts):
        assert c.size == ((N + 15) // 16) * (K // 256)
        assert (c == 1).all(), f"N={N} K={K} R={R}: steps taken {np.bincount(c)}"
    if R == 12:
        # Q|K|V, gate|up and the head in one chunk; O (K = 8192) in two, down (K = 25600) in five
        assert chunks.tolist() == [1, 2, 1, 5, 1]
    if R == 16:
        assert chunks.tolist() == [2, 2, 2, 10, 2]
    if R == 24:
        # two row tiles (one piece slot each): 10 blocks per chunk fit, down (100 blocks) goes in 10
        assert chunks.tolist() == [2, 4, 2, 10, 2]
    if R == 48:
        assert chunks.tolist() == [4, 8, 4, 20, 4]


def test_one_row_tile_takes_at_most_16_chunks():
    """At one row tile the last chunk to arrive adds a sub-tile's partial tiles in
    one round of 16 loads, so the planner never cuts a GEMM into more chunks there:
    K = 34 blocks at 16 rows (fitting only as 17 chunks of 2) is refused, and at 17
    rows (two row tiles, 32 chunks allowed) it runs in 17."""
    _, ch16 = emu.pass_coverage([(64, 34 * 256)], 16, P=256)
    _, ch17 = emu.pass_coverage([(64, 34 * 256)], 17, P=256)
    assert ch16.tolist() == [0] and ch17.tolist() == [17]


@pytest.mark.parametrize("P", [1, 3, 7, 64, 250])
def test_odd_shapes_take_every_step_once(P):
    rng = np.random.default_rng(P)
    shapes = [(int(rng.integers(1, 700)), 256 * int(rng.integers(1, 40))) for _ in range(12)] + [(1, 256), (17, 512)]
    counts, chunks = emu.pass_coverage(shapes, 12, P=P, x_area=4 * 6656)
    planned = 0
    for (N, K), c, S in zip(shapes, counts, chunks):
        if S == 0:                     # no chunking fits (the library refuses such a sequence)
            KB = K // 256
            assert not any(KB % S2 == 0 and KB // S2 <= 4 for S2 in range(1, min(P, emu.pass_max_chunks(12), KB) + 1))
            assert (c == 0).all()
            continue
        planned += 1
        assert (K // 256) % S == 0 and K // 256 // S <= 4 and S <= min(P, emu.pass_max_chunks(12))
        assert (c == 1).all(), f"P={P} N={N} K={K} S={S}"
    assert planned >= 2


@pytest.mark.parametrize("msum", [False, True])
@pytest.mark.parametrize("P,x_blocks", [(7, 3), (16, 2), (5, 40), (1, 8)])
def test_pass_replay_matches_oracle(orc, P, x_blocks, msum):
    """A 4-GEMM sequence on few workgroups (several units each, some with none),
    with an LDS area of x_blocks blocks, so that some GEMMs run in K chunks; the
    min term in either form."""
    R = 12
    shapes = [(300, 1024), (64, 2048), (520, 512), (33, 1536)]
    mats, xs = [], []
    for i, (N, K) in enumerate(shapes):
        mats.append((synth.matrix_rows(6, 20 + i, N, K), N, K))
        xs.append(synth.x_bf16(6, 30 + i, R, K, outlier_p=0.01))
    x_area = x_blocks * emu.pass_block_bytes(R)
    ys = emu.pass_run(mats, xs, P, x_area=x_area, msum=msum)
    for (canon, N, K), x, y in zip(mats, xs, ys):
        m = assert_parity(y, orc.gemm(canon, N, K, x), f"pass replay P={P} N={N} K={K}")
        assert m["rel_l2"] < 2e-6


@pytest.mark.parametrize("R,P,x_blocks", [(24, 7, 3), (33, 16, 2), (48, 5, 4), (17, 3, 6)])
def test_pass_replay_with_row_tiles_matches_oracle(orc, R, P, x_blocks):
    """Rows beyond 16 in two or three row tiles (each step feeds every tile, the
    pieces and partial tiles carry all of them), some GEMMs in K chunks."""
    shapes = [(300, 1024), (64, 2048), (40, 512)]
    mats, xs = [], []
    for i, (N, K) in enumerate(shapes):
        mats.append((synth.matrix_rows(7, 60 + i, N, K), N, K))
        xs.append(synth.x_bf16(7, 70 + i, R, K, outlier_p=0.01))
    ys = emu.pass_run(mats, xs, P, x_area=x_blocks * emu.pass_block_bytes(R))
    for (canon, N, K), x, y in zip(mats, xs, ys):
        m = assert_parity(y, orc.gemm(canon, N, K, x), f"pass replay R={R} P={P} N={N} K={K}")
        assert m["rel_l2"] < 2e-6


@pytest.mark.parametrize("R", range(1, 49))
def test_in_place_conversion_touches_only_its_own_raw_pair(R):
    """The pass kernel converts a slot in place: raw row pair q (2 x 512 bytes of
    bf16) lands at 1056 q, where its two 528-byte operand rows go (a missing odd
    row included), and the 8 R fp32 sums go to 528 times R rounded up to even.
    Pairs are dealt to all waves in any order, so replayed byte by byte: the
    writes of pair q fall on no other pair's raw bytes, and everything stays in
    the slot (the reads of a pair come before its writes, in one wave)."""
    sb = emu.pass_block_bytes(R)
    row, pairs = 528, (R + 1) // 2
    R2 = 2 * pairs
    owner = np.full(sb, -1)                       # raw pair whose bytes lie here
    for q in range(pairs):
        assert 1056 * q + 1024 <= sb
        owner[1056 * q:1056 * q + 1024] = q
    for q in range(pairs):
        writes = []
        for r in (2 * q, 2 * q + 1):
            writes.append((row * r, row * r + 512))                          # operands of row r
            if r < R:
                writes += [(row * R2 + (gg * R + r) * 8, row * R2 + (gg * R + r) * 8 + 8) for gg in range(4)]
        for lo, hi in writes:
            assert 0 <= lo and hi <= sb, f"R={R} pair {q}: write [{lo}, {hi}) outside the slot of {sb}"
            hit = set(owner[lo:hi].tolist()) - {-1, q}
            assert not hit, f"R={R} pair {q}: write [{lo}, {hi}) over the raw bytes of pairs {hit}"


@pytest.mark.parametrize("R,P", [(12, 256), (16, 256), (1, 256), (12, 100), (16, 37), (24, 256), (48, 256), (48, 61)])
def test_gated_wait_sets_hold_exactly_the_producers(R, P):
    """With gated inputs, K chunk c of down (25600 inputs) waits for the
    workgroups holding gate|up outputs [256 kbc c, 256 kbc (c + 1)) and the same
    + 25600: derived here from the deal of every workgroup's units, each chunk's
    wait set must be exactly those holders."""
    from synth import workloads as W
    gu, dn = W.layer_mats(0)[2], W.layer_mats(0)[3]
    x_area = emu.PASS_X_AREA
    _, chunks = emu.pass_coverage([(gu.N, gu.K), (dn.N, dn.K)], R, P=P, x_area=x_area)
    Sp, Sc = int(chunks[0]), int(chunks[1])
    NSp, kbc, half = gu.N // 16, dn.K // 256 // Sc, dn.K // 16
    rot_p = (2 * 37) % P                         # the gate|up GEMM's rotation at index 2 of a layer
    holders = {}                                 # output sub-tile -> workgroups holding a unit of it
    for q in range(P):
        _, ns0, ns1 = emu.pass_units(q, Sp, P, NSp, rot_p)
        for ns in range(ns0, ns1):
            holders.setdefault(ns, set()).add(q)
    assert sorted(holders) == list(range(NSp))
    for c in range(Sc):
        need = set()
        for ns in list(range(16 * kbc * c, 16 * kbc * (c + 1))) + list(range(half + 16 * kbc * c, half + 16 * kbc * (c + 1))):
            need |= holders[ns]
        assert emu.pass_gated_mask(c, kbc, half, P, NSp, Sp, rot_p) == need, (R, P, c)


def _replay_piece_protocol(n, kbc, seed, NC=8, NH=4, PIECES=2):
    """The pass kernel's piece protocol for one workgroup's n steps in units of
    kbc steps, replayed with its waits and a random interleaving: compute wave
    w writes one piece per unit its sub-range touches, piece j into slot
    j mod PIECES once piece j - PIECES has been taken; helper h takes the
    single-piece units of waves h and h + NH as they are written and the first
    piece of the last wave of each unit those two waves begin and later waves
    finish, then adds each such unit's pieces in wave order.  Returns per unit
    the waves whose pieces were added, in order, and per helper its units;
    fails on a deadlock or a piece taken out of turn."""
    rng = np.random.default_rng(seed)
    first = [emu.pass_wave_first(w, NC, n) for w in range(NC + 1)]
    owner = lambda i: emu.pass_step_owner(i, NC, n)
    written = [0] * NC
    taken = [[0] * PIECES for _ in range(NC)]
    sums, mine = {}, {h: [] for h in range(NH)}

    def take(w, j):
        assert written[w] > j and taken[w][j % PIECES] == j // PIECES, (w, j)
        taken[w][j % PIECES] = j // PIECES + 1

    def wave(w):
        a, b = first[w], first[w + 1]
        for j in range(((b - 1) // kbc + 1 - a // kbc) if a < b else 0):
            for _ in range(int(rng.integers(0, 3))):
                yield "busy"
            while j >= PIECES and taken[w][j % PIECES] < j // PIECES:
                yield "blocked"
            written[w] = j + 1
            yield "progress"

    def helper(h):
        ws = [h, h + NH]
        A, B = [first[w] for w in ws], [first[w + 1] for w in ws]
        f = [a // kbc for a in A]
        u = [(a + kbc - 1) // kbc for a in A]
        e = [B[i] // kbc if A[i] < B[i] else u[i] for i in range(2)]
        ul, wl = [], []
        for i in range(2):
            last = (B[i] - 1) // kbc
            shared = A[i] < B[i] and last * kbc >= A[i] and (last + 1) * kbc > B[i]
            ul.append(last if shared else -1)
            wl.append(owner((last + 1) * kbc - 1) if shared else ws[i])
        have = [x < 0 for x in ul]
        while True:
            moved = pending = False
            for i in range(2):
                if u[i] < e[i]:
                    j = u[i] - f[i]
                    if written[ws[i]] > j:
                        take(ws[i], j)
                        sums[u[i]] = [ws[i]]
                        mine[h].append(u[i])
                        u[i] += 1
                        moved = True
                    pending = pending or u[i] < e[i]
                if not have[i]:
                    if written[wl[i]] > 0:
                        take(wl[i], 0)
                        have[i] = moved = True
                    else:
                        pending = True
            if not pending:
                break
            yield "progress" if moved else "blocked"
        for i in range(2):
            if ul[i] < 0:
                continue
            order, j = [ws[i]], ul[i] - f[i]
            while written[ws[i]] <= j:
                yield "blocked"
            take(ws[i], j)
            for ww in range(ws[i] + 1, wl[i]):
                if first[ww] == first[ww + 1]:
                    continue
                while written[ww] <= 0:
                    yield "blocked"
                take(ww, 0)
                order.append(ww)
            order.append(wl[i])
            sums[ul[i]] = order
            mine[h].append(ul[i])
            yield "progress"

    live = [wave(w) for w in range(NC)] + [helper(h) for h in range(NH)]
    while live:
        moved = False
        for k in rng.permutation(len(live)):
            if live[k] is None:
                continue
            try:
                moved = next(live[k]) != "blocked" or moved
            except StopIteration:
                live[k] = None
                moved = True
        live = [g for g in live if g is not None]
        assert moved or not live, f"deadlock at n={n} kbc={kbc}"
    return sums, mine


@pytest.mark.parametrize("pieces", [2, 1])
@pytest.mark.parametrize("units,kbc", [(25, 10), (13, 20), (12, 20), (3, 20), (2, 20), (3, 16), (7, 20), (38, 20),
                                       (1, 20), (7, 1), (8, 3), (1, 1), (1, 32), (125, 4), (5, 7)])
def test_piece_protocol_takes_every_unit_once_in_wave_order(units, kbc, pieces):
    """Every unit's pieces are added once, in wave order, whatever the
    interleaving; no wave waits forever for a slot (two slots per wave at one
    row tile, one from two on); and a helper's units are the ones whose first
    step lies in its two waves (the units whose chunk partials it arrives with)."""
    n = units * kbc
    for seed in range(6):
        sums, mine = _replay_piece_protocol(n, kbc, seed, PIECES=pieces)
        assert sorted(sums) == list(range(units))
        for u, order in sums.items():
            touching = sorted({emu.pass_step_owner(i, 8, n) for i in range(u * kbc, (u + 1) * kbc)})
            assert order == touching, (u, order, touching)
        for h, us in mine.items():
            assert sorted(us) == [u for u in range(units) if emu.pass_step_owner(u * kbc, 8, n) % 4 == h]
