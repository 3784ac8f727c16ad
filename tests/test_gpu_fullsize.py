"""Parity at the full workload sizes, in the launch configuration the benchmark
times (R rows, automatic kernel choice).  The layer's four GEMMs and the output
head are compared with the oracle on every output; the full 257-GEMM pass runs
through the benchmark's own call (graph-replayed sequence with the head's row
argmax and the draft check) and is compared on every output of layers 0 and 63
and of the head, on sampled outputs of the other GEMMs (the oracle recomputes
only the sampled weight rows), and on the argmax and the emitted tokens."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from synth import workloads as W
from tests import gpu_util as G
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu


def fused_canon(seed, m):
    return np.concatenate([synth.matrix_rows(seed, mid, n, m.K) for mid, n in zip(m.mids, m.splits)])


def sampled_rows(seed, m, ns):
    """Canonical bytes of output rows ns of a (possibly fused) matrix."""
    out = []
    bounds = np.cumsum((0,) + m.splits)
    for n in ns:
        p = int(np.searchsorted(bounds, n, side="right") - 1)
        local = n - bounds[p]
        out.append(synth.matrix_rows(seed, m.mids[p], m.splits[p], m.K, n0=local, n1=local + 1))
    return np.concatenate(out)


def sample_ns(N, count, seed):
    rng = np.random.default_rng(seed)
    ns = set(rng.choice(N, size=min(N, count), replace=False).tolist())
    ns |= {0, 1, 15, 16, N - 1, N - 16}
    return np.array(sorted(n for n in ns if 0 <= n < N))


LAYER_RS = (1, 3, 12, 24, 48)
_layer_refs = {}


def layer_ref(orc, which):
    """(matrix, canonical bytes, x of 48 rows, oracle y of 48 rows) of one of layer
    0's GEMMs.  The activation rows of a smaller R are the first rows of the
    48-row x, and the oracle's rows are independent (pinned bitwise), so its
    first R rows are the reference at R."""
    if which not in _layer_refs:
        _layer_refs.clear()                    # keep one matrix's reference on the host at a time
        seed = W.SEED_LAYER
        m = {mm.name: mm for mm in W.layer_mats(0)}[which]
        canon = fused_canon(seed, m)
        x = synth.x_bf16(seed, W.X_STREAM[m.K], max(LAYER_RS), m.K)
        print(f"oracle {which} N={m.N} K={m.K} R={max(LAYER_RS)}", flush=True)
        _layer_refs[which] = (m, canon, x, orc.gemm(canon, m.N, m.K, x))
    return _layer_refs[which]


@pytest.mark.parametrize("which", ["qkv", "o", "gate_up", "down"])
def test_layer_matrix_all_outputs(orc, which):
    """Every output of the full-size layer GEMMs at R = 1, 3, 12, 24 and 48 on the
    automatic choice (streaming kernel, whole-tile and stream-K ranges, K chunks,
    and from 24 rows the row-tiled kernel), and at R = 1 and 3 on the vector-unit
    kernel."""
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import qgemm as Q
    m, canon, x48, ref48 = layer_ref(orc, which)
    packed = G.upload_packed(canon, m.N, m.K)
    g = wsg.QGemm(packed, m.N, m.K, max_R=max(LAYER_RS))
    for R in LAYER_RS:
        info = g.query(R)
        print(f"layer {which} N={m.N} K={m.K} R={R} path={info['path']} wgs={info['workgroups']} "
              f"chunks={info['k_chunks']} sums={info['min_term_sums']}", flush=True)
        y = G.run(g, x48[:R])
        assert_parity(y, ref48[:R], f"{which} R={R} path={info['path']}")
    for R in (1, 3):
        print(f"layer {which} R={R} vector-unit kernel", flush=True)
        assert_parity(G.run(g, x48[:R], path=Q.PATH_VALU), ref48[:R], f"valu {which} R={R}")
    # the same GEMM in the persistent pass kernel: one, two and three row tiles, in K
    # chunks from 24 rows on, with several of a helper's chunk sums added per round
    import torch
    seq = wsg.Seq([g], persistent=True)
    xd = G.to_dev(x48)
    y = torch.empty((max(LAYER_RS), m.N), dtype=torch.float32, device="cuda")
    for R in (12, 24, 48):
        print(f"layer {which} R={R} persistent pass kernel", flush=True)
        y.fill_(-7.0)
        seq.run([xd[:R]], [y[:R]], R)
        torch.cuda.synchronize()
        assert_parity(y[:R].cpu().numpy(), ref48[:R], f"persistent {which} R={R}")
    assert seq.errors() == 0
    seq.close()
    g.close()


def test_vector_unit_k_chunks_sampled(orc):
    """A shape whose step ranges outgrow LDS at R = 4 even with 8 wave columns:
    the vector-unit kernel runs K in two chunks."""
    from weight_streaming_gemm_amd import qgemm as Q
    import weight_streaming_gemm_amd as wsg
    N, K, R = 32768, 16384, 4
    print(f"valu chunks N={N} K={K} R={R}", flush=True)
    canon = synth.matrix_rows(11, 2, N, K)
    packed = G.upload_packed(canon, N, K)
    g = wsg.QGemm(packed, N, K, max_R=R)
    info = g.query(R, Q.PATH_VALU)
    assert info["k_chunks"] == 2, info
    x = synth.x_bf16(11, 3, R, K, outlier_p=0.01)
    y = G.run(g, x, path=Q.PATH_VALU)
    ns = sample_ns(N, 96, 5)
    rows = np.concatenate([synth.matrix_rows(11, 2, N, K, n0=n, n1=n + 1) for n in ns])
    ref = orc.gemm(rows, len(ns), K, x)
    assert_parity(y[:, ns], ref, "valu chunks")
    g.close()


def test_ragged_schedule_sampled_steps(orc):
    """The agent schedule (R_t = 3 a_t, fresh activations with 1 % outliers per
    step) through one graph-mode sequence over layer 0's GEMMs: R changes from
    step to step; every output of every checked step is compared with the oracle,
    and a repeated step gives the same bits."""
    import torch
    import weight_streaming_gemm_amd as wsg
    seed = W.SEED_RAGGED
    sched = W.ragged_schedule(seed, 100)
    steps = [sched.index(R) for R in (3, 6, 9, 12)] + [10, 11]
    mats = W.layer_mats(0)
    gs, canons = [], []
    for m in mats:
        canon = fused_canon(seed, m)
        gs.append(wsg.QGemm(G.upload_packed(canon, m.N, m.K), m.N, m.K, max_R=12))
        canons.append(canon)
    seq = wsg.Seq(gs)
    ys = [torch.empty((12, m.N), dtype=torch.float32, device="cuda") for m in mats]
    first = {}
    for t in steps + steps[:1]:
        R = sched[t]
        print(f"ragged step {t} R={R}", flush=True)
        xs_np = [synth.x_bf16(seed, 1000 * (t + 1) + W.X_STREAM[m.K], R, m.K, outlier_p=0.01) for m in mats]
        seq.run([G.to_dev(x) for x in xs_np], [y[:R] for y in ys], R)
        torch.cuda.synchronize()
        got = [y[:R].cpu().numpy() for y in ys]
        if t in first:
            for a, b in zip(got, first[t]):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
            continue
        first[t] = got
        for i, m in enumerate(mats):
            assert_parity(got[i], orc.gemm(canons[i], m.N, m.K, xs_np[i]), f"ragged t={t} {m.name}")
    seq.close()
    for g in gs:
        g.close()


@pytest.mark.parametrize("R", [W.R_DEFAULT, 24])
def test_output_head_argmax_and_sampled_parity(orc, R):
    """All 151936 outputs against the oracle and the row argmax; at 24 rows (8
    agents) the head takes the row-tiled kernel."""
    import torch
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import qgemm as Q
    seed = W.SEED_PASS
    m = W.lm_head()
    print(f"lm_head N={m.N} K={m.K} R={R}", flush=True)
    canon = fused_canon(seed, m)
    packed = G.upload_packed(canon, m.N, m.K)
    g = wsg.QGemm(packed, m.N, m.K, max_R=R)
    assert g.query(R)["path"] == (Q.PATH_TILED if R >= 24 else Q.PATH_MFMA)
    x = synth.x_bf16(seed, W.X_STREAM[m.K], R, m.K)
    xd = G.to_dev(x)
    y = torch.empty((R, m.N), dtype=torch.float32, device="cuda")
    g.run(xd, y)
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    wsg.argmax_rows(y, idx)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    ref = orc.gemm(canon, m.N, m.K, x)             # all 151936 outputs, fp64
    assert_parity(yh, ref, "lm_head")
    ref_idx = orc.argmax_rows(ref)
    top2 = np.sort(ref, axis=1)[:, -2:]
    margin = top2[:, 1] - top2[:, 0]
    err = np.abs(yh - ref).max()
    got_idx = idx.cpu().numpy()
    clear = margin > 10 * err
    for r in range(R):
        print(f"row {r}: argmax {ref_idx[r]} margin {margin[r]:.3e} vs max|dy| {err:.3e}"
              f"{'' if clear[r] else ' (ambiguous within the error bound)'}", flush=True)
    if R == W.R_DEFAULT:
        assert clear.all(), "an argmax of the 12-row step is ambiguous within the error bound"
    assert clear.mean() >= 0.9
    # exact wherever the oracle's top two are apart by more than 10x the observed error
    assert np.array_equal(got_idx[clear], ref_idx[clear])
    g.close()


def test_shared_tile_counters_rearm_over_repeats(orc):
    """Tiles shared by several workgroups reuse their arrival counters launch after launch."""
    import torch
    import weight_streaming_gemm_amd as wsg
    m = {mm.name: mm for mm in W.layer_mats(0)}["down"]
    canon = fused_canon(5, m)
    packed = G.upload_packed(canon, m.N, m.K)
    g = wsg.QGemm(packed, m.N, m.K, max_R=12)
    q = g.query(12)
    assert q["steps"] % q["workgroups"] != 0 or (q["steps"] // q["workgroups"]) % (m.K // 256) != 0   # tiles are shared
    x = synth.x_bf16(5, 1, 12, m.K)
    xd = G.to_dev(x)
    ys = [torch.empty((12, m.N), dtype=torch.float32, device="cuda") for _ in range(6)]
    for y in ys:
        g.run(xd, y)
    torch.cuda.synchronize()
    first = ys[0].cpu().numpy()
    for y in ys[1:]:
        assert np.array_equal(y.cpu().numpy().view(np.uint32), first.view(np.uint32))
    ns = sample_ns(m.N, 64, 1)
    assert_parity(first[:, ns], orc.gemm(sampled_rows(5, m, ns), len(ns), m.K, x), "down repeats")
    g.close()


@pytest.mark.parametrize("persistent", [False, True])
def test_full_pass_run_verify(orc, persistent):
    """The benchmark's timed call itself: all 257 GEMMs of the pass resident (17.99
    GB), one qgemm_seq_run_verify at 12 rows (4 agents x (token + 2 drafts)) with
    the head's row argmax and the greedy draft check, graph-replayed or as one
    persistent launch.  Every output
    of layers 0 and 63 and of the head is compared with the oracle, 16 sampled
    outputs of every other GEMM, the argmax exactly, and the emitted tokens with
    the oracle's greedy check.  The drafts are made from the oracle's argmax so
    that agents accept two, one and none of their drafts."""
    import torch
    import weight_streaming_gemm_amd as wsg
    seed, R, D = W.SEED_PASS, W.R_DEFAULT, W.ROWS_PER_AGENT - 1
    mats = W.full_pass()
    print(f"full pass: {len(mats)} GEMMs, R={R}, persistent={persistent}", flush=True)
    gs, packs = [], []
    for i, m in enumerate(mats):
        packed = G.upload_packed(fused_canon(seed, m), m.N, m.K)
        packs.append(packed)
        gs.append(wsg.QGemm(packed, m.N, m.K, max_R=R))
        if i % 64 == 0:
            print(f"  resident {i + 1}/{len(mats)}", flush=True)
    xs = {K: synth.x_bf16(seed, sid, R, K) for K, sid in W.X_STREAM.items()}
    xd = {K: G.to_dev(x) for K, x in xs.items()}
    ys = [torch.empty((R, m.N), dtype=torch.float32, device="cuda") for m in mats]
    head = mats[-1]
    print("oracle: head", flush=True)
    head_canon = fused_canon(seed, head)
    ref_head = orc.gemm(head_canon, head.N, head.K, xs[head.K])
    ref_idx = orc.argmax_rows(ref_head)
    A = R // (D + 1)
    drafts = np.zeros((A, D), np.int32)
    for a in range(A):
        base = a * (D + 1)
        accept = max(0, D - a)                       # agent 0 accepts 2, agent 1 one, agents 2, 3 none
        for i in range(D):
            drafts[a, i] = ref_idx[base + i] if i < accept else (ref_idx[base + i] + 1) % head.N
    tok_ref, n_ref = orc.verify_greedy(ref_idx, drafts, D)
    idx = torch.empty(R, dtype=torch.int32, device="cuda")
    tokens = torch.empty((A, D + 1), dtype=torch.int32, device="cuda")
    n_new = torch.empty(A, dtype=torch.int32, device="cuda")
    seq = wsg.Seq(gs, persistent=persistent)
    seq.run_verify([xd[m.K] for m in mats], ys, R, idx, G.to_dev(drafts), D, tokens, n_new)
    torch.cuda.synchronize()
    assert seq.errors() == 0
    print("pass done; comparing", flush=True)
    full = set(range(4)) | set(range(4 * 63, 4 * 64)) | {len(mats) - 1}
    for i, m in enumerate(mats):
        y = ys[i].cpu().numpy()
        assert np.isfinite(y).all(), f"GEMM {i} {m.name}: non-finite output"
        if i == len(mats) - 1:
            assert_parity(y, ref_head, "head")
        elif i in full:
            print(f"oracle: GEMM {i} ({m.name}), all outputs", flush=True)
            assert_parity(y, orc.gemm(fused_canon(seed, m), m.N, m.K, xs[m.K]), f"GEMM {i} {m.name}")
        else:
            ns = sample_ns(m.N, 16, i)
            assert_parity(y[:, ns], orc.gemm(sampled_rows(seed, m, ns), len(ns), m.K, xs[m.K]),
                          f"GEMM {i} {m.name} sampled")
    top2 = np.sort(ref_head, axis=1)[:, -2:]
    err = np.abs(ys[-1].cpu().numpy() - ref_head).max()
    assert (top2[:, 1] - top2[:, 0] > 10 * err).all(), "an argmax is ambiguous within the error bound"
    assert np.array_equal(idx.cpu().numpy(), ref_idx)
    assert np.array_equal(tokens.cpu().numpy(), tok_ref) and np.array_equal(n_new.cpu().numpy(), n_ref)
    assert sorted(n_ref.tolist()) == [1, 1, 2, 3]
    seq.close()
    if persistent:
        # with gated inputs (each down projection waits only for the gate|up
        # outputs it reads) every output is bitwise the same
        print("persistent pass with gated inputs", flush=True)
        ys2 = [torch.empty_like(y) for y in ys]
        idx2, tokens2, n_new2 = torch.empty_like(idx), torch.empty_like(tokens), torch.empty_like(n_new)
        seq2 = wsg.Seq(gs, persistent=True, gated_inputs=True)
        seq2.run_verify([xd[m.K] for m in mats], ys2, R, idx2, G.to_dev(drafts), D, tokens2, n_new2)
        torch.cuda.synchronize()
        assert seq2.errors() == 0
        for i in range(len(mats)):
            assert torch.equal(ys2[i].view(torch.int32), ys[i].view(torch.int32)), f"GEMM {i}"
        assert torch.equal(idx2, idx) and torch.equal(tokens2, tokens) and torch.equal(n_new2, n_new)
        seq2.close()
        del ys2
    for g in gs:
        g.close()
    del packs, ys
    torch.cuda.empty_cache()
