#!/usr/bin/env python3
"""Benchmark of the weight-streaming Q4_K-style GEMM on one MI355X.

A step is one full decode-step weight pass: 64 transformer layers of four
projections (Q|K|V fused, O, gate|up fused, down; hidden 5120, 64 query heads
and 8 key/value heads of 128, MLP 25600) and a 5120 -> 151936 output head with
its row argmax and the greedy check of each agent's two draft tokens, for R
stacked activation rows (4 agents x (1 token + 2 drafts)
= 12 by default).  Weights are streamed once per step; 17,990,737,920 packed
bytes (144 B per 256 weights).  Inputs are seeded synthetic data of those
shapes and distributions, resident in HBM before timing.

A pass runs as one cooperative launch of the pass kernel where it serves the
row count (up to 48 rows), else as a replayed graph of one streaming-kernel
launch per GEMM (--launch picks one of them for every row count).

Prints one JSON line (rank 0): effective weight GB/s and ms per pass, with a
roofline record for the dominant kernel (and the device's practical read
ceiling from a plain read kernel) and the fp64 CPU oracle timed on a bounded
sample beside it.  Extra detail goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s and % HBM peak at R=12; ms per full 27B weight pass"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_pass(R_max: int, seed: int):
    """Generate, upload and pack all 257 matrices; return handles and buffers."""
    import numpy as np
    import torch
    import synth
    from synth import workloads as W
    import weight_streaming_gemm_amd as wsg

    dev = torch.device("cuda:0")
    mats = W.full_pass()
    max_bytes = max(m.weights // 256 * 144 for m in mats)
    host = torch.empty(max_bytes, dtype=torch.uint8, pin_memory=True)
    host_np = host.numpy()
    canon_d = torch.empty(max_bytes, dtype=torch.uint8, device=dev)
    gemms, packed = [], []
    t0 = time.time()
    for i, m in enumerate(mats):
        off = 0
        for mid, n_part in zip(m.mids, m.splits):
            nb = n_part * (m.K // 256) * 144
            synth.matrix_rows(seed, mid, n_part, m.K, out=host_np[off:off + nb])
            off += nb
        canon_d[:off].copy_(host[:off], non_blocking=False)
        p = torch.empty(wsg.packed_size(m.N, m.K), dtype=torch.uint8, device=dev)
        wsg.pack(canon_d, p, m.N, m.K)
        torch.cuda.synchronize()
        packed.append(p)
        gemms.append(wsg.QGemm(p, m.N, m.K, max_R=R_max))
        if i % 64 == 0:
            log(f"[setup] packed {i + 1}/{len(mats)} matrices, {time.time() - t0:.1f}s")
    del canon_d, host
    xs_by_width = {}
    for width, sid in W.X_STREAM.items():
        xb = synth.x_bf16(seed, sid, R_max, width)
        xs_by_width[width] = torch.from_numpy(xb.view(np.int16)).to(dev)
    xs = [xs_by_width[m.K] for m in mats]
    ys = [torch.empty((R_max, m.N), dtype=torch.float32, device=dev) for m in mats]
    idx = torch.empty(R_max, dtype=torch.int32, device=dev)
    log(f"[setup] {len(mats)} matrices resident, {sum(p.numel() for p in packed) / 1e9:.3f} GB packed, "
        f"{time.time() - t0:.1f}s")
    return mats, gemms, packed, xs, ys, idx


def draft_check(R: int, seed: int):
    """Device buffers for the step's draft check: R rows as agents of a token and
    two drafts (when R is a multiple of 3, else no drafts); seeded draft tokens."""
    import numpy as np
    import torch
    from synth import workloads as W
    D = W.ROWS_PER_AGENT - 1 if R % W.ROWS_PER_AGENT == 0 else 0
    A = R // (D + 1)
    rng = np.random.default_rng(seed)
    drafts = torch.from_numpy(rng.integers(0, W.VOCAB, size=(A, max(D, 1))).astype(np.int32)[:, :D].copy()).cuda()
    tokens = torch.empty((A, D + 1), dtype=torch.int32, device="cuda")
    n_new = torch.empty(A, dtype=torch.int32, device="cuda")
    return D, drafts, tokens, n_new


def time_pass(seq, xs, ys, idx, R: int, steps: int, warmup: int):
    """ms per decode step: the 257 GEMMs, the head's row argmax and the greedy
    check of the agents' drafts (one graph replay)."""
    import torch
    xr = [x[:R] for x in xs]
    yr = [y[:R] for y in ys]
    D, drafts, tokens, n_new = draft_check(R, 7)

    def one():
        seq.run_verify(xr, yr, R, idx, drafts, D, tokens, n_new)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        one()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_dominant_kernel(gemms, xs, ys, R: int, reps: int):
    """Average duration of the streaming kernel (qgemm_run enqueues exactly one
    kernel) over back-to-back launches across all 257 matrices, timed with HIP
    events on the stream the kernels run on (torch's current stream)."""
    import torch
    st = torch.cuda.current_stream()
    for g, x, y in zip(gemms, xs, ys):
        g.run(x[:R], y[:R])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        for g, x, y in zip(gemms, xs, ys):
            g.run(x[:R], y[:R])
    e1.record(st)
    torch.cuda.synchronize()
    launches = reps * len(gemms)
    return e0.elapsed_time(e1) / launches, launches


def time_paths(gemms, xs, ys, Rs, reps: int = 5):
    """ms per pass (the 257 streaming kernels, no argmax) on each kernel path for
    each R: the measurement behind the automatic choice between the vector-unit
    and matrix-core kernels.  One graph of the pass per (path, R), replayed."""
    import torch
    from weight_streaming_gemm_amd import qgemm as Q
    out = {}
    for R in Rs:
        rec = {}
        for name, path in (("valu", Q.PATH_VALU), ("mfma", Q.PATH_MFMA)):
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                for g, x, y in zip(gemms, xs, ys):
                    g.run(x[:R], y[:R], R, path=path)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for g, x, y in zip(gemms, xs, ys):
                    g.run(x[:R], y[:R], R, path=path)
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            rec[name + "_ms"] = round(e0.elapsed_time(e1) / reps, 4)
            del graph
        rec["auto"] = "valu" if gemms[0].query(R)["path"] == Q.PATH_VALU else "mfma"
        out[str(R)] = rec
    return out


def graph_ms(calls, reps: int = 5) -> float:
    """ms per replay of a graph of the given launches (captured once, warmed once)."""
    import torch
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for c in calls:
            c()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / reps


def layer_report(seed: int, edge: int, Rs, copies: int):
    """One layer's four GEMMs (Q|K|V, O, gate|up, down), `copies` rotating weight
    copies so that no replay is served from the 256 MB Infinity Cache: per-matrix
    and per-layer time, GB/s and % of 8 TB/s for each R, on the matrix-core path
    and (R <= 4) on the vector-unit path; useful TFLOP/s against the fp16 dense
    matrix-core peak."""
    import numpy as np
    import torch
    import synth
    from synth import workloads as W
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import qgemm as Q
    from weight_streaming_gemm_amd import roofline as RF
    dev = torch.device("cuda:0")
    R_max = max(Rs)
    mats = W.layer_mats(0)
    per = []
    for m in mats:
        canon = np.concatenate([synth.matrix_rows(seed, mid, n, m.K, edge_mode=edge) for mid, n in zip(m.mids, m.splits)])
        cd = torch.from_numpy(canon).to(dev)
        pk = torch.empty(wsg.packed_size(m.N, m.K), dtype=torch.uint8, device=dev)
        wsg.pack(cd, pk, m.N, m.K)
        torch.cuda.synchronize()
        del cd
        pks = [pk] + [pk.clone() for _ in range(copies - 1)]
        gs = [wsg.QGemm(q, m.N, m.K, max_R=R_max) for q in pks]
        x = torch.from_numpy(synth.x_bf16(seed, W.X_STREAM[m.K], R_max, m.K).view(np.int16)).to(dev)
        y = torch.empty((R_max, m.N), dtype=torch.float32, device=dev)
        per.append((m, pks, gs, x, y))
    layer_bytes = sum(m.packed_bytes for m in mats)
    out = {}
    for R in Rs:
        rec = {}
        for pname, path in (("mfma", Q.PATH_MFMA), ("valu", Q.PATH_VALU), ("auto", Q.PATH_AUTO)):
            if path == Q.PATH_VALU and R > 4:
                continue
            if path == Q.PATH_AUTO and R < Q.TILED_MIN_R:
                continue          # the automatic choice is the streaming kernel here
            if path == Q.PATH_AUTO:
                log(f"[layer] R={R} automatic choice: " +
                    ", ".join(f"{m.name} {'tiled' if gs[0].query(R)['path'] == Q.PATH_TILED else 'streaming'}"
                              for m, pks, gs, x, y in per))
            prec = {}
            for m, pks, gs, x, y in per:
                us = graph_ms([lambda g=g, x=x, y=y: g.run(x[:R], y[:R], R, path=path) for g in gs]) / copies * 1e3
                prec[m.name] = {"us": round(us, 2), "GB_s": round(m.packed_bytes / us / 1e3, 1),
                                "pct_hbm_peak": round(m.packed_bytes / us / 1e3 / RF.HBM_PEAK_GBS * 100, 1)}
                if pname != "valu":
                    prec[m.name]["useful_tflop_s"] = round(2 * R * m.N * m.K / us / 1e6, 1)
            calls = []
            for c in range(copies):
                for m, pks, gs, x, y in per:
                    calls.append(lambda g=gs[c], x=x, y=y: g.run(x[:R], y[:R], R, path=path))
            us = graph_ms(calls) / copies * 1e3
            prec["layer"] = {"us": round(us, 2), "GB_s": round(layer_bytes / us / 1e3, 1),
                             "pct_hbm_peak": round(layer_bytes / us / 1e3 / RF.HBM_PEAK_GBS * 100, 1)}
            if pname != "valu":
                flops = sum(2 * R * m.N * m.K for m in mats)
                prec["layer"]["useful_tflop_s"] = round(flops / us / 1e6, 1)
                prec["layer"]["pct_fp16_mfma_peak"] = round(flops / us / 1e6 / RF.MFMA_F16_DENSE_TFLOPS * 100, 2)
            rec[pname] = prec
            log(f"[layer seed={seed} edge={edge}] R={R:2d} {pname}: " +
                ", ".join(f"{k} {v['us']:.1f} us" for k, v in prec.items()))
        out[str(R)] = rec
    for m, pks, gs, x, y in per:
        for g in gs:
            g.close()
    return {"seed": seed, "edge_blocks": bool(edge), "copies": copies, "layer_packed_bytes": layer_bytes,
            "by_R": out}


def prefill_report(seed: int, chunks, copies: int = 2):
    """Prompt-chunk rows sharing the weight pass: one layer's four GEMMs at
    R = 12 decode rows + P prompt rows through the row-tiled kernel
    (qgemm_run_prefill), per matrix and per layer: time, useful TFLOP/s against
    the fp16 dense matrix-core peak, and weight GB/s; next to the layer at the
    12 decode rows alone on the streaming kernel."""
    import numpy as np
    import torch
    import synth
    from synth import workloads as W
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import roofline as RF
    dev = torch.device("cuda:0")
    Rs = [12 + c for c in chunks]
    R_max = max(Rs)
    mats = W.layer_mats(0)
    per = []
    for m in mats:
        canon = np.concatenate([synth.matrix_rows(seed, mid, n, m.K) for mid, n in zip(m.mids, m.splits)])
        cd = torch.from_numpy(canon).to(dev)
        pk = torch.empty(wsg.packed_size(m.N, m.K), dtype=torch.uint8, device=dev)
        wsg.pack(cd, pk, m.N, m.K)
        torch.cuda.synchronize()
        del cd
        pks = [pk] + [pk.clone() for _ in range(copies - 1)]
        gs = [wsg.QGemm(q, m.N, m.K, max_R=12) for q in pks]
        x = torch.from_numpy(synth.x_bf16(seed, W.X_STREAM[m.K], R_max, m.K).view(np.int16)).to(dev)
        y = torch.empty((R_max, m.N), dtype=torch.float32, device=dev)
        # one K-chunk workspace per matrix, sized for the largest need over the row counts
        ws = torch.empty(max(16, max(gs[0].prefill_workspace_size(R) for R in Rs)), dtype=torch.uint8, device=dev)
        per.append((m, pks, gs, x, (y, ws)))
    layer_bytes = sum(m.packed_bytes for m in mats)
    calls = [lambda g=gs[c], x=x, y=y: g.run(x[:12], y[0][:12], 12) for c in range(copies) for m, pks, gs, x, y in per]
    base_us = graph_ms(calls) / copies * 1e3
    log(f"[prefill] decode rows alone (R=12, streaming kernel): {base_us:.1f} us per layer")
    out = {}
    for P, R in zip(chunks, Rs):
        rec = {}
        for m, pks, gs, x, y in per:
            us = graph_ms([lambda g=g, x=x, y=y: g.run_prefill(x[:R], y[0][:R], R, workspace=y[1])
                           for g in gs]) / copies * 1e3
            tf = 2 * R * m.N * m.K / us / 1e6
            rec[m.name] = {"us": round(us, 2), "useful_tflop_s": round(tf, 1),
                           "pct_fp16_mfma_peak": round(tf / RF.MFMA_F16_DENSE_TFLOPS * 100, 1),
                           "weight_GB_s": round(m.packed_bytes / us / 1e3, 1)}
        calls = [lambda g=gs[c], x=x, y=y: g.run_prefill(x[:R], y[0][:R], R, workspace=y[1])
                 for c in range(copies) for m, pks, gs, x, y in per]
        us = graph_ms(calls) / copies * 1e3
        flops = sum(2 * R * m.N * m.K for m in mats)
        rec["layer"] = {"us": round(us, 2), "useful_tflop_s": round(flops / us / 1e6, 1),
                        "pct_fp16_mfma_peak": round(flops / us / 1e6 / RF.MFMA_F16_DENSE_TFLOPS * 100, 1),
                        "weight_GB_s": round(layer_bytes / us / 1e3, 1),
                        "prompt_rows_per_s_per_layer_pass": round(P / us * 1e6, 1)}
        out[str(P)] = rec
        log(f"[prefill] P={P:5d} (R={R}): " + ", ".join(f"{k} {v['us']:.1f} us {v['useful_tflop_s']:.0f} TF/s"
                                                      for k, v in rec.items()))
    for m, pks, gs, x, y in per:
        for g in gs:
            g.close()
    return {"seed": seed, "copies": copies, "decode_rows": 12, "layer_packed_bytes": layer_bytes,
            "decode_only_us_per_layer": round(base_us, 2), "by_prompt_rows": out}


def ragged_report(seed: int, steps: int):
    """The full pass under a seeded schedule of active agents: step t runs R_t =
    3 * a_t rows (a_t uniform in 1..4), with fresh activations per step (1 % of
    them scaled by 50).  Each step is one persistent launch of the 257 GEMMs
    and the head's argmax (one descriptor table per row count, uploaded before
    timing); the timed events bracket the pass only, not the copy of the step's
    activations."""
    import numpy as np
    import torch
    import synth
    from synth import workloads as W
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import roofline as RF
    sched = W.ragged_schedule(seed, steps)
    mats, gemms, packed, _, ys, idx = build_pass(max(sched), seed)
    dev = torch.device("cuda:0")
    # every step's activations, resident; before its pass a step's are copied
    # into the fixed input buffers of its row count (outside the timed events),
    # so that the sequence replays one graph per row count
    xs_t = [{w: torch.from_numpy(synth.x_bf16(seed, 1000 * (t + 1) + sid, R, w, outlier_p=0.01).view(np.int16))
             .to(dev) for w, sid in W.X_STREAM.items()} for t, R in enumerate(sched)]
    xbuf = {R: {w: torch.empty((R, w), dtype=torch.int16, device=dev) for w in W.X_STREAM} for R in set(sched)}
    seq = wsg.Seq(gemms, persistent=max(sched) <= 48)   # one cooperative launch per step (rows <= 48)

    def one_step(t, R, ev=None):
        for w in W.X_STREAM:
            xbuf[R][w].copy_(xs_t[t][w])
        if ev:
            ev[0].record()
        seq.run([xbuf[R][m.K] for m in mats], [y[:R] for y in ys], R, argmax_idx=idx)
        if ev:
            ev[1].record()

    for t, R in enumerate(sched):                                  # warm: one graph per row count
        one_step(t, R)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in sched]
    t0 = time.perf_counter()
    for t, R in enumerate(sched):
        one_step(t, R, ev[t])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    pass_bytes = W.pass_bytes()
    by_r = {str(R): round(float(ms[np.array(sched) == R].mean()), 4) for R in sorted(set(sched))}
    seq.close()
    for g in gemms:
        g.close()
    return {"seed": seed, "steps": steps, "rows_by_step": sched,
            "ms_per_step": {"mean": round(float(ms.mean()), 4), "median": round(float(np.median(ms)), 4),
                            "min": round(float(ms.min()), 4), "max": round(float(ms.max()), 4),
                            "p90": round(float(np.percentile(ms, 90)), 4)},
            "ms_per_step_by_R": by_r,
            "GB_s_mean": round(pass_bytes / ms.mean() / 1e6, 1),
            "pct_hbm_peak_mean": round(pass_bytes / ms.mean() / 1e6 / RF.HBM_PEAK_GBS * 100, 2),
            "rows_tok_per_s": round(sum(sched) / (ms.sum() / 1e3), 1),
            "wall_s": round(wall, 3)}


def attention_report(seed: int, reps: int = 20):
    """Decode attention of 4 agents x 3 step rows over about 23K cached positions
    each (a length mix), 64 query heads over 8 key/value heads of 128: time per
    step (split and combine kernels) over two rotating cache copies, the KV bytes
    it must read, and the fp64 oracle on one agent beside it."""
    import numpy as np
    import torch
    import weight_streaming_gemm_amd as wsg
    from oracle import attention as at
    from weight_streaming_gemm_amd import roofline as RF
    rng = np.random.default_rng(seed)
    lengths = [23000, 21877, 23549, 20001]
    A, rows, Hkv, d, cap = 4, 3, 8, 128, 23552
    max_len = cap - rows

    def bf(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)

    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(a.view(np.int16)).to(dev)  # noqa: E731
    q = bf((A, rows, 8 * Hkv, d))
    kv = [(t(bf((A, Hkv, cap, d))), t(bf((A, Hkv, cap, d)))) for _ in range(2)]     # head-major caches
    qd = t(q)
    ln = torch.tensor(lengths, dtype=torch.int32, device=dev)
    out = torch.empty((A, rows, 8 * Hkv, d), dtype=torch.float32, device=dev)
    ws = torch.empty(wsg.attention_workspace_size(A, rows, Hkv, max_len), dtype=torch.uint8, device=dev)
    for c in range(2):
        wsg.decode_attention(qd, kv[c][0], kv[c][1], ln, out, ws, max_len)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        wsg.decode_attention(qd, kv[r % 2][0], kv[r % 2][1], ln, out, ws, max_len)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    kv_bytes = sum((L + rows) * Hkv * d * 2 * 2 for L in lengths)
    # the oracle on agent 0 (a quarter of the work), all host cores via numpy
    # (the oracle takes [agent, position, head, dim])
    k0 = np.ascontiguousarray(kv[0][0][:1].cpu().numpy().view(np.uint16).transpose(0, 2, 1, 3))
    v0 = np.ascontiguousarray(kv[0][1][:1].cpu().numpy().view(np.uint16).transpose(0, 2, 1, 3))
    t0 = time.perf_counter()
    at.decode_attention(q[:1], k0, v0, lengths[:1])
    cpu_s = time.perf_counter() - t0
    cpu_bytes = (lengths[0] + rows) * Hkv * d * 2 * 2
    return {"agents": A, "rows_per_agent": rows, "q_heads": 8 * Hkv, "kv_heads": Hkv, "head_dim": d,
            "lengths": lengths, "us_per_step": round(us, 2), "kv_bytes": kv_bytes,
            "GB_s": round(kv_bytes / us / 1e3, 1), "pct_hbm_peak": round(kv_bytes / us / 1e3 / RF.HBM_PEAK_GBS * 100, 1),
            "cpu_baseline": {"value": round(cpu_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "kind": "oracle",
                             "sample": f"agent 0 ({lengths[0]} positions), fp64 numpy, {cpu_s:.2f}s"}}


# the sources the streaming kernel and its launches are built from (the decode
# attention and the row-tiled prompt kernel live in files of their own)
# the dominant kernel of each launch mode: (name prefix in traces, sources whose
# code the counters describe, summary file under profiles/)
KERNELS = {
    "pass": ("qg::pass_kernel<", ("layout.h", "operand.h", "pass.hip", "pass_sched.h", "qgemm_api.cpp",
                                  "qgemm_internal.h"), "pass_kernel_full_pass_R12.md"),
    "stream": ("qg::stream_kernel<1, 1, 8", ("layout.h", "operand.h", "qgemm_api.cpp", "qgemm_internal.h",
                                             "qgemm_kernels.hip", "stream_sched.h"), "stream_kernel_full_pass_R12.md"),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_digest(kind: str) -> str:
    """sha256 over a kernel's sources with comments and blank space removed:
    identifies the code a counter run measured (a comment edit does not make the
    counters stale; any code change does)."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "weight_streaming_gemm_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(KERNELS[kind][1]):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)      # the sources hold no "//" or "/*" in literals
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(kind: str, R: int):
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE runs, scaled by a copy kernel of known
    size), or None when the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kind)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("kernel_source_sha256") != kernel_source_digest(kind) or rec.get("R") != R:
        return None
    return rec.get("bytes_per_launch")


def _read_csv(path: str):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find_csv(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for name in files:
            if name.endswith(suffix):
                return os.path.join(root, name)
    raise FileNotFoundError(f"no *{suffix} under {d}")


INST_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_WAVES")


def summarize_profiles(kind: str, trace_dir: str, fetch_dir: str, write_dir: str, copy_mib: int, R: int,
                       commands: dict, inst_dir: str = None) -> dict:
    """Turn one kernel-trace run and two counter runs (FETCH_SIZE, WRITE_SIZE in KiB per
    dispatch) into a record for profiles/traffic.json and a markdown summary.  The
    counters are scaled so that the plain device copy of copy_mib MiB reads and writes
    exactly that many bytes; the dominant kernel's figures are averages over its
    dispatches.  With inst_dir, a run of INST_COUNTERS adds the instructions issued
    per weight step (16 outputs x 256 weights: 2304 packed bytes)."""
    prefix, _, summary = KERNELS[kind]
    stats = _read_csv(_find_csv(trace_dir, "kernel_stats.csv"))
    per = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for row in _read_csv(_find_csv(d, "counter_collection.csv")):
            if row["Counter_Name"] != name:
                continue
            k = per.setdefault(row["Kernel_Name"], {})
            k.setdefault(name, []).append(float(row["Counter_Value"]))
    copy_kib = copy_mib * 1024.0
    cp = per[COPY_KERNEL]
    # the copy runs three times; its largest dispatch is the full-size one
    scale = {c: copy_kib / max(cp[c]) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    fetch, write = [], []
    for kname, v in per.items():
        if prefix in kname:
            fetch += v.get("FETCH_SIZE", [])
            write += v.get("WRITE_SIZE", [])
    fetch_b = sum(fetch) / len(fetch) * 1024 * scale["FETCH_SIZE"]
    write_b = sum(write) / len(write) * 1024 * scale["WRITE_SIZE"]
    calls = tot_ns = 0.0
    for row in stats:
        if prefix in row["Name"]:
            calls += float(row["Calls"])
            tot_ns += float(row["TotalDurationNs"])
    avg_us = tot_ns / calls / 1e3
    launch_bytes = 17990737920 if kind == "pass" else 17990737920 / 257
    rec = {
        "kernel": {"pass": "pass_kernel (one launch per pass: all 257 GEMMs)",
                   "stream": "stream_kernel (all variants of the pass, one launch per GEMM)"}[kind],
        "R": R,
        "kernel_source_sha256": kernel_source_digest(kind),
        "digest": "sha256 of the kernel's csrc sources with comments and blank space removed "
                  "(bench.kernel_source_digest)",
        "fetch_bytes_per_launch": int(round(fetch_b)),
        "write_bytes_per_launch": int(round(write_b)),
        "bytes_per_launch": int(round(fetch_b + write_b)),
        "algorithmic_bytes_per_launch": int(round(launch_bytes)),
        "avg_launch_us_trace": round(avg_us, 3),
        "scale": {"FETCH_SIZE": round(scale["FETCH_SIZE"], 4), "WRITE_SIZE": round(scale["WRITE_SIZE"], 4),
                  "from": f"{COPY_KERNEL} of {copy_mib} MiB"},
        "summary": f"profiles/{summary}",
    }
    title = {"pass": f"Pass kernel (one cooperative launch per 257-GEMM weight pass) at R = {R}",
             "stream": f"Streaming kernel over the full 257-GEMM weight pass at R = {R}"}[kind]
    lines = [f"# {title}", "",
             "Kernel-trace summary (`rocprofv3 --kernel-trace --stats`, run from the repository root with TMPDIR=/tmp):", "",
             "```", commands["trace"], "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for row in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{row['Name'][:90]}` | {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | "
                     f"{float(row['MinNs']) / 1e3:.2f} | {float(row['MaxNs']) / 1e3:.2f} | "
                     f"{float(row['Percentage']):.1f} % |")
    lines += ["", "Hardware counters, one `--pmc` pass per counter (KiB per dispatch, averaged over the "
              "dispatches of each kernel):", "", "```", commands["fetch"], commands["write"], "```", "",
              "| kernel | dispatches | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |", "|---|---|---|---|"]
    for kname, v in sorted(per.items()):
        f_ = v.get("FETCH_SIZE", [0.0])
        w_ = v.get("WRITE_SIZE", [0.0])
        lines.append(f"| `{kname[:90]}` | {len(f_)} | {sum(f_) / len(f_):.1f} | {sum(w_) / len(w_):.1f} |")
    lines += ["", "Reading the numbers (MI355X, one GPU):", "",
              f"- The {kind} kernel averages {avg_us:.2f} us per launch over {int(calls)} launches in the trace; "
              f"a launch moves {launch_bytes / 1e6:.1f} MB of packed weights, i.e. {launch_bytes / avg_us / 1e3:.0f} "
              f"GB/s ({launch_bytes / avg_us / 1e3 / 80:.1f} % of 8 TB/s).",
              f"- Counter scale from the {copy_mib} MiB device copy ({COPY_KERNEL}): FETCH_SIZE x "
              f"{scale['FETCH_SIZE']:.3f}, WRITE_SIZE x {scale['WRITE_SIZE']:.3f}.",
              f"- Scaled, per launch on average: {fetch_b / 1e6:.1f} MB fetched "
              f"({fetch_b / launch_bytes:.3f}x the algorithmic weight bytes; the rest is activations and partial "
              f"tiles), {write_b / 1e6:.2f} MB written (outputs and partial tiles).", ""]
    for row in stats:
        if "read_probe_kernel" in row["Name"]:
            nb = 4 << 30
            rec["read_probe"] = {"bytes": nb, "avg_us_trace": round(float(row["AverageNs"]) / 1e3, 2),
                                 "min_us_trace": round(float(row["MinNs"]) / 1e3, 2)}
            lines[-1:-1] = [f"- Practical read ceiling: the plain read kernel (`read_probe_kernel`, the bench's "
                            f"`roofline.practical_peak`) reads {nb} B in {float(row['AverageNs']) / 1e3:.1f} us on "
                            f"average over {row['Calls']} calls ({nb / float(row['AverageNs']):.0f} GB/s; "
                            f"{nb / float(row['MinNs']):.0f} GB/s at its fastest), against 8000 GB/s on paper."]
    if inst_dir:
        inst = {}
        for row in _read_csv(_find_csv(inst_dir, "counter_collection.csv")):
            if prefix in row["Kernel_Name"] and row["Counter_Name"] in INST_COUNTERS:
                inst.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
        steps = launch_bytes / 2304
        per_step = {c: round(sum(v) / len(v) / steps, 2) for c, v in inst.items() if c != "SQ_WAVES"}
        rec["instructions_per_weight_step"] = per_step
        lines += ["Instructions issued per weight step (wave instructions of all waves, the counters summed over "
                  "the device per dispatch and averaged over the dispatches, divided by the "
                  f"{steps:.0f} steps of a launch; SQ_INSTS_VALU counts the matrix-core instructions too):",
                  "", "```", commands["inst"], "```", "",
                  "| counter | per launch | per weight step |", "|---|---|---|"]
        for c in INST_COUNTERS:
            if c in inst:
                v = sum(inst[c]) / len(inst[c])
                lines.append(f"| {c} | {v:.4g} | {'-' if c == 'SQ_WAVES' else f'{v / steps:.1f}'} |")
        lines.append("")
    rec["summary_text"] = "\n".join(lines)
    return rec


def cpu_baseline(seed: int):
    """The fp64 oracle as it stands on the host cores, on a bounded sample set.
    All cores: the single matrix (256 x 1024) at R in 1, 3, 12, 24, 48; layer 0's
    four GEMMs whole at R in 1, 3, 12 and cut to the first eighth of each
    matrix's outputs at R in 24, 48; the output head's first eighth at R = 12.
    One thread: the single matrix at every R and the first 1/64 of layer 0's
    outputs per matrix at R = 12.  Cut samples are scaled to whole matrices by
    bytes (the oracle's time is linear in the outputs) and labelled so; the full
    pass at R = 12 is extrapolated (64 x layer 0 + the head); `value` is that
    extrapolated all-core rate."""
    import numpy as np
    import synth
    import oracle
    from synth import workloads as W
    o = oracle.get()
    threads = len(os.sched_getaffinity(0))
    Rs = (1, 3, 12, 24, 48)
    t_start = time.perf_counter()

    def timed(canon, N, K, x, th, frac=1):
        rows = N if frac == 1 else max(1, N // frac)
        t0 = time.perf_counter()
        o.gemm(canon[:rows * (K // 256) * 144], rows, K, x, threads=th)
        return time.perf_counter() - t0, rows * (K // 256) * 144

    def entry(t, nbytes, whole_bytes):
        e = {"s": round(t, 5), "sample_bytes": nbytes, "GB_s": round(nbytes / t / 1e9, 5)}
        if nbytes != whole_bytes:
            e["whole_s_scaled"] = round(t * whole_bytes / nbytes, 3)
        return e

    sm = W.SMALL
    one = W.Mat("single", sm["N"], sm["K"], (sm["mid"],), (sm["N"],))
    c0 = synth.matrix_rows(sm["seed"], sm["mid"], one.N, one.K)
    x0 = synth.x_bf16(sm["seed"], 0, max(Rs), one.K)
    layer = [(m, np.concatenate([synth.matrix_rows(seed, mid, n, m.K) for mid, n in zip(m.mids, m.splits)]),
              synth.x_bf16(seed, W.X_STREAM[m.K], max(Rs), m.K)) for m in W.layer_mats(0)]
    layer_bytes = sum(m.packed_bytes for m, _, _ in layer)
    rec = {"all_cores": {}, "one_thread": {}}
    for R in Rs:
        rec["all_cores"][f"single_matrix_R{R}"] = entry(*timed(c0, one.N, one.K, x0[:R], threads), one.packed_bytes)
        rec["one_thread"][f"single_matrix_R{R}"] = entry(*timed(c0, one.N, one.K, x0[:R], 1), one.packed_bytes)

    def layer_run(R, th, frac):
        t = nb = 0
        for m, c, x in layer:
            dt, b = timed(c, m.N, m.K, x[:R], th, frac)
            t += dt
            nb += b
        return t, nb

    for R in Rs:
        frac = 1 if R <= 12 else 8
        rec["all_cores"][f"layer0_R{R}" + ("" if frac == 1 else "_first_eighth")] = entry(*layer_run(R, threads, frac),
                                                                                        layer_bytes)
    head = W.lm_head()
    ch = np.concatenate([synth.matrix_rows(seed, mid, n, head.K) for mid, n in zip(head.mids, head.splits)])
    xh = synth.x_bf16(seed, W.X_STREAM[head.K], 12, head.K)
    th_, hb = timed(ch, head.N, head.K, xh, threads, 8)
    rec["all_cores"]["head_R12_first_eighth"] = entry(th_, hb, head.packed_bytes)
    t1, b1 = layer_run(12, 1, 64)
    rec["one_thread"]["layer0_R12_first_64th"] = entry(t1, b1, layer_bytes)
    t_layer = rec["all_cores"]["layer0_R12"]["s"]
    t_head = th_ * head.packed_bytes / hb
    full_s = 64 * t_layer + t_head
    full_1t = (64 * layer_bytes + head.packed_bytes) / (b1 / t1)
    rec["full_pass_R12_extrapolated"] = {
        "all_cores_s": round(full_s, 2), "all_cores_GB_s": round(W.pass_bytes() / full_s / 1e9, 5),
        "one_thread_s": round(full_1t, 1), "one_thread_GB_s": round(W.pass_bytes() / full_1t / 1e9, 5),
        "how": "all cores: 64 x layer 0 at R=12 + the head at R=12 scaled from its first eighth; one thread: "
               "the first-64th sample of layer 0 at R=12, scaled by bytes"}
    spent = time.perf_counter() - t_start
    return {"value": round(W.pass_bytes() / full_s / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 dequantize-then-dot on {threads} threads: single matrix 256x1024 at R in 1,3,12,24,48; "
                      f"layer 0 (Q|K|V, O, gate|up, down) whole at R in 1,3,12 and its first eighth at R in 24,48; "
                      f"the head's first eighth at R=12; one thread: single matrix at every R and layer 0's first "
                      f"64th at R=12. value = full pass at R=12 extrapolated from layer 0 and the head "
                      f"({spent:.1f}s of CPU work in all)",
            "detail": rec}


def read_ceiling(nbytes: int = 4 << 30, reps: int = 5):
    """The practical HBM read ceiling: the library's plain read kernel over a
    buffer far larger than the caches, best of `reps` (GB/s, ms)."""
    import torch
    import weight_streaming_gemm_amd as wsg
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.empty(16384, dtype=torch.uint8, device="cuda")
    wsg.read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    best = 1e9
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        wsg.read_probe(buf, nbytes, sink)
        e1.record(st)
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del buf, sink
    return nbytes / best / 1e6, best


def time_pass_kernel(seq, xs, ys, R: int, reps: int):
    """Average duration of the persistent pass kernel (seq.run without the argmax
    enqueues exactly one kernel: all 257 GEMMs), with HIP events on the stream it
    runs on."""
    import torch
    xr = [x[:R] for x in xs]
    yr = [y[:R] for y in ys]
    seq.run(xr, yr, R)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        seq.run(xr, yr, R)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps, reps


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--R", type=int, default=12)
    ap.add_argument("--sweep", default="1,3,12,24,48",
                    help="extra row counts timed over the full pass (flatness; 24 and 48 rows = 8 and 16 agents)")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch", choices=["auto", "persistent", "graph"], default="auto",
                    help="how a pass is launched: one cooperative launch of the pass kernel (persistent, up to "
                         "48 rows), a replayed graph of one streaming-kernel launch per GEMM (graph), or the "
                         "persistent launch where it serves the row count and the graph elsewhere (auto)")
    ap.add_argument("--persistent", action="store_true", help="same as --launch persistent")
    ap.add_argument("--kernel-only", action="store_true",
                    help="skip the timed passes: only the dominant kernel's launches at --R (the pass kernel, "
                         "or the streaming kernels with --launch graph) and the copy calibration, for "
                         "hardware-counter runs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain device-to-device copy of MIB MiB three times: a kernel of known "
                         "traffic for scaling the HBM byte counters of a profiler run")
    ap.add_argument("--rows", default="",
                    help="with --report layer: only these row counts (comma-separated), e.g. for counter runs")
    ap.add_argument("--no-paths", action="store_true",
                    help="skip timing the pass on each kernel path for R = 1..4 (for profiler runs of one R)")
    ap.add_argument("--report", choices=["layer", "ragged", "attention", "prefill"],
                    help="instead of the pass: 'layer' = one layer's GEMMs per matrix and R on both kernel paths "
                         "(plain weights, seed 1, R in 1,2,3,4,12,24,48; then edge-block weights, seed 4, R in "
                         "24,48); 'ragged' = 100 passes under the seeded 1..4-agent schedule (seed 3); "
                         "'attention' = decode attention of 4 agents x 3 rows over ~23K cached positions; "
                         "'prefill' = one layer at 12 decode rows + a prompt chunk of 64..2048 rows on the "
                         "row-tiled kernel")
    ap.add_argument("--summarize-profiles", nargs="+", metavar="DIR",
                    help="no GPU work: TRACE_DIR FETCH_DIR WRITE_DIR [INST_DIR]: read the rocprofv3 CSVs of a "
                         "kernel-trace run, of the FETCH_SIZE and WRITE_SIZE counter runs (each made with "
                         "--copy-calibration, size given by that flag) and optionally of a run of the "
                         "instruction counters, and rewrite profiles/traffic.json and the dominant kernel's "
                         "summary under profiles/")
    args = ap.parse_args()

    if args.persistent:
        args.launch = "persistent"
    kind = "stream" if args.launch == "graph" else "pass"

    if args.summarize_profiles:
        lf = f"--launch {args.launch}"
        cmds = {
            "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace -o bench -- "
                     f"python3 bench.py {lf} --steps 5 --warmup 1 --no-cpu-baseline --sweep 12 --no-paths",
            "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fetch -o bench -- "
                     f"python3 bench.py {lf} --kernel-only --no-cpu-baseline --sweep 12 "
                     f"--copy-calibration {args.copy_calibration}",
            "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_write -o bench -- "
                     f"python3 bench.py {lf} --kernel-only --no-cpu-baseline --sweep 12 "
                     f"--copy-calibration {args.copy_calibration}",
            "inst": f"rocprofv3 --pmc {' '.join(INST_COUNTERS)} --output-format csv -d gpurun_out/prof_inst -o bench -- "
                    f"python3 bench.py {lf} --kernel-only --no-cpu-baseline --sweep 12",
        }
        dirs = args.summarize_profiles
        if len(dirs) not in (3, 4):
            ap.error("--summarize-profiles takes TRACE_DIR FETCH_DIR WRITE_DIR [INST_DIR]")
        rec = summarize_profiles(kind, *dirs[:3], args.copy_calibration or 1024, args.R, cmds,
                                 inst_dir=dirs[3] if len(dirs) == 4 else None)
        text = rec.pop("summary_text")
        with open(os.path.join(ROOT, "profiles", KERNELS[kind][2]), "w") as f:
            f.write(text)
        path = os.path.join(ROOT, "profiles", "traffic.json")
        try:
            with open(path) as f:
                allrec = json.load(f)
            if "kernel_source_sha256" in allrec:           # a record of the older single-kernel form
                allrec = {}
        except (OSError, ValueError):
            allrec = {}
        allrec[kind] = rec
        with open(path, "w") as f:
            json.dump(allrec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the weight pass runs on a single GPU and is not sharded "
              "across GPUs; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import weight_streaming_gemm_amd as wsg
    from weight_streaming_gemm_amd import roofline as RF
    from synth import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.report == "layer":
        only = {int(v) for v in args.rows.split(",") if v}
        plain = [r for r in (1, 2, 3, 4, 12, 24, 48) if not only or r in only]
        edge = [r for r in (24, 48) if not only or r in only]
        rep = {"report": "layer", "unit": "us per GEMM (graph replay over rotating weight copies)",
               "layer": layer_report(W.SEED_LAYER, 0, plain, copies=6) if plain else None,
               "large_R_edge_blocks": layer_report(W.SEED_LARGE_R, 2, edge, copies=6) if edge else None}
        print(json.dumps(rep), flush=True)
        return
    if args.report == "prefill":
        rep = prefill_report(1, [64, 128, 256, 512, 1024, 2048])
        print(json.dumps({"report": "prefill", **rep}))
        return
    if args.report == "attention":
        rep = attention_report(args.seed)
        log(f"[attention] {rep['us_per_step']:.1f} us per step, {rep['GB_s']:.0f} GB/s of KV "
            f"({rep['pct_hbm_peak']:.1f} % of 8 TB/s)")
        print(json.dumps({"report": "attention", **rep}), flush=True)
        return
    if args.report == "ragged":
        print(json.dumps({"report": "ragged", **ragged_report(W.SEED_RAGGED, 100)}), flush=True)
        return
    sweep = sorted({int(v) for v in args.sweep.split(",") if v} | {args.R})
    P_MAX = 48                                   # rows the persistent pass kernel serves (three row tiles)
    if args.launch == "persistent" and max(sweep) > P_MAX:
        sweep = [r for r in sweep if r <= P_MAX]
        log(f"[pass] persistent launch: row counts {sweep}")

    def mode_of(R):
        return "persistent" if args.launch != "graph" and R <= P_MAX else "graph"

    R_max = max(sweep)
    mats, gemms, packed, xs, ys, idx = build_pass(R_max, args.seed)
    seqs = {"graph": wsg.Seq(gemms)}
    if any(mode_of(R) == "persistent" for R in sweep) or args.R <= P_MAX:
        seqs["persistent"] = wsg.Seq(gemms, persistent=True)
    pass_bytes = W.pass_bytes()
    if args.copy_calibration > 0:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[calib] copied {nb} bytes three times")
        del src, dst

    head_mode = mode_of(args.R)
    if args.kernel_only:
        if head_mode == "persistent":
            kern_ms, launches = time_pass_kernel(seqs["persistent"], xs, ys, args.R, reps=2)
            per_launch = pass_bytes
        else:
            kern_ms, launches = time_dominant_kernel(gemms, xs, ys, args.R, reps=1)
            per_launch = pass_bytes / len(gemms)
        log(f"[kernel] {launches} launches, {kern_ms * 1e3:.2f} us average")
        print(json.dumps({"kernel_only": True, "R": args.R, "launch": head_mode,
                          "avg_launch_us": round(kern_ms * 1e3, 3), "bytes_per_launch": round(per_launch)}),
              flush=True)
        return
    results, modes = {}, {}
    for R in sweep:
        modes[R] = mode_of(R)
        ms, wall = time_pass(seqs[modes[R]], xs, ys, idx, R, args.steps if R == args.R else max(5, args.steps // 2),
                             args.warmup)
        results[R] = ms
        log(f"[pass] R={R:3d} ({modes[R]}): {ms:.4f} ms/pass, {pass_bytes / ms / 1e6:.1f} GB/s "
            f"({pass_bytes / ms / 1e6 / RF.HBM_PEAK_GBS * 100:.1f}% of 8 TB/s), "
            f"{R * 1000 / ms:.0f} rows*tok/s")
    ms = results[args.R]
    gbs = pass_bytes / ms / 1e6
    # both launch modes at the headline row count
    by_mode = {head_mode: round(ms, 5)}
    for other in ("graph", "persistent"):
        if other != head_mode and other in seqs:
            o_ms, _ = time_pass(seqs[other], xs, ys, idx, args.R, max(5, args.steps // 2), args.warmup)
            by_mode[other] = round(o_ms, 5)
            log(f"[pass] R={args.R} ({other}): {o_ms:.4f} ms/pass")
    # both dependency models of the persistent launch: every GEMM after the whole
    # previous one (the headline), and down projections waiting only for the
    # gate|up outputs they read
    by_dep = None
    if "persistent" in seqs and args.R <= P_MAX:
        gated = wsg.Seq(gemms, persistent=True, gated_inputs=True)
        g_ms, _ = time_pass(gated, xs, ys, idx, args.R, max(5, args.steps // 2), args.warmup)
        gated.close()
        by_dep = {"after_whole_previous_gemm": by_mode["persistent"], "gated_mlp_inputs": round(g_ms, 5)}
        log(f"[pass] R={args.R} (persistent, gated inputs of the down projections): {g_ms:.4f} ms/pass")

    if head_mode == "persistent":
        kern_ms, launches = time_pass_kernel(seqs["persistent"], xs, ys, args.R, reps=10)
        bytes_per_launch = pass_bytes
        kname = "pass_kernel<8, false> (one cooperative launch per pass: all 257 GEMMs)"
    else:
        kern_ms, launches = time_dominant_kernel(gemms, xs, ys, args.R, reps=3)
        bytes_per_launch = pass_bytes / len(gemms)
        info = gemms[0].query(args.R)
        kname = (f"stream_kernel<{info['row_tiles']}, {info['subtiles_per_wave']}, {info['waves_per_workgroup']}, "
                 f"*, 0> (both min-term variants, all 257 GEMMs)")
    achieved = bytes_per_launch / (kern_ms * 1e-3) / 1e9
    log(f"[kernel] {kname}: {kern_ms * 1e3:.2f} us average over {launches} launches, "
        f"{bytes_per_launch / 1e6:.2f} MB/launch, {achieved:.1f} GB/s")
    ceiling, ceiling_ms = read_ceiling()
    log(f"[ceiling] plain read kernel: {ceiling:.1f} GB/s ({ceiling / RF.HBM_PEAK_GBS * 100:.1f}% of 8 TB/s)")

    paths = None if args.no_paths else time_paths(gemms, xs, ys, [r for r in (1, 2, 3, 4) if r <= R_max])
    for R, rec in (paths or {}).items():
        log(f"[paths] R={R}: vector-unit {rec['valu_ms']:.4f} ms/pass, matrix-core {rec['mfma_ms']:.4f} "
            f"ms/pass, automatic choice {rec['auto']}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.seed)
        log(f"[cpu] oracle {cpu['value']:.4f} GB/s on {cpu['cores']} threads ({cpu['sample']})")

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q4k->f16 mfma, f32 acc",
        "data": "synthetic",
        "config": {
            "workload": "full decode-step weight pass: 64 layers (hidden 5120, q 8192, kv 2x1024, "
                        "mlp 2x25600 / 25600) + lm-head 5120->151936, Q4_K-style 4.5 bit, "
                        "257 GEMMs + row argmax",
            "R": args.R,
            "pass_launch": head_mode,
            "pass_launch_by_R": {str(k): v for k, v in modes.items()},
            "ms_per_pass_by_launch": by_mode,
            "dependency_model": "each GEMM starts after the previous one has finished everywhere",
            "persistent_ms_per_pass_by_dependency_model": by_dep,
            "step_epilogue": "head row argmax (chunked) + greedy check of 2 drafts per agent",
            "packed_bytes": pass_bytes,
            "pct_hbm_peak": round(gbs / RF.HBM_PEAK_GBS * 100, 2),
            "rows_tok_per_s": round(args.R * 1000 / ms, 1),
            "ms_per_pass_by_R": {str(k): round(v, 5) for k, v in results.items()},
            "GB_s_by_R": {str(k): round(pass_bytes / v / 1e6, 1) for k, v in results.items()},
            "pct_hbm_peak_by_R": {str(k): round(pass_bytes / v / 1e6 / RF.HBM_PEAK_GBS * 100, 2)
                                  for k, v in results.items()},
            "rows_tok_per_s_by_R": {str(k): round(k * 1000 / v, 1) for k, v in results.items()},
            "row_tiled_gemms_by_R": {str(k): (sum(1 for g in gemms if g.query(k)["path"] == wsg.PATH_TILED)
                                              if modes[k] == "graph" else 0) for k in results},
            "flatness_t12_over_t1": round(results[12] / results[1], 4) if 1 in results and 12 in results else None,
            "kernel_paths_ms_per_pass_by_R": paths,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kname,
            "achieved": round(achieved, 1),
            "peak": RF.HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / RF.HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(kind if head_mode == "persistent" else "stream", args.R),
            "avg_launch_us": round(kern_ms * 1e3, 3),
            "bytes_per_launch": round(bytes_per_launch),
            "practical_peak": round(ceiling, 1),
            "practical_peak_kernel": "read_probe_kernel: 4 GiB, one 512-thread workgroup per CU, 16-byte "
                                     "nontemporal loads, best of 5",
            "frac_of_practical_peak": round(achieved / ceiling, 4),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    for sq in seqs.values():
        sq.close()
    for g in gemms:
        g.close()


if __name__ == "__main__":
    main()
