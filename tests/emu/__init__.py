"""Builds and loads the CPU emulation of the kernels' data flow (test-only)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libqgemm_emu.so")
CLANG = "/opt/rocm/llvm/bin/clang++"


def build(force: bool = False) -> str:
    if os.environ.get("QG_EMU_LIB"):                    # a prebuilt (instrumented) copy: load it as is
        return os.environ["QG_EMU_LIB"]
    src = os.path.join(HERE, "qgemm_emu.cpp")
    deps = [src] + [os.path.join(HERE, "..", "..", "weight_streaming_gemm_amd", "csrc", f)
                    for f in ("layout.h", "operand.h", "stream_sched.h", "prefill_plan.h", "pass_sched.h")]
    if force or not os.path.exists(LIB) or any(os.path.getmtime(d) > os.path.getmtime(LIB) for d in deps):
        tmp = LIB + ".tmp"
        subprocess.check_call([CLANG, "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
                               src, "-o", tmp])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        L.emu_stream_seq.restype = ctypes.c_int
        L.emu_stream_seq.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_uint64]
        L.emu_stream.restype = ctypes.c_int
        L.emu_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p]
        L.emu_dequant.restype = ctypes.c_int
        L.emu_dequant.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.emu_pack.restype = ctypes.c_int
        L.emu_pack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        L.emu_prefill_plan.restype = ctypes.c_int
        L.emu_prefill_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.emu_pass_coverage.restype = ctypes.c_int
        L.emu_pass_coverage.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        L.emu_pass.restype = ctypes.c_int
        L.emu_pass.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int]
        L.emu_pass_block_bytes.restype = ctypes.c_int
        L.emu_pass_block_bytes.argtypes = [ctypes.c_int]
        L.emu_pass_wave_first.restype = ctypes.c_int
        L.emu_pass_wave_first.argtypes = [ctypes.c_int] * 3
        L.emu_pass_step_owner.restype = ctypes.c_int
        L.emu_pass_step_owner.argtypes = [ctypes.c_int] * 3
        L.emu_pass_units.restype = None
        L.emu_pass_units.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p]
        L.emu_pass_gated_mask.restype = None
        L.emu_pass_gated_mask.argtypes = [ctypes.c_int] * 7 + [ctypes.c_void_p]
        L.emu_prefill.restype = ctypes.c_int
        L.emu_prefill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
        _lib = L
    return _lib


PLAN_FIELDS = ("wm", "wn", "mt", "nt", "S", "kc", "img_bytes", "ws_bytes", "rtw")


def prefill_plan(N, K, R, cus=256):
    out = np.zeros(9, np.int64)
    lib().emu_prefill_plan(N, K, R, cus, out.ctypes.data)
    return dict(zip(PLAN_FIELDS, (int(v) for v in out)))


def prefill(canon, N, K, x_bits, cus=256):
    R = x_bits.shape[0]
    y = np.zeros((R, N), np.float32)
    xb = np.ascontiguousarray(x_bits.view(np.uint16))
    lib().emu_prefill(np.ascontiguousarray(canon).ctypes.data, N, K, xb.ctypes.data, R, cus, y.ctypes.data)
    return y


def stream(canon, N, K, x_bits, NT=2, NW=4, V=8, order_seed=0, nwn=1, aligned=0, msum=1, chunks=1):
    """One GEMM through the emulated streaming kernel (NW waves in an nwn x NW/nwn
    grid, NT sub-tiles per wave, V ranges: equal step ranges, or whole-tile ranges
    when aligned; min term from sub-block sums when msum; K in `chunks` chunks)."""
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R = x_bits.shape[0]
    y = np.empty((R, N), dtype=np.float32)
    rc = lib().emu_stream(canon.ctypes.data, N, K, x_bits.ctypes.data, R, NT, NW, nwn, V, aligned,
                             msum, chunks, order_seed, y.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"emu_stream failed ({rc})")
    return y


def stream_seq(mats, xs, NT=2, NW=4, Vs=None, order_seed=0, nwns=None, aligned=None, msums=None, chunks=None):
    """Several GEMMs in one emulated launch; mats = [(canon, N, K)], xs = [bf16 bits (R x K)]."""
    G = len(mats)
    canons = [np.ascontiguousarray(c, dtype=np.uint8) for c, _, _ in mats]
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in xs]
    R = xs[0].shape[0]
    ys = [np.empty((R, N), dtype=np.float32) for _, N, _ in mats]
    P_ = ctypes.c_void_p * G
    Ns = np.array([N for _, N, _ in mats], dtype=np.int64)
    Ks = np.array([K for _, _, K in mats], dtype=np.int64)
    Vs = np.array(Vs if Vs is not None else [8] * G, dtype=np.int64)
    nwns = np.array(nwns if nwns is not None else [1] * G, dtype=np.int32)
    aligned = np.array(aligned if aligned is not None else [0] * G, dtype=np.int32)
    msums = np.array(msums if msums is not None else [1] * G, dtype=np.int32)
    chunks = np.array(chunks if chunks is not None else [1] * G, dtype=np.int32)
    rc = lib().emu_stream_seq(G, P_(*[c.ctypes.data for c in canons]), Ns.ctypes.data, Ks.ctypes.data,
                              P_(*[x.ctypes.data for x in xs]), P_(*[y.ctypes.data for y in ys]), R, NT, NW,
                              nwns.ctypes.data, Vs.ctypes.data, aligned.ctypes.data, msums.ctypes.data,
                              chunks.ctypes.data, order_seed)
    if rc != 0:
        raise RuntimeError(f"emu_stream_seq failed ({rc})")
    return ys


# the persistent pass kernel's constants (qgemm_internal.h): compute waves per
# workgroup, piece slots per wave, most K chunks, most rows; LDS bytes for
# activations at R rows (row tiles of 16)
PASS_NC = 8
PASS_PIECES = 2
PASS_MAX_CHUNKS = 32
PASS_MAX_R = 48


def pass_max_chunks(R):
    """Most K chunks of a GEMM at R rows (16 at one row tile: one round of loads)."""
    return 16 if R <= 16 else PASS_MAX_CHUNKS


def pass_pieces(R):
    """Piece slots per compute wave at R rows (one from two row tiles on)."""
    return PASS_PIECES if R <= 16 else 1


def pass_x_area(R):
    return 160 * 1024 - PASS_NC * pass_pieces(R) * ((R + 15) // 16) * 1024 - 256


PASS_X_AREA = pass_x_area(16)


def pass_coverage(shapes, R, P=256, x_area=None, max_chunks=None):
    """(per-GEMM step hit counts [NS * KB], chunks) of the pass kernel's schedule
    (x_area: the kernel's LDS area at R rows unless given)."""
    x_area = pass_x_area(R) if x_area is None else x_area
    max_chunks = pass_max_chunks(R) if max_chunks is None else max_chunks
    G = len(shapes)
    Ns = np.array([N for N, _ in shapes], np.int64)
    Ks = np.array([K for _, K in shapes], np.int64)
    sizes = [((N + 15) // 16) * (K // 256) for N, K in shapes]
    counts = np.zeros(sum(sizes), np.int32)
    chunks = np.zeros(G, np.int32)
    rc = lib().emu_pass_coverage(G, Ns.ctypes.data, Ks.ctypes.data, R, P, PASS_NC, x_area, max_chunks,
                                 counts.ctypes.data, chunks.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"emu_pass_coverage failed ({rc})")
    out, o = [], 0
    for n in sizes:
        out.append(counts[o:o + n])
        o += n
    return out, chunks


def pass_units(p, S, P, NS, rot):
    """(chunk, ns0, ns1) of workgroup p in the pass kernel's deal."""
    out = np.zeros(3, np.int32)
    lib().emu_pass_units(p, S, P, NS, rot, out.ctypes.data)
    return tuple(int(v) for v in out)


def pass_gated_mask(c, kbc, half, P, NSp, Sp, rot_p):
    """The set of workgroups chunk c of a gated GEMM waits for."""
    w = np.zeros(4, np.uint64)
    lib().emu_pass_gated_mask(c, kbc, half, P, NSp, Sp, rot_p, w.ctypes.data)
    return {q for q in range(256) if (int(w[q // 64]) >> (q % 64)) & 1}


def pass_wave_first(w, NC, n):
    """First step of compute wave w's sub-range when a workgroup's n steps are split over NC waves."""
    return lib().emu_pass_wave_first(w, NC, n)


def pass_step_owner(i, NC, n):
    """The compute wave whose sub-range holds step i."""
    return lib().emu_pass_step_owner(i, NC, n)


def pass_block_bytes(R):
    """LDS bytes of one block's activations in the pass kernel at R rows."""
    return lib().emu_pass_block_bytes(R)


def pass_run(mats, xs, P, x_area=None, max_chunks=None, msum=False):
    """The pass kernel replayed over GEMMs mats = [(canon, N, K)] with activations
    xs (bf16 bits, R x K each), the min term from sub-block sums (msum, and
    always beyond 16 rows, as in the kernel) or from products with the mins: the
    list of y."""
    G = len(mats)
    canons = [np.ascontiguousarray(c, dtype=np.uint8) for c, _, _ in mats]
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in xs]
    R = xs[0].shape[0]
    x_area = pass_x_area(R) if x_area is None else x_area
    max_chunks = pass_max_chunks(R) if max_chunks is None else max_chunks
    ys = [np.full((R, N), np.nan, dtype=np.float32) for _, N, _ in mats]
    P_ = ctypes.c_void_p * G
    Ns = np.array([N for _, N, _ in mats], dtype=np.int64)
    Ks = np.array([K for _, _, K in mats], dtype=np.int64)
    rc = lib().emu_pass(G, P_(*[c.ctypes.data for c in canons]), Ns.ctypes.data, Ks.ctypes.data,
                        P_(*[x.ctypes.data for x in xs]), P_(*[y.ctypes.data for y in ys]), R, P, PASS_NC, x_area,
                        max_chunks, int(msum))
    if rc != 0:
        raise RuntimeError(f"emu_pass failed ({rc})")
    return ys


def dequant(canon, N, K):
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    w = np.empty((N, K), dtype=np.float32)
    lib().emu_dequant(canon.ctypes.data, N, K, w.ctypes.data)
    return w


def pack(canon, N, K):
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    Np = (N + 15) // 16 * 16
    out = np.empty(Np * (K // 256) * 144, dtype=np.uint8)
    lib().emu_pack(canon.ctypes.data, out.ctypes.data, N, K)
    return out
