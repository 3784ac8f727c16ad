"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This package holds no GEMM arithmetic: it draws random fields, writes them in
the canonical Q4_K-style super-block byte layout (see ``synth.c`` for the
layout) and draws bf16 activation rows.  ``workloads`` names the matrix shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QG_SYNTH_LIB names a prebuilt copy to load instead (the sanitizer test's instrumented build)
LIB_PATH = os.environ.get("QG_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
SB_BYTES = 144
SB_WEIGHTS = 256


def build(force: bool = True) -> str:
    """Compile libsynth.so in-tree with gcc (plain C, -O2)."""
    if force or not os.path.exists(LIB_PATH):
        src = os.path.join(_HERE, "synth.c")
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11",
                               src, "-o", tmp, "-lm", "-lpthread"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_mix64.restype = ctypes.c_uint64
        lib.synth_mix64.argtypes = [ctypes.c_uint64]
        lib.synth_f64_to_f16.restype = ctypes.c_uint16
        lib.synth_f64_to_f16.argtypes = [ctypes.c_double]
        lib.synth_f64_to_bf16.restype = ctypes.c_uint16
        lib.synth_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.synth_matrix_rows.restype = ctypes.c_int
        lib.synth_matrix_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
        lib.synth_x.restype = ctypes.c_int
        lib.synth_x.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def mix64(z: int) -> int:
    return int(_load().synth_mix64(z & 0xFFFFFFFFFFFFFFFF))


def f64_to_f16_bits(v: float) -> int:
    return int(_load().synth_f64_to_f16(float(v)))


def f64_to_bf16_bits(v: float) -> int:
    return int(_load().synth_f64_to_bf16(float(v)))


def matrix_rows(seed: int, mid: int, N: int, K: int, n0: int = 0, n1: int | None = None,
                edge_mode: int = 0, out: np.ndarray | None = None,
                threads: int | None = None) -> np.ndarray:
    """Canonical super-block bytes (uint8, (n1-n0)*K/256*144) of rows [n0, n1)."""
    if n1 is None:
        n1 = N
    if K % SB_WEIGHTS:
        raise ValueError("K must be a multiple of 256")
    nbytes = (n1 - n0) * (K // SB_WEIGHTS) * SB_BYTES
    if out is None:
        out = np.empty(nbytes, dtype=np.uint8)
    elif out.nbytes < nbytes or out.dtype != np.uint8 or not out.flags.c_contiguous:
        raise ValueError("out buffer too small or not contiguous uint8")
    rc = _load().synth_matrix_rows(seed, mid, N, K, n0, n1, edge_mode,
                                   out.ctypes.data, threads or default_threads())
    if rc != 0:
        raise ValueError("synth_matrix_rows: bad arguments")
    return out[:nbytes]


def x_bf16(seed: int, sid: int, R: int, K: int, outlier_p: float = 0.0,
           outlier_scale: float = 50.0) -> np.ndarray:
    """Activation rows as bf16 bit patterns, uint16 array of shape (R, K)."""
    out = np.empty((R, K), dtype=np.uint16)
    rc = _load().synth_x(seed, sid, R, K, outlier_p, outlier_scale, out.ctypes.data)
    if rc != 0:
        raise ValueError("synth_x: bad arguments")
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: bf16 is the top half of fp32)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
