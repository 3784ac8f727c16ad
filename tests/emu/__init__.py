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
    src = os.path.join(HERE, "qgemm_emu.cpp")
    deps = [src] + [os.path.join(HERE, "..", "..", "weight_streaming_gemm_amd", "csrc", f)
                    for f in ("layout.h", "operand.h", "stream_sched.h")]
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
        L.emu_gemm.restype = ctypes.c_int
        L.emu_gemm.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.emu_stream.restype = ctypes.c_int
        L.emu_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p]
        L.emu_dequant.restype = ctypes.c_int
        L.emu_dequant.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.emu_pack.restype = ctypes.c_int
        L.emu_pack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
        _lib = L
    return _lib


def gemm(canon, N, K, x_bits, NT=2, S=1):
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R = x_bits.shape[0]
    y = np.empty((R, N), dtype=np.float32)
    lib().emu_gemm(canon.ctypes.data, N, K, x_bits.ctypes.data, R, NT, S, y.ctypes.data)
    return y


def stream(canon, N, K, x_bits, NT=2, P=8, order_seed=0):
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    R = x_bits.shape[0]
    y = np.empty((R, N), dtype=np.float32)
    rc = lib().emu_stream(canon.ctypes.data, N, K, x_bits.ctypes.data, R, NT, P, order_seed, y.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"emu_stream failed ({rc})")
    return y


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
