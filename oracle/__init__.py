"""fp64 CPU oracle for the fused Q4_K-style dequantize-and-multiply.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The HIP library never imports, links or
calls anything here, and this package never touches the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, fp64); this wrapper only
marshals numpy arrays.  ``tiny_exact`` is an independent exact-rational
brute force used to pin the C oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QG_ORACLE_LIB names a prebuilt copy to load instead (the sanitizer test's instrumented build)
LIB_PATH = os.environ.get("QG_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

ORACLE_EARG, ORACLE_EINEXACT = -1, -2


def build(force: bool = True, mutant: int = 0, path: str | None = None) -> str:
    """Compile the oracle with gcc -O2 (no intrinsics).  ``mutant`` != 0 builds a
    deliberately wrong variant for the pin tests (never the default)."""
    path = path or LIB_PATH
    if force or not os.path.exists(path):
        src = os.path.join(_HERE, "oracle.c")
        tmp = path + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off",
                               f"-DORACLE_MUTANT={int(mutant)}", src, "-o", tmp,
                               "-lm", "-lpthread"])
        os.replace(tmp, path)
    return path


class Oracle:
    def __init__(self, path: str | None = None):
        path = path or LIB_PATH
        if not os.path.exists(path):
            build(path=path)
        lib = ctypes.CDLL(path)
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_dequant_block.restype = ctypes.c_int
        lib.oracle_dequant_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        for fn in (lib.oracle_dequant, lib.oracle_dequant_f32):
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                           ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_gemm.restype = ctypes.c_int
        lib.oracle_gemm.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_verify_greedy.restype = ctypes.c_int
        lib.oracle_verify_greedy.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_argmax_rows.restype = ctypes.c_int
        lib.oracle_argmax_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_void_p]
        self.lib = lib

    @staticmethod
    def _check(rc: int, what: str):
        if rc == ORACLE_EINEXACT:
            raise ArithmeticError(f"{what}: block outside the oracle's exact fp64 domain")
        if rc != 0:
            raise ValueError(f"{what}: bad arguments ({rc})")

    def f16(self, bits: int) -> float:
        return self.lib.oracle_f16_to_f64(bits)

    def bf16(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_f64(bits)

    def dequant_block(self, sb: np.ndarray) -> np.ndarray:
        sb = np.ascontiguousarray(sb, dtype=np.uint8)
        assert sb.size == 144
        w = np.empty(256, dtype=np.float64)
        self._check(self.lib.oracle_dequant_block(sb.ctypes.data, w.ctypes.data), "dequant_block")
        return w

    def dequant(self, canon: np.ndarray, N: int, K: int, n0: int = 0, n1: int | None = None,
                f32: bool = False) -> np.ndarray:
        n1 = N if n1 is None else n1
        canon = np.ascontiguousarray(canon, dtype=np.uint8)
        if canon.size < N * (K // 256) * 144:
            raise ValueError("canonical buffer too small")
        w = np.empty((n1 - n0, K), dtype=np.float32 if f32 else np.float64)
        fn = self.lib.oracle_dequant_f32 if f32 else self.lib.oracle_dequant
        self._check(fn(canon.ctypes.data, N, K, n0, n1, w.ctypes.data), "dequant")
        return w

    def gemm(self, canon: np.ndarray, N: int, K: int, x_bits: np.ndarray,
             threads: int | None = None) -> np.ndarray:
        """y (float64, R x N) for canonical weights and bf16 activations x (R x K bits)."""
        canon = np.ascontiguousarray(canon, dtype=np.uint8)
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        R = x_bits.shape[0]
        if x_bits.shape[1] != K or canon.size < N * (K // 256) * 144:
            raise ValueError("shape mismatch")
        y = np.empty((R, N), dtype=np.float64)
        if threads is None:
            threads = len(os.sched_getaffinity(0))
        self._check(self.lib.oracle_gemm(canon.ctypes.data, N, K, x_bits.ctypes.data, R,
                                         y.ctypes.data, threads), "gemm")
        return y

    def argmax_rows(self, y: np.ndarray) -> np.ndarray:
        y = np.ascontiguousarray(y, dtype=np.float64)
        R, N = y.shape
        idx = np.empty(R, dtype=np.int32)
        self._check(self.lib.oracle_argmax_rows(y.ctypes.data, R, N, idx.ctypes.data), "argmax")
        return idx


    def verify_greedy(self, argmax_rows, drafts, drafts_per_agent: int):
        """(tokens [A, D + 1] int32, -1 past n_new; n_new [A] int32) for argmax rows
        [A (D + 1)] and drafts [A, D]."""
        D = int(drafts_per_agent)
        am = np.ascontiguousarray(argmax_rows, dtype=np.int32).ravel()
        A = am.size // (D + 1)
        dr = np.ascontiguousarray(drafts, dtype=np.int32).reshape(A, D) if D > 0 else np.zeros((A, 0), np.int32)
        tokens = np.empty((A, D + 1), dtype=np.int32)
        n_new = np.empty(A, dtype=np.int32)
        self._check(self.lib.oracle_verify_greedy(am.ctypes.data, am.size, dr.ctypes.data if D > 0 else None, D,
                                                  tokens.ctypes.data, n_new.ctypes.data), "verify")
        return tokens, n_new


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
