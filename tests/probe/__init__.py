"""Test-only probe library of gfx950 builtin layouts and rounding (probe.hip)."""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libprobe.so")


def build() -> str:
    from weight_streaming_gemm_amd.build import HIPCC, DEVICE_FLAGS, ARCH
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "-O2", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
                           *DEVICE_FLAGS, os.path.join(HERE, "probe.hip"), "-o", tmp],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    os.replace(tmp, LIB)
    return LIB


def lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} missing: run the build step")
    L = ctypes.CDLL(LIB)
    vp = ctypes.c_void_p
    L.probe_mfma_16x16x32_f16.argtypes = [vp, vp, vp]
    L.probe_mfma_16x16x4_f32.argtypes = [vp, vp, vp]
    L.probe_pk_fma_f16.argtypes = [vp, vp, vp, vp, ctypes.c_int]
    for f in (L.probe_mfma_16x16x32_f16, L.probe_mfma_16x16x4_f32, L.probe_pk_fma_f16):
        f.restype = ctypes.c_int
    return L
