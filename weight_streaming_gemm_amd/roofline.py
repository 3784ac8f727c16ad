"""Roofline bookkeeping for the weight stream (host arithmetic only).

The hot path is bound by HBM bandwidth: every packed weight byte is read once
per step and serves all R rows (OpenJet multi-agent serving page, section on
moving the weights only once, where a full read of the quantised weights at the
card's nominal bandwidth is estimated as the step's floor).
"""
from __future__ import annotations

SB_WEIGHTS = 256
SB_BYTES = 144                       # canonical Q4_K-style super-block
BYTES_PER_WEIGHT = SB_BYTES / SB_WEIGHTS   # 0.5625 B = 4.5 bits

# MI355X published peaks
HBM_PEAK_GBS = 8000.0                # 8 TB/s HBM3E
MFMA_F16_DENSE_TFLOPS = 2500.0       # dense fp16/bf16 matrix peak
FP32_VECTOR_TFLOPS = 157.3
CUS = 256
CLOCK_GHZ = 2.4


def packed_bytes(N: int, K: int) -> int:
    """Algorithmic weight bytes of an N x K matrix: 144 B per 256 weights."""
    if K % SB_WEIGHTS:
        raise ValueError("K must be a multiple of 256")
    return N * (K // SB_WEIGHTS) * SB_BYTES


def ideal_seconds(nbytes: float, bandwidth_bytes_per_s: float) -> float:
    """Time to stream nbytes once at the given bandwidth."""
    return nbytes / bandwidth_bytes_per_s


def effective_gbs(nbytes: float, seconds: float) -> float:
    return nbytes / seconds / 1e9


def frac_of_peak(gbs: float, peak_gbs: float = HBM_PEAK_GBS) -> float:
    return gbs / peak_gbs


def useful_flops(R: int, N: int, K: int) -> int:
    return 2 * R * N * K


def io_bytes(R: int, N: int, K: int) -> int:
    """Activation reads (bf16) plus output writes (fp32), reported apart from weights."""
    return 2 * R * K + 4 * R * N
