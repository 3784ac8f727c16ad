"""Helpers for the GPU tests: upload synthetic inputs, run through the C ABI."""
from __future__ import annotations

import numpy as np

import synth

_dev = None


def dev():
    global _dev
    if _dev is None:
        import torch
        assert torch.cuda.is_available(), "GPU test run without a GPU"
        _dev = torch.device("cuda:0")
    return _dev


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def upload_packed(canon: np.ndarray, N: int, K: int):
    """Canonical bytes -> device packed buffer (packed on the GPU)."""
    import torch
    import weight_streaming_gemm_amd as wsg
    c = to_dev(canon)
    packed = torch.empty(wsg.packed_size(N, K), dtype=torch.uint8, device=dev())
    wsg.pack(c, packed, N, K)
    torch.cuda.synchronize()
    del c
    return packed


def make(seed: int, mid: int, N: int, K: int, max_R: int = 64, edge_mode: int = 0):
    import weight_streaming_gemm_amd as wsg
    canon = synth.matrix_rows(seed, mid, N, K, edge_mode=edge_mode)
    packed = upload_packed(canon, N, K)
    return canon, wsg.QGemm(packed, N, K, max_R=max_R)


def run(g, x_bits: np.ndarray, path: int = 0) -> np.ndarray:
    import torch
    R = x_bits.shape[0]
    xd = to_dev(x_bits)
    y = torch.empty((R, g.N), dtype=torch.float32, device=dev())
    g.run(xd, y, path=path)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def dequant(g) -> np.ndarray:
    import torch
    w = torch.empty((g.N, g.K), dtype=torch.float32, device=dev())
    g.dequantize(w)
    torch.cuda.synchronize()
    return w.cpu().numpy()
