"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import weight_streaming_gemm_amd as wsg
from weight_streaming_gemm_amd import qgemm as Q

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "qgemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemm_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 13
    L = Q.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in qgemm.h but not exported"
    assert set(names) == set(Q.EXPORTS)


def test_status_strings():
    for code in range(0, -9, -1):
        s = wsg.status_string(code)
        assert s and s != "unknown status"
    assert wsg.status_string(-99) == "unknown status"


def test_packed_size():
    assert wsg.packed_size(256, 1024) == 147456
    assert wsg.packed_size(151936, 5120) == 437_575_680
    assert wsg.packed_size(17, 256) == 32 * 144          # N padded to 16
    for N, K in ((0, 256), (16, 100), (16, 0), (-1, 256), (16, 255)):
        with pytest.raises(Q.QGemmError) as e:
            wsg.packed_size(N, K)
        assert e.value.status == Q.QGEMM_ESHAPE
    assert Q.lib().qgemm_packed_size(16, 256, None) == Q.QGEMM_EINVAL


def test_host_validation_codes():
    L = Q.lib()
    vp = ctypes.c_void_p
    assert L.qgemm_pack(None, vp(4096), 16, 256, None) == Q.QGEMM_EINVAL
    assert L.qgemm_pack(vp(4096), vp(4096), 16, 100, None) == Q.QGEMM_ESHAPE
    assert L.qgemm_pack(vp(4097), vp(4096), 16, 256, None) == Q.QGEMM_EALIGN
    h = vp()
    assert L.qgemm_create(ctypes.byref(h), vp(4096), 16, 256, 0, 0) == Q.QGEMM_ERANGE_R
    assert L.qgemm_create(ctypes.byref(h), vp(4096), 16, 256, 65, 0) == Q.QGEMM_ERANGE_R
    assert L.qgemm_create(ctypes.byref(h), vp(4096), 16, 256, 12, 1) == Q.QGEMM_EINVAL
    assert L.qgemm_create(ctypes.byref(h), vp(4104), 16, 256, 12, 0) == Q.QGEMM_EALIGN
    assert L.qgemm_create(None, vp(4096), 16, 256, 12, 0) == Q.QGEMM_EINVAL
    assert L.qgemm_run(None, vp(4096), vp(4096), 1, None) == Q.QGEMM_EINVAL
    assert L.qgemm_run_path(None, vp(4096), vp(4096), 1, 2, None) == Q.QGEMM_EINVAL
    # the allocation-free entry point rejects bad arguments before any HIP call
    assert L.qgemm_run_static(None, 16, 256, vp(4096), vp(4096), 1, None) == Q.QGEMM_EINVAL
    assert L.qgemm_run_static(vp(4096), 16, 100, vp(4096), vp(4096), 1, None) == Q.QGEMM_ESHAPE
    assert L.qgemm_run_static(vp(4096), 16, 256, vp(4096), vp(4096), 65, None) == Q.QGEMM_ERANGE_R
    assert L.qgemm_run_static(vp(4096), 16, 256, vp(4096), vp(4096), -1, None) == Q.QGEMM_ERANGE_R
    assert L.qgemm_run_static(vp(4096), 16, 256, None, vp(4096), 1, None) == Q.QGEMM_EINVAL
    assert L.qgemm_run_static(vp(4104), 16, 256, vp(4096), vp(4096), 1, None) == Q.QGEMM_EALIGN
    assert L.qgemm_run_static(vp(4096), 16, 256, vp(4096), vp(4100), 1, None) == Q.QGEMM_EALIGN
    assert L.qgemm_run_static(vp(4096), 16, 256, None, None, 0, None) == Q.QGEMM_OK      # R = 0: no-op
    assert Q.STATIC_SCRATCH_BYTES == 16 << 20
    # the read probe checks its arguments before any HIP call
    assert L.qgemm_read_probe(None, 4096, vp(4096), None) == Q.QGEMM_EINVAL
    assert L.qgemm_read_probe(vp(4096), 4100, vp(4096), None) == Q.QGEMM_EINVAL
    assert L.qgemm_read_probe(vp(4096), 1 << 40, vp(4096), None) == Q.QGEMM_EINVAL
    assert L.qgemm_read_probe(vp(4104), 4096, vp(4096), None) == Q.QGEMM_EALIGN
    assert L.qgemm_read_probe(vp(4096), 4096, None, None) == Q.QGEMM_EINVAL
    assert L.qgemm_run_prefill(None, vp(4096), vp(4096), 100, None, 0, None) == Q.QGEMM_EINVAL
    assert L.qgemm_prefill_workspace_size(None, 100, ctypes.byref(sz0 := ctypes.c_size_t())) == Q.QGEMM_EINVAL
    assert L.qgemm_dequantize(None, vp(4096), None) == Q.QGEMM_EINVAL
    assert L.qgemm_query(None, 1, 0, None) == Q.QGEMM_EINVAL
    assert L.qgemm_argmax_rows(vp(4096), -1, 10, vp(4096), None) == Q.QGEMM_ERANGE_R
    assert L.qgemm_argmax_rows(vp(4096), 2, 0, vp(4096), None) == Q.QGEMM_ESHAPE
    assert L.qgemm_argmax_rows(None, 2, 10, vp(4096), None) == Q.QGEMM_EINVAL
    assert L.qgemm_argmax_rows(None, 0, 10, None, None) == Q.QGEMM_OK        # R = 0: no-op
    # chunked argmax and draft verification: size arithmetic and argument checks (no GPU call)
    assert wsg.argmax_workspace_size(12, 151936) == 1888          # 12 x 19 chunks x 8 B + 13 counters, 16 B multiple
    assert wsg.argmax_workspace_size(1, 1) == 16
    sz = ctypes.c_size_t()
    assert L.qgemm_argmax_workspace_size(65, 10, ctypes.byref(sz)) == Q.QGEMM_ERANGE_R
    assert L.qgemm_argmax_workspace_size(2, 0, ctypes.byref(sz)) == Q.QGEMM_ESHAPE
    assert L.qgemm_argmax_workspace_size(2, 10, None) == Q.QGEMM_EINVAL
    assert L.qgemm_argmax_rows_ws(vp(4096), 2, 10, vp(4096), vp(4096), 8, None) == Q.QGEMM_EINVAL   # too small
    assert L.qgemm_argmax_rows_ws(vp(4096), 2, 10, vp(4096), vp(4104), 4096, None) == Q.QGEMM_EALIGN
    assert L.qgemm_argmax_rows_ws(None, 0, 10, None, None, 0, None) == Q.QGEMM_OK
    assert L.qgemm_verify_greedy(vp(4096), 10, vp(4096), 2, vp(4096), vp(4096), None) == Q.QGEMM_EINVAL  # 10 % 3
    assert L.qgemm_verify_greedy(vp(4096), 12, None, 2, vp(4096), vp(4096), None) == Q.QGEMM_EINVAL      # no drafts
    assert L.qgemm_verify_greedy(vp(4096), 12, vp(4096), -1, vp(4096), vp(4096), None) == Q.QGEMM_EINVAL
    assert L.qgemm_verify_greedy(vp(4096), 65, vp(4096), 0, vp(4096), vp(4096), None) == Q.QGEMM_ERANGE_R
    assert L.qgemm_verify_greedy(None, 0, None, 0, vp(4096), vp(4096), None) == Q.QGEMM_OK
    assert L.qgemm_seq_run_verify(None, None, None, 12, vp(4096), vp(4096), 2, vp(4096), vp(4096),
                                  None) == Q.QGEMM_EINVAL
    # decode attention: workspace arithmetic and shape checks (no GPU call)
    # 4 agents x 8 heads: 8 splits each at most (256 in all), of 2880 positions (23003 / 8 rounded up to
    # 32), so 8 splits
    assert wsg.attention_workspace_size(4, 3, 8, 23000) == 4 * 8 * 8 * 32 * 130 * 4
    assert wsg.attention_workspace_size(1, 1, 1, 0) == 1 * 1 * 1 * 32 * 130 * 4
    assert L.qgemm_attention_workspace_size(4, 5, 8, 100, ctypes.byref(sz)) == Q.QGEMM_ESHAPE
    att = lambda **kw: L.qgemm_decode_attention(  # noqa: E731
        vp(4096), vp(4096), vp(4096), vp(4096), kw.get("A", 2), kw.get("rows", 3), kw.get("hq", 16),
        kw.get("hkv", 2), kw.get("d", 128), kw.get("cap", 100), kw.get("max_len", 50), vp(4096),
        vp(kw.get("ws", 4096)), kw.get("ws_bytes", 1 << 30), None)
    assert att(d=64) == Q.QGEMM_ESHAPE
    assert att(hq=12) == Q.QGEMM_ESHAPE
    assert att(rows=5) == Q.QGEMM_ESHAPE
    assert att(cap=52) == Q.QGEMM_ESHAPE                      # cap < max_len + rows
    assert att(A=64, cap=1 << 20, max_len=100) == Q.QGEMM_ESHAPE  # caches beyond 2 GiB
    assert att(ws_bytes=16) == Q.QGEMM_EINVAL
    assert att(ws=4104) == Q.QGEMM_EALIGN
    assert att(A=0) == Q.QGEMM_OK
    s = vp()
    assert L.qgemm_seq_create(ctypes.byref(s), None, 1, 0) == Q.QGEMM_EINVAL
    assert L.qgemm_seq_create(ctypes.byref(s), None, 1, 4) == Q.QGEMM_EINVAL
    assert L.qgemm_seq_create(ctypes.byref(s), None, 1, 8) == Q.QGEMM_EINVAL
    assert L.qgemm_seq_run(None, None, None, 1, None, None) == Q.QGEMM_EINVAL
    assert L.qgemm_destroy(None) == Q.QGEMM_OK
    assert L.qgemm_seq_destroy(None) == Q.QGEMM_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(Q, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(Q, "_lib", None)
    with pytest.raises(RuntimeError):
        Q.lib()
