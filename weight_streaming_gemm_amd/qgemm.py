"""Thin ctypes binding of libqgemm.so (include/qgemm.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch provides device memory (tensor.data_ptr()) and the current
stream; nothing else from torch is used.  If the library is missing, loading
fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemm.so")

QGEMM_OK, QGEMM_EINVAL, QGEMM_ESHAPE, QGEMM_EALIGN = 0, -1, -2, -3
QGEMM_ERANGE_R, QGEMM_ENOMEM, QGEMM_EHIP, QGEMM_EPATH, QGEMM_ESCRATCH = -4, -5, -6, -7, -8
STATIC_SCRATCH_BYTES = 16 << 20
PATH_AUTO, PATH_VALU, PATH_MFMA, PATH_TILED = 0, 1, 2, 3
TILED_MIN_R = 24
SEQ_PERSISTENT = 1
SEQ_SUB_BLOCK_SUMS = 2
SEQ_GATED_INPUTS = 4
MAX_R = 64
MAX_PREFILL_R = 8192

# every symbol include/qgemm.h declares
EXPORTS = (
    "qgemm_packed_size", "qgemm_pack", "qgemm_create", "qgemm_run", "qgemm_run_path", "qgemm_run_static",
    "qgemm_run_prefill",
    "qgemm_prefill_workspace_size",
    "qgemm_dequantize", "qgemm_argmax_rows", "qgemm_argmax_workspace_size", "qgemm_argmax_rows_ws",
    "qgemm_verify_greedy", "qgemm_attention_workspace_size", "qgemm_decode_attention", "qgemm_query",
    "qgemm_destroy",
    "qgemm_seq_create", "qgemm_seq_run", "qgemm_seq_run_verify", "qgemm_seq_errors", "qgemm_seq_destroy",
    "qgemm_read_probe",
    "qgemm_status_string",
)


class QGemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("row_tiles", ctypes.c_int), ("subtiles_per_wave", ctypes.c_int),
                ("tiles", ctypes.c_int64), ("workgroups", ctypes.c_int64), ("steps", ctypes.c_int64),
                ("kernels", ctypes.c_int), ("workspace_bytes", ctypes.c_size_t), ("ranges", ctypes.c_int64),
                ("waves_per_workgroup", ctypes.c_int), ("wave_columns", ctypes.c_int),
                ("whole_tile_ranges", ctypes.c_int), ("k_chunks", ctypes.c_int),
                ("min_term_sums", ctypes.c_int)]


_lib = None


def lib():
    """Load libqgemm.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "qgemm_packed_size": [i64, i64, ctypes.POINTER(ctypes.c_size_t)],
            "qgemm_pack": [vp, vp, i64, i64, vp],
            "qgemm_create": [ctypes.POINTER(vp), vp, i64, i64, i32, ctypes.c_uint32],
            "qgemm_run": [vp, vp, vp, i32, vp],
            "qgemm_run_path": [vp, vp, vp, i32, i32, vp],
            "qgemm_run_static": [vp, i64, i64, vp, vp, i32, vp],
            "qgemm_run_prefill": [vp, vp, vp, i32, vp, ctypes.c_size_t, vp],
            "qgemm_prefill_workspace_size": [vp, i32, ctypes.POINTER(ctypes.c_size_t)],
            "qgemm_dequantize": [vp, vp, vp],
            "qgemm_argmax_rows": [vp, i32, i64, vp, vp],
            "qgemm_argmax_workspace_size": [i32, i64, ctypes.POINTER(ctypes.c_size_t)],
            "qgemm_argmax_rows_ws": [vp, i32, i64, vp, vp, ctypes.c_size_t, vp],
            "qgemm_verify_greedy": [vp, i32, vp, i32, vp, vp, vp],
            "qgemm_attention_workspace_size": [i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)],
            "qgemm_decode_attention": [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, ctypes.c_size_t, vp],
            "qgemm_query": [vp, i32, i32, ctypes.POINTER(Info)],
            "qgemm_destroy": [vp],
            "qgemm_seq_create": [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, ctypes.c_uint32],
            "qgemm_seq_run": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, vp],
            "qgemm_seq_run_verify": [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, vp, i32, vp, vp, vp],
            "qgemm_seq_errors": [vp, ctypes.POINTER(ctypes.c_uint32)],
            "qgemm_seq_destroy": [vp],
            "qgemm_read_probe": [vp, ctypes.c_uint64, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.qgemm_status_string.argtypes = [ctypes.c_int]
        L.qgemm_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qgemm_status_string(status).decode()


def _check(rc: int, what: str):
    if rc != QGEMM_OK:
        raise QGemmError(rc, what)


def _stream(stream=None) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream) or 0


def _ptr(t) -> int:
    return 0 if t is None else (t if isinstance(t, int) else t.data_ptr())


def packed_size(N: int, K: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().qgemm_packed_size(N, K, ctypes.byref(out)), "qgemm_packed_size")
    return out.value


def pack(canon_dev, packed_dev, N: int, K: int, stream=None):
    _check(lib().qgemm_pack(_ptr(canon_dev), _ptr(packed_dev), N, K, _stream(stream)), "qgemm_pack")
    return packed_dev


def run_static(packed_dev, N: int, K: int, x, y, R: int | None = None, stream=None):
    """qgemm_run without a handle, on the library's fixed scratch (no allocation)."""
    R = x.shape[0] if R is None else R
    _check(lib().qgemm_run_static(_ptr(packed_dev), N, K, _ptr(x), _ptr(y), R, _stream(stream)),
           "qgemm_run_static")


def read_probe(buf, nbytes: int, sink, stream=None):
    """Read nbytes of device memory at buf once at full speed (a measurement aid:
    the practical HBM read ceiling); sink is 16 KiB of device scratch."""
    _check(lib().qgemm_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "qgemm_read_probe")


def argmax_rows(y, idx, R: int | None = None, stream=None):
    R = y.shape[0] if R is None else R
    N = y.shape[1]
    _check(lib().qgemm_argmax_rows(_ptr(y), R, N, _ptr(idx), _stream(stream)), "qgemm_argmax_rows")
    return idx


def argmax_workspace_size(R: int, N: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().qgemm_argmax_workspace_size(R, N, ctypes.byref(out)), "qgemm_argmax_workspace_size")
    return out.value


def argmax_rows_ws(y, idx, workspace, R: int | None = None, stream=None):
    R = y.shape[0] if R is None else R
    N = y.shape[1]
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qgemm_argmax_rows_ws(_ptr(y), R, N, _ptr(idx), _ptr(workspace), nbytes, _stream(stream)),
           "qgemm_argmax_rows_ws")
    return idx


def verify_greedy(argmax_idx, drafts, drafts_per_agent: int, tokens, n_new, R: int | None = None, stream=None):
    R = argmax_idx.shape[0] if R is None else R
    _check(lib().qgemm_verify_greedy(_ptr(argmax_idx), R, _ptr(drafts), drafts_per_agent, _ptr(tokens), _ptr(n_new),
                                     _stream(stream)), "qgemm_verify_greedy")
    return tokens, n_new


def attention_workspace_size(agents: int, rows: int, kv_heads: int, max_len: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().qgemm_attention_workspace_size(agents, rows, kv_heads, max_len, ctypes.byref(out)),
           "qgemm_attention_workspace_size")
    return out.value


def decode_attention(q, k_cache, v_cache, lengths, out, workspace, max_len: int, stream=None):
    """q [A, rows, Hq, 128], caches [A, Hkv, cap, 128] (bf16 bit patterns on the device),
    lengths [A] int32 on the device, out [A, rows, Hq, 128] fp32."""
    A, rows, Hq, d = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().qgemm_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lengths), A, rows, Hq, Hkv, d,
                                        cap, max_len, _ptr(out), _ptr(workspace), nbytes, _stream(stream)),
           "qgemm_decode_attention")
    return out


class QGemm:
    """One packed weight matrix (borrowed device buffer) and its workspace."""

    def __init__(self, packed_dev, N: int, K: int, max_R: int = MAX_R, flags: int = 0):
        self.N, self.K, self.max_R = N, K, max_R
        self._packed = packed_dev            # keep the borrowed buffer alive
        h = ctypes.c_void_p()
        _check(lib().qgemm_create(ctypes.byref(h), _ptr(packed_dev), N, K, max_R, flags), "qgemm_create")
        self.h = h

    def run(self, x, y, R: int | None = None, path: int = PATH_AUTO, stream=None):
        R = x.shape[0] if R is None else R
        _check(lib().qgemm_run_path(self.h, _ptr(x), _ptr(y), R, path, _stream(stream)), "qgemm_run")
        return y

    def prefill_workspace_size(self, R: int) -> int:
        n = ctypes.c_size_t()
        _check(lib().qgemm_prefill_workspace_size(self.h, R, ctypes.byref(n)), "qgemm_prefill_workspace_size")
        return n.value

    def run_prefill(self, x, y, R: int | None = None, workspace=None, stream=None):
        """Many rows (a prompt chunk with the decode rows): the row-tiled kernel.
        workspace: a device buffer of at least prefill_workspace_size(R) bytes
        (torch allocates one here when none is given)."""
        R = x.shape[0] if R is None else R
        need = self.prefill_workspace_size(R)
        if need and workspace is None:
            import torch
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().qgemm_run_prefill(self.h, _ptr(x), _ptr(y), R, _ptr(workspace), nbytes, _stream(stream)),
               "qgemm_run_prefill")
        return y

    def dequantize(self, w, stream=None):
        _check(lib().qgemm_dequantize(self.h, _ptr(w), _stream(stream)), "qgemm_dequantize")
        return w

    def query(self, R: int, path: int = PATH_AUTO) -> dict:
        info = Info()
        _check(lib().qgemm_query(self.h, R, path, ctypes.byref(info)), "qgemm_query")
        return {f: getattr(info, f) for f, _ in Info._fields_}

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().qgemm_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Seq:
    """A full weight pass: the GEMMs run in order, as a replayed graph of one launch
    per GEMM, or (persistent=True) as one cooperative launch, whose min term comes
    from products with the mins or (sub_block_sums=True) from staged sub-block sums,
    and where (gated_inputs=True) a down projection after a fused gate|up waits only
    for the outputs it reads."""

    def __init__(self, gemms, persistent: bool = False, sub_block_sums: bool = False, gated_inputs: bool = False):
        self.gemms = list(gemms)
        arr = (ctypes.c_void_p * len(self.gemms))(*[g.h.value for g in self.gemms])
        s = ctypes.c_void_p()
        flags = ((SEQ_PERSISTENT if persistent else 0) | (SEQ_SUB_BLOCK_SUMS if sub_block_sums else 0) |
                 (SEQ_GATED_INPUTS if gated_inputs else 0))
        _check(lib().qgemm_seq_create(ctypes.byref(s), arr, len(self.gemms), flags), "qgemm_seq_create")
        self.s = s

    def run(self, xs, ys, R: int, argmax_idx=None, stream=None):
        n = len(self.gemms)
        xa = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
        ya = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
        _check(lib().qgemm_seq_run(self.s, xa, ya, R, _ptr(argmax_idx), _stream(stream)), "qgemm_seq_run")

    def run_verify(self, xs, ys, R: int, argmax_idx, drafts, drafts_per_agent: int, tokens, n_new, stream=None):
        n = len(self.gemms)
        xa = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
        ya = (ctypes.c_void_p * n)(*[_ptr(y) for y in ys])
        _check(lib().qgemm_seq_run_verify(self.s, xa, ya, R, _ptr(argmax_idx), _ptr(drafts), drafts_per_agent,
                                          _ptr(tokens), _ptr(n_new), _stream(stream)), "qgemm_seq_run_verify")

    def errors(self) -> int:
        """Barrier waits that gave up since the last call (synchronises the device)."""
        n = ctypes.c_uint32()
        _check(lib().qgemm_seq_errors(self.s, ctypes.byref(n)), "qgemm_seq_errors")
        return n.value

    def close(self):
        if getattr(self, "s", None) is not None and self.s.value:
            lib().qgemm_seq_destroy(self.s)
            self.s = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
