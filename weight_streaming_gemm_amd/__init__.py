"""Weight-streaming Q4_K-style GEMM for MI355X (gfx950).

The C ABI is include/qgemm.h; ``qgemm`` is its ctypes binding (same names).
``roofline`` holds the host-side bandwidth bookkeeping.
"""
from . import roofline  # noqa: F401
from .qgemm import (PATH_AUTO, PATH_MFMA, PATH_VALU, PATH_TILED, MAX_R, QGemm, QGemmError, Seq,  # noqa: F401
                    argmax_rows, argmax_rows_ws, argmax_workspace_size, pack, packed_size, read_probe, run_static, status_string,
                    verify_greedy, attention_workspace_size, decode_attention)
