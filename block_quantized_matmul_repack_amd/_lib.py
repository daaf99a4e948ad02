"""ctypes loader for libtiledq.so: argument types of every C-ABI entry point.

No compute happens here; a missing library is an error (there is no fallback).
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtiledq.so")

_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64
INT = ctypes.c_int
SZ = ctypes.c_size_t

SIGNATURES = {
    "tq_tile_bytes": (SZ, [INT]),
    "tq_block_bytes": (SZ, [INT]),
    "tq_tiled_bytes": (SZ, [INT, I64, I64]),
    "tq_flat_bytes": (SZ, [INT, I64, I64]),
    "tq_supported": (INT, [INT, I64, I64, I64, INT]),
    "tq_status_string": (ctypes.c_char_p, [INT]),
    "tq_repack_tiles": (INT, [INT, P, I64, I64, P, P]),
    "tq_quantize_act": (INT, [INT, P, I64, I64, I64, P, P, P]),
    "tq_qgemv_workspace_bytes": (SZ, [INT, I64, I64, I64]),
    "tq_qgemv": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P, SZ, P]),
    "tq_qgemv_noalloc": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P]),
    "tq_qgemv_x": (INT, [INT, P, I64, I64, INT, P, I64, I64, P, P, I64, P, SZ, P]),
    "tq_qgemm": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P]),
    "tq_matmul": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P, SZ, P]),
    "tq_matmul_path": (INT, [INT, I64, I64, I64]),
    "tq_matmul_workspace_bytes": (SZ, [INT, I64, I64, I64]),
    "tq_matmul_x_workspace_bytes": (SZ, [INT, I64, I64, I64]),
    "tq_matmul_x": (INT, [INT, P, I64, I64, INT, P, I64, I64, P, P, I64, P, SZ, P]),
    "tq_block_dots": (INT, [INT, P, I64, I64, P, I64, P, P, INT, P]),
    "tq_unpack_tiles": (INT, [INT, P, I64, I64, P, P]),
    "tq_quantize_act_mx": (INT, [INT, P, I64, I64, I64, P, P, P]),
    "tq_qgemm_mx": (INT, [P, I64, I64, P, P, I64, P, I64, P]),
    "tq_matmul_mx_workspace_bytes": (SZ, [I64, I64, I64]),
    "tq_matmul_mx": (INT, [P, I64, I64, P, P, I64, P, I64, P, SZ, P]),
    "tq_stream_read": (INT, [P, SZ, P, P]),
    "tq_qgemv_flat": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P]),
    "tq_qgemm_flat": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P]),
    "tq_matmul_flat": (INT, [INT, P, I64, I64, P, P, I64, P, P, I64, P]),
}


class TiledqError(RuntimeError):
    pass


def lib():
    """Load libtiledq.so (built by block_quantized_matmul_repack_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise TiledqError(
                f"{LIB_PATH} is not built; run `python -m block_quantized_matmul_repack_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status, what):
    if status != 0:
        msg = lib().tq_status_string(status).decode()
        raise TiledqError(f"{what}: {msg} (status {status})")
