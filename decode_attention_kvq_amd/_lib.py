"""ctypes loader for libkvq.so (the HIP library built in-tree by build.py).

There is no fallback: if the library is missing or fails to load, every entry point
raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
NOALLOC_SCRATCH_BYTES = 32 << 20
STATUS_NAMES = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID_ARG", -2: "KVQ_ERR_UNSUPPORTED",
                -3: "KVQ_ERR_WORKSPACE", -4: "KVQ_ERR_HIP"}
EXPORTS = ("kvq_block_bytes", "kvq_quantize_append", "kvq_decode_workspace_bytes",
           "kvq_decode_step_workspace_bytes",
           "kvq_decode_attn", "kvq_decode_attn_noalloc", "kvq_decode_step", "kvq_dequant", "kvq_window_bytes", "kvq_window_prefill",
           "kvq_window_workspace_bytes", "kvq_window_decode_attn", "kvq_window_decode_step",
           "kvq_status_string", "kvq_last_error")


class KvqCacheDesc(C.Structure):
    _fields_ = [("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("page_size", C.c_int32),
                ("bits_k", C.c_int32), ("bits_v", C.c_int32), ("quant_k", C.c_int32),
                ("quant_v", C.c_int32), ("p_lo", C.c_float), ("p_hi", C.c_float),
                ("alpha_k", C.c_float), ("alpha_v", C.c_float), ("num_pages", C.c_int64),
                ("k_pages", C.c_void_p), ("v_pages", C.c_void_p)]


class KvqWindowDesc(C.Structure):
    _fields_ = [("sink", C.c_int32), ("keep", C.c_int32), ("flush", C.c_int32), ("num_rows", C.c_int32),
                ("dtype", C.c_int32), ("k_win", C.c_void_p), ("v_win", C.c_void_p)]


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m decode_attention_kvq_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    D = C.POINTER(KvqCacheDesc)
    L.kvq_block_bytes.restype = sz
    L.kvq_block_bytes.argtypes = [i32]
    L.kvq_quantize_append.restype = i32
    L.kvq_quantize_append.argtypes = [D, P, P, i32, i64, P, P, i32, P]
    L.kvq_decode_workspace_bytes.restype = sz
    L.kvq_decode_workspace_bytes.argtypes = [D, i32, i32, i32]
    L.kvq_decode_step_workspace_bytes.restype = sz
    L.kvq_decode_step_workspace_bytes.argtypes = [D, i32, i32, i32]
    L.kvq_decode_attn.restype = i32
    L.kvq_decode_attn.argtypes = [D, P, i32, i32, i32, P, P, i32, P, i32, f32, P, P, sz, P]
    L.kvq_decode_attn_noalloc.restype = i32
    L.kvq_decode_attn_noalloc.argtypes = [D, P, i32, i32, i32, P, P, i32, P, i32, f32, P, P]
    L.kvq_decode_step.restype = i32
    L.kvq_decode_step.argtypes = [D, P, P, P, i32, i32, i32, P, P, i32, P, P, i32, P, i32, f32, P, P, sz, P]
    L.kvq_dequant.restype = i32
    L.kvq_dequant.argtypes = [D, i32, P, i64, P, P]
    W = C.POINTER(KvqWindowDesc)
    L.kvq_window_bytes.restype = sz
    L.kvq_window_bytes.argtypes = [D, W]
    L.kvq_window_prefill.restype = i32
    L.kvq_window_prefill.argtypes = [D, W, P, P, i32, P, i64, P, i32, P, P, P]
    L.kvq_window_workspace_bytes.restype = sz
    L.kvq_window_workspace_bytes.argtypes = [D, W, i32, i32, i32]
    L.kvq_window_decode_attn.restype = i32
    L.kvq_window_decode_attn.argtypes = [D, W, P, i32, i32, P, P, i32, P, P, i32, f32, P, P, sz, P]
    L.kvq_window_decode_step.restype = i32
    L.kvq_window_decode_step.argtypes = [D, W, P, P, P, i32, i32, P, P, P, i32, P, P, i32, f32, P, P, sz, P]
    L.kvq_status_string.restype = C.c_char_p
    L.kvq_status_string.argtypes = [i32]
    L.kvq_last_error.restype = C.c_char_p
    L.kvq_last_error.argtypes = []
    _lib = L
    return L


def check(status: int) -> None:
    if status != KVQ_OK:
        msg = load().kvq_last_error().decode()
        raise KvqError(status, msg)
