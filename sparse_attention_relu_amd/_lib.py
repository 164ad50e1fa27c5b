"""ctypes loader for libsparse_mla.so (the HIP library built in-tree).

Loading fails loudly when the library is missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_mla.so")

c_i32, c_i64, c_f32, c_sz, c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class LayerDesc(ctypes.Structure):
    _fields_ = [("is_full", c_i32), ("q_idx", c_p), ("w", c_p), ("k_idx", c_p), ("idx", c_p),
                ("q_abs", c_p), ("kv", c_p), ("w_uv", c_p), ("out", c_p)]


class BatchDesc(ctypes.Structure):
    _fields_ = [("seq_start", c_p), ("q_seq", c_p), ("q_pos", c_p), ("n_q", c_i32), ("n_seq", c_i32),
                ("ld", c_i64)]


class StageEvents(ctypes.Structure):
    _fields_ = [("indexer_begin", c_p), ("indexer_end", c_p), ("topk_begin", c_p), ("topk_end", c_p),
                ("attn_begin", c_p), ("attn_end", c_p)]


SIGNATURES = {
    "sa_version": (c_i32, []),
    "sa_status_string": (ctypes.c_char_p, [c_i32]),
    "sa_last_error_message": (ctypes.c_char_p, []),
    "sa_layer_is_full": (c_i32, [c_i32]),
    "sa_indexer_score": (c_i32, [c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_i32, c_p, c_i64, c_p]),
    "sa_indexer_score_algo": (c_i32, [c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_i32, c_p, c_i64, c_i32, c_p]),
    "sa_topk_workspace_size": (c_sz, [c_i32, c_i64, c_i32]),
    "sa_topk_select": (c_i32, [c_p, c_i64, c_p, c_i32, c_i32, c_p, c_p, c_sz, c_p]),
    "sa_topk_select_algo": (c_i32, [c_p, c_i64, c_p, c_i32, c_i32, c_p, c_p, c_sz, c_i32, c_p]),
    "sa_mla_workspace_size": (c_sz, [c_i32, c_i32]),
    "sa_mla_sparse_attn": (c_i32, [c_p, c_p, c_p, c_p, c_p, c_i32, c_i32, c_p, c_f32, c_p, c_p, c_p, c_sz, c_p]),
    "sa_cache_write": (c_i32, [c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_i32, c_p, c_p, c_p]),
    "sa_layer_stack_workspace_size": (c_sz, [c_i32, c_i64, c_i32]),
    "sa_layer_stack": (c_i32, [ctypes.POINTER(LayerDesc), c_i32, ctypes.POINTER(BatchDesc), c_i32, c_f32, c_p,
                               c_sz, ctypes.POINTER(StageEvents), c_p]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_relu_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class SparseMLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.sa_last_error_message().decode()
        super().__init__(f"{fn} failed with status {status} ({L.sa_status_string(status).decode()}): {msg}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != 0:
        raise SparseMLAError(fn, status)
