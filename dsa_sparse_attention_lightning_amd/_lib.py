"""ctypes declarations of libdsa_indexcache.so (the C ABI in include/dsa_indexcache.h)."""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa_indexcache.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "dsa_indexcache.h")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_BF16, DSA_FP8_E4M3 = 0, 1
DSA_PROXY_OUTPUT, DSA_PROXY_MISS = 0, 1
DSA_PROBE_TILES, DSA_PROBE_STRIDE = 0, 1
STATUS_NAMES = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
                3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}

c_int, c_i64, c_f32, c_vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
c_size_p = ctypes.POINTER(ctypes.c_size_t)


class Layer(ctypes.Structure):
    _fields_ = [("q_idx", c_vp), ("q_idx_scale", c_vp), ("w", c_vp), ("k_idx", c_vp),
                ("k_idx_scale", c_vp), ("q", c_vp), ("kv", c_vp), ("out", c_vp), ("lse", c_vp)]


class StackShape(ctypes.Structure):
    _fields_ = [("B", c_int), ("T", c_int), ("H", c_int), ("D", c_int), ("Lmax", c_int),
                ("k", c_int), ("Hq", c_int), ("d_qk", c_int), ("d_v", c_int),
                ("idx_dtype", c_int), ("scale", c_f32), ("flags", c_int)]

DSA_STACK_UNFUSED_TOPK = 1
DSA_NOALLOC_SCRATCH_BYTES = 64 << 20


class StackStats(ctypes.Structure):
    _fields_ = [("n_indexer_calls", c_int), ("n_topk_calls", c_int), ("n_attn_calls", c_int)]


SIGNATURES = {
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_version": (ctypes.c_char_p, []),
    "dsa_indexer_scores": (c_int, [c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                   c_int, c_int, c_vp, c_i64, c_vp]),
    "dsa_topk_workspace_size": (c_int, [c_int, c_int, c_int, c_int, c_size_p]),
    "dsa_topk": (c_int, [c_vp, c_i64, c_vp, c_int, c_int, c_int, c_int, c_vp, c_vp,
                         ctypes.c_size_t, c_vp]),
    "dsa_indexer_topk_workspace_size": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                                c_size_p]),
    "dsa_indexer_topk": (c_int, [c_vp, c_int, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                 c_int, c_int, c_int, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "dsa_sparse_attn_workspace_size": (c_int, [c_int, c_int, c_int, c_int, c_int, c_size_p]),
    "dsa_sparse_attn": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                c_int, c_f32, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "dsa_kv_append": (c_int, [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_vp,
                              c_vp, c_vp, c_vp]),
    "dsa_probe_stream_read": (c_int, [c_vp, c_i64, c_int, c_int, c_vp, c_vp]),
    "indexcache_stack_workspace_size": (c_int, [ctypes.POINTER(StackShape), c_size_p]),
    "indexcache_stack_fuses_topk": (c_int, [ctypes.POINTER(StackShape),
                                            ctypes.POINTER(ctypes.c_int)]),
    "indexcache_run_stack": (c_int, [ctypes.c_char_p, c_int, ctypes.POINTER(Layer),
                                     ctypes.POINTER(StackShape), c_vp, c_vp, c_vp, c_i64, c_vp,
                                     ctypes.c_size_t, ctypes.POINTER(StackStats), c_vp]),
    "indexcache_run_stack_noalloc": (c_int, [ctypes.c_char_p, c_int, ctypes.POINTER(Layer),
                                             ctypes.POINTER(StackShape), c_vp, c_vp, c_vp, c_i64,
                                             ctypes.POINTER(StackStats), c_vp]),
    "indexcache_reuse_costs_workspace_size": (c_int, [ctypes.POINTER(StackShape), c_int, c_int,
                                                      c_size_p]),
    "indexcache_reuse_costs": (c_int, [c_int, ctypes.POINTER(Layer), ctypes.POINTER(StackShape),
                                       c_vp, c_int, c_vp, c_vp, c_i64, c_vp, ctypes.c_size_t,
                                       c_vp]),
    "indexcache_pattern_cost": (c_int, [c_vp, c_int, ctypes.c_char_p,
                                        ctypes.POINTER(ctypes.c_double)]),
    "indexcache_greedy_search": (c_int, [c_vp, c_int, c_int, c_vp, c_vp]),
}

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m dsa_sparse_attention_lightning_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
        return lib


class DSAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int) -> None:
    if status != DSA_OK:
        raise DSAError(status, load().dsa_last_error().decode(errors="replace"))
