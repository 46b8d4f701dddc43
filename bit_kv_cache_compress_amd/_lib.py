"""ctypes binding of libkvcompress.so (the C ABI declared in include/kv_compress.h).

Only argument marshalling lives here.  The library must have been built in-tree
(``python -m bit_kv_cache_compress_amd.build``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvcompress.so")

KV_OK, KV_ERR_ARG, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE, KV_ERR_HIP = 0, -1, -2, -3, -4
KV_ROT_DENSE, KV_ROT_HADAMARD = 0, 1
KV_F16, KV_F32 = 0, 1

EXPORTS = ("kv_compress_append", "kv_decode_attend", "kv_decode_attend_ex", "kv_decode_attend_noalloc",
           "kv_decode_attend_tail",
           "kv_decode_workspace_bytes", "kv_workspace_bytes", "kv_hp_update",
           "kv_tail_append", "kv_tail_retire", "kv_topp_select", "kv_topp_workspace_bytes", "kv_last_error",
           "kv_version")


class KVCacheDesc(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("value_group", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("rot_kind", ctypes.c_int32),
        ("rot", ctypes.c_void_p),
        ("keys", ctypes.c_void_p),
        ("vals", ctypes.c_void_p),
        ("keys_f16", ctypes.c_void_p),
        ("key_center", ctypes.c_void_p),
        ("sketch_dim", ctypes.c_int32),
    ]


class KVDebug(ctypes.Structure):
    _fields_ = [
        ("q_codes", ctypes.c_void_p),
        ("q_params", ctypes.c_void_p),
        ("q_sumu", ctypes.c_void_p),
        ("iscores", ctypes.c_void_p),
        ("scores", ctypes.c_void_p),
        ("sel_count", ctypes.c_void_p),
        ("sel_idx", ctypes.c_void_p),
        ("sel_bins", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
        ("bin_dist", ctypes.c_void_p),
        ("chunk_top", ctypes.c_void_p),
    ]


class KVTailDesc(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("len", ctypes.c_void_p),
        ("capacity", ctypes.c_int32),
        ("mass", ctypes.c_void_p),
    ]


class KVHpDesc(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("saved", ctypes.c_void_p),
        ("mass", ctypes.c_void_p),
        ("capacity", ctypes.c_int32),
    ]


class KVAppendArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("n_new", ctypes.c_int32),
        ("start_pos", ctypes.c_void_p),
    ]


class KVDecodeOpts(ctypes.Structure):
    _fields_ = [
        ("tail", ctypes.POINTER(KVTailDesc)),
        ("q_dither", ctypes.c_void_p),
        ("hp", ctypes.POINTER(KVHpDesc)),
        ("append", ctypes.POINTER(KVAppendArgs)),
    ]


STAGES = ("query", "score", "hist", "select", "attend", "merge")


class KVCompressError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libkvcompress error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    """Loads the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_kv_cache_compress_amd.build` "
                          "(there is no fallback path)")
    # torch ships its own HIP runtime; loading torch first makes the library bind to that
    # same runtime instance (one HIP runtime per process, shared streams and events)
    import torch  # noqa: F401

    L = ctypes.CDLL(LIB_PATH)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.kv_compress_append.argtypes = [ctypes.POINTER(KVCacheDesc), i32, P, P, i32, i32, P, P, i32, P]
    L.kv_compress_append.restype = ctypes.c_int
    L.kv_decode_attend.argtypes = [ctypes.POINTER(KVCacheDesc), P, i32, i32, P, i32, P, i32, f32, P,
                                   ctypes.POINTER(KVDebug), P, sz, P]
    L.kv_decode_attend.restype = ctypes.c_int
    L.kv_decode_attend_tail.argtypes = [ctypes.POINTER(KVCacheDesc), ctypes.POINTER(KVTailDesc), P, i32, i32, P, i32,
                                        P, i32, f32, P, ctypes.POINTER(KVDebug), P, sz, P]
    L.kv_decode_attend_tail.restype = ctypes.c_int
    L.kv_decode_attend_ex.argtypes = [ctypes.POINTER(KVCacheDesc), ctypes.POINTER(KVDecodeOpts), P, i32, i32, P, i32,
                                      P, i32, f32, P, ctypes.POINTER(KVDebug), P, sz, P]
    L.kv_decode_attend_ex.restype = ctypes.c_int
    L.kv_decode_attend_noalloc.argtypes = [ctypes.POINTER(KVCacheDesc), ctypes.POINTER(KVDecodeOpts), P, i32, i32, P,
                                           i32, P, i32, f32, P, ctypes.POINTER(KVDebug), P]
    L.kv_decode_attend_noalloc.restype = ctypes.c_int
    L.kv_hp_update.argtypes = [ctypes.POINTER(KVCacheDesc), ctypes.POINTER(KVHpDesc), ctypes.POINTER(KVTailDesc), i32,
                               i32, P, P, i32, P]
    L.kv_hp_update.restype = ctypes.c_int
    L.kv_tail_append.argtypes = [ctypes.POINTER(KVTailDesc), i32, i32, i32, P, P, i32, i32, P]
    L.kv_tail_append.restype = ctypes.c_int
    L.kv_tail_retire.argtypes = [ctypes.POINTER(KVTailDesc), i32, i32, i32, i32, P, P]
    L.kv_tail_retire.restype = ctypes.c_int
    L.kv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, f32]
    L.kv_decode_workspace_bytes.restype = sz
    L.kv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, f32]
    L.kv_workspace_bytes.restype = sz
    L.kv_topp_select.argtypes = [P, i32, P, i32, i32, i32, f32, P, P, P, sz, P]
    L.kv_topp_select.restype = ctypes.c_int
    L.kv_topp_workspace_bytes.argtypes = [i32, i32, i32]
    L.kv_topp_workspace_bytes.restype = sz
    L.kv_last_error.argtypes = []
    L.kv_last_error.restype = ctypes.c_char_p
    L.kv_version.argtypes = []
    L.kv_version.restype = ctypes.c_int
    _lib = L
    return L


def check(rc: int):
    if rc != KV_OK:
        raise KVCompressError(rc, lib().kv_last_error().decode())
    return rc


def last_error() -> str:
    return lib().kv_last_error().decode()
