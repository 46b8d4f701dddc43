"""Decode attention over a 1-bit-key / 4-bit-value compressed KV cache on AMD Instinct
MI355X (gfx950).

The computation lives in libkvcompress.so (hand-written HIP kernels behind the C ABI of
include/kv_compress.h); this package is its thin PyTorch binding.
"""
from ._lib import (KV_ERR_ARG, KV_ERR_HIP, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE, KV_OK, KVCompressError,  # noqa: F401
                   LIB_PATH, lib)
from .api import (HEAD_DIM, DecodeDebug, HPTier, KVCache, StageTimer, Tail, append, decode_attend,  # noqa: F401
                  decode_workspace_bytes, topp_select, topp_workspace_bytes)

__all__ = ["KVCache", "Tail", "HPTier", "append", "decode_attend", "topp_select", "decode_workspace_bytes",
           "topp_workspace_bytes", "DecodeDebug", "KVCompressError", "lib", "LIB_PATH", "HEAD_DIM"]
