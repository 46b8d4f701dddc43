"""PyTorch-facing wrappers of the C ABI: shape and dtype checks, device pointers, the
current HIP stream, and allocation of outputs/workspace with torch.  Every step of the
computation runs in the library's HIP kernels."""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib as L
from ._lib import lib

HEAD_DIM = 128


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class KVCache:
    """Paged packed cache (device memory owned by torch tensors).

    Token t of sequence b lives in physical page ``page_table[b][t // page_size]``, slot
    ``t % page_size``.  Two arrays of records (per page, KV head, slot): ``keys`` int32
    [..., 5] = 4 sign words and the binary16 norm | binary16 correction << 16 word; ``vals``
    uint8 [..., 64 + 4 * 128 / value_group] = 64 bytes of 4-bit codes, then one binary16
    scale | binary16 zero << 16 word per value group.  ``key_bits``, ``key_nc``,
    ``val_codes`` and ``val_sz`` are views of the fields.

    ``rotation``: dense -> float16 [128, 128] orthogonal matrix; hadamard -> 4 uint32 sign
    words (given as an int32 or uint32 array/tensor).

    ``exact_keys``: also keep the keys in binary16 (``keys_f16`` [..., 128]); appends fill
    it, and a Top-p decode then scores the selected tokens exactly with it.  ``proxy_desc``
    is the descriptor without it (proxy scores throughout).

    ``sketch_dim``: sign bits per key, 128 (the whole rotation) or 64 (a narrow sketch of
    the first 64 rotated coordinates, 12-byte key records).

    ``key_center``: optional float32 [Hkv, 128] per-head key centers (kept on the device as
    ``key_center``).  Appends encode k - c_h instead of k; the proxy scores then estimate
    <q, k - c_h>, a per-head shift that the softmax ignores (tails are moved to that frame).
    """

    def __init__(self, num_pages: int, num_kv_heads: int, rotation, rot_kind: str = "dense",
                 page_size: int = 256, value_group: int = 32, device="cuda", exact_keys: bool = False,
                 key_center=None, sketch_dim: int = HEAD_DIM):
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = device
        D = HEAD_DIM
        self.num_pages, self.num_kv_heads = int(num_pages), int(num_kv_heads)
        self.page_size, self.value_group = int(page_size), int(value_group)
        self.rot_kind = L.KV_ROT_DENSE if rot_kind == "dense" else L.KV_ROT_HADAMARD
        if self.rot_kind == L.KV_ROT_DENSE:
            r = torch.as_tensor(rotation)
            if r.dtype != torch.float16 or tuple(r.shape) != (D, D):
                raise ValueError("dense rotation must be a float16 [128, 128] matrix")
            self.rot = r.to(device).contiguous()
        else:
            r = torch.as_tensor(rotation.astype("int64") if hasattr(rotation, "astype") else rotation)
            r = r.to(torch.int64)
            if r.numel() != D // 32:
                raise ValueError("hadamard rotation must hold 4 sign words")
            r = torch.where(r >= 2**31, r - 2**32, r).to(torch.int32)
            self.rot = r.to(device).contiguous()
        if sketch_dim not in (HEAD_DIM, 64):
            raise ValueError("sketch_dim must be 128 or 64")
        self.sketch_dim = int(sketch_dim)
        shp = (self.num_pages, self.num_kv_heads, self.page_size)
        self.keys = torch.zeros(shp + (self.sketch_dim // 32 + 1,), dtype=torch.int32, device=device)
        self.vals = torch.zeros(shp + (D // 2 + 4 * (D // self.value_group),), dtype=torch.uint8, device=device)
        self.keys_f16 = torch.zeros(shp + (D,), dtype=torch.float16, device=device) if exact_keys else None
        self.key_center = None
        if key_center is not None:
            kc = torch.as_tensor(key_center)
            if kc.dtype != torch.float32 or tuple(kc.shape) != (self.num_kv_heads, D):
                raise ValueError(f"key_center must be a float32 [{self.num_kv_heads}, {D}] array")
            self.key_center = kc.to(device).contiguous()
        kcp = self.key_center.data_ptr() if self.key_center is not None else None
        self.desc = L.KVCacheDesc(D, self.num_kv_heads, self.value_group, self.page_size, self.num_pages,
                                  self.rot_kind, self.rot.data_ptr(), self.keys.data_ptr(), self.vals.data_ptr(),
                                  self.keys_f16.data_ptr() if exact_keys else None, kcp, self.sketch_dim)
        self.proxy_desc = L.KVCacheDesc(D, self.num_kv_heads, self.value_group, self.page_size, self.num_pages,
                                        self.rot_kind, self.rot.data_ptr(), self.keys.data_ptr(),
                                        self.vals.data_ptr(), None, kcp, self.sketch_dim)

    @property
    def key_bits(self) -> torch.Tensor:
        return self.keys[..., :self.sketch_dim // 32]

    @property
    def key_nc(self) -> torch.Tensor:
        return self.keys[..., self.sketch_dim // 32]

    @property
    def val_codes(self) -> torch.Tensor:
        return self.vals[..., :HEAD_DIM // 2]

    @property
    def val_sz(self) -> torch.Tensor:
        return self.vals[..., HEAD_DIM // 2:].view(torch.int32)

    def nbytes(self) -> int:
        return self.keys.numel() * 4 + self.vals.numel() + (0 if self.keys_f16 is None else self.keys_f16.numel() * 2)


def _append_args(cache: KVCache, k: torch.Tensor, v: torch.Tensor, start_pos: torch.Tensor, B=None):
    """Checks the new tokens of an append -> (dtype, k, v, n_new, start_pos) for the C ABI."""
    dev = cache.device
    if k.dim() != 4 or k.shape[2] != cache.num_kv_heads or k.shape[3] != HEAD_DIM:
        raise ValueError(f"k must be [B, n_new, {cache.num_kv_heads}, {HEAD_DIM}], got {tuple(k.shape)}")
    if B is not None and k.shape[0] != B:
        raise ValueError(f"k must have the decode's batch of {B}")
    dtype = {torch.float16: L.KV_F16, torch.float32: L.KV_F32}.get(k.dtype)
    if dtype is None:
        raise TypeError("k, v must be float16 or float32")
    _need(k, "k", k.dtype, dev)
    _need(v, "v", k.dtype, dev, k.shape)
    _need(start_pos, "start_pos", torch.int32, dev, (int(k.shape[0]),))
    return dtype, _ptr(k), _ptr(v), int(k.shape[1]), _ptr(start_pos)


def append(cache: KVCache, k: torch.Tensor, v: torch.Tensor, start_pos: torch.Tensor,
           page_table: torch.Tensor) -> None:
    """Encodes k, v [B, n_new, Hkv, 128] (float16 or float32) at positions start_pos[b] + i."""
    dev = cache.device
    dtype, _, _, n_new, _ = _append_args(cache, k, v, start_pos)
    B = int(k.shape[0])
    _need(page_table, "page_table", torch.int32, dev)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    L.check(L.lib().kv_compress_append(ctypes.byref(cache.desc), dtype, _ptr(k), _ptr(v), B, n_new, _ptr(start_pos),
                                       _ptr(page_table), int(page_table.shape[1]), _stream(dev)))


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, max_seq_len: int, top_p: float = 1.0) -> int:
    n = L.lib().kv_decode_workspace_bytes(B, Hq, Hkv, max_seq_len, HEAD_DIM, float(top_p))
    if n == 0:
        raise ValueError(L.last_error() or "invalid decode shape")
    return int(n)


@dataclass
class DecodeDebug:
    """Intermediate outputs of one decode step (stage-wise checks)."""
    q_codes: torch.Tensor
    q_params: torch.Tensor
    q_sumu: torch.Tensor
    iscores: Optional[torch.Tensor]
    scores: Optional[torch.Tensor]
    sel_count: Optional[torch.Tensor] = None
    sel_idx: Optional[torch.Tensor] = None
    sel_bins: Optional[torch.Tensor] = None
    bin_dist: Optional[torch.Tensor] = None
    chunk_top: Optional[torch.Tensor] = None

    @staticmethod
    def allocate(B, Hq, ld, topp: bool, device, scores: bool = True, dist: bool = False) -> "DecodeDebug":
        """Debug outputs of one decode.  scores=False leaves out the per-token scores, so the
        decode runs the same score kernels as without debug output.  dist=True (Top-p) also
        returns what the score pass wrote: bin_dist uint16 [B, Hq, ld] (returned as int32
        bits of an int16 tensor) and chunk_top int32 [B, Hq, ceil(ld / 512)]."""
        z = lambda *s, dt=torch.int32: torch.zeros(s, dtype=dt, device=device)
        dist = dist and topp
        return DecodeDebug(q_codes=z(B, Hq, HEAD_DIM, dt=torch.uint8), q_params=z(B, Hq, 4, dt=torch.float32),
                           q_sumu=z(B, Hq), iscores=z(B, Hq, ld) if scores else None,
                           scores=z(B, Hq, ld, dt=torch.float32) if scores else None,
                           sel_count=z(B, Hq) if topp else None, sel_idx=z(B, Hq, ld) - 1 if topp else None,
                           sel_bins=z(B, Hq, 2) if topp else None,
                           bin_dist=z(B, Hq, ld, dt=torch.int16) if dist else None,
                           chunk_top=z(B, Hq, (ld + 511) // 512) if dist else None)

    def struct(self) -> L.KVDebug:
        ptrs = [None if t is None else t.data_ptr() for t in
                (self.q_codes, self.q_params, self.q_sumu, self.iscores, self.scores, self.sel_count, self.sel_idx,
                 self.sel_bins)]
        return L.KVDebug(*ptrs, None, *[None if t is None else t.data_ptr() for t in (self.bin_dist, self.chunk_top)])


def _loaded_hip_runtime() -> str:
    """Path of the HIP runtime already mapped into this process (the one torch and the
    library use); opening another copy would create a second, separate runtime."""
    lib().kv_version()  # make sure the library and its HIP runtime are loaded
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1]
            if "libamdhip64.so" in path:
                return path
    raise RuntimeError("no HIP runtime is mapped in this process")


class StageTimer:
    """HIP events that the library records around each decode stage (kv_debug.stage_events).
    Pass ``timer.struct()`` as ``debug_struct`` to decode_attend; read ``timer.elapsed_ms()``
    after synchronizing."""

    def __init__(self):
        self._hip = ctypes.CDLL(_loaded_hip_runtime())
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipGetLastError.argtypes = []
        n = 2 * len(L.STAGES)
        self.events = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events[i] = ev
        self._dbg = L.KVDebug(None, None, None, None, None, None, None, None,
                              ctypes.cast(self.events, ctypes.c_void_p))

    def struct(self) -> L.KVDebug:
        return self._dbg

    def elapsed_ms(self, stages=None) -> dict:
        """Elapsed time of each recorded stage (pass the names of the stages the call ran;
        events of stages that never ran must not be queried)."""
        out = {}
        for s, name in enumerate(L.STAGES):
            if stages is not None and name not in stages:
                continue
            a, b = self.events[2 * s], self.events[2 * s + 1]
            ms = ctypes.c_float(0.0)
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0:
                out[name] = float(ms.value)
        self._hip.hipGetLastError()  # leave no error state behind for the next HIP call
        return out


def decode_attend(cache: KVCache, q: torch.Tensor, seq_lens: torch.Tensor, page_table: torch.Tensor,
                  top_p: float = 1.0, max_seq_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, debug: Optional[DecodeDebug] = None,
                  debug_struct: Optional[L.KVDebug] = None, proxy: bool = False,
                  tail: Optional["Tail"] = None, q_dither: Optional[torch.Tensor] = None,
                  hp: Optional["HPTier"] = None, append: Optional[tuple] = None,
                  noalloc: bool = False) -> torch.Tensor:
    """One decode step: q [B, Hq, 128] float32 -> out [B, Hq, 128] float32.  Under Top-p, a
    cache with binary16 keys scores the selected tokens exactly unless ``proxy`` is set.
    With ``tail``, each sequence's binary16 tail tokens follow its seq_lens compressed ones.
    ``q_dither`` (float32 [B, Hq, 128], uniforms in [0, 1)): stochastic rounding of the int4
    query codes, floor(t + U) instead of rint(t).  ``hp``: the high-precision tier, attended
    exactly next to the tail; the tail (created with mass=True) and the tier accumulate mass.
    ``append`` = (k, v, start_pos): new tokens written into the cache first, as ``append``
    would write them (seq_lens must count them), inside the decode's first launch.
    ``noalloc``: run kv_decode_attend_noalloc, whose workspace is the library's static
    per-device array (``workspace`` must then be None; pass ``out`` to allocate nothing)."""
    dev = cache.device
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be [B, Hq, {HEAD_DIM}]")
    _need(q, "q", torch.float32, dev)
    B, Hq = int(q.shape[0]), int(q.shape[1])
    _need(seq_lens, "seq_lens", torch.int32, dev, (B,))
    _need(page_table, "page_table", torch.int32, dev)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B, max_pages]")
    max_pages = int(page_table.shape[1])
    if max_seq_len is None:
        max_seq_len = max_pages * cache.page_size
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, (B, Hq, HEAD_DIM))
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc decodes use the library's static workspace")
    else:
        need = decode_workspace_bytes(B, Hq, cache.num_kv_heads, max_seq_len, top_p)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _need(workspace, "workspace", torch.uint8, dev)
    if debug is not None:
        debug_struct = debug.struct()
    dbg = ctypes.byref(debug_struct) if debug_struct is not None else None
    desc = cache.proxy_desc if proxy else cache.desc
    if tail is not None and (tail.k.shape[0] != B or tail.k.shape[2] != cache.num_kv_heads):
        raise ValueError(f"tail must be [{B}, capacity, {cache.num_kv_heads}, {HEAD_DIM}]")
    if hp is not None and (hp.B != B or hp.num_kv_heads != cache.num_kv_heads):
        raise ValueError(f"tier must be [{B}, {cache.num_kv_heads}, capacity]")
    app = None
    if append is not None:
        ak, av, asp = append
        app = L.KVAppendArgs(*_append_args(cache, ak, av, asp, B))
    if noalloc or q_dither is not None or hp is not None or app is not None:
        if q_dither is not None:
            _need(q_dither, "q_dither", torch.float32, dev, (B, Hq, HEAD_DIM))
        opts = L.KVDecodeOpts(ctypes.pointer(tail.desc) if tail is not None else None,
                              _ptr(q_dither) if q_dither is not None else None,
                              ctypes.pointer(hp.desc) if hp is not None else None,
                              ctypes.pointer(app) if app is not None else None)
        if noalloc:
            L.check(L.lib().kv_decode_attend_noalloc(ctypes.byref(desc), ctypes.byref(opts), _ptr(q), B, Hq,
                                                     _ptr(seq_lens), int(max_seq_len), _ptr(page_table), max_pages,
                                                     float(top_p), _ptr(out), dbg, _stream(dev)))
        else:
            L.check(L.lib().kv_decode_attend_ex(ctypes.byref(desc), ctypes.byref(opts), _ptr(q), B, Hq,
                                                _ptr(seq_lens), int(max_seq_len), _ptr(page_table), max_pages,
                                                float(top_p), _ptr(out), dbg, _ptr(workspace), workspace.numel(),
                                                _stream(dev)))
    elif tail is None:
        L.check(L.lib().kv_decode_attend(ctypes.byref(desc), _ptr(q), B, Hq, _ptr(seq_lens), int(max_seq_len),
                                         _ptr(page_table), max_pages, float(top_p), _ptr(out), dbg,
                                         _ptr(workspace), workspace.numel(), _stream(dev)))
    else:
        L.check(L.lib().kv_decode_attend_tail(ctypes.byref(desc), ctypes.byref(tail.desc), _ptr(q), B, Hq,
                                              _ptr(seq_lens), int(max_seq_len), _ptr(page_table), max_pages,
                                              float(top_p), _ptr(out), dbg, _ptr(workspace), workspace.numel(),
                                              _stream(dev)))
    return out


class Tail:
    """Binary16 tail of uncompressed recent tokens (device memory owned by torch tensors):
    ``k``, ``v`` float16 [B, capacity, Hkv, 128] (token j of sequence b's tail at [b, j]),
    ``len`` int32 [B].  ``page(b, j, n)`` views tokens j .. j+n-1 of sequence b's tail as the
    [1, n, Hkv, 128] input of ``append`` (to compress them into the cache)."""

    def __init__(self, B: int, capacity: int, num_kv_heads: int, device="cuda", mass: bool = False):
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = device
        self.B, self.num_kv_heads = int(B), int(num_kv_heads)
        self.k = torch.zeros((B, capacity, num_kv_heads, HEAD_DIM), dtype=torch.float16, device=device)
        self.v = torch.zeros_like(self.k)
        self.len = torch.zeros(B, dtype=torch.int32, device=device)
        self.capacity = int(capacity)
        # attention mass per (sequence, tail token, KV head), for the high-precision tier
        self.mass = torch.zeros((B, capacity, num_kv_heads), dtype=torch.float32, device=device) if mass else None
        self.desc = L.KVTailDesc(self.k.data_ptr(), self.v.data_ptr(), self.len.data_ptr(), self.capacity,
                                 self.mass.data_ptr() if mass else None)

    def page(self, b: int, j: int, n: int):
        return self.k[b:b + 1, j:j + n], self.v[b:b + 1, j:j + n]

    def append(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """Writes k, v [B, n_new, Hkv, 128] (float16 or float32) after each sequence's tail."""
        if k.dim() != 4 or k.shape[0] != self.B or k.shape[2] != self.num_kv_heads or k.shape[3] != HEAD_DIM:
            raise ValueError(f"k must be [{self.B}, n_new, {self.num_kv_heads}, {HEAD_DIM}]")
        dtype = {torch.float16: L.KV_F16, torch.float32: L.KV_F32}.get(k.dtype)
        if dtype is None:
            raise TypeError("k, v must be float16 or float32")
        _need(k, "k", k.dtype, self.device)
        _need(v, "v", k.dtype, self.device, k.shape)
        L.check(L.lib().kv_tail_append(ctypes.byref(self.desc), self.num_kv_heads, HEAD_DIM, dtype, _ptr(k), _ptr(v),
                                       self.B, int(k.shape[1]), _stream(self.device)))

    def retire(self, n: int, seq_lens: Optional[torch.Tensor] = None) -> None:
        """Drops the first n tokens of every tail (after they were compressed into the cache)
        and adds n to seq_lens when given."""
        if seq_lens is not None:
            _need(seq_lens, "seq_lens", torch.int32, self.device, (self.B,))
        L.check(L.lib().kv_tail_retire(ctypes.byref(self.desc), self.num_kv_heads, HEAD_DIM, self.B, int(n),
                                       _ptr(seq_lens) if seq_lens is not None else None,
                                       _stream(self.device)))


class HPTier:
    """High-precision tier: per (sequence, KV head) up to ``capacity`` tokens kept in binary16
    (``k``, ``v`` float16 [B, Hkv, capacity, 128]), with their positions ``pos`` (int32, -1 =
    empty), the saved norm/correction words of their marked compressed records ``saved``
    and their accumulated attention mass ``mass`` (float32)."""

    def __init__(self, B: int, capacity: int, num_kv_heads: int, device="cuda"):
        device = torch.device(device)
        if device.type == "cuda" and device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        self.device = device
        self.B, self.num_kv_heads, self.capacity = int(B), int(num_kv_heads), int(capacity)
        shp = (B, num_kv_heads, capacity)
        self.k = torch.zeros(shp + (HEAD_DIM,), dtype=torch.float16, device=device)
        self.v = torch.zeros_like(self.k)
        self.pos = torch.full(shp, -1, dtype=torch.int32, device=device)
        self.saved = torch.zeros(shp, dtype=torch.int32, device=device)
        self.mass = torch.zeros(shp, dtype=torch.float32, device=device)
        self.desc = L.KVHpDesc(self.k.data_ptr(), self.v.data_ptr(), self.pos.data_ptr(), self.saved.data_ptr(),
                               self.mass.data_ptr(), self.capacity)

    def update(self, cache: "KVCache", tail: "Tail", n: int, seq_lens: torch.Tensor, page_table: torch.Tensor) -> None:
        """Promotion step after tail tokens 0..n-1 were compressed into ``cache`` (at positions
        seq_lens[b] + j) and before ``tail.retire(n)``."""
        if tail.mass is None:
            raise ValueError("the tail needs mass=True")
        _need(seq_lens, "seq_lens", torch.int32, self.device, (self.B,))
        _need(page_table, "page_table", torch.int32, self.device)
        L.check(L.lib().kv_hp_update(ctypes.byref(cache.desc), ctypes.byref(self.desc), ctypes.byref(tail.desc),
                                     self.B, int(n), _ptr(seq_lens), _ptr(page_table), int(page_table.shape[1]),
                                     _stream(self.device)))


def topp_workspace_bytes(B: int, Hq: int, ld: int) -> int:
    n = L.lib().kv_topp_workspace_bytes(B, Hq, ld)
    if n == 0:
        raise ValueError("invalid top-p shape")
    return int(n)


def topp_select(scores: torch.Tensor, seq_lens: torch.Tensor, top_p: float, head_dim: int = HEAD_DIM,
                workspace: Optional[torch.Tensor] = None):
    """Adaptive Top-p over scores [B, Hq, ld] -> (sel_idx [B, Hq, ld] ascending, padded
    with -1; sel_count [B, Hq])."""
    dev = scores.device
    _need(scores, "scores", torch.float32, dev)
    if scores.dim() != 3:
        raise ValueError("scores must be [B, Hq, ld]")
    B, Hq, ld = (int(x) for x in scores.shape)
    _need(seq_lens, "seq_lens", torch.int32, dev, (B,))
    sel_idx = torch.full((B, Hq, ld), -1, dtype=torch.int32, device=dev)
    sel_count = torch.zeros((B, Hq), dtype=torch.int32, device=dev)
    need = topp_workspace_bytes(B, Hq, ld)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    L.check(L.lib().kv_topp_select(_ptr(scores), ld, _ptr(seq_lens), B, Hq, head_dim, float(top_p), _ptr(sel_idx),
                                   _ptr(sel_count), _ptr(workspace), workspace.numel(), _stream(dev)))
    return sel_idx, sel_count
