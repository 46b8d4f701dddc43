"""Seeded synthetic workloads for the compressed-KV decode path.

This module only draws random inputs and describes their shapes: it holds none of the
method's arithmetic, and it is the one module that both the oracle-side tests and the GPU
side use.  Random numbers that the method itself needs (the rotation) are drawn here and
passed in as inputs.

Seeds: stream s of workload c uses ``np.random.default_rng(1000 * c + s)`` on the host, or a
``torch.Generator`` seeded with the same number on the device:
    0 = K, 1 = V, 2 = q, 3 = rotation, 4 = outlier channels, 5 = spike positions,
    6 = sequence lengths, 7 = page permutation, 8 = Hadamard signs.

The five workloads mirror the pages' long-context decode setting with synthetic data (no
model weights or evaluation sets are used): a single head at 4k context with fp32 K/V;
a 7B-shaped 32-head layer at 8k with fp16 K/V and 4 outlier channels per head scaled by 8;
grouped-query attention (32 query / 8 KV heads) at 128k with batch 4 and 1% "spike"
tokens correlated with the query, decoded with adaptive Top-p 0.9; batched serving of 32
sequences with lengths uniform in [1024, 32768] in shuffled 256-token pages; and a
32768-token x 32-head prefill append with a randomized Hadamard rotation followed by a
1,048,576-token decode over 8 KV heads with Top-p 0.95.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

S_K, S_V, S_Q, S_ROT, S_OUTLIER, S_SPIKE, S_LEN, S_PERM, S_SIGNS = range(9)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    Hq: int
    Hkv: int
    L: int                       # context length (maximum, for variable lengths)
    D: int = 128
    kv_dtype: str = "f16"        # "f16" or "f32"
    rot: str = "dense"           # "dense" or "hadamard"
    Gv: int = 32                 # value group
    P: int = 256                 # page size in tokens
    top_p: float = 1.0           # >= 1 means full softmax
    len_range: Optional[Tuple[int, int]] = None  # variable lengths, uniform, inclusive
    shuffle_pages: bool = False
    outlier_channels: int = 0
    outlier_scale: float = 8.0
    spike_frac: float = 0.0
    spike_gamma: float = 2.83
    append_tokens: int = 0       # prefill-append workload (n_new) ...
    append_heads: int = 0        # ... over this many KV heads

    def seed(self, stream: int) -> int:
        return 1000 * self.index + stream

    def rng(self, stream: int) -> np.random.Generator:
        return np.random.default_rng(self.seed(stream))

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv


CONFIGS = [
    Workload("single-head-4k-fp32", 0, B=1, Hq=1, Hkv=1, L=4096, kv_dtype="f32", rot="dense", Gv=32),
    Workload("7b-layer-32h-8k-outliers", 1, B=1, Hq=32, Hkv=32, L=8192, kv_dtype="f16", rot="dense",
             Gv=32, outlier_channels=4, outlier_scale=8.0),
    Workload("gqa-32q8kv-128k-b4-spikes-topp0.9", 2, B=4, Hq=32, Hkv=8, L=131072, kv_dtype="f16",
             rot="dense", Gv=32, top_p=0.9, spike_frac=0.01, spike_gamma=2.83),
    Workload("batched-32x32h-len1k-32k-paged256-g64", 3, B=32, Hq=32, Hkv=32, L=32768, kv_dtype="f16",
             rot="dense", Gv=64, P=256, len_range=(1024, 32768), shuffle_pages=True),
    Workload("hadamard-append32k-decode1m-8kv-topp0.95", 4, B=1, Hq=32, Hkv=8, L=1048576,
             kv_dtype="f16", rot="hadamard", Gv=32, top_p=0.95, append_tokens=32768, append_heads=32),
]


# ----------------------------------------------------------------------------------------
# Rotation draws
# ----------------------------------------------------------------------------------------
def haar_orthogonal(rng: np.random.Generator, D: int) -> np.ndarray:
    """A Haar-distributed D x D orthogonal matrix (float64): QR of a Gaussian matrix with the
    signs of R's diagonal moved into Q (sign(0) taken as +1)."""
    G = rng.standard_normal((D, D))
    Q, R = np.linalg.qr(G)
    d = np.sign(np.diag(R))
    d[d == 0] = 1.0
    return Q * d[None, :]


def haar_orthogonal_batch(rng: np.random.Generator, n: int, D: int) -> np.ndarray:
    G = rng.standard_normal((n, D, D))
    Q, R = np.linalg.qr(G)
    d = np.sign(np.diagonal(R, axis1=1, axis2=2))
    d[d == 0] = 1.0
    return Q * d[:, None, :]


def draw_rotation(wl: Workload):
    """Returns ("dense", R16 float16 D x D) or ("hadamard", signs uint32 D/32)."""
    if wl.rot == "dense":
        return "dense", haar_orthogonal(wl.rng(S_ROT), wl.D).astype(np.float16)
    signs = wl.rng(S_SIGNS).integers(0, 2**32, size=wl.D // 32, dtype=np.uint64).astype(np.uint32)
    return "hadamard", signs


# ----------------------------------------------------------------------------------------
# Lengths and pages
# ----------------------------------------------------------------------------------------
def draw_seq_lens(wl: Workload) -> np.ndarray:
    if wl.len_range is None:
        return np.full(wl.B, wl.L, dtype=np.int32)
    lo, hi = wl.len_range
    return wl.rng(S_LEN).integers(lo, hi, size=wl.B, endpoint=True).astype(np.int32)


def page_layout(wl: Workload, seq_lens: np.ndarray, reserve: int = 0):
    """(page_table int32 [B][max_pages], num_pages).  Each sequence gets ceil((len+reserve)/P)
    pages; with shuffle_pages the physical page ids are a seeded permutation of the pool."""
    P = wl.P
    need = [(int(l) + reserve + P - 1) // P for l in seq_lens]
    max_pages = max(1, max(need))
    pool = sum(need)
    ids = np.arange(pool, dtype=np.int32)
    if wl.shuffle_pages:
        ids = wl.rng(S_PERM).permutation(pool).astype(np.int32)
    pt = np.zeros((wl.B, max_pages), dtype=np.int32)
    o = 0
    for b, n in enumerate(need):
        pt[b, :n] = ids[o:o + n]
        o += n
    return pt, max(pool, 1)


# ----------------------------------------------------------------------------------------
# Host (numpy) draws, for sizes the oracle can handle
# ----------------------------------------------------------------------------------------
def draw_host(wl: Workload, L: Optional[int] = None):
    """K, V (B, L, Hkv, D) in the workload's dtype, q (B, Hq, D) float32, seq_lens."""
    L = wl.L if L is None else L
    seq_lens = np.minimum(draw_seq_lens(wl), L).astype(np.int32)
    kvt = np.float16 if wl.kv_dtype == "f16" else np.float32
    q = wl.rng(S_Q).standard_normal((wl.B, wl.Hq, wl.D)).astype(np.float32)
    K = wl.rng(S_K).standard_normal((wl.B, L, wl.Hkv, wl.D))
    V = wl.rng(S_V).standard_normal((wl.B, L, wl.Hkv, wl.D))
    if wl.outlier_channels:
        r = wl.rng(S_OUTLIER)
        for h in range(wl.Hkv):
            ch = r.choice(wl.D, wl.outlier_channels, replace=False)
            K[:, :, h, ch] *= wl.outlier_scale
            V[:, :, h, ch] *= wl.outlier_scale
    if wl.spike_frac > 0:
        r = wl.rng(S_SPIKE)
        n = int(math.ceil(wl.spike_frac * L))
        G = wl.group
        for b in range(wl.B):
            for h in range(wl.Hkv):
                pos = r.choice(L, n, replace=False)
                qbar = q[b, h * G:(h + 1) * G].astype(np.float64).mean(axis=0)
                K[b, pos, h, :] += wl.spike_gamma * qbar[None, :]
    return K.astype(kvt), V.astype(kvt), q, seq_lens


# ----------------------------------------------------------------------------------------
# Device (torch) draws, for full sizes
# ----------------------------------------------------------------------------------------
def draw_device(wl: Workload, device, L: Optional[int] = None, Hkv: Optional[int] = None,
                B: Optional[int] = None):
    """Same recipe as draw_host, drawn by torch's seeded device generator (different numbers
    from the host draw; identical between runs)."""
    import torch

    L = wl.L if L is None else L
    Hkv = wl.Hkv if Hkv is None else Hkv
    B = wl.B if B is None else B
    kvt = torch.float16 if wl.kv_dtype == "f16" else torch.float32

    def gen(stream):
        g = torch.Generator(device=device)
        g.manual_seed(wl.seed(stream))
        return g

    q = torch.randn((B, wl.Hq, wl.D), generator=gen(S_Q), device=device, dtype=torch.float32)
    K = torch.randn((B, L, Hkv, wl.D), generator=gen(S_K), device=device, dtype=torch.float32)
    K = K.to(kvt) if wl.spike_frac == 0 and not wl.outlier_channels else K
    V = torch.randn((B, L, Hkv, wl.D), generator=gen(S_V), device=device, dtype=torch.float32)
    if wl.outlier_channels:
        r = wl.rng(S_OUTLIER)
        for h in range(Hkv):
            ch = torch.as_tensor(r.choice(wl.D, wl.outlier_channels, replace=False), device=device)
            K[:, :, h, ch] *= wl.outlier_scale
            V[:, :, h, ch] *= wl.outlier_scale
    if wl.spike_frac > 0:
        g = gen(S_SPIKE)
        n = int(math.ceil(wl.spike_frac * L))
        G = wl.Hq // Hkv
        for b in range(B):
            for h in range(Hkv):
                pos = torch.randperm(L, generator=g, device=device)[:n]
                qbar = q[b, h * G:(h + 1) * G].double().mean(dim=0).float()
                K[b, pos, h, :] += wl.spike_gamma * qbar[None, :]
    return K.to(kvt).contiguous(), V.to(kvt).contiguous(), q.contiguous()
