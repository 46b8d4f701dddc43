"""Oracle for the compressed-KV decode path -- TEST INFRASTRUCTURE ONLY.

Plain, slow CPU reference of what the GPU library computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it; the
product package never does.  The arithmetic lives in ``kvc_oracle.c`` (built by
``oracle/build.py`` into ``oracle/libkvc_oracle.so``); this module only marshals numpy
arrays, and places per-token records into the paged cache layout and gathers them back.

Every function follows a passage of the pages (cited by title and section in the C file):
keys are stored as the sign bits of a random rotation with a binary16 norm and correction
("RaBitQCache" abstract; "H1B-KV" key design), values as per-group 4-bit linear codes
("H1B-KV" key design), scores come from binary x INT4 dot products ("RaBitQCache" key
design), an adaptive Top-p selects tokens ("RaBitQCache" abstract), and the output is the
softmax-weighted sum of the decoded 4-bit values ("H1B-KV" technical framework).  With the
keys also kept in binary16, the selected tokens are attended with exact scores <q, k>
("RaBitQCache" abstract: proxy scores that estimate the attention weights retrieve the set
for sparse attention); that path is plain numpy in binary64.

Parity pins: every function here is checked against something other than itself in
``tests/test_oracle_*.py`` (brute force, closed forms, library routines, statistics).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

ROT_DENSE = 0
ROT_HADAMARD = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkvc_oracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.orc_f16_from_f64.argtypes = [ctypes.c_double]
    lib.orc_f16_from_f64.restype = ctypes.c_uint16
    lib.orc_f64_from_f16.argtypes = [ctypes.c_uint16]
    lib.orc_f64_from_f16.restype = ctypes.c_double
    lib.orc_rotate_f64.argtypes = [i32, i32, P, P, P, i64, P]
    lib.orc_key_encode.argtypes = [i32, i32, i32, P, P, P, i64, P, P]
    lib.orc_value_encode.argtypes = [i32, i32, P, i64, P, P]
    lib.orc_query_encode.argtypes = [i32, i32, i32, P, P, P, i64, P, P, P, P, P]
    lib.orc_scores.argtypes = [i32, P, P, i64, P, f32, f32, P, P, P]
    lib.orc_kbin.argtypes = [i32]
    lib.orc_kbin.restype = f32
    lib.orc_bin.argtypes = [f32, f32]
    lib.orc_bin.restype = i32
    lib.orc_bins.argtypes = [i32, P, i64, P]
    lib.orc_weight_table.argtypes = [P]
    lib.orc_topp.argtypes = [i32, P, i64, f32, P, P, P, P, P]
    lib.orc_topp.restype = i64
    lib.orc_attend.argtypes = [i32, i32, P, P, P, i64, P, i64, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------------------
# Rotation description
# ----------------------------------------------------------------------------------------
class Rotation:
    """A key/query rotation: dense binary16 D x D matrix, or randomized Hadamard signs.

    dense:    ``R16`` (np.float16, D x D, row-major); k' = R k.
    hadamard: ``signs`` (np.uint32, D/32 words); bit j set means sigma_j = -1;
              k' = H diag(sigma) k / sqrt(D) with H the Sylvester-order Hadamard matrix.
    """

    def __init__(self, kind, D, R16=None, signs=None):
        self.kind = kind
        self.D = D
        if kind == ROT_DENSE:
            self.Rf = _c(np.asarray(R16, dtype=np.float16).astype(np.float32), np.float32)
            self.signs = np.zeros(max(1, D // 32), dtype=np.uint32)
        else:
            self.Rf = np.zeros(1, dtype=np.float32)
            self.signs = _c(signs, np.uint32)


# ----------------------------------------------------------------------------------------
# binary16
# ----------------------------------------------------------------------------------------
def f16_bits(x: float) -> int:
    return int(_load().orc_f16_from_f64(float(x)))


def f16_value(bits: int) -> float:
    return float(_load().orc_f64_from_f16(int(bits)))


def f16_bits_array(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float64).ravel()
    return np.array([lib.orc_f16_from_f64(float(v)) for v in x], dtype=np.uint16)


# ----------------------------------------------------------------------------------------
# Per-vector steps
# ----------------------------------------------------------------------------------------
def rotate_f64(rot: Rotation, x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32).reshape(-1, rot.D), np.float32)
    y = np.empty(x.shape, dtype=np.float64)
    _load().orc_rotate_f64(rot.D, rot.kind, _p(rot.Rf), _p(rot.signs), _p(x), x.shape[0], _p(y))
    return y


def key_encode(rot: Rotation, k, sk=None):
    """k: (n, D) float -> bits (n, sk/32) uint32, nc (n, 2) uint16 (norm, corr); sk is the
    sketch width (the first sk rotated coordinates; default D)."""
    D = rot.D
    sk = D if sk is None else int(sk)
    k = _c(np.asarray(k).astype(np.float32).reshape(-1, D), np.float32)
    n = k.shape[0]
    bits = np.empty((n, sk // 32), dtype=np.uint32)
    nc = np.empty((n, 2), dtype=np.uint16)
    _load().orc_key_encode(D, sk, rot.kind, _p(rot.Rf), _p(rot.signs), _p(k), n, _p(bits), _p(nc))
    return bits, nc


def value_encode(v, D: int, Gv: int):
    """v: (n, D) float -> codes (n, D/2) uint8, sz (n, D/Gv, 2) uint16 (scale, zero)."""
    v = _c(np.asarray(v).astype(np.float32).reshape(-1, D), np.float32)
    n = v.shape[0]
    codes = np.empty((n, D // 2), dtype=np.uint8)
    sz = np.empty((n, D // Gv, 2), dtype=np.uint16)
    _load().orc_value_encode(D, Gv, _p(v), n, _p(codes), _p(sz))
    return codes, sz


def query_encode(rot: Rotation, q, dither=None, sk=None):
    """q: (m, D) float32 -> dict(u (m, D) uint8, vl, delta, c0, c1 (m,) f32, sumu (m,), qrot).
    dither: optional (m, D) float32 uniforms in [0, 1) for stochastic rounding of the codes;
    sk: the keys' sketch width (default D): codes past it are 0."""
    D = rot.D
    sk = D if sk is None else int(sk)
    q = _c(np.asarray(q, dtype=np.float32).reshape(-1, D), np.float32)
    m = q.shape[0]
    if dither is not None:
        dither = _c(np.asarray(dither, dtype=np.float32).reshape(m, D), np.float32)
    u = np.empty((m, D), dtype=np.uint8)
    par = np.empty((m, 4), dtype=np.float32)
    sumu = np.empty(m, dtype=np.int32)
    qrot = np.empty((m, D), dtype=np.float32)
    _load().orc_query_encode(D, sk, rot.kind, _p(rot.Rf), _p(rot.signs), _p(q), m,
                             _p(dither) if dither is not None else None, _p(u), _p(par), _p(sumu), _p(qrot))
    return dict(u=u, vl=par[:, 0].copy(), delta=par[:, 1].copy(), c0=par[:, 2].copy(),
                c1=par[:, 3].copy(), sumu=sumu, qrot=qrot)


def scores(bits, nc, u, c0, c1, D: int, sk=None):
    """One encoded query against L encoded keys (sketches of sk bits, default D) -> (A, P,
    score) arrays of length L."""
    sk = D if sk is None else int(sk)
    bits = _c(bits, np.uint32).reshape(-1, sk // 32)
    nc = _c(nc, np.uint16).reshape(-1, 2)
    u = _c(u, np.uint8).reshape(D)
    L = bits.shape[0]
    A = np.empty(L, dtype=np.int32)
    P = np.empty(L, dtype=np.int32)
    s = np.empty(L, dtype=np.float32)
    _load().orc_scores(sk, _p(bits), _p(nc), L, _p(u), float(c0), float(c1), _p(A), _p(P), _p(s))
    return A, P, s


def kbin(D: int) -> float:
    return float(_load().orc_kbin(D))


def score_bin(s: float, D: int) -> int:
    lib = _load()
    return int(lib.orc_bin(float(s), lib.orc_kbin(D)))


def bins(s, D: int) -> np.ndarray:
    """Top-p bins e_i = floor(s_i * kbin) (clamped; see score_bin) of an array of scores."""
    s = _c(s, np.float32).ravel()
    e = np.empty(s.shape[0], dtype=np.int32)
    _load().orc_bins(D, _p(s), s.shape[0], _p(e))
    return e


def weight_table() -> np.ndarray:
    T = np.empty(256, dtype=np.uint64)
    _load().orc_weight_table(_p(T))
    return T


def topp(s, p: float, D: int):
    """Top-p over one head's scores -> dict(idx ascending int32, emax, bstar, Z, Tp)."""
    s = _c(s, np.float32).ravel()
    L = s.shape[0]
    idx = np.empty(max(L, 1), dtype=np.int32)
    emax = ctypes.c_int32(0)
    bstar = ctypes.c_int32(0)
    Z = ctypes.c_uint64(0)
    Tp = ctypes.c_uint64(0)
    n = _load().orc_topp(D, _p(s), L, float(p), _p(idx), ctypes.byref(emax), ctypes.byref(bstar),
                         ctypes.byref(Z), ctypes.byref(Tp))
    return dict(idx=idx[:n].copy(), emax=emax.value, bstar=bstar.value, Z=Z.value, Tp=Tp.value)


def attend(s, codes, sz, D: int, Gv: int, idx=None) -> np.ndarray:
    """Softmax(s/sqrt(D)) over all tokens (idx None) or over idx, times the decoded values."""
    s = _c(s, np.float32).ravel()
    codes = _c(codes, np.uint8).reshape(-1, D // 2)
    sz = _c(sz, np.uint16).reshape(-1, D // Gv, 2)
    L = s.shape[0]
    out = np.empty(D, dtype=np.float64)
    if idx is None:
        _load().orc_attend(D, Gv, _p(s), _p(codes), _p(sz), L, None, 0, _p(out))
    else:
        idx = _c(idx, np.int32)
        _load().orc_attend(D, Gv, _p(s), _p(codes), _p(sz), L, _p(idx), idx.shape[0], _p(out))
    return out


def value_decode(codes, sz, D: int, Gv: int) -> np.ndarray:
    """The 4-bit values of n tokens in binary64: code * scale + zero with the group's binary16
    scale and zero point ("H1B-KV" key design, 4-bit linear values).  codes (n, D/2) uint8 with
    the even dim in the low nibble; sz (n, D/Gv, 2) uint16 (scale, zero)."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, D // 2)
    sz = np.asarray(sz, dtype=np.uint16).reshape(-1, D // Gv, 2)
    c = np.empty((codes.shape[0], D), dtype=np.float64)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    scale = sz[..., 0].view(np.float16).astype(np.float64)
    zero = sz[..., 1].view(np.float16).astype(np.float64)
    return c * np.repeat(scale, Gv, axis=1) + np.repeat(zero, Gv, axis=1)


def exact_scores(q, k16) -> np.ndarray:
    """<q, k> in binary64 for a binary32 query q (D,) and binary16 keys k16 (n, D)."""
    k = np.asarray(k16, dtype=np.float16).astype(np.float64)
    return k @ np.asarray(q, dtype=np.float32).astype(np.float64)


def attend_exact(q, k16, codes, sz, D: int, Gv: int, idx) -> np.ndarray:
    """Attention over a retrieved token set with exact scores ("RaBitQCache" abstract: the
    proxy scores estimate the attention weights so as to retrieve the tokens that sparse
    attention then runs over): softmax(<q, k_i> / sqrt(D)) over i in idx, times the decoded
    4-bit values, in binary64.  An empty set gives zeros."""
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return np.zeros(D)
    s = exact_scores(q, np.asarray(k16)[idx])
    w = np.exp((s - s.max()) / np.sqrt(D))
    return (w @ value_decode(np.asarray(codes)[idx], np.asarray(sz)[idx], D, Gv)) / w.sum()


def attend_with_tail(s_sel, vals_sel, q, tk, tv, D: int, shift: float = 0.0, weights: bool = False):
    """One softmax over the attended compressed tokens (scores s_sel, decoded values vals_sel)
    and the binary16 tail tokens (exact scores <q, k> - shift, their binary16 values), in
    binary64: the lazy updates of "RaBitQCache" (abstract) leave the newest tokens
    uncompressed, and a decode attends them next to the cache.  shift = <q, c> puts the tail
    in the frame of proxy scores of keys centered at c.  No tokens at all gives zeros.
    weights=True also returns the tail tokens' softmax weights (normalized over everything)."""
    ntk = np.asarray(tk).reshape(-1, D).shape[0]
    s = np.concatenate([np.asarray(s_sel, dtype=np.float64).ravel(),
                        exact_scores(q, np.asarray(tk).reshape(-1, D)) - float(shift)])
    if s.size == 0:
        return (np.zeros(D), np.zeros(ntk)) if weights else np.zeros(D)
    vals = np.concatenate([np.asarray(vals_sel, dtype=np.float64).reshape(-1, D),
                           np.asarray(tv, dtype=np.float16).astype(np.float64).reshape(-1, D)])
    w = np.exp((s - s.max()) / np.sqrt(D))
    out = (w @ vals) / w.sum()
    return (out, w[s.size - ntk:] / w.sum()) if weights else out


# ----------------------------------------------------------------------------------------
# Paged cache: per (physical page, KV head) structure-of-arrays
# ----------------------------------------------------------------------------------------
class PagedCache:
    """The paged packed cache.  Token t of sequence b lives in physical page
    page_table[b][t // P], slot t % P.  Per (page, KV head):
      key_bits  uint32 [P][sk/32]    sign bits of the first sk rotated coordinates (the
                                     sketch; sk = D unless a narrower sketch is asked for)
      key_nc    uint32 [P]           binary16 norm (low half) | binary16 corr (high half)
      val_codes uint8  [P][D/2]      4-bit value codes, even dim in the low nibble
      val_sz    uint32 [P][D/Gv]     binary16 scale (low half) | binary16 zero (high half)
      key_f16   float16 [P][D]       with exact_keys: the keys rounded to binary16 (nearest even)
    key_center (optional, float32 [Hkv][D]): per-head key centers.  Appends encode the
    binary32 difference k - c_h instead of k (key_f16 keeps k); the proxy scores then
    estimate <q, k - c_h>, which differs from <q, k> by a constant per query head.
    """

    def __init__(self, num_pages, Hkv, P, D, Gv, exact_keys=False, key_center=None, sketch=None):
        self.num_pages, self.Hkv, self.P, self.D, self.Gv = num_pages, Hkv, P, D, Gv
        self.sk = D if sketch is None else int(sketch)  # sketch width: sign bits per key
        self.key_center = None if key_center is None else np.asarray(key_center, dtype=np.float32).reshape(Hkv, D)
        self.key_f16 = np.zeros((num_pages, Hkv, P, D), dtype=np.float16) if exact_keys else None
        self.key_bits = np.zeros((num_pages, Hkv, P, self.sk // 32), dtype=np.uint32)
        self.key_nc = np.zeros((num_pages, Hkv, P), dtype=np.uint32)
        self.val_codes = np.zeros((num_pages, Hkv, P, D // 2), dtype=np.uint8)
        self.val_sz = np.zeros((num_pages, Hkv, P, D // Gv), dtype=np.uint32)

    def locate(self, b, t, page_table):
        t = np.asarray(t)
        return np.asarray(page_table)[b, t // self.P], t % self.P

    def gather(self, b, kvh, L, page_table):
        """Records of tokens 0..L-1 of sequence b, KV head kvh."""
        pg, sl = self.locate(b, np.arange(L), page_table)
        bits = self.key_bits[pg, kvh, sl]
        ncw = self.key_nc[pg, kvh, sl]
        nc = np.stack([(ncw & 0xFFFF).astype(np.uint16), (ncw >> 16).astype(np.uint16)], axis=-1)
        codes = self.val_codes[pg, kvh, sl]
        szw = self.val_sz[pg, kvh, sl]
        sz = np.stack([(szw & 0xFFFF).astype(np.uint16), (szw >> 16).astype(np.uint16)], axis=-1)
        return bits, nc, codes, sz


def append(cache: PagedCache, rot: Rotation, k, v, start_pos, page_table):
    """Encode k, v (B, n_new, Hkv, D) and write token start_pos[b] + i of sequence b."""
    k = np.asarray(k)
    v = np.asarray(v)
    B, n_new, Hkv, D = k.shape
    for b in range(B):
        t = int(start_pos[b]) + np.arange(n_new)
        pg, sl = cache.locate(b, t, page_table)
        for h in range(Hkv):
            kh = k[b, :, h, :]
            if cache.key_center is not None:
                # centering before the rotation: one binary32 subtraction per dim
                kh = kh.astype(np.float32) - cache.key_center[h]
            bits, nc = key_encode(rot, kh, cache.sk)
            codes, sz = value_encode(v[b, :, h, :], D, cache.Gv)
            cache.key_bits[pg, h, sl] = bits
            cache.key_nc[pg, h, sl] = nc[:, 0].astype(np.uint32) | (nc[:, 1].astype(np.uint32) << 16)
            cache.val_codes[pg, h, sl] = codes
            cache.val_sz[pg, h, sl] = sz[..., 0].astype(np.uint32) | (sz[..., 1].astype(np.uint32) << 16)
            if cache.key_f16 is not None:
                cache.key_f16[pg, h, sl] = k[b, :, h, :].astype(np.float16)


def decode_head(cache: PagedCache, rot: Rotation, q_h, b, h, Hq, L, page_table, top_p, proxy=False, tail=None,
                dither=None):
    """One (sequence, query head) decode step.  Query head h reads KV head h*Hkv//Hq.  Under
    Top-p, a cache with binary16 keys attends the selected set with exact scores (out), and
    the proxy-score output is kept as out_proxy; proxy=True ignores the binary16 keys.
    tail = (binary16 keys, binary16 values) of the uncompressed tokens that follow the L
    compressed ones: out is then the one softmax over both (the cache-only output stays as
    out_cache).  With key centers, the proxy scores are those of the centered keys and the
    tail's exact scores are moved by <q, c> into their frame (not when exact scores of the
    compressed tokens are in use).  dither: uniforms of the stochastic query rounding."""
    res = _decode_head_cache(cache, rot, q_h, b, h, Hq, L, page_table, top_p, proxy, dither)
    if tail is None:
        return res
    D, Gv = cache.D, cache.Gv
    if L <= 0:
        s_sel, vals_sel = np.zeros(0), np.zeros((0, D))
    else:
        # all live tokens (marked records of the high-precision tier have NaN scores) or the
        # Top-p set
        sel = np.nonzero(~np.isnan(res["score"]))[0] if res["idx"] is None else res["idx"]
        bits, nc, codes, sz = cache.gather(b, res["kvh"], L, page_table)
        if cache.key_f16 is not None and top_p < 1.0 and not proxy:
            pg, sl = cache.locate(b, np.arange(L), page_table)
            s_sel = exact_scores(q_h, cache.key_f16[pg, res["kvh"], sl][sel])
        else:
            s_sel = res["score"][sel]
        vals_sel = value_decode(codes[sel], sz[sel], D, Gv)
    res["out_cache"] = res["out"]
    exact = cache.key_f16 is not None and top_p < 1.0 and not proxy
    shift = 0.0
    if cache.key_center is not None and not exact:
        shift = float(np.dot(np.asarray(q_h, np.float64), cache.key_center[res["kvh"]].astype(np.float64)))
    res["out"], res["w_tail"] = attend_with_tail(s_sel, vals_sel, q_h, tail[0], tail[1], D, shift, weights=True)
    return res


def _decode_head_cache(cache: PagedCache, rot: Rotation, q_h, b, h, Hq, L, page_table, top_p, proxy, dither=None):
    D, Gv = cache.D, cache.Gv
    kvh = h * cache.Hkv // Hq
    qe = query_encode(rot, q_h, dither, cache.sk)
    res = dict(u=qe["u"][0], vl=qe["vl"][0], delta=qe["delta"][0], c0=qe["c0"][0],
               c1=qe["c1"][0], sumu=int(qe["sumu"][0]), kvh=kvh)
    if L <= 0:
        res.update(out=np.zeros(D), A=np.zeros(0, np.int32), score=np.zeros(0, np.float32),
                   idx=None)
        return res
    bits, nc, codes, sz = cache.gather(b, kvh, L, page_table)
    A, P, s = scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], D, cache.sk)
    res.update(A=A, P=P, score=s)
    if top_p < 1.0:
        tp = topp(s, top_p, D)
        res.update(idx=tp["idx"], emax=tp["emax"], bstar=tp["bstar"], Z=tp["Z"], Tp=tp["Tp"])
        res["out"] = attend(s, codes, sz, D, Gv, tp["idx"])
        if cache.key_f16 is not None and not proxy:
            pg, sl = cache.locate(b, np.arange(L), page_table)
            res["out_proxy"] = res["out"]
            res["out"] = attend_exact(q_h, cache.key_f16[pg, kvh, sl], codes, sz, D, Gv, tp["idx"])
    else:
        res["idx"] = None
        live = ~np.isnan(s)  # a NaN score marks a record held in the high-precision tier
        res["out"] = attend(s, codes, sz, D, Gv) if live.all() else attend(s, codes, sz, D, Gv, np.nonzero(live)[0])
    return res


class HPTier:
    """High-precision tier ("H1IB-KV" high-precision layer): per (sequence, KV head) up to C
    tokens kept in binary16, read here as the ones with the largest accumulated attention
    mass.  k16, v16 float16 [B][Hkv][C][D]; pos int [B][Hkv][C] (-1 empty); saved uint32
    [B][Hkv][C]: the norm/correction word of the token's compressed key record, which holds
    MARKER while the token is in the tier; mass float64 [B][Hkv][C]."""

    MARKER = 0x7E007E00  # binary16 NaN norm and correction

    def __init__(self, B, Hkv, C, D):
        self.B, self.Hkv, self.C, self.D = B, Hkv, C, D
        self.k16 = np.zeros((B, Hkv, C, D), np.float16)
        self.v16 = np.zeros((B, Hkv, C, D), np.float16)
        self.pos = np.full((B, Hkv, C), -1, np.int64)
        self.saved = np.zeros((B, Hkv, C), np.uint32)
        self.mass = np.zeros((B, Hkv, C), np.float64)


def hp_update(cache: PagedCache, hp: HPTier, tail_k, tail_v, tail_mass, n, seq_lens, page_table):
    """Promotion step, once tail tokens 0..n-1 of every sequence (positions seq_lens[b] + j)
    are compressed into the cache: per (sequence, KV head) the C candidates with the largest
    mass among the tier's entries and those n tokens hold the tier afterwards (equal mass:
    lower position first; empty entries last).  Leaving entries get their record word back;
    entering tokens take the free entries in ascending order (in ascending j), with their
    binary16 key and value, their mass, and their record word saved and replaced by MARKER."""
    C = hp.C
    for b in range(hp.B):
        L0 = int(seq_lens[b])
        for h in range(hp.Hkv):
            cand = []  # (sort key, kind, index)
            for i in range(C):
                if hp.pos[b, h, i] >= 0:
                    cand.append(((-hp.mass[b, h, i], int(hp.pos[b, h, i]), i), "entry", i))
                else:
                    cand.append(((np.inf, 2**62, i), "entry", i))
            for j in range(n):
                cand.append(((-float(tail_mass[b, j, h]), L0 + j, C + j), "tail", j))
            cand.sort(key=lambda c: c[0])
            chosen = cand[:C]
            stay = {i for _, kind, i in chosen if kind == "entry" and hp.pos[b, h, i] >= 0}
            enter = sorted(j for _, kind, j in chosen if kind == "tail")
            for i in range(C):
                if hp.pos[b, h, i] >= 0 and i not in stay:
                    pg, sl = cache.locate(b, int(hp.pos[b, h, i]), page_table)
                    cache.key_nc[pg, h, sl] = hp.saved[b, h, i]
                    hp.pos[b, h, i] = -1
            free = [i for i in range(C) if hp.pos[b, h, i] < 0]
            for f, j in zip(free, enter):
                pos = L0 + j
                pg, sl = cache.locate(b, pos, page_table)
                hp.k16[b, h, f] = np.asarray(tail_k)[b, j, h]
                hp.v16[b, h, f] = np.asarray(tail_v)[b, j, h]
                hp.saved[b, h, f] = cache.key_nc[pg, h, sl]
                cache.key_nc[pg, h, sl] = HPTier.MARKER
                hp.pos[b, h, f] = pos
                hp.mass[b, h, f] = float(tail_mass[b, j, h])


def add_mass(res, tail_mass, hp: HPTier, Hq):
    """Adds each query head's softmax weights of its tail tokens and tier entries (from
    decode(..., hp=...)) to tail_mass [B][cap][Hkv] and hp.mass: the mass accumulates the
    weights of the KV head's query heads, step after step."""
    for (b, h), r in res.items():
        kvh = h * hp.Hkv // Hq
        wt, wh = r["w_tail_only"], r["w_hp"]
        if tail_mass is not None and wt.size:
            tail_mass[b, :wt.size, kvh] += wt
        hp.mass[b, kvh] += wh


def decode(cache: PagedCache, rot: Rotation, q, seq_lens, page_table, top_p, heads=None, proxy=False,
           tail=None, dither=None, hp: HPTier = None):
    """Decode step for q (B, Hq, D).  Returns {(b, h): decode_head(...)} for the requested
    (b, h) pairs (all by default).  tail = (tail_k, tail_v, tail_len): binary16 [B][cap][Hkv][D]
    keys and values and int [B] lengths of the uncompressed tokens after seq_lens[b].
    dither: optional (B, Hq, D) uniforms in [0, 1) for stochastic rounding of the query codes.
    hp: the high-precision tier, whose valid entries of the head's KV head are attended like
    tail tokens after them; each result then holds w_tail_only (the tail tokens' weights) and
    w_hp [C] (the entries' weights, 0 for empty entries)."""
    q = np.asarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    out = {}
    for (b, h) in heads:
        th = None
        kvh = h * cache.Hkv // Hq
        nt = 0
        if tail is not None:
            nt = int(tail[2][b])
            th = (np.asarray(tail[0])[b, :nt, kvh], np.asarray(tail[1])[b, :nt, kvh])
        if hp is not None:
            live = np.nonzero(hp.pos[b, kvh] >= 0)[0]
            tk_ = np.zeros((0, D), np.float16) if th is None else th[0]
            tv_ = np.zeros((0, D), np.float16) if th is None else th[1]
            th = (np.concatenate([tk_, hp.k16[b, kvh, live]]), np.concatenate([tv_, hp.v16[b, kvh, live]]))
        dh = None if dither is None else np.asarray(dither, dtype=np.float32)[b, h]
        r = decode_head(cache, rot, q[b, h], b, h, Hq, int(seq_lens[b]), page_table, top_p, proxy, th, dh)
        if hp is not None:
            w = r["w_tail"]
            r["w_tail_only"] = w[:nt]
            r["w_hp"] = np.zeros(hp.C)
            r["w_hp"][live] = w[nt:]
        out[(b, h)] = r
    return out
