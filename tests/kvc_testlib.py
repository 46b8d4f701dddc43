"""Shared helpers of the GPU parity tests: build a case from a seeded workload, run the
oracle and the library on it, move caches between them, and compare results."""
from __future__ import annotations

import numpy as np

import oracle
import workloads as W


class Case:
    def __init__(self, wl: W.Workload, L=None, seq_lens=None, reserve=0):
        self.wl = wl
        K, V, q, lens = W.draw_host(wl, L)
        if seq_lens is not None:
            lens = np.asarray(seq_lens, dtype=np.int32)
        self.K, self.V, self.q, self.lens = K, V, q, lens
        self.L = K.shape[1]
        self.pt, self.npages = W.page_layout(wl, np.maximum(lens, 1), reserve=reserve)
        kind, r = W.draw_rotation(wl)
        self.rot_kind = kind
        self.rot_raw = r
        if kind == "dense":
            self.orot = oracle.Rotation(oracle.ROT_DENSE, wl.D, R16=r)
        else:
            self.orot = oracle.Rotation(oracle.ROT_HADAMARD, wl.D, signs=r)

    @property
    def max_len(self):
        return int(max(1, self.lens.max()))

    def oracle_cache(self, exact_keys=False, key_center=None, sketch=None):
        c = oracle.PagedCache(self.npages, self.wl.Hkv, self.wl.P, self.wl.D, self.wl.Gv, exact_keys=exact_keys,
                              key_center=key_center, sketch=sketch)
        for b in range(self.wl.B):
            n = int(self.lens[b])
            if n:
                oracle.append(c, self.orot, self.K[b:b + 1, :n], self.V[b:b + 1, :n], np.zeros(1, np.int32),
                              self.pt[b:b + 1])
        return c

    def oracle_decode(self, cache, top_p, heads=None):
        return oracle.decode(cache, self.orot, self.q, self.lens, self.pt, top_p, heads=heads)


def gpu_empty_cache(case: Case, device="cuda", exact_keys=False, key_center=None, sketch=None):
    from bit_kv_cache_compress_amd import KVCache

    rot = case.rot_raw
    return KVCache(case.npages, case.wl.Hkv, rot, rot_kind=case.rot_kind, page_size=case.wl.P,
                   value_group=case.wl.Gv, device=device, exact_keys=exact_keys, key_center=key_center,
                   sketch_dim=sketch or case.wl.D)


def gpu_append(case: Case, chunk=None, device="cuda", exact_keys=False, key_center=None, sketch=None):
    """The library's append of every sequence (optionally in chunks of `chunk` tokens)."""
    import torch

    from bit_kv_cache_compress_amd import append

    cache = gpu_empty_cache(case, device, exact_keys=exact_keys, key_center=key_center, sketch=sketch)
    for b in range(case.wl.B):
        n = int(case.lens[b])
        step = n if chunk is None else chunk
        for s0 in range(0, n, max(step, 1)):
            e = min(n, s0 + step)
            k = torch.from_numpy(np.ascontiguousarray(case.K[b:b + 1, s0:e])).to(device)
            v = torch.from_numpy(np.ascontiguousarray(case.V[b:b + 1, s0:e])).to(device)
            sp = torch.tensor([s0], dtype=torch.int32, device=device)
            pt = torch.from_numpy(np.ascontiguousarray(case.pt[b:b + 1])).to(device)
            append(cache, k, v, sp, pt)
    torch.cuda.synchronize()
    return cache


def upload(cache_o: oracle.PagedCache, case: Case, device="cuda"):
    """A library cache holding the oracle's bytes."""
    import torch

    g = gpu_empty_cache(case, device, exact_keys=cache_o.key_f16 is not None, key_center=cache_o.key_center,
                        sketch=cache_o.sk)
    if cache_o.key_f16 is not None:
        g.keys_f16.copy_(torch.from_numpy(cache_o.key_f16))
    g.key_bits.copy_(torch.from_numpy(cache_o.key_bits.view(np.int32)))
    g.key_nc.copy_(torch.from_numpy(cache_o.key_nc.view(np.int32)))
    g.val_codes.copy_(torch.from_numpy(cache_o.val_codes))
    g.val_sz.copy_(torch.from_numpy(cache_o.val_sz.view(np.int32)))
    torch.cuda.synchronize()
    return g


def download(g):
    return dict(key_bits=g.key_bits.cpu().numpy().view(np.uint32), key_nc=g.key_nc.cpu().numpy().view(np.uint32),
                val_codes=g.val_codes.cpu().numpy(), val_sz=g.val_sz.cpu().numpy().view(np.uint32))


def oracle_cache_of(gpu: dict, case: Case, sketch=None):
    """An oracle cache holding the bytes the library wrote (download()), so that the oracle's
    query encode, scores, Top-p and attention run on exactly the GPU-built records."""
    c = oracle.PagedCache(case.npages, case.wl.Hkv, case.wl.P, case.wl.D, case.wl.Gv, sketch=sketch)
    c.key_bits[...] = gpu["key_bits"]
    c.key_nc[...] = gpu["key_nc"]
    c.val_codes[...] = gpu["val_codes"]
    c.val_sz[...] = gpu["val_sz"]
    return c


def chunk_dists(s, D: int, chunk: int = 512):
    """What the Top-p score pass writes for one query head's L scores, from the oracle's bins:
    (bin distance of every token to the top bin of its chunk, saturated at 8192, and 8192 past
    L in the last chunk; the chunks' top bins)."""
    e = oracle.bins(s, D).astype(np.int64)
    L = e.shape[0]
    nch = (L + chunk - 1) // chunk
    top = np.array([e[c * chunk:(c + 1) * chunk].max() for c in range(nch)], dtype=np.int64)
    d = np.full(nch * chunk, 8192, dtype=np.int64)
    d[:L] = np.minimum(np.repeat(top, chunk)[:L] - e, 8192)
    return d.astype(np.uint16), top.astype(np.int32)


def check_bins(dbg, b: int, h: int, s, D: int, ld: int):
    """The score pass's bin distances and chunk top bins of (b, h) (DecodeDebug with
    dist=True) against the oracle's bins of the scores s of its L tokens (bit-exact)."""
    d, top = chunk_dists(s, D)
    if top.size == 0:
        return
    got_d = dbg.bin_dist[b, h].cpu().numpy().view(np.uint16)
    got_t = dbg.chunk_top[b, h].cpu().numpy()
    n = min(d.shape[0], ld)
    np.testing.assert_array_equal(got_d[:n], d[:n])
    np.testing.assert_array_equal(got_t[:top.shape[0]], top)


def written_slots(case: Case):
    """(page, slot) index arrays of every written token, per sequence."""
    pg, sl = [], []
    for b in range(case.wl.B):
        t = np.arange(int(case.lens[b]))
        pg.append(case.pt[b, t // case.wl.P])
        sl.append(t % case.wl.P)
    return np.concatenate(pg).astype(np.int64), np.concatenate(sl).astype(np.int64)


def compare_caches(gpu: dict, ocache: oracle.PagedCache, case: Case):
    """Value bytes, scales and norms bit-exact; key bits bit-exact (a coordinate whose
    binary64 rotated value is within 2^-40 of sum|R k| of zero may differ); corr within one
    binary16 ulp.  Returns a dict of counts."""
    stats = {}
    np.testing.assert_array_equal(gpu["val_codes"], ocache.val_codes)
    np.testing.assert_array_equal(gpu["val_sz"], ocache.val_sz)
    ncg, nco = gpu["key_nc"], ocache.key_nc
    np.testing.assert_array_equal(ncg & 0xFFFF, nco & 0xFFFF)
    cg = (ncg >> 16).astype(np.int64)
    co = (nco >> 16).astype(np.int64)
    assert np.all(np.abs(cg - co) <= 1), "correction differs by more than one binary16 ulp"
    stats["corr_ulp_diffs"] = int(np.count_nonzero(cg != co))
    diff = gpu["key_bits"] != ocache.key_bits
    stats["key_word_diffs"] = int(np.count_nonzero(diff))
    if stats["key_word_diffs"]:
        pg, sl = written_slots(case)
        for h in range(case.wl.Hkv):
            bad = np.nonzero(diff[pg, h, sl].any(-1))[0]
            for i in bad:
                b, t = _token_of(case, pg[i], sl[i])
                k = case.K[b, t, h].astype(np.float32)
                y = oracle.rotate_f64(case.orot, k[None, :])[0]
                if case.rot_kind == "dense":
                    mag = np.abs(case.orot.Rf.astype(np.float64)) @ np.abs(k.astype(np.float64))
                else:
                    mag = np.full(case.wl.D, np.abs(k.astype(np.float64)).sum() / np.sqrt(case.wl.D))
                xb = np.bitwise_xor(gpu["key_bits"][pg[i], h, sl[i]], ocache.key_bits[pg[i], h, sl[i]])
                for w in range(xb.shape[-1]):  # the record's sign words (a sketch may hold fewer)
                    for bit in range(32):
                        if (int(xb[w]) >> bit) & 1:
                            r = 32 * w + bit
                            assert abs(y[r]) <= 2.0**-40 * mag[r], f"sign of coordinate {r} differs outside the band"
    return stats


def _token_of(case, page, slot):
    for b in range(case.wl.B):
        hits = np.nonzero(case.pt[b, :(int(case.lens[b]) + case.wl.P - 1) // case.wl.P] == page)[0]
        if len(hits):
            return b, int(hits[0]) * case.wl.P + int(slot)
    raise KeyError(page)


def rel_err(out, ref):
    """max_j |out - ref| / max_j |ref| per row."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref).max(-1), 1e-30)
    return np.abs(out - ref).max(-1) / den
