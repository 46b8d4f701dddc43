"""Pins of the oracle's paged cache: placement through the page table, the chunked-append
invariant, and an end-to-end decode on a small workload checked against a direct binary64
evaluation (fp64 softmax over the oracle's own per-token records)."""
import numpy as np
import torch

import oracle
import workloads as W


def _rot(wl):
    kind, r = W.draw_rotation(wl)
    if kind == "dense":
        return oracle.Rotation(oracle.ROT_DENSE, wl.D, R16=r)
    return oracle.Rotation(oracle.ROT_HADAMARD, wl.D, signs=r)


def test_chunked_append_equals_single_append_and_pages_are_honoured():
    wl = W.CONFIGS[3].scaled(B=3, Hq=4, Hkv=2, L=300, len_range=(100, 300), P=16)
    K, V, q, lens = W.draw_host(wl)
    pt, npages = W.page_layout(wl, lens)
    rot = _rot(wl)
    one = oracle.PagedCache(npages, wl.Hkv, wl.P, wl.D, wl.Gv)
    chunked = oracle.PagedCache(npages, wl.Hkv, wl.P, wl.D, wl.Gv)
    n = int(lens.min())
    oracle.append(one, rot, K[:, :n], V[:, :n], np.zeros(wl.B, np.int32), pt)
    for s0 in range(0, n, 37):
        e = min(n, s0 + 37)
        oracle.append(chunked, rot, K[:, s0:e], V[:, s0:e], np.full(wl.B, s0, np.int32), pt)
    for a in ("key_bits", "key_nc", "val_codes", "val_sz"):
        np.testing.assert_array_equal(getattr(one, a), getattr(chunked, a))
    # token t of sequence b sits in page pt[b][t // P], slot t % P
    b, t, h = 2, 45, 1
    bits, nc = oracle.key_encode(rot, K[b, t, h][None, :].astype(np.float32))
    assert np.array_equal(one.key_bits[pt[b, t // wl.P], h, t % wl.P], bits[0])
    assert one.key_nc[pt[b, t // wl.P], h, t % wl.P] == (int(nc[0, 0]) | (int(nc[0, 1]) << 16))


def test_decode_matches_direct_fp64_attention():
    wl = W.CONFIGS[2].scaled(B=2, L=700, P=64)
    K, V, q, lens = W.draw_host(wl)
    pt, npages = W.page_layout(wl, lens)
    rot = _rot(wl)
    cache = oracle.PagedCache(npages, wl.Hkv, wl.P, wl.D, wl.Gv)
    oracle.append(cache, rot, K, V, np.zeros(wl.B, np.int32), pt)
    res = oracle.decode(cache, rot, q, lens, pt, 1.0, heads=[(0, 0), (1, 31)])
    for (b, h), r in res.items():
        kvh = h * wl.Hkv // wl.Hq
        bits, nc, codes, sz = cache.gather(b, kvh, int(lens[b]), pt)
        codes_u = np.stack([codes & 15, codes >> 4], -1).reshape(len(codes), wl.D).astype(np.float64)
        sc = np.repeat(sz[..., 0].view(np.float16).astype(np.float64), wl.Gv, axis=1)
        zr = np.repeat(sz[..., 1].view(np.float16).astype(np.float64), wl.Gv, axis=1)
        vhat = codes_u * sc + zr
        w = torch.softmax(torch.tensor(r["score"], dtype=torch.float64) / np.sqrt(wl.D), 0).numpy()
        np.testing.assert_allclose(r["out"], w @ vhat, rtol=1e-10, atol=1e-12)
        # the proxy scores track the exact inner products (spread ~0.067 |k||q| plus int4)
        exact = K[b, :lens[b], kvh].astype(np.float64) @ q[b, h].astype(np.float64)
        rel = (r["score"] - exact) / (np.linalg.norm(K[b, :lens[b], kvh].astype(np.float64), axis=1)
                                     * np.linalg.norm(q[b, h]))
        assert abs(rel.mean()) < 0.02 and rel.std() < 0.12
    # Top-p: the selection is a subset, and attention renormalises over it
    rp = oracle.decode(cache, rot, q, lens, pt, 0.9, heads=[(1, 5)])[(1, 5)]
    assert 0 < len(rp["idx"]) < lens[1]
    bits, nc, codes, sz = cache.gather(1, 5 * wl.Hkv // wl.Hq, int(lens[1]), pt)
    np.testing.assert_allclose(rp["out"], oracle.attend(rp["score"], codes, sz, wl.D, wl.Gv, rp["idx"]))
