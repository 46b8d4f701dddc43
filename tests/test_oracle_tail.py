"""Pins of the oracle's attention over the compressed cache plus a binary16 tail.

RaBitQCache (abstract) hides its system's overhead with lazy updates: the newest tokens stay
uncompressed until a whole page is compressed, and a decode attends them next to the cache.
Read here as one softmax over the attended compressed tokens (their proxy scores, or exact
scores with binary16 keys, and decoded 4-bit values) and every tail token (exact score
<q, k>, binary16 value).  Checked against the C attention (empty tail), torch.softmax in
binary64 (tail only; both together), permutation invariance, and the cache-only decode.
"""
import numpy as np
import torch

import oracle
import workloads as W

D = 128


def _vals(rng, n, Gv=32):
    codes = rng.integers(0, 256, size=(n, D // 2), dtype=np.uint8)
    scale = rng.uniform(0.01, 0.2, size=(n, D // Gv)).astype(np.float16).view(np.uint16)
    zero = rng.uniform(-1, 1, size=(n, D // Gv)).astype(np.float16).view(np.uint16)
    return codes, np.stack([scale, zero], axis=-1)


def _torch_union(s, vals):
    w = torch.softmax(torch.tensor(s, dtype=torch.float64) / np.sqrt(D), dim=0)
    return (w @ torch.tensor(vals, dtype=torch.float64)).numpy()


def test_empty_tail_is_the_cache_attention():
    rng = np.random.default_rng(1)
    codes, sz = _vals(rng, 50)
    s = (4 * rng.standard_normal(50)).astype(np.float32)
    idx = np.array([1, 4, 9, 30, 49], np.int32)
    q = rng.standard_normal(D).astype(np.float32)
    got = oracle.attend_with_tail(s[idx], oracle.value_decode(codes[idx], sz[idx], D, 32), q,
                                  np.zeros((0, D), np.float16), np.zeros((0, D), np.float16), D)
    np.testing.assert_allclose(got, oracle.attend(s, codes, sz, D, 32, idx), rtol=1e-12, atol=1e-14)


def test_tail_only_against_torch_softmax():
    rng = np.random.default_rng(2)
    q = (2 * rng.standard_normal(D)).astype(np.float32)
    tk = rng.standard_normal((37, D)).astype(np.float16)
    tv = rng.standard_normal((37, D)).astype(np.float16)
    s = tk.astype(np.float64) @ q.astype(np.float64)
    want = _torch_union(s, tv.astype(np.float64))
    got = oracle.attend_with_tail(np.zeros(0), np.zeros((0, D)), q, tk, tv, D)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_cache_and_tail_against_torch_softmax_and_order():
    rng = np.random.default_rng(3)
    q = (2 * rng.standard_normal(D)).astype(np.float32)
    codes, sz = _vals(rng, 20)
    s_sel = (8 * rng.standard_normal(20)).astype(np.float32)
    vals_sel = oracle.value_decode(codes, sz, D, 32)
    tk = rng.standard_normal((11, D)).astype(np.float16)
    tv = rng.standard_normal((11, D)).astype(np.float16)
    s_t = tk.astype(np.float64) @ q.astype(np.float64)
    want = _torch_union(np.concatenate([s_sel.astype(np.float64), s_t]),
                        np.concatenate([vals_sel, tv.astype(np.float64)]))
    got = oracle.attend_with_tail(s_sel, vals_sel, q, tk, tv, D)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)
    perm = rng.permutation(11)
    np.testing.assert_allclose(oracle.attend_with_tail(s_sel, vals_sel, q, tk[perm], tv[perm], D), got,
                               rtol=1e-12, atol=1e-14)


def test_decode_with_tail_keeps_the_cache_decode():
    wl = W.CONFIGS[2].scaled(B=2, Hq=4, Hkv=2, P=64)
    K, V, q, lens = W.draw_host(wl, 600)
    pt, npages = W.page_layout(wl, lens)
    kind, r = W.draw_rotation(wl)
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=r)
    cache = oracle.PagedCache(npages, 2, 64, D, 32)
    oracle.append(cache, rot, K, V, np.zeros(2, np.int32), pt)
    lc = np.array([500, 0], np.int32)  # the second sequence is all tail
    tl = np.array([100, 64], np.int32)
    tk = np.zeros((2, 128, 2, D), np.float16)
    tv = np.zeros_like(tk)
    for b in range(2):
        tk[b, :tl[b]] = K[b, lc[b]:lc[b] + tl[b]].astype(np.float16)
        tv[b, :tl[b]] = V[b, lc[b]:lc[b] + tl[b]].astype(np.float16)
    for top_p in (0.9, 1.0):
        plain = oracle.decode(cache, rot, q, lc, pt, top_p)
        withtail = oracle.decode(cache, rot, q, lc, pt, top_p, tail=(tk, tv, tl))
        for key, r0 in plain.items():
            r1 = withtail[key]
            np.testing.assert_array_equal(r1["out_cache"], r0["out"])
            if r0["idx"] is not None:
                np.testing.assert_array_equal(r1["idx"], r0["idx"])
            assert np.all(np.isfinite(r1["out"]))
