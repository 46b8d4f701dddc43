"""Pins of the oracle's estimator variants: stochastic rounding of the int4 query and per-head
key centering before the rotation (both outside the pages; RaBitQCache's abstract names the
unbiased proxy score they serve).

Stochastic rounding replaces rint(t) by floor(t + U) with a caller-supplied uniform U, so
that every code is floor(t) or floor(t) + 1 with E[u] = t.  Pinned by: the two candidate
codes, agreement with the round-to-nearest path away from ties at U = 1/2, and the means
over many seeded dithers of the dequantized query and of the proxy score, which must reach
the unquantized values (the round-to-nearest path does not).

Centering encodes k - c_h instead of k.  Pinned by an identity that needs no retyped
formula: with every number a short dyadic fraction (exact in binary16 and binary32), a
centered cache of keys c + d holds the same bytes as a plain cache of keys d, and its decode
(plain, Top-p, exact scores, with a binary16 tail t or the tail t - c for the plain cache)
gives the same output, because every score moves by the same <q, c>.
"""
import numpy as np
import pytest

import oracle
import workloads as W

D = 128


def _rotation(kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "dense":
        return oracle.Rotation(oracle.ROT_DENSE, D, R16=W.haar_orthogonal(rng, D).astype(np.float16))
    signs = rng.integers(0, 2**32, size=D // 32, dtype=np.uint64).astype(np.uint32)
    return oracle.Rotation(oracle.ROT_HADAMARD, D, signs=signs)


def _t(qe):
    """(q' - v_l) / delta in binary32, the quantity that is rounded."""
    return ((qe["qrot"] - qe["vl"][:, None]) / qe["delta"][:, None]).astype(np.float32)


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
def test_stochastic_codes_are_floor_or_floor_plus_one(kind):
    rot = _rotation(kind, 1)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((64, D)).astype(np.float32)
    U = rng.random((64, D), dtype=np.float32)
    qe = oracle.query_encode(rot, q, U)
    t = _t(qe)
    lo = np.clip(np.floor(t), 0, 15)
    hi = np.clip(np.floor(t) + 1, 0, 15)
    u = qe["u"].astype(np.float32)
    assert np.all((u == lo) | (u == hi))
    assert np.any(u == lo) and np.any(u == hi)
    # U = 0 truncates
    qe0 = oracle.query_encode(rot, q, np.zeros((64, D), np.float32))
    np.testing.assert_array_equal(qe0["u"], np.clip(np.floor(_t(qe0)), 0, 15).astype(np.uint8))
    # the same rotation and range as the deterministic path
    qr = oracle.query_encode(rot, q)
    np.testing.assert_array_equal(qe["qrot"], qr["qrot"])
    np.testing.assert_array_equal(qe["vl"], qr["vl"])
    np.testing.assert_array_equal(qe["delta"], qr["delta"])
    np.testing.assert_array_equal(qe["sumu"], qe["u"].astype(np.int64).sum(axis=1))


def test_half_dither_is_round_to_nearest_away_from_ties():
    rot = _rotation("dense", 3)
    rng = np.random.default_rng(4)
    q = rng.standard_normal((256, D)).astype(np.float32)
    half = oracle.query_encode(rot, q, np.full((256, D), 0.5, np.float32))
    rne = oracle.query_encode(rot, q)
    t = _t(rne)
    frac = t - np.floor(t)
    # t + 1/2 rounds in binary32 only when t is within an ulp of a tie; leave those out
    away = np.abs(frac - 0.5) > 1e-5
    np.testing.assert_array_equal(half["u"][away], rne["u"][away])
    assert away.mean() > 0.99


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
def test_stochastic_rounding_is_unbiased(kind):
    """Mean over N seeded dithers: the dequantized query reaches the rotated query and the
    proxy score reaches |k| <x, q'> / corr, within 5 standard errors; the round-to-nearest
    query misses the score by more than that for most keys."""
    rot = _rotation(kind, 5)
    rng = np.random.default_rng(6)
    N = 4096
    q = rng.standard_normal(D).astype(np.float32)
    U = rng.random((N, D), dtype=np.float32)
    qe = oracle.query_encode(rot, np.tile(q, (N, 1)), U)
    vl, delta = float(qe["vl"][0]), float(qe["delta"][0])
    deq = vl + delta * qe["u"].astype(np.float64)
    qrot = qe["qrot"][0].astype(np.float64)
    se = delta / (2 * np.sqrt(N))
    assert np.all(np.abs(deq.mean(axis=0) - qrot) <= 5 * se + 1e-6 * delta)

    keys = rng.standard_normal((12, D)).astype(np.float32)
    bits, nc = oracle.key_encode(rot, keys)
    s_sign = np.where((bits[:, np.arange(D) // 32] >> (np.arange(D) % 32)) & 1, 1.0, -1.0)
    r = np.array([oracle.f16_value(n) / oracle.f16_value(c) for n, c in nc])
    want = (s_sign @ qrot) / np.sqrt(D) * r
    acc = np.zeros(len(keys))
    for i in range(N):
        _, _, s = oracle.scores(bits, nc, qe["u"][i], qe["c0"][i], qe["c1"][i], D)
        acc += s
    mean = acc / N
    se_s = delta / (2 * np.sqrt(N)) * r
    assert np.all(np.abs(mean - want) <= 5 * se_s + 1e-5 * np.abs(want))
    qr = oracle.query_encode(rot, q)
    _, _, s_rne = oracle.scores(bits, nc, qr["u"][0], qr["c0"][0], qr["c1"][0], D)
    assert np.mean(np.abs(s_rne - want) > 5 * se_s) > 0.5


def _dyadic(rng, shape, scale=1.0):
    """Multiples of 1/64 in [-4, 4): exact in binary16, and so are sums of two of them."""
    return (np.clip(np.round(scale * rng.standard_normal(shape) * 64), -256, 255) / 64).astype(np.float32)


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
def test_centered_cache_equals_plain_cache_of_differences(kind):
    rot = _rotation(kind, 7)
    rng = np.random.default_rng(8)
    B, L, Hkv, Hq, P, Gv = 2, 300, 2, 8, 64, 32
    c = _dyadic(rng, (Hkv, D), 0.5)
    d = _dyadic(rng, (B, L, Hkv, D))
    k = (c[None, None] + d).astype(np.float32)
    assert np.array_equal(k - c[None, None], d)
    v = rng.standard_normal((B, L, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    wl = W.CONFIGS[2].scaled(B=B, Hq=Hq, Hkv=Hkv, P=P)
    lens = np.array([L, L - 37], np.int32)
    pt, npages = W.page_layout(wl, lens)
    for exact in (False, True):
        cen = oracle.PagedCache(npages, Hkv, P, D, Gv, exact_keys=exact, key_center=c)
        plain = oracle.PagedCache(npages, Hkv, P, D, Gv, exact_keys=exact)
        oracle.append(cen, rot, k, v, np.zeros(B, np.int32), pt)
        oracle.append(plain, rot, d, v, np.zeros(B, np.int32), pt)
        np.testing.assert_array_equal(cen.key_bits, plain.key_bits)
        np.testing.assert_array_equal(cen.key_nc, plain.key_nc)
        np.testing.assert_array_equal(cen.val_codes, plain.val_codes)
        np.testing.assert_array_equal(cen.val_sz, plain.val_sz)
        if exact:  # the binary16 keys stay uncentered
            for b_ in range(B):
                pg, sl = cen.locate(b_, np.arange(L), pt)
                np.testing.assert_array_equal(cen.key_f16[pg, :, sl], k[b_].astype(np.float16))
        # tails: t for the centered cache, t - c for the plain one
        n_t = np.array([5, 0], np.int32)
        e = _dyadic(rng, (B, 8, Hkv, D))
        tk = (c[None, None] + e).astype(np.float16)
        tk_plain = e.astype(np.float16)
        tv = rng.standard_normal((B, 8, Hkv, D)).astype(np.float16)
        for top_p in (0.9, 1.0):
            a = oracle.decode(cen, rot, q, lens, pt, top_p)
            b = oracle.decode(plain, rot, q, lens, pt, top_p)
            at = oracle.decode(cen, rot, q, lens, pt, top_p, tail=(tk, tv, n_t))
            bt = oracle.decode(plain, rot, q, lens, pt, top_p, tail=(tk_plain, tv, n_t))
            for key in a:
                if a[key]["idx"] is not None:
                    np.testing.assert_array_equal(a[key]["idx"], b[key]["idx"])
                np.testing.assert_allclose(a[key]["out"], b[key]["out"], rtol=1e-9, atol=1e-12)
                np.testing.assert_allclose(at[key]["out"], bt[key]["out"], rtol=1e-9, atol=1e-12)
            # the tail matters here, so the shift is exercised
            assert any(np.abs(at[key]["out"] - a[key]["out"]).max() > 1e-3 for key in a if key[0] == 0)


def test_zero_center_is_the_plain_cache():
    rot = _rotation("dense", 9)
    rng = np.random.default_rng(10)
    k = rng.standard_normal((1, 70, 2, D)).astype(np.float16)
    v = rng.standard_normal((1, 70, 2, D)).astype(np.float16)
    pt = np.arange(2, dtype=np.int32)[None]
    cen = oracle.PagedCache(2, 2, 64, D, 32, key_center=np.zeros((2, D), np.float32))
    plain = oracle.PagedCache(2, 2, 64, D, 32)
    oracle.append(cen, rot, k, v, np.zeros(1, np.int32), pt)
    oracle.append(plain, rot, k, v, np.zeros(1, np.int32), pt)
    np.testing.assert_array_equal(cen.key_bits, plain.key_bits)
    np.testing.assert_array_equal(cen.key_nc, plain.key_nc)


def test_centering_changes_the_encoding_per_head():
    """Different centers per head: each head's bits are those of its own difference (a
    center applied to the wrong head, or not at all, fails)."""
    rot = _rotation("hadamard", 11)
    rng = np.random.default_rng(12)
    c = _dyadic(rng, (3, D), 2.0)
    k = _dyadic(rng, (1, 40, 3, D))
    v = np.zeros((1, 40, 3, D), np.float32)
    pt = np.zeros((1, 1), np.int32)
    cen = oracle.PagedCache(1, 3, 64, D, 32, key_center=c)
    oracle.append(cen, rot, k, v, np.zeros(1, np.int32), pt)
    for h in range(3):
        bits, nc = oracle.key_encode(rot, k[0, :, h] - c[h])
        np.testing.assert_array_equal(cen.key_bits[0, h, :40], bits)
        other, _ = oracle.key_encode(rot, k[0, :, h] - c[(h + 1) % 3])
        assert not np.array_equal(cen.key_bits[0, h, :40], other)


def test_centering_lowers_the_score_error_of_offset_keys():
    """Keys with a common offset (k = mu + noise, |mu| = 3 |noise|): the centered proxy score
    plus <q, c> (c = the keys' mean) misses <q, k> by far less than the plain proxy score,
    since the estimator's spread scales with |k - c| instead of |k|."""
    rot = _rotation("dense", 13)
    rng = np.random.default_rng(14)
    n = 2000
    mu = rng.standard_normal(D)
    mu *= 3 * np.sqrt(D) / np.linalg.norm(mu)
    k = (mu[None] + rng.standard_normal((1, n, 1, D))).astype(np.float32)
    v = np.zeros_like(k)
    c = k[0, :, 0].astype(np.float64).mean(axis=0).astype(np.float32)[None]
    pt = np.arange((n + 255) // 256, dtype=np.int32)[None]
    plain = oracle.PagedCache(pt.size, 1, 256, D, 32)
    cen = oracle.PagedCache(pt.size, 1, 256, D, 32, key_center=c)
    oracle.append(plain, rot, k, v, np.zeros(1, np.int32), pt)
    oracle.append(cen, rot, k, v, np.zeros(1, np.int32), pt)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    exact = k[0, :, 0].astype(np.float64) @ q[0, 0].astype(np.float64)
    sp = oracle.decode(plain, rot, q, [n], pt, 1.0)[(0, 0)]["score"].astype(np.float64)
    sc = oracle.decode(cen, rot, q, [n], pt, 1.0)[(0, 0)]["score"].astype(np.float64)
    sc += float(q[0, 0].astype(np.float64) @ c[0].astype(np.float64))
    e_plain = np.sqrt(np.mean((sp - exact) ** 2))
    e_cen = np.sqrt(np.mean((sc - exact) ** 2))
    assert e_cen < 0.5 * e_plain, (e_cen, e_plain)
