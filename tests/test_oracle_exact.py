"""Pins of the oracle's exact-score attention over the Top-p set.

RaBitQCache (abstract) uses the proxy scores to estimate the attention weights and so to
retrieve the token set that sparse attention runs over.  With the keys also kept in binary16
the oracle attends that set with the exact scores <q, k>: softmax(<q, k_i> / sqrt(D)) over
the set, times the decoded 4-bit values, in binary64.  Checked here against the C oracle's
attention (an independent implementation) fed the same scores, brute-force dot products, a
two-token closed form, special cases, the IEEE rounding of the stored binary16 keys, and the
proxy-score decode (same sets).
"""
import math

import numpy as np

import oracle
import workloads as W

D = 128


def _tokens(rng, n, Gv):
    codes = rng.integers(0, 256, size=(n, D // 2), dtype=np.uint8)
    scale = rng.uniform(0.01, 0.2, size=(n, D // Gv)).astype(np.float16).view(np.uint16)
    zero = rng.uniform(-1, 1, size=(n, D // Gv)).astype(np.float16).view(np.uint16)
    return codes, np.stack([scale, zero], axis=-1)


def test_value_decode_matches_c_attention_of_one_token():
    rng = np.random.default_rng(1)
    for Gv in (32, 64):
        codes, sz = _tokens(rng, 7, Gv)
        s = rng.standard_normal(7).astype(np.float32)
        vals = oracle.value_decode(codes, sz, D, Gv)
        for i in range(7):
            np.testing.assert_array_equal(oracle.attend(s, codes, sz, D, Gv, np.array([i])), vals[i])


def test_exact_scores_brute_force():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(D).astype(np.float32)
    k16 = rng.standard_normal((5, D)).astype(np.float16)
    got = oracle.exact_scores(q, k16)
    for i in range(5):
        want = math.fsum(float(q[d]) * float(k16[i, d]) for d in range(D))
        assert abs(got[i] - want) <= 1e-12 * max(1.0, abs(want))


def test_attend_exact_matches_c_attention_on_the_same_scores():
    rng = np.random.default_rng(3)
    for Gv in (32, 64):
        n = 300
        q = (3 * rng.standard_normal(D)).astype(np.float32)
        k16 = rng.standard_normal((n, D)).astype(np.float16)
        codes, sz = _tokens(rng, n, Gv)
        idx = np.sort(rng.choice(n, 40, replace=False)).astype(np.int32)
        s32 = oracle.exact_scores(q, k16).astype(np.float32)
        want = oracle.attend(s32, codes, sz, D, Gv, idx)
        got = oracle.attend_exact(q, k16, codes, sz, D, Gv, idx)
        # the C path sees the scores rounded to binary32: weights move by < 1e-6 relative
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6 * np.abs(want).max())


def test_two_token_closed_form():
    rng = np.random.default_rng(4)
    q = np.zeros(D, np.float32)
    q[0] = 2.0
    k16 = np.zeros((2, D), np.float16)
    k16[0, 0] = 3.0   # <q, k0> = 6
    k16[1, 0] = -1.5  # <q, k1> = -3
    codes, sz = _tokens(rng, 2, 32)
    v = oracle.value_decode(codes, sz, D, 32)
    r = math.exp((-3.0 - 6.0) / math.sqrt(D))
    want = (v[0] + r * v[1]) / (1.0 + r)
    np.testing.assert_allclose(oracle.attend_exact(q, k16, codes, sz, D, 32, [0, 1]), want, rtol=1e-13)


def test_single_token_and_empty_set():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(D).astype(np.float32)
    k16 = rng.standard_normal((3, D)).astype(np.float16)
    codes, sz = _tokens(rng, 3, 64)
    np.testing.assert_array_equal(oracle.attend_exact(q, k16, codes, sz, D, 64, [2]),
                                  oracle.value_decode(codes, sz, D, 64)[2])
    np.testing.assert_array_equal(oracle.attend_exact(q, k16, codes, sz, D, 64, []), np.zeros(D))


def test_stored_binary16_keys_round_to_nearest_even():
    cache = oracle.PagedCache(1, 1, 16, D, 32, exact_keys=True)
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=np.eye(D, dtype=np.float16))
    k = np.zeros((1, 4, 1, D), np.float32)
    k[0, 0, 0, 0] = 1 + 2.0**-11      # halfway between 1 and 1 + 2^-10: to even, 1
    k[0, 1, 0, 0] = 1 + 3 * 2.0**-11  # halfway between 1 + 2^-10 and 1 + 2^-9: to even, 1 + 2^-9
    k[0, 2, 0, 0] = 65520.0           # halfway to the next binade above 65504: overflows to inf
    k[0, 3, 0, 0] = -2.0**-25         # half the smallest subnormal: to even, -0
    with np.errstate(over="ignore"):
        oracle.append(cache, rot, k, np.ones_like(k), np.zeros(1, np.int32), np.zeros((1, 1), np.int32))
    bits = cache.key_f16[0, 0, :4, 0].view(np.uint16)
    assert [int(x) for x in bits] == [0x3C00, 0x3C02, 0x7C00, 0x8000]


def test_exact_decode_keeps_the_proxy_sets():
    wl = W.CONFIGS[2].scaled(B=1, Hq=4, Hkv=1, P=64)
    K, V, q, lens = W.draw_host(wl, 700)
    pt, npages = W.page_layout(wl, lens)
    kind, r = W.draw_rotation(wl)
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=r)
    exact = oracle.PagedCache(npages, 1, 64, D, 32, exact_keys=True)
    plain = oracle.PagedCache(npages, 1, 64, D, 32)
    for c in (exact, plain):
        oracle.append(c, rot, K, V, np.zeros(1, np.int32), pt)
    re = oracle.decode(exact, rot, q, lens, pt, 0.9)
    rp = oracle.decode(plain, rot, q, lens, pt, 0.9)
    rx = oracle.decode(exact, rot, q, lens, pt, 0.9, proxy=True)
    for key in re:
        np.testing.assert_array_equal(re[key]["idx"], rp[key]["idx"])
        np.testing.assert_array_equal(re[key]["out_proxy"], rp[key]["out"])
        np.testing.assert_array_equal(rx[key]["out"], rp[key]["out"])
        pg, sl = exact.locate(0, np.arange(int(lens[0])), pt)
        k16 = exact.key_f16[pg, 0, sl]
        np.testing.assert_array_equal(k16, K[0, :int(lens[0]), 0].astype(np.float16))
        b, h = key
        codes, sz = exact.gather(0, 0, int(lens[0]), pt)[2:]
        np.testing.assert_array_equal(re[key]["out"],
                                      oracle.attend_exact(q[b, h], k16, codes, sz, D, 32, re[key]["idx"]))
