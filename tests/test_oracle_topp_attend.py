"""Pins of the oracle's adaptive Top-p selection and of its attention output.

Top-p ("RaBitQCache", abstract: adaptive Top-p retrieval sets the token budget from the
actual attention sparsity) is read as the textbook nucleus: the smallest set of tokens,
heaviest first, whose softmax mass reaches p.  The oracle evaluates masses on integer
weights at a bin resolution of 2^(1/256); here it is checked against a binary64 nucleus
computed by sorting, against exact high-precision weights, and on special cases.
Attention ("H1B-KV", technical framework: weights from the 1-bit sketch, output from the
4-bit values) is checked against torch.softmax in float64 times the decoded values.
"""
import decimal

import numpy as np
import pytest
import torch

import oracle

D = 128


def test_weight_table_against_high_precision():
    decimal.getcontext().prec = 60
    T = oracle.weight_table()
    ln2 = decimal.Decimal(2).ln()
    for j in range(256):
        exact = (ln2 * (decimal.Decimal(32) - decimal.Decimal(j) / 256)).exp()
        assert int(T[j]) == int(exact.to_integral_value(rounding=decimal.ROUND_HALF_EVEN)), j
        # every entry is far from a rounding tie, so any faithful exp2 gives the same table
        frac = exact - exact.to_integral_value(rounding=decimal.ROUND_FLOOR)
        assert abs(frac - decimal.Decimal("0.5")) > decimal.Decimal("1e-6"), j
    assert int(T[0]) == 2**32


def test_kbin_constant():
    kb = np.float32(oracle.kbin(128))
    assert kb.view(np.uint32) == 0x420293EE
    # one bin is a factor 2^(1/256) of softmax weight exp(s / sqrt(D))
    np.testing.assert_allclose(float(kb) / 256, np.log2(np.e) / np.sqrt(128), rtol=2.0**-24)


def test_bin_is_floor_and_clamped():
    kb = oracle.kbin(D)
    for s in (0.0, 1e-3, -1e-3, 3.7, -3.7, 100.0):
        x = np.float32(np.float32(s) * np.float32(kb))
        assert oracle.score_bin(s, D) == int(np.floor(x))
    assert oracle.score_bin(1e30, D) == 2**29
    assert oracle.score_bin(-1e30, D) == -(2**29)
    assert oracle.score_bin(float("nan"), D) == -(2**29)


def test_bins_vector_matches_scalar():
    """The array form of the bins agrees with the scalar bin, clamps and NaN included."""
    rng = np.random.default_rng(7)
    s = np.concatenate([rng.normal(0, 30, 500), [0.0, -0.0, 1e30, -1e30, np.nan, np.inf, -np.inf]]).astype(np.float32)
    np.testing.assert_array_equal(oracle.bins(s, D), [oracle.score_bin(float(x), D) for x in s])


def _nucleus_masses(s, S, p):
    """Binary64 softmax masses of S and of S minus its lowest bin."""
    w = np.exp((s.astype(np.float64) - s.max()) / np.sqrt(D))
    w /= w.sum()
    return w[S].sum()


@pytest.mark.parametrize("p", [0.5, 0.9, 0.95, 0.99])
@pytest.mark.parametrize("dist", ["normal", "spiky", "wide"])
def test_topp_against_fp64_nucleus(p, dist):
    rng = np.random.default_rng(20)
    L = 20000
    if dist == "normal":
        s = rng.standard_normal(L) * np.sqrt(D)
    elif dist == "spiky":
        s = rng.standard_normal(L) * np.sqrt(D)
        pos = rng.choice(L, 200, replace=False)
        s[pos] += 8 * np.sqrt(D)
    else:
        s = rng.standard_normal(L) * 4 * np.sqrt(D)
    s = s.astype(np.float32)
    r = oracle.topp(s, p, D)
    idx = r["idx"]
    assert np.all(np.diff(idx) > 0)
    bins = np.array([oracle.score_bin(x, D) for x in s])
    d = r["emax"] - bins
    np.testing.assert_array_equal(idx, np.nonzero(d <= r["bstar"])[0])
    delta = 0.003  # a bin is a factor 2^(1/256) = 1.0027 of weight
    w = np.exp((s.astype(np.float64) - s.max()) / np.sqrt(D))
    w /= w.sum()
    assert w[idx].sum() >= p - delta
    inner = np.nonzero(d < r["bstar"])[0]
    assert w[inner].sum() < p + delta
    # the binary64 nucleus (sort, smallest prefix reaching p) agrees up to the boundary bin
    order = np.argsort(-s.astype(np.float64), kind="stable")
    k = int(np.searchsorted(np.cumsum(w[order]), p)) + 1
    nuc = set(order[:k].tolist())
    sel = set(idx.tolist())
    boundary = set(np.nonzero(np.abs(d - r["bstar"]) <= 2)[0].tolist())
    assert (nuc ^ sel) <= boundary


def test_topp_special_cases():
    rng = np.random.default_rng(21)
    L = 5000
    s = (rng.standard_normal(L) * np.sqrt(D)).astype(np.float32)
    s[1234] = s.max() + 30 * np.sqrt(D)  # 30 logits above the rest
    r = oracle.topp(s, 0.99, D)
    assert list(r["idx"]) == [1234]
    eq = np.full(L, 3.25, dtype=np.float32)
    r = oracle.topp(eq, 0.5, D)
    np.testing.assert_array_equal(r["idx"], np.arange(L))
    s2 = (rng.standard_normal(L) * np.sqrt(D)).astype(np.float32)
    r = oracle.topp(s2, 1e-9, D)
    bins = np.array([oracle.score_bin(x, D) for x in s2])
    np.testing.assert_array_equal(r["idx"], np.nonzero(bins == bins.max())[0])
    assert r["bstar"] == 0
    one = oracle.topp(np.array([7.0], np.float32), 0.9, D)
    assert list(one["idx"]) == [0]


def test_topp_integer_mass_bookkeeping():
    """Z and the threshold follow from exact integer weights recomputed here with Python
    integers from the high-precision table."""
    rng = np.random.default_rng(22)
    s = (rng.standard_normal(3000) * np.sqrt(D)).astype(np.float32)
    p = 0.9
    r = oracle.topp(s, p, D)
    decimal.getcontext().prec = 60
    ln2 = decimal.Decimal(2).ln()
    T = [int((ln2 * (32 - decimal.Decimal(j) / 256)).exp().to_integral_value(decimal.ROUND_HALF_EVEN))
         for j in range(256)]
    bins = [oracle.score_bin(float(x), D) for x in s]
    em = max(bins)
    W = [(T[(em - e) % 256] >> ((em - e) // 256)) if em - e < 8192 else 0 for e in bins]
    Z = sum(W)
    assert r["Z"] == Z
    pfx = int(round(p * 2**24))
    assert r["Tp"] == -(-(Z * pfx) // 2**24)
    F = lambda b: sum(w for w, e in zip(W, bins) if em - e <= b)
    assert F(r["bstar"]) >= r["Tp"] and (r["bstar"] == 0 or F(r["bstar"] - 1) < r["Tp"])


def _random_cache(rng, L, Gv=32):
    codes = rng.integers(0, 256, size=(L, D // 2), dtype=np.uint8)
    sc = (np.abs(rng.standard_normal((L, D // Gv))) * 0.2 + 0.01).astype(np.float16)
    zr = (rng.standard_normal((L, D // Gv))).astype(np.float16)
    sz = np.stack([sc.view(np.uint16), zr.view(np.uint16)], axis=-1)
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(L, D).astype(np.float64)
    vhat = c * np.repeat(sc.astype(np.float64), Gv, axis=1) + np.repeat(zr.astype(np.float64), Gv, axis=1)
    return codes, sz, vhat


@pytest.mark.parametrize("Gv", [32, 64])
def test_attend_matches_torch_softmax(Gv):
    rng = np.random.default_rng(23)
    L = 777
    codes, sz, vhat = _random_cache(rng, L, Gv)
    s = (rng.standard_normal(L) * 30).astype(np.float32)
    out = oracle.attend(s, codes, sz, D, Gv)
    w = torch.softmax(torch.tensor(s, dtype=torch.float64) / np.sqrt(D), dim=0)
    ref = (w[:, None] * torch.tensor(vhat)).sum(0).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    idx = np.sort(rng.choice(L, 100, replace=False)).astype(np.int32)
    out2 = oracle.attend(s, codes, sz, D, Gv, idx)
    w2 = torch.softmax(torch.tensor(s[idx], dtype=torch.float64) / np.sqrt(D), dim=0)
    ref2 = (w2[:, None] * torch.tensor(vhat[idx])).sum(0).numpy()
    np.testing.assert_allclose(out2, ref2, rtol=1e-12, atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(24)
    codes, sz, vhat = _random_cache(rng, 50)
    s = rng.standard_normal(50).astype(np.float32)
    np.testing.assert_allclose(oracle.attend(s[:1], codes[:1], sz[:1], D, 32), vhat[0], rtol=1e-15)
    eq = np.full(50, -2.5, np.float32)
    np.testing.assert_allclose(oracle.attend(eq, codes, sz, D, 32), vhat.mean(0), rtol=1e-12)
    np.testing.assert_array_equal(oracle.attend(s, codes, sz, D, 32, np.zeros(0, np.int32)), np.zeros(D))
