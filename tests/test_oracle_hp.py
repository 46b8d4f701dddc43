"""Pins of the oracle's high-precision tier ("H1IB-KV": a high-precision layer for the most
important key-value pairs next to the one-bit layer; importance read as accumulated
attention mass).

The tier's rules are checked against identities that need no retyped formula:
  * a compressed record marked with the NaN norm behaves as if the token were not in the
    cache at all (the decode is invariant under token order, so the token can be removed);
  * tier entries behave exactly as tail tokens, and a token moved from the cache into the
    tier leaves the decode as if it had been a tail token from the start;
  * the weights reported for tail tokens are the closed-form softmax ratios and sum to 1;
  * the promotion keeps the top-C by mass (brute-force sorted), prefers lower positions on
    ties, and promotion followed by eviction of everything gives back the original bytes;
  * a head whose scores are all NaN has an empty Top-p set.
"""
import numpy as np
import pytest

import oracle
import workloads as W

D = 128


def _setup(L=300, B=2, Hkv=2, Hq=4, P=64, seed=0, kind="dense", exact=False):
    rng = np.random.default_rng(seed)
    wl = W.CONFIGS[2].scaled(B=B, Hq=Hq, Hkv=Hkv, P=P)
    if kind == "dense":
        rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=W.haar_orthogonal(rng, D).astype(np.float16))
    else:
        rot = oracle.Rotation(oracle.ROT_HADAMARD, D,
                              signs=rng.integers(0, 2**32, size=D // 32, dtype=np.uint64).astype(np.uint32))
    K = rng.standard_normal((B, L, Hkv, D)).astype(np.float16)
    V = rng.standard_normal((B, L, Hkv, D)).astype(np.float16)
    q = (1.5 * rng.standard_normal((B, Hq, D))).astype(np.float32)
    lens = np.full(B, L, np.int32)
    pt, npages = W.page_layout(wl, lens)
    cache = oracle.PagedCache(npages, Hkv, P, D, 32, exact_keys=exact)
    oracle.append(cache, rot, K, V, np.zeros(B, np.int32), pt)
    return rng, rot, K, V, q, lens, pt, npages, cache


def _mark(cache, b, h, t, pt):
    pg, sl = cache.locate(b, t, pt)
    old = int(cache.key_nc[pg, h, sl])
    cache.key_nc[pg, h, sl] = oracle.HPTier.MARKER
    return old


@pytest.mark.parametrize("top_p", [1.0, 0.9])
def test_marked_record_is_an_absent_token(top_p):
    rng, rot, K, V, q, lens, pt, npages, cache = _setup(seed=1)
    B, L, Hkv = K.shape[0], K.shape[1], K.shape[2]
    drop = {(b, h): sorted(rng.choice(L, 7, replace=False).tolist()) for b in range(B) for h in range(Hkv)}
    for (b, h), ts in drop.items():
        for t in ts:
            _mark(cache, b, h, t, pt)
    res = oracle.decode(cache, rot, q, lens, pt, top_p)
    Hq = q.shape[1]
    for (b, hq), r in res.items():
        h = hq * Hkv // Hq
        keep = np.setdiff1d(np.arange(L), drop[(b, h)])
        # the same head without the dropped tokens, as a cache of its own
        c2 = oracle.PagedCache(npages, 1, cache.P, D, 32)
        oracle.append(c2, rot, K[b:b + 1, keep][:, :, h:h + 1], V[b:b + 1, keep][:, :, h:h + 1],
                      np.zeros(1, np.int32), pt[b:b + 1])
        r2 = oracle.decode_head(c2, rot, q[b, hq], 0, 0, 1, keep.size, pt[b:b + 1], top_p)
        np.testing.assert_allclose(r["out"], r2["out"], rtol=1e-12, atol=1e-14)
        if top_p < 1.0:
            np.testing.assert_array_equal(keep[r2["idx"]], r["idx"])


@pytest.mark.parametrize("exact", [False, True])
def test_tier_entries_are_tail_tokens(exact):
    """Tokens moved into the tier (records marked) decode as tail tokens of a cache that never
    held them; a real tail and the tier together, too."""
    rng, rot, K, V, q, lens, pt, npages, cache = _setup(seed=2, exact=exact)
    B, L, Hkv = K.shape[0], K.shape[1], K.shape[2]
    Hq = q.shape[1]
    C = 8
    hp = oracle.HPTier(B, Hkv, C, D)
    chosen = {}
    for b in range(B):
        for h in range(Hkv):
            ts = sorted(rng.choice(L - 20, 5, replace=False).tolist())
            chosen[(b, h)] = ts
            for i, t in enumerate(ts):
                slot = [1, 3, 4, 6, 7][i]  # scattered entries, the rest empty
                hp.saved[b, h, slot] = _mark(cache, b, h, t, pt)
                hp.pos[b, h, slot] = t
                hp.k16[b, h, slot] = K[b, t, h]
                hp.v16[b, h, slot] = V[b, t, h]
    nt = np.array([20, 3], np.int32)
    lc = (lens - nt).astype(np.int32)
    tk = np.zeros((B, 32, Hkv, D), np.float16)
    tv = np.zeros_like(tk)
    for b in range(B):
        tk[b, :nt[b]] = K[b, lc[b]:lens[b]]
        tv[b, :nt[b]] = V[b, lc[b]:lens[b]]
    for top_p in (1.0, 0.9):
        res = oracle.decode(cache, rot, q, lc, pt, top_p, tail=(tk, tv, nt), hp=hp)
        for (b, hq), r in res.items():
            h = hq * Hkv // Hq
            # the reference: the chosen tokens were never compressed, they are tail tokens
            keep = np.setdiff1d(np.arange(lc[b]), chosen[(b, h)])
            c2 = oracle.PagedCache(npages, 1, cache.P, D, 32, exact_keys=exact)
            oracle.append(c2, rot, K[b:b + 1, keep][:, :, h:h + 1], V[b:b + 1, keep][:, :, h:h + 1],
                          np.zeros(1, np.int32), pt[b:b + 1])
            extra = np.array(chosen[(b, h)])
            t2k = np.concatenate([tk[b, :nt[b], h], K[b, extra, h]])
            t2v = np.concatenate([tv[b, :nt[b], h], V[b, extra, h]])
            r2 = oracle.decode_head(c2, rot, q[b, hq], 0, 0, 1, keep.size, pt[b:b + 1], top_p, tail=(t2k, t2v))
            np.testing.assert_allclose(r["out"], r2["out"], rtol=1e-12, atol=1e-14)
            w2 = r2["w_tail"]
            np.testing.assert_allclose(r["w_tail_only"], w2[:nt[b]], rtol=1e-12, atol=1e-15)
            slots = [1, 3, 4, 6, 7]
            np.testing.assert_allclose(r["w_hp"][slots], w2[nt[b]:], rtol=1e-12, atol=1e-15)
            assert np.all(r["w_hp"][[0, 2, 5]] == 0)


def test_tail_weights_closed_form():
    rng = np.random.default_rng(3)
    q = (2 * rng.standard_normal(D)).astype(np.float32)
    tk = rng.standard_normal((9, D)).astype(np.float16)
    tv = rng.standard_normal((9, D)).astype(np.float16)
    out, w = oracle.attend_with_tail(np.zeros(0), np.zeros((0, D)), q, tk, tv, D, weights=True)
    s = np.array([sum(float(q[j]) * float(tk[i, j]) for j in range(D)) for i in range(9)])
    assert abs(w.sum() - 1.0) < 1e-12
    for i in range(9):
        for j in range(9):
            assert w[i] / w[j] == pytest.approx(np.exp((s[i] - s[j]) / np.sqrt(D)), rel=1e-10)
    np.testing.assert_allclose(out, w @ tv.astype(np.float64), rtol=1e-12)


def _state(seed, C=6, n=10, B=2, Hkv=2, L0=64):
    rng, rot, K, V, q, lens, pt, npages, cache = _setup(L=L0 + n, B=B, Hkv=Hkv, seed=seed)
    hp = oracle.HPTier(B, Hkv, C, D)
    tk = np.zeros((B, n, Hkv, D), np.float16)
    tv = np.zeros_like(tk)
    for b in range(B):
        tk[b] = K[b, L0:L0 + n]
        tv[b] = V[b, L0:L0 + n]
    return rng, K, V, pt, cache, hp, tk, tv, np.full(B, L0, np.int32)


def test_promotion_keeps_the_top_c_by_mass():
    rng, K, V, pt, cache, hp, tk, tv, seq = _state(4)
    before = cache.key_nc.copy()
    C, n = hp.C, tk.shape[1]
    # entries: 4 of the 6 hold older tokens with masses; the tail has distinct masses
    for b in range(2):
        for h in range(2):
            for i, t in enumerate([5, 17, 30, 41]):
                hp.saved[b, h, i] = _mark(cache, b, h, t, pt)
                hp.pos[b, h, i] = t
                hp.mass[b, h, i] = [0.5, 0.05, 0.2, 0.01][i]
                hp.k16[b, h, i] = K[b, t, h]
    tmass = rng.permutation(np.linspace(0.001, 0.4, n * 4)).reshape(2, n, 2).astype(np.float32)
    old = {(b, h): {int(p): float(m) for p, m in zip(hp.pos[b, h], hp.mass[b, h]) if p >= 0}
           for b in range(2) for h in range(2)}
    oracle.hp_update(cache, hp, tk, tv, tmass, n, seq, pt)
    for b in range(2):
        for h in range(2):
            allc = dict(old[(b, h)])
            allc.update({int(seq[b]) + j: float(tmass[b, j, h]) for j in range(n)})
            want = set(sorted(allc, key=lambda p: (-allc[p], p))[:C])
            got = {int(p) for p in hp.pos[b, h] if p >= 0}
            assert got == want
            for i in range(C):
                p = int(hp.pos[b, h, i])
                pg, sl = cache.locate(b, p, pt)
                assert cache.key_nc[pg, h, sl] == oracle.HPTier.MARKER
                assert hp.saved[b, h, i] == before[pg, h, sl]
                assert hp.mass[b, h, i] == pytest.approx(allc[p])
                src = K[b, p, h]
                np.testing.assert_array_equal(hp.k16[b, h, i], src)
            # everything else is unmarked and unchanged
            for p in set(allc) - want:
                pg, sl = cache.locate(b, p, pt)
                assert cache.key_nc[pg, h, sl] == before[pg, h, sl]


def test_promotion_ties_prefer_lower_positions_and_empty_entries_fill_first():
    rng, K, V, pt, cache, hp, tk, tv, seq = _state(5, C=4, n=6)
    tmass = np.full((2, 6, 2), 0.25, np.float32)
    oracle.hp_update(cache, hp, tk, tv, tmass, 6, seq, pt)
    for b in range(2):
        for h in range(2):
            # four empty entries, six equal masses: the first four positions, in entries 0..3
            assert hp.pos[b, h].tolist() == [int(seq[b]) + j for j in range(4)]


def test_promote_then_evict_everything_restores_the_cache():
    rng, K, V, pt, cache, hp, tk, tv, seq = _state(6, C=5, n=8)
    before = cache.key_nc.copy()
    tmass = rng.random((2, 8, 2)).astype(np.float32) + 1.0
    oracle.hp_update(cache, hp, tk, tv, tmass, 8, seq, pt)
    assert (cache.key_nc != before).sum() == 2 * 2 * 5
    # a heavier batch at 8 other positions (the same binary16 rows) evicts every entry
    seq2 = seq - 16
    oracle.hp_update(cache, hp, tk, tv, tmass + 10.0, 8, seq2, pt)
    for b in range(2):
        for h in range(2):
            assert all(int(p) < int(seq[b]) for p in hp.pos[b, h] if p >= 0)
    # emptying the tier through its saved words gives back the original bytes
    for b in range(2):
        for h in range(2):
            for i in range(hp.C):
                if hp.pos[b, h, i] >= 0:
                    pg, sl = cache.locate(b, int(hp.pos[b, h, i]), pt)
                    cache.key_nc[pg, h, sl] = hp.saved[b, h, i]
    np.testing.assert_array_equal(cache.key_nc, before)


def test_all_nan_scores_give_an_empty_topp_set():
    s = np.full(50, np.nan, np.float32)
    r = oracle.topp(s, 0.9, D)
    assert r["idx"].size == 0 and r["bstar"] == -1
    s[7] = 1.0
    r = oracle.topp(s, 0.9, D)
    assert r["idx"].tolist() == [7]
