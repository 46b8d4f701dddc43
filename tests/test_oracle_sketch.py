"""Pins of the oracle's narrow key sketch: sk < D sign bits per key, the first sk rotated
coordinates (rows 0..sk-1 of the rotation: a non-square random projection, read from
"H1B-KV" key design, a 1-bit key sketch by random projection).  The estimator keeps its
form with sk in place of D in the sign part (x = sign(k'_{<sk})/sqrt(sk)); the norm is the
whole key's and the softmax temperature stays 1/sqrt(D).

Checked against:
  * the full encoding: the sketch bits are its first sk/32 words;
  * a closed form: with the randomized Hadamard rotation, k = diag(sigma) H s / D for a sign
    vector s has k' = s / sqrt(D) exactly, so bits = s >= 0, norm = 1, corr = sqrt(sk/D),
    and the score of k against itself is 1 (= <k, k>) up to the binary16 correction;
  * the binary64 estimator of oracle.ideal on the same binary16 rotation (scores);
  * statistics over Haar rotations: unbiased within 4 standard errors, with a spread that
    grows as sqrt(1 - c^2) / c, c ~ sqrt(2 sk / (pi D)) the correction (about 1.9 times the
    full sketch's at sk = D/2).
"""
import numpy as np
import pytest

import oracle
from oracle import ideal
from workloads import haar_orthogonal, haar_orthogonal_batch

D = 128


def _hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("sk", [32, 64, 96])
def test_sketch_bits_are_a_prefix_of_the_full_encoding(sk):
    rng = np.random.default_rng(1)
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=haar_orthogonal(rng, D).astype(np.float16))
    k = rng.standard_normal((50, D)).astype(np.float32)
    full, ncf = oracle.key_encode(rot, k)
    part, ncp = oracle.key_encode(rot, k, sk)
    np.testing.assert_array_equal(part, full[:, :sk // 32])
    np.testing.assert_array_equal(ncp[:, 0], ncf[:, 0])  # the whole key's norm
    # a narrower sketch sums fewer |k'_r| but divides by a smaller sqrt(sk)
    assert not np.array_equal(ncp[:, 1], ncf[:, 1])


@pytest.mark.parametrize("sk", [32, 64, 128])
def test_closed_form_with_the_hadamard_rotation(sk):
    rng = np.random.default_rng(2)
    sig_bits = rng.integers(0, 2, D)
    signs = np.zeros(D // 32, np.uint32)
    for j in range(D):
        signs[j // 32] |= np.uint32(int(sig_bits[j]) << (j % 32))
    rot = oracle.Rotation(oracle.ROT_HADAMARD, D, signs=signs)
    sigma = np.where(sig_bits == 1, -1.0, 1.0)
    s = np.where(rng.random(D) < 0.5, -1.0, 1.0)
    k = (sigma * (_hadamard(D) @ s) / D).astype(np.float32)  # entries in (1/128) Z: exact
    assert abs(np.linalg.norm(k.astype(np.float64)) - 1.0) < 1e-12
    bits, nc = oracle.key_encode(rot, k[None], sk)
    want = np.zeros(sk // 32, np.uint32)
    for r in range(sk):
        if s[r] > 0:
            want[r // 32] |= np.uint32(1 << (r % 32))
    np.testing.assert_array_equal(bits[0], want)
    assert oracle.f16_value(nc[0, 0]) == 1.0
    assert nc[0, 1] == oracle.f16_bits(np.sqrt(sk / D))
    qe = oracle.query_encode(rot, k[None], sk=sk)
    assert np.all(qe["u"][0, sk:] == 0)
    _, _, sc = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], D, sk)
    assert sc[0] == pytest.approx(1.0, rel=2e-3)


@pytest.mark.parametrize("sk", [64, 96])
def test_scores_match_the_binary64_estimator(sk):
    """The binary32 pipeline (binary16 norm and correction, int4 query) against the binary64
    estimator on the same binary16 rotation, exact query: close, and much closer than the
    full-width estimator would be (the widths differ)."""
    rng = np.random.default_rng(3)
    R16 = haar_orthogonal(rng, D).astype(np.float16)
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=R16)
    k = rng.standard_normal((200, D)).astype(np.float32)
    q = rng.standard_normal(D).astype(np.float32)
    bits, nc = oracle.key_encode(rot, k, sk)
    qe = oracle.query_encode(rot, q[None], sk=sk)
    _, _, sc = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], D, sk)
    Q = R16.astype(np.float64)
    est = np.array([ideal.estimate(Q, k[i], q, "rne", sk=sk)[0] for i in range(len(k))])
    full = np.array([ideal.estimate(Q, k[i], q, "rne")[0] for i in range(len(k))])
    err = np.abs(sc - est) / np.sqrt(np.mean(est ** 2))
    assert err.max() < 5e-3
    assert np.median(np.abs(sc - full)) > 20 * np.median(np.abs(sc - est))


def test_sketch_estimator_unbiased_with_larger_spread():
    rng = np.random.default_rng(4)
    Qs = np.concatenate([haar_orthogonal_batch(rng, 1000, D) for _ in range(6)])
    k = rng.standard_normal(D)
    e = rng.standard_normal(D)
    e -= (e @ k) / (k @ k) * k
    q = 0.3 * k / np.linalg.norm(k) + np.sqrt(1 - 0.09) * e / np.linalg.norm(e)
    q *= np.linalg.norm(k)
    truth = k @ q
    sd = {}
    for sk in (128, 64, 32):
        est, _ = ideal.estimate(Qs, k, q, "exact", sk=sk)
        se = est.std() / np.sqrt(len(est))
        assert abs(est.mean() - truth) < 4 * se, (sk, est.mean(), truth, se)
        sd[sk] = est.std()
    # given the rotated key, the error is |k| beta <x, P Q e> / c with Var <x, P Q e> =
    # (1 - c^2) / (D - 1), so its spread goes as sqrt(1 - c^2) / c, c ~ sqrt(2 sk / (pi D))
    def spread(sk):
        c = np.sqrt(2 * sk / (np.pi * D))
        return np.sqrt(1 - c * c) / c
    assert sd[64] / sd[128] == pytest.approx(spread(64) / spread(128), rel=0.15)   # ~1.94
    assert sd[32] / sd[64] == pytest.approx(spread(32) / spread(64), rel=0.15)     # ~1.57
