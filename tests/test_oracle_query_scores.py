"""Pins of the oracle's query encoding and binary x int4 proxy score.

Independent checks: rotations against fp64 library products with a rigorous rounding bound;
the integer score against the bit-plane popcount identity and hand cases; the binary32
score against a binary64 evaluation of the same estimator and a closed-form special case.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from workloads import haar_orthogonal

D = 128


def _dense(seed=10):
    R16 = haar_orthogonal(np.random.default_rng(seed), D).astype(np.float16)
    return oracle.Rotation(oracle.ROT_DENSE, D, R16=R16), R16


def _hadamard(seed=11, d=D):
    signs = np.random.default_rng(seed).integers(0, 2**32, size=d // 32, dtype=np.uint64).astype(np.uint32)
    return oracle.Rotation(oracle.ROT_HADAMARD, d, signs=signs), signs


def test_dense_query_rotation_within_fp32_bound():
    rot, R16 = _dense()
    q = np.random.default_rng(12).standard_normal((40, D)).astype(np.float32)
    qe = oracle.query_encode(rot, q)
    R = R16.astype(np.float64)
    exact = q.astype(np.float64) @ R.T
    # sequential fused chain of D terms: |err| <= gamma_D * sum_j |R_rj q_j|
    u = 2.0**-24
    gamma = D * u / (1 - D * u)
    bound = gamma * (np.abs(q.astype(np.float64)) @ np.abs(R).T)
    assert np.all(np.abs(qe["qrot"] - exact) <= bound)


@pytest.mark.parametrize("d", [32, 128])
def test_hadamard_query_rotation_within_fp32_bound(d):
    rot, signs = _hadamard(d=d)
    q = np.random.default_rng(13).standard_normal((40, d)).astype(np.float32)
    qe = oracle.query_encode(rot, q)
    sigma = np.array([-1.0 if (signs[j // 32] >> (j % 32)) & 1 else 1.0 for j in range(d)])
    H = scipy.linalg.hadamard(d).astype(np.float64)
    exact = (q.astype(np.float64) * sigma) @ H.T / np.sqrt(d)
    # log2(d) levels of binary32 additions plus one multiply
    u = 2.0**-24
    lv = int(np.log2(d)) + 1
    bound = ((1 + u) ** lv - 1) * (np.abs(q.astype(np.float64)) @ np.abs(H).T) / np.sqrt(d) + 1e-30
    assert np.all(np.abs(qe["qrot"] - exact) <= bound * 1.0001)


def test_query_int4_quantization_properties():
    rot, _ = _dense()
    q = np.random.default_rng(14).standard_normal((200, D)).astype(np.float32)
    qe = oracle.query_encode(rot, q)
    qr = qe["qrot"].astype(np.float64)
    vl, dl = qe["vl"].astype(np.float64), qe["delta"].astype(np.float64)
    u = qe["u"].astype(np.float64)
    assert u.min() == 0 and u.max() == 15
    np.testing.assert_array_equal(vl, qr.min(1))
    np.testing.assert_array_equal(qe["u"][np.arange(200), qr.argmin(1)], 0)
    np.testing.assert_array_equal(qe["u"][np.arange(200), qr.argmax(1)], 15)
    qbar = vl[:, None] + dl[:, None] * u
    assert np.all(np.abs(qbar - qr) <= dl[:, None] / 2 * (1 + 1e-5))
    np.testing.assert_array_equal(qe["sumu"], qe["u"].astype(np.int64).sum(1))
    isd = np.float32(1 / np.sqrt(D))
    np.testing.assert_array_equal(qe["c0"], (qe["vl"] * isd).astype(np.float32))
    np.testing.assert_array_equal(qe["c1"], (qe["delta"] * isd).astype(np.float32))


def test_constant_query_gives_zero_codes():
    rot = oracle.Rotation(oracle.ROT_DENSE, 32, R16=np.eye(32, dtype=np.float16))
    qe = oracle.query_encode(rot, np.full((1, 32), 0.5, np.float32))
    assert np.all(qe["u"] == 0) and qe["delta"][0] == 0 and qe["sumu"][0] == 0


def _bits_from_signs(s):
    """(n, D) array of +-1 -> (n, D/32) uint32 words, element r at word r/32 bit r%32."""
    n, d = s.shape
    b = (s > 0).astype(np.uint64).reshape(n, d // 32, 32)
    return (b << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)


def test_integer_score_popcount_identity():
    """A = 2 * sum_j 2^j popcount(bits & plane_j) - sum(u): the bit-plane form of the
    binary x int4 product ("RaBitQCache" key design: binary-INT4 arithmetic)."""
    rng = np.random.default_rng(15)
    for d in (32, 64, 128):
        L = 3000
        s = rng.choice([-1, 1], size=(L, d))
        bits = _bits_from_signs(s)
        u = rng.integers(0, 16, size=d).astype(np.uint8)
        nc = np.tile(np.array([[0x3C00, 0x3C00]], np.uint16), (L, 1))
        A, P, _ = oracle.scores(bits, nc, u, 0.0, 0.0, d)
        planes = [_bits_from_signs(((u.astype(np.int64) >> j) & 1)[None, :] * 2 - 1)[0] for j in range(4)]
        ip = np.zeros(L, dtype=np.int64)
        for j in range(4):
            ip += (1 << j) * np.bitwise_count(bits & planes[j][None, :]).sum(1).astype(np.int64)
        np.testing.assert_array_equal(A, 2 * ip - int(u.astype(np.int64).sum()))
        np.testing.assert_array_equal(P, 2 * np.bitwise_count(bits).sum(1).astype(np.int64) - d)


def test_integer_score_hand_cases():
    d = 32
    u = np.arange(32, dtype=np.uint8) % 16
    su = int(u.sum())
    nc = np.array([[0x3C00, 0x3C00]] * 3, np.uint16)
    bits = np.array([[0xFFFFFFFF], [0x0], [1 << 5]], dtype=np.uint32)
    A, P, _ = oracle.scores(bits, nc, u, 0.0, 0.0, d)
    assert list(A) == [su, -su, 2 * int(u[5]) - su]
    assert list(P) == [32, -32, -30]


def test_binary32_score_matches_binary64_estimator():
    """score = |k| <x, q~> / corr with q~ the dequantized query, evaluated in binary64 on the
    oracle's own encodings: agrees to the binary32 rounding of the combine."""
    rot, R16 = _dense()
    rng = np.random.default_rng(16)
    k = rng.standard_normal((500, D)).astype(np.float16)
    q = rng.standard_normal((1, D)).astype(np.float32)
    bits, nc = oracle.key_encode(rot, k)
    qe = oracle.query_encode(rot, q)
    A, P, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], D)
    sg = np.array([[1.0 if (bits[i, r // 32] >> (r % 32)) & 1 else -1.0 for r in range(D)]
                   for i in range(len(k))])
    qt = qe["vl"][0].astype(np.float64) + qe["delta"][0].astype(np.float64) * qe["u"][0].astype(np.float64)
    nrm = nc[:, 0].view(np.float16).astype(np.float64)
    cor = nc[:, 1].view(np.float16).astype(np.float64)
    ref = nrm * (sg @ qt / np.sqrt(D)) / cor
    scale = nrm * (np.abs(qt).sum() / np.sqrt(D)) / cor
    assert np.all(np.abs(s - ref) <= 8 * 2.0**-24 * scale)


def test_score_of_key_with_itself_closed_form():
    """For k = +-a (all magnitudes equal) and identity rotation, q = k is exactly on the
    int4 grid (codes 0 and 15), corr = 1, and the estimate equals |k|^2 up to the binary16
    rounding of |k|."""
    d = 128
    rot = oracle.Rotation(oracle.ROT_DENSE, d, R16=np.eye(d, dtype=np.float16))
    rng = np.random.default_rng(17)
    for a in (0.5, 1.0, 3.0):
        sg = rng.choice([-1.0, 1.0], size=d)
        k = (a * sg).astype(np.float32)[None, :]
        bits, nc = oracle.key_encode(rot, k)
        assert nc[0, 1] == np.float16(1.0).view(np.uint16)
        qe = oracle.query_encode(rot, k)
        assert set(np.unique(qe["u"][0])) <= {0, 15}
        _, _, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], d)
        nrm16 = float(np.float16(a * np.sqrt(d)))
        np.testing.assert_allclose(s[0], nrm16 * a * np.sqrt(d), rtol=4 * 2.0**-24)
