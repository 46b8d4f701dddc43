"""Pins of the oracle's storage format: binary16 rounding, key bit order, value nibbles,
rotations.  Each expected value comes from a library routine, a hand-worked fixture under
tests/golden/ (with its citation) or a closed form -- never from the oracle itself."""
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from workloads import haar_orthogonal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            out[key] = rest.split()
    return out


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.integers(-30, 17, 20000)),
        np.float16(rng.standard_normal(2000)).astype(np.float64) * (1 + 2.0**-11),  # ties
        np.float16(rng.standard_normal(2000)).astype(np.float64) * (1 - 2.0**-12),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0**-24, 2.0**-25,
                  2.0**-25 * 1.0000001, 3 * 2.0**-25, 6.1e-5, 2.0**-14 - 2.0**-25]),
    ])
    got = oracle.f16_bits_array(x)
    ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got, ref)
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    finite = h[(h & 0x7C00) != 0x7C00]
    dec = np.array([oracle.f16_value(int(b)) for b in finite])
    np.testing.assert_array_equal(dec, finite.view(np.float16).astype(np.float64))


def test_key_bit_order_matches_h1ib_bitmap_fixture():
    fx = _read_fixture("bitmap_h1ib.txt")
    signs = fx["signs"][0]
    want = bytes(int(b, 16) for b in fx["bytes"])
    D = 32
    k = np.array([1.0 if c == "+" else -1.0 for c in signs], dtype=np.float32)[None, :]
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=np.eye(D, dtype=np.float16))
    bits, nc = oracle.key_encode(rot, k)
    assert bits.astype("<u4").tobytes() == want
    # decoding the bytes with the page's rule returns the signs
    raw = np.frombuffer(want, dtype=np.uint8)
    dec = np.array([1.0 if (raw[i // 8] >> (i % 8)) & 1 else -1.0 for i in range(D)])
    np.testing.assert_array_equal(dec, k[0])
    # |k| = sqrt(32); corr = sum|k'| / (sqrt(D)|k|) = 32 / 32 = 1
    assert nc[0, 0] == np.float16(np.sqrt(32.0)).view(np.uint16)
    assert nc[0, 1] == np.float16(1.0).view(np.uint16)


def test_zero_counts_as_plus_one_and_zero_key():
    D = 32
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=np.eye(D, dtype=np.float16))
    k = np.zeros((1, D), dtype=np.float32)
    k[0, 3] = -1.0
    bits, nc = oracle.key_encode(rot, k)
    assert bits[0, 0] == 0xFFFFFFFF & ~(1 << 3)
    bits0, nc0 = oracle.key_encode(rot, np.zeros((1, D), np.float32))
    assert bits0[0, 0] == 0xFFFFFFFF
    assert nc0[0, 0] == 0 and nc0[0, 1] == np.float16(1.0).view(np.uint16)


def test_value_nibble_fixture():
    fx = _read_fixture("value_nibbles.txt")
    v = np.array([float(x) for x in fx["values"]], dtype=np.float32)[None, :]
    codes, sz = oracle.value_encode(v, 32, 32)
    assert codes[0].tobytes() == bytes(int(b, 16) for b in fx["bytes"])
    assert sz[0, 0, 0] == int(fx["scale"][0], 16) and sz[0, 0, 1] == int(fx["zero"][0], 16)


@pytest.mark.parametrize("Gv", [32, 64])
def test_value_reconstruction_bound(Gv):
    rng = np.random.default_rng(2)
    D = 128
    v = (rng.standard_normal((500, D)) * np.exp2(rng.integers(-6, 6, (500, 1)))).astype(np.float16)
    codes, sz = oracle.value_encode(v, D, Gv)
    c = np.stack([codes & 15, codes >> 4], axis=-1).reshape(500, D).astype(np.float64)
    sc = sz[..., 0].view(np.float16).astype(np.float64)
    zr = sz[..., 1].view(np.float16).astype(np.float64)
    vf = v.astype(np.float64).reshape(500, D // Gv, Gv)
    vhat = c.reshape(500, D // Gv, Gv) * sc[..., None] + zr[..., None]
    mn, mx = vf.min(-1), vf.max(-1)
    # rounding to the nearest code costs at most half a step, plus the binary16 error of
    # the zero point, plus 15 codes' worth of the binary16 error of the step
    bound = sc / 2 + np.abs(zr - mn) + 15 * np.abs(sc - (mx - mn) / 15) + 1e-12
    err = np.abs(vhat - vf).max(-1)
    assert np.all(err <= bound[...] * (1 + 1e-6))
    assert c.min() >= 0 and c.max() <= 15
    # the max of each group decodes to within half a step, the min to the zero point
    assert np.all(np.abs(zr - mn) <= np.abs(mn) * 2.0**-11 + 2.0**-24)


def test_value_exact_on_grid():
    rng = np.random.default_rng(3)
    D, Gv = 128, 32
    zero = np.float16(-1.25)
    step = np.float16(0.125)
    c = rng.integers(0, 16, (64, D))
    c[:, ::Gv] = 0
    c[:, 1::Gv] = 15
    v = (float(zero) + c * float(step)).astype(np.float32)
    codes, sz = oracle.value_encode(v, D, Gv)
    got = np.stack([codes & 15, codes >> 4], axis=-1).reshape(64, D)
    np.testing.assert_array_equal(got, c)
    assert np.all(sz[..., 0] == step.view(np.uint16)) and np.all(sz[..., 1] == zero.view(np.uint16))


def test_constant_group_gives_zero_scale():
    v = np.full((1, 32), 0.7, dtype=np.float32)
    codes, sz = oracle.value_encode(v, 32, 32)
    assert np.all(codes == 0) and sz[0, 0, 0] == 0 and sz[0, 0, 1] == np.float16(0.7).view(np.uint16)


def test_dense_rotation_matches_numpy_matmul():
    rng = np.random.default_rng(4)
    D = 128
    R16 = haar_orthogonal(rng, D).astype(np.float16)
    rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=R16)
    k = rng.standard_normal((50, D)).astype(np.float16)
    y = oracle.rotate_f64(rot, k)
    ref = k.astype(np.float64) @ R16.astype(np.float64).T
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_hadamard_rotation_matches_scipy(D):
    rng = np.random.default_rng(5)
    signs = rng.integers(0, 2**32, size=D // 32, dtype=np.uint64).astype(np.uint32)
    rot = oracle.Rotation(oracle.ROT_HADAMARD, D, signs=signs)
    sigma = np.array([-1.0 if (signs[j // 32] >> (j % 32)) & 1 else 1.0 for j in range(D)])
    H = scipy.linalg.hadamard(D).astype(np.float64)
    k = rng.standard_normal((20, D)).astype(np.float16)
    y = oracle.rotate_f64(rot, k)
    ref = (k.astype(np.float64) * sigma) @ H.T / np.sqrt(D)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)
    # the rotation preserves norms
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(k.astype(np.float64), axis=1),
                               rtol=1e-12)


def test_key_norm_and_corr_closed_forms():
    rng = np.random.default_rng(6)
    D = 128
    signs = rng.integers(0, 2**32, size=D // 32, dtype=np.uint64).astype(np.uint32)
    rot = oracle.Rotation(oracle.ROT_HADAMARD, D, signs=signs)
    k = rng.standard_normal((300, D)).astype(np.float16)
    bits, nc = oracle.key_encode(rot, k)
    kn = np.linalg.norm(k.astype(np.float64), axis=1)
    np.testing.assert_array_equal(nc[:, 0], kn.astype(np.float16).view(np.uint16))
    corr = nc[:, 1].view(np.float16).astype(np.float64)
    # <x, k'/|k|> with x a sign vector / sqrt(D): between 1/sqrt(D) and 1 (Cauchy-Schwarz)
    assert np.all(corr >= 1 / np.sqrt(D) * (1 - 1e-3)) and np.all(corr <= 1.0)
    # the sign bits reproduce |k'| sum: sum_r s_r k'_r = sum_r |k'_r| = corr sqrt(D) |k|
    y = oracle.rotate_f64(rot, k)
    s = np.array([[1.0 if (bits[i, r // 32] >> (r % 32)) & 1 else -1.0 for r in range(D)]
                  for i in range(len(k))])
    np.testing.assert_allclose((s * y).sum(1), np.abs(y).sum(1), rtol=1e-12)
    np.testing.assert_allclose(corr, np.abs(y).sum(1) / (np.sqrt(D) * kn), rtol=2.0**-11)
