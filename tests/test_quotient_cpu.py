"""The device's norm/corr quotient (a reciprocal refined by one fma) against IEEE division.

The GPU computes n / c for the binary16 pair of a key record as q0 = n*y, e = fma(-c, q0, n),
q1 = fma(e, y, q0) with y = rcp(c), an approximation within one ulp of 1/c, and takes q0
where q1 is NaN or zero.  The argument for it: q0 is within three ulps of n/c, the remainder
is exact, q1 differs from n/c by less than 2^-20 ulp, and a quotient of two binary16 numbers
is never that close to a rounding midpoint of binary32.  Here the same steps run in numpy
(float64 with one rounding to float32 per step is exact for these fma operands, see below)
for y = RN(1/c) and its two float32 neighbours, over every binary16 numerator and a spread of
binary16 denominators (every exponent, the extreme mantissas, random others, signs, zeros,
infinities and NaN), and the result is compared bit for bit with numpy's float32 division.
"""
import numpy as np


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _fma32(a, b, c):
    # a*b is exact in float64 for float32 a, b (48-bit product).  For the remainder
    # fma(-c, q0, n) the exact sum has a handful of significant bits, so the float64 sum is
    # exact too.  For fma(e, y, q0) the float64 sum may round, by at most 2^-29 float32 ulps,
    # while the exact value lies more than 2^-13 ulps from any float32 rounding midpoint (the
    # argument above), so rounding the double to float32 gives the fused result.
    return _f32(a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64))


def _quotient(n, c, y):
    with np.errstate(invalid="ignore", over="ignore"):  # the zero, infinite and NaN operands
        q0 = _f32(n.astype(np.float64) * y.astype(np.float64))
        e = _fma32(-c, q0, n)
        q1 = _fma32(e, y, q0)
    take0 = np.isnan(q1) | (q1 == 0)
    return np.where(take0, q0, q1)


def _denominators():
    rng = np.random.default_rng(5)
    bits = set()
    for sign in (0, 0x8000):
        for exp in range(32):
            for man in (0, 1, 2, 0x155, 0x2AA, 0x3FD, 0x3FE, 0x3FF):
                bits.add(sign | (exp << 10) | man)
    bits.update(int(b) for b in rng.integers(0, 65536, 1500))
    return np.array(sorted(bits), dtype=np.uint16)


def test_refined_reciprocal_equals_division():
    n = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    checked = 0
    for cb in _denominators():
        c = np.array([cb], dtype=np.uint16).view(np.float16).astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
            ref = n / c[0]
            r0 = _f32(1.0 / c.astype(np.float64))
        ys = [r0]
        if np.isfinite(r0[0]) and r0[0] != 0:
            ys += [np.nextafter(r0, np.float32(np.inf)), np.nextafter(r0, np.float32(-np.inf))]
        for y in ys:
            cc = np.full_like(n, c[0])
            yy = np.full_like(n, y[0])
            q = _quotient(n, cc, yy)
            same = (q.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(q) & np.isnan(ref))
            assert same.all(), (hex(int(cb)), float(y[0]), np.nonzero(~same)[0][:5])
            checked += n.size
    assert checked > 2e8


def test_sign_of_zero_needs_the_fallback():
    # -0 / c: the remainder sum gives +0, so the device takes q0 (which keeps the sign)
    n = np.array([-0.0], np.float32)
    c = np.array([2.0 ** -18], np.float32)
    y = _f32(1.0 / c.astype(np.float64))
    q0 = _f32(n.astype(np.float64) * y.astype(np.float64))
    q1 = _fma32(_fma32(-c, q0, n), y, q0)
    assert np.signbit(q0[0]) and not np.signbit(q1[0])
    assert np.signbit(_quotient(n, c, y)[0])
