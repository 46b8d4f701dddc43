"""Binary64 "ideal" form of the rotated-binary score estimator -- TEST INFRASTRUCTURE ONLY.

Used by the statistical pins (unbiasedness, spread, closed-form mean of the correction).
It evaluates the estimator exactly as defined, with an exact (binary64) orthogonal
rotation and an optional int4 query:

    k' = Q k, q' = Q q, x = sign(k') / sqrt(D)          (sign(0) = +1)
    corr = <x, k' / |k|>
    est  = |k| <x, q~> / corr,   q~ = q' or its int4 dequantization
With a sketch of sk < D coordinates, k' and q' are the first sk rotated coordinates and
x = sign(k')/sqrt(sk); the estimate stays unbiased (the part of q orthogonal to k has
conditional mean zero given the rotated key) and its spread goes as sqrt(1 - corr^2)/corr,
corr ~ sqrt(2 sk / (pi D)): about 1.9 times the full sketch's at sk = D/2.

"RaBitQCache" (abstract; key design) states that its proxy score from randomized rotated
binary quantization is an unbiased estimator of the attention score with a proven error
bound; the exact form above is that of the RaBitQ method (Gao & Long, SIGMOD 2024), which
the pages do not print [outside the pages].
"""
from __future__ import annotations

import numpy as np


def sign_pm1(x):
    return np.where(x < 0, -1.0, 1.0)


def int4_dequant(qp, mode="rne", uniforms=None):
    """Per-vector min/max int4 quantization of the rotated query, returned dequantized.
    mode "rne": round half to even; "stochastic": floor(t + U), U ~ U[0,1) passed in."""
    qp = np.asarray(qp, dtype=np.float64)
    vl = qp.min(axis=-1, keepdims=True)
    vr = qp.max(axis=-1, keepdims=True)
    delta = (vr - vl) / 15.0
    t = np.where(delta > 0, (qp - vl) / np.where(delta > 0, delta, 1.0), 0.0)
    if mode == "rne":
        u = np.clip(np.rint(t), 0, 15)
    else:
        u = np.clip(np.floor(t + uniforms), 0, 15)
    return vl + delta * u


def estimate(Q, k, q, query="exact", uniforms=None, sk=None):
    """Estimator of <k, q> for a batch of rotations Q (n, D, D) or one rotation (D, D).
    sk: sketch width, the first sk rotated coordinates only (default D): a non-square
    projection whose rows are the first sk rows of Q."""
    Q = np.asarray(Q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    D = k.shape[-1]
    sk = D if sk is None else int(sk)
    kp = (Q @ k)[..., :sk]
    qp = (Q @ q)[..., :sk]
    nk = np.linalg.norm(k)
    x = sign_pm1(kp) / np.sqrt(sk)
    corr = np.sum(x * kp, axis=-1) / nk
    if query == "exact":
        qt = qp
    elif query == "rne":
        qt = int4_dequant(qp, "rne")
    else:
        qt = int4_dequant(qp, "stochastic", uniforms)
    return nk * np.sum(x * qt, axis=-1) / corr, corr
