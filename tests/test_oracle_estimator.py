"""Statistical pins of the rotated-binary score estimator.

"RaBitQCache" (abstract; key design) states that its proxy score, built from randomized
rotated binary quantization, is an unbiased estimator of the attention score with a proven
error bound.  The pages do not print the estimator; its form is that of RaBitQ (Gao & Long,
SIGMOD 2024) [outside the pages].  Checked here over many Haar-random rotations:
  * unbiasedness (exact and stochastically rounded int4 query): mean error within 4 SE;
  * closed form of E[corr] = sqrt(D) Gamma(D/2) / (sqrt(pi) Gamma((D+1)/2)) = 0.79944 (D=128);
  * spread of the normalised error ~ sqrt((1 - E[corr]^2)/(D - 1)) / E[corr] = 0.067;
  * est(k, k) = |k|^2 exactly;
  * the oracle's binary32 pipeline (binary16 rotation and scalars, int4 query) on the same
    rotations has no gross bias (a missing or wrong normaliser shows up as ~20%).
"""
import numpy as np
import pytest
from scipy.special import gammaln

import oracle
from oracle import ideal
from workloads import haar_orthogonal_batch

D = 128
S = 20000


def _pair(rng, cos=0.3):
    k = rng.standard_normal(D)
    e = rng.standard_normal(D)
    e -= (e @ k) / (k @ k) * k
    q = cos * k / np.linalg.norm(k) + np.sqrt(1 - cos**2) * e / np.linalg.norm(e)
    return k, q * np.linalg.norm(k) * 0.9


@pytest.fixture(scope="module")
def rotations():
    rng = np.random.default_rng(30)
    return np.concatenate([haar_orthogonal_batch(rng, 1000, D) for _ in range(S // 1000)])


def test_ecorr_closed_form():
    ec = np.exp(0.5 * np.log(D) + gammaln(D / 2) - 0.5 * np.log(np.pi) - gammaln((D + 1) / 2))
    assert abs(ec - 0.79944) < 1e-5
    assert abs(np.sqrt(2 / np.pi) - 0.79788) < 1e-5


def test_unbiased_and_spread(rotations):
    rng = np.random.default_rng(31)
    k, q = _pair(rng)
    truth = k @ q
    est, corr = ideal.estimate(rotations, k, q, "exact")
    err = est - truth
    se = err.std() / np.sqrt(S)
    assert abs(err.mean()) < 4 * se, (err.mean(), se)
    ec = np.exp(0.5 * np.log(D) + gammaln(D / 2) - 0.5 * np.log(np.pi) - gammaln((D + 1) / 2))
    assert abs(corr.mean() - ec) < 4 * corr.std() / np.sqrt(S)
    cos = truth / (np.linalg.norm(k) * np.linalg.norm(q))
    spread = (err / (np.linalg.norm(k) * np.linalg.norm(q) * np.sqrt(1 - cos**2))).std()
    pred = np.sqrt((1 - ec**2) / (D - 1)) / ec
    assert abs(pred - 0.067) < 0.001
    assert abs(spread - pred) < 0.05 * pred, (spread, pred)
    # stochastic int4 rounding of the rotated query keeps the estimator unbiased
    U = np.random.default_rng(32).random((S, D))
    est_sr, _ = ideal.estimate(rotations, k, q, "stochastic", U)
    e2 = est_sr - truth
    assert abs(e2.mean()) < 4 * e2.std() / np.sqrt(S)


def test_estimate_of_key_with_itself_is_norm_squared(rotations):
    rng = np.random.default_rng(33)
    k = rng.standard_normal(D)
    est, _ = ideal.estimate(rotations[:100], k, k, "exact")
    np.testing.assert_allclose(est, k @ k, rtol=1e-12)


def test_binary32_pipeline_has_no_gross_bias(rotations):
    rng = np.random.default_rng(34)
    k, q = _pair(rng)
    k16 = k.astype(np.float16)
    truth = k16.astype(np.float64) @ q.astype(np.float32).astype(np.float64)
    n = 2000
    est = np.empty(n)
    for i in range(n):
        rot = oracle.Rotation(oracle.ROT_DENSE, D, R16=rotations[i].astype(np.float16))
        bits, nc = oracle.key_encode(rot, k16[None, :])
        qe = oracle.query_encode(rot, q.astype(np.float32)[None, :])
        _, _, s = oracle.scores(bits, nc, qe["u"][0], qe["c0"][0], qe["c1"][0], D)
        est[i] = s[0]
    err = est - truth
    scale = np.linalg.norm(k) * np.linalg.norm(q)
    # deterministic rounding of the query may carry a small bias; it is reported, and only
    # a gross bias (above 2% of |k||q|, ~6 standard errors) fails
    assert abs(err.mean()) < 0.02 * scale, (err.mean() / scale)
    assert 0.03 < (err / scale).std() < 0.12
