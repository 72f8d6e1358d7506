"""Pins of the oracle's stochastic drafting and rejection-sampling
verification (oracle/pe_sampling.py).

  * the counter-based generator against the published known-answer vectors;
  * Gumbel-max draws against the softmax they must follow (chi-square);
  * the guarantee the pages state -- the verified output keeps the verifier's
    distribution -- checked by Monte Carlo over seeds: the first emitted token
    follows softmax(target / T), and the first draft is kept with probability
    sum_v min(p, q);
  * closed cases: drafter == verifier keeps every draft; a drafter whose
    mass sits where the verifier has none is rejected at once."""
import os

import numpy as np
import pytest
from scipy import stats

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def test_philox_known_answers():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        v = [int(x, 16) for x in r]
        got = O.philox4x32(np.array(v[0:4]), np.array(v[4:6]))
        assert [int(x) for x in got] == v[6:10]


def test_uniform_range_and_streams():
    u = O.uniform(1234, O.STREAM_DRAFT, np.arange(200000), 7)
    assert np.all(u > 0) and np.all(u < 1)
    assert abs(u.mean() - 0.5) < 3e-3 and abs(u.var() - 1 / 12) < 2e-3
    # 23-bit lattice, exact in float32: U * 2^23 - 1/2 is an integer
    assert np.all(np.abs(u * 2 ** 23 - 0.5 - np.round(u * 2 ** 23 - 0.5)) == 0)
    np.testing.assert_array_equal(u.astype(np.float32).astype(np.float64), u)
    u2 = O.uniform(1234, O.STREAM_ACCEPT, np.arange(1000), 7)
    u3 = O.uniform(1235, O.STREAM_DRAFT, np.arange(1000), 7)
    assert not np.array_equal(u[:1000], u2) and not np.array_equal(u[:1000], u3)
    np.testing.assert_array_equal(u[:1000], O.uniform(1234, O.STREAM_DRAFT, np.arange(1000), 7))
    # token uniforms: the four words of block v div 4, in order
    tu = O.token_uniforms(99, O.STREAM_RESIDUAL, 12, 5)
    blk = O.philox4x32(np.array([[c, 5, 0, O.STREAM_RESIDUAL] for c in range(3)]), np.array([99, 0]))
    np.testing.assert_array_equal(tu, (np.floor(blk.reshape(-1).astype(np.float64) / 512) + 0.5) / 2 ** 23)


def _chi2_ok(counts, probs):
    exp = probs * counts.sum()
    return stats.chisquare(counts, exp).pvalue > 1e-4


def test_gumbel_max_draws_follow_the_softmax():
    z = np.array([[1.0, 0.2, -0.5, 2.0, 0.0]])
    T = 0.8
    p = np.exp(O.log_softmax(z, T))[0]
    draws = np.array([O.sample_drafts(z, T, seed)[0] for seed in range(6000)])
    assert _chi2_ok(np.bincount(draws, minlength=5).astype(float), p)


def _rounds(zq, zp, T, n):
    first, kept = [], []
    B, K, V = zq.shape
    for seed in range(n):
        t = O.sample_drafts(zq.reshape(B * K, V), T, seed).reshape(B, K)
        a, nxt = O.rejection_verify(t, zq, zp, T, seed)
        first.append(t[0, 0] if a[0] >= 1 else nxt[0])
        kept.append(a[0] >= 1)
    return np.array(first), np.array(kept)


def test_rejection_sampling_keeps_the_verifier_distribution():
    rng = np.random.default_rng(3)
    V, K, T = 6, 2, 1.0
    zq = rng.normal(0, 1.2, (1, K, V))
    zp = rng.normal(0, 1.2, (1, K + 1, V))
    first, kept = _rounds(zq, zp, T, 6000)
    p0 = np.exp(O.log_softmax(zp[0, 0], T))
    q0 = np.exp(O.log_softmax(zq[0, 0], T))
    assert _chi2_ok(np.bincount(first, minlength=V).astype(float), p0)
    acc = np.minimum(p0, q0).sum()
    assert abs(kept.mean() - acc) < 4 * np.sqrt(acc * (1 - acc) / len(kept))


def test_identical_drafter_keeps_every_draft():
    rng = np.random.default_rng(4)
    V, K = 7, 3
    z = rng.normal(0, 1, (2, K + 1, V))
    for seed in range(50):
        t = O.sample_drafts(z[:, :K].reshape(-1, V), 1.3, seed).reshape(2, K)
        a, nxt = O.rejection_verify(t, z[:, :K], z, 1.3, seed)
        assert np.all(a == K)


def test_disjoint_drafter_is_rejected_at_once_and_the_residual_is_the_verifier():
    V, K = 5, 2
    zq = np.full((1, K, V), -40.0)
    zq[..., 4] = 10.0                       # the drafter always proposes token 4
    zp = np.zeros((1, K + 1, V))
    zp[..., 4] = -40.0                      # which the verifier never takes
    outs = []
    for seed in range(3000):
        t = O.sample_drafts(zq.reshape(-1, V), 1.0, seed).reshape(1, K)
        assert np.all(t == 4)
        a, nxt = O.rejection_verify(t, zq, zp, 1.0, seed)
        assert a[0] == 0 and nxt[0] != 4
        outs.append(nxt[0])
    assert _chi2_ok(np.bincount(outs, minlength=V)[:4].astype(float), np.full(4, 0.25))
