"""Pins of the oracle's draft depth selection: the expected tokens per round
against a Monte Carlo of the acceptance process and its closed forms, and
the choice against its limits (alpha = 0 takes the cheapest round, a free
draft takes the deepest)."""
import numpy as np
import pytest

import oracle as O


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.75, 1.0])
def test_expected_tokens_closed_form(alpha):
    for K in (1, 3, 7, 15):
        want = K + 1 if alpha == 1.0 else (1 - alpha ** (K + 1)) / (1 - alpha)
        assert abs(O.expected_tokens(K, alpha) - want) < 1e-12


def test_expected_tokens_monte_carlo():
    rng = np.random.default_rng(0)
    alpha, K, n = 0.7, 7, 200000
    kept = (rng.random((n, K)) < alpha).cumprod(axis=1).sum(axis=1)
    assert abs((kept + 1).mean() - O.expected_tokens(K, alpha)) < 4 * (kept.std() / np.sqrt(n))


def test_choose_depth_limits_and_ties():
    Ks, t = [1, 3, 5, 7], [100.0, 150.0, 200.0, 250.0]
    assert O.choose_depth(Ks, t, 0.0, 0.0, 0.0)[0] == 1          # nothing is ever kept
    assert O.choose_depth(Ks, [100.0] * 4, 0.9, 0.0, 0.0)[0] == 7  # a free deeper draft
    assert O.choose_depth([3, 1], [10.0, 10.0], 0.0, 5.0, 0.0)[0] == 1  # tie: the smaller K
    k, rate = O.choose_depth(Ks, t, 0.8, 1000.0, 2.0)
    rates = [O.expected_tokens(K, 0.8) / (ti + 1000.0 + 2.0 * (K + 1)) for K, ti in zip(Ks, t)]
    assert k == Ks[int(np.argmax(rates))] and abs(rate - max(rates)) < 1e-15
