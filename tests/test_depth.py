"""pe_choose_depth (host-only C ABI call, no GPU needed) against the oracle's
choose_depth on random costs and acceptance rates, and its argument errors."""
import numpy as np
import pytest

import oracle as O
from drafting_pe_prepare_amd import binding as pb


def test_choose_depth_matches_oracle():
    rng = np.random.default_rng(1)
    for _ in range(300):
        Ks = sorted(rng.choice(np.arange(1, 33), size=rng.integers(1, 8), replace=False).tolist())
        t = (rng.uniform(100, 2000, len(Ks)) * (1 + 0.1 * np.array(Ks))).tolist()
        alpha = float(rng.choice([0.0, 1.0, rng.uniform(0, 1)]))
        vf, vt = float(rng.uniform(0, 5000)), float(rng.uniform(0, 50))
        k, rate = pb.pe_choose_depth(Ks, t, alpha, vf, vt)
        ko, ro = O.choose_depth(Ks, t, alpha, vf, vt)
        rates = sorted(O.expected_tokens(K, alpha) / (ti + vf + vt * (K + 1)) for K, ti in zip(Ks, t))
        if len(rates) < 2 or rates[-1] - rates[-2] > 1e-12 * rates[-1]:
            assert k == ko
        assert abs(rate - ro) <= 1e-12 * ro


@pytest.mark.parametrize("args", [
    ([], [], 0.5), ([3], [100.0], 1.5), ([3], [100.0], -0.1), ([0], [100.0], 0.5), ([40], [100.0], 0.5),
    ([3], [0.0], 0.5),
])
def test_choose_depth_errors(args):
    with pytest.raises(RuntimeError):
        pb.pe_choose_depth(*args)
