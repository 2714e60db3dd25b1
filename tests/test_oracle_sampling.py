"""Pins of the oracle's temperature sampler (mht18 essay, section 3.2: a
random draw from the softmax of the logits, the temperature scaling them).

- the draw generator against splitmix64's published outputs;
- temperature -> 0 reduces to the greedy argmax exactly;
- the drawn tokens follow softmax(logits / T): a chi-square test over many
  seeds against the probabilities computed directly from the definition.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "splitmix64_vectors.json")


def test_splitmix64_published_outputs():
    g = json.load(open(GOLDEN))
    for v in g["vectors"]:
        for k, want in enumerate(v["outputs"], start=1):
            assert oracle.splitmix64(v["seed"], k) == int(want, 0), (v["seed"], k)


def test_uniform_draws_lie_in_open_unit_interval_and_are_not_degenerate():
    u = np.array([oracle.uniform(7, k) for k in range(1, 20001)])
    assert (u > 0).all() and (u < 1).all()
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005


def test_zero_and_tiny_temperature_give_the_argmax():
    rng = np.random.default_rng(3)
    for trial in range(50):
        lg = rng.standard_normal(300).astype(np.float32)
        want = int(np.argmax(lg))
        assert oracle.sample(lg, 0.0, trial, trial) == want
        # logit / 1e-30 dwarfs any Gumbel draw (|g| < 40 for u in (2^-54, 1))
        assert oracle.sample(lg, 1e-30, trial, trial) == want


@pytest.mark.parametrize("temperature", [0.8, 1.5])
def test_draws_follow_softmax_of_scaled_logits(temperature):
    lg = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.5], np.float32)
    p = np.exp(lg.astype(np.float64) / temperature)
    p /= p.sum()
    n = 30000
    counts = np.zeros(lg.size)
    for s in range(n):
        counts[oracle.sample(lg, temperature, 1000 + s, s % 7)] += 1
    expected = n * p
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    # 5 degrees of freedom: P(chi2 > 25.7) = 1e-4
    assert chi2 < 25.7, (chi2, counts / n, p)


def test_sample_is_the_argmax_of_the_scores():
    rng = np.random.default_rng(5)
    lg = rng.standard_normal(1000).astype(np.float32)
    for pos in range(5):
        sc = oracle.sample_scores(lg, 0.9, 42, pos)
        assert oracle.sample(lg, 0.9, 42, pos) == int(np.argmax(sc))
