"""Pins of the reference nucleus sampler (oracle/sampling.py) against hand-computed cases,
closed forms and the exact distribution it must draw from."""
import math

import numpy as np

from oracle import sampling


def test_hand_computed_example():
    # logits [2, 1, 0, 1, -1] at temperature 1: p0 = e^2 / (e^2 + 2e + 1 + e^-1) ~ 0.5206,
    # p1 = p3 ~ 0.1915 (a tie), p2 ~ 0.0705, p4 ~ 0.0259
    lg = np.array([2.0, 1.0, 0.0, 1.0, -1.0])
    den = math.e ** 2 + 2 * math.e + 1 + math.e ** -1
    p0, p1 = math.e ** 2 / den, math.e / den
    r = sampling.sample(lg, 1.0, 0.5, 0.99)  # p0 alone reaches 0.5
    assert r["token"] == 0 and r["kept"].tolist() == [True, False, False, False, False]
    assert abs(r["mass"] - p0) < 1e-15
    # top_p 0.6 needs a second token: tau = p1, and the tie p3 is kept too
    r = sampling.sample(lg, 1.0, 0.6, 0.6)
    assert r["kept"].tolist() == [True, True, False, True, False]
    assert abs(r["tau"] - p1) < 1e-15 and abs(r["mass"] - (p0 + 2 * p1)) < 1e-15
    assert r["token"] == 1  # 0.6 * mass = 0.542 lies past p0 = 0.521, before p0 + p1
    assert sampling.sample(lg, 1.0, 0.6, 0.9)["token"] == 3  # 0.813: past p0 + p1 = 0.712
    assert sampling.sample(lg, 1.0, 0.6, 0.0)["token"] == 0


def test_top_p_one_keeps_everything_and_u_zero_takes_the_first():
    lg = np.array([0.3, -2.0, 1.5, 0.0])
    r = sampling.sample(lg, 0.7, 1.0, 0.0)
    assert r["kept"].all() and abs(r["mass"] - 1.0) < 1e-15 and r["token"] == 0


def test_small_temperature_is_greedy():
    rng = np.random.default_rng(0)
    lg = rng.normal(size=200)
    for u in (0.0, 0.3, 0.999):
        assert sampling.sample(lg, 1e-3, 0.9, u)["token"] == int(np.argmax(lg))


def test_uniform_logits_are_one_tie():
    V = 1000
    for top_p in (0.05, 0.5, 1.0):
        for u in (0.0, 0.2501, 0.70005, 0.9999):  # off the boundaries u * V = integer
            r = sampling.sample(np.zeros(V), 1.3, top_p, u)
            assert r["kept"].all()  # every token is tied with tau
            assert r["token"] == int(u * V)


def test_draws_follow_the_truncated_distribution():
    # a fine grid of u draws each kept token with frequency p / mass, never a dropped one
    rng = np.random.default_rng(1)
    lg = rng.normal(size=50) * 2
    T, top_p, N = 0.7, 0.8, 200000
    ref = sampling.sample(lg, T, top_p, 0.5)
    p, kept, mass = ref["p"], ref["kept"], ref["mass"]
    counts = np.zeros(50)
    for k in range(N):
        counts[sampling.sample(lg, T, top_p, (k + 0.5) / N)["token"]] += 1
    assert np.all(counts[~kept] == 0)
    np.testing.assert_allclose(counts[kept] / N, p[kept] / mass, atol=2.0 / N)


def test_nucleus_is_minimal():
    rng = np.random.default_rng(2)
    for trial in range(50):
        lg = rng.normal(size=300) * rng.uniform(0.1, 3)
        top_p = rng.uniform(0.05, 1.0)
        r = sampling.sample(lg, rng.uniform(0.3, 2.0), top_p, 0.5)
        p, kept, tau = r["p"], r["kept"], r["tau"]
        assert r["mass"] >= top_p - 1e-12
        # dropping the tokens tied at tau leaves less than top_p
        assert p[kept & (p > tau)].sum() < top_p
        assert np.all(p[kept] >= tau) and np.all(p[~kept] < tau)
