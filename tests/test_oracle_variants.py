"""Pins of the oracle's forward variants against facts other than the oracle itself.

SiLU: closed forms (sigmoid(ln 3) = 3/4; SiLU(x) - SiLU(-x) = x since sigmoid(x) +
sigmoid(-x) = 1). Gaussian router noise: two separate implementations (Python-integer Philox
with the math module, vectorised numpy) agree, and the draws pass a Kolmogorov-Smirnov test
against scipy's standard normal. Temperature schedule: the values the pages' formula gives at
the steps where it is easy to read off. Shared expert: the layer with a shared expert equal to
expert 0, when every token routes to expert 0 with weight 1, is exactly twice the layer
without it; the dense loop and the dispatch path agree with a shared expert and SiLU.
"""
import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import philox


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    ln3 = math.log(3.0)
    assert oracle.silu(np.array([ln3]))[0] == pytest.approx(0.75 * ln3, rel=1e-15)
    x = np.random.default_rng(1).normal(size=1000) * 6
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)
    # tails: SiLU(x) -> x for large x, -> -|x| e^-|x| for very negative x
    assert oracle.silu(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    v = oracle.silu(np.array([-30.0]))[0]
    assert v == pytest.approx(-30.0 * math.exp(-30.0), rel=1e-12)


def test_gaussian_noise_two_implementations_agree():
    seed, T, E, sd = 0x1234_5678_9ABC, 37, 11, 0.05
    g = philox.gaussian_f32(seed, T, E, sd)
    for t, e in [(0, 0), (5, 3), (36, 10), (17, 7)]:
        assert g[t, e] == philox.gaussian_scalar(seed, t, e, sd)
    # the t0 offset addresses the same counters
    np.testing.assert_array_equal(philox.gaussian_f32(seed, 10, E, sd, t0=20), g[20:30])


def test_gaussian_noise_is_standard_normal():
    g2 = philox.gaussian_f32(7, 400, 250, 1.0).astype(np.float64)
    g = g2.ravel()
    n = g.size
    assert abs(g.mean()) < 5 / math.sqrt(n)
    assert abs(g.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert stats.kstest(g, "norm").pvalue > 1e-3
    # noise_std scales the draw (one float32 rounding on each side)
    a = philox.gaussian_f32(7, 50, 20, 0.3).astype(np.float64)
    np.testing.assert_allclose(a, 0.3 * g2[:50, :20], rtol=2 ** -22)


def test_temperature_schedule_values():
    # lpnh.cn page, section 3.3: tau = max(0.5, 1.0 - 0.0001 * step)
    assert oracle.temperature_at(0) == 1.0
    assert oracle.temperature_at(2500) == pytest.approx(0.75)
    assert oracle.temperature_at(5000) == pytest.approx(0.5)
    assert oracle.temperature_at(100_000) == 0.5
    # aberweb.com page, section 3.3: the same floor with rate 0.001
    assert oracle.temperature_at(250, rate=1e-3) == pytest.approx(0.75)
    assert oracle.temperature_at(600, rate=1e-3) == 0.5


def _problem(T=40, d=16, E=4, dff=24, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, d))
    Wg = rng.normal(size=(E, d)) * 0.3
    W1 = rng.normal(size=(E, dff, d)) / math.sqrt(d)
    b1 = rng.normal(size=(E, dff)) * 0.1
    W2 = rng.normal(size=(E, d, dff)) / math.sqrt(dff)
    b2 = rng.normal(size=(E, d)) * 0.1
    return x, Wg, W1, b1, W2, b2


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_shared_expert_doubles_when_it_copies_the_only_routed_expert(act):
    x, Wg, W1, b1, W2, b2 = _problem()
    Wg = np.zeros_like(Wg)                   # all logits 0: every token picks expert 0 (k = 1)
    kw = dict(k=1, capacity_factor=float(Wg.shape[0]), act=act)
    plain = oracle.forward(x, Wg, None, W1, b1, W2, b2, **kw)
    assert np.all(plain["idx"] == 0) and np.all(plain["w"] == 1.0) and plain["drops"].sum() == 0
    with_shared = oracle.forward(x, Wg, None, W1, b1, W2, b2, shared=(W1[0], b1[0], W2[0], b2[0]), **kw)
    np.testing.assert_array_equal(with_shared["y"], 2.0 * plain["y"])


@pytest.mark.parametrize("act", ["gelu", "silu"])
def test_dense_loop_matches_dispatch_path_with_shared_expert(act):
    x, Wg, W1, b1, W2, b2 = _problem(T=50, E=5, seed=11)
    rng = np.random.default_rng(2)
    shared = (rng.normal(size=(32, 16)) / 4, rng.normal(size=32) * 0.1, rng.normal(size=(16, 32)) / 6, None)
    kw = dict(k=2, capacity_factor=0.7, act=act, shared=shared, noise_std=0.2, seed=9, tau=0.8)
    a = oracle.forward(x, Wg, None, W1, b1, W2, b2, **kw)
    assert a["drops"].sum() > 0
    b = oracle.brute_dense(x, Wg, None, W1, b1, W2, b2, **kw)
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)
    rows = [0, 7, 31, 49]
    c = oracle.forward_rows(rows, x, Wg, None, W1, b1, W2, b2, **kw)
    np.testing.assert_allclose(c["y_rows"], a["y"][rows], rtol=1e-12, atol=1e-12)


def test_gaussian_noise_moves_the_routing():
    x, Wg, W1, b1, W2, b2 = _problem(T=200, E=8, seed=4)
    base = oracle.route(x, Wg, None, 2)
    noisy = oracle.route(x, Wg, None, 2, seed=5, noise_std=0.5)
    diff = noisy["s"].astype(np.float64) - base["s"].astype(np.float64)
    # the scores move by the noise itself (tau = 1), so their spread is about noise_std
    assert 0.4 < diff.std() < 0.6
    assert (noisy["idx"] != base["idx"]).any()
