"""Pins of the oracle's routing statistics by closed forms on constructed batches.

Uniform routing (every expert gets k T / E slots, every p = 1/E): loss_sq = k^2 / E, loss_var =
0, usage_std = 0, entropy = ln E. Evenly spaced usage u_e = e / (E - 1): the q-quantile with
linear interpolation is q itself, so loss_quant = 0.5 * 0.5 + 0.3 * 0.9 + 0.2 * 0.99 = 0.718.
Two experts: loss_var = (a - b)^2 / 2, usage_std = |a - b| / (2 T), entropy of (q, 1 - q) =
-q ln q - (1 - q) ln (1 - q). A one-hot p gives entropy 0 (0 ln 0 = 0).
"""
import math

import numpy as np
import pytest

import oracle


def test_uniform_routing():
    T, E, k = 96, 8, 2
    counts = np.full(E, k * T // E)
    p = np.full((T, E), 1.0 / E)
    st = oracle.routing_stats(counts, p)
    assert st["loss_sq"] == pytest.approx(k * k / E, rel=1e-15)
    assert st["loss_var"] == 0.0 and st["usage_std"] == 0.0
    assert st["entropy"] == pytest.approx(math.log(E), rel=1e-14)
    assert st["loss_quant"] == pytest.approx(k / E, rel=1e-15)    # every quantile of a constant


def test_quantile_loss_on_evenly_spaced_usage():
    E, T = 11, 1000
    counts = np.arange(E) * T // (E - 1)                          # usage e / 10, exactly
    st = oracle.routing_stats(counts[::-1].copy(), np.full((T, E), 1.0 / E))   # order of experts is irrelevant
    assert st["loss_quant"] == pytest.approx(0.5 * 0.5 + 0.3 * 0.9 + 0.2 * 0.99, rel=1e-12)


def test_two_experts_closed_forms():
    T = 200
    a, b = 150, 50
    q = 0.3
    p = np.tile([q, 1.0 - q], (T, 1))
    st = oracle.routing_stats(np.array([a, b]), p)
    assert st["loss_var"] == pytest.approx((a - b) ** 2 / 2)
    assert st["usage_std"] == pytest.approx(abs(a - b) / (2 * T))
    assert st["loss_sq"] == pytest.approx((a / T) ** 2 + (b / T) ** 2)
    assert st["entropy"] == pytest.approx(-q * math.log(q) - (1 - q) * math.log(1 - q), rel=1e-14)


def test_one_hot_probabilities_have_zero_entropy():
    T, E = 10, 4
    p = np.zeros((T, E))
    p[:, 2] = 1.0
    assert oracle.routing_stats(np.array([0, 0, T, 0]), p)["entropy"] == 0.0
