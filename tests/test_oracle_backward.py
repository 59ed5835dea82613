"""Pins of the oracle's backward pass against facts other than its own formulas.

1. Central finite differences of the oracle's forward objective J = sum(dy * y) + lam * L
   along random directions, for every input and parameter tensor. The routing decisions are
   piecewise constant, so the difference quotient is the derivative as long as no decision
   flips inside +-eps (checked). Router tensors use the oracle's float64-score mode, where J
   is smooth; the expert tensors do not touch the routing and use the default float32 scores.
2. torch.autograd on a dense, masked torch formulation of the same layer (every expert on
   every token, masked by the kept slots; the discrete decisions enter as constants, which is
   the pages' statement of what carries gradient).
3. Closed forms of the activation derivatives (GeLU'(0) = 1/2, SiLU'(0) = 1/2, the tails) and
   torch's own derivatives of nn.GELU / nn.SiLU.
"""
import math

import numpy as np
import pytest
import torch

import oracle

D, DFF = 8, 12


def _problem(T=24, E=4, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.normal(size=(T, D)) * scale,
        Wg=rng.normal(size=(E, D)) * 0.7,
        bg=rng.normal(size=E) * 0.3,
        W1=rng.normal(size=(E, DFF, D)) / math.sqrt(D),
        b1=rng.normal(size=(E, DFF)) * 0.2,
        W2=rng.normal(size=(E, D, DFF)) / math.sqrt(DFF),
        b2=rng.normal(size=(E, D)) * 0.2,
        dy=rng.normal(size=(T, D)),
    )


NAMES = ("x", "Wg", "bg", "W1", "b1", "W2", "b2")
GRAD = {"x": "dx", "Wg": "dWg", "bg": "dbg", "W1": "dW1", "b1": "db1", "W2": "dW2", "b2": "db2"}

CASES = [
    # (k, capacity_factor, lam, tau, act, gumbel, noise_std, policy)
    (2, 0.75, 0.3, 0.8, "gelu", False, 0.0, "token"),
    (2, 0.75, 0.0, 1.0, "silu", False, 0.0, "token"),
    (1, 0.6, 1.5, 1.0, "gelu", True, 0.0, "token"),
    (2, 0.6, 0.5, 0.7, "silu", False, 0.4, "random"),
    (2, 0.6, 0.2, 1.0, "gelu", False, 0.0, "reroute"),
    (3, 0.5, 0.1, 1.3, "gelu", False, 0.0, "reroute"),
    (4, 2.0, 0.4, 1.0, "gelu", False, 0.0, "token"),          # k = E, nothing dropped
]


def _kw(case, exact):
    k, c, lam, tau, act, gumbel, noise, policy = case
    return dict(k=k, capacity_factor=c, tau=tau, act=act, gumbel=gumbel, seed=5, noise_std=noise,
                policy=policy, exact_scores=exact)


def _objective(prob, kw, lam):
    out = oracle.forward(*(prob[n] for n in NAMES), **kw)
    return float(np.sum(prob["dy"] * out["y"]) + lam * out["L"]), out


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}-k{c[0]}-{c[4]}" for c in CASES])
def test_directional_finite_differences(case):
    lam = case[2]
    prob = _problem(E=4, seed=CASES.index(case))
    rng = np.random.default_rng(1)
    for name in NAMES:
        exact = name in ("x", "Wg", "bg")
        kw = _kw(case, exact)
        g = oracle.backward(*(prob[n] for n in NAMES), prob["dy"], lam=lam, **{k: v for k, v in kw.items()})
        _, base = _objective(prob, kw, lam)
        assert base["drops"].sum() > 0 or case[1] >= 2.0
        for trial in range(2):
            v = rng.normal(size=prob[name].shape)
            eps = 1e-6
            vals = []
            for sgn in (1, -1):
                p2 = dict(prob)
                p2[name] = prob[name] + sgn * eps * v
                J, out = _objective(p2, kw, lam)
                # no routing decision may flip inside the difference
                np.testing.assert_array_equal(out["idx"], base["idx"])
                np.testing.assert_array_equal(out["dest"], base["dest"])
                vals.append(J)
            fd = (vals[0] - vals[1]) / (2 * eps)
            an = float(np.sum(g[GRAD[name]] * v))
            assert an == pytest.approx(fd, rel=2e-6, abs=1e-8), (name, an, fd)


def _torch_objective(prob, case, g, lam):
    """Dense masked torch formulation; g holds the oracle's routing decisions and noise."""
    k, c, _, tau, act, gumbel, noise, policy = case
    t = {n: torch.tensor(prob[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    E = prob["Wg"].shape[0]
    T = prob["x"].shape[0]
    z = t["x"] @ t["Wg"].T + t["bg"]
    s = (z + torch.tensor(g["noise"], dtype=torch.float64)) / tau
    p = torch.softmax(s, dim=1)
    final = torch.tensor(g["final_idx"], dtype=torch.int64)
    keep = torch.tensor(g["dest"] >= 0)
    pf = torch.gather(p, 1, final)
    w = pf / pf.sum(dim=1, keepdim=True)
    actf = torch.nn.GELU() if act == "gelu" else torch.nn.SiLU()
    y = torch.zeros((T, D), dtype=torch.float64)
    for e in range(E):
        he = actf(t["x"] @ t["W1"][e].T + t["b1"][e])
        oe = he @ t["W2"][e].T + t["b2"][e]
        for j in range(k):
            m = (keep[:, j] & (final[:, j] == e)).to(torch.float64)
            y = y + (m * w[:, j])[:, None] * oe
    f = torch.tensor(g["counts"] / (k * T), dtype=torch.float64)
    L = E * torch.sum(f * p.mean(dim=0))
    J = torch.sum(torch.tensor(prob["dy"]) * y) + lam * L
    J.backward()
    return {GRAD[n]: t[n].grad.numpy() for n in NAMES}


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}-k{c[0]}-{c[4]}" for c in CASES])
def test_matches_torch_autograd(case):
    lam = case[2]
    prob = _problem(T=40, E=4, seed=7)
    kw = _kw(case, True)
    ref = oracle.backward(*(prob[n] for n in NAMES), prob["dy"], lam=lam, **kw)
    z = oracle.logits(prob["x"], prob["Wg"], prob["bg"])
    # the noise the oracle added: recover it from its float64 scores
    noise = ref["route"]["s"] * case[3] - z
    dec = {"noise": noise, "final_idx": ref["final_idx"], "dest": ref["dest"], "counts": ref["dispatch"]["counts"]}
    got = _torch_objective(prob, case, dec, lam)
    for key, val in got.items():
        np.testing.assert_allclose(ref[key], val, rtol=1e-9, atol=1e-11, err_msg=key)


def test_given_float32_scores_match_autograd_through_the_scores():
    # with the device's float32 scores given, the router gradient is that of softmax(s) in s
    prob = _problem(T=30, E=5, seed=3)
    kw = dict(k=2, capacity_factor=0.7, tau=0.9, act="gelu")
    s32 = oracle.route(prob["x"], prob["Wg"], prob["bg"], 2, tau=0.9)["s"]
    g = oracle.backward(*(prob[n] for n in NAMES), prob["dy"], lam=0.25, given_scores=s32, **kw)
    st = torch.tensor(s32.astype(np.float64), requires_grad=True)
    p = torch.softmax(st, dim=1)
    final = torch.tensor(g["final_idx"])
    pf = torch.gather(p, 1, final)
    w = pf / pf.sum(dim=1, keepdim=True)
    keep = torch.tensor((g["dest"] >= 0).astype(np.float64))
    T, E = s32.shape
    f = torch.tensor(g["dispatch"]["counts"] / (2 * T))
    J = torch.sum(torch.tensor(g["dw"]) * w * keep) + 0.25 * E * torch.sum(f * p.mean(dim=0))
    J.backward()
    np.testing.assert_allclose(g["dz"] * 0.9, st.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_activation_derivatives():
    assert oracle.gelu_grad(np.array([0.0]))[0] == 0.5
    assert oracle.silu_grad(np.array([0.0]))[0] == 0.5
    assert oracle.gelu_grad(np.array([40.0]))[0] == pytest.approx(1.0, abs=1e-15)
    assert oracle.silu_grad(np.array([-40.0]))[0] == pytest.approx(0.0, abs=1e-15)
    v = np.linspace(-6, 6, 301)
    for name, mod in (("gelu", torch.nn.GELU()), ("silu", torch.nn.SiLU())):
        tv = torch.tensor(v, requires_grad=True)
        mod(tv).sum().backward()
        ours = oracle.gelu_grad(v) if name == "gelu" else oracle.silu_grad(v)
        np.testing.assert_allclose(ours, tv.grad.numpy(), rtol=1e-13, atol=1e-15)


def test_router_gradient_vanishes_for_one_expert():
    # E = 1: p = 1 whatever the logits, so W_g and b_g get no gradient
    prob = _problem(T=10, E=1, seed=2)
    g = oracle.backward(*(prob[n] for n in NAMES), prob["dy"], k=1, capacity_factor=1.0, lam=0.7)
    assert np.all(g["dWg"] == 0.0) and np.all(g["dbg"] == 0.0)


def test_balance_term_alone():
    # dy = 0: only lam * L drives the router; dz = lam * E / T * p * (f - <p, f>) / tau
    prob = _problem(T=50, E=6, seed=9)
    prob["dy"] = np.zeros_like(prob["dy"])
    lam, tau = 0.8, 1.7
    g = oracle.backward(*(prob[n] for n in NAMES), prob["dy"], k=2, capacity_factor=0.8, lam=lam, tau=tau)
    p = g["route"]["p"]
    f = g["dispatch"]["counts"] / (2 * 50)
    want = lam * 6 / 50 * p * (f[None, :] - (p * f[None, :]).sum(1, keepdims=True)) / tau
    np.testing.assert_allclose(g["dz"], want, rtol=1e-12, atol=1e-15)
    assert np.all(g["dW1"] == 0.0) and np.all(g["dW2"] == 0.0)


@pytest.mark.parametrize("policy", ["token", "random", "reroute"])
def test_sampled_entries_equal_the_full_backward(policy):
    prob = _problem(T=40, E=5, seed=11)
    kw = dict(k=2, capacity_factor=0.7, lam=0.4, tau=0.9, act="silu", policy=policy, seed=3)
    full = oracle.backward(*(prob[n] for n in NAMES), prob["dy"], **kw)
    tokens = [0, 7, 39, 21]
    w2_rows = [(3, 1), (0, 5), (3, 7), (1, 0)]
    w1_rows = [(2, 11), (0, 0), (4, 3)]
    got = oracle.backward_entries(*(prob[n] for n in NAMES), prob["dy"], tokens=tokens, w2_rows=w2_rows,
                                  w1_rows=w1_rows, **kw)
    np.testing.assert_allclose(got["dx"], full["dx"][tokens], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["dz"], full["dz"][tokens], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["dW2"], [full["dW2"][e, m] for e, m in w2_rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["db2"], [full["db2"][e, m] for e, m in w2_rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["dW1"], [full["dW1"][e, n] for e, n in w1_rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(got["db1"], [full["db1"][e, n] for e, n in w1_rows], rtol=1e-12, atol=1e-14)
