"""Pins of the CPU oracle to things other than itself (closed forms, library routines,
brute force, the pages' stated invariants and hand-worked fixtures under tests/golden/).

Each test names the oracle function it pins and the kind of mistake it would catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy import stats as sstats
from scipy.special import expit

import oracle
from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ capacity
def test_capacity_golden():
    g = _golden("capacity.json")
    for case in g["cases"]:
        C = oracle.capacity(case["T"], case["E"], case["k"], case["c"])
        assert C == case["C"], case
        # the page's code form int(c*T*k/E)+1 differs exactly where c*k*T/E is an integer
        assert int(case["c"] * case["T"] * case["k"] / case["E"]) + 1 == case["int_plus_one"]


def test_capacity_is_exact_on_the_float_value():
    # 1.1 is stored as 1.100000000000000088817841970012523...; 1.1 * 10 / 11 is then just
    # above 1, so the exact ceiling is 2 (a float evaluation would give 1.0000000000000002 -> 2
    # too, but an evaluation that rounds first could give 1).
    assert oracle.capacity(10, 11, 1, 1.1) == 2
    assert oracle.capacity(8, 8, 1, 1.0) == 1
    assert oracle.capacity(3, 7, 1, 1e-300) == 1
    with pytest.raises(ValueError):
        oracle.capacity(4, 2, 1, 0.0)


# ------------------------------------------------------------------ logits
def test_logits_one_hot_router_selects_columns():
    # W_g rows one-hot on column c_e: z[t, e] = x[t, c_e] + b_e. Catches a transposed W_g
    # or a wrong bias axis.
    rng = _rng(1)
    T, d, E = 7, 5, 3
    x = rng.standard_normal((T, d))
    cols = [4, 0, 2]
    Wg = np.zeros((E, d))
    for e, c in enumerate(cols):
        Wg[e, c] = 1.0
    bg = np.array([0.5, -1.0, 2.0])
    z = oracle.logits(x, Wg, bg)
    assert z.shape == (T, E)
    np.testing.assert_array_equal(z, x[:, cols] + bg[None, :])


def test_logits_against_torch_linear():
    rng = _rng(2)
    x = rng.standard_normal((9, 6))
    Wg = rng.standard_normal((4, 6))
    bg = rng.standard_normal(4)
    lin = torch.nn.Linear(6, 4).double()
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(Wg))
        lin.bias.copy_(torch.from_numpy(bg))
        ref = lin(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(oracle.logits(x, Wg, bg), ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ scores / softmax
def test_softmax_uniform_is_exactly_one_over_E():
    for E in (1, 2, 4, 8, 16, 64):
        p = oracle.softmax(np.zeros((3, E), np.float32))
        assert np.all(p == 1.0 / E)


def test_softmax_two_experts_is_logistic():
    rng = _rng(3)
    s = rng.standard_normal((50, 2)) * 5
    p = oracle.softmax(s)
    np.testing.assert_allclose(p[:, 0], expit(s[:, 0] - s[:, 1]), rtol=1e-13, atol=1e-15)


def test_softmax_shift_invariant_and_no_overflow():
    rng = _rng(4)
    s = rng.standard_normal((10, 6))
    np.testing.assert_allclose(oracle.softmax(s), oracle.softmax(s + 700.0), rtol=1e-12)
    p = oracle.softmax(np.array([[1000.0, 0.0, -1000.0]]))
    assert np.all(np.isfinite(p)) and abs(p.sum() - 1) < 1e-15 and p[0, 0] == 1.0


def test_softmax_against_torch():
    rng = _rng(5)
    s = rng.standard_normal((20, 7)) * 3
    ref = torch.softmax(torch.from_numpy(s), dim=-1).numpy()
    np.testing.assert_allclose(oracle.softmax(s), ref, rtol=1e-13, atol=1e-16)


def test_scores_temperature_and_noise_rounding():
    z = np.array([[1.0, 2.0, 3.0]], np.float32)
    g = np.array([[0.5, -0.25, 0.125]], np.float32)
    s = oracle.scores(z, 0.5, g)
    assert s.dtype == np.float32
    np.testing.assert_array_equal(s, np.array([[3.0, 3.5, 6.25]], np.float32))
    np.testing.assert_array_equal(oracle.scores(z), z)


# ------------------------------------------------------------------ top-k
def _topk_bruteforce(row, k):
    # enumerate the key (-s_i, i) by Python's tuple ordering (independent of numpy sort)
    keyed = sorted(range(len(row)), key=lambda i: (-float(row[i]) + 0.0, i))
    return keyed[:k]


def test_topk_matches_bruteforce_with_ties():
    rng = _rng(6)
    for trial in range(200):
        E = int(rng.integers(1, 10))
        k = int(rng.integers(1, E + 1))
        row = rng.integers(-3, 4, size=E).astype(np.float32)   # many exact ties
        if trial % 7 == 0:
            row[:] = 0.0
            row[rng.integers(0, E)] = -0.0
        got = oracle.topk(row[None, :], k)[0].tolist()
        assert got == _topk_bruteforce(row, k), (row, k)


def test_topk_invariant_and_lowest_index_ties():
    s = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, 3.0]], np.float32)
    assert oracle.topk(s, 4)[0].tolist() == [1, 2, 5, 0]
    assert oracle.topk(s, 6)[0].tolist() == [1, 2, 5, 0, 3, 4]    # -0.0 ties +0.0
    assert oracle.topk(np.zeros((1, 5), np.float32), 3)[0].tolist() == [0, 1, 2]
    rng = _rng(7)
    s = rng.standard_normal((100, 16)).astype(np.float32)
    idx = oracle.topk(s, 5)
    for t in range(100):
        sel = set(idx[t].tolist())
        for i in sel:
            for j in range(16):
                if j not in sel:
                    assert s[t, i] > s[t, j] or (s[t, i] == s[t, j] and i < j)
        assert all(s[t, idx[t, a]] >= s[t, idx[t, a + 1]] for a in range(4))


def test_topk_on_logits_equals_topk_on_probabilities():
    # kwkr.cn page, section 2.1: softmax is monotone, so selecting on logits or on
    # probabilities gives the same experts in the same order.
    rng = _rng(8)
    s = rng.standard_normal((300, 12)).astype(np.float32)
    p = oracle.softmax(s)
    idx_s = oracle.topk(s, 3)
    idx_p = np.argsort(-p, axis=1, kind="stable")[:, :3]
    np.testing.assert_array_equal(idx_s, idx_p)
    # and against torch.topk on probabilities (distinct values, so order is unique)
    _, idx_t = torch.topk(torch.from_numpy(p), 3, dim=-1)
    np.testing.assert_array_equal(idx_s, idx_t.numpy())


# ------------------------------------------------------------------ renormalisation
def test_renormalised_weights_sum_to_one_and_keep_ratios():
    rng = _rng(9)
    s = rng.standard_normal((64, 8)).astype(np.float32)
    p = oracle.softmax(s)
    idx = oracle.topk(s, 3)
    w = oracle.renormalise(p, idx)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-15)
    sel = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(w[:, 0] / w[:, 1], sel[:, 0] / sel[:, 1], rtol=1e-13)
    assert np.all(w[:, 0] >= w[:, 1]) and np.all(w[:, 1] >= w[:, 2])


def test_renormalise_special_cases():
    rng = _rng(10)
    s = rng.standard_normal((20, 5)).astype(np.float32)
    p = oracle.softmax(s)
    w1 = oracle.renormalise(p, oracle.topk(s, 1))
    assert np.all(w1 == 1.0)                                   # k = 1: weight exactly 1
    idx = oracle.topk(s, 5)
    wE = oracle.renormalise(p, idx)                            # k = E: weights are p
    np.testing.assert_allclose(wE, np.take_along_axis(p, idx, 1), rtol=1e-14)


# ------------------------------------------------------------------ dispatch
def test_dispatch_golden():
    for case in _golden("dispatch_worked.json")["cases"]:
        idx = np.array(case["idx"])
        C = oracle.capacity(case["T"], case["E"], case["k"], case["c"])
        assert C == case["C"]
        dsp = oracle.dispatch(idx, case["E"], C)
        for key in ("counts", "kept", "offsets", "drops", "dest", "perm"):
            np.testing.assert_array_equal(dsp[key], np.array(case[key]), err_msg=f"{case['name']}:{key}")
        st = oracle.balance_stats(dsp["counts"], np.full((case["T"], case["E"]), 1.0 / case["E"]), case["k"])
        np.testing.assert_allclose(st["f"], case["f"], rtol=1e-15)


def _random_idx(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)])


def test_dispatch_against_quadratic_definition():
    rng = _rng(11)
    for _ in range(40):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 30))
        C = int(rng.integers(1, T + 2))
        idx = _random_idx(rng, T, E, k)
        dsp = oracle.dispatch(idx, E, C)
        # rank from the definition: number of earlier tokens that chose the same expert
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                r = sum(1 for t2 in range(t) if e in idx[t2])
                if r < C:
                    assert dsp["dest"][t, j] == dsp["offsets"][e] + r
                    assert dsp["perm"][dsp["dest"][t, j]] == t
                else:
                    assert dsp["dest"][t, j] == -1
        assert dsp["counts"].sum() == T * k
        assert dsp["kept"].sum() == T * k - dsp["drops"].sum()
        np.testing.assert_array_equal(dsp["kept"], np.minimum(dsp["counts"], C))
        # perm is sorted by (expert, token) and is a bijection onto the kept slots
        rows_e = np.repeat(np.arange(E), dsp["kept"])
        keys = list(zip(rows_e.tolist(), dsp["perm"].tolist()))
        assert keys == sorted(keys) and len(set(keys)) == len(keys)


def test_dispatch_special_cases():
    rng = _rng(12)
    idx = _random_idx(rng, 50, 6, 2)
    dsp = oracle.dispatch(idx, 6, 50)                          # C >= T: nothing dropped
    assert dsp["drops"].sum() == 0 and np.all(dsp["dest"] >= 0)
    dsp1 = oracle.dispatch(idx, 6, 1)                          # C = 1: first arrival only
    for e in range(6):
        first = min(t for t in range(50) if e in idx[t])
        assert dsp1["perm"][dsp1["offsets"][e]] == first
    assert dsp1["kept"].tolist() == [1] * 6


# ------------------------------------------------------------------ experts and GeLU
def test_gelu_against_torch_exact_gelu():
    v = np.linspace(-8, 8, 1001)
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(v), ref, rtol=1e-12, atol=1e-15)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0


def _torch_expert(xr, W1e, b1e, W2e, b2e):
    d, dff = W1e.shape[1], W1e.shape[0]
    net = torch.nn.Sequential(torch.nn.Linear(d, dff), torch.nn.GELU(), torch.nn.Linear(dff, d)).double()
    with torch.no_grad():
        net[0].weight.copy_(torch.from_numpy(W1e))
        net[0].bias.copy_(torch.from_numpy(b1e))
        net[2].weight.copy_(torch.from_numpy(W2e))
        net[2].bias.copy_(torch.from_numpy(b2e))
        return net(torch.from_numpy(xr)).numpy()


def test_single_expert_layer_is_a_dense_ffn():
    # E = 1, k = 1, C >= T: the layer reduces to the textbook FFN Linear -> GELU -> Linear.
    rng = _rng(13)
    T, d, dff = 17, 12, 20
    x = rng.standard_normal((T, d))
    Wg = rng.standard_normal((1, d))
    W1 = rng.standard_normal((1, dff, d)) / math.sqrt(d)
    b1 = rng.standard_normal((1, dff))
    W2 = rng.standard_normal((1, d, dff)) / math.sqrt(dff)
    b2 = rng.standard_normal((1, d))
    out = oracle.forward(x, Wg, None, W1, b1, W2, b2, k=1, capacity_factor=1.0)
    ref = _torch_expert(x, W1[0], b1[0], W2[0], b2[0])
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    assert out["L"] == 1.0


def test_all_experts_layer_is_the_dense_softmax_mixture():
    # k = E and C >= T: y = sum_e softmax(z)_e * FFN_e(x), built here from torch modules.
    rng = _rng(14)
    T, d, dff, E = 11, 8, 16, 3
    x = rng.standard_normal((T, d))
    Wg = rng.standard_normal((E, d))
    bg = rng.standard_normal(E)
    W1 = rng.standard_normal((E, dff, d)) / math.sqrt(d)
    b1 = rng.standard_normal((E, dff))
    W2 = rng.standard_normal((E, d, dff)) / math.sqrt(dff)
    b2 = rng.standard_normal((E, d))
    out = oracle.forward(x, Wg, bg, W1, b1, W2, b2, k=E, capacity_factor=2.0)
    z32 = torch.from_numpy(x @ Wg.T + bg).float().double()     # the oracle routes on fp32 logits
    p = torch.softmax(z32, dim=-1).numpy()
    ref = sum(p[:, e, None] * _torch_expert(x, W1[e], b1[e], W2[e], b2[e]) for e in range(E))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)
    assert abs(out["L"] - 1.0) < 1e-14                        # f uniform when k = E


# ------------------------------------------------------------------ combine vs brute force
def _tiny_problem(rng, T, d, dff, E, with_bias=True, ties=False):
    x = rng.standard_normal((T, d))
    Wg = rng.standard_normal((E, d)) * 0.5
    if ties:
        Wg[:] = 0.0
        Wg[:, 0] = np.round(rng.standard_normal(E))
    bg = rng.standard_normal(E) if with_bias else None
    W1 = rng.standard_normal((E, dff, d)) / math.sqrt(d)
    W2 = rng.standard_normal((E, d, dff)) / math.sqrt(dff)
    b1 = rng.standard_normal((E, dff)) if with_bias else None
    b2 = rng.standard_normal((E, d)) if with_bias else None
    return x, Wg, bg, W1, b1, W2, b2


def test_forward_equals_brute_dense_loop():
    rng = _rng(15)
    for trial in range(25):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 25))
        c = float(rng.choice([0.05, 0.3, 0.75, 1.0, 1.25, 4.0]))
        args = _tiny_problem(rng, T, 6, 10, E, with_bias=bool(trial % 2), ties=(trial % 5 == 0))
        a = oracle.forward(*args, k=k, capacity_factor=c)
        b = oracle.brute_dense(*args, k=k, capacity_factor=c)
        np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(a["dest"] >= 0, b["keep"])
        dropped_all = np.all(a["dest"] < 0, axis=1)
        assert np.all(a["y"][dropped_all] == 0.0)


def test_forward_rows_matches_forward():
    rng = _rng(16)
    args = _tiny_problem(rng, 40, 8, 12, 5)
    a = oracle.forward(*args, k=2, capacity_factor=0.6)
    rows = [0, 3, 17, 39]
    b = oracle.forward_rows(rows, *args, k=2, capacity_factor=0.6)
    np.testing.assert_allclose(b["y_rows"], a["y"][rows], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ balance statistics
def test_balance_golden_uniform():
    for case in _golden("balance_uniform.json")["cases"]:
        E = case["E"]
        f = np.array(case.get("f", [case.get("f_each")] * E), np.float64)
        P = np.array(case.get("P", [case.get("P_each")] * E), np.float64)
        assert abs(E * np.sum(f * P) - case["L"]) < 1e-15
    # through the oracle: W_g = 0 and b_g = 0 make P uniform (exactly 1/E), so L = 1 for any f
    rng = _rng(17)
    T, E, k = 32, 8, 2
    p = oracle.softmax(np.zeros((T, E), np.float32))
    counts = np.bincount(_random_idx(rng, T, E, k).reshape(-1), minlength=E)
    st = oracle.balance_stats(counts, p, k)
    assert st["L"] == 1.0 and np.all(st["P"] == 1.0 / E) and abs(st["f"].sum() - 1) < 1e-15


def test_balance_collapsed_router_gives_E_times_P0():
    # every token to expert 0 (k = 1): f = (1, 0, ...), so L = E * P_0 exactly.
    T, E = 10, 4
    s = np.zeros((T, E), np.float32)
    s[:, 0] = 30.0
    p = oracle.softmax(s)
    st = oracle.balance_stats(np.array([T, 0, 0, 0]), p, 1)
    assert abs(st["L"] - E * p[:, 0].mean()) < 1e-15 and st["L"] > 0.999 * E


def test_balance_matches_pages_one_hot_form():
    # intelliparadigm.com page, section 2.3: (one_hot(idx).mean(0) * softmax.mean(0)).sum() * E
    # for top-1 routing, written with torch ops.
    rng = _rng(18)
    logits = torch.from_numpy(rng.standard_normal((50, 6)).astype(np.float32))
    idx1 = torch.argmax(logits, dim=-1)
    ref = (torch.nn.functional.one_hot(idx1, 6).double().mean(0)
           * torch.softmax(logits.double(), -1).mean(0)).sum() * 6
    s = logits.numpy()
    idx = oracle.topk(s, 1)
    counts = np.bincount(idx[:, 0], minlength=6)
    st = oracle.balance_stats(counts, oracle.softmax(s), 1)
    assert abs(st["L"] - float(ref)) < 1e-12
