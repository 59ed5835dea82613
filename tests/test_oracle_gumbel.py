"""Pins of the oracle's Philox-4x32-10 and Gumbel noise.

* Two separately written Philox implementations (Python integers, vectorised numpy) agree.
* Both agree with rocRAND's Philox-4x32-10 engine, called as a library through its public
  seeding API (tests/helpers/rocrand_philox.cpp, built here with the host compiler).
* The Gumbel draws follow the Gumbel(0, 1) law: mean = Euler's gamma, variance = pi^2/6,
  Kolmogorov-Smirnov against exp(-exp(-g)).
* Gumbel-max: argmax(z + g) picks expert i with probability softmax(z)_i.
* The aberweb.com page's form (logits + g) / tau and the mhpn.cn page's form
  exp((log p_i + g_i)/tau) / sum_j exp((log p_j + g_j)/tau) give the same distribution.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats as sstats

import oracle
from oracle import philox

HELPER = os.path.join(os.path.dirname(__file__), "helpers", "rocrand_philox.cpp")


def test_philox_scalar_and_vector_agree():
    rng = np.random.default_rng(0)
    cs = rng.integers(0, 2 ** 32, size=(300, 4), dtype=np.uint64)
    ks = rng.integers(0, 2 ** 32, size=(300, 2), dtype=np.uint64)
    for c, k in zip(cs, ks):
        a = philox.philox4x32_10(tuple(int(v) for v in c), (int(k[0]), int(k[1])))
        b = philox.philox4x32_10_np(c[0], c[1], c[2], c[3], k[0], k[1])
        assert a == tuple(int(v) for v in b)


def test_philox_is_a_bijection_on_counters_sample():
    # a keyed bijection: distinct counters under one key give distinct blocks
    t = np.arange(4096, dtype=np.uint64)
    w = philox.philox4x32_10_np(t, 0, 0, 0, 7, 9)
    blocks = set(zip(*(a.tolist() for a in w)))
    assert len(blocks) == 4096


def _rocrand_binary(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    inc = "/opt/rocm/include"
    if cxx is None or not os.path.isdir(os.path.join(inc, "rocrand")):
        pytest.skip("no host compiler or rocRAND headers")
    out = str(tmp_path_factory.mktemp("rocrand") / "rocrand_philox")
    subprocess.run([cxx, "-O1", "-D__HIP_PLATFORM_AMD__", "-I", inc, HELPER, "-o", out],
                   check=True, capture_output=True)
    return out


def test_philox_matches_rocrand_library(tmp_path_factory):
    exe = _rocrand_binary(tmp_path_factory)
    rng = np.random.default_rng(1)
    rows = []
    for i in range(400):
        c = [int(v) for v in rng.integers(0, 2 ** 32, size=4)]
        c[1] &= (1 << 30) - 1                     # the helper's (offset, subsequence) form needs c1 < 2^30
        k = [int(v) for v in rng.integers(0, 2 ** 32, size=2)]
        if i < 3:
            c, k = [[0, 0, 0, 0], [i, 5, 0, 0], [65535, 15, 0, 0]][i], [[0, 0], [0, 0], [0, 0]][i]
        rows.append(c + k)
    text = "\n".join(" ".join(str(v) for v in r) for r in rows) + "\n"
    res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    got = [tuple(int(v) for v in line.split()) for line in res.stdout.strip().split("\n")]
    for r, g in zip(rows, got):
        assert philox.philox4x32_10(tuple(r[:4]), tuple(r[4:])) == g, r


def test_gumbel_layout_matches_scalar_path():
    g = philox.gumbel_f32(12345, 33, 7)
    for t in (0, 5, 32):
        for e in (0, 3, 6):
            assert g[t, e] == philox.gumbel_scalar(12345, t, e)
    g2 = philox.gumbel_f32(12345, 10, 7, t0=20)
    np.testing.assert_array_equal(g2, g[20:30])


def test_gumbel_distribution_closed_forms():
    g = philox.gumbel_f32(0, 1000, 1000).astype(np.float64).reshape(-1)   # 10^6 draws
    n = g.size
    assert abs(g.mean() - np.euler_gamma) < 5 * np.sqrt(np.pi ** 2 / 6 / n)
    assert abs(g.var() - np.pi ** 2 / 6) < 0.02
    ks = sstats.kstest(g, lambda v: np.exp(-np.exp(-v)))
    assert ks.pvalue > 1e-3
    assert g.min() > -3.2 and g.max() < 23.0          # u in (0,1) open: bounded noise


def test_gumbel_max_samples_softmax():
    # For k = 1 the noisy top-1 is a sample of softmax(z): chi-square over 200k tokens.
    z = np.array([1.0, 0.0, -0.5, 2.0, 0.3], np.float32)
    T = 200_000
    g = philox.gumbel_f32(99, T, 5)
    s = oracle.scores(np.broadcast_to(z, (T, 5)), 1.0, g)
    idx = oracle.topk(s, 1)[:, 0]
    obs = np.bincount(idx, minlength=5)
    exp = oracle.softmax(z[None, :].astype(np.float64))[0] * T
    chi = sstats.chisquare(obs, exp)
    assert chi.pvalue > 1e-4


def test_gumbel_forms_agree_on_selection():
    # (z + g)/tau and (log softmax(z) + g)/tau differ by a per-row constant over tau, so the
    # top-k and the softmax are the same; selection does not depend on tau > 0.
    rng = np.random.default_rng(3)
    z = rng.standard_normal((500, 9))
    g = philox.gumbel_f32(5, 500, 9).astype(np.float64)
    logp = np.log(oracle.softmax(z))
    for tau in (0.5, 1.0, 2.0):
        a = (z + g) / tau
        b = (logp + g) / tau
        np.testing.assert_array_equal(oracle.topk(a, 3), oracle.topk(b, 3))
        np.testing.assert_allclose(oracle.softmax(a), oracle.softmax(b), rtol=1e-9, atol=1e-15)
    s1 = oracle.scores(z.astype(np.float32), 1.0, g.astype(np.float32))
    s5 = oracle.scores(z.astype(np.float32), 0.5, g.astype(np.float32))
    np.testing.assert_array_equal(oracle.topk(s1, 2), oracle.topk(s5, 2))
