"""Seeded synthetic inputs for the MoE layer.

Every tensor has its own numpy PCG64 stream, ``SeedSequence(seed, spawn_key=(stream, chunk))``,
drawn in float32 in chunks of 2**22 elements (so the chunks can be drawn in parallel and the
result does not depend on the thread count), then stored either as float32 or as bfloat16 bit
patterns rounded to nearest even. These arrays are the inputs of both the GPU path and the
oracle; this module holds none of the layer's arithmetic.

Recipes (the second parameter of N(mu, sigma) is the standard deviation):
  gauss      x ~ N(0, 1); W_g ~ N(0, wg_std) or N(0, 1/sqrt(d)); W1 ~ N(0, 1/sqrt(d));
             W2 ~ N(0, 1/sqrt(d_ffn)); no biases.
  zipf_bias  as gauss, plus a router bias b_e = 0.5 * ln(w_e) with Zipf(1.1) weights
             w_e = (e+1)^-1.1 / sum_r r^-1.1 over the expert rank e+1.
  clusters   512 centres mu_m ~ N(0, 1)^d; token t belongs to cluster m_t drawn with
             probability proportional to (m+1)^-1.2; x_t = mu_{m_t} + N(0, 0.1)^d.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import MoEShape

_CHUNK = 1 << 22

# One stream id per tensor.
STREAM_X, STREAM_WG, STREAM_BG, STREAM_W1, STREAM_B1, STREAM_W2, STREAM_B2 = 0, 1, 2, 3, 4, 5, 6
STREAM_CENTRES, STREAM_CLUSTER, STREAM_NOISE = 7, 8, 9
STREAM_W1S, STREAM_B1S, STREAM_W2S, STREAM_B2S = 10, 11, 12, 13
STREAM_DY = 14

N_CLUSTERS = 512
CLUSTER_ZIPF_S = 1.2
CLUSTER_NOISE_STD = 0.1
ROUTER_ZIPF_S = 1.1


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std) array; chunk c of the flat array comes from spawn_key (stream, c)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c: int) -> None:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _bf16_rne(u: np.ndarray) -> np.ndarray:
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    n = u.size
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def conv(c: int) -> bool:
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        if not np.all(np.isfinite(a.reshape(-1)[lo:hi])):
            return False
        out[lo:hi] = _bf16_rne(u[lo:hi])
        return True

    if nchunks <= 1:
        ok = all(conv(c) for c in range(nchunks))
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            ok = all(ex.map(conv, range(nchunks)))
    if not ok:
        raise ValueError("inputs must be finite")
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float64(arr: np.ndarray | None, dtype: str) -> np.ndarray | None:
    """Exact float64 value of a stored tensor (bf16 bit patterns or float32)."""
    if arr is None:
        return None
    if dtype == "bf16" and arr.dtype == np.uint16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def zipf_router_bias(E: int, s: float = ROUTER_ZIPF_S) -> np.ndarray:
    ranks = np.arange(1, E + 1, dtype=np.float64)
    w = ranks ** (-s)
    w /= w.sum()
    return (0.5 * np.log(w)).astype(np.float32)


def cluster_tokens(seed: int, T: int, d: int) -> np.ndarray:
    centres = normal_f32(seed, STREAM_CENTRES, (N_CLUSTERS, d), 1.0)
    pi = np.arange(1, N_CLUSTERS + 1, dtype=np.float64) ** (-CLUSTER_ZIPF_S)
    pi /= pi.sum()
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(STREAM_CLUSTER, 0))))
    m = g.choice(N_CLUSTERS, size=T, p=pi)
    x = normal_f32(seed, STREAM_NOISE, (T, d), CLUSTER_NOISE_STD)
    x += centres[m]
    return x


def make_inputs(cfg: MoEShape, bias_std: float = 0.0) -> dict:
    """All layer inputs of ``cfg`` in storage form.

    Returns a dict with x [T,d], Wg [E,d], bg [E] float32 or None, W1 [E,d_ffn,d],
    b1 [E,d_ffn] or None, W2 [E,d,d_ffn], b2 [E,d] or None. x, W* and b1/b2 are in the
    storage dtype (uint16 bf16 bits or float32); bg is always float32.
    ``bias_std`` > 0 adds N(0, bias_std) expert and router biases (used by small tests).
    """
    T, d, E, dff, seed, dt = cfg.T, cfg.d, cfg.E, cfg.d_ffn, cfg.seed, cfg.dtype
    if cfg.recipe == "clusters":
        x = cluster_tokens(seed, T, d)
    else:
        x = normal_f32(seed, STREAM_X, (T, d), 1.0)
    wg_std = cfg.wg_std if cfg.wg_std is not None else 1.0 / np.sqrt(d)
    Wg = normal_f32(seed, STREAM_WG, (E, d), wg_std)
    W1 = normal_f32(seed, STREAM_W1, (E, dff, d), 1.0 / np.sqrt(d))
    W2 = normal_f32(seed, STREAM_W2, (E, d, dff), 1.0 / np.sqrt(dff))
    bg = b1 = b2 = None
    if cfg.recipe == "zipf_bias":
        bg = zipf_router_bias(E)
    if bias_std > 0.0:
        extra = normal_f32(seed, STREAM_BG, (E,), bias_std)
        bg = extra if bg is None else (bg + extra).astype(np.float32)
        b1 = _store(normal_f32(seed, STREAM_B1, (E, dff), bias_std), dt)
        b2 = _store(normal_f32(seed, STREAM_B2, (E, d), bias_std), dt)
    return {
        "x": _store(x, dt), "Wg": _store(Wg, dt), "bg": bg,
        "W1": _store(W1, dt), "b1": b1, "W2": _store(W2, dt), "b2": b2,
    }


def make_shared_expert(cfg: MoEShape, d_ffn_s: int, bias_std: float = 0.0) -> dict:
    """Weights of one shared expert for ``cfg`` in storage form: W1s [d_ffn_s, d] ~ N(0, 1/sqrt(d)),
    W2s [d, d_ffn_s] ~ N(0, 1/sqrt(d_ffn_s)); b1s, b2s ~ N(0, bias_std) when bias_std > 0."""
    d, seed, dt = cfg.d, cfg.seed, cfg.dtype
    W1s = normal_f32(seed, STREAM_W1S, (d_ffn_s, d), 1.0 / np.sqrt(d))
    W2s = normal_f32(seed, STREAM_W2S, (d, d_ffn_s), 1.0 / np.sqrt(d_ffn_s))
    b1s = b2s = None
    if bias_std > 0.0:
        b1s = _store(normal_f32(seed, STREAM_B1S, (d_ffn_s,), bias_std), dt)
        b2s = _store(normal_f32(seed, STREAM_B2S, (d,), bias_std), dt)
    return {"W1s": _store(W1s, dt), "b1s": b1s, "W2s": _store(W2s, dt), "b2s": b2s}


def make_upstream_grad(cfg: MoEShape, std: float = 1.0) -> np.ndarray:
    """The gradient arriving at the layer's output for the backward pass: dy [T, d] ~ N(0, std),
    in storage form."""
    return _store(normal_f32(cfg.seed, STREAM_DY, (cfg.T, cfg.d), std), cfg.dtype)
