"""Philox-4x32-10 and the Gumbel noise the router draws from it.

TEST INFRASTRUCTURE. Nothing in the product path imports this module: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may use it.

Philox-4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11), written here from that paper's
definition: a 4 x 32-bit counter and a 2 x 32-bit key; each of the ten rounds multiplies
counter words 0 and 2 by two fixed odd constants, and builds the next counter from the high
and low halves of those products, XORed with the other two words and the key; the key gets a
Weyl increment (the golden ratio and sqrt(3) - 1 scaled to 32 bits) before every round but
the first.

Gumbel noise (the Gumbel-softmax router of "Mixture of Experts (MoE) 原理与工程落地全指南",
lpnh.cn, section 2.2, and the Top-K Gumbel-Softmax row of chapter 1's table on the aberweb.com
page "为什么92%的AI团队误用MoE？…") is g = -log(-log(u)) with u uniform on (0, 1). Reading
taken here, for a token t, an expert e and a 64-bit seed:
  key = (seed mod 2^32, seed >> 32), counter = (t, e, 0, 0), w0 = word 0 of the output,
  u = (w0 + 1/2) * 2^-32 in float64 (strictly inside (0, 1), so no clamp is needed),
  g = -log(-log(u)) in float64, rounded once to float32.

Gaussian noise (the training-time router noise of the kwkr.cn page on sparse activation,
section 3.3: a standard normal draw per (token, expert) times noise_std, added to the
logits). Reading taken here: from the same block (counter (t, e, 0, 0)), u1 and u2 are words 0
and 1 mapped as above, and n = sqrt(-2 ln u1) cos(2 pi u2) (the Box-Muller transform, G. E. P.
Box and M. E. Muller, "A Note on the Generation of Random Normal Deviates", Ann. Math. Statist.
29, 1958), in float64; noise_std is a float32 parameter (its float32 value is used), and the
noise noise_std * n is rounded once to float32.

Two implementations follow: one on Python integers, one vectorised in numpy. They are
written separately and checked against each other (and against rocRAND's Philox, called as
a library) by the tests.
"""
from __future__ import annotations

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10


def philox4x32_10(counter, key):
    """One Philox-4x32-10 block on Python integers: 4 counter words, 2 key words -> 4 words."""
    x0, x1, x2, x3 = (int(v) & MASK32 for v in counter)
    k0, k1 = (int(v) & MASK32 for v in key)
    for rnd in range(ROUNDS):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        prod0 = PHILOX_M0 * x0
        prod1 = PHILOX_M1 * x2
        x0, x1, x2, x3 = ((prod1 >> 32) ^ x1 ^ k0, prod1 & MASK32,
                          (prod0 >> 32) ^ x3 ^ k1, prod0 & MASK32)
    return x0, x1, x2, x3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox-4x32-10: arrays of counter words (broadcastable) -> 4 uint32 arrays."""
    m = np.uint64(MASK32)
    x = [np.asarray(v, dtype=np.uint64) & m for v in (c0, c1, c2, c3)]
    x0, x1, x2, x3 = np.broadcast_arrays(*x)
    x0, x1, x2, x3 = (a.copy() for a in (x0, x1, x2, x3))
    key0 = np.uint64(int(k0) & MASK32)
    key1 = np.uint64(int(k1) & MASK32)
    sh = np.uint64(32)
    for rnd in range(ROUNDS):
        if rnd > 0:
            key0 = np.uint64((int(key0) + PHILOX_W0) & MASK32)
            key1 = np.uint64((int(key1) + PHILOX_W1) & MASK32)
        p0 = x0 * np.uint64(PHILOX_M0)     # < 2^64: exact in uint64
        p1 = x2 * np.uint64(PHILOX_M1)
        n0 = (p1 >> sh) ^ x1 ^ key0
        n1 = p1 & m
        n2 = (p0 >> sh) ^ x3 ^ key1
        n3 = p0 & m
        x0, x1, x2, x3 = n0, n1, n2, n3
    return tuple(a.astype(np.uint32) for a in (x0, x1, x2, x3))


def seed_key(seed: int) -> tuple[int, int]:
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & MASK32, seed >> 32


def uniform_open(w0) -> np.ndarray:
    """u = (w0 + 1/2) / 2^32 in float64, exactly representable and strictly inside (0, 1)."""
    return (np.asarray(w0, dtype=np.float64) + 0.5) * (2.0 ** -32)


def gumbel_f32(seed: int, T: int, E: int, t0: int = 0) -> np.ndarray:
    """float32 Gumbel noise g[t, e] for tokens t0 .. t0+T-1 and experts 0 .. E-1."""
    k0, k1 = seed_key(seed)
    t = np.arange(t0, t0 + T, dtype=np.uint64)[:, None]
    e = np.arange(E, dtype=np.uint64)[None, :]
    w0, _, _, _ = philox4x32_10_np(t, e, 0, 0, k0, k1)
    u = uniform_open(w0)
    return (-np.log(-np.log(u))).astype(np.float32)


def gumbel_scalar(seed: int, t: int, e: int) -> np.float32:
    """The same g[t, e] through the Python-integer Philox (for cross-checks on a few entries)."""
    import math
    w0 = philox4x32_10((t, e, 0, 0), seed_key(seed))[0]
    u = (w0 + 0.5) * 2.0 ** -32
    return np.float32(-math.log(-math.log(u)))


def gaussian_f32(seed: int, T: int, E: int, noise_std: float, t0: int = 0) -> np.ndarray:
    """float32 Gaussian noise noise_std * n[t, e] for tokens t0 .. t0+T-1, experts 0 .. E-1."""
    k0, k1 = seed_key(seed)
    t = np.arange(t0, t0 + T, dtype=np.uint64)[:, None]
    e = np.arange(E, dtype=np.uint64)[None, :]
    w0, w1, _, _ = philox4x32_10_np(t, e, 0, 0, k0, k1)
    u1, u2 = uniform_open(w0), uniform_open(w1)
    n = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return (float(np.float32(noise_std)) * n).astype(np.float32)


def gaussian_scalar(seed: int, t: int, e: int, noise_std: float) -> np.float32:
    """The same noise through the Python-integer Philox and the math module."""
    import math
    w0, w1, _, _ = philox4x32_10((t, e, 0, 0), seed_key(seed))
    u1, u2 = (w0 + 0.5) * 2.0 ** -32, (w1 + 0.5) * 2.0 ** -32
    sd = float(np.float32(noise_std))
    return np.float32(sd * math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * u2))


def drop_priority(seed: int, T: int, E: int) -> np.ndarray:
    """uint32 priority of slot (token t, expert e) for random capacity dropping: word 2 of the
    Philox block of counter (t, e, 0, 0) (the block the router noise draws words 0 and 1 from)."""
    k0, k1 = seed_key(seed)
    t = np.arange(T, dtype=np.uint64)[:, None]
    e = np.arange(E, dtype=np.uint64)[None, :]
    _, _, w2, _ = philox4x32_10_np(t, e, 0, 0, k0, k1)
    return w2
