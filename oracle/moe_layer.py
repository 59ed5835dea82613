"""Plain CPU oracle of the sparse MoE FFN layer's forward pass, in float64.

TEST INFRASTRUCTURE. Nothing in the product path imports this module: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg may use it. It shares no
code with the HIP path. Inputs are the stored tensor values converted exactly to float64;
nothing is rounded between steps except where a step below says so.

Sources (pages cited by title or address and section):
  [G]  the kwkr.cn page on sparse activation (news/623730; the page prints no title),
       sections 2.1-2.3
       (gate softmax, top-k on logits, second normalisation, combine, L_balance, capacity,
       dropping) and 3.1-3.2 (Linear-GELU-Linear experts, stable sort by expert, per-expert
       contiguous segments truncated at capacity, weighted scatter-add back to tokens).
  [D]  "MoE模型：动态计算架构解析与实践指南" (intelliparadigm.com), sections 2.1 (expert =
       Linear -> GeLU -> Linear), 2.3 (balance loss = E * sum(one-hot mean * softmax mean)),
       3.1 (dense loop: every expert on every token, masked by routing).
  [L]  "Mixture of Experts (MoE) 原理与工程落地全指南" (lpnh.cn), sections 2.2 (Gumbel noise
       added to the logits, divided by a temperature, then softmax), 2.3 (a shared expert that
       every token uses, plus the routed experts), 2.4 (the squared-usage balance loss and its
       quantile-weighted form), 3.2 (experts Linear -> SiLU -> Linear), 3.3 (the temperature
       schedule tau = max(0.5, 1.0 - 0.0001 * step)), 3.6 (load standard deviation and routing
       entropy as monitored quantities).
  [A]  "为什么92%的AI团队误用MoE？…" (aberweb.com), section 3.3: the same schedule with rate
       0.001.
  [M]  "MoE架构揭秘：参数规模≠计算量…" (mhpn.cn): section 3.1's load-variance loss.
Forward variants (the plain layer is the default of each): SiLU experts ([L] 3.2); Gaussian
router noise noise_std * N(0, 1) added to the logits ([G] 3.3; generator in philox.py); a
shared expert whose output is added to every token's routed sum ([L] 2.3).

Readings taken where the pages leave a step open:
  * top-k selects on the float32 scores s (logits, plus Gumbel noise, over tau); ties go to
    the lower expert index; +0.0 and -0.0 are equal ([G] 2.1 says logits and probabilities
    give the same order and that selection on logits is the safer one).
  * the k selected probabilities are divided by their sum with no epsilon ([G] 2.1).
  * C = ceil(c*k*T/E) from the exact value of the float c ([G] 2.3's formula).
  * slots are ordered token-major (slot = t*k + j) and stably sorted by expert; within an
    expert the first C slots (lowest token index) are kept ([G] 3.2).
  * a dropped slot contributes 0 and the surviving weights are not renormalised ([G] 2.3).
  * f_e = counts before dropping / (k*T); P_e = mean over tokens of the full softmax;
    L = E * sum_e f_e * P_e, without the small outside coefficient ([G] 2.2, [D] 2.3).
  * GeLU is the exact erf form 0.5 v (1 + erf(v / sqrt 2)) (nn.GELU's default; [G] 3.1).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
from scipy.special import erf, expit

from . import philox

SQRT1_2 = 1.0 / math.sqrt(2.0)


# ---------------------------------------------------------------- capacity ([G] 2.3)
def capacity(T: int, E: int, k: int, c: float) -> int:
    """C = ceil(c * k * T / E), in exact rational arithmetic on the float c."""
    if not (T >= 1 and E >= 1 and k >= 1) or not (c > 0) or not math.isfinite(c):
        raise ValueError("bad capacity arguments")
    return math.ceil(Fraction(c) * k * T / E)


# ---------------------------------------------------------------- router ([G] 2.1, [L] 2.2)
def logits(x: np.ndarray, Wg: np.ndarray, bg: np.ndarray | None = None) -> np.ndarray:
    """z[t, e] = sum_c x[t, c] * Wg[e, c] (+ bg[e]); Wg has nn.Linear's [out=E, in=d] layout."""
    z = np.asarray(x, np.float64) @ np.asarray(Wg, np.float64).T
    if bg is not None:
        z = z + np.asarray(bg, np.float64)[None, :]
    return z


def scores(z32: np.ndarray, tau: float = 1.0, g32: np.ndarray | None = None) -> np.ndarray:
    """float32 scores s = ((z + g) / tau), each operation rounded to float32.

    z32 is the float32 logit; g32 the float32 Gumbel noise (None: no noise)."""
    s = np.asarray(z32, np.float32)
    if g32 is not None:
        s = (s + np.asarray(g32, np.float32)).astype(np.float32)
    if tau != 1.0:
        s = (s / np.float32(tau)).astype(np.float32)
    return s


def softmax(s: np.ndarray) -> np.ndarray:
    """Row softmax in float64: exp(s - max s) / sum exp(s - max s)."""
    s = np.asarray(s, np.float64)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, largest first, lower index first on ties."""
    s = np.asarray(s)
    T, E = s.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # Sort key (-s, e): a stable sort of -s keeps ascending e among equal values.
    neg = -np.asarray(s, np.float64)
    neg = np.where(neg == 0.0, 0.0, neg)          # fold -0.0 into +0.0
    order = np.argsort(neg, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def renormalise(p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, idx[t, j]] / sum_j' p[t, idx[t, j']] (no epsilon)."""
    sel = np.take_along_axis(np.asarray(p, np.float64), idx, axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route_from_scores(s: np.ndarray, k: int, exact: bool = False) -> dict:
    """Softmax, top-k and renormalised weights from float32 scores s [T,E] (float64 scores,
    unrounded, when ``exact``)."""
    s = np.asarray(s, np.float64 if exact else np.float32)
    p = softmax(s)
    idx = topk(s, k)
    w = renormalise(p, idx)
    return {"s": s, "p": p, "idx": idx, "w": w}


def route(x, Wg, bg, k, tau=1.0, gumbel=False, seed=0, given_scores=None, noise_std=0.0, exact_scores=False):
    """Router step. Returns z (float64 logits), s (float32 scores), p, idx, w.

    Noise: Gumbel when ``gumbel``, else Gaussian noise of std ``noise_std`` when it is > 0,
    else none. With ``given_scores`` (float32 [T,E]) the routing is re-derived from those
    scores instead of the oracle's own logits (z is still the oracle's float64 logit). With
    ``exact_scores`` the scores are (z + g) / tau in float64, never rounded to float32 (the
    method's definition without the device's float32 scores; smooth in the inputs)."""
    z = logits(x, Wg, bg)
    exact = exact_scores and given_scores is None
    if given_scores is not None:
        s = np.asarray(given_scores, np.float32)
    else:
        if gumbel:
            g32 = philox.gumbel_f32(seed, z.shape[0], z.shape[1])
        elif noise_std > 0.0:
            g32 = philox.gaussian_f32(seed, z.shape[0], z.shape[1], noise_std)
        else:
            g32 = None
        if exact:
            s = (z + (0.0 if g32 is None else np.asarray(g32, np.float64))) / float(tau)
        else:
            s = scores(z.astype(np.float32), tau, g32)
    out = route_from_scores(s, k, exact=exact)
    out["z"] = z
    return out


# ---------------------------------------------------------------- dispatch ([G] 2.3, 3.2)
def dispatch(idx: np.ndarray, E: int, C: int) -> dict:
    """Capacity-limited stable dispatch of the flattened slots (slot = t*k + j).

    Returns counts, kept, offsets, drops [E]; dest [T,k] (row in the expert-sorted buffer,
    -1 when dropped); perm [sum kept] (source token of each row)."""
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    order = np.argsort(flat, kind="stable")          # slots grouped by expert, token order kept
    seg_start = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.empty(T * k, dtype=np.int64)
    rank[order] = np.arange(T * k) - seg_start[flat[order]]
    kept = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)[:-1]]).astype(np.int64)
    keep = rank < C
    dest = np.where(keep, offsets[flat] + rank, -1).reshape(T, k)
    perm = np.empty(int(kept.sum()), dtype=np.int64)
    tok = np.repeat(np.arange(T), k)
    perm[dest.reshape(-1)[keep]] = tok[keep]
    return {"counts": counts, "kept": kept, "offsets": offsets, "drops": counts - kept,
            "dest": dest, "perm": perm, "C": C}


# ---------------------------------------------------------------- experts ([G] 3.1, [D] 2.1)
def gelu(v: np.ndarray) -> np.ndarray:
    return 0.5 * v * (1.0 + erf(v * SQRT1_2))


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v) ([L] 3.2's nn.SiLU); the sigmoid is scipy's expit."""
    return v * expit(v)


ACTIVATIONS = {"gelu": gelu, "silu": silu}


def expert(xr, W1e, b1e, W2e, b2e, act: str = "gelu") -> np.ndarray:
    """One expert on rows xr: Linear(d -> d_ffn) -> activation -> Linear(d_ffn -> d)."""
    h = np.asarray(xr, np.float64) @ np.asarray(W1e, np.float64).T
    if b1e is not None:
        h = h + np.asarray(b1e, np.float64)
    h = ACTIVATIONS[act](h)
    y = h @ np.asarray(W2e, np.float64).T
    if b2e is not None:
        y = y + np.asarray(b2e, np.float64)
    return y


def expert_ffn(x_perm, kept, offsets, W1, b1, W2, b2, act: str = "gelu") -> np.ndarray:
    """Each expert e runs on its own contiguous segment of the expert-sorted rows."""
    y_perm = np.zeros((x_perm.shape[0], W2.shape[1]), dtype=np.float64)
    for e in range(len(kept)):
        n = int(kept[e])
        if n == 0:
            continue
        lo = int(offsets[e])
        y_perm[lo:lo + n] = expert(x_perm[lo:lo + n], W1[e], None if b1 is None else b1[e],
                                   W2[e], None if b2 is None else b2[e], act)
    return y_perm


# ---------------------------------------------------------------- combine ([G] 2.1, 3.2)
def combine(y_perm: np.ndarray, dest: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[t] = sum over kept slots j (in j order) of w[t, j] * y_perm[dest[t, j]]."""
    T, k = dest.shape
    y = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        m = dest[:, j] >= 0
        y[m] += w[m, j, None] * y_perm[dest[m, j]]
    return y


# ---------------------------------------------------------------- statistics ([G] 2.2, [D] 2.3)
def balance_stats(counts: np.ndarray, p: np.ndarray, k: int) -> dict:
    """f_e = counts_e / (k T); P_e = mean_t p[t, e]; L = E * sum_e f_e P_e."""
    T, E = p.shape
    f = np.asarray(counts, np.float64) / float(k * T)
    P = np.asarray(p, np.float64).mean(axis=0)
    return {"f": f, "P": P, "L": float(E * np.sum(f * P))}


# ---------------------------------------------------------------- capacity policies ([M] 3.x)
def dispatch_random(idx: np.ndarray, E: int, C: int, seed: int) -> dict:
    """Random capacity dropping: expert e keeps the C slots with the smallest (priority, t),
    priority = philox.drop_priority(seed)[t, e] (a uniformly random subset of its slots when
    over capacity); kept rows are stored in token order. Same outputs as dispatch()."""
    T, k = idx.shape
    prio = philox.drop_priority(seed, T, E)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int64)
    kept = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)[:-1]]).astype(np.int64)
    dest = np.full((T, k), -1, dtype=np.int64)
    perm = np.empty(int(kept.sum()), dtype=np.int64)
    for e in range(E):
        slots = [(t, j) for t in range(T) for j in range(k) if idx[t, j] == e]      # token order
        chosen = sorted(slots, key=lambda tj: (int(prio[tj[0], e]), tj[0]))[:C]
        keep = sorted(chosen)                                                        # back to token order
        for r, (t, j) in enumerate(keep):
            dest[t, j] = offsets[e] + r
            perm[offsets[e] + r] = t
    return {"counts": counts, "kept": kept, "offsets": offsets, "dest": dest, "perm": perm,
            "drops": counts - kept, "C": C}


def dispatch_reroute(idx: np.ndarray, idx_next: np.ndarray, E: int, C: int) -> dict:
    """Rerouting over-capacity slots to the next-best experts: pass 1 is dispatch() (token
    order); the slots it drops move, in j order within a token, to idx_next[t, 0], idx_next[t,
    1], ... (the token's (k+1)-th, (k+2)-th, ... ranked experts; -1 past the last expert:
    dropped), and pass 2 assigns those slots in slot order (t*k + j) to the capacity left after
    pass 1. Expert e's segment holds its pass-1 rows, then its pass-2 rows. Returns dispatch()'s
    fields (counts are pass-1 counts; kept, drops final) plus `final_idx` [T,k], the expert
    each slot ends at (its pass-1 choice when it had no next expert)."""
    T, k = idx.shape
    d1 = dispatch(idx, E, C)
    rank1 = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if d1["dest"][t, j] >= 0:
                e = idx[t, j]
                rank1[t, j] = d1["dest"][t, j] - d1["offsets"][e]
    kept1 = d1["kept"]
    room = C - kept1
    kept2 = np.zeros(E, dtype=np.int64)
    rank2 = np.full((T, k), -1, dtype=np.int64)
    final_idx = idx.copy()
    for t in range(T):
        m = 0                                       # the token's dropped slots so far
        for j in range(k):
            if d1["dest"][t, j] >= 0:
                continue
            e2 = idx_next[t, m]
            m += 1
            if e2 < 0:
                continue
            final_idx[t, j] = e2
            if kept2[e2] < room[e2]:
                rank2[t, j] = kept2[e2]
                kept2[e2] += 1
    kept = kept1 + kept2
    offsets = np.concatenate([[0], np.cumsum(kept)[:-1]]).astype(np.int64)
    dest = np.full((T, k), -1, dtype=np.int64)
    perm = np.empty(int(kept.sum()), dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if rank1[t, j] >= 0:
                r = offsets[idx[t, j]] + rank1[t, j]
            elif rank2[t, j] >= 0:
                e2 = final_idx[t, j]
                r = offsets[e2] + kept1[e2] + rank2[t, j]
            else:
                continue
            dest[t, j] = r
            perm[r] = t
    # drops[e]: slots that chose e in pass 1 and have no row at the end
    drops = np.bincount(idx[dest < 0].ravel(), minlength=E).astype(np.int64)
    return {"counts": d1["counts"], "kept": kept, "offsets": offsets, "dest": dest, "perm": perm,
            "drops": drops, "C": C, "final_idx": final_idx, "kept1": kept1, "kept2": kept2}


def next_choices(s: np.ndarray, k: int) -> np.ndarray:
    """[T,k]: the (k+1)-th ... (2k)-th ranked experts of each token by score (lower index first
    on ties); -1 past the E-th."""
    T, E = s.shape
    out = np.full((T, k), -1, dtype=np.int64)
    m = min(2 * k, E) - k
    if m > 0:
        out[:, :m] = topk(s, k + m)[:, k:]
    return out


def reweight(p: np.ndarray, final_idx: np.ndarray) -> np.ndarray:
    """w[t, j] = p[t, final_idx[t, j]] / sum_j' p[t, final_idx[t, j']] (renormalise() on the
    experts the slots end at)."""
    return renormalise(p, final_idx)


# ---------------------------------------------------------------- routing statistics
def routing_stats(counts: np.ndarray, p: np.ndarray) -> dict:
    """Load statistics of one batch, none with an outer coefficient (lambda):

      usage_e    = counts_e / T (slots routed to e before capacity, over the tokens; [L] 2.4)
      loss_sq    = sum_e usage_e^2                                   ([L] 2.4, standard form)
      loss_quant = 0.5 Q50(usage) + 0.3 Q90(usage) + 0.2 Q99(usage)  ([L] 2.4, improved form);
                   Qq over the E experts, linear interpolation between order statistics
      loss_var   = sum_e (counts_e - mean_e counts)^2                ([M] 3.1)
      usage_std  = population standard deviation of usage            ([L] 3.6)
      entropy    = mean over tokens of -sum_e p ln p, 0 ln 0 = 0     ([L] 3.6)"""
    counts = np.asarray(counts, np.float64)
    p = np.asarray(p, np.float64)
    T = p.shape[0]
    usage = counts / T
    srt = np.sort(usage)
    E = len(srt)

    def quantile(q):
        h = (E - 1) * q
        lo = int(math.floor(h))
        hi = min(lo + 1, E - 1)
        return srt[lo] + (h - lo) * (srt[hi] - srt[lo])

    plogp = np.where(p > 0.0, p * np.log(np.where(p > 0.0, p, 1.0)), 0.0)
    return {
        "usage": usage,
        "loss_sq": float(np.sum(usage ** 2)),
        "loss_quant": float(0.5 * quantile(0.5) + 0.3 * quantile(0.9) + 0.2 * quantile(0.99)),
        "loss_var": float(np.sum((counts - counts.mean()) ** 2)),
        "usage_std": float(np.sqrt(np.mean((usage - usage.mean()) ** 2))),
        "entropy": float(np.mean(-plogp.sum(axis=1))),
    }


# ---------------------------------------------------------------- whole layer
def shared_expert(x, shared, act: str = "gelu"):
    """The shared expert ([L] 2.3) on every token; ``shared`` = (W1s, b1s, W2s, b2s) or None."""
    if shared is None:
        return None
    W1s, b1s, W2s, b2s = shared
    return expert(x, W1s, b1s, W2s, b2s, act)


def dispatch_policy(r: dict, E: int, C: int, k: int, policy: str, seed: int) -> tuple[dict, np.ndarray]:
    """Dispatch under a capacity policy ("token": dispatch(); "random": dispatch_random();
    "reroute": dispatch_reroute()); returns the dispatch and the combine weights."""
    if policy == "token":
        return dispatch(r["idx"], E, C), r["w"]
    if policy == "random":
        return dispatch_random(r["idx"], E, C, seed), r["w"]
    if policy == "reroute":
        dsp = dispatch_reroute(r["idx"], next_choices(r["s"], k), E, C)
        return dsp, reweight(r["p"], dsp["final_idx"])
    raise ValueError(policy)


def forward(x, Wg, bg, W1, b1, W2, b2, *, k, capacity_factor, tau=1.0, gumbel=False,
            seed=0, given_scores=None, act="gelu", noise_std=0.0, shared=None, policy="token",
            exact_scores=False) -> dict:
    """The layer: route -> dispatch -> gather -> experts -> combine (+ shared expert), plus
    f, P, L and the routing statistics."""
    T, d = x.shape
    E = Wg.shape[0]
    r = route(x, Wg, bg, k, tau, gumbel, seed, given_scores, noise_std, exact_scores)
    C = capacity(T, E, k, capacity_factor)
    dsp, w = dispatch_policy(r, E, C, k, policy, seed)
    x_perm = np.asarray(x, np.float64)[dsp["perm"]]
    y_perm = expert_ffn(x_perm, dsp["kept"], dsp["offsets"], W1, b1, W2, b2, act)
    y = combine(y_perm, dsp["dest"], w)
    ys = shared_expert(x, shared, act)
    if ys is not None:
        y = y + ys
    st = balance_stats(dsp["counts"], r["p"], k)
    out = dict(r)
    out["w"] = w
    out["stats"] = routing_stats(dsp["counts"], r["p"])
    out.update(dsp)
    out.update(st)
    out.update({"x_perm": x_perm, "y_perm": y_perm, "y": y})
    return out


def forward_rows(rows, x, Wg, bg, W1, b1, W2, b2, *, k, capacity_factor, tau=1.0,
                 gumbel=False, seed=0, given_scores=None, act="gelu", noise_std=0.0, shared=None,
                 policy="token") -> dict:
    """The layer's output for selected tokens only, at any size.

    Routing and dispatch are done for all tokens (they decide which slots survive); each
    expert then runs only on the selected tokens' kept slots that chose it, and each
    selected token sums its slots in j order."""
    T, d = x.shape
    E = Wg.shape[0]
    r = route(x, Wg, bg, k, tau, gumbel, seed, given_scores, noise_std)
    C = capacity(T, E, k, capacity_factor)
    dsp, w = dispatch_policy(r, E, C, k, policy, seed)
    final_idx = dsp.get("final_idx", r["idx"])
    rows = np.asarray(rows, np.int64)
    contrib = np.zeros((len(rows), k, W2.shape[1]), dtype=np.float64)
    for e in range(E):
        sel = [(i, j) for i, t in enumerate(rows) for j in range(k)
               if final_idx[t, j] == e and dsp["dest"][t, j] >= 0]
        if not sel:
            continue
        xe = np.asarray(x[[rows[i] for i, _ in sel]], np.float64)
        ye = expert(xe, W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e], act)
        for n, (i, j) in enumerate(sel):
            contrib[i, j] = w[rows[i], j] * ye[n]
    y = np.zeros((len(rows), W2.shape[1]), dtype=np.float64)
    for j in range(k):
        y += contrib[:, j]
    ys = shared_expert(np.asarray(x[rows], np.float64), shared, act)
    if ys is not None:
        y = y + ys
    st = balance_stats(dsp["counts"], r["p"], k)
    out = dict(r)
    out["w"] = w
    out.update(dsp)
    out.update(st)
    out["y_rows"] = y
    return out


# ---------------------------------------------------------------- brute force (tiny sizes)
def brute_dense(x, Wg, bg, W1, b1, W2, b2, *, k, capacity_factor, tau=1.0, gumbel=False,
                seed=0, given_scores=None, act="gelu", noise_std=0.0, shared=None) -> dict:
    """Every expert on every token, masked by routing and capacity ([D] 3.1's dense loop).

    Capacity is applied from its definition: slot (t, j) with expert e survives iff fewer
    than C earlier tokens t' < t chose e. O(T^2 k^2); tiny inputs only."""
    T, d = x.shape
    E = Wg.shape[0]
    r = route(x, Wg, bg, k, tau, gumbel, seed, given_scores, noise_std)
    C = capacity(T, E, k, capacity_factor)
    idx, w = r["idx"], r["w"]
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            earlier = sum(1 for t2 in range(t) if e in idx[t2])
            keep[t, j] = earlier < C
    y = np.zeros((T, W2.shape[1]), dtype=np.float64)
    for e in range(E):
        ye = expert(x, W1[e], None if b1 is None else b1[e], W2[e], None if b2 is None else b2[e], act)
        mask = np.zeros(T, dtype=np.float64)
        for j in range(k):
            mask += np.where((idx[:, j] == e) & keep[:, j], w[:, j], 0.0)
        y += mask[:, None] * ye
    if shared is not None:                   # the shared expert, also on every token
        W1s, b1s, W2s, b2s = shared
        y += expert(x, W1s, b1s, W2s, b2s, act)
    return {"y": y, "keep": keep, "idx": idx, "w": w, "C": C}


# ---------------------------------------------------------------- temperature schedule
def temperature_at(step: int, tau0: float = 1.0, tau_min: float = 0.5, rate: float = 1e-4) -> float:
    """tau_t = max(tau_min, tau0 - rate * t) ([L] 3.3: 0.5, 1.0, 1e-4; [A] 3.3: rate 1e-3)."""
    return max(float(tau_min), float(tau0) - float(rate) * float(step))


# ---------------------------------------------------------------- backward ([G] 2.2, 2.3, 3.3)
def gelu_grad(v: np.ndarray) -> np.ndarray:
    """d/dv of the exact GeLU 0.5 v (1 + erf(v / sqrt 2)): Phi(v) + v phi(v)."""
    return 0.5 * (1.0 + erf(v * SQRT1_2)) + v * np.exp(-0.5 * v * v) / math.sqrt(2.0 * math.pi)


def silu_grad(v: np.ndarray) -> np.ndarray:
    """d/dv of v sigmoid(v): sigmoid(v) (1 + v (1 - sigmoid(v)))."""
    sg = expit(v)
    return sg * (1.0 + v * (1.0 - sg))


ACTIVATION_GRADS = {"gelu": gelu_grad, "silu": silu_grad}


def backward(x, Wg, bg, W1, b1, W2, b2, dy, *, k, capacity_factor, lam=0.0, tau=1.0, gumbel=False, seed=0,
             given_scores=None, act="gelu", noise_std=0.0, policy="token", exact_scores=False) -> dict:
    """Gradients of J = sum(dy * y) + lam * L with respect to x, W_g, b_g, W1, b1, W2, b2.

    What carries gradient ([G] 2.2, 2.3, 3.3): the routing decisions (top-k, capacity, the
    policy) and f are discrete and held fixed; the weights w and the balance term's P are
    continuous. A dropped slot gets no expert-path gradient (its output is masked to zero),
    but its probability still sits in the denominator of the token's weights. Steps:
      o_r = FFN_e(x_t) for each kept slot at row r of expert e; y_t = sum_j w_tj o_r
      dO_r = w_tj dy_t;  dw_tj = <dy_t, o_r> (0 for a dropped slot)
      dW2_e = sum_r dO_r^T h_r; db2_e = sum_r dO_r; da_r = (dO_r W2_e) * act'(a_r)
      dW1_e = sum_r da_r^T x_t; db1_e = sum_r da_r; dx_t += da_r W1_e
      w_tj = p_t,e_j / S_t (S_t = sum over the token's k final experts) =>
      dp_t,e_m += (dw_tm - sum_j dw_tj w_tj) / S_t
      dp_t,e += lam * E f_e / T (L = E sum_e f_e P_e, P_e = mean_t p_t,e)
      ds_t = p_t * (dp_t - <p_t, dp_t>) (softmax); dz = ds / tau (the noise is a constant)
      dW_g = dz^T x; db_g = sum_t dz_t; dx_t += dz_t W_g
    Returns the gradients (float64) and the intermediates dz, dw."""
    x64 = np.asarray(x, np.float64)
    dy64 = np.asarray(dy, np.float64)
    T, d = x64.shape
    E = Wg.shape[0]
    r = route(x, Wg, bg, k, tau, gumbel, seed, given_scores, noise_std, exact_scores)
    C = capacity(T, E, k, capacity_factor)
    dsp, w = dispatch_policy(r, E, C, k, policy, seed)
    final_idx = dsp.get("final_idx", r["idx"])
    dest = dsp["dest"]
    grad = ACTIVATION_GRADS[act]
    fwd = ACTIVATIONS[act]
    dx = np.zeros((T, d))
    dW1 = np.zeros(W1.shape)
    db1 = np.zeros(W1.shape[:2])
    dW2 = np.zeros(W2.shape)
    db2 = np.zeros(W2.shape[:2])
    dw = np.zeros((T, k))
    for e in range(E):
        slots = sorted((int(dest[t, j]), t, j) for t in range(T) for j in range(k)
                       if final_idx[t, j] == e and dest[t, j] >= 0)           # row order of the segment
        if not slots:
            continue
        ts = np.array([t for _, t, _ in slots])
        js = np.array([j for _, _, j in slots])
        W1e, W2e = np.asarray(W1[e], np.float64), np.asarray(W2[e], np.float64)
        a = x64[ts] @ W1e.T
        if b1 is not None:
            a = a + np.asarray(b1[e], np.float64)
        h = fwd(a)
        o = h @ W2e.T
        if b2 is not None:
            o = o + np.asarray(b2[e], np.float64)
        dw[ts, js] = np.sum(dy64[ts] * o, axis=1)
        dO = w[ts, js][:, None] * dy64[ts]
        dW2[e] = dO.T @ h
        db2[e] = dO.sum(axis=0)
        da = (dO @ W2e) * grad(a)
        dW1[e] = da.T @ x64[ts]
        db1[e] = da.sum(axis=0)
        np.add.at(dx, ts, da @ W1e)
    p = r["p"]
    S = np.take_along_axis(p, final_idx, axis=1).sum(axis=1)
    corr = np.sum(dw * w, axis=1)
    dp = np.zeros((T, E))
    for j in range(k):
        np.add.at(dp, (np.arange(T), final_idx[:, j]), (dw[:, j] - corr) / S)
    f = dsp["counts"] / (k * T)
    dp = dp + lam * E * f[None, :] / T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    dz = ds / float(tau)
    dWg = dz.T @ x64
    dbg = dz.sum(axis=0)
    dx = dx + dz @ np.asarray(Wg, np.float64)
    return {"dx": dx, "dWg": dWg, "dbg": dbg, "dW1": dW1, "db1": db1, "dW2": dW2, "db2": db2, "dz": dz, "dw": dw,
            "w": w, "dest": dest, "final_idx": final_idx, "route": r, "dispatch": dsp}


def backward_entries(x, Wg, bg, W1, b1, W2, b2, dy, *, tokens, w2_rows, w1_rows, k, capacity_factor, lam=0.0,
                     tau=1.0, gumbel=False, seed=0, given_scores=None, act="gelu", noise_std=0.0,
                     policy="token") -> dict:
    """Selected entries of backward()'s gradients at any size, by the same steps restricted to
    what they depend on: dx and dz rows of ``tokens``; rows m of dW2_e (and db2_e[m]) for
    (e, m) in ``w2_rows``; rows n of dW1_e (and db1_e[n]) for (e, n) in ``w1_rows``.
    Routing and dispatch cover all tokens; an expert's hidden layer is computed on all its
    rows only when a dW2 row of it is asked for."""
    x64 = np.asarray(x, np.float64)
    dy64 = np.asarray(dy, np.float64)
    T, d = x64.shape
    E = Wg.shape[0]
    r = route(x, Wg, bg, k, tau, gumbel, seed, given_scores, noise_std)
    C = capacity(T, E, k, capacity_factor)
    dsp, w = dispatch_policy(r, E, C, k, policy, seed)
    final_idx = dsp.get("final_idx", r["idx"])
    dest = dsp["dest"]
    grad, fwd = ACTIVATION_GRADS[act], ACTIVATIONS[act]
    p = r["p"]
    f = dsp["counts"] / (k * T)

    def pre(e, xs):
        a = xs @ np.asarray(W1[e], np.float64).T
        return a + np.asarray(b1[e], np.float64) if b1 is not None else a

    def out(e, h):
        o = h @ np.asarray(W2[e], np.float64).T
        return o + np.asarray(b2[e], np.float64) if b2 is not None else o

    def rows_of(e):                      # (t, j) of expert e's kept slots in row order
        sl = sorted((int(dest[t, j]), t, j) for t in range(T) for j in range(k)
                    if final_idx[t, j] == e and dest[t, j] >= 0)
        return np.array([t for _, t, _ in sl], dtype=np.int64), np.array([j for _, _, j in sl], dtype=np.int64)

    res = {"tokens": np.asarray(tokens), "dx": [], "dz": []}
    for t in tokens:
        dxt = np.zeros(d)
        dw = np.zeros(k)
        for j in range(k):
            if dest[t, j] < 0:
                continue
            e = final_idx[t, j]
            a = pre(e, x64[t][None, :])[0]
            dw[j] = dy64[t] @ out(e, fwd(a)[None, :])[0]
            da = (w[t, j] * dy64[t] @ np.asarray(W2[e], np.float64)) * grad(a)
            dxt += da @ np.asarray(W1[e], np.float64)
        S = p[t, final_idx[t]].sum()
        dp = np.zeros(E)
        corr = float(np.sum(dw * w[t]))
        for j in range(k):
            dp[final_idx[t, j]] += (dw[j] - corr) / S
        dp += lam * E * f / T
        dz = p[t] * (dp - np.sum(p[t] * dp)) / float(tau)
        res["dz"].append(dz)
        res["dx"].append(dxt + dz @ np.asarray(Wg, np.float64))
    res["dx"], res["dz"] = np.array(res["dx"]).reshape(len(tokens), d), np.array(res["dz"]).reshape(len(tokens), E)
    res["dW2"], res["db2"] = [], []
    for e in sorted({e for e, _ in w2_rows}):
        ts, js = rows_of(e)
        h = fwd(pre(e, x64[ts])) if len(ts) else np.zeros((0, W1.shape[1]))
        dO = w[ts, js][:, None] * dy64[ts]
        for ee, m in w2_rows:
            if ee == e:
                res["dW2"].append(dO[:, m] @ h)
                res["db2"].append(dO[:, m].sum())
    res["dW1"], res["db1"] = [], []
    for e, n in w1_rows:
        ts, js = rows_of(e)
        xs = x64[ts]
        a_n = xs @ np.asarray(W1[e][n], np.float64) + (float(b1[e][n]) if b1 is not None else 0.0)
        dh_n = (w[ts, js][:, None] * dy64[ts]) @ np.asarray(W2[e][:, n], np.float64)
        da_n = dh_n * grad(a_n)
        res["dW1"].append(da_n @ xs)
        res["db1"].append(da_n.sum())
    # entries in the order of the requests (dW2 rows grouped by expert above: restore)
    order2 = sorted(range(len(w2_rows)), key=lambda i: (w2_rows[i][0], i))
    dW2 = [None] * len(w2_rows)
    db2 = [None] * len(w2_rows)
    for pos, i in enumerate(order2):
        dW2[i], db2[i] = res["dW2"][pos], res["db2"][pos]
    res["dW2"], res["db2"] = np.array(dW2), np.array(db2)
    res["dW1"], res["db1"] = np.array(res["dW1"]), np.array(res["db1"])
    res["dispatch"], res["route"] = dsp, r
    return res
