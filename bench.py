#!/usr/bin/env python3
"""Throughput of the sparse MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gumbel_longtail]
                    [--others mixtral_like,switch_skew,decode,tiny_fp32]

One step is one moe_forward call (router + softmax + top-k, capacity dispatch, grouped expert
GEMMs with GeLU, combine and the balance statistic) over one batch of seeded synthetic input
already resident in HBM. Per workload: W untimed warm-up steps, then K cold-cache steps (each
preceded by a 1 GiB write that evicts L2 and the 256 MB MALL and a 512 MiB read that leaves
them clean, timed with HIP events recorded by moe_forward on its stream), then K warm steps
back to back between two device
synchronisations. Prints one JSON line for the headline workload (the largest one by default):
  value          tokens/s of the whole layer from the median cold step (T tokens per step);
  warm           the back-to-back figures beside it;
  row_major      the headline workload again with W1 and W2 in nn.Linear's layout, as a caller
                 hands them over (the headline packs them once, before its warm-up);
  stage_ms       per-stage medians of the cold steps;
  roofline       the headline's dominant expert GEMM kernel: algorithmic flops (2 d d_ffn per
                 kept row) over its mean cold-step duration, against the bf16 dense MFMA peak;
  workloads      the other workloads measured the same way, each with the roofline of its own
                 bound (MFMA; weight streaming for switch_skew, max of the two; weight GB/s for
                 the decode-sized GEMV path);
  measured_peaks what this chip sustains: a plain copy kernel and an MFMA-only loop;
  cpu_baseline   the CPU oracle (numpy float64) on a bounded sample of the headline workload,
                 per stage, with the host's CPU model and thread count.
Where the shape allows it (bf16, d and d_ffn multiples of 256) the forward takes W1 and W2
packed by moe_pack_expert_weights, once before the warm-up, as a server packs them at load.

    python bench.py --summarize-trace DIR --bench-log FILE
prints the rocprofv3 --kernel-trace summary of a traced run of this script (DIR: the -d
directory; FILE: that run's stdout): per-workload averages of the expert kernels over the
timed cold steps, matched to the launches in order.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = "gumbel_longtail"
OTHERS = "mixtral_like,switch_skew,decode,tiny_fp32"
FLUSH_BYTES = 1 << 30
SCRUB_BYTES = 1 << 29
# default size of the CPU oracle's sample (tokens): about 10-30 s of host work
CPU_SAMPLE = {"gumbel_longtail": 32768, "mixtral_like": 4096, "switch_skew": 16384, "decode": 128, "tiny_fp32": 256}


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--others", default=OTHERS,
                    help="comma-separated workloads also measured after the headline one ('' = none)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens of the headline batch the CPU oracle is timed on (-1 = the whole batch, 0 = skip; "
                         "default: a per-workload sample of about 10-30 s)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy and MFMA peak probes")
    ap.add_argument("--traffic", default=None,
                    help="JSON with rocprofv3-measured HBM bytes per launch "
                         "(default: profiles/traffic_<workload>.json)")
    ap.add_argument("--activation", choices=("gelu", "silu"), default="gelu",
                    help="expert activation (forward variant)")
    ap.add_argument("--noise-std", type=float, default=0.0,
                    help="Gaussian router noise std (forward variant; needs a workload without Gumbel noise)")
    ap.add_argument("--shared-d-ffn", type=int, default=0,
                    help="hidden width of a shared expert every token uses (forward variant; 0 = none)")
    ap.add_argument("--drop-policy", choices=("token", "random", "reroute"), default="token",
                    help="what happens to slots past capacity (variant; token = the first C in token order)")
    ap.add_argument("--route-stats", action="store_true",
                    help="also compute the five routing statistics in the timed steps and report them")
    ap.add_argument("--capacity-factor", type=float, default=None,
                    help="override the headline workload's capacity factor (reported in config)")
    ap.add_argument("--train", action="store_true",
                    help="time the training step instead: moe_forward_train + moe_backward (one JSON line)")
    ap.add_argument("--lam", type=float, default=0.01, help="weight of the balance loss in the training step")
    ap.add_argument("--weights", choices=("packed", "row-major"), default="packed",
                    help="expert weight layout of the timed forwards (packed where the shape allows it)")
    ap.add_argument("--no-row-major", action="store_true",
                    help="skip the headline's second measurement with row-major weights (the traffic "
                         "counter runs use this: both layouts' GEMM1 launches share one kernel name)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run the probe copy kernel over this many MiB (3 times) and exit: the "
                         "known-size reference for the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-trace", default=None, help="rocprofv3 output directory of a traced bench run")
    ap.add_argument("--bench-log", default=None, help="stdout of that traced run (its JSON line)")
    ap.add_argument("--summarize-counters", default=None, metavar="FETCH,WRITE,CAL_FETCH,CAL_WRITE",
                    help="four rocprofv3 --pmc output directories (FETCH_SIZE and WRITE_SIZE of a bench run of "
                         "--workload, then of --calibrate-copy-mib 1024): print the traffic JSON")
    return ap.parse_args()


# Sources whose change invalidates a stored traffic measurement of the expert GEMMs.
GEMM_SOURCES = ("sparse_mixture_experts_41_amd/csrc/expert_gemm.hip", "sparse_mixture_experts_41_amd/csrc/moe_common.h",
                "sparse_mixture_experts_41_amd/csrc/tile_plan.h")


def gemm_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(path: str, kernel: str, weights: str):
    """Measured HBM bytes per launch of `kernel`, or None if absent or taken on other code or on
    the other weight layout."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("gemm_source_sha256") != gemm_source_digest() or rec.get("weights", "row-major") != weights:
        return None
    return rec.get("bytes_per_launch", {}).get(kernel)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _median(v):
    v = sorted(v)
    n = len(v)
    return 0.5 * (v[(n - 1) // 2] + v[n // 2])


# ----------------------------------------------------------------------------------- CPU oracle
def cpu_baseline(shape, arrays, n_tokens: int, variant: dict | None = None) -> dict:
    """The oracle as it stands, timed on the host cores on the first n_tokens tokens, stage by
    stage (its forward's own sequence of calls). ``variant``: activation, noise_std, drop policy
    and shared-expert arrays of a forward variant."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from workloads import CONFIGS, bf16_bits_to_f32, make_inputs

    cores = len(os.sched_getaffinity(0))
    dt = shape.dtype

    def val(a):
        if a is None:
            return None
        return bf16_bits_to_f32(a) if (dt == "bf16" and a.dtype == np.uint16) else np.asarray(a, np.float32)

    x = val(arrays["x"])[:n_tokens]
    Wg, bg, W1, b1, W2, b2 = (val(arrays["Wg"]), arrays["bg"], val(arrays["W1"]), val(arrays["b1"]),
                              val(arrays["W2"]), val(arrays["b2"]))
    v = variant or {}
    act, noise, policy = v.get("activation", "gelu"), v.get("noise_std", 0.0), v.get("drop_policy", "token")
    shared = v.get("shared")
    shared = None if shared is None else tuple(val(shared[n]) for n in ("W1s", "b1s", "W2s", "b2s"))
    stages = {}
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        r = oracle.route(x, Wg, bg, shape.k, shape.temperature, shape.gumbel, shape.seed, noise_std=noise)
        t1 = time.perf_counter()
        C = oracle.capacity(n_tokens, shape.E, shape.k, shape.capacity_factor)
        dsp, w = oracle.dispatch_policy(r, shape.E, C, shape.k, policy, shape.seed)
        t2 = time.perf_counter()
        x_perm = np.asarray(x, np.float64)[dsp["perm"]]
        t3 = time.perf_counter()
        y_perm = oracle.expert_ffn(x_perm, dsp["kept"], dsp["offsets"], W1, b1, W2, b2, act)
        t4 = time.perf_counter()
        y = oracle.combine(y_perm, dsp["dest"], w)
        ys = oracle.shared_expert(x, shared, act)
        if ys is not None:
            y = y + ys
        t5 = time.perf_counter()
        st = oracle.balance_stats(dsp["counts"], r["p"], shape.k)
        t6 = time.perf_counter()
        blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                for i in threadpool_info()]
    assert np.isfinite(y).all() and np.isfinite(st["L"])
    stages = {"route": t1 - t0, "dispatch": t2 - t1, "gather": t3 - t2, "experts": t4 - t3, "combine": t5 - t4,
              "stats": t6 - t5}
    total = t6 - t0
    # the tiny float32 configuration, whole, on one thread
    tiny = CONFIGS["tiny_fp32"]
    ta = make_inputs(tiny)
    with threadpool_limits(limits=1):
        s0 = time.perf_counter()
        oracle.forward(ta["x"], ta["Wg"], ta["bg"], ta["W1"], ta["b1"], ta["W2"], ta["b2"], k=tiny.k,
                       capacity_factor=tiny.capacity_factor)
        s1 = time.perf_counter()
    return {"value": n_tokens / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"the whole {shape.name} batch ({n_tokens} tokens)" if n_tokens == shape.T else
                       f"first {n_tokens} of the {shape.T} tokens of the {shape.name} input as one batch "
                       f"(capacity recomputed for {n_tokens} tokens)") + ", numpy float64",
            "seconds": total, "stage_seconds": stages, "cpu_model": cpu_model(), "blas": blas,
            "tiny_fp32_one_thread": {"tokens_per_s": tiny.T / (s1 - s0), "seconds": s1 - s0}}


# --------------------------------------------------------------------------------- training step
def train_step(args, shape, cfg, tensors, variant, ops, torch) -> int:
    """The training step: moe_forward_train then moe_backward on synthetic dy, K timed steps."""
    from workloads import make_upstream_grad

    plan = ops.TrainPlan(cfg, *tensors, keep_routing=False, variant=variant)
    a = make_upstream_grad(shape)
    dy = (torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16) if shape.dtype == "bf16"
          else torch.from_numpy(a).cuda())
    for _ in range(args.warmup):
        plan.run()
        plan.backward(dy, args.lam)
    torch.cuda.synchronize()
    fev = [ops.StageEvents() for _ in range(args.steps)]
    bev = [ops.StageEvents(ops.MOE_BACKWARD_STAGES) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        plan.run(events=fev[i])
        plan.backward(dy, args.lam, events=bev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    fst = {n: 0.0 for n in ops.STAGE_NAMES}
    bst = {n: 0.0 for n in ops.BWD_STAGE_NAMES}
    for evs, acc, names in ((fev, fst, ops.STAGE_NAMES), (bev, bst, ops.BWD_STAGE_NAMES)):
        for ev in evs:
            for n, v in zip(names, ev.accumulate()):
                acc[n] += v / args.steps
            ev.close()
    kept = int(plan.out["kept"].sum().item())
    T, d, E, k, dff = shape.T, shape.d, shape.E, shape.k, shape.d_ffn
    gemm = 2.0 * d * dff * kept                   # one expert product over the kept rows
    bwd_gemms = {n: gemm for n in ("dact_gemm", "dx_gemm", "wgrad_W2", "wgrad_W1")}
    tflops = {n: f / (bst[n] * 1e-3) / 1e12 for n, f in bwd_gemms.items()}
    dom = max(bwd_gemms, key=lambda n: bst[n])
    fwd_ms, bwd_ms = sum(fst.values()), sum(bst.values())
    line = {
        "metric": "MoE-layer training step tokens/sec (forward + backward, bf16, 1 GPU)",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; workloads.make_inputs, make_upstream_grad)",
        "config": {"workload": shape.name, "T": T, "d": d, "E": E, "k": k, "d_ffn": dff,
                   "capacity_factor": shape.capacity_factor, "lam": args.lam, "parallelism": "none (one GPU)"},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": tflops[dom], "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops[dom] / PEAK_BF16_TFLOPS, "traffic": None},
        "forward_ms": fwd_ms,
        "backward_ms": bwd_ms,
        "backward_gemm_tflops": tflops,
        "backward_gemm_frac": {n: v / PEAK_BF16_TFLOPS for n, v in tflops.items()},
        "training_flops_frac": 12.0 * d * dff * kept / ((fwd_ms + bwd_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stage_ms": fst,
        "backward_stage_ms": bst,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


# ------------------------------------------------------------------------------------ peaks
def measure_peaks(ops, torch) -> dict:
    """The probe kernels: a 1 GiB copy (read + write bytes over its time, median of 5) and the
    MFMA-only loop (flops over its time, median of 3)."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ops.probe_copy(src, dst)                                   # warm-up
    copy_ms = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ops.probe_copy(src, dst)
        b.record()
        b.synchronize()
        copy_ms.append(a.elapsed_time(b))
    del src, dst
    wgs, iters = 2048, 8000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    ops.probe_mfma(out, wgs, 100)                              # warm-up
    mfma_ms, flops = [], 0.0
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        flops = ops.probe_mfma(out, wgs, iters)
        b.record()
        b.synchronize()
        mfma_ms.append(a.elapsed_time(b))
    copy_gbs = 2 * n / (_median(copy_ms) * 1e-3) / 1e9
    mfma_tf = flops / (_median(mfma_ms) * 1e-3) / 1e12
    return {"copy_GB/s": copy_gbs, "copy_frac_of_spec": copy_gbs / PEAK_HBM_GBS, "copy_bytes": 2 * n,
            "mfma_bf16_TFLOP/s": mfma_tf, "mfma_frac_of_spec": mfma_tf / PEAK_BF16_TFLOPS,
            "mfma_probe": f"{wgs} workgroups x 4 waves x 16 chains x {iters} v_mfma_f32_16x16x32_bf16",
            "kernels": "probe_copy_kernel, probe_mfma_kernel (csrc/probe.hip)"}


# ------------------------------------------------------------------------------ one workload
class Measured:
    pass


def measure_workload(shape, args, ops, torch, variant_args=None, capacity_factor=None, arrays=None,
                     weights=None) -> Measured:
    """Inputs (or the given arrays of the same shape), plan, W warm-up steps, K cold steps
    (events), K warm steps (host clock). `weights` overrides args.weights."""
    import numpy as np

    from workloads import make_inputs, make_shared_expert

    if capacity_factor is not None:
        shape = shape.with_(capacity_factor=capacity_factor)
    if arrays is None:
        arrays = make_inputs(shape)

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    tensors = [dev(arrays[n]) for n in ("x", "Wg", "bg", "W1", "b1", "W2", "b2")]
    cfg = ops.make_config(shape.T, shape.d, shape.E, shape.k, shape.d_ffn, shape.capacity_factor,
                          shape.temperature, shape.gumbel, shape.seed, shape.dtype)
    m = Measured()
    m.shape, m.arrays, m.cfg, m.variant_host, m.route_stats = shape, arrays, cfg, None, None
    va = variant_args
    with_variant = va is not None and (va.activation != "gelu" or va.noise_std > 0.0 or va.shared_d_ffn > 0
                                       or va.drop_policy != "token" or va.route_stats)
    shared = None
    if with_variant:
        m.variant_host = {"activation": va.activation, "noise_std": va.noise_std, "shared": None,
                          "drop_policy": va.drop_policy}
        if va.route_stats:
            m.route_stats = torch.zeros((len(ops.ROUTE_STAT_NAMES),), dtype=torch.float32, device="cuda")
        if va.shared_d_ffn > 0:
            sh = make_shared_expert(shape, va.shared_d_ffn)
            shared = tuple(dev(sh[n]) for n in ("W1s", "b1s", "W2s", "b2s"))
            m.variant_host["shared"] = sh
    m.with_variant = with_variant
    if args.train:
        variant = (ops.make_variant(cfg, va.activation, va.noise_std, shared, va.drop_policy, m.route_stats)
                   if with_variant else None)
        m.train = (cfg, tensors, variant)
        return m
    m.packed = ((weights or args.weights) == "packed" and shape.dtype == "bf16" and shape.d % 256 == 0
                and shape.d_ffn % 256 == 0)
    m.pack_ms = None
    if m.packed:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        W1p, W2p = ops.pack_expert_weights(tensors[3]), ops.pack_expert_weights(tensors[5])
        b.record()
        b.synchronize()
        m.pack_ms = a.elapsed_time(b)
        tensors = tensors[:3] + [W1p, tensors[4], W2p, tensors[6]]
    variant = None
    if with_variant or m.packed:
        va_act = va.activation if with_variant else "gelu"
        va_noise = va.noise_std if with_variant else 0.0
        va_pol = va.drop_policy if with_variant else "token"
        variant = ops.make_variant(cfg, va_act, va_noise, shared, va_pol, m.route_stats, packed_weights=m.packed)
    plan = ops.ForwardPlan(cfg, *tensors, keep_routing=False, variant=variant)
    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize()
    # cold: each step follows a 1 GiB write (L2 and the MALL hold none of its inputs), then a
    # 512 MiB read, so that the write's dirty lines are written back before the step starts
    # rather than during its first kernel
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda")
    # K cold steps with moe_forward's per-stage events (the stage breakdown and the GEMM
    # durations), then K cold steps timed by two events around the call alone: the step time.
    # Each stage event adds a few microseconds to the step it splits.
    events = [ops.StageEvents() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush.fill_(i & 255)
        scrub.sum()
        plan.run(events=events[i])
    torch.cuda.synchronize()
    cold_stage = [ev.accumulate() for ev in events]
    for ev in events:
        ev.close()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush.fill_(i & 255)
        scrub.sum()
        pairs[i][0].record()
        plan.run()
        pairs[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del flush, scrub
    # warm: back to back, host clock (no events), then with the stage events for the breakdown
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        plan.run()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    wev = [ops.StageEvents() for _ in range(args.steps)]
    for i in range(args.steps):
        plan.run(events=wev[i])
    torch.cuda.synchronize()
    warm_stage = [ev.accumulate() for ev in wev]
    for ev in wev:
        ev.close()
    names = ops.STAGE_NAMES
    m.cold_step_ms = [a.elapsed_time(b) for a, b in pairs]
    m.cold_ms = _median(m.cold_step_ms)
    m.cold_staged_ms = _median([sum(s) for s in cold_stage])
    m.cold_stage_median = {n: _median([s[i] for s in cold_stage]) for i, n in enumerate(names)}
    m.cold_stage_mean = {n: sum(s[i] for s in cold_stage) / len(cold_stage) for i, n in enumerate(names)}
    m.cold_host_ms = (t1 - t0) * 1e3 / args.steps
    m.warm_ms = (t3 - t2) * 1e3 / args.steps
    m.warm_stage_mean = {n: sum(s[i] for s in warm_stage) / len(warm_stage) for i, n in enumerate(names)}
    m.kept = int(plan.out["kept"].sum().item())
    m.counts = plan.out["counts"].cpu().numpy()
    m.kept_e = plan.out["kept"].cpu().numpy()
    m.C = ops.capacity(cfg)
    m.forwards = args.warmup + 4 * args.steps
    if m.route_stats is not None:
        m.route_stats_values = dict(zip(ops.ROUTE_STAT_NAMES, m.route_stats.cpu().tolist()))
    del plan
    return m


def path_of(m: Measured) -> str:
    """Which expert kernels the forward runs: 'gemm' (bf16 MFMA), 'gemv' (decode-sized) or 'f32'."""
    if m.shape.dtype != "bf16":
        return "f32"
    return "gemm" if min(m.C, m.shape.T) > 16 else "gemv"


def rooflines(m: Measured, shared_d_ffn: int = 0) -> dict:
    """Roofline of the workload's dominant expert kernel, by the bound its shape sets, plus the
    HBM rates of the memory-bound stages. Times: mean of the cold steps."""
    sh = m.shape
    T, d, E, k, dff = sh.T, sh.d, sh.E, sh.k, sh.d_ffn
    st = m.cold_stage_mean
    sx = 2 if sh.dtype == "bf16" else 4
    kept = m.kept
    active = int((m.kept_e > 0).sum())
    g1, g2 = st["expert_gemm1_gelu"], st["expert_gemm2"]
    flops = 2.0 * d * dff * kept                       # per expert product, kept rows only
    shared_flops = 4.0 * d * shared_d_ffn * T
    path = path_of(m)
    w_bytes = active * d * dff * sx                    # one expert matrix (W1 or W2) of every active expert
    out = {"path": path}
    if path == "gemv":
        # decode: both launches stream the active experts' W1 and W2 once
        achieved = 2 * w_bytes / ((g1 + g2) * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": "expert_gemv (W1 and W2 launches)", "achieved": achieved,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                           "bytes_per_step": 2 * w_bytes, "active_experts": active}
    elif path == "gemm":
        stage_flops = {"expert_gemm1_gelu": flops, "expert_gemm2": flops + shared_flops}
        dom = "expert_gemm1_gelu" if g1 >= g2 else "expert_gemm2"
        t = st[dom] * 1e-3
        # HBM bytes the product must move at least: the active experts' weight matrix, the rows
        # it reads and writes (gathered x and bf16 H for GEMM1; bf16 H and float y_perm for GEMM2)
        io = kept * (d * sx + dff * sx) if dom == "expert_gemm1_gelu" else kept * (dff * sx + d * 4)
        bytes_min = w_bytes + io
        t_mfma = stage_flops[dom] / (PEAK_BF16_TFLOPS * 1e12)
        t_hbm = bytes_min / (PEAK_HBM_GBS * 1e9)
        tflops = stage_flops[dom] / t / 1e12
        if t_hbm > t_mfma:
            achieved = bytes_min / t / 1e9
            out["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": t_hbm / t, "algorithmic_bytes": bytes_min,
                               "tflops": tflops, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
                               "rule": "max(F/peak, B/BW): B/BW is larger"}
        else:
            out["roofline"] = {"bound": "mfma", "kernel": dom, "achieved": tflops, "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                               "algorithmic_flops": stage_flops[dom]}
        tot = 2 * flops + shared_flops
        out["grouped_gemm"] = {"tflops": tot / ((g1 + g2) * 1e-3) / 1e12,
                               "frac_of_peak": tot / ((g1 + g2) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "gemm1_ms": g1, "gemm2_ms": g2,
                               "gemm1_frac": flops / (g1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "gemm2_frac": (flops + shared_flops) / (g2 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                               "kept_rows": kept, "dropped_slots": int(k * T - kept)}
    else:
        out["roofline"] = None                          # launch-latency-bound correctness path
    ng = (T + 15) // 16
    router_bytes = T * d * sx + E * d * sx + T * E * 4 + T * k * 8 + ng * E * 8
    gather_fused = path == "gemv" or (path == "gemm" and T * d * 2 < 2 ** 31)
    dispatch_bytes = T * k * 4 + T * k * 4 + kept * 4 + (0 if gather_fused else 2 * kept * d * sx)
    combine_bytes = kept * d * 4 + T * k * 8 + T * d * sx
    disp_ms = st["scan"] + st["permute_gather"]
    out["hbm_stages"] = {
        "router": {"GB/s": router_bytes / (st["route"] * 1e-3) / 1e9, "bytes": router_bytes, "ms": st["route"]},
        "dispatch": {"GB/s": dispatch_bytes / (disp_ms * 1e-3) / 1e9, "bytes": dispatch_bytes, "ms": disp_ms,
                     "gather_fused_into_gemm1": gather_fused},
        "combine": {"GB/s": combine_bytes / (st["combine"] * 1e-3) / 1e9, "bytes": combine_bytes,
                    "ms": st["combine"]},
        "peak_GB/s": PEAK_HBM_GBS,
    }
    return out


def workload_entry(m: Measured, shared_d_ffn: int = 0) -> dict:
    sh = m.shape
    e = {"config": {"T": sh.T, "d": sh.d, "E": sh.E, "k": sh.k, "d_ffn": sh.d_ffn,
                    "capacity_factor": sh.capacity_factor, "temperature": sh.temperature, "gumbel": sh.gumbel,
                    "dtype": sh.dtype, "weights": "packed" if m.packed else "row-major", "capacity": m.C},
         "tokens_per_s": sh.T / (m.cold_ms * 1e-3), "ms_per_step": m.cold_ms,
         "ms_per_step_with_stage_events": m.cold_staged_ms,
         "warm": {"tokens_per_s": sh.T / (m.warm_ms * 1e-3), "ms_per_step": m.warm_ms},
         "stage_ms": m.cold_stage_median,
         "counts_minmax": [int(m.counts.min()), int(m.counts.max())]}
    e.update(rooflines(m, shared_d_ffn))
    return e


# ----------------------------------------------------------------------------------- main
def main() -> int:
    args = _args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.bench_log))
        return 0
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters.split(","), args.workload, args.weights), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported: the library has no "
              "collectives or sharding (expert-parallel sharding of the layer is described, not implemented).",
              file=sys.stderr)
        return 2

    import torch

    from sparse_mixture_experts_41_amd import ops
    from workloads import CONFIGS

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            ops.probe_copy(src, dst)
        torch.cuda.synchronize()
        for _ in range(3):   # the runtime's own device copy: ordinary (cached) loads, like the GEMMs'
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 3, "kernels": ["probe_copy_kernel", "runtime copy"]}),
              flush=True)
        return 0

    head = measure_workload(CONFIGS[args.workload], args, ops, torch, variant_args=args,
                            capacity_factor=args.capacity_factor)
    shape = head.shape
    if args.train:
        cfg, tensors, variant = head.train
        return train_step(args, shape, cfg, tensors, variant, ops, torch)
    launches = [{"workload": shape.name, "forwards": head.forwards, "warmup": args.warmup, "cold": args.steps,
                 "warm": args.steps}]
    entry = workload_entry(head, args.shared_d_ffn)
    # the headline workload again with the expert weights in nn.Linear's layout, as the caller
    # hands them over (the headline packs them once before its warm-up)
    row_major = None
    if head.packed and not args.no_row_major:
        rm = measure_workload(head.shape, args, ops, torch, variant_args=args, arrays=head.arrays,
                              weights="row-major")
        launches.append({"workload": f"{shape.name} (row-major weights)", "forwards": rm.forwards,
                         "warmup": args.warmup, "cold": args.steps, "warm": args.steps})
        rm_entry = workload_entry(rm, args.shared_d_ffn)
        row_major = {"tokens_per_s": shape.T / (rm.cold_ms * 1e-3), "ms_per_step": rm.cold_ms,
                     "warm_ms_per_step": rm.warm_ms, "stage_ms": rm.cold_stage_median,
                     "grouped_gemm": rm_entry.get("grouped_gemm")}
        del rm
        torch.cuda.empty_cache()
    traffic = None
    if entry.get("roofline") and not head.with_variant and args.capacity_factor is None:
        traffic_path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{shape.name}.json")
        traffic = stored_traffic(traffic_path, entry["roofline"]["kernel"], "packed" if head.packed else "row-major")
    roof = dict(entry["roofline"]) if entry.get("roofline") else None
    if roof is not None:
        roof["traffic"] = traffic
        roof["timing"] = "mean kernel duration over the cold steps (HIP events on the layer's stream)"
    others = {}
    for name in [w for w in args.others.split(",") if w and w != shape.name]:
        m = measure_workload(CONFIGS[name], args, ops, torch)
        launches.append({"workload": name, "forwards": m.forwards, "warmup": args.warmup, "cold": args.steps,
                         "warm": args.steps})
        others[name] = workload_entry(m)
        del m
        torch.cuda.empty_cache()
    peaks = None if args.no_peaks else measure_peaks(ops, torch)
    if peaks and roof is not None:
        roof["frac_of_measured_peak"] = roof["achieved"] / (
            peaks["mfma_bf16_TFLOP/s"] if roof["unit"] == "TFLOP/s" else peaks["copy_GB/s"])
    T = shape.T
    line = {
        "metric": "MoE-layer tokens/sec (bf16, 1 GPU) + grouped-GEMM % of bf16 MFMA peak",
        "value": T / (head.cold_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.cold_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; workloads.make_inputs)",
        "config": {"workload": shape.name, "T": T, "d": shape.d, "E": shape.E, "k": shape.k, "d_ffn": shape.d_ffn,
                   "capacity_factor": shape.capacity_factor, "temperature": shape.temperature,
                   "gumbel": shape.gumbel, "parallelism": "none (one GPU)",
                   "weights": "packed" if head.packed else "row-major",
                   **({"variant": {"activation": args.activation, "noise_std": args.noise_std,
                                   "shared_d_ffn": args.shared_d_ffn, "drop_policy": args.drop_policy,
                                   "route_stats": args.route_stats}} if head.with_variant else {})},
        "timing": {"headline": "median of K cold-cache steps, each timed by two HIP events around moe_forward",
                   "cold_step_ms": head.cold_step_ms, "host_ms_per_cold_iteration_incl_flush": head.cold_host_ms,
                   "ms_per_step_with_stage_events": head.cold_staged_ms,
                   "flush_bytes": FLUSH_BYTES, "scrub_read_bytes": SCRUB_BYTES},
        "warm": {"tokens_per_s": T / (head.warm_ms * 1e-3), "ms_per_step": head.warm_ms,
                 "stage_ms": head.warm_stage_mean},
        "roofline": roof,
        "grouped_gemm": entry.get("grouped_gemm"),
        "hbm_stages": entry["hbm_stages"],
        "stage_ms": head.cold_stage_median,
        "stage_ms_mean": head.cold_stage_mean,
        "pack_ms": head.pack_ms,
        "row_major": row_major,
        "counts_minmax": entry["counts_minmax"],
        "measured_peaks": peaks,
        "workloads": others,
        "launches": launches,
    }
    if getattr(head, "route_stats_values", None):
        line["route_stats"] = head.route_stats_values
    n_cpu = args.cpu_sample_tokens
    if n_cpu is None:
        n_cpu = CPU_SAMPLE.get(shape.name, min(T, 4096))
    if n_cpu != 0:
        n_cpu = T if n_cpu < 0 else min(n_cpu, T)
        line["cpu_baseline"] = cpu_baseline(shape, head.arrays, n_cpu, head.variant_host)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


# ------------------------------------------------------------------------ trace summary
def summarize_trace(trace_dir: str, bench_log: str | None) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace run of this script: every kernel's calls
    and mean duration, then per workload the expert kernels' mean over the timed cold steps
    (dispatches matched in order to the forwards the JSON line's `launches` lists) against the
    bench line's own figures."""
    traces = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not traces:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    rows = []
    for path in traces:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    line = None
    if bench_log:
        with open(bench_log) as f:
            for ln in f:
                if ln.startswith("{") and '"metric"' in ln:
                    line = json.loads(ln)
    def clean(name):
        return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("moe::", "")

    stats = {}
    for s, e, name in rows:
        short = clean(name)
        st = stats.setdefault(short, [0, 0.0])
        st[0] += 1
        st[1] += (e - s) / 1e3
    out = [f"Kernel trace: {len(rows)} dispatches from {len(traces)} file(s).", "",
           "| kernel | calls | mean µs | total ms |", "|---|---:|---:|---:|"]
    for name, (n, tot) in sorted(stats.items(), key=lambda kv: -kv[1][1]):
        out.append(f"| `{name}` | {n} | {tot / n:.2f} | {tot / 1e3:.3f} |")
    if line is None:
        return "\n".join(out)

    def kind(name):
        # template argument 0 / 2: the activation epilogue (GEMM1), 1: the linear one (GEMM2)
        for base in ("grouped_gemm_bf16_kernel<", "grouped_gemv_bf16_kernel<", "grouped_gemm_f32_kernel<"):
            if name.startswith(base):
                epi = name[len(base):].split(",")[0].split(">")[0].strip()
                return {"0": "gemm1", "2": "gemm1", "1": "gemm2"}.get(epi)
        return None

    seq = {"gemm1": [], "gemm2": []}
    for s, e, name in rows:
        kd = kind(clean(name))
        if kd:
            seq[kd].append((e - s) / 1e3)
    out += ["", "Expert kernels per workload over the timed cold steps (dispatches matched in launch order; "
            "one GEMM1 and one GEMM2 launch per forward):", "",
            "| workload | kernel | cold launches | trace mean µs | bench events mean µs | trace / events | "
            "algorithmic work | trace frac of peak |", "|---|---|---:|---:|---:|---:|---|---:|"]
    pos = 0
    for l in line["launches"]:
        w = l["workload"]
        entry = line if w == line["config"]["workload"] else line["workloads"].get(w, {})
        if w.endswith("(row-major weights)") and line.get("row_major"):
            rmj = line["row_major"]
            entry = {"stage_ms": rmj["stage_ms"], "grouped_gemm": rmj["grouped_gemm"], "roofline": line["roofline"],
                     "config": line["config"]}
        stage = (line.get("stage_ms_mean") if w == line["config"]["workload"] else None) or entry.get("stage_ms", {})
        roof = entry.get("roofline")
        gg = entry.get("grouped_gemm") or {}
        lo, hi = pos + l["warmup"], pos + l["warmup"] + l["cold"]
        pos += l["forwards"]
        for kd, stage_name in (("gemm1", "expert_gemm1_gelu"), ("gemm2", "expert_gemm2")):
            d = seq[kd][lo:hi]
            if not d:
                continue
            mean = sum(d) / len(d)
            ev = stage.get(stage_name)
            work, frac = "", ""
            if gg and roof:
                cfg = line["config"] if w == line["config"]["workload"] else entry["config"]
                flops = 2.0 * cfg["d"] * cfg["d_ffn"] * gg["kept_rows"]
                work = f"{flops / 1e12:.4f} TFLOP"
                frac = f"{flops / (mean * 1e-6) / 1e12 / PEAK_BF16_TFLOPS:.3f}"
            elif roof and roof.get("unit") == "GB/s" and "bytes_per_step" in roof:
                work = f"{roof['bytes_per_step'] / 2e9:.3f} GB (one launch's weights)"
                frac = f"{roof['bytes_per_step'] / 2 / (mean * 1e-6) / 1e9 / PEAK_HBM_GBS:.3f} of HBM"
            ratio = f"{mean / (ev * 1e3):.3f}" if ev else ""
            out.append(f"| {w} | {stage_name} | {len(d)} | {mean:.1f} | {ev * 1e3 if ev else float('nan'):.1f} | "
                       f"{ratio} | {work} | {frac} |")
    hr = line.get("roofline") or {}
    out += ["", f"Bench line of the traced run: value {line['value']:.0f} tokens/s, {line['ms_per_step']:.4f} ms per "
            f"cold step; roofline {hr.get('kernel')} {hr.get('achieved', 0):.1f} {hr.get('unit')} = frac "
            f"{hr.get('frac', 0):.4f}."]
    return "\n".join(out)


def _counter_means(d: str, counter: str) -> dict:
    """Mean per dispatch of `counter` (summed over its instances) for every kernel in a
    rocprofv3 --pmc output directory: {clean kernel name: (mean KiB, dispatches)}."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for path in files:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = (path, r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, _, name), v in per.items():
        n = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("moe::", "")
        tot, cnt = out.get(n, (0.0, 0))
        out[n] = (tot + v, cnt + 1)
    return {n: (tot / cnt, cnt) for n, (tot, cnt) in out.items()}


def summarize_counters(dirs, workload: str, weights: str) -> dict:
    """Traffic JSON: calibrated HBM bytes per launch of the headline's expert GEMMs. Each counter
    (FETCH_SIZE, WRITE_SIZE, in KiB per dispatch) is scaled by the bytes a 1 GiB copy moves over
    what the same counter reads for it. Two copies are counted: the runtime's device copy
    (ordinary loads and stores, as the GEMMs issue; its factors scale the GEMMs' counters) and
    the non-temporal probe copy (recorded beside it)."""
    fetch, write, cfetch, cwrite = (_counter_means(d, c) for d, c in zip(
        dirs, ("FETCH_SIZE", "WRITE_SIZE", "FETCH_SIZE", "WRITE_SIZE")))
    copy_bytes = 1 << 30

    def runtime_copy(counts):
        # the runtime's copy kernel: 3 dispatches of the 1 GiB copy (the fills run other kernels)
        cands = [(v, n) for n, v in counts.items() if "copy" in n.lower() and n != "probe_copy_kernel" and v[1] >= 3]
        return max(cands)[0][0] if cands else None

    probe = {"fetch_factor": copy_bytes / (cfetch["probe_copy_kernel"][0] * 1024),
             "write_factor": copy_bytes / (cwrite["probe_copy_kernel"][0] * 1024)}
    rf, rw = runtime_copy(cfetch), runtime_copy(cwrite)
    plain = ({"fetch_factor": copy_bytes / (rf * 1024), "write_factor": copy_bytes / (rw * 1024)}
             if rf and rw else None)
    use = plain or probe
    cal_f, cal_w = use["fetch_factor"], use["write_factor"]
    names = {"expert_gemm1_gelu": "grouped_gemm_bf16_kernel<0,", "expert_gemm2": "grouped_gemm_bf16_kernel<1,"}
    res = {"workload": workload, "weights": weights, "gemm_source_sha256": gemm_source_digest(),
           "bytes_per_launch": {}, "counters_kib_per_launch": {},
           "calibration": {"copy_bytes": copy_bytes, "fetch_factor": cal_f, "write_factor": cal_w,
                           "kernel": "runtime copy" if plain else "probe_copy_kernel",
                           "runtime_copy": plain, "probe_copy_kernel": probe}}
    for stage, prefix in names.items():
        fk = [v for n, v in fetch.items() if n.startswith(prefix)]
        wk = [v for n, v in write.items() if n.startswith(prefix)]
        if fk and wk:
            f_kib, nf = fk[0]
            w_kib, nw = wk[0]
            res["bytes_per_launch"][stage] = f_kib * 1024 * cal_f + w_kib * 1024 * cal_w
            res["counters_kib_per_launch"][stage] = {"FETCH_SIZE": f_kib, "WRITE_SIZE": w_kib, "dispatches": [nf, nw]}
    return res


if __name__ == "__main__":
    sys.exit(main())
