#!/usr/bin/env python3
"""Throughput of the sparse MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral_like]

One step is one moe_forward call (router + softmax + top-k, capacity dispatch, grouped expert
GEMMs with GeLU, combine and the balance statistic) over one batch of seeded synthetic input
already resident in HBM. W untimed warm-up steps, then exactly K timed steps between two
device synchronisations. Prints one JSON line:
  value         tokens/s of the whole layer (T tokens per step);
  stage_ms      per-stage means from HIP events recorded inside moe_forward on its stream;
  roofline      the dominant expert GEMM kernel: algorithmic FLOPs (2 d d_ffn per kept row)
                over its measured duration, against the bf16 dense MFMA peak (2.5 PFLOP/s);
  cpu_baseline  the CPU oracle (numpy float64) on a bounded sample of the same workload;
  cold_cache    the median event-measured forward when each call follows a 1 GiB write that
                evicts L2 and the MALL (value and stage_ms are warm, back-to-back steps);
  weights       where the shape allows it (bf16, d and d_ffn multiples of 256) the timed
                forward takes W1 and W2 in the panel layout of moe_pack_expert_weights, packed
                once before the warm-up as a server does when it loads the weights (pack_ms).
                With --weights both (the default) row_major holds the same timing with
                nn.Linear's layout, run first; both layouts give bit-identical outputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_like")
    ap.add_argument("--cpu-sample-tokens", type=int, default=-1,
                    help="tokens in the batch the CPU oracle is timed on (-1 = the whole batch, 0 = skip)")
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
                    help="override the workload's capacity factor (reported in config)")
    ap.add_argument("--train", action="store_true",
                    help="time the training step instead: moe_forward_train + moe_backward (one JSON line)")
    ap.add_argument("--lam", type=float, default=0.01, help="weight of the balance loss in the training step")
    ap.add_argument("--weights", choices=("both", "packed", "row-major"), default="both",
                    help="expert weight layout of the timed forward (packed where the shape allows it); "
                         "both: also time the row-major layout first")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="after the timed steps, this many forwards each preceded by a 1 GiB write that "
                         "evicts L2 and the 256 MB MALL, timed with HIP events (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit: the "
                         "known-size reference for the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# Sources whose change invalidates a stored traffic measurement of the expert GEMMs.
GEMM_SOURCES = ("sparse_mixture_experts_41_amd/csrc/expert_gemm.hip", "sparse_mixture_experts_41_amd/csrc/moe_common.h")


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


def cpu_baseline(shape, arrays, n_tokens: int, variant: dict | None = None) -> dict:
    """The oracle as it stands, timed on the host cores on the first n_tokens tokens.
    ``variant``: activation, noise_std and shared-expert arrays of a forward variant."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from workloads import bf16_bits_to_f32

    cores = len(os.sched_getaffinity(0))
    dt = shape.dtype

    def val(a):
        if a is None:
            return None
        return bf16_bits_to_f32(a) if (dt == "bf16" and a.dtype == np.uint16) else np.asarray(a, np.float32)

    x = val(arrays["x"])[:n_tokens]
    args = (x, val(arrays["Wg"]), arrays["bg"], val(arrays["W1"]), val(arrays["b1"]), val(arrays["W2"]),
            val(arrays["b2"]))
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        vkw = {}
        if variant:
            shared = variant.get("shared")
            vkw = dict(act=variant["activation"], noise_std=variant["noise_std"], policy=variant["drop_policy"],
                       shared=None if shared is None else tuple(val(shared[n]) for n in ("W1s", "b1s", "W2s", "b2s")))
        out = oracle.forward(*args, k=shape.k, capacity_factor=shape.capacity_factor, tau=shape.temperature,
                             gumbel=shape.gumbel, seed=shape.seed, **vkw)
        t1 = time.perf_counter()
        blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()]
    assert np.isfinite(out["y"]).all()
    return {"value": n_tokens / (t1 - t0), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"the whole {shape.name} batch ({n_tokens} tokens)" if n_tokens == shape.T else
                       f"first {n_tokens} tokens of the {shape.name} input as one batch (C recomputed)")
                      + f", numpy float64, {', '.join(blas)}",
            "seconds": t1 - t0}


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
        "training_flops_frac": 6.0 * d * dff * kept / ((fwd_ms + bwd_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stage_ms": fst,
        "backward_stage_ms": bst,
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    args = _args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported by this build "
              "(no collectives or sharding are implemented).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sparse_mixture_experts_41_amd import ops
    from workloads import CONFIGS, make_inputs, make_shared_expert

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 3}), flush=True)
        return 0
    shape = CONFIGS[args.workload]
    if args.capacity_factor is not None:
        shape = shape.with_(capacity_factor=args.capacity_factor)
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
    with_variant = (args.activation != "gelu" or args.noise_std > 0.0 or args.shared_d_ffn > 0
                    or args.drop_policy != "token" or args.route_stats)
    variant = None
    variant_host = None
    route_stats = None
    if with_variant:
        shared = None
        variant_host = {"activation": args.activation, "noise_std": args.noise_std, "shared": None,
                        "drop_policy": args.drop_policy}
        if args.route_stats:
            route_stats = torch.zeros((len(ops.ROUTE_STAT_NAMES),), dtype=torch.float32, device="cuda")
        if args.shared_d_ffn > 0:
            sh = make_shared_expert(shape, args.shared_d_ffn)
            shared = tuple(dev(sh[n]) for n in ("W1s", "b1s", "W2s", "b2s"))
            variant_host["shared"] = sh
        variant = ops.make_variant(cfg, args.activation, args.noise_std, shared, args.drop_policy, route_stats)
    if args.train:
        return train_step(args, shape, cfg, tensors, variant, ops, torch)

    def timed(plan):
        """W warm-up steps, then K timed steps: (host ms per step, mean stage ms, the events)."""
        for _ in range(args.warmup):
            plan.run()
        torch.cuda.synchronize()
        events = [ops.StageEvents() for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            plan.run(events=events[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        stage = {n: 0.0 for n in ops.STAGE_NAMES}
        for ev in events:
            for n, v in zip(ops.STAGE_NAMES, ev.accumulate()):
                stage[n] += v / args.steps
            ev.close()
        return (t1 - t0) * 1e3 / args.steps, stage, events

    packed = (args.weights != "row-major" and shape.dtype == "bf16" and shape.d % 256 == 0
              and shape.d_ffn % 256 == 0)
    row_major = None
    pack_ms = None
    if packed:
        if args.weights == "both":
            rm_ms, rm_stage, _ = timed(ops.ForwardPlan(cfg, *tensors, keep_routing=False, variant=variant))
            row_major = {"ms_per_step": rm_ms, "tokens_per_s": shape.T / (rm_ms * 1e-3),
                         "expert_gemm1_gelu_ms": rm_stage["expert_gemm1_gelu"],
                         "expert_gemm2_ms": rm_stage["expert_gemm2"]}
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        W1p, W2p = ops.pack_expert_weights(tensors[3]), ops.pack_expert_weights(tensors[5])
        end.record()
        torch.cuda.synchronize()
        pack_ms = start.elapsed_time(end)
        tensors = tensors[:3] + [W1p, tensors[4], W2p, tensors[6]]
        shared = variant[1].get("shared") if variant is not None else None
        variant = ops.make_variant(cfg, args.activation, args.noise_std, shared, args.drop_policy, route_stats,
                                   packed_weights=True)
    plan = ops.ForwardPlan(cfg, *tensors, keep_routing=False, variant=variant)
    ms_per_step, stage, events = timed(plan)

    # warm: the median event-measured forward of the timed steps; cold: forwards that each follow
    # a 1 GiB write (L2 and MALL hold none of the inputs or weights when they start)
    warm_event_ms = float(np.median([sum(ev.totals) / max(ev.samples, 1) for ev in events]))
    cold = None
    if args.cold_reps > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold_ms = []
        for r in range(args.cold_reps):
            flush.fill_(r & 255)
            ev = ops.StageEvents()
            plan.run(events=ev)
            cold_ms.append(sum(ev.accumulate()))
            ev.close()
        del flush
        cold_med = float(np.median(cold_ms))
        cold = {"ms_per_step": cold_med, "tokens_per_s": shape.T / (cold_med * 1e-3), "reps": args.cold_reps,
                "flush_bytes": 1 << 30, "warm_event_ms_per_step": warm_event_ms}
    kept = int(plan.out["kept"].sum().item())
    counts = plan.out["counts"].cpu().numpy()
    T, d, E, k, dff = shape.T, shape.d, shape.E, shape.k, shape.d_ffn
    sx = 2 if shape.dtype == "bf16" else 4
    gemm_flops = 2.0 * d * dff * kept                       # per GEMM launch, kept rows only
    shared_flops = 4.0 * d * args.shared_d_ffn * T          # both shared-expert GEMMs, every token
    g1, g2 = stage["expert_gemm1_gelu"], stage["expert_gemm2"]
    # the shared expert's two GEMMs run inside the second stage
    stage_flops = {"expert_gemm1_gelu": gemm_flops, "expert_gemm2": gemm_flops + shared_flops}
    dom_name, dom_ms = ("expert_gemm1_gelu", g1) if g1 >= g2 else ("expert_gemm2", g2)
    achieved = stage_flops[dom_name] / (dom_ms * 1e-3) / 1e12
    traffic_path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{shape.name}.json")
    traffic = (None if (with_variant or args.capacity_factor is not None)
               else stored_traffic(traffic_path, dom_name, "packed" if packed else "row-major"))
    ng = (T + 15) // 16
    router_bytes = T * d * sx + E * d * sx + T * E * 4 + T * k * 8 + ng * E * 8
    # GEMM1 reads the token rows through the permutation (no gathered copy) on the bf16 MFMA
    # path while x is addressable by 32-bit offsets; otherwise dispatch also copies the rows
    C = ops.capacity(cfg)
    gather_fused = shape.dtype == "bf16" and min(C, T) > 16 and T * d * 2 < 2 ** 31
    dispatch_bytes = T * k * 4 + T * k * 4 + kept * 4 + (0 if gather_fused else 2 * kept * d * sx)
    combine_bytes = kept * d * 4 + T * k * 8 + T * d * sx
    disp_ms = stage["scan"] + stage["permute_gather"]
    line = {
        "metric": "MoE-layer tokens/sec (bf16, 1 GPU) + grouped-GEMM % of bf16 MFMA peak",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded; workloads.make_inputs)",
        "config": {"workload": shape.name, "T": T, "d": d, "E": E, "k": k, "d_ffn": dff,
                   "capacity_factor": shape.capacity_factor, "temperature": shape.temperature,
                   "gumbel": shape.gumbel, "parallelism": "none (one GPU)",
                   "weights": "packed" if packed else "row-major",
                   **({"variant": {"activation": args.activation, "noise_std": args.noise_std,
                                   "shared_d_ffn": args.shared_d_ffn, "drop_policy": args.drop_policy,
                                   "route_stats": args.route_stats}} if with_variant else {})},
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic},
        "grouped_gemm": {"tflops": (2 * gemm_flops + shared_flops) / ((g1 + g2) * 1e-3) / 1e12,
                         "frac_of_peak": (2 * gemm_flops + shared_flops) / ((g1 + g2) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "kept_rows": kept, "dropped_slots": int(k * T - kept)},
        "hbm_stages": {
            "router": {"GB/s": router_bytes / (stage["route"] * 1e-3) / 1e9, "bytes": router_bytes},
            "dispatch": {"GB/s": dispatch_bytes / (disp_ms * 1e-3) / 1e9, "bytes": dispatch_bytes,
                         "gather_fused_into_gemm1": gather_fused},
            "combine": {"GB/s": combine_bytes / (stage["combine"] * 1e-3) / 1e9, "bytes": combine_bytes},
            "peak_GB/s": PEAK_HBM_GBS,
        },
        "stage_ms": stage,
        "cold_cache": cold,
        "row_major": row_major,
        "pack_ms": pack_ms,
        "counts_minmax": [int(counts.min()), int(counts.max())],
    }
    if route_stats is not None:
        line["route_stats"] = dict(zip(ops.ROUTE_STAT_NAMES, route_stats.cpu().tolist()))
    if args.cpu_sample_tokens != 0:
        n_cpu = T if args.cpu_sample_tokens < 0 else min(args.cpu_sample_tokens, T)
        line["cpu_baseline"] = cpu_baseline(shape, arrays, n_cpu, variant_host)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
