"""GPU parity of the capacity policies and the routing statistics (moe_forward_ex) against the
CPU oracle (MI355X).

Random dropping and rerouting to the next-ranked experts: counts, kept, offsets, dest and perm
bit-exact against oracle.dispatch_policy on the GPU's own scores; weights (renormalised over
the final experts when rerouting) and outputs to the tolerances of tests/parity.py. Cases span
the MFMA GEMM, GEMV and float32 expert paths, all four router kernels (one-kernel 16-token,
K-sliced, 64-token wide, float32), ragged token counts, heavy skew (one expert far over
capacity), k = E (no next expert), k = 8 of 64 experts, noise and temperature (scores differ
from logits), token counts that take the scan's two-level path, and the full-size layers on
sampled rows.
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_41_amd import ops
from workloads import CONFIGS, MoEShape

from .parity import Problem, check_forward_full, check_forward_sampled, run_forward

pytestmark = pytest.mark.gpu

S = MoEShape
CASES = {
    # name: (shape, bias_std, policy, stats, noise_std)
    "random_gemm": (S("random_gemm", T=1000, d=256, E=8, k=2, d_ffn=384, capacity_factor=0.7), 0.1, "random",
                    True, 0.0),
    "random_f32": (S("random_f32", T=300, d=96, E=6, k=2, d_ffn=200, capacity_factor=0.6, dtype="f32", seed=7), 0.1,
                   "random", True, 0.0),
    "random_small_gemv": (S("random_small_gemv", T=50, d=128, E=16, k=2, d_ffn=128, capacity_factor=0.5,
                            wg_std=None), 0.05, "random", False, 0.0),
    "random_skew_ragged": (S("random_skew_ragged", T=777, d=192, E=64, k=1, d_ffn=128, capacity_factor=1.0,
                             recipe="zipf_bias", wg_std=None, seed=3), 0.0, "random", True, 0.0),
    "reroute_gemm": (S("reroute_gemm", T=1000, d=256, E=8, k=2, d_ffn=384, capacity_factor=0.8), 0.1, "reroute",
                     True, 0.0),
    "reroute_top1_skew": (S("reroute_top1_skew", T=777, d=192, E=64, k=1, d_ffn=128, capacity_factor=1.0,
                            recipe="zipf_bias", wg_std=None, seed=5), 0.0, "reroute", False, 0.0),
    "reroute_k_eq_E": (S("reroute_k_eq_E", T=200, d=64, E=4, k=4, d_ffn=64, capacity_factor=0.5, dtype="f32"), 0.1,
                       "reroute", True, 0.0),
    "reroute_k8_E64": (S("reroute_k8_E64", T=500, d=128, E=64, k=8, d_ffn=64, capacity_factor=0.5, wg_std=None),
                       0.05, "reroute", True, 0.0),
    "reroute_noise_tau": (S("reroute_noise_tau", T=700, d=128, E=6, k=2, d_ffn=192, capacity_factor=0.7,
                            temperature=0.9, seed=21), 0.0, "reroute", True, 0.3),
    "reroute_gumbel_f32": (S("reroute_gumbel_f32", T=300, d=64, E=5, k=2, d_ffn=96, capacity_factor=0.8,
                             dtype="f32", gumbel=True, temperature=0.7, seed=9), 0.1, "reroute", False, 0.0),
    "stats_sliced_router": (S("stats_sliced_router", T=300, d=1024, E=24, k=3, d_ffn=128, capacity_factor=1.0,
                              seed=5, wg_std=None), 0.0, "token", True, 0.0),
    "stats_f32": (S("stats_f32", T=256, d=128, E=4, k=2, d_ffn=512, capacity_factor=1.25, dtype="f32"), 0.0,
                  "token", True, 0.0),
    # enough 16-token groups for the two-level scan (more than 256 groups of 64 experts, 1024 of
    # 16), with a ragged last chunk
    "random_two_level": (S("random_two_level", T=5000, d=64, E=64, k=2, d_ffn=64, capacity_factor=0.8,
                           wg_std=None, seed=11), 0.05, "random", True, 0.0),
    "reroute_two_level": (S("reroute_two_level", T=5000, d=64, E=64, k=2, d_ffn=64, capacity_factor=0.7,
                            wg_std=None, seed=12), 0.0, "reroute", True, 0.0),
    "stats_two_level_e16": (S("stats_two_level_e16", T=17000, d=64, E=16, k=2, d_ffn=64, capacity_factor=1.0,
                              seed=13), 0.0, "token", True, 0.0),
    # 257 groups of 64 experts: the first count that takes two levels, its last chunk one group
    "random_two_level_edge": (S("random_two_level_edge", T=4112, d=64, E=64, k=2, d_ffn=64, capacity_factor=0.9,
                                wg_std=None, seed=14), 0.0, "random", True, 0.0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_policy(name):
    shape, bias, policy, stats, noise = CASES[name]
    print(f"[gpu] policy {name} {shape} policy={policy} stats={stats} noise={noise}", flush=True)
    p = Problem(shape, bias_std=bias, noise_std=noise, drop_policy=policy, route_stats=stats)
    res = check_forward_full(p)
    print(f"[gpu]   {name}: {res}", flush=True)
    if policy != "token":
        assert res["drops"] > 0 or policy == "reroute", "the case should overflow some expert"


def test_random_with_room_is_token_order():
    shape = S("room", T=900, d=128, E=6, k=2, d_ffn=256, capacity_factor=6.0, seed=2)
    print(f"[gpu] random with room {shape}", flush=True)
    a = run_forward(Problem(shape, bias_std=0.05))
    b = run_forward(Problem(shape, bias_std=0.05, drop_policy="random"))
    assert torch.equal(a["y_raw"], b["y_raw"])
    for key in ("counts", "kept", "offsets", "dest", "perm", "topk_w"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)


def test_reroute_keeps_more_than_token_order():
    shape = S("more", T=1000, d=128, E=8, k=2, d_ffn=128, capacity_factor=0.9, seed=4, wg_std=None)
    a = run_forward(Problem(shape))
    b = run_forward(Problem(shape, drop_policy="reroute"))
    assert b["kept"].sum() > a["kept"].sum()
    np.testing.assert_array_equal(a["counts"], b["counts"])
    assert np.all(b["kept"] <= ops.capacity(Problem(shape).cfg))


FULL = {
    "mixtral_like_random": (CONFIGS["mixtral_like"].with_(capacity_factor=0.9), "random"),
    "mixtral_like_reroute": (CONFIGS["mixtral_like"].with_(capacity_factor=0.9), "reroute"),
    "switch_skew_random": (CONFIGS["switch_skew"], "random"),
    "switch_skew_reroute": (CONFIGS["switch_skew"], "reroute"),
}


@pytest.mark.parametrize("name", sorted(FULL))
def test_policy_full_size(name):
    shape, policy = FULL[name]
    print(f"[gpu] full-size policy {name} {shape}", flush=True)
    p = Problem(shape, drop_policy=policy, route_stats=True)
    res = check_forward_sampled(p)
    print(f"[gpu]   {name}: {res}", flush=True)
