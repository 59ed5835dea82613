"""GPU parity of every stage and of the whole layer against the CPU oracle (MI355X).

Small shapes (the oracle runs on every token) span several tiles and ragged tails, drops,
k = 1, k = E, C = 1, the decode-sized path, float32, Gumbel noise and exact ties. The five
named workloads run at full size with routing checked on every token; outputs are compared on
every token, except on gumbel_longtail (65536 tokens), where one token of every (expert,
256-row tile) and 256 uniform tokens are compared. Tolerances are those of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_mixture_experts_41_amd import ops
from workloads import CONFIGS, MoEShape

from .parity import (Problem, check_forward_full, check_forward_sampled, check_logits, check_output, check_routing,
                     run_forward)

pytestmark = pytest.mark.gpu

SMALL = {
    # several 128-row tiles per expert, ragged tail, some drops, all biases set
    "ragged_bias": (MoEShape("ragged_bias", T=1000, d=256, E=8, k=2, d_ffn=384, capacity_factor=1.0), 0.1),
    # heavy drops, k = 3 of 5, Gumbel noise at tau = 0.7
    "gumbel_drops": (MoEShape("gumbel_drops", T=700, d=128, E=5, k=3, d_ffn=192, capacity_factor=0.6,
                              temperature=0.7, gumbel=True, seed=12345), 0.0),
    # 64 experts, top-1, C = 13 <= 16: the decode-sized (GEMV) expert path
    "gemv_path": (MoEShape("gemv_path", T=777, d=192, E=64, k=1, d_ffn=128, capacity_factor=1.0,
                           wg_std=None), 0.05),
    # k = E: every expert on every token, no drops
    "k_equals_E": (MoEShape("k_equals_E", T=200, d=64, E=3, k=3, d_ffn=64, capacity_factor=2.0), 0.0),
    # C = 1: each expert keeps only its first token
    "capacity_one": (MoEShape("capacity_one", T=130, d=64, E=16, k=2, d_ffn=128, capacity_factor=0.05), 0.0),
    # a single token and a single expert
    "single_token": (MoEShape("single_token", T=1, d=64, E=1, k=1, d_ffn=64, capacity_factor=1.0), 0.0),
    # float32 with Gumbel noise and a temperature
    "f32_gumbel": (MoEShape("f32_gumbel", T=300, d=96, E=6, k=2, d_ffn=200, capacity_factor=0.9, temperature=0.5,
                            gumbel=True, dtype="f32", seed=7), 0.1),
    # few tokens over a wide d: the router cuts d into K slices (4 here) and adds them in a
    # second kernel; E = 24 spans two 16-expert MFMA tiles; Gumbel noise at tau = 0.8
    "router_slices": (MoEShape("router_slices", T=300, d=1024, E=24, k=3, d_ffn=128, capacity_factor=1.0,
                               temperature=0.8, gumbel=True, seed=3, wg_std=None), 0.2),
    # E > 32 with more than 1024 token groups: the router takes 64 tokens per workgroup; the last
    # workgroup holds one 16-token group
    "router_wide_tiles": (MoEShape("router_wide_tiles", T=16400, d=128, E=40, k=2, d_ffn=64, capacity_factor=1.0,
                                   wg_std=None), 0.1),
    # tokens spanning many 16-token routing groups and 64-token permutation waves, E not a multiple of 16
    "many_blocks": (MoEShape("many_blocks", T=3000, d=128, E=37, k=4, d_ffn=128, capacity_factor=1.1,
                             wg_std=None), 0.0),
    # tiled-panel edges: C = 256, two experts keep exactly one full 256-row panel (kept 249, 256,
    # 256); d = 192 and d_ffn = 320 leave partial column panels and a 6-step K
    "panel_256": (MoEShape("panel_256", T=768, d=192, E=3, k=1, d_ffn=320, capacity_factor=1.0, wg_std=None), 0.05),
    # C = 257: two experts spill one row into a second panel (kept 249, 257, 257)
    "panel_257": (MoEShape("panel_257", T=771, d=192, E=3, k=1, d_ffn=320, capacity_factor=1.0, wg_std=None), 0.05),
    # d_ffn = 8192: GEMM1 over 32 column panels with pair-staged A rows read through the
    # permutation, two row panels per expert
    "wide_ffn": (MoEShape("wide_ffn", T=600, d=128, E=3, k=2, d_ffn=8192, capacity_factor=1.0, wg_std=None), 0.05),
    # the streaming router (W_g in LDS, waves owning whole 16-token groups): 2501 groups over
    # 2048 wave slots, so some waves take two groups; a last group of 3 tokens; E = 12 pads the
    # expert tile; Gumbel noise at tau = 0.6
    "router_stream": (MoEShape("router_stream", T=40003, d=128, E=12, k=2, d_ffn=64, capacity_factor=1.0,
                               temperature=0.6, gumbel=True, seed=11, wg_std=None), 0.1),
    # GEMM2 over K = 8192 (256 K steps) on 40 row tiles: each XCD's 5 tiles are split into 6 K
    # parts of 42 or 44 steps, pair-staged W2 rows ending exactly at the end of W2
    "split_p6": (MoEShape("split_p6", T=4800, d=256, E=8, k=2, d_ffn=8192, capacity_factor=1.25), 0.05),
    # C = 119: every row tile holds at most 128 rows and runs WIDE (the four waves side by side,
    # 64 columns each), some at most 64; d = 320 and d_ffn = 192 leave waves with part or none
    # of their columns inside N; biases set
    "wide_tiles": (MoEShape("wide_tiles", T=1900, d=320, E=32, k=2, d_ffn=192, capacity_factor=1.0), 0.1),
    # WIDE tiles under the tail split: GEMM2 has 4 tiles, each cut into 8 K parts written to the
    # side buffer and added by the fixup kernel
    "wide_split": (MoEShape("wide_split", T=200, d=256, E=4, k=2, d_ffn=2048, capacity_factor=1.0), 0.05),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_small(name):
    shape, bias = SMALL[name]
    print(f"[gpu] forward small {name} {shape}", flush=True)
    stats = check_forward_full(Problem(shape, bias_std=bias))
    print(f"[gpu]   {name}: {stats}", flush=True)


def test_exact_ties_route_to_lowest_index():
    # W_g = 0, no bias: every logit is 0, so every token picks experts 0..k-1, p = 1/E exactly,
    # and L = E * sum f P = 1 exactly (P uniform).
    shape = MoEShape("ties", T=256, d=64, E=8, k=3, d_ffn=64, capacity_factor=4.0)
    p = Problem(shape)
    p.arrays["Wg"][:] = 0
    p = Problem(shape, arrays=p.arrays)
    gpu = run_forward(p)
    assert np.all(gpu["topk_idx"] == np.arange(3)[None, :])
    assert np.all(gpu["logits"] == 0.0)
    assert np.all(gpu["P"] == np.float32(1.0 / 8)) and gpu["L"][0] == 1.0
    check_forward_full(p, gpu)


STAGE_SHAPES = {
    "one_level_scan": MoEShape("stages", T=900, d=128, E=6, k=2, d_ffn=256, capacity_factor=0.8, temperature=0.8,
                               gumbel=True, seed=99),
    # 313 groups of 64 experts: the scan and the route stage's column sums take two levels
    "two_level_scan": MoEShape("stages2", T=5000, d=64, E=64, k=2, d_ffn=64, capacity_factor=0.8, temperature=0.8,
                               gumbel=True, seed=98, wg_std=None),
}


@pytest.mark.parametrize("which", sorted(STAGE_SHAPES))
def test_stages_match_forward_and_oracle(which):
    """moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine: bitwise equal to moe_forward,
    and each stage checked against the oracle on its own inputs."""
    shape = STAGE_SHAPES[which]
    print(f"[gpu] stages {which} {shape}", flush=True)
    p = Problem(shape, bias_std=0.05)
    cfg = p.cfg
    x, Wg, bg, W1, b1, W2, b2 = p.args()
    ws = ops.workspace(cfg, x.device)
    r = ops.route(cfg, x, Wg, bg, ws=ws)
    dsp = ops.dispatch(cfg, r["topk_idx"], x, ws=ws)
    y_perm = ops.expert_ffn(cfg, dsp["x_perm"], dsp["kept"], dsp["offsets"], W1, b1, W2, b2, ws=ws)
    cmb = ops.combine(cfg, y_perm, dsp["dest"], r["topk_w"], dsp["counts"], r["prob_colsum"], ws=ws)
    torch.cuda.synchronize()
    fwd = run_forward(p)
    for key, a in (("logits", r["logits"]), ("scores", r["scores"]), ("topk_idx", r["topk_idx"]),
                   ("topk_w", r["topk_w"]), ("prob_colsum", r["prob_colsum"]), ("counts", dsp["counts"]),
                   ("kept", dsp["kept"]), ("offsets", dsp["offsets"]), ("dest", dsp["dest"]), ("f", cmb["f"]),
                   ("P", cmb["P"]), ("L", cmb["L"])):
        np.testing.assert_array_equal(a.cpu().numpy(), fwd[key], err_msg=key)
    assert torch.equal(cmb["y"], fwd["y_raw"])
    # stage by stage against the oracle
    host = p.host
    z_ref = oracle.logits(host["x"], host["Wg"], host["bg"])
    check_logits(r["logits"].cpu().numpy(), z_ref)
    gpu = {k: v.cpu().numpy() for k, v in r.items()}
    gpu.update({k: v.cpu().numpy() for k, v in dsp.items() if k != "x_perm"})
    gpu.update({k: v.cpu().numpy() for k, v in cmb.items() if k != "y"})
    chk = check_routing(p, gpu)
    n = int(chk["dispatch"]["kept"].sum())
    xp = dsp["x_perm"].float().cpu().numpy()[:n]
    np.testing.assert_array_equal(xp, host["x"][chk["dispatch"]["perm"]])          # gather is a pure copy
    y_perm_ref = oracle.expert_ffn(xp.astype(np.float64), chk["dispatch"]["kept"], chk["dispatch"]["offsets"],
                                   host["W1"], host["b1"], host["W2"], host["b2"])
    check_output(y_perm.cpu().numpy()[:n], y_perm_ref, "bf16", "y_perm")
    y_ref = oracle.combine(y_perm.cpu().numpy()[:n].astype(np.float64), chk["dispatch"]["dest"],
                           r["topk_w"].cpu().numpy().astype(np.float64))
    # combine alone: float32 accumulation of the GPU's own y_perm, one bf16 rounding
    err = np.abs(cmb["y"].float().cpu().numpy() - y_ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(y_ref) + 1e-6)


def test_dispatch_from_given_indices_is_bit_exact():
    # moe_dispatch on indices chosen here (skewed to force drops), against the oracle dispatch
    rng = np.random.default_rng(5)
    T, E, k, d = 2500, 12, 3, 64
    shape = MoEShape("dispatch", T=T, d=d, E=E, k=k, d_ffn=64, capacity_factor=0.7)
    p = Problem(shape)
    weights = np.arange(1, E + 1, dtype=np.float64) ** -1.0
    idx = np.stack([rng.choice(E, size=k, replace=False, p=weights / weights.sum()) for _ in range(T)])
    idx_dev = torch.from_numpy(idx.astype(np.int32)).cuda()
    out = ops.dispatch(p.cfg, idx_dev, p.dev["x"])
    torch.cuda.synchronize()
    C = oracle.capacity(T, E, k, 0.7)
    ref = oracle.dispatch(idx, E, C)
    assert ref["drops"].sum() > 0
    for key in ("counts", "kept", "offsets", "dest"):
        np.testing.assert_array_equal(out[key].cpu().numpy(), ref[key], err_msg=key)
    n = int(ref["kept"].sum())
    np.testing.assert_array_equal(out["perm"].cpu().numpy()[:n], ref["perm"])
    np.testing.assert_array_equal(out["x_perm"].float().cpu().numpy()[:n], p.host["x"][ref["perm"]])


DET_SHAPES = {
    "full_tiles": MoEShape("det", T=2048, d=256, E=8, k=2, d_ffn=512, capacity_factor=1.0, gumbel=True,
                           temperature=0.5),
    # about 125 rows per expert: WIDE GEMM tiles, and the permutation fused into the scan
    "wide_fused": MoEShape("det_wide", T=1000, d=192, E=16, k=2, d_ffn=320, capacity_factor=1.0, gumbel=True,
                           temperature=0.7),
}


@pytest.mark.parametrize("name", sorted(DET_SHAPES))
def test_forward_is_deterministic(name):
    shape = DET_SHAPES[name]
    p = Problem(shape, bias_std=0.05)
    a = run_forward(p)
    b = run_forward(p)
    for key in a:
        if key == "y_raw":
            assert torch.equal(a[key], b[key])
        else:
            np.testing.assert_array_equal(a[key], b[key], err_msg=key)


@pytest.mark.parametrize("name", ["tiny_fp32", "mixtral_like", "switch_skew", "decode", "gumbel_longtail"])
def test_named_workloads(name):
    shape = CONFIGS[name]
    print(f"[gpu] named workload {name} {shape}", flush=True)
    p = Problem(shape)
    if name == "tiny_fp32":
        stats = check_forward_full(p)
        # the tiny config also matches the brute-force dense loop (every expert on every token)
        gpu = run_forward(p)
        bf = oracle.brute_dense(*p.host_args(), k=shape.k, capacity_factor=shape.capacity_factor,
                                given_scores=gpu["scores"])
        check_output(gpu["y"], bf["y"], "f32", "tiny_fp32_brute_dense")
    elif name == "gumbel_longtail":
        # 65536 tokens: every token's routing; outputs of one token in every (expert, 256-row
        # tile) of the grouped GEMMs plus 256 uniform ones (the rms estimate)
        stats = check_forward_sampled(p, n_random=256)
    else:
        # every token's output against the oracle's whole-batch forward
        stats = check_forward_full(p)
    print(f"[gpu]   {name}: {stats}", flush=True)
