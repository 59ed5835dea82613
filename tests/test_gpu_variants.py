"""GPU parity of the forward variants (moe_forward_ex) against the CPU oracle (MI355X).

SiLU experts on the MFMA GEMM, the decode-sized GEMV and the float32 paths; Gaussian router
noise on the one-kernel and the K-sliced router; a shared expert on the MFMA, GEMV and float32
paths, alone and combined with SiLU and noise; the Mixtral-like layer with a shared expert at
full size (sampled rows). Tolerances are those of tests/parity.py.
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_41_amd import ops
from workloads import CONFIGS, MoEShape

from .parity import Problem, check_forward_full, check_forward_sampled, run_forward

pytestmark = pytest.mark.gpu

CASES = {
    # name: (shape, bias_std, activation, noise_std, shared_d_ffn)
    "silu_gemm": (MoEShape("silu_gemm", T=1000, d=256, E=8, k=2, d_ffn=384, capacity_factor=1.0), 0.1,
                  "silu", 0.0, 0),
    "silu_gemv": (MoEShape("silu_gemv", T=777, d=192, E=64, k=1, d_ffn=128, capacity_factor=1.0, wg_std=None), 0.05,
                  "silu", 0.0, 0),
    "silu_f32": (MoEShape("silu_f32", T=300, d=96, E=6, k=2, d_ffn=200, capacity_factor=0.9, dtype="f32", seed=7),
                 0.1, "silu", 0.0, 0),
    "gaussian": (MoEShape("gaussian", T=700, d=128, E=6, k=2, d_ffn=192, capacity_factor=0.8, temperature=0.9,
                          seed=21), 0.0, "gelu", 0.3, 0),
    "gaussian_sliced_router": (MoEShape("gaussian_sliced_router", T=300, d=1024, E=24, k=3, d_ffn=128,
                                        capacity_factor=1.0, seed=5, wg_std=None), 0.0, "gelu", 0.2, 0),
    "shared": (MoEShape("shared", T=900, d=128, E=6, k=2, d_ffn=256, capacity_factor=0.8), 0.1, "gelu", 0.0, 320),
    "shared_silu_noise": (MoEShape("shared_silu_noise", T=1000, d=256, E=8, k=2, d_ffn=384, capacity_factor=0.7,
                                   temperature=0.8, seed=3), 0.05, "silu", 0.1, 512),
    "shared_gemv": (MoEShape("shared_gemv", T=12, d=128, E=4, k=2, d_ffn=64, capacity_factor=1.0), 0.1, "gelu",
                    0.0, 128),
    "shared_f32": (MoEShape("shared_f32", T=200, d=64, E=5, k=2, d_ffn=96, capacity_factor=0.9, dtype="f32"), 0.1,
                   "silu", 0.0, 72),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_forward_variant(name):
    shape, bias, act, noise, ds = CASES[name]
    print(f"[gpu] variant {name} {shape} act={act} noise={noise} shared={ds}", flush=True)
    p = Problem(shape, bias_std=bias, activation=act, noise_std=noise, shared_d_ffn=ds)
    stats = check_forward_full(p)
    print(f"[gpu]   {name}: {stats}", flush=True)


def test_zero_variant_is_moe_forward():
    shape = MoEShape("plain", T=900, d=128, E=6, k=2, d_ffn=256, capacity_factor=0.8, gumbel=True, temperature=0.7)
    p = Problem(shape, bias_std=0.05)
    a = run_forward(p)
    plan = ops.ForwardPlan(p.cfg, *p.args(), variant=ops.make_variant(p.cfg))
    b = plan.run()
    torch.cuda.synchronize()
    assert torch.equal(a["y_raw"], b["y"])
    for key in ("topk_idx", "dest", "kept", "f", "P", "L"):
        np.testing.assert_array_equal(a[key], b[key].cpu().numpy(), err_msg=key)


def test_mixtral_like_with_shared_expert_and_silu():
    shape = CONFIGS["mixtral_like"]
    print(f"[gpu] named workload mixtral_like + shared expert 14336 + SiLU", flush=True)
    p = Problem(shape, activation="silu", shared_d_ffn=14336)
    stats = check_forward_sampled(p)
    print(f"[gpu]   {stats}", flush=True)
