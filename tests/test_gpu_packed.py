"""Packed expert weights (moe_pack_expert_weights, MOE_WEIGHTS_PACKED) on the GPU (MI355X).

The pack is pure data movement, so its output is compared bit for bit with the layout's
definition written out in numpy: W [E, rows, cols] viewed as [E, rows/256, 256, cols/32, 32]
with the 256-row and 32-column block axes swapped. The forward on packed weights feeds the same
values to the same MFMA and GEMV kernels in the same summation order as the row-major forward,
so every output must equal that forward's bit for bit: on the MFMA path (ragged row tiles, the
split tail of GEMM2, biases), on the decode-sized GEMV path, with a shared expert and SiLU, and
on the Mixtral-like layer at full size. Two cases also go through the oracle parity check of
tests/parity.py directly.
"""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_41_amd import ops
from workloads import CONFIGS, MoEShape

from .parity import Problem, check_forward_full, run_forward

pytestmark = pytest.mark.gpu


def _packed_reference(W: np.ndarray) -> np.ndarray:
    E, rows, cols = W.shape
    return W.reshape(E, rows // 256, 256, cols // 32, 32).transpose(0, 1, 3, 2, 4).reshape(E, rows, cols)


@pytest.mark.parametrize("E,rows,cols", [(1, 256, 32), (3, 512, 96), (2, 768, 4096)])
def test_pack_matches_the_layout_definition(E, rows, cols):
    print(f"[gpu] pack E={E} rows={rows} cols={cols}", flush=True)
    g = torch.Generator().manual_seed(E * 1000 + cols)
    bits = torch.randint(-32768, 32768, (E, rows, cols), generator=g, dtype=torch.int32).to(torch.int16)
    W = bits.view(torch.bfloat16).cuda()             # every bit pattern, NaNs included
    Wp = ops.pack_expert_weights(W)
    torch.cuda.synchronize()
    got = Wp.view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(got, _packed_reference(bits.numpy()))


CASES = {
    # name: (shape, bias_std, activation, shared_d_ffn)
    "gemm_ragged_bias": (MoEShape("gemm_ragged_bias", T=1000, d=256, E=6, k=2, d_ffn=512, capacity_factor=1.0), 0.1,
                         "gelu", 0),
    "gemm_drops": (MoEShape("gemm_drops", T=1500, d=512, E=8, k=2, d_ffn=768, capacity_factor=0.6, seed=4), 0.0,
                   "gelu", 0),
    "gemv_decode": (MoEShape("gemv_decode", T=40, d=256, E=16, k=2, d_ffn=512, capacity_factor=1.0, seed=9), 0.05,
                    "gelu", 0),
    "shared_silu": (MoEShape("shared_silu", T=900, d=256, E=6, k=2, d_ffn=256, capacity_factor=0.8, seed=2), 0.1,
                    "silu", 320),
}


def _same(a: dict, b: dict, name: str):
    assert torch.equal(a["y_raw"].view(torch.int16), b["y_raw"].view(torch.int16)), f"{name}: y differs"
    for key in ("f", "P", "L", "counts", "kept", "dest", "topk_idx", "topk_w"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=f"{name}: {key}")


@pytest.mark.parametrize("name", sorted(CASES))
def test_packed_forward_equals_row_major(name):
    shape, bias, act, ds = CASES[name]
    print(f"[gpu] packed vs row-major {name} {shape} act={act} shared={ds}", flush=True)
    row = Problem(shape, bias_std=bias, activation=act, shared_d_ffn=ds)
    packed = Problem(shape, bias_std=bias, arrays=row.arrays, activation=act, shared_d_ffn=ds, packed_weights=True)
    _same(run_forward(row), run_forward(packed), name)


@pytest.mark.parametrize("name", ["gemm_ragged_bias", "gemv_decode"])
def test_packed_forward_parity_with_the_oracle(name):
    shape, bias, act, ds = CASES[name]
    print(f"[gpu] packed parity {name}", flush=True)
    stats = check_forward_full(Problem(shape, bias_std=bias, activation=act, shared_d_ffn=ds, packed_weights=True))
    print(f"[gpu]   {name}: {stats}", flush=True)


def test_packed_forward_equals_row_major_mixtral_like():
    shape = CONFIGS["mixtral_like"]
    print("[gpu] packed vs row-major mixtral_like (full size)", flush=True)
    row = Problem(shape)
    a = run_forward(row)
    packed = Problem(shape, arrays=row.arrays, packed_weights=True)
    _same(a, run_forward(packed), "mixtral_like")
