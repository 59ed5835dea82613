"""moe_forward_noalloc on the GPU: the allocation-free forward (its workspace is the library's
static device scratch) gives bit for bit the outputs of moe_forward with a caller workspace,
on consecutive calls on one device whose inputs shrink (the scratch keeps the previous call's
intermediates; nothing in it may leak into the next result) and on both expert paths (the
MFMA grouped GEMM and the decode-sized GEMV). Called through the C ABI with ctypes."""
import ctypes

import pytest
import torch

from sparse_mixture_experts_41_amd import _lib, ops
from workloads import MoEShape

from .parity import Problem

pytestmark = pytest.mark.gpu

SHAPES = [
    # MFMA path with Gumbel routing, drops and biases; about 20 MB of workspace
    (MoEShape("noalloc_gemm", T=1000, d=256, E=8, k=2, d_ffn=512, capacity_factor=1.0, gumbel=True,
              temperature=0.7, seed=5), 0.05),
    # a smaller input right after it
    (MoEShape("noalloc_smaller", T=130, d=128, E=4, k=2, d_ffn=256, capacity_factor=1.25, seed=6), 0.05),
    # decode-sized: C = 8, the GEMV path
    (MoEShape("noalloc_gemv", T=64, d=512, E=16, k=2, d_ffn=256, capacity_factor=1.0, seed=7), 0.05),
]


def _noalloc(p: Problem) -> dict:
    cfg = p.cfg
    x, Wg, bg, W1, b1, W2, b2 = p.args()
    T, d, E = cfg.T, cfg.d, cfg.E
    dev = x.device
    out = {"y": torch.empty((T, d), dtype=x.dtype, device=dev),
           "f": torch.empty((E,), dtype=torch.float32, device=dev),
           "P": torch.empty((E,), dtype=torch.float32, device=dev),
           "L": torch.empty((1,), dtype=torch.float32, device=dev),
           "counts": torch.empty((E,), dtype=torch.int32, device=dev),
           "kept": torch.empty((E,), dtype=torch.int32, device=dev)}
    ptr = lambda t: None if t is None else t.data_ptr()
    status = _lib.load().moe_forward_noalloc(
        ctypes.byref(cfg), ptr(x), ptr(Wg), ptr(bg), ptr(W1), ptr(b1), ptr(W2), ptr(b2), ptr(out["y"]),
        ptr(out["f"]), ptr(out["P"]), ptr(out["L"]), ptr(out["counts"]), ptr(out["kept"]), None,
        torch.cuda.current_stream().cuda_stream)
    _lib.check(status)
    return out


def test_noalloc_equals_moe_forward_on_consecutive_calls():
    for shape, bias in SHAPES:
        print(f"[gpu] noalloc {shape}", flush=True)
        p = Problem(shape, bias_std=bias)
        assert ops.workspace_size(p.cfg) <= _lib.MOE_NOALLOC_SCRATCH_BYTES
        ref = ops.ForwardPlan(p.cfg, *p.args(), keep_routing=False).run()
        got = _noalloc(p)
        torch.cuda.synchronize()
        assert torch.equal(got["y"].view(torch.int16), ref["y"].view(torch.int16)), shape.name
        for key in ("f", "P", "L", "counts", "kept"):
            assert torch.equal(got[key], ref[key]), (shape.name, key)
        assert int(got["kept"].sum()) > 0


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    shape = MoEShape("noalloc_too_big", T=4096, d=1024, E=8, k=2, d_ffn=4096, capacity_factor=1.25)
    p = Problem(shape)
    assert ops.workspace_size(p.cfg) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(_lib.MoeError) as exc:
        _noalloc(p)
    assert exc.value.status == _lib.MOE_EUNSUPPORTED and "static scratch" in exc.value.detail
