"""The peak probes of include/moe_probe.h on the GPU: the copy kernel copies exactly, and the
MFMA loop writes finite values that repeat bit for bit (it is a timing kernel; its result only
has to exist)."""
import pytest
import torch

from sparse_mixture_experts_41_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (64 << 20) + 48])
def test_probe_copy_copies(nbytes):
    print(f"[gpu] probe copy {nbytes} bytes", flush=True)
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8).cuda()
    dst = torch.zeros_like(src)
    ops.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_mfma_is_finite_and_repeatable():
    print("[gpu] probe mfma", flush=True)
    out = torch.empty(64 * 256, dtype=torch.float32, device="cuda")
    flops = ops.probe_mfma(out, 64, 50)
    torch.cuda.synchronize()
    a = out.clone()
    ops.probe_mfma(out, 64, 50)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, out)
    assert flops == 64 * 4 * 16 * 50 * 16 * 16 * 32 * 2
