"""The C-ABI library without a GPU: it loads, exports every symbol include/moe.h declares,
computes the capacity and workspace size on the host, and rejects bad arguments before any
HIP call. No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import oracle
from sparse_mixture_experts_41_amd import _lib
from sparse_mixture_experts_41_amd._lib import (MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_OK, MoeConfig,
                                                make_config)
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmoe.so is not built (python -m sparse_mixture_experts_41_amd.build)")
    return _lib.load()


HEADERS = sorted(os.path.join(ROOT, "include", n) for n in os.listdir(os.path.join(ROOT, "include"))
                 if n.endswith(".h"))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward", "moe_capacity",
              "moe_workspace_size", "moe_status_str", "moe_last_error", "moe_probe_copy", "moe_probe_mfma"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_struct_layout_matches_header(lib):
    assert ctypes.sizeof(MoeConfig) == 72
    assert MoeConfig.seed.offset == 56 and MoeConfig.dtype.offset == 64


def _cfg(name):
    c = CONFIGS[name]
    return make_config(c.T, c.d, c.E, c.k, c.d_ffn, c.capacity_factor, c.temperature, c.gumbel, c.seed, c.dtype)


def test_capacity_matches_the_oracle_formula(lib):
    for name, c in CONFIGS.items():
        assert lib.moe_capacity(ctypes.byref(_cfg(name))) == oracle.capacity(c.T, c.E, c.k, c.capacity_factor)
    for (T, E, k, cf) in [(10, 11, 1, 1.1), (10, 3, 2, 1.0), (5, 8, 1, 0.5), (1000, 7, 3, 1.37), (3, 7, 1, 1e-300),
                          (12345, 64, 8, 0.999), (1, 1, 1, 3.0)]:
        cfg = make_config(T, 64, E, k, 64, cf)
        assert lib.moe_capacity(ctypes.byref(cfg)) == oracle.capacity(T, E, k, cf), (T, E, k, cf)


def test_workspace_size_is_positive_and_monotone(lib):
    n = ctypes.c_size_t()
    sizes = {}
    for name in CONFIGS:
        assert lib.moe_workspace_size(ctypes.byref(_cfg(name)), ctypes.byref(n)) == MOE_OK
        sizes[name] = n.value
        assert n.value % 256 == 0 and n.value > 0
    assert sizes["gumbel_longtail"] > sizes["mixtral_like"] > sizes["tiny_fp32"]


@pytest.mark.parametrize("field,value,status", [
    ("T", 0, MOE_EINVAL), ("d", 0, MOE_EINVAL), ("E", 0, MOE_EINVAL), ("k", 0, MOE_EINVAL),
    ("k", 9, MOE_EINVAL),                     # k > E (E = 8)
    ("capacity_factor", 0.0, MOE_EINVAL), ("capacity_factor", -1.0, MOE_EINVAL),
    ("capacity_factor", float("inf"), MOE_EINVAL), ("capacity_factor", float("nan"), MOE_EINVAL),
    ("temperature", 0.0, MOE_EINVAL), ("temperature", float("nan"), MOE_EINVAL),
    ("gumbel", 2, MOE_EINVAL), ("dtype", 7, MOE_EINVAL), ("reserved", 1, MOE_EINVAL),
    ("E", 65, MOE_EUNSUPPORTED), ("d", 4100, MOE_EUNSUPPORTED), ("d_ffn", 100, MOE_EUNSUPPORTED),
    ("capacity_factor", 3.0e6, MOE_EUNSUPPORTED),
])
def test_invalid_configs_are_rejected(lib, field, value, status):
    cfg = _cfg("mixtral_like")
    setattr(cfg, field, value)
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)) == status
    assert lib.moe_capacity(ctypes.byref(cfg)) == -1
    assert lib.moe_last_error() != b""


def test_k_above_8_and_token_overflow(lib):
    cfg = make_config(16, 64, 16, 9, 64, 1.0)
    assert lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(ctypes.c_size_t())) == MOE_EUNSUPPORTED
    cfg = make_config(1 << 29, 64, 16, 4, 64, 1.0)
    assert lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(ctypes.c_size_t())) == MOE_EINVAL
    f32 = make_config(1 << 17, 64, 4, 2, 64, 1.0, dtype="f32")
    assert lib.moe_workspace_size(ctypes.byref(f32), ctypes.byref(ctypes.c_size_t())) == MOE_EUNSUPPORTED


# Fake device addresses: never dereferenced, because each call below fails validation first.
A16 = 0x100000
MIS = 0x100004


def _route_args(cfg, **over):
    args = dict(x=A16, Wg=A16, bg=None, logits=A16, scores=None, idx=A16, w=A16, colsum=A16, ws=A16, ws_bytes=0)
    args.update(over)
    return (ctypes.byref(cfg), args["x"], args["Wg"], args["bg"], args["logits"], args["scores"], args["idx"],
            args["w"], args["colsum"], args["ws"], args["ws_bytes"], None)


def test_null_misaligned_and_workspace_checks(lib):
    cfg = _cfg("mixtral_like")
    assert lib.moe_route(*_route_args(cfg, x=None)) == MOE_EINVAL
    assert b"x is NULL" in lib.moe_last_error()
    assert lib.moe_route(*_route_args(cfg, Wg=MIS)) == MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()
    assert lib.moe_route(*_route_args(cfg, ws_bytes=1024)) == MOE_EWORKSPACE
    n = ctypes.c_size_t()
    lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n))
    assert lib.moe_route(*_route_args(cfg, ws=A16 + 16, ws_bytes=n.value)) == MOE_EINVAL   # ws not 256-aligned
    bad = _cfg("mixtral_like")
    bad.k = 0
    assert lib.moe_route(*_route_args(bad)) == MOE_EINVAL
    # the other entry points reject a NULL config and NULL required pointers the same way
    assert lib.moe_dispatch(None, A16, A16, A16, A16, A16, A16, A16, A16, A16, 0, None) == MOE_EINVAL
    assert lib.moe_dispatch(ctypes.byref(cfg), None, A16, A16, A16, A16, A16, A16, A16, A16, 0, None) == MOE_EINVAL
    assert lib.moe_expert_ffn(ctypes.byref(cfg), A16, A16, A16, None, None, A16, None, A16, A16, 0, None) == MOE_EINVAL
    assert lib.moe_combine(ctypes.byref(cfg), A16, A16, A16, None, None, A16, A16, None, None, A16, 0,
                           None) == MOE_EINVAL                                     # f given without P, L
    assert lib.moe_forward(ctypes.byref(cfg), A16, A16, None, A16, None, A16, None, A16, A16, A16, A16, A16, A16,
                           None, A16, 0, None) == MOE_EWORKSPACE


def test_status_strings(lib):
    for s in range(5):
        assert lib.moe_status_str(s).startswith(b"MOE_")


def test_variant_struct_layout(lib):
    from sparse_mixture_experts_41_amd._lib import MoeVariant
    assert ctypes.sizeof(MoeVariant) == 64
    assert MoeVariant.noise_std.offset == 4 and MoeVariant.shared_d_ffn.offset == 8 and MoeVariant.W1s.offset == 16
    assert MoeVariant.b2s.offset == 40
    assert MoeVariant.drop_policy.offset == 48 and MoeVariant.weight_layout.offset == 52
    assert MoeVariant.route_stats.offset == 56


def _ws_ex(lib, cfg, v):
    n = ctypes.c_size_t()
    return lib.moe_workspace_size_ex(ctypes.byref(cfg), ctypes.byref(v) if v is not None else None, ctypes.byref(n)), n


def test_variant_validation(lib):
    from sparse_mixture_experts_41_amd._lib import MoeVariant
    cfg = _cfg("mixtral_like")
    st, plain = _ws_ex(lib, cfg, None)
    assert st == MOE_OK
    n0 = ctypes.c_size_t()
    lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n0))
    assert plain.value == n0.value                       # a NULL variant is the plain layer
    assert _ws_ex(lib, cfg, MoeVariant())[1].value == n0.value
    assert _ws_ex(lib, cfg, MoeVariant(activation=2))[0] == MOE_EINVAL
    assert _ws_ex(lib, cfg, MoeVariant(noise_std=-0.1))[0] == MOE_EINVAL
    assert _ws_ex(lib, cfg, MoeVariant(noise_std=float("nan")))[0] == MOE_EINVAL
    assert _ws_ex(lib, _cfg("gumbel_longtail"), MoeVariant(noise_std=0.1))[0] == MOE_EINVAL   # two noises
    assert _ws_ex(lib, cfg, MoeVariant(shared_d_ffn=100))[0] == MOE_EUNSUPPORTED             # bf16: 64 | d_ffn_s
    assert _ws_ex(lib, cfg, MoeVariant(shared_d_ffn=-64))[0] == MOE_EINVAL
    st, with_shared = _ws_ex(lib, cfg, MoeVariant(shared_d_ffn=14336))
    assert st == MOE_OK and with_shared.value >= n0.value + cfg.T * 14336 * 2 + cfg.T * cfg.d * 4
    # moe_forward_ex: a shared expert needs its weights (checked before any HIP call)
    v = MoeVariant(shared_d_ffn=1024)
    args = (A16, A16, None, A16, None, A16, None, A16, A16, A16, A16, A16, A16, None, A16, 1 << 40, None)
    assert lib.moe_forward_ex(ctypes.byref(cfg), ctypes.byref(v), *args) == MOE_EINVAL
    assert b"W1s is NULL" in lib.moe_last_error()
    v.W1s, v.W2s, v.b1s = A16, A16, MIS + 1
    assert lib.moe_forward_ex(ctypes.byref(cfg), ctypes.byref(v), *args) == MOE_EINVAL      # b1s misaligned
    assert b"b1s" in lib.moe_last_error()


def test_variant_policy_and_stats_validation(lib):
    from sparse_mixture_experts_41_amd._lib import MOE_DROP_RANDOM, MOE_DROP_REROUTE, MoeVariant
    cfg = _cfg("mixtral_like")
    n0 = _ws_ex(lib, cfg, None)[1].value
    assert _ws_ex(lib, cfg, MoeVariant(drop_policy=3))[0] == MOE_EINVAL
    assert _ws_ex(lib, cfg, MoeVariant(drop_policy=-1))[0] == MOE_EINVAL
    assert _ws_ex(lib, cfg, MoeVariant(weight_layout=2))[0] == MOE_EINVAL
    assert _ws_ex(lib, cfg, MoeVariant(route_stats=MIS + 2))[0] == MOE_EINVAL
    assert b"route_stats" in lib.moe_last_error()
    ng, TE = (cfg.T + 15) // 16, cfg.T * cfg.k
    st, rnd = _ws_ex(lib, cfg, MoeVariant(drop_policy=MOE_DROP_RANDOM))
    assert st == MOE_OK and rnd.value >= n0 + 2 * ng * cfg.E * 4 + cfg.E * 8
    st, rr = _ws_ex(lib, cfg, MoeVariant(drop_policy=MOE_DROP_REROUTE, route_stats=A16))
    assert st == MOE_OK and rr.value >= n0 + 2 * TE * 4 + 2 * ng * cfg.E * 4 + cfg.E * 4 + ng * 4


def test_packed_weight_layout_validation(lib):
    """Packed weights: bf16 only, d and d_ffn multiples of 256, forward only; the pack entry point
    checks its sizes and pointers before it launches anything."""
    from sparse_mixture_experts_41_amd._lib import MOE_WEIGHTS_PACKED, MoeVariant
    packed = MoeVariant(weight_layout=MOE_WEIGHTS_PACKED)
    for name in ("mixtral_like", "switch_skew", "decode", "gumbel_longtail"):
        c = CONFIGS[name]
        want = MOE_OK if (c.d % 256 == 0 and c.d_ffn % 256 == 0) else MOE_EUNSUPPORTED
        assert _ws_ex(lib, _cfg(name), packed)[0] == want, name
    assert _ws_ex(lib, _cfg("tiny_fp32"), packed)[0] == MOE_EUNSUPPORTED          # float32
    assert b"bf16" in lib.moe_last_error()
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size_train(ctypes.byref(_cfg("mixtral_like")), ctypes.byref(packed),
                                        ctypes.byref(n)) == MOE_EUNSUPPORTED
    assert b"row-major" in lib.moe_last_error()
    pack = lib.moe_pack_expert_weights
    assert pack(8, 14336, 4096, None, A16, None) == MOE_EINVAL
    assert pack(8, 14336, 4096, A16, MIS + 2, None) == MOE_EINVAL                  # misaligned
    assert pack(0, 256, 32, A16, A16 + (1 << 30), None) == MOE_EINVAL
    assert pack(8, 100, 4096, A16, A16 + (1 << 30), None) == MOE_EUNSUPPORTED      # rows % 256
    assert pack(8, 256, 40, A16, A16 + (1 << 30), None) == MOE_EUNSUPPORTED        # cols % 32
    assert pack(1 << 21, 256, 32, A16, A16 + (1 << 40), None) == MOE_EINVAL        # too large
    assert pack(2, 256, 32, A16, A16 + 256 * 32 * 2, None) == MOE_EINVAL           # overlap
    assert b"overlap" in lib.moe_last_error()


def test_temperature_schedule_matches_the_oracle(lib):
    import numpy as np
    for step, rate in [(0, 1e-4), (2500, 1e-4), (5000, 1e-4), (10 ** 6, 1e-4), (250, 1e-3), (333, 1e-3)]:
        assert lib.moe_temperature_at(step, 1.0, 0.5, rate) == np.float32(oracle.temperature_at(step, rate=rate))


def test_training_entry_points_validate_on_the_host(lib):
    from sparse_mixture_experts_41_amd._lib import MoeBackwardAux, MoeVariant
    assert ctypes.sizeof(MoeBackwardAux) == 16
    cfg = _cfg("mixtral_like")
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size_train(ctypes.byref(cfg), None, ctypes.byref(n)) == MOE_OK
    n_fwd = ctypes.c_size_t()
    lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n_fwd))
    c = CONFIGS["mixtral_like"]
    R = min(c.k * c.T, c.E * oracle.capacity(c.T, c.E, c.k, c.capacity_factor))
    # saved pre-activations and the transposed activations at least; the bf16 MFMA path reads the
    # weights as given, so the workspace holds no transposed copy of them (2 E d d_ffn bf16)
    need = n_fwd.value + R * c.d_ffn * 2 + 2 * (c.d + c.d_ffn) * R * 2
    wt = 2 * c.E * c.d * c.d_ffn * 2
    assert need <= n.value < need + wt
    # the float32 path multiplies transposed weights: its workspace holds both copies
    cfg32 = _cfg("tiny_fp32")
    n32, n32_fwd = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.moe_workspace_size_train(ctypes.byref(cfg32), None, ctypes.byref(n32)) == MOE_OK
    lib.moe_workspace_size(ctypes.byref(cfg32), ctypes.byref(n32_fwd))
    t = CONFIGS["tiny_fp32"]
    assert n32.value >= n32_fwd.value + 2 * t.E * t.d * t.d_ffn * 4
    shared = MoeVariant(shared_d_ffn=1024)
    assert lib.moe_workspace_size_train(ctypes.byref(cfg), ctypes.byref(shared), ctypes.byref(n)) == MOE_EUNSUPPORTED
    # moe_backward rejects bad arguments before any HIP call
    args = [A16, A16, A16, A16, A16, ctypes.c_float(0.1), A16, A16, None, A16, None, A16, None, None, A16,
            ctypes.c_size_t(1 << 40), None]
    bad = list(args)
    bad[4] = None                                                   # dy
    assert lib.moe_backward(ctypes.byref(cfg), None, *bad) == MOE_EINVAL
    assert b"dy is NULL" in lib.moe_last_error()
    bad = list(args)
    bad[5] = ctypes.c_float(float("inf"))
    assert lib.moe_backward(ctypes.byref(cfg), None, *bad) == MOE_EINVAL
    bad = list(args)
    bad[15] = ctypes.c_size_t(1024)                                 # workspace too small
    assert lib.moe_backward(ctypes.byref(cfg), None, *bad) == MOE_EWORKSPACE
    assert lib.moe_backward(ctypes.byref(cfg), ctypes.byref(shared), *args) == MOE_EUNSUPPORTED


def test_probes_reject_bad_arguments_before_any_launch(lib):
    # every check runs before the first HIP call, so these return without touching a GPU
    dummy = ctypes.c_void_p(1 << 20)
    assert lib.moe_probe_copy(None, dummy, 1024, None) == MOE_EINVAL
    assert lib.moe_probe_copy(dummy, ctypes.c_void_p((1 << 20) + 4096), 1000, None) == MOE_EINVAL   # not 16 k
    assert lib.moe_probe_copy(dummy, ctypes.c_void_p((1 << 20) + 512), 1024, None) == MOE_EINVAL    # overlap
    assert lib.moe_probe_copy(ctypes.c_void_p((1 << 20) + 8), ctypes.c_void_p(1 << 24), 1024, None) == MOE_EINVAL
    assert lib.moe_probe_mfma(None, 4, 10, None) == MOE_EINVAL
    assert lib.moe_probe_mfma(dummy, 0, 10, None) == MOE_EINVAL
    assert lib.moe_probe_mfma(dummy, 4, 0, None) == MOE_EINVAL
    assert lib.moe_probe_mfma(dummy, (1 << 20) + 1, 10, None) == MOE_EINVAL
    assert b"iters" in lib.moe_last_error() or b"workgroups" in lib.moe_last_error()


def test_noalloc_rejects_a_large_workspace_before_any_hip_call(lib):
    # the Mixtral-like layer needs far more workspace than the static scratch: refused up front
    cfg = _cfg("mixtral_like")
    n = ctypes.c_size_t()
    assert lib.moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)) == MOE_OK
    assert n.value > _lib.MOE_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(1 << 20)
    st = lib.moe_forward_noalloc(ctypes.byref(cfg), p, p, None, p, None, p, None, p, p, p, p, p, p, None, None)
    assert st == MOE_EUNSUPPORTED
    assert b"static scratch" in lib.moe_last_error()
