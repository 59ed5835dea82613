"""Torch-facing binding of the MoE C ABI: argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the layer runs in the
library's HIP kernels. Each function mirrors one entry point of include/moe.h and allocates
its outputs (and, unless one is passed, a workspace) with torch on the inputs' device.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (BWD_STAGE_NAMES, MOE_BACKWARD_STAGES, MOE_FORWARD_STAGES, STAGE_NAMES, MoeBackwardAux, MoeConfig,
                   MoeForwardAux, make_config)

__all__ = ["make_config", "capacity", "workspace_size", "workspace", "route", "dispatch", "expert_ffn", "combine",
           "forward", "ForwardPlan", "StageEvents", "STAGE_NAMES", "MoeConfig", "make_variant", "workspace_size_ex",
           "temperature_at", "DROP_POLICIES", "ROUTE_STAT_NAMES", "TrainPlan", "BWD_STAGE_NAMES",
           "MOE_BACKWARD_STAGES", "workspace_size_train", "probe_copy", "probe_mfma"]


def _storage_dtype(cfg: MoeConfig) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == _lib.MOE_BF16 else torch.float32


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("MoE tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("MoE tensors must be contiguous")
    return t.data_ptr()


def _expect(t: torch.Tensor | None, name: str, shape, dtype, optional=False) -> None:
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def capacity(cfg: MoeConfig) -> int:
    c = _lib.load().moe_capacity(ctypes.byref(cfg))
    if c < 0:
        _lib.check(_lib.load().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(ctypes.c_size_t())))
    return int(c)


def workspace_size(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.load().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)))
    return int(n.value)


def workspace(cfg: MoeConfig, device) -> torch.Tensor:
    return torch.empty(workspace_size(cfg), dtype=torch.uint8, device=device)


def rows_max(cfg: MoeConfig) -> int:
    """Rows of the expert-sorted buffers: min(k*T, E*C)."""
    C = min(capacity(cfg), cfg.T)
    return min(cfg.k * cfg.T, cfg.E * C)


def route(cfg: MoeConfig, x, Wg, bg=None, ws=None, want_scores=True) -> dict:
    sd = _storage_dtype(cfg)
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    _expect(x, "x", (T, d), sd)
    _expect(Wg, "Wg", (E, d), sd)
    _expect(bg, "bg", (E,), torch.float32, optional=True)
    dev = x.device
    ws = workspace(cfg, dev) if ws is None else ws
    out = {
        "logits": torch.empty((T, E), dtype=torch.float32, device=dev),
        "scores": torch.empty((T, E), dtype=torch.float32, device=dev) if want_scores else None,
        "topk_idx": torch.empty((T, k), dtype=torch.int32, device=dev),
        "topk_w": torch.empty((T, k), dtype=torch.float32, device=dev),
        "prob_colsum": torch.empty((E,), dtype=torch.float32, device=dev),
    }
    _lib.check(_lib.load().moe_route(
        ctypes.byref(cfg), _ptr(x), _ptr(Wg), _ptr(bg), _ptr(out["logits"]), _ptr(out["scores"]),
        _ptr(out["topk_idx"]), _ptr(out["topk_w"]), _ptr(out["prob_colsum"]), _ptr(ws), ws.numel(), _stream()))
    return out


def dispatch(cfg: MoeConfig, topk_idx, x, ws=None) -> dict:
    sd = _storage_dtype(cfg)
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    _expect(topk_idx, "topk_idx", (T, k), torch.int32)
    _expect(x, "x", (T, d), sd)
    dev = x.device
    ws = workspace(cfg, dev) if ws is None else ws
    R = rows_max(cfg)
    out = {
        "counts": torch.empty((E,), dtype=torch.int32, device=dev),
        "kept": torch.empty((E,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((E,), dtype=torch.int32, device=dev),
        "dest": torch.empty((T, k), dtype=torch.int32, device=dev),
        "perm": torch.full((R,), -1, dtype=torch.int32, device=dev),
        "x_perm": torch.zeros((R, d), dtype=sd, device=dev),
    }
    _lib.check(_lib.load().moe_dispatch(
        ctypes.byref(cfg), _ptr(topk_idx), _ptr(x), _ptr(out["counts"]), _ptr(out["kept"]), _ptr(out["offsets"]),
        _ptr(out["dest"]), _ptr(out["perm"]), _ptr(out["x_perm"]), _ptr(ws), ws.numel(), _stream()))
    return out


def expert_ffn(cfg: MoeConfig, x_perm, kept, offsets, W1, b1, W2, b2, ws=None) -> torch.Tensor:
    sd = _storage_dtype(cfg)
    E, d, dff = cfg.E, cfg.d, cfg.d_ffn
    R = rows_max(cfg)
    _expect(x_perm, "x_perm", (R, d), sd)
    _expect(kept, "kept", (E,), torch.int32)
    _expect(offsets, "offsets", (E,), torch.int32)
    _expect(W1, "W1", (E, dff, d), sd)
    _expect(b1, "b1", (E, dff), sd, optional=True)
    _expect(W2, "W2", (E, d, dff), sd)
    _expect(b2, "b2", (E, d), sd, optional=True)
    dev = x_perm.device
    ws = workspace(cfg, dev) if ws is None else ws
    y_perm = torch.zeros((R, d), dtype=torch.float32, device=dev)
    _lib.check(_lib.load().moe_expert_ffn(
        ctypes.byref(cfg), _ptr(x_perm), _ptr(kept), _ptr(offsets), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
        _ptr(y_perm), _ptr(ws), ws.numel(), _stream()))
    return y_perm


def combine(cfg: MoeConfig, y_perm, dest, topk_w, counts=None, prob_colsum=None, ws=None) -> dict:
    sd = _storage_dtype(cfg)
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    _expect(y_perm, "y_perm", (rows_max(cfg), d), torch.float32)
    _expect(dest, "dest", (T, k), torch.int32)
    _expect(topk_w, "topk_w", (T, k), torch.float32)
    stats = counts is not None
    dev = y_perm.device
    ws = workspace(cfg, dev) if ws is None else ws
    out = {"y": torch.empty((T, d), dtype=sd, device=dev)}
    if stats:
        _expect(counts, "counts", (E,), torch.int32)
        _expect(prob_colsum, "prob_colsum", (E,), torch.float32)
        out.update(f=torch.empty((E,), dtype=torch.float32, device=dev),
                   P=torch.empty((E,), dtype=torch.float32, device=dev),
                   L=torch.empty((1,), dtype=torch.float32, device=dev))
    _lib.check(_lib.load().moe_combine(
        ctypes.byref(cfg), _ptr(y_perm), _ptr(dest), _ptr(topk_w), _ptr(counts), _ptr(prob_colsum), _ptr(out["y"]),
        _ptr(out.get("f")), _ptr(out.get("P")), _ptr(out.get("L")), _ptr(ws), ws.numel(), _stream()))
    return out


class StageEvents:
    """n_stages + 1 HIP events for per-stage timing (moe_forward's MOE_FORWARD_STAGES by default)."""

    def __init__(self, n_stages: int = MOE_FORWARD_STAGES):
        self.n = n_stages
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.array = (ctypes.c_void_p * (self.n + 1))()
        for i in range(self.n + 1):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.array[i] = ev
        self.totals = [0.0] * self.n
        self.samples = 0

    def accumulate(self) -> list[float]:
        """Per-stage milliseconds of the last recorded forward (synchronises on the last event)."""
        if self._hip.hipEventSynchronize(self.array[self.n]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = []
        for i in range(self.n):
            t = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(t), self.array[i], self.array[i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            ms.append(t.value)
            self.totals[i] += t.value
        self.samples += 1
        return ms

    def mean_ms(self) -> dict:
        n = max(1, self.samples)
        return {name: self.totals[i] / n for i, name in enumerate(STAGE_NAMES)}

    def close(self):
        for i in range(self.n + 1):
            if self.array[i]:
                self._hip.hipEventDestroy(self.array[i])
                self.array[i] = None


DROP_POLICIES = {"token": _lib.MOE_DROP_TOKEN_ORDER, "random": _lib.MOE_DROP_RANDOM, "reroute": _lib.MOE_DROP_REROUTE}
ROUTE_STAT_NAMES = ("loss_sq", "loss_quant", "loss_var", "usage_std", "entropy")


def make_variant(cfg: MoeConfig, activation: str = "gelu", noise_std: float = 0.0, shared=None,
                 drop_policy: str = "token", route_stats=None, packed_weights: bool = False):
    """A moe_variant: expert activation ("gelu" or "silu"), Gaussian router noise std, an
    optional shared expert ``shared = (W1s [ds,d], b1s [ds] or None, W2s [d,ds], b2s [d] or
    None)``, the capacity policy ("token", "random", "reroute"), an optional float32 device
    tensor of MOE_ROUTE_STATS elements for the routing statistics (ROUTE_STAT_NAMES order), and
    whether W1 and W2 come from pack_expert_weights (MOE_WEIGHTS_PACKED).
    Returns (variant, tensors kept alive for it)."""
    sd = _storage_dtype(cfg)
    v = _lib.MoeVariant()
    v.activation = {"gelu": _lib.MOE_ACT_GELU, "silu": _lib.MOE_ACT_SILU}[activation]
    v.noise_std = float(noise_std)
    v.drop_policy = DROP_POLICIES[drop_policy]
    v.weight_layout = _lib.MOE_WEIGHTS_PACKED if packed_weights else _lib.MOE_WEIGHTS_LINEAR
    keep = {}
    if shared is not None:
        W1s, b1s, W2s, b2s = shared
        ds = W1s.shape[0]
        _expect(W1s, "W1s", (ds, cfg.d), sd)
        _expect(b1s, "b1s", (ds,), sd, optional=True)
        _expect(W2s, "W2s", (cfg.d, ds), sd)
        _expect(b2s, "b2s", (cfg.d,), sd, optional=True)
        v.shared_d_ffn = int(ds)
        v.W1s, v.b1s, v.W2s, v.b2s = _ptr(W1s), _ptr(b1s), _ptr(W2s), _ptr(b2s)
        keep["shared"] = tuple(shared)
    if route_stats is not None:
        _expect(route_stats, "route_stats", (_lib.MOE_ROUTE_STATS,), torch.float32)
        v.route_stats = _ptr(route_stats)
        keep["route_stats"] = route_stats
    return v, keep


def pack_expert_weights(W, stream=None):
    """moe_pack_expert_weights: a new tensor of W's shape [E, rows, cols] (bf16, on W's device)
    holding W's values in the packed panel order that moe_forward_ex reads when the variant says
    packed_weights. Its element order is not W's: it is meant only for that call."""
    if W.dtype != torch.bfloat16 or W.dim() != 3 or not W.is_contiguous():
        raise ValueError("W must be a contiguous [E, rows, cols] bfloat16 tensor")
    out = torch.empty_like(W)
    E, rows, cols = W.shape
    _lib.check(_lib.load().moe_pack_expert_weights(int(E), int(rows), int(cols), _ptr(W), _ptr(out),
                                                    _stream(stream)))
    return out


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """moe_probe_copy: dst's bytes = src's bytes (contiguous device tensors of the same byte size,
    a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _lib.check(_lib.load().moe_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def probe_mfma(out: torch.Tensor, workgroups: int, iters: int, stream=None) -> float:
    """moe_probe_mfma into out (float32, workgroups * 256 elements); returns the flops issued."""
    _expect(out, "out", (int(workgroups) * 256,), torch.float32)
    _lib.check(_lib.load().moe_probe_mfma(_ptr(out), int(workgroups), int(iters), _stream(stream)))
    return float(workgroups) * 4 * _lib.MOE_PROBE_CHAINS * iters * 16 * 16 * 32 * 2


def workspace_size_ex(cfg: MoeConfig, variant) -> int:
    n = ctypes.c_size_t()
    _lib.check(_lib.load().moe_workspace_size_ex(ctypes.byref(cfg), ctypes.byref(variant), ctypes.byref(n)))
    return n.value


def temperature_at(step: int, tau0: float = 1.0, tau_min: float = 0.5, rate: float = 1e-4) -> float:
    """moe_temperature_at: max(tau_min, tau0 - rate * step), rounded to float32."""
    return float(_lib.load().moe_temperature_at(int(step), float(tau0), float(tau_min), float(rate)))


class ForwardPlan:
    """Preallocated outputs and workspace for repeated moe_forward calls on fixed tensors.
    ``variant`` (from make_variant) selects moe_forward_ex."""

    def __init__(self, cfg: MoeConfig, x, Wg, bg, W1, b1, W2, b2, keep_routing: bool = True, variant=None,
                 workspace_bytes: int | None = None):
        sd = _storage_dtype(cfg)
        T, d, E, k, dff = cfg.T, cfg.d, cfg.E, cfg.k, cfg.d_ffn
        _expect(x, "x", (T, d), sd)
        _expect(Wg, "Wg", (E, d), sd)
        _expect(bg, "bg", (E,), torch.float32, optional=True)
        _expect(W1, "W1", (E, dff, d), sd)
        _expect(b1, "b1", (E, dff), sd, optional=True)
        _expect(W2, "W2", (E, d, dff), sd)
        _expect(b2, "b2", (E, d), sd, optional=True)
        dev = x.device
        self.cfg = cfg
        self.inputs = (x, Wg, bg, W1, b1, W2, b2)
        self.variant = variant
        if workspace_bytes is not None:
            self.ws = torch.empty((workspace_bytes,), dtype=torch.uint8, device=dev)
        elif variant is None:
            self.ws = workspace(cfg, dev)
        else:
            self.ws = torch.empty((workspace_size_ex(cfg, variant[0]),), dtype=torch.uint8, device=dev)
        f32, i32 = torch.float32, torch.int32
        self.out = {
            "y": torch.empty((T, d), dtype=sd, device=dev),
            "f": torch.empty((E,), dtype=f32, device=dev),
            "P": torch.empty((E,), dtype=f32, device=dev),
            "L": torch.empty((1,), dtype=f32, device=dev),
            "counts": torch.empty((E,), dtype=i32, device=dev),
            "kept": torch.empty((E,), dtype=i32, device=dev),
        }
        if variant is not None and "route_stats" in variant[1]:
            self.out["route_stats"] = variant[1]["route_stats"]
        self.aux = MoeForwardAux()
        if keep_routing:
            R = rows_max(cfg)
            self.out.update(
                logits=torch.empty((T, E), dtype=f32, device=dev),
                scores=torch.empty((T, E), dtype=f32, device=dev),
                topk_idx=torch.empty((T, k), dtype=i32, device=dev),
                topk_w=torch.empty((T, k), dtype=f32, device=dev),
                offsets=torch.empty((E,), dtype=i32, device=dev),
                dest=torch.empty((T, k), dtype=i32, device=dev),
                perm=torch.full((R,), -1, dtype=i32, device=dev),
                prob_colsum=torch.empty((E,), dtype=f32, device=dev),
            )
            for name in ("logits", "scores", "topk_idx", "topk_w", "offsets", "dest", "perm", "prob_colsum"):
                setattr(self.aux, name, self.out[name].data_ptr())
        self._args = None

    def run(self, events: StageEvents | None = None, stream=None) -> dict:
        self.aux.stage_events = ctypes.cast(events.array, ctypes.c_void_p).value if events is not None else None
        x, Wg, bg, W1, b1, W2, b2 = self.inputs
        o = self.out
        args = (_ptr(x), _ptr(Wg), _ptr(bg), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                _ptr(o["y"]), _ptr(o["f"]), _ptr(o["P"]), _ptr(o["L"]), _ptr(o["counts"]), _ptr(o["kept"]),
                ctypes.byref(self.aux), _ptr(self.ws), self.ws.numel(), _stream(stream))
        self._call(_lib.load(), ctypes.byref(self.cfg), args)
        return o

    def _call(self, lib, cfg, args):
        if self.variant is None:
            _lib.check(lib.moe_forward(cfg, *args))
        else:
            _lib.check(lib.moe_forward_ex(cfg, ctypes.byref(self.variant[0]), *args))


def forward(cfg: MoeConfig, x, Wg, bg, W1, b1, W2, b2, keep_routing: bool = True, variant=None) -> dict:
    """The whole layer (moe_forward, or moe_forward_ex with a variant); returns y, f, P, L,
    counts, kept (+ routing arrays)."""
    return ForwardPlan(cfg, x, Wg, bg, W1, b1, W2, b2, keep_routing=keep_routing, variant=variant).run()


def workspace_size_train(cfg: MoeConfig, variant=None) -> int:
    n = ctypes.c_size_t()
    v = ctypes.byref(variant[0]) if variant is not None else None
    _lib.check(_lib.load().moe_workspace_size_train(ctypes.byref(cfg), v, ctypes.byref(n)))
    return n.value


class TrainPlan(ForwardPlan):
    """moe_forward_train then moe_backward on fixed tensors: ``run()`` is the training forward
    (outputs as ForwardPlan), ``backward(dy, lam)`` the gradients (float32 weight gradients,
    dx in the storage dtype). The workspace holds the forward's saved state in between."""

    def __init__(self, cfg: MoeConfig, x, Wg, bg, W1, b1, W2, b2, keep_routing: bool = True, variant=None,
                 bias_grads: bool = True):
        super().__init__(cfg, x, Wg, bg, W1, b1, W2, b2, keep_routing=keep_routing, variant=variant,
                         workspace_bytes=workspace_size_train(cfg, variant))
        T, d, E, dff = cfg.T, cfg.d, cfg.E, cfg.d_ffn
        dev = x.device
        f32 = torch.float32
        self.grads = {
            "dx": torch.empty((T, d), dtype=_storage_dtype(cfg), device=dev),
            "dWg": torch.empty((E, d), dtype=f32, device=dev),
            "dW1": torch.empty((E, dff, d), dtype=f32, device=dev),
            "dW2": torch.empty((E, d, dff), dtype=f32, device=dev),
            "dz": torch.empty((T, E), dtype=f32, device=dev),
        }
        if bias_grads:
            self.grads.update(dbg=torch.empty((E,), dtype=f32, device=dev),
                              db1=torch.empty((E, dff), dtype=f32, device=dev),
                              db2=torch.empty((E, d), dtype=f32, device=dev))
        self.baux = MoeBackwardAux()
        self.baux.dz = self.grads["dz"].data_ptr()

    def _call(self, lib, cfg, args):
        v = ctypes.byref(self.variant[0]) if self.variant is not None else None
        _lib.check(lib.moe_forward_train(cfg, v, *args))

    def backward(self, dy, lam: float = 0.0, events: StageEvents | None = None, stream=None) -> dict:
        _expect(dy, "dy", (self.cfg.T, self.cfg.d), _storage_dtype(self.cfg))
        x, Wg, bg, W1, b1, W2, b2 = self.inputs
        g = self.grads
        self.baux.stage_events = ctypes.cast(events.array, ctypes.c_void_p).value if events is not None else None
        v = ctypes.byref(self.variant[0]) if self.variant is not None else None
        _lib.check(_lib.load().moe_backward(
            ctypes.byref(self.cfg), v, _ptr(x), _ptr(Wg), _ptr(W1), _ptr(W2), _ptr(dy), float(lam),
            _ptr(g["dx"]), _ptr(g["dWg"]), _ptr(g.get("dbg")), _ptr(g["dW1"]), _ptr(g.get("db1")), _ptr(g["dW2"]),
            _ptr(g.get("db2")), ctypes.byref(self.baux), _ptr(self.ws), self.ws.numel(), _stream(stream)))
        return g
