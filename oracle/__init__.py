"""CPU oracle of the sparse MoE FFN layer forward (numpy, float64).

TEST INFRASTRUCTURE: a plain, slow, obviously correct implementation that the GPU path is
checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
cpu_baseline leg may import it; the product path never does, and the oracle imports nothing
from the product package.

Parity status: every function here is pinned by ``tests/test_oracle_*.py`` to something other
than itself (closed forms, library routines, brute force, the pages' stated invariants,
hand-worked fixtures under ``tests/golden/``). The Philox generator is pinned to rocRAND's
Philox-4x32-10 called as a library.
"""
from . import philox
from .moe_layer import (backward, backward_entries, balance_stats, brute_dense, capacity, combine, dispatch, dispatch_policy, dispatch_random,
                        dispatch_reroute, expert, next_choices, reweight,
                        expert_ffn, forward, forward_rows, gelu, gelu_grad, logits, renormalise, route,
                        route_from_scores, routing_stats, scores, shared_expert, silu, silu_grad, softmax, temperature_at, topk)

__all__ = ["philox", "capacity", "logits", "scores", "softmax", "topk", "renormalise", "route", "route_from_scores",
           "dispatch", "expert", "expert_ffn", "gelu", "silu", "combine", "balance_stats", "forward",
           "forward_rows", "brute_dense", "shared_expert", "temperature_at", "routing_stats", "dispatch_random",
           "dispatch_reroute", "dispatch_policy", "next_choices", "reweight", "backward", "backward_entries", "gelu_grad",
           "silu_grad"]
