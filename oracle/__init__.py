"""CPU oracle of the MoE-layer hot path (route, dispatch, expert SwiGLU MLP, combine), and of the
fp8 block-scaled token rows an fp8 dispatch ships (oracle/fp8.py), and of the combine with
sender-side partial accumulation (oracle/sender_combine.py).

TEST INFRASTRUCTURE ONLY: plain, slow, float64 reference code. Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it. It shares no code with the HIP path and never imports it.

Parity pins: every function here is pinned by tests that do not re-run its own formula (brute force
over tiny inputs, closed forms, invariants the pages state, and special cases that reduce to library
routines); see tests/test_oracle_*.py.
"""
from .moe import (Layout, combine, dispatch, expert_mlp, moe_layer, router_logits, routing_weights,
                  row_experts, silu, topk_select, topk_softmax)
from . import fp8, sender_combine
from .numerics import (bf16_bits_to_f64, f64_to_bf16_bits, from_f64, round_to_bf16, round_to_f32,
                       to_f64)

__all__ = ["fp8", "sender_combine", "Layout", "combine", "dispatch", "expert_mlp", "moe_layer", "router_logits",
           "routing_weights", "row_experts", "silu", "topk_select", "topk_softmax",
           "bf16_bits_to_f64", "f64_to_bf16_bits", "from_f64", "round_to_bf16", "round_to_f32",
           "to_f64"]
