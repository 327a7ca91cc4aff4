"""fp64 CPU oracle for the dropless MoE layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU
baseline, never by the GPU library.  It shares no code with the GPU path; the only thing both
sides see is the seeded input arrays from the ``workloads`` package.

Every function is pinned by CPU tests against properties the pages and the mathematics fix
(library sort routines, dense-MLP closed forms, finite differences, conservation identities);
the pages themselves print no worked values.
"""
from .formats import (bf16_to_f64, e4m3_to_f64, dequant_rows_1x128, dequant_blocks_128x128, e8m0_to_f64,
                      e4m3_encode_rne, mx_block_exponent, mx_quantize, mx_dequantize, mx_roundtrip_rows)
from .moe_ref import (route, plan, Plan, forward, backward, token_forward, token_backward,
                      weight_grad_entries, expert_weight_grads, d_logits_from_dw, router_logits,
                      router_backward)

__all__ = ["bf16_to_f64", "e4m3_to_f64", "dequant_rows_1x128", "dequant_blocks_128x128", "e8m0_to_f64",
           "e4m3_encode_rne", "mx_block_exponent", "mx_quantize", "mx_dequantize", "mx_roundtrip_rows", "route",
           "plan", "Plan", "forward", "backward", "token_forward", "token_backward",
           "weight_grad_entries", "expert_weight_grads", "d_logits_from_dw", "router_logits", "router_backward"]
