"""CPU oracle for the MoE-layer forward -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 numpy implementation of what the layer computes, written
from the pages' description of the method.  It shares no code with the HIP
library and imports nothing from it.  Only the tests, the smoke check of the
entry module and the CPU-baseline leg of the benchmark may import or run it;
the product path never does.

Every function is pinned by CPU tests against something other than itself
(brute force on tiny inputs, closed forms, invariants, library routines).
See moe.py for the passages each step follows.
"""
from .moe import (  # noqa: F401
    widen, e4m3_decode, dequant_blocks, e4m3_round, fp8_block_scale_exponents, fp8_quantize_rows,
    router_logits, select_topk, gate_weights,
    route, permute, silu, expert_ffn, combine, moe_forward, moe_forward_view,
    moe_forward_tokens,
    InputsView, rel_frobenius, near_tie_tokens,
)
