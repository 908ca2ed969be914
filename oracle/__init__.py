"""CPU oracle of the DeepSeekMoE layer forward: TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package.  It shares no code with the HIP library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (NEAR_TIE, Routing, Perm, ForwardResult, lift, router_affinity,
                         biased_scores, group_scores, select_experts, gate_values, permute,
                         route, silu, expert_ffn, expert_ffn_fp8, expert_f64, dequant_blocks, forward,
                         bias_update, load_ratio, e4m3_decode, e4m3_quantize, quantize_1x128,
                         dequantize_1x128, fake_quant_1x128, max_row_rel_err, E4M3_MAX)
