"""CPU oracle (test infrastructure only; see moe_oracle's header)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (combine, dequant, dequant_q4_0, dequant_q8_0,  # noqa: F401
                         expert_ffn, lru_simulate, moe_ffn_pairs, moe_layer,
                         permute, renormalize, route, router_logits, silu,
                         softmax, topk_gap, topk_select)
