"""CPU oracle (test infrastructure only; see moe_oracle's header)."""
from .moe_oracle import (activation, combine, expert_ffn, gather_rows, gelu, moe_layer,
                         moe_layer_expert_major,
                         permute, route_topk, silu)

__all__ = ["activation", "combine", "expert_ffn", "gather_rows", "gelu", "moe_layer",
           "moe_layer_expert_major",
           "permute", "route_topk", "silu"]
