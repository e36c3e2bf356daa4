"""Oracle package -- test infrastructure only (see moe_oracle.py)."""
from .moe_oracle import (dequant_int4, dispatch, forward, gate_weights, route, router_logits,
                         select_topk, silu, swiglu_ffn, topk_gap)

__all__ = ["dequant_int4", "dispatch", "forward", "gate_weights", "route", "router_logits",
           "select_topk", "silu", "swiglu_ffn", "topk_gap"]
