"""CPU oracle of the MoE expert layer -- test infrastructure only.

Imported only by the tests, the smoke check and the benchmark's CPU-baseline
leg; the product path never imports it.  See moe_oracle.py.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (widen, store, route_select, route_weights, route, slot_map,  # noqa: F401
                         slot_map_ranks, rank_base_offsets, dispatch, swiglu_up, down_proj, expert_ffn, combine,
                         forward, combine_bwd, swiglu_bwd, input_grad, expert_ffn_bwd_data,
                         expert_ffn_bwd_weight, dispatch_bwd, route_bwd, backward,
                         tokens_forward, tokens_backward, expert_wgrad_columns)
