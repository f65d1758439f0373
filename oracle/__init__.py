"""CPU float64 oracle of the GLM-5.2 MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY: importable by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package.
"""
from . import mx
from .moe import (Routing, bf16_bits_to_f64, block_ffn, decode, dense_ffn, expert_load,
                  expert_hidden_mx, expert_mlp, expert_mlp_mx, forward, forward_arrays, forward_mx,
                  forward_mx_on_hidden, group_scores,
                  rmsnorm, round_bf16, route, select_topk, select_topk_grouped, sigmoid, silu,
                  topk_gap)

__all__ = ["Routing", "bf16_bits_to_f64", "block_ffn", "decode", "dense_ffn", "expert_load",
           "expert_hidden_mx", "expert_mlp", "expert_mlp_mx", "forward", "forward_arrays",
           "forward_mx", "forward_mx_on_hidden",
           "group_scores", "mx", "rmsnorm", "round_bf16", "route", "select_topk",
           "select_topk_grouped", "sigmoid", "silu", "topk_gap"]
