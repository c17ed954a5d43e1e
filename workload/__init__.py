"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package only draws numbers and lays them out in the canonical input
formats; it holds none of the method's arithmetic (no routing, no dequant,
no matmul, no cache policy).
"""
from .gen import (  # noqa: F401
    ROOT_SEED,
    Workload,
    WORKLOADS,
    expert_bytes,
    q4_matrix,
    expert_weights,
    layer_weights,
    router_weights,
    activations,
    step_activations,
    zipf_logits,
    zipf_popularity,
    rank_permutation,
    frequency_table,
)
