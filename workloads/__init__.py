"""Seeded synthetic inputs for the sparse lightning-indexer KL-loss backward.

This package only draws random inputs (queries, keys, head weights, top-k index
lists, target distributions).  It holds none of the operator's arithmetic, so
both the fp64 CPU oracle and the GPU path can be fed from it without sharing
any computation.
"""
from .gen import (  # noqa: F401
    ATTN_P_WORKLOADS,
    AttnPInputs,
    AttnPWorkload,
    DENSE_WORKLOADS,
    DenseInputs,
    Inputs,
    Workload,
    WORKLOADS,
    make_attn_p_inputs,
    make_dense_inputs,
    make_inputs,
    round_to_bf16,
    round_to_f16,
    workload,
)
