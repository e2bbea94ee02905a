"""Seeded synthetic workloads for the paged-KV hot path.

This package only draws random numbers and lays out the order of block-manager
operations; it holds none of the attention, block-allocation or copy-on-write
arithmetic. Both the oracle side (tests, CPU baseline) and the GPU side consume
exactly the values produced here.
"""
from .synth import (  # noqa: F401
    DTYPES,
    Workload,
    AddOp,
    AppendOp,
    ForkOp,
    FreeOp,
    SwapOutOp,
    SwapInOp,
    make_swap_workload,
    make_workload,
    make_decode_workload,
    make_ragged_workload,
    make_churn_workload,
    CONFIG_NAMES,
    gen_kv,
    gen_q,
    round_to_dtype,
    dtype_nbytes,
)
