"""Seeded synthetic inputs for the NVFP4 routed-MoE layer.

This package only draws random numbers in the shapes, sizes and distributions
of the layer's workloads. It holds none of the layer's arithmetic (no decoding
of codes, no routing, no GEMM), so both the fp64 oracle tests and the HIP path
can take their inputs from it without sharing any of the method.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    DECODE_TS,
    MoEWorkload,
    ROUTER_SCALE2,
    RouterBank,
    WeightBank,
    make_router,
    make_weights,
    make_workload,
    workload_for,
)
