"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This package holds random-number generation and workload shapes only: none of
the MoE method's arithmetic lives here.
"""
from .gen import (  # noqa: F401
    splitmix64_ref,
    uniform,
    normal,
    make_x,
    make_logits,
    make_weight,
    make_expert_weights,
)
from .workloads import WORKLOADS, Workload  # noqa: F401
