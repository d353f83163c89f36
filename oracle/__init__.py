"""CPU oracle for the block-scaled MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg, never by the product package.
"""
from . import reference  # noqa: F401
