"""Seeded synthetic inputs shared by the GPU library's tests/bench and the oracle.

This package draws inputs and lays them out; it holds none of the method's
arithmetic.  See ``workloads.gen``.
"""
from .gen import (  # noqa: F401
    MODULE_NAMES, ModuleSpec, Workload, bf16_bits, bf16_to_f32, make_workload,
    WORKLOADS, normal_bf16, build_workload, build_workload_for_tests,
)
