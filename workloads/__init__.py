"""Seeded synthetic inputs shared by the HIP path's tests/benchmarks and the CPU oracle.

This package draws input tensors only; it contains none of the attention
method's arithmetic.
"""
from .configs import WORKLOADS, Workload, get
from .synth import bf16_bits, head_tensors, make_inputs, round_to_bf16

__all__ = ["WORKLOADS", "Workload", "get", "make_inputs", "head_tensors", "round_to_bf16", "bf16_bits"]
