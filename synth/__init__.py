"""Seeded synthetic workloads for the MoE expert layer.

This package is shared by the CPU oracle's tests, the GPU parity tests and
the benchmark.  It holds workload shapes and random-number recipes only: no
routing, GEMM, combine or hashing arithmetic of the method lives here.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .inputs import make_inputs, make_router_inputs, make_batch, f32_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
