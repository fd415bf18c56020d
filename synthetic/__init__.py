"""Seeded synthetic inputs for the APB-V approximate-attention prefill.

This package is shared by the tests, the benchmark and the oracle's callers. It holds only
workload shapes, the random draws and the bf16 rounding of inputs: none of the method's
arithmetic (scoring, selection, gathering or attention) lives here.
"""
from .configs import CONFIGS, Workload, sweep_layouts, workload
from .gen import Inputs, generate, bf16_bits, bf16_round, frame_partition

__all__ = ["CONFIGS", "Workload", "sweep_layouts", "workload", "Inputs", "generate", "bf16_bits",
           "bf16_round", "frame_partition"]
