"""Seeded synthetic inputs for the ReLU-gated FFN workloads.

This package holds only input generation (random draws, bf16 rounding of the
draws, per-neuron gate biases that set a target activation probability). It
holds none of the FFN's arithmetic, and it is shared by the CPU oracle, the
tests and the benchmark.
"""
from .synth import CONFIGS, Workload, make_workload, round_bf16, bf16_bits

__all__ = ["CONFIGS", "Workload", "make_workload", "round_bf16", "bf16_bits"]
