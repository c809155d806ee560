"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and rounds them to the storage type the
workload names (bf16, or fp32 for the MXFP4 workload whose quantisation is
part of the method).  It holds none of the attention arithmetic: no scores,
no softmax, no quantiser.  Both the CPU oracle and the GPU path receive the
exact same bytes from here.
"""

from .gen import bf16_bits_to_f64, f32_to_bf16_bits, normal_bf16, normal_f32
from .configs import CONFIGS, Workload, workload

__all__ = [
    "CONFIGS",
    "Workload",
    "workload",
    "normal_bf16",
    "normal_f32",
    "f32_to_bf16_bits",
    "bf16_bits_to_f64",
]
