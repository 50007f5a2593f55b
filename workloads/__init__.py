"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path's
tests and benchmark.  Nothing here computes any part of the attention step."""
from .synth import (RequestSpec, Workload, build_workload, normal_bf16, float32_to_bf16_bits,
                    bf16_bits_to_float32, align_up, BF16_NAN)
from . import configs

__all__ = ["RequestSpec", "Workload", "build_workload", "normal_bf16", "float32_to_bf16_bits",
           "bf16_bits_to_float32", "align_up", "BF16_NAN", "configs"]
