"""Seeded synthetic workloads for the fused GEMM + epilogue path.

This module only describes the transformer-layer workloads (shapes,
storage dtypes, value distributions, the ordered epilogue program as plain
data) and draws seeded inputs for them.  It holds none of the method's
arithmetic: the HIP path and the CPU oracle each turn the symbolic program
into their own representation and compute independently.

Distributions follow the workload descriptions of the CODA pages' experiment
section (GPT-2 / BERT / LLaMA shaped layers; "CODA: Rewriting Transformer
Blocks as GEMM-Epilogue Programs", section 4).  ``N(0, v)`` is read with ``v``
the variance, so that ``W ~ N(0, 1/K)`` keeps unit output variance.
"""
from .spec import CONFIGS, WorkloadSpec, TensorSpec, get_config, scaled_config
from .gen import make_inputs, bf16_bits_from_f64, bf16_bits_to_f64, draw_tensor

__all__ = [
    "CONFIGS", "WorkloadSpec", "TensorSpec", "get_config", "scaled_config",
    "make_inputs", "bf16_bits_from_f64", "bf16_bits_to_f64", "draw_tensor",
]
