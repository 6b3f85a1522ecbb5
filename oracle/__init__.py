"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .coda_oracle import (
    gelu_tanh, gelu_tanh_grad, sigmoid, silu, swiglu_pair, rms, rmsnorm,
    deferred_rmsnorm_gemm, rmsnorm_backward, layernorm, ln_fold, deferred_layernorm_gemm,
    logical_b, gemm, apply_epilogue, forward,
    philox4x64, philox4x64_scalar, dropout, dropout_keep, dropout_words, dropout_threshold,
)
from .run import run_workload, resolve_program

__all__ = [
    "gelu_tanh", "gelu_tanh_grad", "sigmoid", "silu", "swiglu_pair", "rms", "rmsnorm",
    "deferred_rmsnorm_gemm", "rmsnorm_backward", "layernorm", "ln_fold", "deferred_layernorm_gemm", "logical_b", "gemm", "apply_epilogue", "forward",
    "philox4x64", "philox4x64_scalar", "dropout", "dropout_keep", "dropout_words", "dropout_threshold",
    "run_workload", "resolve_program",
]
