"""Declarative description of the workloads.

Each workload is: GEMM shape (M, N, K) where N is the width the contraction
computes, the storage layout of B, storage dtypes, the tensors to draw (in the
order they are drawn), and the ordered epilogue program as a list of
``(op_name, args)`` pairs whose arguments name tensors.  Op names:

  scale(alpha)              v *= alpha
  scale_row(vec)            v[i,j] *= vec[i]
  scale_col(vec)            v[i,j] *= vec[j]
  rms_rowscale(gamma, eps)  deferred RMSNorm row scale (must come first)
  ln_rowscale(gamma, beta, eps)  deferred LayerNorm of A's rows with gain gamma
                            and shift beta (must come first)
  add_col(vec)              v[i,j] += vec[j]
  add_row(vec)              v[i,j] += vec[i]
  add_mat(mat, beta)        v[i,j] += beta * mat[i,j]
  gelu_tanh                 tanh-approximated GELU
  silu                      x * sigmoid(x)
  swiglu_pair               out[i,j] = silu(v[i,2j]) * v[i,2j+1]
  mul_dgelu_tanh(mat)       v[i,j] *= GELU_tanh'(mat[i,j])
  row_sum/row_sumsq/row_mean(out, col)   fp32 per-row reduction written to
                            out[i, col] of an [M x ncols] fp32 array
  dropout(p, seed, offset)  inverted dropout with a counter-based mask (element
                            (i, j) kept with probability 1 - p, kept values
                            scaled by 1 / (1 - p))
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: Tuple[int, ...]
    dist: str            # "normal", "abs_normal", "one_plus_normal", "row_shift_normal"
    var: float           # variance of the underlying normal
    dtype: str           # "bf16" | "f32"


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    index: int
    name: str
    M: int
    N: int               # GEMM width (columns of logical B)
    K: int
    b_layout: str        # "KN": B stored row-major [K x N]; "NK": stored [N x K] (used as its transpose)
    ab_dtype: str        # storage dtype of A and B
    d_dtype: str         # storage dtype of D
    a_name: str
    b_name: str
    tensors: Tuple[TensorSpec, ...]          # drawn in this order
    program: Tuple[Tuple[str, Dict], ...]    # ordered epilogue
    outputs: Tuple[Tuple[str, Tuple[int, ...]], ...]  # fp32 reduction outputs (name, shape)

    @property
    def out_width(self) -> int:
        return self.N // 2 if any(op == "swiglu_pair" for op, _ in self.program) else self.N

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _normal(name, shape, var, dtype):
    return TensorSpec(name, tuple(shape), "normal", var, dtype)


def _build(index: int, M: int, N: int, K: int) -> WorkloadSpec:
    """Build workload ``index`` (1..6) at the given GEMM shape."""
    if index == 1:
        dt = "f32"
        tensors = (
            _normal("X", (M, K), 1.0, dt),
            TensorSpec("gamma", (K,), "one_plus_normal", 0.01, dt),
            _normal("W", (K, N), 1.0 / K, dt),
            _normal("bias", (N,), 0.02, dt),
            _normal("R", (M, N), 1.0, dt),
        )
        program = (
            ("rms_rowscale", {"gamma": "gamma", "eps": 1e-6}),
            ("add_col", {"vec": "bias"}),
            ("gelu_tanh", {}),
            ("add_mat", {"mat": "R", "beta": 1.0}),
        )
        return WorkloadSpec(1, "tiny_fwd_f32", M, N, K, "KN", dt, dt, "X", "W",
                            tensors, program, ())
    if index == 2:
        dt = "bf16"
        tensors = (
            _normal("X", (M, K), 1.0, dt),
            _normal("W", (K, N), 1.0 / K, dt),
            TensorSpec("gamma", (K,), "one_plus_normal", 0.01, dt),
            _normal("bias", (N,), 0.02, dt),
        )
        program = (
            ("rms_rowscale", {"gamma": "gamma", "eps": 1e-6}),
            ("add_col", {"vec": "bias"}),
            ("gelu_tanh", {}),
        )
        return WorkloadSpec(2, "gpt2s_mlp_up", M, N, K, "KN", dt, dt, "X", "W",
                            tensors, program, ())
    if index == 3:
        dt = "bf16"
        tensors = (
            TensorSpec("H", (M, K), "abs_normal", 1.0, dt),
            _normal("W", (K, N), 1.0 / K, dt),
            _normal("bias", (N,), 0.02, dt),
            _normal("R", (M, N), 1.0, dt),
        )
        program = (
            ("add_col", {"vec": "bias"}),
            ("add_mat", {"mat": "R", "beta": 1.0}),
            ("row_sum", {"out": "stats", "col": 0}),
            ("row_sumsq", {"out": "stats", "col": 1}),
        )
        return WorkloadSpec(3, "bertl_mlp_down", M, N, K, "KN", dt, dt, "H", "W",
                            tensors, program, (("stats", (M, 2)),))
    if index == 4:
        dt = "bf16"
        if N % 2:
            raise ValueError("the gate/up workload needs an even GEMM width")
        tensors = (
            _normal("X", (M, K), 1.0, dt),
            _normal("W", (K, N), 1.0 / K, dt),   # column 2j = gate_j, 2j+1 = up_j
            TensorSpec("gamma", (K,), "one_plus_normal", 0.01, dt),
        )
        program = (
            ("rms_rowscale", {"gamma": "gamma", "eps": 1e-6}),
            ("swiglu_pair", {}),
        )
        return WorkloadSpec(4, "llama7b_swiglu_gate_up", M, N, K, "KN", dt, dt, "X", "W",
                            tensors, program, ())
    if index == 5:
        dt = "bf16"
        # dH = dY @ W2^T: W2 is stored [N x K] = [4096 x 1024] and used transposed.
        tensors = (
            _normal("dY", (M, K), 1.0, dt),
            _normal("W2", (N, K), 1.0 / N, dt),   # 1/4096 at the full shape
            _normal("P", (M, N), 1.0, dt),
        )
        program = (
            ("mul_dgelu_tanh", {"mat": "P"}),
            ("row_sum", {"out": "rowsum", "col": 0}),
        )
        return WorkloadSpec(5, "gpt2m_mlp_bwd_act", M, N, K, "NK", dt, dt, "dY", "W2",
                            tensors, program, (("rowsum", (M, 1)),))
    if index == 6:
        dt = "bf16"
        # the GPT-2-small MLP up-projection with the LayerNorm GPT-2 actually
        # uses in front of it; rows of X carry a mean of the order of their spread
        tensors = (
            TensorSpec("X", (M, K), "row_shift_normal", 1.0, dt),
            _normal("W", (K, N), 1.0 / K, dt),
            TensorSpec("gamma", (K,), "one_plus_normal", 0.01, dt),
            _normal("beta", (K,), 0.01, dt),
            _normal("bias", (N,), 0.02, dt),
        )
        program = (
            ("ln_rowscale", {"gamma": "gamma", "beta": "beta", "eps": 1e-5}),
            ("add_col", {"vec": "bias"}),
            ("gelu_tanh", {}),
        )
        return WorkloadSpec(6, "gpt2s_mlp_up_layernorm", M, N, K, "KN", dt, dt, "X", "W",
                            tensors, program, ())
    raise ValueError(f"unknown workload index {index}")


# Full-size shapes of the workloads (M, GEMM N, K).
FULL_SHAPES = {
    1: (256, 256, 256),
    2: (8192, 3072, 768),
    3: (8192, 1024, 4096),
    4: (4096, 22016, 4096),
    5: (8192, 4096, 1024),
    6: (8192, 3072, 768),
}

CONFIGS: Dict[int, WorkloadSpec] = {i: _build(i, *FULL_SHAPES[i]) for i in FULL_SHAPES}


def get_config(index: int) -> WorkloadSpec:
    return CONFIGS[index]


def scaled_config(index: int, M: int, N: int, K: int) -> WorkloadSpec:
    """Same workload recipe (distributions, program) at another shape."""
    return _build(index, M, N, K)
