"""Run the oracle on a seeded workload (test infrastructure only).

Rows of the output depend only on the same rows of A and of the row-shaped
side operands, so a subset of rows can be computed exactly on its own; that is
how full-size workloads are checked on sampled rows.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from workloads.gen import to_f64

from .coda_oracle import COLUMN_REDUCTION_OPS, forward


def _row_shaped(spec, name: str) -> bool:
    t = next(t for t in spec.tensors if t.name == name)
    return len(t.shape) == 2 and t.shape[0] == spec.M and name != spec.b_name


def resolve_program(spec, inputs: Dict[str, np.ndarray], rows: Optional[np.ndarray] = None):
    """Turn the symbolic program into (name, args) with fp64 array arguments."""
    dtypes = {t.name: t.dtype for t in spec.tensors}

    def arr(name):
        a = to_f64(inputs[name], dtypes[name])
        if rows is not None and _row_shaped(spec, name):
            a = a[rows]
        return a

    ops = []
    for name, args in spec.program:
        r = dict(args)
        for key in ("gamma", "beta", "vec", "mat"):
            # tensor arguments are names; add_mat's beta is a number
            if isinstance(r.get(key), str):
                r[key] = arr(r[key])
        ops.append((name, r))
    return ops


def run_workload(spec, inputs: Dict[str, np.ndarray], rows: Optional[Sequence[int]] = None):
    """fp64 oracle outputs of ``spec`` on ``inputs`` (optionally only ``rows``).

    Returns (D, outs) where D is fp64 [rows x out_width] and outs maps each
    reduction output name to an fp64 [rows x ncols] array.
    """
    dtypes = {t.name: t.dtype for t in spec.tensors}
    rows_arr = None if rows is None else np.asarray(rows, dtype=np.int64)
    A = to_f64(inputs[spec.a_name], dtypes[spec.a_name])
    if rows_arr is not None:
        A = A[rows_arr]
    B = to_f64(inputs[spec.b_name], dtypes[spec.b_name])
    ops = resolve_program(spec, inputs, rows_arr)
    D, reds = forward(A, B, ops, spec.b_layout, row_ids=rows_arr)
    # outputs of column reductions are indexed by column (over the rows given);
    # all others by row
    col_outs = {args["out"] for name, args in spec.program if name in COLUMN_REDUCTION_OPS}
    outs = {}
    for oname, shape in spec.outputs:
        outs[oname] = np.full((shape[0] if oname in col_outs else A.shape[0], shape[1]), np.nan)
    for name, args, val in reds:
        outs[args["out"]][:, args["col"]] = val
    return D, outs
