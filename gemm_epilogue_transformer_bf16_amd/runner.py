"""Marshal a workload (device tensors + ordered op list) into a coda_epi_desc.

Argument marshalling only: buffers are torch device tensors, the descriptor
is filled with their pointers, and the calls go to libcoda.so.  Every step of
the computation runs in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import coda as C

OPCODES = {
    "scale": C.CODA_OP_SCALE,
    "scale_row": C.CODA_OP_SCALE_ROW,
    "scale_col": C.CODA_OP_SCALE_COL,
    "rms_rowscale": C.CODA_OP_RMS_ROWSCALE,
    "add_col": C.CODA_OP_ADD_COL,
    "add_row": C.CODA_OP_ADD_ROW,
    "add_mat": C.CODA_OP_ADD_MAT,
    "gelu_tanh": C.CODA_OP_GELU_TANH,
    "silu": C.CODA_OP_SILU,
    "swiglu_pair": C.CODA_OP_SWIGLU_PAIR,
    "mul_dgelu_tanh": C.CODA_OP_MUL_DGELU_TANH,
    "row_sum": C.CODA_OP_ROW_SUM,
    "row_sumsq": C.CODA_OP_ROW_SUMSQ,
    "row_mean": C.CODA_OP_ROW_MEAN,
    "ln_rowscale": C.CODA_OP_LN_ROWSCALE,
    "col_sum": C.CODA_OP_COL_SUM,
    "col_sumsq": C.CODA_OP_COL_SUMSQ,
    "row_dot": C.CODA_OP_ROW_DOT,
    "rms_bwd": C.CODA_OP_RMS_BWD,
    "rms_dgamma": C.CODA_OP_RMS_DGAMMA,
    "dropout": C.CODA_OP_DROPOUT,
}

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
CODA_DT = {torch.bfloat16: C.CODA_BF16, torch.float32: C.CODA_F32}


def storage_to_tensor(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored numpy array (bf16 as uint16 bits, or float32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to(device)


def tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def current_stream_ptr() -> int:
    return int(torch.cuda.current_stream().cuda_stream)


class Call:
    """Descriptor plus the device tensors it points at, for one (A, B, ops) call.

    ``ops`` is a list of (name, args) where array arguments are device tensors:
    ``gamma``/``vec``/``mat`` inputs, ``out`` a 2-D fp32 tensor with ``col``
    selecting the column a reduction writes (its rows index the output's rows
    for row_* reductions and the output's columns for col_* reductions).  Scalars: ``alpha``, ``beta``, ``eps``.
    ``rms_rowscale`` / ``ln_rowscale`` may take given row statistics: ``row_ss``
    a 2-D fp32 tensor with the sums of squares in column ``row_ss_col`` and
    (LayerNorm) the sums in column ``row_s_col`` (with ``fold_gain``).
    ``ln_rowscale`` takes ``gamma``, ``eps`` and an optional shift ``beta``
    tensor: the call computes u = gamma^T B and c = beta^T B once with
    coda_ln_fold and passes LN_ROWSCALE(gamma, u) followed by ADD_COL(c).
    With ``fold_gain``, an ``rms_rowscale`` gain is folded into a copy of B once
    (coda_fold_gain) and the op is passed with gamma NULL.
    """

    def __init__(self, A: torch.Tensor, B: torch.Tensor, ops: Sequence[Tuple[str, Dict]], b_layout: str,
                 D: Optional[torch.Tensor] = None, d_dtype: Optional[torch.dtype] = None, tile: int = 0,
                 M: Optional[int] = None, N: Optional[int] = None, K: Optional[int] = None,
                 lda: Optional[int] = None, ldb: Optional[int] = None, flags: int = 0,
                 fold_gain: bool = False, a_layout: str = "MK"):
        self.A, self.B = A, B
        # a_layout "KM": A is given as its [K x M] storage (the X of X^T dY)
        akm = a_layout == "KM"
        self.M = (A.shape[1] if akm else A.shape[0]) if M is None else M
        self.K = (A.shape[0] if akm else A.shape[1]) if K is None else K
        if N is None:
            N = B.shape[1] if b_layout == "KN" else B.shape[0]
        self.N = N
        self.b_layout = b_layout
        self._keep: List[torch.Tensor] = []
        if lda is None:
            inner_a = self.M if akm else self.K
            lda = A.stride(0) if A.dim() == 2 and A.shape[0] > 0 and A.shape[1] > 0 else max((inner_a + 7) // 8 * 8, 8)
        if ldb is None:
            inner = self.N if b_layout == "KN" else self.K
            ldb = B.stride(0) if B.dim() == 2 and B.numel() > 0 else max((inner + 7) // 8 * 8, 8)
        if fold_gain and ops and ops[0][0] == "ln_rowscale":
            B, ldb = self._fold_layernorm(B, ldb, list(ops))
            self.B = B
        else:
            self.ops = self._expand_layernorm(list(ops), B, ldb)
        if fold_gain:
            B, ldb = self._fold_gain(B, ldb)
            self.B = B
        width = self.N // 2 if any(n == "swiglu_pair" for n, _ in self.ops) else self.N
        self.out_width = width
        d_dtype = d_dtype or A.dtype
        if D is None:
            # rows padded to a multiple of 8 elements (16-byte aligned row starts)
            ldd = max((width + 7) // 8 * 8, 8)
            D = torch.empty((self.M, ldd), dtype=d_dtype, device=A.device)[:, :width]
        self.D = D
        d = C.coda_epi_desc()
        d.ab_dtype = CODA_DT[A.dtype]
        d.d_dtype = CODA_DT[D.dtype]
        d.b_layout = C.CODA_B_KN if b_layout == "KN" else C.CODA_B_NK
        d.lda = lda
        d.a_layout = C.CODA_A_KM if akm else C.CODA_A_MK
        d.ldb = ldb
        d.ldd = D.stride(0) if D.dim() == 2 and D.shape[0] > 0 else max(width, 8)
        d.D = D.data_ptr() if D.numel() else None
        if len(self.ops) > C.CODA_MAX_OPS:
            raise ValueError(f"at most {C.CODA_MAX_OPS} ops")
        d.n_ops = len(self.ops)
        self._validate_operands(width_in=self.N)
        for i, (name, args) in enumerate(self.ops):
            o = d.ops[i]
            o.kind = OPCODES[name]
            for key in ("gamma", "vec", "mat"):
                if args.get(key) is not None:
                    t = args[key]
                    self._keep.append(t)
                    o.in_ = t.data_ptr()
                    o.in_dtype = CODA_DT[t.dtype]
                    if key == "mat":
                        o.ld = t.stride(0)
            if name == "scale":
                o.scalar = float(args["alpha"])
            elif name == "add_mat":
                o.scalar = float(args.get("beta", 1.0))
            elif name in ("rms_rowscale", "ln_rowscale"):
                o.scalar = float(args["eps"])
            elif name == "dropout":
                o.scalar = float(args["p"])
                o.seed = int(args.get("seed", 0)) & ((1 << 64) - 1)
                o.offset = int(args.get("offset", 0)) & ((1 << 64) - 1)
            if name == "ln_rowscale":
                o.in2 = args["u"].data_ptr()
            if name in ("rms_rowscale", "ln_rowscale") and args.get("row_ss") is not None:
                # given row statistics: columns of a 2-D fp32 tensor, the sums of
                # squares in `row_ss_col` and (LayerNorm) the sums in `row_s_col`
                t = args["row_ss"]
                self._keep.append(t)
                o.row_sumsq = t.data_ptr() + 4 * int(args.get("row_ss_col", 0))
                if name == "ln_rowscale":
                    o.row_sum = t.data_ptr() + 4 * int(args["row_s_col"])
                o.row_ld = t.stride(0)
            if name == "rms_bwd":
                # in = x [M x width], in2 = gamma [width] (x's dtype); the row
                # statistics are columns of a 2-D fp32 tensor: the sums of squares
                # of x in `sumsq_col`, t in `t_col`
                x, g, st = args["x"], args["gamma"], args["stats"]
                if g.dtype != x.dtype:
                    raise ValueError("rms_bwd: gamma must have x's dtype")
                self._keep += [x, g, st]
                o.in_ = x.data_ptr()
                o.in_dtype = CODA_DT[x.dtype]
                o.ld = x.stride(0)
                o.in2 = g.data_ptr()
                o.scalar = float(args["eps"])
                o.row_sumsq = st.data_ptr() + 4 * int(args.get("sumsq_col", 0))
                o.row_sum = st.data_ptr() + 4 * int(args.get("t_col", 1))
                o.row_ld = st.stride(0)
            if name == "rms_dgamma":
                # in = x [M x width]; the sums of squares of x in column
                # `sumsq_col` of a 2-D fp32 tensor
                x, st = args["x"], args["stats"]
                self._keep += [x, st]
                o.in_ = x.data_ptr()
                o.in_dtype = CODA_DT[x.dtype]
                o.ld = x.stride(0)
                o.scalar = float(args["eps"])
                o.row_sumsq = st.data_ptr() + 4 * int(args.get("sumsq_col", 0))
                o.row_ld = st.stride(0)
            if name in ("row_sum", "row_sumsq", "row_mean", "col_sum", "col_sumsq", "row_dot", "rms_dgamma"):
                out = args["out"]
                self._keep.append(out)
                col = int(args.get("col", 0))
                o.out = out.data_ptr() + 4 * col
                o.out_stride = out.stride(0)
        d.tile = tile
        d.flags = flags
        self.desc = d
        self.ws = {}
        for unfused in (0, 1):
            nbytes = C.coda_workspace_size(self.M, self.N, self.K, d, unfused)
            self.ws[unfused] = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=A.device) if nbytes else None

    def _validate_operands(self, width_in: int):
        """Shapes, dtypes and strides of every tensor an op reads or writes.

        The C ABI sees raw pointers only and cannot check extents, so a tensor
        that is too small, of the wrong dtype or with a strided inner dimension
        is rejected here, before a descriptor points at it.
        """
        M, K = self.M, self.K
        width = width_in

        def check(t, what, *, rows=None, cols=None, length=None, dtype=None):
            if not isinstance(t, torch.Tensor):
                raise ValueError(f"{what}: expected a tensor, got {type(t).__name__}")
            if dtype is not None and t.dtype != dtype:
                raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
            if t.dtype not in CODA_DT:
                raise ValueError(f"{what}: dtype {t.dtype} is neither bfloat16 nor float32")
            if length is not None:
                if t.dim() != 1 or t.shape[0] < length or (t.numel() > 1 and t.stride(0) != 1):
                    raise ValueError(f"{what}: expected a contiguous vector of at least {length} elements, "
                                     f"got shape {tuple(t.shape)}")
                return
            if t.dim() != 2:
                raise ValueError(f"{what}: expected a 2-D tensor, got shape {tuple(t.shape)}")
            if t.shape[1] > 1 and t.stride(1) != 1:
                raise ValueError(f"{what}: the inner dimension must be contiguous (stride {t.stride(1)})")
            if rows is not None and t.shape[0] < rows:
                raise ValueError(f"{what}: {t.shape[0]} rows, at least {rows} needed")
            if cols is not None and t.shape[1] < cols:
                raise ValueError(f"{what}: {t.shape[1]} columns, at least {cols} needed")

        def check_col(t, col, what):
            if not 0 <= int(col) < t.shape[1]:
                raise ValueError(f"{what}: column {col} outside 0..{t.shape[1] - 1}")

        for name, args in self.ops:
            if name not in OPCODES:
                raise ValueError(f"unknown op {name!r}")
            if name in ("rms_rowscale", "ln_rowscale"):
                if args.get("gamma") is not None:
                    check(args["gamma"], f"{name} gamma", length=K, dtype=self.A.dtype)
                if args.get("u") is not None:
                    check(args["u"], f"{name} u", length=self.N, dtype=torch.float32)
                if args.get("row_ss") is not None:
                    st = args["row_ss"]
                    check(st, f"{name} row statistics", rows=M, dtype=torch.float32)
                    check_col(st, args.get("row_ss_col", 0), f"{name} row_ss_col")
                    if name == "ln_rowscale":
                        check_col(st, args["row_s_col"], f"{name} row_s_col")
            elif name in ("scale_row", "add_row"):
                check(args["vec"], f"{name} vec", length=M)
            elif name in ("scale_col", "add_col"):
                check(args["vec"], f"{name} vec", length=width)
            elif name in ("add_mat", "mul_dgelu_tanh", "row_dot"):
                check(args["mat"], f"{name} mat", rows=M, cols=width)
            elif name in ("rms_bwd", "rms_dgamma"):
                check(args["x"], f"{name} x", rows=M, cols=width)
                st = args["stats"]
                check(st, f"{name} stats", rows=M, dtype=torch.float32)
                check_col(st, args.get("sumsq_col", 0), f"{name} sumsq_col")
                if name == "rms_bwd":
                    check(args["gamma"], f"{name} gamma", length=width)
                    check_col(st, args.get("t_col", 1), f"{name} t_col")
            elif name == "dropout":
                p = float(args["p"])
                if not 0.0 <= p < 1.0:
                    raise ValueError(f"dropout probability {p} outside [0, 1)")
            if name in ("row_sum", "row_sumsq", "row_mean", "row_dot", "col_sum", "col_sumsq", "rms_dgamma"):
                out = args["out"]
                col_red = name in ("col_sum", "col_sumsq", "rms_dgamma")
                check(out, f"{name} out", rows=width if col_red else M, dtype=torch.float32)
                check_col(out, args.get("col", 0), f"{name} out col")
            if name == "swiglu_pair":
                width //= 2

    def _expand_layernorm(self, ops, B: torch.Tensor, ldb: int):
        """ln_rowscale(gamma, beta, eps) -> LN_ROWSCALE(gamma, u) [+ ADD_COL(c)],
        with u, c from coda_ln_fold on the current stream."""
        if not ops or ops[0][0] != "ln_rowscale" or "u" in ops[0][1]:
            return ops
        args = dict(ops[0][1])
        gamma, beta = args["gamma"], args.pop("beta", None)
        n = max(self.N, 1)
        u = torch.empty(n, dtype=torch.float32, device=B.device)
        c = torch.empty(n, dtype=torch.float32, device=B.device) if beta is not None else None
        self._keep += [t for t in (gamma, beta, u, c) if t is not None]
        st = C.coda_ln_fold(B.data_ptr() if B.numel() else None, self.K, self.N, ldb,
                            C.CODA_B_KN if self.b_layout == "KN" else C.CODA_B_NK, CODA_DT[B.dtype],
                            gamma.data_ptr() if gamma.numel() else None,
                            None if beta is None else beta.data_ptr(), u.data_ptr(),
                            None if c is None else c.data_ptr(), current_stream_ptr())
        C.check(st, "coda_ln_fold")
        args["u"] = u
        out = [("ln_rowscale", args)]
        if c is not None:
            out.append(("add_col", {"vec": c}))
        return out + list(ops[1:])

    def _fold_layernorm(self, B: torch.Tensor, ldb: int, ops):
        """ln_rowscale(gamma, beta) on B -> LN_ROWSCALE(NULL, u') on B' = diag(gamma) B
        with u' the column sums of B' and, with beta, ADD_COL(beta^T B)."""
        args = dict(ops[0][1])
        gamma = args["gamma"]
        layout = C.CODA_B_KN if self.b_layout == "KN" else C.CODA_B_NK
        Bf = torch.empty_like(B)
        ldo = Bf.stride(0) if Bf.dim() == 2 and Bf.numel() else ldb
        self._keep += [gamma, B]
        st = C.coda_fold_gain(B.data_ptr() if B.numel() else None, self.K, self.N, ldb, layout, CODA_DT[B.dtype],
                              gamma.data_ptr() if gamma.numel() else None, Bf.data_ptr() if Bf.numel() else None,
                              ldo, current_stream_ptr())
        C.check(st, "coda_fold_gain")
        ones = torch.ones(max(self.K, 1), dtype=B.dtype, device=B.device)
        u = torch.empty(max(self.N, 1), dtype=torch.float32, device=B.device)
        self._keep += [ones, u]
        st = C.coda_ln_fold(Bf.data_ptr() if Bf.numel() else None, self.K, self.N, ldo, layout, CODA_DT[B.dtype],
                            ones.data_ptr(), None, u.data_ptr(), None, current_stream_ptr())
        C.check(st, "coda_ln_fold (column sums of the folded weights)")
        out = [("ln_rowscale", {"gamma": None, "eps": args["eps"], "u": u,
                                **{k: args[k] for k in ("row_ss", "row_ss_col", "row_s_col") if k in args}})]
        beta = args.get("beta")
        if beta is not None:
            c = torch.empty(max(self.N, 1), dtype=torch.float32, device=B.device)
            uu = torch.empty_like(c)
            self._keep += [beta, c, uu]
            st = C.coda_ln_fold(B.data_ptr() if B.numel() else None, self.K, self.N, ldb, layout, CODA_DT[B.dtype],
                                gamma.data_ptr() if gamma.numel() else None, beta.data_ptr(), uu.data_ptr(),
                                c.data_ptr(), current_stream_ptr())
            C.check(st, "coda_ln_fold")
            out.append(("add_col", {"vec": c}))
        self.ops = out + list(ops[1:])
        return Bf, ldo

    def _fold_gain(self, B: torch.Tensor, ldb: int):
        """rms_rowscale(gamma) on B -> rms_rowscale(NULL) on diag(gamma) B."""
        if not self.ops or self.ops[0][0] != "rms_rowscale" or self.ops[0][1].get("gamma") is None:
            return B, ldb
        args = dict(self.ops[0][1])
        gamma = args["gamma"]
        Bf = torch.empty_like(B)
        self._keep += [gamma, B]
        st = C.coda_fold_gain(B.data_ptr() if B.numel() else None, self.K, self.N, ldb,
                              C.CODA_B_KN if self.b_layout == "KN" else C.CODA_B_NK, CODA_DT[B.dtype],
                              gamma.data_ptr() if gamma.numel() else None, Bf.data_ptr() if Bf.numel() else None,
                              Bf.stride(0) if Bf.dim() == 2 and Bf.numel() else ldb, current_stream_ptr())
        C.check(st, "coda_fold_gain")
        args["gamma"] = None
        self.ops = [("rms_rowscale", args)] + self.ops[1:]
        return Bf, (Bf.stride(0) if Bf.dim() == 2 and Bf.numel() else ldb)

    def _set_ws(self, unfused: int):
        w = self.ws[unfused]
        self.desc.workspace = None if w is None else w.data_ptr()
        self.desc.workspace_bytes = 0 if w is None else w.numel()

    def _ptrs(self):
        a = self.A.data_ptr() if self.A.numel() else None
        b = self.B.data_ptr() if self.B.numel() else None
        return a, b

    def fused(self, stream: Optional[int] = None) -> int:
        self._set_ws(0)
        a, b = self._ptrs()
        return C.coda_gemm_epi(a, b, self.M, self.N, self.K, self.desc,
                               current_stream_ptr() if stream is None else stream)

    def unfused(self, stream: Optional[int] = None) -> int:
        self._set_ws(1)
        a, b = self._ptrs()
        return C.coda_gemm_unfused(a, b, self.M, self.N, self.K, self.desc,
                                   current_stream_ptr() if stream is None else stream)


class WorkloadCall(Call):
    """A ``workloads`` spec with its seeded inputs uploaded to the device."""

    def __init__(self, spec, inputs: Dict[str, np.ndarray], device="cuda", tile: int = 0, flags: int = 0,
                 fold_gain: bool = False):
        dtypes = {t.name: t.dtype for t in spec.tensors}
        self.spec = spec
        self.tensors = {name: storage_to_tensor(arr, dtypes[name], device) for name, arr in inputs.items()}
        self.outputs = {name: torch.zeros(shape, dtype=torch.float32, device=device) for name, shape in spec.outputs}
        ops = []
        for name, args in spec.program:
            a = dict(args)
            for key in ("gamma", "beta", "vec", "mat"):
                if isinstance(a.get(key), str):   # tensor names (add_mat's beta is a number)
                    a[key] = self.tensors[a[key]]
            if "out" in a:
                a["out"] = self.outputs[a["out"]]
            ops.append((name, a))
        super().__init__(self.tensors[spec.a_name], self.tensors[spec.b_name], ops, spec.b_layout,
                         d_dtype=TORCH_DT[spec.d_dtype], tile=tile, M=spec.M, N=spec.N, K=spec.K, flags=flags,
                         fold_gain=fold_gain)
