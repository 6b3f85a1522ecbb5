"""A text front end for epilogue programs: statements on the running value,
lowered to the ordered op list the C ABI's descriptor takes.

The form follows the epilogue-as-statements style of the d9bl.com page
(section 3.2): each statement assigns a new value of ``output`` computed from
the previous one (``input`` names the GEMM result), and a reduction writes a
column of a named output array.  Argument marshalling only: lowering resolves
names to the tensors the caller binds and picks the primitive from the
operand's shape; nothing is computed here.

Grammar (whitespace and ``//`` comments ignored; the braces are optional)::

    program := ["EPILOGUE"] "{" stmt* "}" | stmt*
    stmt    := "output" "=" value ";"  |  NAME "[" INT "]" "=" reduce ";"
    reduce  := REDUCE "(" "output" ")"
             | "rowdot" "(" "output" "," NAME ")"
             | "rmsdgamma" "(" "output" "," NAME "," NAME "," NUMBER ")"
    value   := FN "(" ("input" | "output") ")"
             | "rmsnorm_backward" "(" "output" "," NAME "," NAME "," NAME "," NUMBER ")"
             | "rmsnorm" "(" "input" "," NAME "," NUMBER ")"          (first statement only)
             | "layernorm" "(" "input" "," NAME ["," NAME] "," NUMBER ")"   (first statement only)
             | "output" ("+" | "*") term  |  term ("+" | "*") "output"
             | "output" "*" "dgelu" "(" NAME ")"
             | "dropout" "(" "output" "," NUMBER ["," INT] ")"
    term    := NUMBER | NAME | NUMBER "*" NAME | "row" "(" NAME ")" | "col" "(" NAME ")"
    FN      := "gelu" | "silu" | "swiglu"
    REDUCE  := "rowsum" | "rowsumsq" | "rowmean" | "colsum" | "colsumsq"

``input`` (the GEMM result) may appear only in the first statement: later
statements see the running value ``output``.  ``output + NAME`` adds a matrix
(residual), a column vector [width] (bias) or a row vector [M];
``output * NAME`` scales by a column or row vector; ``output + b * NAME`` adds
b times a matrix.  When M equals the running width a vector's length does not
say which it is: write ``col(NAME)`` or ``row(NAME)`` (an unmarked vector is
then an error).  ``dropout(output, p[, seed])`` zeroes each element with
probability p and scales the kept ones by 1 / (1 - p); the mask comes from the
counter-based Philox-4x64-10 generator keyed by the seed (default 0, or the
``seed`` argument of ``lower``) and counted by the element's row and column, so
it is reproducible and needs no stored state.  The RMS norm's backward:
``rowdot(output, P)`` is the row sum of output times the matrix P;
``rmsnorm_backward(output, x, gamma, stats, eps)`` turns dL/dY into dL/dx given
``stats`` [M x 2] (column 0 the sums of squares of x, column 1 t = rowdot of
the upstream gradient with P); ``rmsdgamma(output, x, stats, eps)`` is the
gain gradient, one value per column.
"""
from __future__ import annotations

import re
from typing import Dict, List, Tuple

_TOKEN = re.compile(r"\s*(?:(//[^\n]*)|(\d+\.\d*(?:[eE][-+]?\d+)?|\d*\.\d+(?:[eE][-+]?\d+)?|\d+(?:[eE][-+]?\d+)?)"
                    r"|([A-Za-z_][A-Za-z_0-9]*)|(.))")

_FUNCS = {"gelu": "gelu_tanh", "silu": "silu", "swiglu": "swiglu_pair"}
_REDUCE = {"rowsum": "row_sum", "rowsumsq": "row_sumsq", "rowmean": "row_mean",
           "colsum": "col_sum", "colsumsq": "col_sumsq"}
# reductions with operands: name -> (op, number of arguments after output)
_REDUCE_ARGS = {"rowdot": ("row_dot", 1), "rmsdgamma": ("rms_dgamma", 3)}


class FrontendError(ValueError):
    pass


def _tokens(text: str) -> List[str]:
    out = []
    pos = 0
    while pos < len(text):
        m = _TOKEN.match(text, pos)
        if not m or m.end() == pos:
            break
        pos = m.end()
        comment, num, name, sym = m.groups()
        if comment:
            continue
        tok = num or name or sym
        if tok is not None and tok.strip():
            out.append(tok)
    return out


class _Parser:
    def __init__(self, text: str):
        self.t = _tokens(text)
        self.i = 0

    def peek(self, k: int = 0):
        return self.t[self.i + k] if self.i + k < len(self.t) else None

    def take(self, want=None):
        tok = self.peek()
        if tok is None or (want is not None and tok != want):
            raise FrontendError(f"expected {want!r}, found {tok!r} (token {self.i})")
        self.i += 1
        return tok

    @staticmethod
    def is_number(tok) -> bool:
        return tok is not None and re.fullmatch(r"\d+\.?\d*(?:[eE][-+]?\d+)?|\d*\.\d+(?:[eE][-+]?\d+)?", tok) is not None

    def program(self):
        if self.peek() == "EPILOGUE":
            self.take()
        braced = self.peek() == "{"
        if braced:
            self.take("{")
        stmts = []
        while self.peek() is not None and self.peek() != "}":
            stmts.append(self.stmt(first=not stmts))
        if braced:
            self.take("}")
        if self.peek() is not None:
            raise FrontendError(f"unexpected {self.peek()!r} after the program")
        return stmts

    def stmt(self, first: bool):
        target = self.take()
        if target == "output":
            self.take("=")
            st = self.value(first)
        else:
            self.take("[")
            col = self.take()
            if not col.isdigit():
                raise FrontendError(f"column index must be an integer, found {col!r}")
            self.take("]")
            self.take("=")
            fn = self.take()
            if fn not in _REDUCE and fn not in _REDUCE_ARGS:
                raise FrontendError(f"{target}[{col}] must be assigned a reduction "
                                    f"({', '.join(list(_REDUCE) + list(_REDUCE_ARGS))})")
            self.take("(")
            self.take("output")
            args = []
            while self.peek() == ",":
                self.take(",")
                args.append(self.take())
            self.take(")")
            if fn in _REDUCE:
                if args:
                    raise FrontendError(f"{fn} takes only the running value")
                st = ("reduce", _REDUCE[fn], target, int(col))
            else:
                op, nargs = _REDUCE_ARGS[fn]
                if len(args) != nargs:
                    raise FrontendError(f"{fn} takes output and {nargs} more argument(s)")
                st = ("reduce", op, target, int(col), tuple(args))
        self.take(";")
        return st

    def term(self):
        tok = self.take()
        if tok in ("row", "col") and self.peek() == "(":
            self.take("(")
            name = self.take()
            self.take(")")
            return ("vec", tok, name)
        if self.is_number(tok):
            if self.peek() == "*" and self.peek(1) not in (None, "output"):
                self.take("*")
                return ("scaled", float(tok), self.take())
            return ("number", float(tok))
        return ("name", tok)

    def value(self, first: bool):
        tok = self.peek()
        if tok == "dropout":
            self.take()
            self.take("(")
            self.take("output")
            self.take(",")
            p = self.take()
            if not self.is_number(p):
                raise FrontendError(f"dropout probability must be a number, found {p!r}")
            seed = None
            if self.peek() == ",":
                self.take(",")
                seed = self.take()
                if not seed.isdigit():
                    raise FrontendError(f"dropout seed must be a non-negative integer, found {seed!r}")
                seed = int(seed)
            self.take(")")
            if not 0.0 <= float(p) < 1.0:
                raise FrontendError(f"dropout probability must be in [0, 1), found {p}")
            return ("dropout", float(p), seed)
        if tok in ("rmsnorm", "layernorm"):
            if not first:
                raise FrontendError(f"{tok} normalises the GEMM's A operand and must be the first statement")
            self.take()
            self.take("(")
            self.take("input")
            self.take(",")
            gamma = self.take()
            beta = None
            if tok == "layernorm" and self.peek() == "," and not self.is_number(self.peek(1)):
                self.take(",")
                beta = self.take()
            self.take(",")
            eps = self.take()
            if not self.is_number(eps):
                raise FrontendError(f"eps must be a number, found {eps!r}")
            self.take(")")
            return ("norm", "rms_rowscale" if tok == "rmsnorm" else "ln_rowscale", gamma, beta, float(eps))
        if tok == "rmsnorm_backward":
            self.take()
            self.take("(")
            self.take("output")
            names = []
            for _ in range(3):
                self.take(",")
                names.append(self.take())
            self.take(",")
            eps = self.take()
            if not self.is_number(eps):
                raise FrontendError(f"eps must be a number, found {eps!r}")
            self.take(")")
            return ("rmsbwd", *names, float(eps))
        if tok in _FUNCS:
            self.take()
            self.take("(")
            arg = self.take()
            if arg not in ("input", "output"):
                raise FrontendError(f"{tok} applies to the running value, found {arg!r}")
            if arg == "input" and not first:
                raise FrontendError(f"'input' names the GEMM result and is valid only in the first statement; "
                                    f"use {tok}(output)")
            self.take(")")
            return ("func", _FUNCS[tok])
        if tok == "output":
            self.take()
            opsym = self.take()
            if opsym not in ("+", "*"):
                raise FrontendError(f"expected + or * after output, found {opsym!r}")
            if opsym == "*" and self.peek() == "dgelu":
                self.take()
                self.take("(")
                name = self.take()
                self.take(")")
                return ("dgelu", name)
            return ("bin", opsym, self.term())
        t = self.term()
        opsym = self.take()
        if opsym not in ("+", "*"):
            raise FrontendError(f"expected + or *, found {opsym!r}")
        self.take("output")
        return ("bin", opsym, t)


def parse(text: str):
    """The statements of ``text`` as tuples (no name resolution)."""
    return _Parser(text).program()


def lower(text: str, operands: Dict[str, object], M: int, N: int, seed: int = 0) -> List[Tuple[str, Dict]]:
    """Lower a program to the op list of ``runner.Call`` / the workloads vocabulary.

    ``operands`` maps names to bound values (tensors or arrays: anything with
    ``.shape``); M and N are the GEMM's output rows and columns, used to tell a
    row vector [M] from a column vector [N] and a matrix [M x width].  ``seed``
    keys every dropout statement that names no seed of its own.
    """
    ops: List[Tuple[str, Dict]] = []
    width = N

    def get(name):
        if name not in operands:
            raise FrontendError(f"unbound name {name!r}")
        return operands[name]

    def shape(name):
        return tuple(getattr(get(name), "shape", ()))

    for st in parse(text):
        kind = st[0]
        if kind == "norm":
            _, op, gamma, beta, eps = st
            args = {"gamma": get(gamma), "eps": eps}
            if beta is not None:
                args["beta"] = get(beta)
            ops.append((op, args))
        elif kind == "func":
            ops.append((st[1], {}))
            if st[1] == "swiglu_pair":
                width //= 2
        elif kind == "dgelu":
            ops.append(("mul_dgelu_tanh", {"mat": get(st[1])}))
        elif kind == "dropout":
            _, p, own_seed = st
            ops.append(("dropout", {"p": p, "seed": seed if own_seed is None else own_seed}))
        elif kind == "rmsbwd":
            _, x, gamma, stats, eps = st
            ops.append(("rms_bwd", {"x": get(x), "gamma": get(gamma), "stats": get(stats), "eps": eps,
                                    "sumsq_col": 0, "t_col": 1}))
        elif kind == "reduce":
            op, target, col = st[1], st[2], st[3]
            args = {"out": get(target), "col": col}
            if op == "row_dot":
                args["mat"] = get(st[4][0])
            elif op == "rms_dgamma":
                x, stats, eps = st[4]
                if not _Parser.is_number(eps):
                    raise FrontendError(f"eps must be a number, found {eps!r}")
                args.update({"x": get(x), "stats": get(stats), "eps": float(eps), "sumsq_col": 0})
            ops.append((op, args))
        else:   # ("bin", sym, term)
            _, sym, term = st
            if term[0] == "vec":
                _, which, name = term
                shp = shape(name)
                want = width if which == "col" else M
                if len(shp) != 1 or shp[0] != want:
                    raise FrontendError(f"{which}({name}) must be a vector of length {want}, found shape {shp}")
                if which == "col":
                    ops.append(("add_col" if sym == "+" else "scale_col", {"vec": get(name)}))
                else:
                    ops.append(("add_row" if sym == "+" else "scale_row", {"vec": get(name)}))
                continue
            if term[0] == "number":
                if sym == "*":
                    ops.append(("scale", {"alpha": term[1]}))
                else:
                    raise FrontendError("adding a constant is not a primitive; add a column vector instead")
            elif term[0] == "scaled":
                if sym != "+":
                    raise FrontendError("b * NAME is only valid as an addend")
                if len(shape(term[2])) != 2:
                    raise FrontendError(f"{term[2]!r} must be a matrix for output + b * {term[2]}")
                ops.append(("add_mat", {"mat": get(term[2]), "beta": term[1]}))
            else:
                name = term[1]
                shp = shape(name)
                if len(shp) == 2 and shp[0] == M:
                    if sym == "*":
                        raise FrontendError("elementwise products with a matrix are not a primitive (use dgelu)")
                    ops.append(("add_mat", {"mat": get(name), "beta": 1.0}))
                elif len(shp) == 1 and shp[0] == width == M:
                    raise FrontendError(f"{name!r} of length {shp[0]} could be a row vector [M] or a column vector "
                                        f"[width]; write row({name}) or col({name})")
                elif len(shp) == 1 and shp[0] == width:
                    ops.append(("add_col" if sym == "+" else "scale_col", {"vec": get(name)}))
                elif len(shp) == 1 and shp[0] == M:
                    ops.append(("add_row" if sym == "+" else "scale_row", {"vec": get(name)}))
                else:
                    raise FrontendError(f"{name!r} of shape {shp} is neither [M x width], [width] nor [M]")
    return ops
