"""fp64 CPU oracle of the fused GEMM + epilogue computation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and has no CPU fallback.

What it computes is the plain definition, in the order the pages state it:

  1. optional RMS normalisation of the rows of A, with the gain gamma applied
     per feature (the row-wise norm of the "augment_me" comment on the zeli.app
     page, and the Transformer operators listed in section 3.1 / Fig. 4 of the
     d9bl.com page);
  2. the GEMM  C = alpha * Y @ B  (section 3.1 of the d9bl.com page, where the
     GEMM is written C = alpha*A*B + beta*C_prev and the epilogue D = f(C));
  3. the epilogue f as an ordered list of primitives, each statement acting on
     the previous value (section 3.2 of the d9bl.com page, the EPILOGUE
     example), drawn from the four primitive families of the agentlenshq.com
     page ("How it works": scaling, reductions, pairwise transformations,
     accumulation).

Everything runs in fp64 on the exact values of the stored inputs; nothing is
rounded.  The GEMM uses numpy's matmul as a library primitive; all other steps
are written out elementwise-vectorised with no blocking or reordering.

Readings of points the pages leave open (each also listed in the design notes):
  * GELU is the tanh approximation, 0.5 v (1 + tanh(sqrt(2/pi)(v + 0.044715 v^3)))
    (Hendrycks & Gimpel 2016); its derivative is the exact derivative of that form.
  * SiLU(v) = v * sigmoid(v) (Elfwing et al. 2017); SwiGLU pairs column 2j
    (gate) with column 2j+1 (up): out_j = SiLU(v_2j) * v_2j+1 (Shazeer 2020).
  * rms(x) = sqrt(mean_k x_k^2 + eps), the mean over the K features of a row,
    eps inside the square root.
  * The RMS row scale precedes every other epilogue op (it is a property of A's
    rows and only commutes past the matmul, not past a nonlinearity).
  * LayerNorm (ln_rowscale) is the mean-centred norm: mu and the 1/K variance
    of the row's deviations, eps inside the root, gain gamma and shift beta
    per feature (beta optional, zero when absent).
  * A reduction observes the running value at its position in the list, over
    the current width (half the GEMM width after swiglu_pair).
  * The RMS norm's backward (rmsnorm_backward, the rms_bwd op) is the
    chain-rule gradient of that same forward form.
  * Dropout (the dropout step of the d9bl.com page's section 3.2 EPILOGUE
    example) zeroes an element with probability p and scales
    the kept ones by 1 / (1 - p) (inverted dropout, so the expectation is
    unchanged).  The pages name no generator; the mask here is drawn from the
    counter-based Philox-4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel
    random numbers: as easy as 1, 2, 3", SC 2011), keyed by (seed, 0) and
    counted by (column // 8, row, offset, 0) of the element in the running
    value; column j takes the 32-bit word j % 8 of the block (the low half of
    64-bit word (j % 8) // 2 for even j % 8, the high half for odd), and the
    element is kept when that word is >= floor(p * 2^32), p taken at fp32.
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715

# op names understood by the oracle (its own vocabulary; the HIP path has its own enum)
ELEMENTWISE_OPS = ("scale", "scale_row", "scale_col", "add_col", "add_row", "add_mat",
                   "gelu_tanh", "silu", "swiglu_pair", "mul_dgelu_tanh", "rms_bwd", "dropout")
# row_dot: sum over the row of the running value times a matrix operand
REDUCTION_OPS = ("row_sum", "row_sumsq", "row_mean", "row_dot")
# reductions over the rows of the output, one value per column (the bias
# gradient of a backward layer is the column sum of its output gradient)
COLUMN_REDUCTION_OPS = ("col_sum", "col_sumsq", "rms_dgamma")


# --- pairwise / elementwise transforms (agentlenshq.com, "How it works": pairwise) ---

def gelu_tanh(v: np.ndarray) -> np.ndarray:
    """tanh-approximated GELU (Hendrycks & Gimpel 2016)."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(SQRT_2_OVER_PI * (v + GELU_CUBIC * v ** 3)))


def gelu_tanh_grad(p: np.ndarray) -> np.ndarray:
    """Exact derivative of ``gelu_tanh`` at p (product rule on 0.5 p (1 + t(p)))."""
    p = np.asarray(p, dtype=np.float64)
    t = np.tanh(SQRT_2_OVER_PI * (p + GELU_CUBIC * p ** 3))
    dinner = SQRT_2_OVER_PI * (1.0 + 3.0 * GELU_CUBIC * p ** 2)
    return 0.5 * (1.0 + t) + 0.5 * p * (1.0 - t * t) * dinner


def sigmoid(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU / Swish with beta = 1: v * sigmoid(v)."""
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


def swiglu_pair(v: np.ndarray) -> np.ndarray:
    """Column-interleaved SwiGLU: out[:, j] = SiLU(v[:, 2j]) * v[:, 2j+1]."""
    if v.shape[1] % 2:
        raise ValueError("swiglu_pair needs an even width")
    gate = v[:, 0::2]
    up = v[:, 1::2]
    return silu(gate) * up


# --- dropout's generator: Philox-4x64-10 (Salmon et al., SC 2011) ---

MASK32 = np.uint64(0xFFFFFFFF)
# round multipliers and the two key increments (the golden ratio and sqrt(3) - 1
# as 64-bit fractions), as the generator's definition gives them
PHILOX_M0, PHILOX_M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157
PHILOX_W0, PHILOX_W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B
PHILOX_ROUNDS = 10


def philox4x64_scalar(counter, key, rounds: int = PHILOX_ROUNDS):
    """One Philox-4x64 block on Python integers (small cases and pins).

    Each round multiplies counter words 0 and 2 by the two multipliers into
    128-bit products (hi, lo); the new counter is (hi(M1 c2) ^ c1 ^ k0,
    lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key then advances by
    (W0, W1) modulo 2^64.
    """
    m64 = (1 << 64) - 1
    c = [int(x) & m64 for x in counter]
    k0, k1 = (int(x) & m64 for x in key)
    for _ in range(rounds):
        p0 = PHILOX_M0 * c[0]
        p1 = PHILOX_M1 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k0, p1 & m64, (p0 >> 64) ^ c[3] ^ k1, p0 & m64]
        k0 = (k0 + PHILOX_W0) & m64
        k1 = (k1 + PHILOX_W1) & m64
    return c


def _mulhilo64(a: np.ndarray, b: int):
    """128-bit products of uint64 arrays by a 64-bit constant, as (hi, lo), from 32-bit limbs."""
    a = a.astype(np.uint64)
    a0, a1 = a & MASK32, a >> np.uint64(32)
    b0, b1 = np.uint64(b & 0xFFFFFFFF), np.uint64(b >> 32)
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> np.uint64(32)) + (p01 & MASK32) + (p10 & MASK32)
    lo = (p00 & MASK32) | ((mid & MASK32) << np.uint64(32))
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64(c0, c1, c2, c3, key, rounds: int = PHILOX_ROUNDS):
    """Philox-4x64 blocks for arrays of counters (broadcast), the key a pair of ints."""
    c = [np.asarray(x, dtype=np.uint64) for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = int(key[0]) & ((1 << 64) - 1), int(key[1]) & ((1 << 64) - 1)
    with np.errstate(over="ignore"):
        for _ in range(rounds):
            hi0, lo0 = _mulhilo64(c[0], PHILOX_M0)
            hi1, lo1 = _mulhilo64(c[2], PHILOX_M1)
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
            k0 = (k0 + PHILOX_W0) & ((1 << 64) - 1)
            k1 = (k1 + PHILOX_W1) & ((1 << 64) - 1)
    return c


def dropout_words(rows: np.ndarray, width: int, seed: int, offset: int = 0) -> np.ndarray:
    """The 32-bit uniform word of every element (row i in ``rows``, column j < width)."""
    rows = np.asarray(rows, dtype=np.uint64)
    nblk = (width + 7) // 8
    blk = np.arange(nblk, dtype=np.uint64)
    words = philox4x64(blk[None, :], rows[:, None], np.uint64(offset), np.uint64(0), (seed, 0))
    # [rows, blocks, 8]: 32-bit word 2w is the low half of 64-bit word w, 2w + 1 the high half
    out = np.empty((len(rows), nblk, 8), dtype=np.uint64)
    for w in range(4):
        out[:, :, 2 * w] = words[w] & MASK32
        out[:, :, 2 * w + 1] = words[w] >> np.uint64(32)
    return out.reshape(len(rows), nblk * 8)[:, :width]


def dropout_threshold(p: float) -> int:
    """floor(p * 2^32) for p taken at fp32: an element is kept when its word is >= this."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(math.floor(p32 * 4294967296.0))


def dropout_keep(rows: np.ndarray, width: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Boolean keep-mask [len(rows) x width]."""
    return dropout_words(rows, width, seed, offset) >= np.uint64(dropout_threshold(p))


def dropout(v: np.ndarray, p: float, seed: int, offset: int = 0, rows=None) -> np.ndarray:
    """Inverted dropout of the running value: kept elements times 1 / (1 - p), the rest 0.

    ``rows`` are the global row indices of v's rows (default 0 .. len(v) - 1).
    """
    v = np.asarray(v, dtype=np.float64)
    rows = np.arange(v.shape[0]) if rows is None else np.asarray(rows)
    keep = dropout_keep(rows, v.shape[1], p, seed, offset)
    p32 = float(np.float32(p))
    return np.where(keep, v / (1.0 - p32), 0.0)


# --- row-wise norm (zeli.app comment; d9bl.com section 3.1 / Fig. 4) ---

def rms(X: np.ndarray, eps: float) -> np.ndarray:
    """Per-row root mean square over the K features, eps inside the root."""
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[1]
    if K == 0:
        raise ValueError("rms of an empty row is undefined")
    ms = np.sum(X * X, axis=1) / K
    return np.sqrt(ms + eps)


def rmsnorm(X: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Normalise-first form: Y[i,k] = X[i,k] / rms_i * gamma[k]."""
    X = np.asarray(X, dtype=np.float64)
    r = rms(X, eps)
    return (X / r[:, None]) * np.asarray(gamma, dtype=np.float64)[None, :]


def deferred_rmsnorm_gemm(X: np.ndarray, gamma: np.ndarray, B: np.ndarray, eps: float) -> np.ndarray:
    """The rewritten form: ((X * gamma) @ B) with each row divided by rms(X) afterwards.

    The zeli.app comment states that a per-row scale of a row-wise norm can be
    pulled past the following projection; this is that form, used only to check
    the oracle's normalise-first form against the identity.
    """
    X = np.asarray(X, dtype=np.float64)
    C = (X * np.asarray(gamma, dtype=np.float64)[None, :]) @ np.asarray(B, dtype=np.float64)
    return C / rms(X, eps)[:, None]


def rmsnorm_backward(X: np.ndarray, gamma: np.ndarray, eps: float, dY: np.ndarray):
    """Gradients of the RMS norm's inputs, given dY = dL/dY for Y = rmsnorm(X, gamma, eps).

    The backward half of the norm: the d9bl.com page's Fig. 4 counts gradients
    among the Transformer operators split into a GEMM and an epilogue, and the
    agentlenshq.com page ("How it works") has the primitives covering nearly
    all non-attention work of both the forward and the backward pass.  The chain
    rule through Y[i,k] = X[i,k] gamma[k] / r_i, with r_i = sqrt(mean_k X[i,k]^2
    + eps) and dr_i/dX[i,k] = X[i,k] / (K r_i), gives

        dgamma[k] = sum_i dY[i,k] X[i,k] / r_i
        dX[i,k]   = gamma[k] dY[i,k] / r_i - X[i,k] * s_i / (K r_i^3),
        s_i       = sum_j gamma[j] dY[i,j] X[i,j].

    Returns (dX, dgamma).
    """
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    K = X.shape[1]
    r = rms(X, eps)
    G = dY * g[None, :]                       # dL/d(X / r): the gain's factor
    s = np.sum(G * X, axis=1)                 # the row dot product of the second term
    dX = G / r[:, None] - X * (s / (K * r ** 3))[:, None]
    dgamma = np.sum(dY * X / r[:, None], axis=0)
    return dX, dgamma


# --- mean-centred row norm (LayerNorm; zeli.app comment, d9bl.com Fig. 4) ---

def layernorm(X: np.ndarray, gamma: np.ndarray, eps: float, beta=None) -> np.ndarray:
    """Normalise-first form: Y[i,k] = (X[i,k] - mu_i) / sqrt(var_i + eps) * gamma[k] + beta[k].

    mu_i is the mean of row i over its K features and var_i the mean of the
    squared deviations from it (the 1/K variance), eps inside the root; beta
    defaults to zero.
    """
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[1]
    if K == 0:
        raise ValueError("layernorm of an empty row is undefined")
    mu = np.sum(X, axis=1) / K
    Xc = X - mu[:, None]
    var = np.sum(Xc * Xc, axis=1) / K
    Y = Xc / np.sqrt(var + eps)[:, None] * np.asarray(gamma, dtype=np.float64)[None, :]
    if beta is not None:
        Y = Y + np.asarray(beta, dtype=np.float64)[None, :]
    return Y


def ln_fold(B: np.ndarray, gamma: np.ndarray, beta: np.ndarray):
    """The two constant rows of the deferred form: u = gamma^T B and c = beta^T B."""
    B = np.asarray(B, dtype=np.float64)
    return (np.asarray(gamma, dtype=np.float64) @ B, np.asarray(beta, dtype=np.float64) @ B)


def deferred_layernorm_gemm(X: np.ndarray, gamma: np.ndarray, beta: np.ndarray, B: np.ndarray,
                            eps: float) -> np.ndarray:
    """The rewritten form: rstd_i * ((X * gamma) @ B - mu_i * u) + c.

    Both per-row factors of the norm move past the projection: the scale
    rstd_i as for RMSNorm, and the shift mu_i as the rank-one term mu_i * u_j
    with u = gamma^T B; beta becomes c = beta^T B.  Used only to check the
    normalise-first form against the identity.
    """
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[1]
    mu = np.sum(X, axis=1) / K
    var = np.sum((X - mu[:, None]) ** 2, axis=1) / K
    u, c = ln_fold(B, gamma, beta)
    P = (X * np.asarray(gamma, dtype=np.float64)[None, :]) @ np.asarray(B, dtype=np.float64)
    return (P - mu[:, None] * u[None, :]) / np.sqrt(var + eps)[:, None] + c[None, :]


# --- the GEMM (d9bl.com section 3.1) ---

def logical_b(B_stored: np.ndarray, b_layout: str) -> np.ndarray:
    """Logical [K x N] operand from its storage: 'KN' as stored, 'NK' transposed."""
    B_stored = np.asarray(B_stored, dtype=np.float64)
    if b_layout == "KN":
        return B_stored
    if b_layout == "NK":
        return B_stored.T
    raise ValueError(b_layout)


def gemm(Y: np.ndarray, B: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    return alpha * (np.asarray(Y, dtype=np.float64) @ np.asarray(B, dtype=np.float64))


# --- the ordered epilogue (d9bl.com section 3.2; agentlenshq.com "How it works") ---

def apply_epilogue(C: np.ndarray, ops: Sequence[Tuple[str, Dict]],
                   row_ids=None) -> Tuple[np.ndarray, List[Tuple[str, Dict, np.ndarray]]]:
    """Apply ``ops`` in order to the running value v = C.

    Returns the final value and, for each reduction op in list order, a tuple
    (op name, its args, the fp64 result): one value per row for row_*, one per
    column (over all rows given) for col_*.  ``rms_rowscale`` is not an
    epilogue op here: the oracle applies it to A before the GEMM.  ``row_ids``
    are the global indices of C's rows (dropout's counter uses them; default
    0 .. rows - 1).
    """
    v = np.array(C, dtype=np.float64, copy=True)
    reductions = []
    for name, args in ops:
        if name == "scale":
            v = v * float(args["alpha"])
        elif name == "scale_row":
            v = v * np.asarray(args["vec"], dtype=np.float64)[:, None]
        elif name == "scale_col":
            v = v * np.asarray(args["vec"], dtype=np.float64)[None, :]
        elif name == "add_col":
            v = v + np.asarray(args["vec"], dtype=np.float64)[None, :]
        elif name == "add_row":
            v = v + np.asarray(args["vec"], dtype=np.float64)[:, None]
        elif name == "add_mat":
            v = v + float(args.get("beta", 1.0)) * np.asarray(args["mat"], dtype=np.float64)
        elif name == "gelu_tanh":
            v = gelu_tanh(v)
        elif name == "silu":
            v = silu(v)
        elif name == "swiglu_pair":
            v = swiglu_pair(v)
        elif name == "mul_dgelu_tanh":
            v = v * gelu_tanh_grad(np.asarray(args["mat"], dtype=np.float64))
        elif name == "dropout":
            v = dropout(v, float(args["p"]), int(args.get("seed", 0)), int(args.get("offset", 0)), row_ids)
        elif name == "rms_bwd":
            # v is dL/dY of Y = rmsnorm(x, gamma, eps); the op's value is dL/dx
            # (the plain gradient; row statistics a caller may pass are ignored)
            v = rmsnorm_backward(args["x"], args["gamma"], float(args["eps"]), v)[0]
        elif name == "row_sum":
            reductions.append((name, args, np.sum(v, axis=1)))
        elif name == "row_sumsq":
            reductions.append((name, args, np.sum(v * v, axis=1)))
        elif name == "row_mean":
            width = v.shape[1]
            if width == 0:
                raise ValueError("row_mean over an empty row is undefined")
            reductions.append((name, args, np.sum(v, axis=1) / width))
        elif name == "row_dot":
            reductions.append((name, args, np.sum(v * np.asarray(args["mat"], dtype=np.float64), axis=1)))
        elif name == "col_sum":
            reductions.append((name, args, np.sum(v, axis=0)))
        elif name == "col_sumsq":
            reductions.append((name, args, np.sum(v * v, axis=0)))
        elif name == "rms_dgamma":
            # v is dL/dY of Y = rmsnorm(x, gamma, eps): dL/dgamma, one value per column
            x = np.asarray(args["x"], dtype=np.float64)
            reductions.append((name, args, np.sum(v * x / rms(x, float(args["eps"]))[:, None], axis=0)))
        elif name in ("rms_rowscale", "ln_rowscale"):
            raise ValueError(f"{name} is applied to A by forward(); it must come first")
        else:
            raise ValueError(f"unknown op {name}")
    return v, reductions


def forward(A: np.ndarray, B_stored: np.ndarray, ops: Sequence[Tuple[str, Dict]],
            b_layout: str = "KN", alpha: float = 1.0, row_ids=None):
    """Normalise (if the list starts with rms_rowscale or ln_rowscale) -> GEMM -> ordered epilogue.

    ``ops`` items are (name, args) with array-valued args already resolved;
    ``row_ids`` are the global indices of A's rows when A is a row subset.
    Returns (D fp64, list of (name, args, fp64 per-row result)).
    """
    A = np.asarray(A, dtype=np.float64)
    ops = list(ops)
    Y = A
    if ops and ops[0][0] in ("rms_rowscale", "ln_rowscale"):
        name, args = ops[0]
        if name == "rms_rowscale":
            Y = rmsnorm(A, args["gamma"], float(args["eps"]))
        else:
            Y = layernorm(A, args["gamma"], float(args["eps"]), args.get("beta"))
        ops = ops[1:]
    for name, _ in ops:
        if name in ("rms_rowscale", "ln_rowscale"):
            raise ValueError(f"{name} must be the first op")
    C = gemm(Y, logical_b(B_stored, b_layout), alpha)
    return apply_epilogue(C, ops, row_ids)
