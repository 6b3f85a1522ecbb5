"""ctypes binding of the C ABI in include/coda.h (argument marshalling only).

Every function here forwards to libcoda.so with the same name; nothing is
computed in Python.  Importing this module loads the library and raises if it
has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libcoda.so")

# ---- constants (mirror coda.h) ----
CODA_MAX_OPS = 16
CODA_MAX_REDUCTIONS = 8
CODA_MAX_COL_REDUCTIONS = 2
CODA_FLAG_NO_SPLIT_K = 1

CODA_OK = 0
CODA_ERR_INVALID_ARG = -1
CODA_ERR_UNSUPPORTED = -2
CODA_ERR_WORKSPACE = -3
CODA_ERR_HIP = -4

CODA_BF16 = 0
CODA_F32 = 1

CODA_A_MK = 0
CODA_A_KM = 1

CODA_B_KN = 0
CODA_B_NK = 1

CODA_OP_SCALE = 0
CODA_OP_SCALE_ROW = 1
CODA_OP_SCALE_COL = 2
CODA_OP_RMS_ROWSCALE = 3
CODA_OP_ADD_COL = 4
CODA_OP_ADD_ROW = 5
CODA_OP_ADD_MAT = 6
CODA_OP_GELU_TANH = 7
CODA_OP_SILU = 8
CODA_OP_SWIGLU_PAIR = 9
CODA_OP_MUL_DGELU_TANH = 10
CODA_OP_ROW_SUM = 11
CODA_OP_ROW_SUMSQ = 12
CODA_OP_ROW_MEAN = 13
CODA_OP_LN_ROWSCALE = 14
CODA_OP_COL_SUM = 15
CODA_OP_COL_SUMSQ = 16
CODA_OP_ROW_DOT = 17
CODA_OP_RMS_BWD = 18
CODA_OP_RMS_DGAMMA = 19
CODA_OP_DROPOUT = 20

EXPORTED = (
    "coda_gemm_epi", "coda_gemm_unfused", "coda_validate", "coda_workspace_size",
    "coda_status_string", "coda_last_error", "coda_num_tile_configs", "coda_tile_config",
    "coda_selected_tile", "coda_ln_fold", "coda_fold_gain", "coda_gemm_epi_noalloc",
)
CODA_NOALLOC_SCRATCH_BYTES = 64 << 20


class coda_op(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("in_", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("scalar", ctypes.c_float),
        ("reserved0", ctypes.c_int32),
        ("out", ctypes.c_void_p),
        ("out_stride", ctypes.c_int64),
        ("in2", ctypes.c_void_p),
        ("row_sum", ctypes.c_void_p),
        ("row_sumsq", ctypes.c_void_p),
        ("row_ld", ctypes.c_int64),
        ("seed", ctypes.c_uint64),
        ("offset", ctypes.c_uint64),
    ]


class coda_epi_desc(ctypes.Structure):
    _fields_ = [
        ("ab_dtype", ctypes.c_int32),
        ("d_dtype", ctypes.c_int32),
        ("b_layout", ctypes.c_int32),
        ("n_ops", ctypes.c_int32),
        ("lda", ctypes.c_int64),
        ("ldb", ctypes.c_int64),
        ("ldd", ctypes.c_int64),
        ("D", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("tile", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("a_layout", ctypes.c_int32),
        ("reserved1", ctypes.c_int32),
        ("ops", coda_op * CODA_MAX_OPS),
    ]


class CodaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {coda_status_string(status)} ({coda_last_error()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with gemm_epilogue_transformer_bf16_amd.build.build() "
            "(hipcc --offload-arch=gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    DESC = ctypes.POINTER(coda_epi_desc)
    lib.coda_gemm_epi.argtypes = [P, P, I64, I64, I64, DESC, P]
    lib.coda_gemm_epi.restype = ctypes.c_int
    lib.coda_gemm_epi_noalloc.argtypes = [P, P, I64, I64, I64, DESC, P]
    lib.coda_gemm_epi_noalloc.restype = ctypes.c_int
    lib.coda_gemm_unfused.argtypes = [P, P, I64, I64, I64, DESC, P]
    lib.coda_gemm_unfused.restype = ctypes.c_int
    lib.coda_validate.argtypes = [P, P, I64, I64, I64, DESC, ctypes.c_int]
    lib.coda_validate.restype = ctypes.c_int
    lib.coda_workspace_size.argtypes = [I64, I64, I64, DESC, ctypes.c_int]
    lib.coda_workspace_size.restype = ctypes.c_size_t
    lib.coda_status_string.argtypes = [ctypes.c_int]
    lib.coda_status_string.restype = ctypes.c_char_p
    lib.coda_last_error.argtypes = []
    lib.coda_last_error.restype = ctypes.c_char_p
    lib.coda_num_tile_configs.argtypes = []
    lib.coda_num_tile_configs.restype = ctypes.c_int
    lib.coda_tile_config.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int)] * 4
    lib.coda_tile_config.restype = ctypes.c_int
    lib.coda_selected_tile.argtypes = [I64, I64, I64, DESC]
    lib.coda_selected_tile.restype = ctypes.c_int
    lib.coda_ln_fold.argtypes = [P, I64, I64, I64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
    lib.coda_ln_fold.restype = ctypes.c_int
    lib.coda_fold_gain.argtypes = [P, I64, I64, I64, ctypes.c_int32, ctypes.c_int32, P, P, I64, P]
    lib.coda_fold_gain.restype = ctypes.c_int
    return lib


lib = _load()


def _desc_ptr(desc):
    return None if desc is None else ctypes.byref(desc)


# ---- same-name forwards ----

def coda_gemm_epi(A: int, B: int, M: int, N: int, K: int, desc: coda_epi_desc, stream: int = 0) -> int:
    return lib.coda_gemm_epi(A, B, M, N, K, _desc_ptr(desc), stream)


def coda_gemm_epi_noalloc(A: int, B: int, M: int, N: int, K: int, desc: coda_epi_desc, stream: int = 0) -> int:
    return lib.coda_gemm_epi_noalloc(A, B, M, N, K, _desc_ptr(desc), stream)


def coda_gemm_unfused(A: int, B: int, M: int, N: int, K: int, desc: coda_epi_desc, stream: int = 0) -> int:
    return lib.coda_gemm_unfused(A, B, M, N, K, _desc_ptr(desc), stream)


def coda_validate(A: int, B: int, M: int, N: int, K: int, desc: coda_epi_desc, unfused: int = 0) -> int:
    return lib.coda_validate(A, B, M, N, K, _desc_ptr(desc), unfused)


def coda_workspace_size(M: int, N: int, K: int, desc: coda_epi_desc, unfused: int = 0) -> int:
    return lib.coda_workspace_size(M, N, K, _desc_ptr(desc), unfused)


def coda_status_string(status: int) -> str:
    return lib.coda_status_string(status).decode()


def coda_last_error() -> str:
    return lib.coda_last_error().decode()


def coda_num_tile_configs() -> int:
    return lib.coda_num_tile_configs()


def coda_tile_config(index: int):
    vals = [ctypes.c_int() for _ in range(4)]
    st = lib.coda_tile_config(index, *[ctypes.byref(v) for v in vals])
    if st != CODA_OK:
        raise CodaError(st, "coda_tile_config")
    return tuple(v.value for v in vals)   # (bm, bn, bk, waves)


def coda_selected_tile(M: int, N: int, K: int, desc: coda_epi_desc) -> int:
    return lib.coda_selected_tile(M, N, K, _desc_ptr(desc))


def coda_ln_fold(B: int, K: int, N: int, ldb: int, b_layout: int, dtype: int, gamma: int, beta,
                 u: int, c, stream: int = 0) -> int:
    return lib.coda_ln_fold(B, K, N, ldb, b_layout, dtype, gamma, beta, u, c, stream)


def coda_fold_gain(B: int, K: int, N: int, ldb: int, b_layout: int, dtype: int, gamma: int, B_out: int,
                   ldo: int, stream: int = 0) -> int:
    return lib.coda_fold_gain(B, K, N, ldb, b_layout, dtype, gamma, B_out, ldo, stream)


def check(status: int, where: str) -> None:
    if status != CODA_OK:
        raise CodaError(status, where)
