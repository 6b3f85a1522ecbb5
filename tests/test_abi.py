"""C-ABI checks that need no GPU: the library loads, exports every function
coda.h declares, the ctypes structs match the C layout, and host validation
returns the documented status codes (also under ASan/UBSan in a host build)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coda.h")
CSRC = os.path.join(ROOT, "gemm_epilogue_transformer_bf16_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")


@pytest.fixture(scope="module")
def C():
    lib = os.path.join(ROOT, "gemm_epilogue_transformer_bf16_amd", "libcoda.so")
    if not os.path.exists(lib):
        from gemm_epilogue_transformer_bf16_amd import build
        build.build()
    from gemm_epilogue_transformer_bf16_amd import coda
    return coda


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coda_[a-z_]+)\s*\(", text)))


def test_header_functions_exported(C):
    names = declared_functions()
    assert set(names) == set(C.EXPORTED)
    lib = ctypes.CDLL(C.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_struct_layout_matches_c(C, tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    src = tmp_path / "layout.c"
    src.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "coda.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(coda_op), offsetof(coda_op, out), offsetof(coda_op, out_stride),
         offsetof(coda_op, in2), offsetof(coda_op, row_ld), sizeof(coda_epi_desc), offsetof(coda_epi_desc, tile),
         offsetof(coda_epi_desc, ops));
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.run([gcc, f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)], check=True)
    vals = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()))
    assert vals == [ctypes.sizeof(C.coda_op), C.coda_op.out.offset, C.coda_op.out_stride.offset, C.coda_op.in2.offset,
                    C.coda_op.row_ld.offset, ctypes.sizeof(C.coda_epi_desc), C.coda_epi_desc.tile.offset,
                    C.coda_epi_desc.ops.offset]


def test_validation_status_codes_via_library(C):
    d = C.coda_epi_desc()
    d.ab_dtype = C.CODA_BF16
    d.d_dtype = C.CODA_BF16
    d.b_layout = C.CODA_B_KN
    d.lda, d.ldb, d.ldd = 64, 128, 128
    d.D = 0x30000000
    A, B = 0x10000000, 0x20000000
    assert C.coda_validate(A, B, 64, 128, 64, d, 0) == C.CODA_OK
    assert C.coda_validate(A, B, 64, 128, 60, d, 0) == C.CODA_ERR_UNSUPPORTED
    assert "multiple of 8" in C.coda_last_error()
    d.n_ops = 1
    d.ops[0].kind = C.CODA_OP_ROW_SUM
    assert C.coda_validate(A, B, 64, 128, 64, d, 0) == C.CODA_ERR_INVALID_ARG
    # an invalid call enqueues nothing and returns before touching the device
    assert C.coda_gemm_epi(A, B, 64, 128, 64, d, None) == C.CODA_ERR_INVALID_ARG
    assert C.coda_gemm_unfused(A, B, 64, 128, 64, d, None) == C.CODA_ERR_INVALID_ARG
    d.n_ops = 0
    # an empty problem is a no-op
    assert C.coda_gemm_epi(A, B, 0, 128, 64, d, None) == C.CODA_OK
    assert C.coda_status_string(C.CODA_ERR_HIP) == "CODA_ERR_HIP"
    assert C.coda_workspace_size(64, 128, 64, d, 0) == 0
    for i in range(1, C.coda_num_tile_configs() + 1):
        bm, bn, bk, waves = C.coda_tile_config(i)
        assert bm % 32 == 0 and bn % 32 == 0 and bk % 16 == 0 and waves in (4, 8)


def test_host_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    exe = tmp_path / "test_plan_host"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "host", "test_plan_host.cpp"), os.path.join(CSRC, "coda_plan.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL OK" in r.stdout
