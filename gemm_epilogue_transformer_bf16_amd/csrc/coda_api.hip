// extern "C" entry points of the C ABI declared in coda.h.
#include "coda_launch.h"

namespace {

int finish(int st) {
  if (st == CODA_ERR_HIP) {
    const hipError_t e = hipGetLastError();
    coda::set_error("HIP launch failed: %s", hipGetErrorString(e));
  }
  return st;
}

}  // namespace

extern "C" {

int coda_gemm_epi(const void* A, const void* B, int64_t M, int64_t N, int64_t K, const coda_epi_desc* desc,
                  void* stream) {
  coda::Plan p;
  const int st = coda::build_plan(A, B, M, N, K, desc, 0, true, &p);
  if (st != CODA_OK) return st;
  return finish(coda::launch_fused(p, static_cast<hipStream_t>(stream)));
}

int coda_gemm_unfused(const void* A, const void* B, int64_t M, int64_t N, int64_t K, const coda_epi_desc* desc,
                      void* stream) {
  coda::Plan p;
  const int st = coda::build_plan(A, B, M, N, K, desc, 1, true, &p);
  if (st != CODA_OK) return st;
  return finish(coda::launch_unfused(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
