// Host-side launch entry points for validated plans (HIP side of the library).
#pragma once

#include <hip/hip_runtime.h>

#include "coda_plan.h"

namespace coda {

// Enqueue the fused kernel for `p` on `stream`.  Returns a coda_status.
int launch_fused(const Plan& p, hipStream_t stream);

// The same, with the cross-workgroup counters taken from `counters` (at least
// grid_m + grid_n + split_tiles words, zero on entry and left zero) instead
// of the workspace, whose counter regions are then unused.
int launch_fused_with_counters(const Plan& p, unsigned* counters, hipStream_t stream);

// Enqueue the unfused sequence for `p` on `stream`.  Returns a coda_status.
int launch_unfused(const Plan& p, hipStream_t stream);

// Enqueue the fused kernel with the epilogue list replaced by nothing: the
// plain GEMM writing d_dtype values to (out, ldo).  Used by the unfused path.
int launch_plain_gemm(const Plan& p, const void* A, int64_t lda, void* out, int64_t ldo,
                      hipStream_t stream);

}  // namespace coda
