// Weight-side preparation of the deferred row norms.
//
// coda_fold_gain: B' = diag(gamma) B, the per-feature gain of a row norm moved
// into the rows of the following projection ((x * gamma) W = x (gamma W), the
// reparameterisation of the zeli.app page's "augment_me" comment), rounded
// once to B's dtype; the fused kernel then feeds A to the MFMAs unchanged.
//
// coda_ln_fold: the constant rows of the deferred LayerNorm, u = gamma^T B
// and c = beta^T B.
//
// Moving a LayerNorm past the projection (the zeli.app page's "augment_me"
// comment moves a row-wise norm's per-row factors past the matmul; the norm is
// the mean-centred one of the Transformer operators in the d9bl.com page's
// Fig. 4) leaves two column vectors that depend on the weights alone: the mean
// term multiplies u, and the shift beta contributes c.  Both are one weighted
// column sum of B, computed here in fp32 (bf16 x bf16 products are exact in
// fp32), reading B once.
#include "coda_device.h"
#include "coda_launch.h"

namespace coda {
namespace dev {

constexpr int kFoldThreads = 256;
constexpr int kFoldSlices = 8;                           // K slices per workgroup (B stored [K x N])
constexpr int kFoldCols = 8 * (kFoldThreads / kFoldSlices);   // columns per workgroup

__device__ __forceinline__ void load8f(const void* p, int dtype, long long i, float (&v)[8]) {
  if (dtype == CODA_BF16) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(w[e]);
      v[2 * e + 1] = bf16_hi(w[e]);
    }
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
}

// B stored [K x N]: thread (slice s, group g) sums rows k = s, s + 8, ... of the
// 8 columns 8g .. 8g+7 of its workgroup's column block; the 8 slices are then
// added in slice order through LDS.
__global__ void __launch_bounds__(kFoldThreads) fold_kn_kernel(const void* B, long long ldb, int K, int N, int dtype,
                                                               const void* gamma, const void* beta, float* u,
                                                               float* c) {
  __shared__ float part[2][kFoldSlices][kFoldCols];
  const int g = threadIdx.x % (kFoldThreads / kFoldSlices);
  const int sl = threadIdx.x / (kFoldThreads / kFoldSlices);
  const long long col = (long long)blockIdx.x * kFoldCols + 8 * g;
  float su[8] = {}, sc[8] = {};
  if (col < N) {   // N % 8 == 0 for this layout, so a group is all in or all out
    for (int k = sl; k < K; k += kFoldSlices) {
      float b[8];
      load8f(B, dtype, (long long)k * ldb + col, b);
      const float gk = load_elem(gamma, dtype, k);
      const float bk = beta ? load_elem(beta, dtype, k) : 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        su[e] = fmaf(gk, b[e], su[e]);
        sc[e] = fmaf(bk, b[e], sc[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    part[0][sl][8 * g + e] = su[e];
    part[1][sl][8 * g + e] = sc[e];
  }
  __syncthreads();
  for (int t = threadIdx.x; t < kFoldCols; t += kFoldThreads) {
    const long long j = (long long)blockIdx.x * kFoldCols + t;
    if (j >= N) continue;
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int s = 0; s < kFoldSlices; ++s) {
      a += part[0][s][t];
      b += part[1][s][t];
    }
    u[j] = a;
    if (c) c[j] = b;
  }
}

// B stored [N x K] (row j of storage is column j of the logical B): one wave
// per column, lanes over 8-element chunks of K, then a wave reduction.
__global__ void __launch_bounds__(kFoldThreads) fold_nk_kernel(const void* B, long long ldb, int K, int N, int dtype,
                                                               const void* gamma, const void* beta, float* u,
                                                               float* c) {
  const int lane = threadIdx.x & 63;
  const long long j = (long long)blockIdx.x * (kFoldThreads / 64) + (threadIdx.x >> 6);
  if (j >= N) return;
  float su = 0.0f, sc = 0.0f;
  for (int k = 8 * lane; k < K; k += 8 * 64) {
    float b[8], gv[8], bv[8] = {};
    load8f(B, dtype, j * ldb + k, b);
    load8f(gamma, dtype, k, gv);
    if (beta) load8f(beta, dtype, k, bv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      su = fmaf(gv[e], b[e], su);
      sc = fmaf(bv[e], b[e], sc);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    su += __shfl_xor(su, off);
    sc += __shfl_xor(sc, off);
  }
  if (lane == 0) {
    u[j] = su;
    if (c) c[j] = sc;
  }
}

// B' = diag(gamma) B, 8 consecutive elements of a storage row per thread
// (the storage rows are K rows of B for [K x N] storage, N rows for [N x K]).
template <bool F32>
__global__ void __launch_bounds__(kFoldThreads) fold_gain_kernel(const void* B, long long ldb, const void* gamma,
                                                                 void* Bo, long long ldo, long long rows, int inner,
                                                                 bool kn) {
  const int cpr = inner / 8;
  const long long t = (long long)blockIdx.x * kFoldThreads + threadIdx.x;
  if (t >= rows * cpr) return;
  const long long r = t / cpr;
  const int c0 = int(t % cpr) * 8;
  float b[8], g[8];
  load8f(B, F32 ? CODA_F32 : CODA_BF16, r * ldb + c0, b);
  if (kn) {
    const float gk = load_elem(gamma, F32 ? CODA_F32 : CODA_BF16, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = gk;
  } else {
    load8f(gamma, F32 ? CODA_F32 : CODA_BF16, c0, g);
  }
  if (F32) {
    f32x4_t lo, hv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = b[e] * g[e];
      hv[e] = b[4 + e] * g[4 + e];
    }
    float* o = static_cast<float*>(Bo) + r * ldo + c0;
    *reinterpret_cast<f32x4_t*>(o) = lo;
    *reinterpret_cast<f32x4_t*>(o + 4) = hv;
  } else {
    u32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(b[2 * e] * g[2 * e], b[2 * e + 1] * g[2 * e + 1]);
    *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(Bo) + r * ldo + c0) = w;
  }
}

}  // namespace dev
}  // namespace coda

extern "C" int coda_fold_gain(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                              const void* gamma, void* B_out, int64_t ldo, void* stream) {
  const int st = coda::validate_fold_gain(B, K, N, ldb, b_layout, dtype, gamma, B_out, ldo);
  if (st != CODA_OK || K == 0 || N == 0) return st;
  const bool kn = b_layout == CODA_B_KN;
  const long long rows = kn ? K : N;
  const int inner = int(kn ? N : K);
  const long long threads = rows * (inner / 8);
  const unsigned blocks = unsigned((threads + coda::dev::kFoldThreads - 1) / coda::dev::kFoldThreads);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == CODA_F32)
    hipLaunchKernelGGL(coda::dev::fold_gain_kernel<true>, dim3(blocks), dim3(coda::dev::kFoldThreads), 0, s, B,
                       (long long)ldb, gamma, B_out, (long long)ldo, rows, inner, kn);
  else
    hipLaunchKernelGGL(coda::dev::fold_gain_kernel<false>, dim3(blocks), dim3(coda::dev::kFoldThreads), 0, s, B,
                       (long long)ldb, gamma, B_out, (long long)ldo, rows, inner, kn);
  if (hipGetLastError() != hipSuccess) {
    coda::set_error("HIP launch failed (coda_fold_gain)");
    return CODA_ERR_HIP;
  }
  return CODA_OK;
}

extern "C" int coda_ln_fold(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                            const void* gamma, const void* beta, float* u, float* c, void* stream) {
  const int st = coda::validate_ln_fold(B, K, N, ldb, b_layout, dtype, gamma, beta, u, c);
  if (st != CODA_OK || N == 0) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (b_layout == CODA_B_KN) {
    const unsigned blocks = unsigned((N + coda::dev::kFoldCols - 1) / coda::dev::kFoldCols);
    hipLaunchKernelGGL(coda::dev::fold_kn_kernel, dim3(blocks), dim3(coda::dev::kFoldThreads), 0, s, B,
                       (long long)ldb, (int)K, (int)N, (int)dtype, gamma, beta, u, c);
  } else {
    const unsigned blocks = unsigned((N + 3) / 4);
    hipLaunchKernelGGL(coda::dev::fold_nk_kernel, dim3(blocks), dim3(coda::dev::kFoldThreads), 0, s, B,
                       (long long)ldb, (int)K, (int)N, (int)dtype, gamma, beta, u, c);
  }
  if (hipGetLastError() != hipSuccess) {
    coda::set_error("HIP launch failed (coda_ln_fold)");
    return CODA_ERR_HIP;
  }
  return CODA_OK;
}
