// Device-side types and helpers shared by the fused and unfused kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "coda.h"

namespace coda {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  bf16 is the top half of an fp32 word, so widening is a shift;
// narrowing uses the gfx950 conversion instruction, which rounds to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return uint16_t(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// Activations, written from their definitions with the identity
// 0.5 * (1 + tanh(z)) = 1 / (1 + exp(-2z)), evaluated with the hardware
// base-2 exponential and reciprocal (about 1 ulp each in fp32).
// ---------------------------------------------------------------------------
constexpr float kSqrt2OverPi = 0.7978845608028654f;   // sqrt(2/pi)
constexpr float kGeluCubic = 0.044715f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sigmoid_f(float x) {
  // 1 / (1 + 2^(-x log2 e)); saturates cleanly to 0 / 1 at the extremes
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

__device__ __forceinline__ float gelu_tanh_f(float v) {
  const float z = kSqrt2OverPi * (v + kGeluCubic * v * v * v);
  return v * sigmoid_f(2.0f * z);
}

__device__ __forceinline__ float silu_f(float v) { return v * sigmoid_f(v); }

// d/dp [0.5 p (1 + tanh(z(p)))] = s + 2 p s (1 - s) z'(p), with s = sigmoid(2 z)
// (since 1 - tanh^2 = 4 s (1 - s)) and z'(p) = sqrt(2/pi) (1 + 3 * 0.044715 p^2).
__device__ __forceinline__ float gelu_tanh_grad_f(float p) {
  const float z = kSqrt2OverPi * (p + kGeluCubic * p * p * p);
  const float s = sigmoid_f(2.0f * z);
  const float dz = kSqrt2OverPi * (1.0f + 3.0f * kGeluCubic * p * p);
  return s + 2.0f * p * s * (1.0f - s) * dz;
}

// ---------------------------------------------------------------------------
// Buffer resources: raw (stride 0) buffers whose out-of-range loads return 0.
// Offsets at or above num_records read as zero instead of faulting, which is
// how tile tails and masked K chunks are zero-filled.
// ---------------------------------------------------------------------------
constexpr int kBufferFlags = 0x00020000;
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  int64_t n = bytes < 0 ? 0 : bytes;
  if (n > 0x7fffffffll) n = 0x7fffffffll;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufferFlags);
}

__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------------------
// Kernel argument blocks (passed by value).
// ---------------------------------------------------------------------------
struct DevOp {
  int kind;
  int dtype;
  const void* in;
  long long ld;
  float scalar;
  int width;            // running width when the op runs
  float* out;
  long long out_stride;
  int red_slot;         // reductions: 0..n_red-1
  int pad_;
  const void* in2;      // RMS_BWD: gamma [width] (dtype)
  const float* row_s;   // RMS_BWD: t per row (row_ld apart)
  const float* row_ss;  // RMS_BWD: sum of squares of x per row
  long long row_ld;
};

struct FusedArgs {
  const void* A;
  const void* B;
  void* D;
  const void* gamma;
  const float* ln_u;    // LayerNorm: u = gamma^T B [N]
  const float* row_ss;  // given row sums of squares: row_ss[i * row_ss_stride]
  const float* row_s;   // LayerNorm: given row sums (same stride)
  long long row_ss_stride;
  float* partials;      // [n_red][grid_n][M]
  unsigned* counters;   // [grid_m]
  long long lda, ldb, ldd;
  int M, N, K;
  int d_dtype;
  int out_width;
  int n_ops;
  int n_red;
  int n_colred;         // column reductions
  int grid_m, grid_n;
  float eps;
  // split of the last round over K (split_s == 1: none)
  int full_tiles;       // workgroups [0, full_tiles) compute whole tiles
  int split_s;          // then split_s workgroups per split tile
  int k_steps;          // K steps of the whole tile
  int pad_;
  float* split_acc;     // [split tiles][split_s][NT][acc registers]
  float* split_ss;      // [split tiles][split_s][BM] (RMS)
  unsigned* split_cnt;  // [split tiles]
  float* col_partials;  // [n_colred][grid_m][N]
  unsigned* col_counters;   // [grid_n]
  DevOp ops[CODA_MAX_OPS];
};

// Loads of epilogue side operands -------------------------------------------

__device__ __forceinline__ float load_elem(const void* p, int dtype, long long i) {
  return dtype == CODA_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i])
                            : static_cast<const float*>(p)[i];
}

// Four consecutive elements p[i .. i+3] (i % 4 == 0, p 16-byte aligned), zero past `limit`.
__device__ __forceinline__ void load4(const void* p, int dtype, long long i, long long limit, float (&v)[4]) {
  if (i + 3 < limit) {
    if (dtype == CODA_BF16) {
      u32x2_t w = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(p) + i);
      v[0] = bf16_lo(w[0]); v[1] = bf16_hi(w[0]); v[2] = bf16_lo(w[1]); v[3] = bf16_hi(w[1]);
    } else {
      f32x4_t w = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
      v[0] = w[0]; v[1] = w[1]; v[2] = w[2]; v[3] = w[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (i + e < limit) ? load_elem(p, dtype, i + e) : 0.0f;
  }
}

// Two consecutive elements p[i], p[i+1] (i % 2 == 0), zero past `limit`.
__device__ __forceinline__ void load2(const void* p, int dtype, long long i, long long limit, float (&v)[2]) {
  if (i + 1 < limit) {
    if (dtype == CODA_BF16) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p) + i);
      v[0] = bf16_lo(w); v[1] = bf16_hi(w);
    } else {
      const float* q = static_cast<const float*>(p) + i;
      v[0] = q[0]; v[1] = q[1];
    }
  } else {
    v[0] = (i < limit) ? load_elem(p, dtype, i) : 0.0f;
    v[1] = 0.0f;
  }
}

}  // namespace dev
}  // namespace coda
