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
// base-2 exponential and reciprocal (about 1 ulp each in fp32).  The constant
// factors are folded: with z = sqrt(2/pi) (v + 0.044715 v^3),
//   -2 z log2(e) = v (kG1 + kG3 v^2),
// so GELU_tanh(v) = v / (1 + 2^(v (kG1 + kG3 v^2))) in 7 operations.
// ---------------------------------------------------------------------------
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kSqrt2OverPiD = 0.79788456080286535588;   // sqrt(2 / pi)
constexpr double kGeluCubicD = 0.044715;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr float kG1 = float(-2.0 * kSqrt2OverPiD * kLog2eD);
constexpr float kG3 = float(-2.0 * kSqrt2OverPiD * kGeluCubicD * kLog2eD);
// d(2z)/dv = kD0 + kD2 v^2
constexpr float kD0 = float(2.0 * kSqrt2OverPiD);
constexpr float kD2 = float(2.0 * kSqrt2OverPiD * 3.0 * kGeluCubicD);

__device__ __forceinline__ float sigmoid_f(float x) {
  // 1 / (1 + 2^(-x log2 e)); saturates cleanly to 0 / 1 at the extremes
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}

// s = sigmoid(2 z(v)) = 0.5 (1 + tanh(z(v)))
__device__ __forceinline__ float gelu_gate_f(float v, float v2) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * fmaf(kG3, v2, kG1)));
}

__device__ __forceinline__ float gelu_tanh_f(float v) { return v * gelu_gate_f(v, v * v); }

__device__ __forceinline__ float silu_f(float v) { return v * sigmoid_f(v); }

// d/dp [0.5 p (1 + tanh(z(p)))] = s + 2 p s (1 - s) z'(p), with s = sigmoid(2 z)
// (since 1 - tanh^2 = 4 s (1 - s)) and 2 z'(p) = kD0 + kD2 p^2.
__device__ __forceinline__ float gelu_tanh_grad_f(float p) {
  const float p2 = p * p;
  const float s = gelu_gate_f(p, p2);
  const float dz2 = p * fmaf(kD2, p2, kD0);   // 2 p z'(p)
  return fmaf(dz2, s * (1.0f - s), s);
}

// ---------------------------------------------------------------------------
// Dropout's generator: Philox-4x64 with 10 rounds (Salmon, Moraes, Dror and
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011).  A round
// multiplies counter words 0 and 2 by the two round multipliers into 128-bit
// products and recombines them with words 1 and 3 and the key; the key then
// advances by the two Weyl increments (the golden ratio and sqrt(3) - 1 as
// 64-bit fractions).
// ---------------------------------------------------------------------------
constexpr unsigned long long kPhiloxM0 = 0xD2E7470EE14C6C93ull, kPhiloxM1 = 0xCA5A826395121157ull;
constexpr unsigned long long kPhiloxW0 = 0x9E3779B97F4A7C15ull, kPhiloxW1 = 0xBB67AE8584CAA73Bull;

__device__ __forceinline__ void philox4x64_10(unsigned long long (&c)[4], unsigned long long k0,
                                              unsigned long long k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const unsigned long long hi0 = __umul64hi(kPhiloxM0, c[0]), lo0 = kPhiloxM0 * c[0];
    const unsigned long long hi1 = __umul64hi(kPhiloxM1, c[2]), lo1 = kPhiloxM1 * c[2];
    c[0] = hi1 ^ c[1] ^ k0;
    c[1] = lo1;
    c[2] = hi0 ^ c[3] ^ k1;
    c[3] = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
}

// Inverted dropout of n consecutive values v[0..n) of row `row`, columns
// col .. col + n - 1, with n = 8 and col % 8 == 0, or n = 4 and col % 4 == 0
// (one generator block either way): the block has key (seed, 0) and counter
// (col / 8, row, offset, 0), column j takes 32-bit word j % 8 (the low half of
// 64-bit word (j % 8) / 2 when even, the high half when odd), and a value is
// kept, times `scale`, when its word is >= thr.
template <int n>
__device__ __forceinline__ void dropout_values(float* v, long long row, long long col, unsigned thr, float scale,
                                               unsigned long long seed, unsigned long long offset) {
  static_assert(n == 8 || n == 4, "one generator block per call");
  unsigned long long c[4] = {(unsigned long long)(col >> 3), (unsigned long long)row, offset, 0ull};
  philox4x64_10(c, seed, 0ull);
  // the upper half of a block (col % 8 == 4) takes 64-bit words 2 and 3; a
  // select rather than a runtime index keeps the words in registers
  const bool upper = n == 4 && (col & 4) != 0;
  const unsigned long long x[4] = {upper ? c[2] : c[0], upper ? c[3] : c[1], c[2], c[3]};
#pragma unroll
  for (int e = 0; e < n; ++e) {
    const unsigned word = unsigned(x[e >> 1] >> (32 * (e & 1)));
    v[e] = word >= thr ? v[e] * scale : 0.0f;
  }
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

// For extents known to be >= 0 (the main loop's): the clamp to 2^31 - 1 is a
// shift test that stays on the scalar unit (a signed 64-bit compare has no
// scalar form and costs vector compares and lane reads every K step).  No
// offset within a tile reaches 2^31, so clamping larger extents loses nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_nonneg(const void* base, int64_t bytes) {
  const uint64_t b = uint64_t(bytes);
  const int n = (b >> 31) ? 0x7fffffff : int(b);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferFlags);
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
  unsigned thr;         // DROPOUT: keep when the element's 32-bit word >= thr
  const void* in2;      // RMS_BWD: gamma [width] (dtype)
  const float* row_s;   // RMS_BWD: t per row (row_ld apart)
  const float* row_ss;  // RMS_BWD: sum of squares of x per row
  long long row_ld;
  unsigned long long seed, offset;   // DROPOUT: key word 0, counter word 2 (scalar = 1 / (1 - p))
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
