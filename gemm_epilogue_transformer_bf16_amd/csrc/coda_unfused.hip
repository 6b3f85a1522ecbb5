// The unfused comparison sequence: one kernel per operator, intermediates in
// global memory (the framework-level execution the agentlenshq.com page
// describes under "The problem": the GEMM output written out and read straight
// back by the next operator's kernel).
//
//   [row norm pass]  ->  plain GEMM (same main loop as the fused kernel)
//   ->  one pass per elementwise op  ->  one pass per row reduction, two per
//   column reduction (partial sums over chunks of rows, then the chunks)
//
// Every pass streams its operands with 16-byte vector accesses.
#include "coda_device.h"
#include "coda_launch.h"

#include <cstring>

namespace coda {
namespace dev {

constexpr int kPassThreads = 256;

// ---- row normalisation of A, one wave per row ----
// RMS: Y = (x * rinv) * gamma with rinv = 1/sqrt(mean(x^2) + eps).
// LN:  Y = ((x - mu) * rstd) * gamma with mu the row mean and rstd = 1/sqrt(var +
//      eps), var the mean squared deviation (a second pass over the row, which
//      is in cache).  The shift beta is left to the epilogue's column term.
template <bool F32>
__device__ __forceinline__ float row_pass(const char* xr, int nch, int lane, float mu, bool sq) {
  float acc = 0.0f;
  for (int c = lane; c < nch; c += 64) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(xr + c * 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float v[2];
      if (F32) {
        v[0] = __uint_as_float(x[w]) - mu;
        v[1] = 0.0f;
      } else {
        v[0] = bf16_lo(x[w]) - mu;
        v[1] = bf16_hi(x[w]) - mu;
      }
      if (sq) {
        acc = fmaf(v[0], v[0], acc);
        acc = fmaf(v[1], v[1], acc);
      } else {
        acc += v[0] + v[1];
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  return acc;
}

template <bool F32, bool LN>
__global__ void __launch_bounds__(kPassThreads) rownorm_kernel(const void* X, long long ldx, const void* gamma,
                                                               float eps, int M, int K, void* Y, long long ldy) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kPassThreads / 64) + (threadIdx.x >> 6);
  if (row >= M) return;
  constexpr int CE = F32 ? 4 : 8;
  const int nch = K / CE;
  const char* xr = static_cast<const char*>(X) + (long long)row * ldx * (F32 ? 4 : 2);
  char* yr = static_cast<char*>(Y) + (long long)row * ldy * (F32 ? 4 : 2);
  const float mu = LN ? row_pass<F32>(xr, nch, lane, 0.0f, false) / float(K) : 0.0f;
  const float ss = row_pass<F32>(xr, nch, lane, mu, true);
  const float rinv = 1.0f / sqrtf(ss / float(K) + eps);
  // gamma NULL: the gain is folded into B, so the pass writes the unit-gain norm
  const char* gp = static_cast<const char*>(gamma);
  const u32x4_t ones = F32 ? u32x4_t{0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u}
                           : u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  for (int c = lane; c < nch; c += 64) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(xr + c * 16);
    const u32x4_t gv = gp ? *reinterpret_cast<const u32x4_t*>(gp + c * 16) : ones;
    u32x4_t y;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (F32) {
        y[w] = __float_as_uint(((__uint_as_float(x[w]) - mu) * rinv) * __uint_as_float(gv[w]));
      } else {
        y[w] = pack_bf16x2(((bf16_lo(x[w]) - mu) * rinv) * bf16_lo(gv[w]),
                           ((bf16_hi(x[w]) - mu) * rinv) * bf16_hi(gv[w]));
      }
    }
    *reinterpret_cast<u32x4_t*>(yr + c * 16) = y;
  }
}

// ---- one elementwise op per pass; each thread owns 8 consecutive input columns ----
__device__ __forceinline__ void load8(const void* p, int dtype, long long i, long long limit, float (&v)[8]) {
  if (dtype == CODA_BF16 && i + 7 < limit) {   // the group's 16 bytes in one access
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(w[e]);
      v[2 * e + 1] = bf16_hi(w[e]);
    }
    return;
  }
  float a[4], b[4];
  load4(p, dtype, i, limit, a);
  load4(p, dtype, i + 4, limit, b);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[4 + e] = b[e];
  }
}

__device__ __forceinline__ void store_n(void* p, int dtype, long long i, long long limit, const float* v, int n) {
  if (dtype == CODA_BF16) {
    uint16_t* d = static_cast<uint16_t*>(p) + i;
    if (n == 8 && i + 7 < limit) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      *reinterpret_cast<u32x4_t*>(d) = w;
    } else if (n == 4 && i + 3 < limit) {
      u32x2_t w;
      w[0] = pack_bf16x2(v[0], v[1]);
      w[1] = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<u32x2_t*>(d) = w;
    } else {
      for (int e = 0; e < n; ++e)
        if (i + e < limit) d[e] = f32_to_bf16_bits(v[e]);
    }
  } else {
    float* d = static_cast<float*>(p) + i;
    if (i + n - 1 < limit) {
      for (int e = 0; e < n; e += 4) {
        f32x4_t w;
        w[0] = v[e]; w[1] = v[e + 1]; w[2] = v[e + 2]; w[3] = v[e + 3];
        *reinterpret_cast<f32x4_t*>(d + e) = w;
      }
    } else {
      for (int e = 0; e < n; ++e)
        if (i + e < limit) d[e] = v[e];
    }
  }
}

// IDX: the index type of the element groups (32-bit when they number under
// 2^31, which keeps the row / column split of an index cheap)
template <class IDX>
__global__ void __launch_bounds__(kPassThreads) ew_kernel(const void* in, long long ldi, int width, int M,
                                                          void* out, long long ldo, int io_dtype, DevOp op) {
  const IDX groups_per_row = IDX((width + 7) / 8);
  const IDX total = groups_per_row * IDX(M);
  for (IDX gid = IDX(blockIdx.x) * kPassThreads + threadIdx.x; gid < total; gid += IDX(gridDim.x) * kPassThreads) {
    const int row = int(gid / groups_per_row);
    const long long c = (long long)(gid % groups_per_row) * 8;
    const int esz = io_dtype == CODA_BF16 ? 2 : 4;
    float v[8];
    load8(static_cast<const char*>(in) + (long long)row * ldi * esz, io_dtype, c, width, v);
    int nout = 8;
    long long oc = c;
    int out_width = width;
    switch (op.kind) {
      case CODA_OP_SCALE:
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= op.scalar;
        break;
      case CODA_OP_SCALE_ROW:
      case CODA_OP_ADD_ROW: {
        const float r = load_elem(op.in, op.dtype, row);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = op.kind == CODA_OP_ADD_ROW ? v[e] + r : v[e] * r;
        break;
      }
      case CODA_OP_SCALE_COL:
      case CODA_OP_ADD_COL: {
        float s[8];
        load8(op.in, op.dtype, c, width, s);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = op.kind == CODA_OP_ADD_COL ? v[e] + s[e] : v[e] * s[e];
        break;
      }
      case CODA_OP_ADD_MAT:
      case CODA_OP_MUL_DGELU_TANH: {
        float s[8];
        const int sz = op.dtype == CODA_BF16 ? 2 : 4;
        load8(static_cast<const char*>(op.in) + (long long)row * op.ld * sz, op.dtype, c, width, s);
        // the variant is chosen outside the element loop (inside it, the
        // compiler branches around every element)
        if (op.kind == CODA_OP_ADD_MAT) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] + op.scalar * s[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = v[e] * gelu_tanh_grad_f(s[e]);
        }
        break;
      }
      case CODA_OP_RMS_BWD: {
        float x[8], g[8];
        const int sz = op.dtype == CODA_BF16 ? 2 : 4;
        load8(static_cast<const char*>(op.in) + (long long)row * op.ld * sz, op.dtype, c, width, x);
        load8(op.in2, op.dtype, c, width, g);
        const long long ro = (long long)row * op.row_ld;
        const float r2 = op.row_ss[ro] / float(width) + op.scalar;
        const float rinv = 1.0f / sqrtf(r2);
        const float coef = op.row_s[ro] / float(width) / r2;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = g[e] * v[e] * rinv - x[e] * coef;
        break;
      }
      case CODA_OP_GELU_TANH:
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = gelu_tanh_f(v[e]);
        break;
      case CODA_OP_DROPOUT:
        dropout_values<8>(v, row, c, op.thr, op.scalar, op.seed, op.offset);
        break;
      case CODA_OP_SILU:
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = silu_f(v[e]);
        break;
      case CODA_OP_SWIGLU_PAIR:
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = silu_f(v[2 * e]) * v[2 * e + 1];
        nout = 4;
        oc = c / 2;
        out_width = width / 2;
        break;
      default:
        break;
    }
    store_n(static_cast<char*>(out) + (long long)row * ldo * esz, io_dtype, oc, out_width, v, nout);
  }
}

// ---- row reduction pass: one wave per row ----
__global__ void __launch_bounds__(kPassThreads) rowred_kernel(const void* in, long long ldi, int width, int M,
                                                              int io_dtype, DevOp op) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kPassThreads / 64) + (threadIdx.x >> 6);
  if (row >= M) return;
  const int esz = io_dtype == CODA_BF16 ? 2 : 4;
  const char* r = static_cast<const char*>(in) + (long long)row * ldi * esz;
  const bool sq = op.kind == CODA_OP_ROW_SUMSQ;
  const bool dot = op.kind == CODA_OP_ROW_DOT;
  const char* mrow = dot ? static_cast<const char*>(op.in) + (long long)row * op.ld * (op.dtype == CODA_BF16 ? 2 : 4)
                         : nullptr;
  float acc = 0.0f;
  for (long long c = lane * 8LL; c < width; c += 64 * 8) {
    float v[8];
    load8(r, io_dtype, c, width, v);
    if (dot) {
      float m[8];
      load8(mrow, op.dtype, c, width, m);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += v[e] * m[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += sq ? v[e] * v[e] : v[e];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) {
    if (op.kind == CODA_OP_ROW_MEAN) acc /= float(width);
    op.out[(long long)row * op.out_stride] = acc;
  }
}

// ---- column reductions over a stored tensor: partial sums over chunks of
// kColChunk rows (8 columns per thread), then the chunks in order per column ----
__global__ void __launch_bounds__(kPassThreads) colred_partial_kernel(const void* in, long long ldi, int width, int M,
                                                                      int io_dtype, DevOp op, float* part,
                                                                      long long ldp) {
  const long long c = ((long long)blockIdx.x * kPassThreads + threadIdx.x) * 8;
  if (c >= width) return;
  const int r0 = blockIdx.y * kColChunk;
  const int r1 = min(M, r0 + kColChunk);
  const int esz = io_dtype == CODA_BF16 ? 2 : 4;
  const bool sq = op.kind == CODA_OP_COL_SUMSQ;
  const bool dg = op.kind == CODA_OP_RMS_DGAMMA;   // sum of v * x / r over the rows
  const int xsz = op.dtype == CODA_BF16 ? 2 : 4;
  float acc[8] = {};
  for (int r = r0; r < r1; ++r) {
    float v[8];
    load8(static_cast<const char*>(in) + (long long)r * ldi * esz, io_dtype, c, width, v);
    if (dg) {
      float x[8];
      load8(static_cast<const char*>(op.in) + (long long)r * op.ld * xsz, op.dtype, c, width, x);
      const float rinv = 1.0f / sqrtf(op.row_ss[(long long)r * op.row_ld] / float(width) + op.scalar);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += v[e] * x[e] * rinv;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += sq ? v[e] * v[e] : v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c + e < width) part[(long long)blockIdx.y * ldp + c + e] = acc[e];
}

__global__ void __launch_bounds__(kPassThreads) colred_final_kernel(const float* part, long long ldp, int chunks,
                                                                    int width, DevOp op) {
  const long long c = (long long)blockIdx.x * kPassThreads + threadIdx.x;
  if (c >= width) return;
  float v = 0.0f;
  for (int k = 0; k < chunks; ++k) v += part[(long long)k * ldp + c];
  op.out[c * op.out_stride] = v;
}

}  // namespace dev

namespace {

bool is_row_reduction(int kind) {
  return kind == CODA_OP_ROW_SUM || kind == CODA_OP_ROW_SUMSQ || kind == CODA_OP_ROW_MEAN ||
         kind == CODA_OP_ROW_DOT;
}

bool is_col_reduction(int kind) {
  return kind == CODA_OP_COL_SUM || kind == CODA_OP_COL_SUMSQ || kind == CODA_OP_RMS_DGAMMA;
}

bool is_reduction(int kind) { return is_row_reduction(kind) || is_col_reduction(kind); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

dev::DevOp to_dev(const Op& q) {
  dev::DevOp d;
  std::memset(&d, 0, sizeof(d));
  d.kind = q.kind;
  d.dtype = q.dtype;
  d.in = q.in;
  d.ld = q.ld;
  d.scalar = q.scalar;
  d.width = (int)q.width;
  d.out = static_cast<float*>(q.out);
  d.out_stride = q.out_stride;
  d.red_slot = q.red_slot;
  d.in2 = q.in2;
  d.row_s = q.row_s;
  d.row_ss = q.row_ss;
  d.row_ld = q.row_ld;
  d.thr = q.thr;
  d.seed = q.seed;
  d.offset = q.offset;
  return d;
}

int check_launch() { return hipGetLastError() == hipSuccess ? CODA_OK : CODA_ERR_HIP; }

}  // namespace

int launch_unfused(const Plan& p, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return CODA_OK;
  char* ws = static_cast<char*>(p.workspace);
  const int M = (int)p.M;
  const void* gA = p.A;
  int64_t glda = p.lda;
  if (p.has_norm) {
    void* Xn = ws;
    ws += align256(size_t(p.M) * size_t(p.K) * dtype_size(p.ab_dtype));
    const unsigned blocks = unsigned((p.M + 3) / 4);
    auto* kern = p.ab_dtype == CODA_F32 ? (p.has_ln ? dev::rownorm_kernel<true, true> : dev::rownorm_kernel<true, false>)
                                        : (p.has_ln ? dev::rownorm_kernel<false, true> : dev::rownorm_kernel<false, false>);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(dev::kPassThreads), 0, stream, p.A, (long long)p.lda, p.gamma,
                       p.eps, M, (int)p.K, Xn, (long long)p.K);
    if (check_launch() != CODA_OK) return CODA_ERR_HIP;
    gA = Xn;
    glda = p.K;
  }
  const int64_t ldi = unfused_ld(p);
  void* bufs[2];
  bufs[0] = ws;
  bufs[1] = ws + align256(size_t(p.M) * size_t(ldi) * dtype_size(p.d_dtype));

  int last_ew = -1;
  for (int i = 0; i < p.n_ops; ++i)
    if (!is_reduction(p.ops[i].kind)) last_ew = i;

  const void* cur;
  int64_t ldc;
  int which = 0;
  if (last_ew < 0) {
    if (launch_plain_gemm(p, gA, glda, p.D, p.ldd, stream) != CODA_OK) return CODA_ERR_HIP;
    cur = p.D;
    ldc = p.ldd;
  } else {
    if (launch_plain_gemm(p, gA, glda, bufs[0], ldi, stream) != CODA_OK) return CODA_ERR_HIP;
    cur = bufs[0];
    ldc = ldi;
  }
  int64_t width = p.N;
  for (int i = 0; i < p.n_ops; ++i) {
    const Op& q = p.ops[i];
    const dev::DevOp d = to_dev(q);
    if (is_row_reduction(q.kind)) {
      const unsigned blocks = unsigned((p.M + 3) / 4);
      hipLaunchKernelGGL(dev::rowred_kernel, dim3(blocks), dim3(dev::kPassThreads), 0, stream, cur, (long long)ldc,
                         (int)width, M, p.d_dtype, d);
      if (check_launch() != CODA_OK) return CODA_ERR_HIP;
      continue;
    }
    if (is_col_reduction(q.kind)) {
      float* part = reinterpret_cast<float*>(static_cast<char*>(p.workspace) + unfused_col_partials_offset(p));
      const int chunks = int((p.M + kColChunk - 1) / kColChunk);
      const unsigned gx = unsigned(((width + 7) / 8 + dev::kPassThreads - 1) / dev::kPassThreads);
      hipLaunchKernelGGL(dev::colred_partial_kernel, dim3(gx, (unsigned)chunks), dim3(dev::kPassThreads), 0, stream,
                         cur, (long long)ldc, (int)width, M, p.d_dtype, d, part, (long long)ldi);
      if (check_launch() != CODA_OK) return CODA_ERR_HIP;
      const unsigned gf = unsigned((width + dev::kPassThreads - 1) / dev::kPassThreads);
      hipLaunchKernelGGL(dev::colred_final_kernel, dim3(gf), dim3(dev::kPassThreads), 0, stream, part,
                         (long long)ldi, chunks, (int)width, d);
      if (check_launch() != CODA_OK) return CODA_ERR_HIP;
      continue;
    }
    void* dst;
    int64_t ldo;
    if (i == last_ew) {
      dst = p.D;
      ldo = p.ldd;
    } else {
      which ^= 1;
      dst = bufs[which];
      ldo = ldi;
    }
    const int64_t groups = ((width + 7) / 8) * p.M;
    int64_t blocks = (groups + dev::kPassThreads - 1) / dev::kPassThreads;
    if (blocks > 65536) blocks = 65536;
    if (groups < (int64_t(1) << 31))
      hipLaunchKernelGGL(dev::ew_kernel<uint32_t>, dim3((unsigned)blocks), dim3(dev::kPassThreads), 0, stream, cur,
                         (long long)ldc, (int)width, M, dst, (long long)ldo, p.d_dtype, d);
    else
      hipLaunchKernelGGL(dev::ew_kernel<long long>, dim3((unsigned)blocks), dim3(dev::kPassThreads), 0, stream, cur,
                         (long long)ldc, (int)width, M, dst, (long long)ldo, p.d_dtype, d);
    if (check_launch() != CODA_OK) return CODA_ERR_HIP;
    cur = dst;
    ldc = ldo;
    if (q.kind == CODA_OP_SWIGLU_PAIR) width /= 2;
  }
  return CODA_OK;
}

}  // namespace coda
