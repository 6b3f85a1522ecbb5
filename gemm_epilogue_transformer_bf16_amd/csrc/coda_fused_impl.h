// Fused GEMM + ordered epilogue for gfx950.
//
// One workgroup computes one bm x bn output tile.  The main loop streams A and
// B tiles global -> registers -> LDS (double buffered: the next K step's loads
// are in flight while MFMA consumes the current one) and accumulates in fp32
// with v_mfma_f32_32x32x16_bf16 (bf16 operands) or v_mfma_f32_32x32x2f32 (fp32
// operands).  The tile is computed transposed (MFMA rows = columns of D), so
// each lane's accumulators hold runs of 4 consecutive output columns of one row:
// side operands are read and D is written as 8/16-byte vectors.
//
// With the deferred RMS op, the A loader multiplies each A element by gamma[k]
// (rounded to the operand dtype) before it goes to LDS and keeps the raw
// element's square in an fp32 per-row sum; after the last K step the per-row
// factor 1/sqrt(sum/K + eps) is applied to the accumulators (the per-row scale
// of a row-wise norm moved past the projection: the zeli.app "augment_me"
// comment; the agentlenshq.com page, "CODA's approach").
//
// The epilogue walks the op list in order on the accumulators (d9bl.com page,
// section 3.2), then stores D once.  Row reductions combine lanes, then waves
// through LDS, then the workgroups of one tile row through a workspace of
// partial sums finished by the last workgroup to arrive (deterministic order).
#pragma once

#include "coda_device.h"

#include <cstring>
#include <type_traits>

namespace coda {
namespace dev {

// Compile-time loop: calls f(std::integral_constant<int, I>) for I in [0, N).
// Used where a loop body is too large for the unroller, so that register-array
// indices stay compile-time constants.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}


// Workgroups are dealt to the 8 XCDs round-robin.  Give each XCD a contiguous
// range of logical tiles, and order the logical tiles in groups of 8 tile rows
// (column-major inside a group), so concurrently resident tiles on one XCD
// share A row panels and B column panels in that XCD's L2.
__device__ __forceinline__ void map_tile(int bid, int gm, int gn, int& tm, int& tn) {
  const int nwg = gm * gn;
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = nwg >> 3, r = nwg & 7;
  const int L = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  constexpr int G = 8;
  const int group = L / (G * gn);
  const int first = group * G;
  const int gsz = min(gm - first, G);
  const int rem = L - group * G * gn;
  tm = first + rem % gsz;
  tn = rem / gsz;
}

template <int BM_, int BN_, int BK_, int WM_, int WN_, bool F32_, bool BKN_, bool RMS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr bool F32 = F32_, BKN = BKN_, RMS = RMS_;
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int ES = F32 ? 4 : 2;     // operand element size
  static constexpr int CE = 16 / ES;         // elements per 16-byte chunk
  static constexpr int KCH = BK / CE;        // chunks per K row of a K-major tile
  // LDS row strides (elements).  bf16: 16-byte pad on K-major rows and 32-byte
  // pad on N-major rows make the MFMA operand reads bank-conflict free.  fp32:
  // one-element pad on K-major rows (element-wise reads and writes).
  static constexpr int SA = F32 ? BK + 1 : BK + 8;
  static constexpr int SB = F32 ? BN + 4 : BN + 16;
  static constexpr int A_ELEMS = BM * SA;
  static constexpr int B_ELEMS = BKN ? BK * SB : BN * SA;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * ES;
  // loader geometry
  static constexpr int A_CH = BM * KCH / NT;          // 16-byte chunks of A per thread
  static constexpr int A_RSTEP = NT / KCH;            // rows between them
  static constexpr int BKN_CPR = BN / CE;             // chunks per row of an N-major B tile
  static constexpr int B_CH = BKN ? BK * BKN_CPR / NT : BN * KCH / NT;
  static constexpr int B_RSTEP = BKN ? NT / BKN_CPR : NT / KCH;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be a multiple of 32");
  static_assert((BM * KCH) % NT == 0 && A_CH >= 1, "A tile must split evenly over threads");
  static_assert(B_CH >= 1, "B tile must split evenly over threads");
  static_assert(NT % KCH == 0 && A_RSTEP % 8 == 0, "loader rows");
  // epilogue scratch (floats), reusing the main-loop LDS
  static constexpr int EPI_FLOATS = BM + CODA_MAX_REDUCTIONS * WN * BM + 4;
  static_assert(EPI_FLOATS * 4 <= LDS_BYTES, "epilogue scratch must fit");
};

// ---------------------------------------------------------------------------
// epilogue on the accumulators
// ---------------------------------------------------------------------------

// The kernel reads its argument block straight from the kernarg segment
// (constant address space): the op list is indexed with a runtime op number,
// and indexing a by-value parameter would make the compiler copy the whole
// block to per-lane scratch memory.
typedef const __attribute__((address_space(4))) FusedArgs* KArgs;

template <class C>
struct Geo {
  int M;
  int m[C::MI];     // global row of each m-block for this lane
  int nb;           // global column of (ni = 0, g = 0, e = 0) for this lane
  int mloc0;        // local row (within the tile) of m-block 0
  int wn;
  int lane;
};

template <class C, bool PAIRED>
__device__ __forceinline__ int col_of(const Geo<C>& g, int ni, int grp) {
  const int c = g.nb + 32 * ni + 8 * grp;
  return PAIRED ? (c >> 1) : c;
}

// Applies ops[o..] to one 32 x 32 accumulator block (m-block mi, n-block ni)
// until the end of the list or a SWIGLU_PAIR (whose index is returned).  One
// block at a time keeps the epilogue's live set to the accumulators plus 16
// side-operand values.  Row reductions add the block's share of each row into
// the wave's slot of `red` (assigned on the first n-block, accumulated after).
template <class C, bool PAIRED>
__device__ __forceinline__ int run_ops(f32x16_t& acc, KArgs a, int o, const Geo<C>& g, int mi, int ni,
                                       float* red) {
  constexpr int EPG = PAIRED ? 2 : 4;   // live elements per group of 4 slots
  const int row = g.m[mi];
  const bool row_ok = row < g.M;
  for (; o < a->n_ops; ++o) {
    const __attribute__((address_space(4))) DevOp& op = a->ops[o];
    const int kind = op.kind;
    if (!PAIRED && kind == CODA_OP_SWIGLU_PAIR) return o;
    const int width = op.width;
    switch (kind) {
      case CODA_OP_SCALE: {
        const float s = op.scalar;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] *= s;
        break;
      }
      case CODA_OP_SCALE_ROW:
      case CODA_OP_ADD_ROW: {
        const bool add = kind == CODA_OP_ADD_ROW;
        const float v = row_ok ? load_elem(op.in, op.dtype, row) : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = add ? acc[r] + v : acc[r] * v;
        break;
      }
      case CODA_OP_SCALE_COL:
      case CODA_OP_ADD_COL: {
        const bool add = kind == CODA_OP_ADD_COL;
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          float v[4];
          if (PAIRED) {
            float t[2];
            load2(op.in, op.dtype, col_of<C, PAIRED>(g, ni, grp), width, t);
            v[0] = t[0]; v[1] = t[1]; v[2] = 0.f; v[3] = 0.f;
          } else {
            load4(op.in, op.dtype, col_of<C, PAIRED>(g, ni, grp), width, v);
          }
#pragma unroll
          for (int e = 0; e < EPG; ++e) {
            const float x = acc[4 * grp + e];
            acc[4 * grp + e] = add ? x + v[e] : x * v[e];
          }
        }
        break;
      }
      case CODA_OP_ADD_MAT:
      case CODA_OP_MUL_DGELU_TANH: {
        if (!row_ok) break;
        const bool addm = kind == CODA_OP_ADD_MAT;
        const float beta = op.scalar;
        const char* base = static_cast<const char*>(op.in) + (long long)row * op.ld * (op.dtype == CODA_BF16 ? 2 : 4);
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int c = col_of<C, PAIRED>(g, ni, grp);
          float v[4];
          if (PAIRED) {
            float t[2];
            load2(base, op.dtype, c, width, t);
            v[0] = t[0]; v[1] = t[1]; v[2] = 0.f; v[3] = 0.f;
          } else {
            load4(base, op.dtype, c, width, v);
          }
#pragma unroll
          for (int e = 0; e < EPG; ++e) {
            const float x = acc[4 * grp + e];
            acc[4 * grp + e] = addm ? x + beta * v[e] : x * gelu_tanh_grad_f(v[e]);
          }
        }
        break;
      }
      case CODA_OP_GELU_TANH:
      case CODA_OP_SILU: {
        const bool gelu = kind == CODA_OP_GELU_TANH;
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
#pragma unroll
          for (int e = 0; e < EPG; ++e) {
            const float x = acc[4 * grp + e];
            acc[4 * grp + e] = gelu ? gelu_tanh_f(x) : silu_f(x);
          }
        break;
      }
      case CODA_OP_ROW_SUM:
      case CODA_OP_ROW_MEAN:
      case CODA_OP_ROW_SUMSQ: {
        const bool sq = kind == CODA_OP_ROW_SUMSQ;
        float p = 0.0f;
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int c = col_of<C, PAIRED>(g, ni, grp);
#pragma unroll
          for (int e = 0; e < EPG; ++e) {
            const float x = acc[4 * grp + e];
            const float t = sq ? x * x : x;
            p += (c + e < width) ? t : 0.0f;
          }
        }
        // lanes l and l+32 hold the same row
        p += __shfl_xor(p, 32);
        if (g.lane < 32) {
          float* dst = red + (op.red_slot * C::WN + g.wn) * C::BM + g.mloc0 + 32 * mi + g.lane;
          *dst = (ni == 0) ? p : *dst + p;
        }
        break;
      }
      default:
        break;
    }
  }
  return o;
}

// out[j] = silu(v[2j]) * v[2j+1] inside each lane's group of 4 columns:
// slot 4g+0 <- pair (4g+0, 4g+1), slot 4g+1 <- pair (4g+2, 4g+3).
__device__ __forceinline__ void swiglu_pair_acc(f32x16_t& acc) {
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const float g0 = acc[4 * grp + 0], u0 = acc[4 * grp + 1];
    const float g1 = acc[4 * grp + 2], u1 = acc[4 * grp + 3];
    acc[4 * grp + 0] = silu_f(g0) * u0;
    acc[4 * grp + 1] = silu_f(g1) * u1;
  }
}

template <class C, bool PAIRED>
__device__ __forceinline__ void store_d(const f32x16_t& acc, KArgs a, const Geo<C>& g, int mi, int ni) {
  const int width = a->out_width;
  const int row = g.m[mi];
  if (row >= g.M) return;
  const long long rowoff = (long long)row * a->ldd;
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    const int c = col_of<C, PAIRED>(g, ni, grp);
    const float v0 = acc[4 * grp + 0], v1 = acc[4 * grp + 1];
    const float v2 = acc[4 * grp + 2], v3 = acc[4 * grp + 3];
    if (a->d_dtype == CODA_BF16) {
      uint16_t* d = static_cast<uint16_t*>(a->D) + rowoff + c;
      if (PAIRED) {
        if (c + 1 < width) {
          *reinterpret_cast<uint32_t*>(d) = pack_bf16x2(v0, v1);
        } else if (c < width) {
          d[0] = f32_to_bf16_bits(v0);
        }
      } else {
        if (c + 3 < width) {
          u32x2_t w;
          w[0] = pack_bf16x2(v0, v1);
          w[1] = pack_bf16x2(v2, v3);
          *reinterpret_cast<u32x2_t*>(d) = w;
        } else {
          const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < width) d[e] = f32_to_bf16_bits(vv[e]);
        }
      }
    } else {
      float* d = static_cast<float*>(a->D) + rowoff + c;
      if (PAIRED) {
        if (c + 1 < width) {
          d[0] = v0;
          d[1] = v1;
        } else if (c < width) {
          d[0] = v0;
        }
      } else {
        if (c + 3 < width) {
          f32x4_t w;
          w[0] = v0; w[1] = v1; w[2] = v2; w[3] = v3;
          *reinterpret_cast<f32x4_t*>(d) = w;
        } else {
          const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (c + e < width) d[e] = vv[e];
        }
      }
    }
  }
}

__device__ __forceinline__ void write_reduction(const __attribute__((address_space(4))) DevOp& op, int row, float v) {
  if (op.kind == CODA_OP_ROW_MEAN) v = v / float(op.width);
  op.out[(long long)row * op.out_stride] = v;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <class C>
__global__ void __launch_bounds__(C::NT) fused_kernel(FusedArgs args) {
  (void)args;
  const KArgs a = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, MI = C::MI, NI = C::NI;
  constexpr int SA = C::SA, SB = C::SB, ES = C::ES, CE = C::CE, KCH = C::KCH;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;

  int tile_m, tile_n;
  map_tile(blockIdx.x, a->grid_m, a->grid_n, tile_m, tile_n);
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int M = a->M, N = a->N, K = a->K;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // ---- loader geometry ----
  const int a_c = tid % KCH, a_r = tid / KCH;
  const int b_c = C::BKN ? tid % C::BKN_CPR : tid % KCH;
  const int b_r = C::BKN ? tid / C::BKN_CPR : tid / KCH;
  const char* Abase = static_cast<const char*>(a->A) + ((long long)m0 * a->lda) * ES;
  const char* Bbase = C::BKN ? static_cast<const char*>(a->B) + (long long)n0 * ES
                             : static_cast<const char*>(a->B) + ((long long)n0 * a->ldb) * ES;
  const uint32_t a_row_bytes = uint32_t(a->lda * ES);
  const uint32_t b_row_bytes = uint32_t(a->ldb * ES);
  const long long a_extent0 = ((long long)(M - 1 - m0) * a->lda + K) * ES;  // bytes from tile base
  const long long b_extent0 = C::BKN ? ((long long)(K - 1) * a->ldb + (N - n0)) * ES
                                     : ((long long)(N - 1 - n0) * a->ldb + K) * ES;

  u32x4_t areg[C::A_CH], breg[C::B_CH];
  u32x4_t greg;           // gamma chunk (RMS)
  float ss[C::A_CH];      // per-row sum of squares (RMS)
#pragma unroll
  for (int i = 0; i < C::A_CH; ++i) ss[i] = 0.0f;

  const int KT = (K + BK - 1) / BK;

  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    const bool kin_a = k0 + a_c * CE < K;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(Abase + (long long)k0 * ES, a_extent0 - (long long)k0 * ES);
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const uint32_t off = uint32_t(a_r + i * C::A_RSTEP) * a_row_bytes + uint32_t(a_c * 16);
      areg[i] = buffer_load16(ra, kin_a ? off : kOobOffset);
    }
    if (C::BKN) {
      const __amdgpu_buffer_rsrc_t rb =
          make_rsrc(Bbase + (long long)k0 * a->ldb * ES, b_extent0 - (long long)k0 * a->ldb * ES);
#pragma unroll
      for (int i = 0; i < C::B_CH; ++i) {
        const uint32_t off = uint32_t(b_r + i * C::B_RSTEP) * b_row_bytes + uint32_t(b_c * 16);
        breg[i] = buffer_load16(rb, off);
      }
    } else {
      const bool kin_b = k0 + b_c * CE < K;
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bbase + (long long)k0 * ES, b_extent0 - (long long)k0 * ES);
#pragma unroll
      for (int i = 0; i < C::B_CH; ++i) {
        const uint32_t off = uint32_t(b_r + i * C::B_RSTEP) * b_row_bytes + uint32_t(b_c * 16);
        breg[i] = buffer_load16(rb, kin_b ? off : kOobOffset);
      }
    }
    if (C::RMS) {
      const __amdgpu_buffer_rsrc_t rg = make_rsrc(a->gamma, (long long)K * ES);
      greg = buffer_load16(rg, uint32_t((k0 + a_c * CE) * ES));
    }
  };

  auto sstore = [&](int buf) {
    char* stage = smem + buf * C::STAGE * ES;
    if constexpr (!C::F32) {
      uint16_t* As = reinterpret_cast<uint16_t*>(stage);
      uint16_t* Bs = As + C::A_ELEMS;
      float gf[8];
      if (C::RMS) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gf[2 * w] = bf16_lo(greg[w]);
          gf[2 * w + 1] = bf16_hi(greg[w]);
        }
      }
#pragma unroll
      for (int i = 0; i < C::A_CH; ++i) {
        u32x4_t x = areg[i];
        if (C::RMS) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float lo = bf16_lo(x[w]), hi = bf16_hi(x[w]);
            ss[i] = fmaf(lo, lo, ss[i]);
            ss[i] = fmaf(hi, hi, ss[i]);
            x[w] = pack_bf16x2(lo * gf[2 * w], hi * gf[2 * w + 1]);
          }
        }
        *reinterpret_cast<u32x4_t*>(As + (a_r + i * C::A_RSTEP) * SA + a_c * 8) = x;
      }
#pragma unroll
      for (int i = 0; i < C::B_CH; ++i) {
        if (C::BKN)
          *reinterpret_cast<u32x4_t*>(Bs + (b_r + i * C::B_RSTEP) * SB + b_c * 8) = breg[i];
        else
          *reinterpret_cast<u32x4_t*>(Bs + (b_r + i * C::B_RSTEP) * SA + b_c * 8) = breg[i];
      }
    } else {
      float* As = reinterpret_cast<float*>(stage);
      float* Bs = As + C::A_ELEMS;
      float gf[4];
      if (C::RMS) {
#pragma unroll
        for (int w = 0; w < 4; ++w) gf[w] = __uint_as_float(greg[w]);
      }
#pragma unroll
      for (int i = 0; i < C::A_CH; ++i) {
        float* dst = As + (a_r + i * C::A_RSTEP) * SA + a_c * 4;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float x = __uint_as_float(areg[i][w]);
          if (C::RMS) {
            ss[i] = fmaf(x, x, ss[i]);
            x = x * gf[w];
          }
          dst[w] = x;
        }
      }
#pragma unroll
      for (int i = 0; i < C::B_CH; ++i) {
        if (C::BKN) {
          *reinterpret_cast<u32x4_t*>(Bs + (b_r + i * C::B_RSTEP) * SB + b_c * 4) = breg[i];
        } else {
          float* dst = Bs + (b_r + i * C::B_RSTEP) * SA + b_c * 4;
#pragma unroll
          for (int w = 0; w < 4; ++w) dst[w] = __uint_as_float(breg[i][w]);
        }
      }
    }
  };

  auto compute = [&](int buf) {
    const char* stage = smem + buf * C::STAGE * ES;
    if constexpr (!C::F32) {
      const uint16_t* As = reinterpret_cast<const uint16_t*>(stage);
      const uint16_t* Bs = As + C::A_ELEMS;
      const int l32 = lane & 31, hi = lane >> 5;
      const int G = lane >> 4, s = lane & 15;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8_t xf[MI], wf[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          xf[mi] = *reinterpret_cast<const bf16x8_t*>(As + (wm * C::WTM + 32 * mi + l32) * SA + 16 * kk + 8 * hi);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          if (C::BKN) {
            // transposing LDS read: lane (G, s) supplies row 16kk + 8(G/2) + 4h + s/4 at
            // column 32ni + 16(G%2) + 4(s%4); lane s of each 16-lane group receives the
            // 4 K-consecutive values of column 16(G%2) + s.
            const int krow = 16 * kk + 8 * (G >> 1) + (s >> 2);
            const int ncol = wn * C::WTN + 32 * ni + 16 * (G & 1) + 4 * (s & 3);
            typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Bs + krow * SB + ncol));
            const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(Bs + (krow + 4) * SB + ncol));
            wf[ni] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            wf[ni] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn * C::WTN + 32 * ni + l32) * SA + 16 * kk + 8 * hi);
          }
        }
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ni], xf[mi], acc[mi][ni], 0, 0, 0);
      }
    } else {
      const float* As = reinterpret_cast<const float*>(stage);
      const float* Bs = As + C::A_ELEMS;
      const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        float xf[MI], wf[NI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) xf[mi] = As[(wm * C::WTM + 32 * mi + l32) * SA + 2 * kk + hi];
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          wf[ni] = C::BKN ? Bs[(2 * kk + hi) * SB + wn * C::WTN + 32 * ni + l32]
                          : Bs[(wn * C::WTN + 32 * ni + l32) * SA + 2 * kk + hi];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(wf[ni], xf[mi], acc[mi][ni], 0, 0, 0);
      }
    }
  };

  // ---- main loop: one barrier per K step ----
  if (KT > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < KT;
      if (more) gload(kt + 1);
      compute(cur);
      if (more) sstore(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue ----
  float* epi = reinterpret_cast<float*>(smem);
  float* rinv = epi;                 // [BM]
  float* red = epi + BM;             // [MAX_RED][WN][BM]
  int* flag = reinterpret_cast<int*>(epi + BM + CODA_MAX_REDUCTIONS * C::WN * BM);

  Geo<C> g;
  g.M = M;
  g.lane = lane;
  g.wn = wn;
  g.mloc0 = wm * C::WTM;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) g.m[mi] = m0 + wm * C::WTM + 32 * mi + (lane & 31);
  g.nb = n0 + wn * C::WTN + 4 * (lane >> 5);

  if (C::RMS) {
    // rows a_r + i*A_RSTEP are shared by the KCH consecutive lanes with equal a_r
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      float v = ss[i];
#pragma unroll
      for (int off = 1; off < KCH; off <<= 1) v += __shfl_xor(v, off);
      if (a_c == 0) rinv[a_r + i * C::A_RSTEP] = 1.0f / sqrtf(v / float(K) + a->eps);
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const float r = rinv[wm * C::WTM + 32 * mi + (lane & 31)];
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[mi][ni][q] *= r;
    }
  }

  static_for<0, MI * NI>([&](auto blk) {
    constexpr int mi = decltype(blk)::value / NI;
    constexpr int ni = decltype(blk)::value % NI;
    const int o = run_ops<C, false>(acc[mi][ni], a, 0, g, mi, ni, red);
    if (o < a->n_ops) {   // SWIGLU_PAIR
      swiglu_pair_acc(acc[mi][ni]);
      run_ops<C, true>(acc[mi][ni], a, o + 1, g, mi, ni, red);
      store_d<C, true>(acc[mi][ni], a, g, mi, ni);
    } else {
      store_d<C, false>(acc[mi][ni], a, g, mi, ni);
    }
  });

  if (a->n_red > 0) {
    __syncthreads();
    const bool multi = a->grid_n > 1;
    for (int q = 0; q < a->n_ops; ++q) {
      const __attribute__((address_space(4))) DevOp& op = a->ops[q];
      if (op.kind < CODA_OP_ROW_SUM) continue;
      const int s = op.red_slot;
      for (int t = tid; t < BM; t += C::NT) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < C::WN; ++w) v += red[(s * C::WN + w) * BM + t];
        const int row = m0 + t;
        if (row < M) {
          if (!multi) {
            write_reduction(op, row, v);
          } else {
            float* dst = a->partials + ((long long)s * a->grid_n + tile_n) * M + row;
            __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    if (multi) {
      __threadfence();
      __syncthreads();
      if (tid == 0) {
        const unsigned old = atomicAdd(a->counters + tile_m, 1u);
        *flag = (old == unsigned(a->grid_n - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (*flag) {
        __threadfence();
        for (int q = 0; q < a->n_ops; ++q) {
          const __attribute__((address_space(4))) DevOp& op = a->ops[q];
          if (op.kind < CODA_OP_ROW_SUM) continue;
          const int s = op.red_slot;
          for (int t = tid; t < BM; t += C::NT) {
            const int row = m0 + t;
            if (row >= M) continue;
            float v = 0.0f;
            for (int tn = 0; tn < a->grid_n; ++tn)
              v += __hip_atomic_load(a->partials + ((long long)s * a->grid_n + tn) * M + row, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
            write_reduction(op, row, v);
          }
        }
        if (tid == 0) atomicExch(a->counters + tile_m, 0u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <class C>
int launch_cfg(const FusedArgs& args, int64_t nwg, hipStream_t stream) {
  hipLaunchKernelGGL(fused_kernel<C>, dim3((unsigned)nwg), dim3(C::NT), 0, stream, args);
  return hipGetLastError() == hipSuccess ? CODA_OK : CODA_ERR_HIP;
}

template <int BM, int BN, int BK, int WM, int WN, bool F32>
int launch_variants(const FusedArgs& args, int64_t nwg, bool bkn, bool rms, hipStream_t s) {
  if (bkn) {
    return rms ? launch_cfg<Cfg<BM, BN, BK, WM, WN, F32, true, true>>(args, nwg, s)
               : launch_cfg<Cfg<BM, BN, BK, WM, WN, F32, true, false>>(args, nwg, s);
  }
  return rms ? launch_cfg<Cfg<BM, BN, BK, WM, WN, F32, false, true>>(args, nwg, s)
             : launch_cfg<Cfg<BM, BN, BK, WM, WN, F32, false, false>>(args, nwg, s);
}

// one function per compiled tile configuration (defined in coda_fused_t*.hip)
int launch_tile1(const FusedArgs& a, int64_t nwg, bool bkn, bool rms, hipStream_t s);
int launch_tile2(const FusedArgs& a, int64_t nwg, bool bkn, bool rms, hipStream_t s);
int launch_tile3(const FusedArgs& a, int64_t nwg, bool bkn, bool rms, hipStream_t s);
int launch_tile4(const FusedArgs& a, int64_t nwg, bool bkn, bool rms, hipStream_t s);
int launch_tile_f32(const FusedArgs& a, int64_t nwg, bool bkn, bool rms, hipStream_t s);

}  // namespace dev
}  // namespace coda
