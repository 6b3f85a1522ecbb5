// Fused GEMM + ordered epilogue for gfx950.
//
// One workgroup computes one bm x bn output tile; its waves form a wm x wn grid
// over the tile.  The tile is computed transposed (MFMA rows = columns of D):
// the W fragment is the MFMA A operand and the X fragment the MFMA B operand,
// so each lane's accumulators hold runs of 4 consecutive output columns.
//
// Main loop (bf16 operands), two LDS stages, one barrier per K step of 64:
//   * operand tiles go global -> LDS with buffer loads that write LDS directly
//     (16 bytes per lane); out-of-range offsets read as zero, which fills the
//     M / N / K tails;
//   * LDS tiles are XOR-swizzled at 16-byte granularity so the MFMA operand
//     reads (ds_read_b128 for K-contiguous tiles, the transposing
//     ds_read_b64_tr_b16 for the N-contiguous W tile) are bank-conflict free:
//     ds_read_b128 serves 16 lanes (256 bytes) per cycle on gfx950, so the
//     16 rows a K-contiguous read touches must land on distinct 16-byte bank
//     slots, which the row swizzle swz(r) = (r & 7) ^ ((r >> 3) & 1) provides;
//   * MFMA fragments for the next k16 step are read while the current step's
//     v_mfma_f32_32x32x16_bf16 instructions run.
// A stored [K x M] (the X^T of a weight gradient) is staged like the
// N-contiguous W tile and read with the same transposing LDS reads.
// Deferred row norms (the per-row factors of a row-wise norm moved past the
// projection: the "augment_me" comment on the zeli.app page; the
// agentlenshq.com page, "CODA's approach"), one compile-time mode each:
//   * gain in the loop (RMS, LayerNorm): raw A comes into registers one K
//     step ahead; each wave multiplies its chunks by gamma[k], rounds them to
//     bf16, writes them into the stage and adds the raw squares (and, for
//     LayerNorm, the values, both about a per-row shift) to fp32 per-row sums;
//   * gain folded into B (RMS, LayerNorm): A reaches the MFMAs unchanged and
//     the sums come from the X fragments the MFMAs read, between the MFMAs;
//   * row sums of squares given (RMS with the gain in B): the plain main loop.
// The epilogue scales each row by 1/rms (RMS) or applies
// rstd * (acc - mean * u) with u the column sums of the gained weights
// (LayerNorm).  fp32 operands (a small tile, v_mfma_f32_32x32x2f32) use a
// register-staged, padded LDS layout.
//
// Epilogue: each wave moves its accumulators, one 32-row block at a time,
// through a private LDS region into a row-major layout where every lane owns
// chunks of 8 consecutive columns.  The op list then runs in order on fp32
// values (d9bl.com page, section 3.2), side operands are read and D is written
// as whole 16-byte row chunks, and row reductions combine the lanes of a row,
// then the waves of the tile through LDS, then the workgroups of a tile row
// through a workspace of partial sums finished by the last workgroup to arrive
// (a fixed summation order, so results are bitwise repeatable).  Column
// reductions combine the lanes of a column, then the row blocks of the tile in
// LDS, then the workgroups of a tile column the same way.
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
// range of logical tiles (of the first nwg), and order the logical tiles in
// groups of 8 tile rows (column-major inside a group), so concurrently
// resident tiles on one XCD share A row panels and B column panels in that
// XCD's L2.
__device__ __forceinline__ int xcd_logical(int bid, int nwg) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = nwg >> 3, r = nwg & 7;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}
__device__ __forceinline__ void tile_of(int L, int gm, int gn, int& tm, int& tn) {
  constexpr int G = 8;
  const int group = L / (G * gn);
  const int first = group * G;
  const int gsz = min(gm - first, G);
  const int rem = L - group * G * gn;
  tm = first + rem % gsz;
  tn = rem / gsz;
}

// The kernel reads its argument block straight from the kernarg segment
// (constant address space): the op list is indexed with a runtime op number,
// and indexing a by-value parameter would make the compiler copy the whole
// block to per-lane scratch memory.
typedef const __attribute__((address_space(4))) FusedArgs* KArgs;
typedef const __attribute__((address_space(4))) DevOp& KOp;
typedef __attribute__((address_space(3))) void* LdsPtr;
typedef __attribute__((address_space(3))) i16x4_t LdsI16x4;

// deferred row norm in front of the GEMM: none, RMSNorm (gain applied to A in
// the main loop), LayerNorm, RMSNorm with the gain already folded into B's rows
constexpr int kNormNone = 0, kNormRms = 1, kNormLn = 2, kNormRmsB = 3;
// RMSNorm with the gain in B and the row sums of squares given (a cross-layer
// chain): the main loop is the plain GEMM
constexpr int kNormRmsGiven = 4;
// LayerNorm with the gain folded into B: row sums and sums of squares (about a
// per-row shift) from the X fragments, like kNormRmsB
constexpr int kNormLnB = 5;
// LayerNorm with the gain in B and the row sums and sums of squares given
constexpr int kNormLnGiven = 6;

template <int BM_, int BN_, int WM_, int WN_, bool F32_, bool BKN_, int NORM_, bool AKM_ = false, bool EXT_ = true,
          bool SIDE_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool F32 = F32_, BKN = BKN_;
  // EXT: the kernel carries the epilogue ops of the backward set (column
  // reductions, ROW_DOT, RMS_BWD, RMS_DGAMMA); lists without them run a
  // variant compiled without their code and registers
  static constexpr bool EXT = EXT_;
  // SIDE: the list's first bf16 side matrix (ADD_MAT / MUL_DGELU_TANH before
  // any SWIGLU_PAIR) is read one 32-row block ahead into registers; variants
  // without it read side matrices chunk by chunk where they are used, and
  // carry no prefetch registers
  static constexpr bool SIDE = SIDE_;
  // AKM: A stored [K x M] (M contiguous) and used transposed, as X^T in the
  // weight gradient X^T dY; its tile is staged and read like an N-major W tile
  static constexpr bool AKM = AKM_;
  static_assert(!AKM || (!F32 && NORM_ == kNormNone), "A stored [K x M]: bf16 operands, no row norm");
  static constexpr int KM_CPR = BM / 8;               // 16-byte chunks per row of an M-major A tile
  static constexpr int KM_RPB = 64 / KM_CPR;          // rows of it per 1 KB block
  // RMS: gain applied to A in the main loop, sums of squares, a row scale in
  // the epilogue; LN: additionally row sums and the mean term of the deferred
  // LayerNorm; SSF: A goes to the MFMAs unchanged (the gain is in B) and the
  // sums of squares come from the X fragments the MFMAs read
  static constexpr bool RMS = NORM_ == kNormRms || NORM_ == kNormLn, LN = NORM_ == kNormLn;
  static constexpr bool LNF = NORM_ == kNormLnB;
  static constexpr bool SSF = NORM_ == kNormRmsB || LNF;   // sums from the X fragments
  static constexpr bool LNE = LN || LNF || NORM_ == kNormLnGiven;   // LayerNorm epilogue
  static constexpr bool GIVEN = NORM_ == kNormRmsGiven || NORM_ == kNormLnGiven;
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  // the bf16 128 x 128 tile of 4 waves runs two workgroups per CU: two waves
  // per SIMD, so VGPRs + AGPRs must stay within 256 (the epilogue's rarely
  // used ops may not push the whole kernel to one wave per SIMD)
  static constexpr int MIN_WAVES_PER_EU = (BM == 128 && BN == 128 && NW == 4 && !F32) ? 2 : 1;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int BK = F32 ? 32 : 64;
  static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be a multiple of 32");

  // ---- bf16 main loop: swizzled, unpadded stages ----
  static constexpr int A_BYTES = BM * 128;            // [BM][64] bf16
  static constexpr int B_BYTES = BN * 128;            // [64][BN] or [BN][64] bf16
  static constexpr int A_BLK = BM / 8;                // 1 KB blocks of A per stage
  static constexpr int B_BLK = BN / 8;
  static_assert(F32 || (A_BLK % NW == 0 && B_BLK % NW == 0), "1 KB blocks must split over the waves");
  static constexpr int A_BPW = A_BLK / NW, B_BPW = B_BLK / NW;   // blocks per wave
  static constexpr int KN_CPR = BN / 8;               // 16-byte chunks per row of an N-major W tile
  static constexpr int KN_RPB = 64 / KN_CPR;          // rows of it per 1 KB block

  // ---- fp32 main loop: register staged, padded ----
  static constexpr int SA32 = BK + 1, SB32 = BN + 4;
  static constexpr int A32_CH = BM * (BK / 4) / NT;    // 16-byte chunks per thread
  static constexpr int B32_CH = BN * (BK / 4) / NT;

  static constexpr int STAGE_BYTES =
      F32 ? (BM * SA32 + (BKN ? BK * SB32 : BN * SA32)) * 4 : A_BYTES + B_BYTES;

  // ---- epilogue ----
  static constexpr int CPR = WTN / 8;                 // 8-column chunks per wave-tile row
  static constexpr int CPL = 32 * CPR / 64;           // chunks per lane per 32-row block
  static constexpr int RSTEP = 64 / CPR;              // rows between a lane's chunks
  static constexpr int REGION_BYTES = 32 * WTN * 4;   // per-wave fp32 staging of one block
  // LDS is two arrays, one per main-loop stage (distinct objects, so the
  // compiler does not make reads of one stage wait for direct-to-LDS loads
  // into the other); the epilogue reuses array 0 for the per-wave regions and
  // array 1 for the reduction partials, 1/rms and a flag.
  static constexpr int EPI_RED_OFF = 0;                // in array 1
  static constexpr int EPI_RINV_OFF = EPI_RED_OFF + CODA_MAX_REDUCTIONS * WN * BM * 4;
  static constexpr int EPI_RMU_OFF = EPI_RINV_OFF + BM * 4;   // LN: mean * rstd per row
  static constexpr int EPI_FLAG_OFF = EPI_RMU_OFF + BM * 4;
  // column reductions: per-block column partials [slot][wm][mi][BN]
  static constexpr int EPI_COL_OFF = EPI_FLAG_OFF + 16;
  static constexpr int EPI_END = EPI_COL_OFF + CODA_MAX_COL_REDUCTIONS * WM * MI * BN * 4;
  static constexpr int ARR0_BYTES = STAGE_BYTES > NW * REGION_BYTES ? STAGE_BYTES : NW * REGION_BYTES;
  static constexpr int ARR1_BYTES = STAGE_BYTES > EPI_END ? STAGE_BYTES : EPI_END;
  // SSF: per-row partial sums of squares, one row of BM per wave column
  // (LNF: then the row sums [WN][BM] and the per-row shift [BM])
  static constexpr int SS_BYTES = (SSF && !F32) ? (LNF ? 2 * WN + 1 : WN) * BM * 4 : 16;
  // (the compiler drops the sums array from variants without SSF)
  static_assert(ARR0_BYTES + ARR1_BYTES + (SSF ? SS_BYTES : 0) <= 160 * 1024, "LDS budget");
  static_assert(CPR >= 4 && CPR <= 16 && (CPR & (CPR - 1)) == 0, "epilogue lane layout");
};

// ---------------------------------------------------------------------------
// epilogue: ops on a lane's row chunks (values v[j][0..7] = columns
// col[j] .. col[j]+7 of row row[j]; after SWIGLU_PAIR the first 4 hold the
// 4 output columns col[j]/2 .. col[j]/2 + 3)
// ---------------------------------------------------------------------------

template <int CPL>
struct Chunks {
  float v[CPL][8];
  int row[CPL];     // global row
  int mloc[CPL];    // row within the tile
  int col;          // global first column of the lane's chunk (same for every j)
};

template <bool PAIRED>
__device__ __forceinline__ void load_cols(const void* p, int dtype, long long col, long long width, float (&x)[8]) {
  if (PAIRED) {
    float t[4];
    load4(p, dtype, col, width, t);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = t[e];
#pragma unroll
    for (int e = 4; e < 8; ++e) x[e] = 0.0f;
  } else {
    float t[4], u[4];
    load4(p, dtype, col, width, t);
    load4(p, dtype, col + 4, width, u);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = t[e];
      x[4 + e] = u[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Lane reductions with DPP row moves (inside the VALU) where the partner lane
// is in the same row of 16, LDS permutes across rows.  The additions pair the
// lanes as the xor butterfly over the same offsets does, so the sums are the
// same bit for bit.  (gfx950's permlane16/32 swaps would serve across rows,
// but the compiler's builtin returns the first half of the swap for both of
// its results, checked on the GPU, so they are not used.)
// ---------------------------------------------------------------------------
template <int ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]: lane i <- lane i ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]: lane i <- lane i ^ 2
constexpr int kDppHalfMirror = 0x141; // lane i of 8 <- lane 7 - i
constexpr int kDppMirror = 0x140;     // lane i of 16 <- lane 15 - i
constexpr int kDppRor8 = 0x128;       // lane i of 16 <- lane (i + 8) % 16 = lane i ^ 8

// sum over each group of n consecutive lanes (n = 4, 8 or 16), in every lane;
// after the quad sums, the mirrors bring the other half's (equal) sums
template <int n>
__device__ __forceinline__ float group_sum(float p) {
  static_assert(n == 4 || n == 8 || n == 16, "group of 4, 8 or 16 lanes");
  p += dpp<kDppXor1>(p);
  p += dpp<kDppXor2>(p);
  if constexpr (n >= 8) p += dpp<kDppHalfMirror>(p);
  if constexpr (n >= 16) p += dpp<kDppMirror>(p);
  return p;
}

// sum over the lanes l with the same l % n (n = 4, 8 or 16), in every lane
template <int n>
__device__ __forceinline__ float stride_sum(float p) {
  static_assert(n == 4 || n == 8 || n == 16, "stride of 4, 8 or 16 lanes");
  if constexpr (n == 4) p += __shfl_xor(p, 4);
  if constexpr (n <= 8) p += dpp<kDppRor8>(p);
  p += __shfl_xor(p, 16);
  return p + __shfl_xor(p, 32);
}

__device__ __forceinline__ bool is_row_reduction(int kind) {
  return (kind >= CODA_OP_ROW_SUM && kind <= CODA_OP_ROW_MEAN) || kind == CODA_OP_ROW_DOT;
}

__device__ __forceinline__ bool is_col_reduction(int kind) {
  return kind == CODA_OP_COL_SUM || kind == CODA_OP_COL_SUMSQ || kind == CODA_OP_RMS_DGAMMA;
}

// Applies ops[o..] until the end of the list or a SWIGLU_PAIR (returned index).
// pf: the prefetched rows of side matrix op pf_op (SIDE variants); pf_used()
// runs as soon as they are consumed, and issues the next block's prefetch into
// the same registers
template <class C, bool PAIRED, class PfUsed>
__device__ __forceinline__ int run_ops(Chunks<C::CPL>& ch, KArgs a, int o, int M, int lane, int wn, float* red,
                                       int pf_op, const u32x4_t (&pf)[C::CPL], float* colp, int wm, int mi,
                                       int cv_op, const float (&cv)[8], PfUsed&& pf_used) {
  constexpr int CPL = C::CPL;
  constexpr int EPC = PAIRED ? 4 : 8;   // live values per chunk
  const int col = PAIRED ? ch.col >> 1 : ch.col;
  for (; o < a->n_ops; ++o) {
    KOp op = a->ops[o];
    const int kind = op.kind;
    if (!PAIRED && kind == CODA_OP_SWIGLU_PAIR) return o;
    const int width = op.width;
    switch (kind) {
      case CODA_OP_SCALE: {
        const float s = op.scalar;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < EPC; ++e) ch.v[j][e] *= s;
        break;
      }
      case CODA_OP_SCALE_ROW:
      case CODA_OP_ADD_ROW: {
        const bool add = kind == CODA_OP_ADD_ROW;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const float x = ch.row[j] < M ? load_elem(op.in, op.dtype, ch.row[j]) : 0.0f;
#pragma unroll
          for (int e = 0; e < EPC; ++e) ch.v[j][e] = add ? ch.v[j][e] + x : ch.v[j][e] * x;
        }
        break;
      }
      case CODA_OP_SCALE_COL:
      case CODA_OP_ADD_COL: {
        const bool add = kind == CODA_OP_ADD_COL;
        float x[8];
        if (!PAIRED && o == cv_op) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = cv[e];   // loaded once per tile
        } else {
          load_cols<PAIRED>(op.in, op.dtype, col, width, x);
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < EPC; ++e) ch.v[j][e] = add ? ch.v[j][e] + x[e] : ch.v[j][e] * x[e];
        break;
      }
      case CODA_OP_ADD_MAT:
      case CODA_OP_MUL_DGELU_TANH: {
        // v + beta x, or v * GELU_tanh'(x): the variant is a compile-time flag,
        // and the side values are applied chunk by chunk so that no whole
        // block of them is live
        auto side_mat = [&](auto addc) {
          constexpr bool ADDM = decltype(addc)::value;
          const float beta = op.scalar;
          auto apply = [&](float& v, float x) {
            if constexpr (ADDM) v = v + beta * x;
            else v = v * gelu_tanh_grad_f(x);
          };
          if (C::SIDE && !PAIRED && o == pf_op) {
            // prefetched bf16 row chunks
#pragma unroll
            for (int j = 0; j < CPL; ++j)
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                apply(ch.v[j][2 * w], bf16_lo(pf[j][w]));
                apply(ch.v[j][2 * w + 1], bf16_hi(pf[j][w]));
              }
            pf_used();
          } else {
            const int esz = op.dtype == CODA_BF16 ? 2 : 4;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              float x[8];
              if (ch.row[j] < M) {
                load_cols<PAIRED>(static_cast<const char*>(op.in) + (long long)ch.row[j] * op.ld * esz, op.dtype,
                                  col, width, x);
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
              }
#pragma unroll
              for (int e = 0; e < EPC; ++e) apply(ch.v[j][e], x[e]);
            }
          }
        };
        if (kind == CODA_OP_ADD_MAT) side_mat(std::true_type{});
        else side_mat(std::false_type{});
        break;
      }
      case CODA_OP_DROPOUT: {
        // the lane's chunk of each row: 8 columns (4 after SWIGLU_PAIR), one
        // generator block
#pragma unroll
        for (int j = 0; j < CPL; ++j) dropout_values<EPC>(ch.v[j], ch.row[j], col, op.thr, op.scalar, op.seed, op.offset);
        break;
      }
      case CODA_OP_GELU_TANH:
      case CODA_OP_SILU: {
        const bool gelu = kind == CODA_OP_GELU_TANH;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int e = 0; e < EPC; ++e) ch.v[j][e] = gelu ? gelu_tanh_f(ch.v[j][e]) : silu_f(ch.v[j][e]);
        break;
      }
      case CODA_OP_ROW_SUM:
      case CODA_OP_ROW_MEAN:
      case CODA_OP_ROW_SUMSQ: {
        const bool sq = kind == CODA_OP_ROW_SUMSQ;
        float* dst = red + (op.red_slot * C::WN + wn) * C::BM;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          float p = 0.0f;
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const float x = ch.v[j][e];
            p += (col + e < width) ? (sq ? x * x : x) : 0.0f;
          }
          // the CPR lanes of a row are consecutive
          p = group_sum<C::CPR>(p);
          if ((lane & (C::CPR - 1)) == 0) dst[ch.mloc[j]] = p;
        }
        break;
      }
      case CODA_OP_ROW_DOT: {
        if constexpr (C::EXT) {
          // ROW_SUM of the running value times the matrix operand
          const int esz = op.dtype == CODA_BF16 ? 2 : 4;
          float* dst = red + (op.red_slot * C::WN + wn) * C::BM;
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            float x[8];
            if (ch.row[j] < M) {
              load_cols<PAIRED>(static_cast<const char*>(op.in) + (long long)ch.row[j] * op.ld * esz, op.dtype, col,
                                width, x);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
            float p = 0.0f;
#pragma unroll
            for (int e = 0; e < EPC; ++e) p += (col + e < width) ? ch.v[j][e] * x[e] : 0.0f;
            p = group_sum<C::CPR>(p);
            if ((lane & (C::CPR - 1)) == 0) dst[ch.mloc[j]] = p;
          }
        }
        break;
      }
      case CODA_OP_RMS_BWD: {
        if constexpr (C::EXT) {
          // v = gamma_j v / r_i - x_ij t_i / (width r_i^2), r_i^2 = sumsq_i / width + eps
          const int esz = op.dtype == CODA_BF16 ? 2 : 4;
          const float inv_w = 1.0f / float(width);
          float g[8];
          load_cols<PAIRED>(op.in2, op.dtype, col, width, g);
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            float x[8];
            float rinv = 0.0f, coef = 0.0f;
            if (ch.row[j] < M) {
              load_cols<PAIRED>(static_cast<const char*>(op.in) + (long long)ch.row[j] * op.ld * esz, op.dtype, col,
                                width, x);
              const long long ro = (long long)ch.row[j] * op.row_ld;
              const float r2 = op.row_ss[ro] * inv_w + op.scalar;
              rinv = 1.0f / sqrtf(r2);
              coef = op.row_s[ro] * inv_w / r2;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) ch.v[j][e] = g[e] * ch.v[j][e] * rinv - x[e] * coef;
          }
        }
        break;
      }
      case CODA_OP_RMS_DGAMMA: {
        if constexpr (C::EXT) {
          // column sums of v * x / r_i, r_i^2 = sumsq_i / width + eps, reduced as COL_SUM
          const int esz = op.dtype == CODA_BF16 ? 2 : 4;
          const float inv_w = 1.0f / float(width);
          float p[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) p[e] = 0.0f;
#pragma unroll
          for (int j = 0; j < CPL; ++j)
            if (ch.row[j] < M) {
              float x[8];
              load_cols<PAIRED>(static_cast<const char*>(op.in) + (long long)ch.row[j] * op.ld * esz, op.dtype, col,
                                width, x);
              const float rinv = 1.0f / sqrtf(op.row_ss[(long long)ch.row[j] * op.row_ld] * inv_w + op.scalar);
#pragma unroll
              for (int e = 0; e < EPC; ++e) p[e] += ch.v[j][e] * x[e] * rinv;
            }
#pragma unroll
          for (int e = 0; e < EPC; ++e) p[e] = stride_sum<C::CPR>(p[e]);
          if (lane < C::CPR) {
            const int tcol = wn * C::WTN + 8 * lane;
            float* dst = colp + ((op.red_slot * C::WM + wm) * C::MI + mi) * C::BN + (PAIRED ? tcol / 2 : tcol);
#pragma unroll
            for (int e = 0; e < EPC; ++e) dst[e] = p[e];
          }
        }
        break;
      }
      case CODA_OP_COL_SUM:
      case CODA_OP_COL_SUMSQ: {
        if constexpr (C::EXT) {
          // the lane's rows, then the lanes that hold the same columns (lane %
          // CPR): the wave's partial for its 32-row block, kept per block in LDS
          const bool sq = kind == CODA_OP_COL_SUMSQ;
          float p[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) p[e] = 0.0f;
#pragma unroll
          for (int j = 0; j < CPL; ++j)
            if (ch.row[j] < M) {
#pragma unroll
              for (int e = 0; e < EPC; ++e) p[e] += sq ? ch.v[j][e] * ch.v[j][e] : ch.v[j][e];
            }
#pragma unroll
          for (int e = 0; e < EPC; ++e) p[e] = stride_sum<C::CPR>(p[e]);
          if (lane < C::CPR) {
            const int tcol = wn * C::WTN + 8 * lane;   // tile-local first column of the chunk
            float* dst = colp + ((op.red_slot * C::WM + wm) * C::MI + mi) * C::BN + (PAIRED ? tcol / 2 : tcol);
#pragma unroll
            for (int e = 0; e < EPC; ++e) dst[e] = p[e];
          }
        }
        break;
      }
      default:
        break;
    }
  }
  return o;
}

template <class C>
__device__ __forceinline__ void swiglu_chunks(Chunks<C::CPL>& ch) {
#pragma unroll
  for (int j = 0; j < C::CPL; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) ch.v[j][e] = silu_f(ch.v[j][2 * e]) * ch.v[j][2 * e + 1];
}

template <class C, bool PAIRED>
__device__ __forceinline__ void store_chunks(const Chunks<C::CPL>& ch, KArgs a, int M) {
  const int width = a->out_width;
  const int col = PAIRED ? ch.col >> 1 : ch.col;
  constexpr int EPC = PAIRED ? 4 : 8;
#pragma unroll
  for (int j = 0; j < C::CPL; ++j) {
    if (ch.row[j] >= M) continue;
    const long long off = (long long)ch.row[j] * a->ldd + col;
    if (a->d_dtype == CODA_BF16) {
      uint16_t* d = static_cast<uint16_t*>(a->D) + off;
      if (col + EPC - 1 < width) {
        if (PAIRED) {
          u32x2_t w;
          w[0] = pack_bf16x2(ch.v[j][0], ch.v[j][1]);
          w[1] = pack_bf16x2(ch.v[j][2], ch.v[j][3]);
          *reinterpret_cast<u32x2_t*>(d) = w;
        } else {
          u32x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(ch.v[j][2 * e], ch.v[j][2 * e + 1]);
          *reinterpret_cast<u32x4_t*>(d) = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (col + e < width) d[e] = f32_to_bf16_bits(ch.v[j][e]);
      }
    } else {
      float* d = static_cast<float*>(a->D) + off;
      if (col + EPC - 1 < width) {
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          f32x4_t w;
          w[0] = ch.v[j][e]; w[1] = ch.v[j][e + 1]; w[2] = ch.v[j][e + 2]; w[3] = ch.v[j][e + 3];
          *reinterpret_cast<f32x4_t*>(d + e) = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (col + e < width) d[e] = ch.v[j][e];
      }
    }
  }
}

// Parts of a tile split over K: at most this many (the plan's limit)
constexpr int kMaxSplitParts = 4;
// cache policy of a buffer load: sc1, coherent at agent scope (the policy of
// this target's agent-scope atomic loads)
constexpr int kCachePolicySc1 = 16;

// Register pairs per round trip when a split tile's partials come through LDS:
// the largest of 8, 4, 2, 1 whose chunk (pairs x threads x 8 bytes) fits a
// part's LDS slot and divides the pairs
constexpr int split_chunk_pairs(int slot_bytes, int nt, int pairs) {
  int c = 8;
  while (c > 1 && (c * nt * 8 > slot_bytes || pairs % c != 0)) c /= 2;
  return c;
}

// The sum p[0] + p[stride] + ... + p[(n - 1) stride], added in index order (so
// the result does not depend on which workgroup adds), read with agent-scope
// loads.  Those loads go to the memory side of the XCD L2s, about a
// microsecond each, so they go out eight at a time ahead of their adds: one
// round trip per eight partials, not one per partial.  (Adding 0 in place of a
// missing partial leaves the sum unchanged: it starts at +0 and never becomes
// -0.)
__device__ __forceinline__ float sum_partials(const float* p, long long stride, int n) {
  float v = 0.0f;
  for (int i = 0; i < n; i += 8) {
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t[j] = i + j < n ? __hip_atomic_load(p + (long long)(i + j) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) v += t[j];
  }
  return v;
}

__device__ __forceinline__ void write_reduction(KOp op, int row, float v) {
  if (op.kind == CODA_OP_ROW_MEAN) v = v / float(op.width);
  op.out[(long long)row * op.out_stride] = v;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <class C>
__global__ void __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::MIN_WAVES_PER_EU)))
fused_kernel(FusedArgs args) {
  (void)args;
  const KArgs a = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, MI = C::MI, NI = C::NI;
  __shared__ __attribute__((aligned(1024))) char smem0[C::ARR0_BYTES];
  __shared__ __attribute__((aligned(1024))) char smem1[C::ARR1_BYTES];
  __shared__ __attribute__((aligned(16))) float smem_ss[C::SS_BYTES / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int l32 = lane & 31, hi = lane >> 5;
  const int swz_l = (l32 & 7) ^ ((l32 >> 3) & 1);   // LDS row swizzle; depends on the row mod 16 only

  // work item: a whole tile, or one part (over K) of a tile of the last round
  int tile_m, tile_n;
  int kt_lo = 0;      // first K step of this workgroup
  int split = -1;     // index of the split tile, -1 for a whole tile
  int part = 0;       // part of the split tile
  const int KT_all = a->k_steps;
  int KT = KT_all;    // K steps of this workgroup
  {
    const int bid = blockIdx.x;
    int L;
    if (bid < a->full_tiles) {
      L = xcd_logical(bid, a->full_tiles);
    } else {
      const int u = bid - a->full_tiles;
      split = u / a->split_s;
      part = u % a->split_s;
      L = a->full_tiles + split;
      kt_lo = (KT_all * part) / a->split_s;
      KT = (KT_all * (part + 1)) / a->split_s - kt_lo;
    }
    tile_of(L, a->grid_m, a->grid_n, tile_m, tile_n);
  }
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int M = a->M, N = a->N, K = a->K;
  const long long lda = a->lda, ldb = a->ldb;

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

  // per-row sums of squares (RMS, LN) and sums (LN) of the A values this lane
  // converts; with bf16 operands LN shifts each row by its first element first
  // SSF: one sum per k16 slice and per row block the wave takes at that slice
  constexpr int NSS = C::F32 ? C::A32_CH : (C::SSF ? 4 * (MI / C::WN) : C::A_BPW);
  float ss[NSS], sx[NSS], sh[NSS];
#pragma unroll
  for (int i = 0; i < NSS; ++i) ss[i] = sx[i] = sh[i] = 0.0f;

  if constexpr (!C::F32) {
    // ================= bf16 main loop =================
    const char* Abase = C::AKM ? static_cast<const char*>(a->A) + (long long)m0 * 2
                               : static_cast<const char*>(a->A) + (long long)m0 * lda * 2;
    const char* Bbase = C::BKN ? static_cast<const char*>(a->B) + (long long)n0 * 2
                               : static_cast<const char*>(a->B) + (long long)n0 * ldb * 2;
    const long long a_ext0 = C::AKM ? ((long long)(K - 1) * lda + (M - m0)) * 2
                                    : ((long long)(M - 1 - m0) * lda + K) * 2;
    const long long b_ext0 = C::BKN ? ((long long)(K - 1) * ldb + (N - n0)) * 2
                                    : ((long long)(N - 1 - n0) * ldb + K) * 2;
    // loader lane geometry: a 1 KB block q holds rows 8q .. 8q+7 of a K-major
    // tile; lane writes physical 16-byte slot (lane & 7) of row 8q + (lane >> 3),
    // which holds logical chunk (lane & 7) ^ swz(row), swz(r) = (r & 7) ^ ((r >> 3) & 1)
    // (NW is even, so q & 1 == wave & 1 for every block a wave loads)
    const int kq_row = lane >> 3;
    const int kq_chunk = (lane & 7) ^ kq_row ^ (wave & 1);
    static_assert(C::F32 || C::NW % 2 == 0, "wave count must be even");
    // N-major W tile: a 1 KB block holds KN_RPB rows of KN_CPR chunks
    const int kn_row = lane / C::KN_CPR;
    const int kn_slot = lane % C::KN_CPR;

    u32x4_t greg;   // RMS: the gamma chunk matching this lane's A chunks
    u32x4_t araw[C::A_BPW];   // RMS: this lane's raw A chunks of the next K step
    const __amdgpu_buffer_rsrc_t rg_all = make_rsrc(C::RMS ? a->gamma : a->A, (long long)K * 2);

    // A straight to LDS (into the stage), or with RMS into registers (the chunk
    // a lane loads is the one it owns in the stage's swizzled block layout, so
    // its converted values go to LDS at the same place); B straight to LDS
    // per-lane offsets of the direct loads within a K step (fixed for the
    // whole loop; the step moves the resource base)
    uint32_t a_off[C::A_BPW], b_off[C::B_BPW];
#pragma unroll
    for (int i = 0; i < C::A_BPW; ++i) {
      const int q = wave + C::NW * i;
      if constexpr (C::AKM) {
        const int k = q * C::KM_RPB + lane / C::KM_CPR;
        a_off[i] = uint32_t(k) * uint32_t(lda * 2) + uint32_t(((lane % C::KM_CPR) ^ (2 * (k & 3))) * 16);
      } else {
        a_off[i] = uint32_t(8 * q + kq_row) * uint32_t(lda * 2) + uint32_t(kq_chunk * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_BPW; ++i) {
      const int q = wave + C::NW * i;
      if constexpr (C::BKN) {
        const int k = q * C::KN_RPB + kn_row;
        b_off[i] = uint32_t(k) * uint32_t(ldb * 2) + uint32_t((kn_slot ^ (2 * (k & 3))) * 16);
      } else {
        b_off[i] = uint32_t(8 * q + kq_row) * uint32_t(ldb * 2) + uint32_t(kq_chunk * 16);
      }
    }
    auto load_a = [&](int kt, char* dst) {
      const int k0 = (kt_lo + kt) * 64;
      if constexpr (C::AKM) {
        // K rows of BM contiguous M values, 16-byte chunk c of row k at slot
        // c ^ 2(k & 3) (rows past K read as zero); the same layout as an
        // N-major W tile
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc_nonneg(Abase + (long long)k0 * lda * 2, a_ext0 - (long long)k0 * lda * 2);
#pragma unroll
        for (int i = 0; i < C::A_BPW; ++i) {
          const int q = wave + C::NW * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(dst + q * 1024), 16, (int)a_off[i], 0, 0, 0);
        }
        return;
      }
      const __amdgpu_buffer_rsrc_t ra = make_rsrc_nonneg(Abase + (long long)k0 * 2, a_ext0 - (long long)k0 * 2);
      // chunks past K read as zero (an offset with the top bit set is out of
      // range); whole K steps take the wave-uniform first branch, so the
      // offsets carry no per-lane select (one compiled as a divergent branch
      // around every load)
      const uint32_t kmask = (k0 + 64 <= K) ? 0u : ((k0 + 8 * kq_chunk < K) ? 0u : kOobOffset);
      if constexpr (C::RMS) {
#pragma unroll
        for (int i = 0; i < C::A_BPW; ++i) araw[i] = buffer_load16(ra, a_off[i] | kmask);
        greg = buffer_load16(rg_all, uint32_t((k0 + 8 * kq_chunk) * 2));
      } else {
#pragma unroll
        for (int i = 0; i < C::A_BPW; ++i) {
          const int q = wave + C::NW * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (LdsPtr)(dst + q * 1024), 16, (int)(a_off[i] | kmask), 0, 0,
                                                   0);
        }
      }
    };
    auto load_b = [&](int kt, char* As) {
      const int k0 = (kt_lo + kt) * 64;
      char* Bs = As + C::A_BYTES;
      if constexpr (C::BKN) {
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc_nonneg(Bbase + (long long)k0 * ldb * 2, b_ext0 - (long long)k0 * ldb * 2);
#pragma unroll
        for (int i = 0; i < C::B_BPW; ++i) {
          const int q = wave + C::NW * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LdsPtr)(Bs + q * 1024), 16, (int)b_off[i], 0, 0, 0);
        }
      } else {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc_nonneg(Bbase + (long long)k0 * 2, b_ext0 - (long long)k0 * 2);
        const uint32_t kmask = (k0 + 64 <= K) ? 0u : ((k0 + 8 * kq_chunk < K) ? 0u : kOobOffset);
#pragma unroll
        for (int i = 0; i < C::B_BPW; ++i) {
          const int q = wave + C::NW * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (LdsPtr)(Bs + q * 1024), 16, (int)(b_off[i] | kmask), 0, 0, 0);
        }
      }
    };

    // RMS: convert this lane's raw A chunks into the stage `As`: fp32 sum of
    // squares of the raw values, then bf16(x * gamma).  Each lane writes only
    // its own chunks, so no barrier is needed between load and conversion.
    // LN: the values converted are x - s, s the mean of the row's first 64 values
    // (taken at the first conversion over the 8 lanes that hold the row; any
    // per-row constant leaves the norm unchanged, and one close to the row mean
    // keeps x - s, and so the bf16 rounding of the operand, small); chunks past K
    // (zeros) use s = 0 so that they add nothing to the sums.
    auto convert_a = [&](char* As, int k0, bool first) {
      const bool kin = k0 + 8 * kq_chunk < K;
#pragma unroll
      for (int i = 0; i < C::A_BPW; ++i) {
        const int q = wave + C::NW * i;
        u32x4_t x = araw[i];
        if constexpr (C::LN) {
          if (first) {
            float t = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w) t += bf16_lo(x[w]) + bf16_hi(x[w]);
            t += __shfl_xor(t, 1);
            t += __shfl_xor(t, 2);
            t += __shfl_xor(t, 4);
            sh[i] = t * (1.0f / 64.0f);
          }
          const float s0 = kin ? sh[i] : 0.0f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float lo = bf16_lo(x[w]) - s0, hv = bf16_hi(x[w]) - s0;
            ss[i] = fmaf(lo, lo, ss[i]);
            ss[i] = fmaf(hv, hv, ss[i]);
            sx[i] += lo + hv;
            x[w] = pack_bf16x2(lo * bf16_lo(greg[w]), hv * bf16_hi(greg[w]));
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float lo = bf16_lo(x[w]), hv = bf16_hi(x[w]);
            ss[i] = fmaf(lo, lo, ss[i]);
            ss[i] = fmaf(hv, hv, ss[i]);
            x[w] = pack_bf16x2(lo * bf16_lo(greg[w]), hv * bf16_hi(greg[w]));
          }
        }
        *reinterpret_cast<u32x4_t*>(As + q * 1024 + lane * 16) = x;
      }
    };

    // MFMA operand read offsets (bytes within a stage)
    // X fragment (MFMA B operand): row wm*WTM + 32 mi + l32, logical chunk 2kk + hi;
    // the row base is a multiple of 32, so swz(row) = swz(l32)
    int xa_off[C::AKM ? MI : 4];
    if constexpr (C::AKM) {
      // M-major A tile: the transposing read of the W fragments below, with
      // rows m of the tile in place of columns n
      const int G = lane >> 4, s = lane & 15;
      const int r = s >> 2;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int krow = 8 * (G >> 1) + r;
        const int m = wm * C::WTM + 32 * mi + 16 * (G & 1) + 4 * (s & 3);
        const int phys = (m >> 3) ^ (2 * r);
        xa_off[mi] = krow * (BM * 2) + phys * 16 + (m & 7) * 2;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        xa_off[kk] = (wm * C::WTM + l32) * 128 + (((2 * kk + hi) ^ swz_l) * 16);
    }
    // W fragment (MFMA A operand)
    int wb_off[C::BKN ? NI : 4];
    if constexpr (C::BKN) {
      // transposing read: lane (G, s) supplies row 16kk + 8(G/2) + 4h + s/4 at
      // column 32ni + 16(G%2) + 4(s%4); lane s of each 16-lane group receives
      // the 4 K-consecutive values of column 16(G%2) + s
      const int G = lane >> 4, s = lane & 15;
      const int r = s >> 2;
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int krow = 8 * (G >> 1) + r;
        const int n = wn * C::WTN + 32 * ni + 16 * (G & 1) + 4 * (s & 3);
        const int phys = (n >> 3) ^ (2 * r);
        wb_off[ni] = C::A_BYTES + krow * (BN * 2) + phys * 16 + (n & 7) * 2;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        wb_off[kk] = C::A_BYTES + (wn * C::WTN + l32) * 128 + (((2 * kk + hi) ^ swz_l) * 16);
    }

    auto read_frags = [&](const char* stage, int kk, bf16x8_t (&xf)[MI], bf16x8_t (&wf)[NI]) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if constexpr (C::AKM) {
          const char* p = stage + xa_off[mi] + kk * 16 * (BM * 2);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsI16x4*)(p));
          const i16x4_t hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsI16x4*)(p + 4 * (BM * 2)));
          xf[mi] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          xf[mi] = *reinterpret_cast<const bf16x8_t*>(stage + xa_off[kk] + mi * 32 * 128);
        }
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if constexpr (C::BKN) {
          const char* p = stage + wb_off[ni] + kk * 16 * (BN * 2);
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsI16x4*)(p));
          const i16x4_t hv = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsI16x4*)(p + 4 * (BN * 2)));
          wf[ni] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hv, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          wf[ni] = *reinterpret_cast<const bf16x8_t*>(stage + wb_off[kk] + ni * 32 * 128);
        }
      }
    };

    // SSF: squares of the X fragments (rows wm*WTM + 32 mi + l32, K indices
    // 16 kk + 8 (lane >> 5) + 0..7).  The WN waves that share those rows split
    // the (row block, slice) pairs: at slice kk wave wn takes the blocks
    // mi = ((wn - kk) mod WN) + WN t, picked with wave-uniform selects so that
    // the work has no branch and can sit between the slice's MFMAs; the sum
    // goes to ss[kk * (MI / WN) + t].
    static_assert(C::F32 || !C::SSF || MI % C::WN == 0, "row blocks must split over the wave columns");
    static_assert(C::F32 || !C::LNF || NSS >= MI, "one shift per row block");
    const int wn_s = __builtin_amdgcn_readfirstlane(wn);
    // LNF: the sums are of x - s, s the row's first element (sh[mi], taken from
    // the first slice of the first K step), over the K indices below K only.
    auto sumsq_frags = [&](auto kkc, const bf16x8_t (&xf)[MI], int k0) {
      constexpr int kk = decltype(kkc)::value;
      constexpr int TPW = MI / C::WN;
      const int sel = (wn_s - kk + 4 * C::WN) % C::WN;   // wave-uniform
      const bool kin = k0 + 16 * kk + 8 * hi < K;
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        u32x4_t v = __builtin_bit_cast(u32x4_t, xf[C::WN * t]);
        uint32_t shb = __float_as_uint(sh[C::WN * t]);
#pragma unroll
        for (int c = 1; c < C::WN; ++c) {
          // a bitwise select on a wave-uniform mask (indexing the fragment
          // array with `sel` would move it to scratch memory)
          const uint32_t m = sel == c ? 0xffffffffu : 0u;
          const u32x4_t o = __builtin_bit_cast(u32x4_t, xf[C::WN * t + c]);
#pragma unroll
          for (int w = 0; w < 4; ++w) v[w] = (o[w] & m) | (v[w] & ~m);
          if constexpr (C::LNF) shb = (__float_as_uint(sh[C::WN * t + c]) & m) | (shb & ~m);
        }
        const float s0 = (C::LNF && kin) ? __uint_as_float(shb) : 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_lo(v[w]) - s0, hv = bf16_hi(v[w]) - s0;
          ss[kk * TPW + t] = fmaf(lo, lo, ss[kk * TPW + t]);
          ss[kk * TPW + t] = fmaf(hv, hv, ss[kk * TPW + t]);
          if constexpr (C::LNF) sx[kk * TPW + t] += lo + hv;
        }
        // keeps the sums computed inside this slice's scheduling region (the
        // arithmetic would otherwise be sunk past the MFMAs of the whole step)
        asm volatile("" ::"v"(ss[kk * TPW + t]));
        if constexpr (C::LNF) asm volatile("" ::"v"(sx[kk * TPW + t]));
      }
    };

    auto compute = [&](const char* stage, int kt) {
      bf16x8_t xf[2][MI], wf[2][NI];
      read_frags(stage, 0, xf[0], wf[0]);
      if constexpr (C::LNF) {
        if (kt == 0) {   // the row's first element: lane l32 (lower half) holds K indices 0..7
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            sh[mi] = __shfl(bf16_lo(__builtin_bit_cast(u32x4_t, xf[0][mi])[0]), l32);
        }
      }
      const int k0 = (kt_lo + kt) * 64;
      static_for<0, 4>([&](auto kkc) {
        constexpr int kk = decltype(kkc)::value;
        // the next step's fragment reads are issued before this step's MFMAs
        // (scheduling barriers keep them there), so their latency is covered
        if constexpr (kk < 3) read_frags(stage, kk + 1, xf[(kk + 1) & 1], wf[(kk + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk & 1][ni], xf[kk & 1][mi], acc[mi][ni], 0, 0, 0);
        if constexpr (C::SSF) {
          // the slice's squares between its MFMAs: one MFMA, then up to 4 VALU
          sumsq_frags(kkc, xf[kk & 1], k0);
#pragma unroll
          for (int q = 0; q < MI * NI; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // Buffer loads (to LDS or to registers) complete in issue order, so a wait
    // for a given load is "at most `later` loads outstanding", `later` being
    // those issued after it.
    auto wait_vm = [&](auto later_c) {
      constexpr int later = decltype(later_c)::value;
      constexpr int enc = (later & 0xF) | (0x7 << 4) | (0xF << 8) | (((later >> 4) & 3) << 14);
      __builtin_amdgcn_s_waitcnt(enc);
    };
    constexpr std::integral_constant<int, C::A_BPW + 1> kAfterB{};   // raw A + gamma of the next step
    constexpr std::integral_constant<int, C::B_BPW> kAfterA{};       // B of the next step

    // RMS: the waves of a workgroup are spread round-robin over the 4 SIMDs, so
    // waves w and w + NW/2 share a SIMD.  The upper half converts A(kt+1) before
    // its MFMAs and the lower half after them: on every SIMD one wave's VALU
    // conversion overlaps the other wave's matrix work.
    const bool convert_first = wave >= C::NW / 2;
    auto convert_phase = [&](int kt, char* nxt) {
      wait_vm(kAfterA);                     // raw A(kt+1) and its gamma have landed
      convert_a(nxt, (kt_lo + kt + 1) * 64, false);
      if (kt + 2 < KT) load_a(kt + 2, nullptr);   // into araw, which the conversion has consumed
    };

    // One K step: tile kt is in `cur`; every wave is done reading `nxt`.
    // RMS order of a wave's loads: B(kt) (to LDS) at the top of step kt-1, then
    // raw A(kt+1) (to registers) and gamma after that wave's conversion in step
    // kt-1; so at the top of step kt only the latter may still be in flight.
    auto step = [&](int kt, char* cur, char* nxt) {
      if constexpr (C::RMS) {
        if (kt + 1 < KT) wait_vm(kAfterB);
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
      const bool more = kt + 1 < KT;
      if (more) {
        if constexpr (!C::RMS) load_a(kt + 1, nxt);
        load_b(kt + 1, nxt);
      }
      if constexpr (C::RMS) {
        if (more && convert_first) convert_phase(kt, nxt);
      }
      compute(cur, kt);
      if constexpr (C::RMS) {
        if (more && !convert_first) convert_phase(kt, nxt);
      }
    };
    if (KT > 0) {
      if constexpr (C::RMS) {
        load_a(0, nullptr);
        load_b(0, smem0);
        wait_vm(kAfterA);
        convert_a(smem0, kt_lo * 64, true);
        if (KT > 1) load_a(1, nullptr);
      } else {
        load_a(0, smem0);
        load_b(0, smem0);
      }
      for (int kt = 0; kt < KT; kt += 2) {   // two steps per trip keep each stage a fixed array
        step(kt, smem0, smem1);
        if (kt + 1 < KT) step(kt + 1, smem1, smem0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    if constexpr (C::SSF) {
      // the two lane halves of a row, then this wave column's LDS row: the pair
      // (block mi, slice kk) was taken by wave column (mi + kk) mod WN only, so
      // the WN rows add up to the whole sum
      constexpr int TPW = MI / C::WN;
      float* col = smem_ss + wn * BM + wm * C::WTM + l32;
      float* colx = col + C::WN * BM;   // LNF: row sums
      if (hi == 0) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          col[32 * mi] = 0.0f;
          if constexpr (C::LNF) colx[32 * mi] = 0.0f;
        }
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const float v = ss[kk * TPW + t] + __shfl_xor(ss[kk * TPW + t], 32);
          const int mi = (wn - kk + 4 * C::WN) % C::WN + C::WN * t;
          if (hi == 0) col[32 * mi] += v;
          if constexpr (C::LNF) {
            const float u = sx[kk * TPW + t] + __shfl_xor(sx[kk * TPW + t], 32);
            if (hi == 0) colx[32 * mi] += u;
          }
        }
      if constexpr (C::LNF) {   // the shifts, once per row (wave column 0)
        if (wn == 0 && hi == 0) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) smem_ss[2 * C::WN * BM + wm * C::WTM + 32 * mi + l32] = sh[mi];
        }
      }
    }
    __syncthreads();
  } else {
    // ================= fp32 main loop (small tile, register staged) =================
    constexpr int SA = C::SA32, SB = C::SB32;
    constexpr int KCH = BK / 4;   // 16-byte chunks per K row
    const int a_c = tid % KCH, a_r = tid / KCH;
    const int bkn_cpr = BN / 4;
    const int b_c = C::BKN ? tid % bkn_cpr : tid % KCH;
    const int b_r = C::BKN ? tid / bkn_cpr : tid / KCH;
    constexpr int A_RSTEP = C::NT / KCH;
    const int B_RSTEP = C::BKN ? C::NT / bkn_cpr : C::NT / KCH;
    const char* Abase = static_cast<const char*>(a->A) + (long long)m0 * lda * 4;
    const char* Bbase = C::BKN ? static_cast<const char*>(a->B) + (long long)n0 * 4
                               : static_cast<const char*>(a->B) + (long long)n0 * ldb * 4;
    const long long a_ext0 = ((long long)(M - 1 - m0) * lda + K) * 4;
    const long long b_ext0 = C::BKN ? ((long long)(K - 1) * ldb + (N - n0)) * 4
                                    : ((long long)(N - 1 - n0) * ldb + K) * 4;
    u32x4_t areg[C::A32_CH], breg[C::B32_CH], greg;

    auto gload = [&](int kt) {
      const int k0 = kt * BK;
      const bool kin_a = k0 + a_c * 4 < K;
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(Abase + (long long)k0 * 4, a_ext0 - (long long)k0 * 4);
#pragma unroll
      for (int i = 0; i < C::A32_CH; ++i) {
        const uint32_t off = uint32_t(a_r + i * A_RSTEP) * uint32_t(lda * 4) + uint32_t(a_c * 16);
        areg[i] = buffer_load16(ra, kin_a ? off : kOobOffset);
      }
      if (C::BKN) {
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(Bbase + (long long)k0 * ldb * 4, b_ext0 - (long long)k0 * ldb * 4);
#pragma unroll
        for (int i = 0; i < C::B32_CH; ++i)
          breg[i] = buffer_load16(rb, uint32_t(b_r + i * B_RSTEP) * uint32_t(ldb * 4) + uint32_t(b_c * 16));
      } else {
        const bool kin_b = k0 + b_c * 4 < K;
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bbase + (long long)k0 * 4, b_ext0 - (long long)k0 * 4);
#pragma unroll
        for (int i = 0; i < C::B32_CH; ++i) {
          const uint32_t off = uint32_t(b_r + i * B_RSTEP) * uint32_t(ldb * 4) + uint32_t(b_c * 16);
          breg[i] = buffer_load16(rb, kin_b ? off : kOobOffset);
        }
      }
      if (C::RMS) {
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(a->gamma, (long long)K * 4);
        greg = buffer_load16(rg, uint32_t((k0 + a_c * 4) * 4));
      }
    };
    // LN: as in the bf16 loop, A - s with s the mean of the row's first BK
    // values (the KCH threads of a row are consecutive lanes)
    auto sstore = [&](int buf, int k0) {
      float* As = reinterpret_cast<float*>(buf ? smem1 : smem0);
      float* Bs = As + BM * SA;
      const bool kin = k0 + a_c * 4 < K;
#pragma unroll
      for (int i = 0; i < C::A32_CH; ++i) {
        float* dst = As + (a_r + i * A_RSTEP) * SA + a_c * 4;
        if (C::LN && k0 == 0) {
          float t = 0.0f;
#pragma unroll
          for (int w = 0; w < 4; ++w) t += __uint_as_float(areg[i][w]);
#pragma unroll
          for (int off = 1; off < KCH; off <<= 1) t += __shfl_xor(t, off);
          sh[i] = t * (1.0f / float(BK));
        }
        const float s0 = (C::LN && kin) ? sh[i] : 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float x = __uint_as_float(areg[i][w]) - s0;
          if (C::RMS || C::SSF) {
            ss[i] = fmaf(x, x, ss[i]);
            if (C::LN) sx[i] += x;
            if (C::RMS) x = x * __uint_as_float(greg[w]);
          }
          dst[w] = x;
        }
      }
#pragma unroll
      for (int i = 0; i < C::B32_CH; ++i) {
        if (C::BKN) {
          *reinterpret_cast<u32x4_t*>(Bs + (b_r + i * B_RSTEP) * SB + b_c * 4) = breg[i];
        } else {
          float* dst = Bs + (b_r + i * B_RSTEP) * SA + b_c * 4;
#pragma unroll
          for (int w = 0; w < 4; ++w) dst[w] = __uint_as_float(breg[i][w]);
        }
      }
    };
    auto compute = [&](int buf) {
      const float* As = reinterpret_cast<const float*>(buf ? smem1 : smem0);
      const float* Bs = As + BM * SA;
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
    };
    if (KT > 0) {
      gload(0);
      sstore(0, 0);
      __syncthreads();
      for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) gload(kt + 1);
        compute(cur);
        if (more) sstore(cur ^ 1, (kt + 1) * BK);
        __syncthreads();
      }
    }
  }

  // ================= parts of a split tile =================
  // Each part stores its fp32 accumulators (and, with RMS, its per-row sums of
  // squares) to the workspace and counts itself in; the part that arrives last
  // adds all parts in part order, so the sum does not depend on the arrival
  // order, and goes on to the epilogue.  The others are done.  The partials go
  // out and come back as agent-scope atomic accesses, which are coherent across
  // the XCDs' L2 caches; waiting for the stores to complete before the count
  // publishes them without writing back or invalidating a whole L2.
  if constexpr (!C::F32 && !C::LNE) {   // LN tiles are never split
    if (split >= 0) {
      const int S = a->split_s;
      constexpr int NG = MI * NI * 8;   // pairs of accumulator registers per thread
      const size_t slot0 = size_t(split) * size_t(S);
      // [slot][pair][thread], 8 bytes per entry: each store or load instruction
      // covers 512 contiguous bytes
      unsigned long long* accp = reinterpret_cast<unsigned long long*>(a->split_acc) + tid;
      static_for<0, NG>([&](auto gc) {
        constexpr int gi = decltype(gc)::value;
        constexpr int mi = gi / (NI * 8), ni = (gi / 8) % NI, g = gi % 8;
        const unsigned long long bits = (unsigned long long)__float_as_uint(acc[mi][ni][2 * g]) |
                                        ((unsigned long long)__float_as_uint(acc[mi][ni][2 * g + 1]) << 32);
        __hip_atomic_store(accp + ((slot0 + part) * NG + gi) * C::NT, bits, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      });
      if constexpr (C::RMS) {
        // rows 8q + (lane >> 3): the 8 lanes of a row are consecutive
#pragma unroll
        for (int i = 0; i < C::A_BPW; ++i) {
          float v = ss[i];
          v += __shfl_xor(v, 1);
          v += __shfl_xor(v, 2);
          v += __shfl_xor(v, 4);
          if ((lane & 7) == 0)
            __hip_atomic_store(a->split_ss + (slot0 + part) * BM + 8 * (wave + C::NW * i) + (lane >> 3), v,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else if constexpr (C::SSF) {
        // this part's row sums of squares (its wave columns in order)
        for (int t = tid; t < BM; t += C::NT) {
          float v = smem_ss[t];
#pragma unroll
          for (int w = 1; w < C::WN; ++w) v += smem_ss[w * BM + t];
          __hip_atomic_store(a->split_ss + (slot0 + part) * BM + t, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      int* last = reinterpret_cast<int*>(smem1 + C::EPI_FLAG_OFF);
      if (tid == 0) {
        const unsigned old =
            __hip_atomic_fetch_add(a->split_cnt + split, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *last = (old == unsigned(S - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (*last == 0) return;
      // the parts in part order (this part's own values from its registers)
      if constexpr (C::RMS) {
        // The in-loop row norm's kernels sit at the register limit, so the
        // other parts' partials come through LDS instead (the stages are free
        // now): direct loads of CH register pairs of every part per round trip,
        // agent-scope coherent like the atomic loads (sc1), then the sums in
        // part order from LDS.  Part pp's slot: array pp / 2, half pp % 2.
        constexpr int SLOT = (C::ARR0_BYTES < C::ARR1_BYTES ? C::ARR0_BYTES : C::ARR1_BYTES) / 2;
        constexpr int CH = split_chunk_pairs(SLOT, C::NT, NG);
        constexpr int KB_PER_PART = CH * C::NT * 8 / 1024;   // 1 KB direct loads per part and chunk
        static_assert(NG % CH == 0 && KB_PER_PART % C::NW == 0 && CH * C::NT * 8 <= SLOT, "split chunk layout");
        static_for<0, NG / CH>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          __syncthreads();   // every read of the previous chunk (or of the flag) is done
          static_for<0, kMaxSplitParts>([&](auto pc) {
            constexpr int pp = decltype(pc)::value;
            if (pp < S && pp != part) {
              char* slot = (pp < 2 ? smem0 : smem1) + (pp & 1) * SLOT;
              const char* src = reinterpret_cast<const char*>(accp - tid) +
                                (((slot0 + pp) * NG + size_t(CH) * c) * C::NT) * 8;
              const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, CH * C::NT * 8);
#pragma unroll
              for (int i = 0; i < KB_PER_PART / C::NW; ++i) {
                const int k = wave + C::NW * i;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(slot + k * 1024), 16, k * 1024 + lane * 16, 0,
                                                         0, kCachePolicySc1);
              }
            }
          });
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          static_for<0, CH>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int gi = CH * c + j;
            constexpr int mi = gi / (NI * 8), ni = (gi / 8) % NI, g = gi % 8;
            float s0 = 0.0f, s1 = 0.0f;
            for (int pp = 0; pp < S; ++pp) {
              float v0 = acc[mi][ni][2 * g], v1 = acc[mi][ni][2 * g + 1];
              if (pp != part) {
                const char* slot = (pp < 2 ? smem0 : smem1) + (pp & 1) * SLOT;
                const unsigned long long bits =
                    *reinterpret_cast<const unsigned long long*>(slot + (j * C::NT + tid) * 8);
                v0 = __uint_as_float(uint32_t(bits));
                v1 = __uint_as_float(uint32_t(bits >> 32));
              }
              s0 = pp == 0 ? v0 : s0 + v0;
              s1 = pp == 0 ? v1 : s1 + v1;
            }
            acc[mi][ni][2 * g] = s0;
            acc[mi][ni][2 * g + 1] = s1;
          });
        });
        __syncthreads();   // the slots' last reads are done before the epilogue's LDS use
      } else {
        // the other parts' values of PB register pairs are loaded together, so a
        // batch costs one round trip to the memory side
        constexpr int PB = 8;
        static_assert(NG % PB == 0, "register pairs come in whole batches");
        static_for<0, NG / PB>([&](auto bc) {
          constexpr int b = decltype(bc)::value;
          // (scheduling barriers keep each batch's loads next to its adds)
          __builtin_amdgcn_sched_barrier(0);
          unsigned long long t[kMaxSplitParts][PB];
          static_for<0, kMaxSplitParts>([&](auto pc) {
            constexpr int pp = decltype(pc)::value;
            if (pp < S && pp != part) {
#pragma unroll
              for (int j = 0; j < PB; ++j)
                t[pp][j] = __hip_atomic_load(accp + ((slot0 + pp) * NG + PB * b + j) * C::NT, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
            }
          });
          static_for<0, PB>([&](auto jc) {
            constexpr int gi = PB * b + decltype(jc)::value;
            constexpr int mi = gi / (NI * 8), ni = (gi / 8) % NI, g = gi % 8;
            const float own0 = acc[mi][ni][2 * g], own1 = acc[mi][ni][2 * g + 1];
            float s0 = 0.0f, s1 = 0.0f;
            static_for<0, kMaxSplitParts>([&](auto pc) {
              constexpr int pp = decltype(pc)::value;
              if (pp < S) {
                float v0 = own0, v1 = own1;
                if (pp != part) {
                  const unsigned long long bits = t[pp][decltype(jc)::value];
                  v0 = __uint_as_float(uint32_t(bits));
                  v1 = __uint_as_float(uint32_t(bits >> 32));
                }
                s0 = pp == 0 ? v0 : s0 + v0;
                s1 = pp == 0 ? v1 : s1 + v1;
              }
            });
            acc[mi][ni][2 * g] = s0;
            acc[mi][ni][2 * g + 1] = s1;
          });
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      if constexpr (C::RMS) {
        // whole-row sums in part order, on the first lane of each row (the row
        // sum below adds the zeros of the other lanes)
#pragma unroll
        for (int i = 0; i < C::A_BPW; ++i) {
          const int row = 8 * (wave + C::NW * i) + (lane >> 3);
          float x[kMaxSplitParts];
#pragma unroll
          for (int pp = 0; pp < kMaxSplitParts; ++pp)
            if (pp < S)
              x[pp] = __hip_atomic_load(a->split_ss + (slot0 + pp) * BM + row, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
          float t = 0.0f;
#pragma unroll
          for (int pp = 0; pp < kMaxSplitParts; ++pp)
            if (pp < S) t = pp == 0 ? x[pp] : t + x[pp];
          ss[i] = (lane & 7) == 0 ? t : 0.0f;
        }
      } else if constexpr (C::SSF) {
        // whole-row sums in part order, left in the first wave column's LDS row
        for (int t = tid; t < BM; t += C::NT) {
          float x[kMaxSplitParts];
#pragma unroll
          for (int pp = 0; pp < kMaxSplitParts; ++pp)
            if (pp < S)
              x[pp] = __hip_atomic_load(a->split_ss + (slot0 + pp) * BM + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          float v = 0.0f;
#pragma unroll
          for (int pp = 0; pp < kMaxSplitParts; ++pp)
            if (pp < S) v = pp == 0 ? x[pp] : v + x[pp];
          smem_ss[t] = v;
#pragma unroll
          for (int w = 1; w < C::WN; ++w) smem_ss[w * BM + t] = 0.0f;
        }
      }
      // leave the counter at zero for the next call
      if (tid == 0) __hip_atomic_store(a->split_cnt + split, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ================= epilogue =================
  char* region = smem0 + wave * C::REGION_BYTES;
  float* red = reinterpret_cast<float*>(smem1 + C::EPI_RED_OFF);
  float* rinv = reinterpret_cast<float*>(smem1 + C::EPI_RINV_OFF);
  float* rmu = reinterpret_cast<float*>(smem1 + C::EPI_RMU_OFF);
  float* colp = reinterpret_cast<float*>(smem1 + C::EPI_COL_OFF);
  // row factors from the sums: RMS 1/sqrt(ss/K + eps); LN rstd = 1/sqrt(var + eps)
  // with mean m = sx/K and var = ss/K - m^2 (of the shifted values), and m * rstd
  // (LNF: the accumulators hold the unshifted product, so the mean term is
  // (shift + m) * rstd)
  auto row_factors = [&](int row, float v, float s, float shift) {
    if constexpr (C::LNE) {
      const float m = s / float(K);
      const float var = fmaxf(v / float(K) - m * m, 0.0f);
      const float r = 1.0f / sqrtf(var + a->eps);
      rinv[row] = r;
      rmu[row] = (shift + m) * r;
    } else {
      rinv[row] = 1.0f / sqrtf(v / float(K) + a->eps);
    }
  };
  int* flag = reinterpret_cast<int*>(smem1 + C::EPI_FLAG_OFF);

  if constexpr (C::GIVEN) {
    for (int t = tid; t < BM; t += C::NT) {
      const int row = m0 + t;
      const float v = row < M ? a->row_ss[(long long)row * a->row_ss_stride] : 0.0f;
      const float sm = (C::LNE && row < M) ? a->row_s[(long long)row * a->row_ss_stride] : 0.0f;
      row_factors(t, v, sm, 0.0f);
    }
    __syncthreads();
  } else if constexpr (C::SSF && !C::F32) {
    for (int t = tid; t < BM; t += C::NT) {
      float v = smem_ss[t], s = 0.0f, shift = 0.0f;
#pragma unroll
      for (int w = 1; w < C::WN; ++w) v += smem_ss[w * BM + t];
      if constexpr (C::LNF) {
#pragma unroll
        for (int w = 0; w < C::WN; ++w) s += smem_ss[(C::WN + w) * BM + t];
        shift = smem_ss[2 * C::WN * BM + t];
      }
      row_factors(t, v, s, shift);
    }
    __syncthreads();
  } else if constexpr (C::RMS || C::SSF) {
    if constexpr (!C::F32) {
      // rows 8q + (lane >> 3): the 8 lanes of a row are consecutive
#pragma unroll
      for (int i = 0; i < C::A_BPW; ++i) {
        float v = ss[i], s = sx[i];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        if constexpr (C::LN) {
          s += __shfl_xor(s, 1);
          s += __shfl_xor(s, 2);
          s += __shfl_xor(s, 4);
        }
        if ((lane & 7) == 0) row_factors(8 * (wave + C::NW * i) + (lane >> 3), v, s, 0.0f);
      }
    } else {
      constexpr int KCH = BK / 4;
#pragma unroll
      for (int i = 0; i < C::A32_CH; ++i) {
        float v = ss[i], s = sx[i];
#pragma unroll
        for (int off = 1; off < KCH; off <<= 1) {
          v += __shfl_xor(v, off);
          if constexpr (C::LN) s += __shfl_xor(s, off);
        }
        if (tid % KCH == 0) row_factors(tid / KCH + i * (C::NT / KCH), v, s, 0.0f);
      }
    }
    __syncthreads();
  }

  // SIDE: the first bf16 side matrix of the list (before any SWIGLU_PAIR) is
  // read ahead: block 0's rows before the block loop, block mi+1's as soon as
  // block mi has consumed its own (one set of registers), so their latency
  // overlaps the rest of the block's ops, its stores and the next restage.
  int pf_op = -1;
  if constexpr (C::SIDE) {
    for (int q = 0; q < a->n_ops; ++q) {
      const int k = a->ops[q].kind;
      if (k == CODA_OP_SWIGLU_PAIR) break;
      if ((k == CODA_OP_ADD_MAT || k == CODA_OP_MUL_DGELU_TANH) && a->ops[q].dtype == CODA_BF16) {
        pf_op = q;
        break;
      }
    }
  }
  u32x4_t pf_buf[C::SIDE ? C::CPL : 1][1];
  u32x4_t(&pfb)[C::CPL] = *reinterpret_cast<u32x4_t(*)[C::CPL]>(&pf_buf[0][0]);
  auto prefetch = [&](int mi_next, u32x4_t (&dst)[C::CPL]) {
    KOp op = a->ops[pf_op];
    // rows from m0 on; reads past the matrix (rows >= M) return zero
    const char* base = static_cast<const char*>(op.in) + (long long)m0 * op.ld * 2;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, ((long long)(M - 1 - m0) * op.ld + op.width) * 2);
    const int colb = wn * C::WTN + 8 * (lane % C::CPR) + n0;
#pragma unroll
    for (int j = 0; j < C::CPL; ++j) {
      const int mloc = wm * C::WTM + 32 * mi_next + lane / C::CPR + C::RSTEP * j;
      dst[j] = buffer_load16(rs, uint32_t(mloc) * uint32_t(op.ld * 2) + uint32_t(colb * 2));
    }
  };
  if (C::SIDE && pf_op >= 0) prefetch(0, pfb);
  // LN: u[j] for the lane's 8 columns (the same in every block)
  float uv[8];
  if constexpr (C::LNE) load_cols<false>(a->ln_u, CODA_F32, n0 + wn * C::WTN + 8 * (lane % C::CPR), N, uv);
  // The first column vector of the list (a bias, before any SWIGLU_PAIR): a
  // lane's 8 columns are the same in every 32-row block, so it is loaded once
  // here instead of once per block with its latency in each block's path.
  int cv_op = -1;
  for (int q = 0; q < a->n_ops; ++q) {
    const int k = a->ops[q].kind;
    if (k == CODA_OP_SWIGLU_PAIR) break;
    if (k == CODA_OP_ADD_COL || k == CODA_OP_SCALE_COL) {
      cv_op = q;
      break;
    }
  }
  float cv[8];
  if (cv_op >= 0) {
    KOp op = a->ops[cv_op];
    load_cols<false>(op.in, op.dtype, n0 + wn * C::WTN + 8 * (lane % C::CPR), op.width, cv);
  }

  static_for<0, MI>([&](auto mic) {
    constexpr int mi = decltype(mic)::value;
    auto next_pf = [&]() {
      if constexpr (C::SIDE && mi + 1 < MI) prefetch(mi + 1, pfb);
    };
    // accumulators of block mi -> the wave's region, row-major [32][WTN] fp32,
    // 16-byte slot s of row r stored at slot s ^ swz(r)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int slot = 8 * ni + 2 * g + hi;
        f32x4_t w;
        w[0] = acc[mi][ni][4 * g + 0];
        w[1] = acc[mi][ni][4 * g + 1];
        w[2] = acc[mi][ni][4 * g + 2];
        w[3] = acc[mi][ni][4 * g + 3];
        *reinterpret_cast<f32x4_t*>(region + l32 * (C::WTN * 4) + ((slot ^ swz_l) * 16)) = w;
      }
    __builtin_amdgcn_wave_barrier();
    Chunks<C::CPL> ch;
    const int c = lane % C::CPR;
    ch.col = n0 + wn * C::WTN + 8 * c;
#pragma unroll
    for (int j = 0; j < C::CPL; ++j) {
      const int r = lane / C::CPR + C::RSTEP * j;
      ch.mloc[j] = wm * C::WTM + 32 * mi + r;
      ch.row[j] = m0 + ch.mloc[j];
      const int sw = (r & 7) ^ ((r >> 3) & 1);
      const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(region + r * (C::WTN * 4) + (((2 * c) ^ sw) * 16));
      const f32x4_t hv = *reinterpret_cast<const f32x4_t*>(region + r * (C::WTN * 4) + (((2 * c + 1) ^ sw) * 16));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ch.v[j][e] = lo[e];
        ch.v[j][4 + e] = hv[e];
      }
      if constexpr (C::LNE) {
        const float s = rinv[ch.mloc[j]], mr = rmu[ch.mloc[j]];
#pragma unroll
        for (int e = 0; e < 8; ++e) ch.v[j][e] = fmaf(ch.v[j][e], s, -mr * uv[e]);
      } else if constexpr (C::RMS || C::SSF || C::GIVEN) {
        const float s = rinv[ch.mloc[j]];
#pragma unroll
        for (int e = 0; e < 8; ++e) ch.v[j][e] *= s;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int o = run_ops<C, false>(ch, a, 0, M, lane, wn, red, pf_op, pfb, colp, wm, mi, cv_op, cv, next_pf);
    if (o < a->n_ops) {   // SWIGLU_PAIR
      swiglu_chunks<C>(ch);
      run_ops<C, true>(ch, a, o + 1, M, lane, wn, red, -1, pfb, colp, wm, mi, -1, cv, [] {});
      store_chunks<C, true>(ch, a, M);
    } else {
      store_chunks<C, false>(ch, a, M);
    }
  });

  if (a->n_red > 0) {
    __syncthreads();
    const bool multi = a->grid_n > 1;
    for (int q = 0; q < a->n_ops; ++q) {
      KOp op = a->ops[q];
      if (!is_row_reduction(op.kind)) continue;
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
      // The partial sums went out as agent-scope atomic stores, which are
      // coherent across the XCDs' L2s.  Waiting for their completion before the
      // counter increment publishes them without a device-wide L2 write-back.
      // This is an ISA-level argument, outside the language memory model
      // (which would ask for a release increment and an acquire read): on
      // gfx950 an agent-scope store is written through to the memory side of
      // the XCD L2s, vmcnt counts a store down only when that write is
      // acknowledged, and the agent-scope loads of the last workgroup read
      // from the same level, never from a stale L2 line.  A release/acquire
      // pair would instead write back and invalidate a whole L2 per workgroup.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) {
        const unsigned old =
            __hip_atomic_fetch_add(a->counters + tile_m, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = (old == unsigned(a->grid_n - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (*flag) {
        // last workgroup of the tile row: sum the partials in tile order
        for (int q = 0; q < a->n_ops; ++q) {
          KOp op = a->ops[q];
          if (!is_row_reduction(op.kind)) continue;
          const int s = op.red_slot;
          for (int t = tid; t < BM; t += C::NT) {
            const int row = m0 + t;
            if (row >= M) continue;
            const float v = sum_partials(a->partials + (long long)s * a->grid_n * M + row, M, a->grid_n);
            write_reduction(op, row, v);
          }
        }
        // leave the counter at zero for the next call
        if (tid == 0) __hip_atomic_store(a->counters + tile_m, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // Column reductions: the tile's partial per column (its row blocks in a
  // fixed order), then across the tile rows of the grid through the workspace,
  // finished in tile order by the last workgroup of the tile column, as for
  // the row reductions.
  if (C::EXT && a->n_colred > 0) {
    __syncthreads();
    const bool multi = a->grid_m > 1;
    for (int q = 0; q < a->n_ops; ++q) {
      KOp op = a->ops[q];
      if (!is_col_reduction(op.kind)) continue;
      const int s = op.red_slot;
      const bool paired = op.width != N;   // after SWIGLU_PAIR: half the columns
      const int cols = paired ? BN / 2 : BN;
      const int c0 = paired ? n0 / 2 : n0;
      for (int t = tid; t < cols; t += C::NT) {
        const int col = c0 + t;
        if (col >= op.width) continue;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < C::WM; ++w)
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) v += colp[((s * C::WM + w) * MI + mi) * BN + t];
        if (!multi) {
          op.out[(long long)col * op.out_stride] = v;
        } else {
          __hip_atomic_store(a->col_partials + ((long long)s * a->grid_m + tile_m) * N + col, v, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    if (multi) {
      // publish the partials (agent-scope atomic stores, coherent across the
      // XCDs' L2s) before the count, as for the row reductions
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) {
        const unsigned old =
            __hip_atomic_fetch_add(a->col_counters + tile_n, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = (old == unsigned(a->grid_m - 1)) ? 1 : 0;
      }
      __syncthreads();
      if (*flag) {
        for (int q = 0; q < a->n_ops; ++q) {
          KOp op = a->ops[q];
          if (!is_col_reduction(op.kind)) continue;
          const int s = op.red_slot;
          const bool paired = op.width != N;
          const int cols = paired ? BN / 2 : BN;
          const int c0 = paired ? n0 / 2 : n0;
          for (int t = tid; t < cols; t += C::NT) {
            const int col = c0 + t;
            if (col >= op.width) continue;
            const float v = sum_partials(a->col_partials + (long long)s * a->grid_m * N + col, N, a->grid_m);
            op.out[(long long)col * op.out_stride] = v;
          }
        }
        // leave the counter at zero for the next call
        if (tid == 0) __hip_atomic_store(a->col_counters + tile_n, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// The backward set's ops (EXT) are compiled into the kernels without a row
// norm only: a list with a row norm and one of those ops is rejected on the
// host (no workload pairs them), which keeps the norm kernels' registers to
// what their own ops need.
template <int BM, int BN, int WM, int WN, bool F32, bool BKN>
int launch_norms(const FusedArgs& args, int64_t nwg, int norm, hipStream_t s) {
  switch (norm) {
    case kNormRms: return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormRms, false, false>>(args, nwg, s);
    case kNormLn: return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormLn, false, false>>(args, nwg, s);
    case kNormRmsB: return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormRmsB, false, false>>(args, nwg, s);
    case kNormRmsGiven: return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormRmsGiven, false, false>>(args, nwg, s);
    case kNormLnB: return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormLnB, false, false>>(args, nwg, s);
    case kNormLnGiven: return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormLnGiven, false, false>>(args, nwg, s);
    default: return CODA_ERR_UNSUPPORTED;
  }
}

// The kernels with a deferred row norm (one per norm kind and B layout).
template <int BM, int BN, int WM, int WN, bool F32>
int launch_norm_variants(const FusedArgs& args, int64_t nwg, bool bkn, int norm, hipStream_t s) {
  return bkn ? launch_norms<BM, BN, WM, WN, F32, true>(args, nwg, norm, s)
             : launch_norms<BM, BN, WM, WN, F32, false>(args, nwg, norm, s);
}

// The kernels without a row norm: A stored [M x K] or [K x M], with or
// without the backward set (ext) and the side-matrix read-ahead (side).
template <int BM, int BN, int WM, int WN, bool F32, bool BKN>
int launch_plain_b(const FusedArgs& args, int64_t nwg, bool akm, bool ext, bool side, hipStream_t s) {
  if constexpr (!F32) {
    if (akm) {   // A stored [K x M]: no row norm (validated on the host)
      return ext ? launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormNone, true, true, true>>(args, nwg, s)
                 : launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormNone, true, false, true>>(args, nwg, s);
    }
  }
  if (ext) return launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormNone, false, true, true>>(args, nwg, s);
  return side ? launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormNone, false, false, true>>(args, nwg, s)
              : launch_cfg<Cfg<BM, BN, WM, WN, F32, BKN, kNormNone, false, false>>(args, nwg, s);
}

template <int BM, int BN, int WM, int WN, bool F32>
int launch_plain_variants(const FusedArgs& args, int64_t nwg, bool bkn, bool akm, bool ext, bool side,
                          hipStream_t s) {
  return bkn ? launch_plain_b<BM, BN, WM, WN, F32, true>(args, nwg, akm, ext, side, s)
             : launch_plain_b<BM, BN, WM, WN, F32, false>(args, nwg, akm, ext, side, s);
}

// every variant of one tile configuration
template <int BM, int BN, int WM, int WN, bool F32>
int launch_variants(const FusedArgs& args, int64_t nwg, bool bkn, int norm, bool akm, bool ext, bool side,
                    hipStream_t s) {
  if (norm == kNormNone) return launch_plain_variants<BM, BN, WM, WN, F32>(args, nwg, bkn, akm, ext, side, s);
  return launch_norm_variants<BM, BN, WM, WN, F32>(args, nwg, bkn, norm, s);
}

// per compiled tile configuration (bf16 configurations 1 - 3, defined in
// coda_fused_t<n>.hip without a row norm and coda_fused_t<n>n.hip with one,
// so that the two halves compile in parallel; fp32 in coda_fused_tf32.hip)
int launch_tile1(const FusedArgs& a, int64_t nwg, bool bkn, bool akm, bool ext, bool side, hipStream_t s);
int launch_tile2(const FusedArgs& a, int64_t nwg, bool bkn, bool akm, bool ext, bool side, hipStream_t s);
int launch_tile3(const FusedArgs& a, int64_t nwg, bool bkn, bool akm, bool ext, bool side, hipStream_t s);
int launch_tile1_norm(const FusedArgs& a, int64_t nwg, bool bkn, int norm, hipStream_t s);
int launch_tile2_norm(const FusedArgs& a, int64_t nwg, bool bkn, int norm, hipStream_t s);
int launch_tile3_norm(const FusedArgs& a, int64_t nwg, bool bkn, int norm, hipStream_t s);
int launch_tile_f32(const FusedArgs& a, int64_t nwg, bool bkn, int norm, bool akm, bool ext, bool side,
                    hipStream_t s);

}  // namespace dev
}  // namespace coda
