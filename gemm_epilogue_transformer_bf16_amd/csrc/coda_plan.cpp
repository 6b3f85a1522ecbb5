// Host-side validation, tile choice and workspace sizing for the C ABI.
// No HIP calls: this file also builds into the host-only test binary.
#include "coda_plan.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace coda {

namespace {

thread_local char g_err[512] = "";

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Tile-relative byte offsets of A and B loads are 32-bit: 256 rows x ld x 4 bytes < 2^31.
constexpr int64_t kMaxLd = int64_t(1) << 21;

bool is_reduction(int kind) {
  return kind == CODA_OP_ROW_SUM || kind == CODA_OP_ROW_SUMSQ || kind == CODA_OP_ROW_MEAN ||
         kind == CODA_OP_ROW_DOT;
}

bool is_col_reduction(int kind) {
  return kind == CODA_OP_COL_SUM || kind == CODA_OP_COL_SUMSQ || kind == CODA_OP_RMS_DGAMMA;
}

bool needs_vector(int kind) {
  return kind == CODA_OP_SCALE_ROW || kind == CODA_OP_SCALE_COL || kind == CODA_OP_ADD_COL ||
         kind == CODA_OP_ADD_ROW;
}

bool needs_matrix(int kind) {
  return kind == CODA_OP_ADD_MAT || kind == CODA_OP_MUL_DGELU_TANH || kind == CODA_OP_ROW_DOT ||
         kind == CODA_OP_RMS_BWD || kind == CODA_OP_RMS_DGAMMA;
}

bool valid_dtype(int dt) { return dt == CODA_BF16 || dt == CODA_F32; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Extent {
  uintptr_t lo, hi;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};

Extent matrix_extent(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t es) {
  if (rows <= 0 || cols <= 0) return {0, 0};
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * static_cast<int64_t>(es))};
}

bool overlap(const Extent& a, const Extent& b) {
  if (a.empty() || b.empty()) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// n elements of `elem` bytes, `stride` bytes apart (a dense block: n = 1)
struct Strided {
  uintptr_t lo;
  int64_t n, stride, elem;
  Extent extent() const {
    if (lo == 0 || n <= 0) return {0, 0};
    return {lo, lo + uintptr_t((n - 1) * stride + elem)};
  }
};

Strided dense(const Extent& e) { return {e.lo, e.empty() ? 0 : 1, 0, int64_t(e.hi - e.lo)}; }
Strided column(const void* p, int64_t n, int64_t stride_elems) {
  return {reinterpret_cast<uintptr_t>(p), n, stride_elems * 4, 4};
}

// Two strided vectors of one stride whose elements fall in disjoint byte
// ranges of every period (columns of one row-major array) do not overlap.
bool strided_overlap(const Strided& a, const Strided& b) {
  if (!overlap(a.extent(), b.extent())) return false;
  if (a.stride == b.stride && a.stride > 0 && a.n > 1 && b.n > 1 && a.elem <= a.stride && b.elem <= b.stride) {
    intptr_t d = (intptr_t(b.lo) - intptr_t(a.lo)) % intptr_t(a.stride);
    if (d < 0) d += intptr_t(a.stride);
    if (d >= a.elem && intptr_t(a.stride) - d >= b.elem) return false;
  }
  return true;
}

// Automatic tile choice, from measurements on MI355X: the 8-wave 256 x 256
// tile (config 3) is fastest once its grid fills the 256 CUs at least once;
// smaller grids do better with 128 x 128 tiles (config 2), which give four
// times as many workgroups (two resident per CU).
}  // namespace

namespace {
// share of the compute units busy over the rounds of a grid of t tiles, one
// workgroup per CU
double round_fill(int64_t t, int64_t per_cu = 1) {
  const int64_t slots = kNumCUs * per_cu;
  const int64_t rounds = (t + slots - 1) / slots;
  return double(t) / double(rounds * slots);
}
}  // namespace

int choose_tile(int64_t M, int64_t N, int64_t K, bool split_allowed) {
  const int64_t t3 = ((M + 255) / 256) * ((N + 255) / 256);   // 256 x 256 tiles
  const int64_t t1 = ((M + 255) / 256) * ((N + 127) / 128);   // 256 x 128 tiles
  const int64_t t2 = ((M + 127) / 128) * ((N + 127) / 128);   // 128 x 128 tiles, two per CU
  if (t1 < kNumCUs) return 2;   // not one round even of 256 x 128
  // under one round of 256 x 256: two 128 x 128 workgroups per CU, one's
  // epilogue beside the other's main loop, unless they fill the rounds worse
  if (t3 < kNumCUs) return round_fill(t2, 2) >= round_fill(t1) ? 2 : 1;
  // the 256 x 256 tile's main loop is the faster one (fewer operand bytes per
  // flop through LDS); the 256 x 128 tile wins where it fills the rounds
  // better.  A last round that the split over K can fill counts as full.
  const bool splittable = split_allowed && (K + 63) / 64 >= 2 * kMinSplitSteps;
  const double fill3 = splittable ? 1.0 : round_fill(t3);
  return fill3 >= kTile1Speed * round_fill(t1) ? 3 : 1;
}

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = 0; }

const char* last_error() { return g_err; }

size_t fused_partials_offset(const Plan&) { return 0; }

namespace {
bool has_row_partials(const Plan& p) { return p.n_red > 0 && p.grid_n > 1; }
}  // namespace

size_t fused_counters_offset(const Plan& p) {
  return has_row_partials(p) ? align256(size_t(p.n_red) * size_t(p.grid_n) * size_t(p.M) * sizeof(float)) : 0;
}

size_t fused_split_acc_offset(const Plan& p) {
  return fused_counters_offset(p) + (has_row_partials(p) ? align256(size_t(p.grid_m) * sizeof(uint32_t)) : 0);
}

size_t fused_split_ss_offset(const Plan& p) {
  return fused_split_acc_offset(p) +
         align256(size_t(p.split_tiles) * size_t(p.split_s) * size_t(p.cfg.bm) * size_t(p.cfg.bn) * sizeof(float));
}

size_t fused_split_counters_offset(const Plan& p) {
  const size_t ss = p.has_norm ? size_t(p.split_tiles) * size_t(p.split_s) * size_t(p.cfg.bm) * sizeof(float) : 0;
  return fused_split_ss_offset(p) + align256(ss);
}

namespace {
bool has_col_partials(const Plan& p) { return p.n_colred > 0 && p.grid_m > 1; }
size_t fused_row_and_split_bytes(const Plan& p) {
  if (p.split_s <= 1) return has_row_partials(p) ? fused_split_acc_offset(p) : 0;
  return fused_split_counters_offset(p) + align256(size_t(p.split_tiles) * sizeof(uint32_t));
}
}  // namespace

size_t fused_col_partials_offset(const Plan& p) { return fused_row_and_split_bytes(p); }

size_t fused_col_counters_offset(const Plan& p) {
  return fused_col_partials_offset(p) +
         (has_col_partials(p) ? align256(size_t(p.n_colred) * size_t(p.grid_m) * size_t(p.N) * sizeof(float)) : 0);
}

size_t fused_workspace_bytes(const Plan& p) {
  if (p.M == 0 || p.N == 0) return 0;
  if (!has_col_partials(p)) return fused_row_and_split_bytes(p);
  return fused_col_counters_offset(p) + align256(size_t(p.grid_n) * sizeof(uint32_t));
}

// Split of the last round (bf16 configurations): with T tiles and `slots`
// workgroups resident at once, the grid runs T / slots full rounds and a last
// round of r = T % slots tiles.  Splitting each of those r tiles over K into s
// parts (s <= slots / r, each part at least kMinSplitSteps K steps) lets the
// last round take about 1/s of a round.
void plan_split(Plan* p, bool allow, int max_split) {
  p->full_tiles = p->grid_m * p->grid_n;
  p->split_tiles = 0;
  p->split_s = 1;
  if (!allow || p->ab_dtype != CODA_BF16 || p->K == 0 || p->has_ln) return;
  const int64_t tiles = p->grid_m * p->grid_n;
  const int64_t slots = int64_t(kNumCUs) * p->cfg.wg_per_cu;
  const int64_t r = tiles % slots;
  if (r == 0) return;
  int64_t s = slots / r;
  if (s > max_split) s = max_split;
  if (s > p->k_steps / kMinSplitSteps) s = p->k_steps / kMinSplitSteps;
  if (s < 2) return;
  p->split_tiles = r;
  p->split_s = int(s);
  p->full_tiles = tiles - r;
}

int64_t unfused_ld(const Plan& p) { return (p.N + 7) / 8 * 8; }

size_t unfused_col_partials_offset(const Plan& p) {
  size_t bytes = 0;
  if (p.has_norm) bytes += align256(size_t(p.M) * size_t(p.K) * dtype_size(p.ab_dtype));
  bytes += 2 * align256(size_t(p.M) * size_t(unfused_ld(p)) * dtype_size(p.d_dtype));
  return bytes;
}

Plan plain_gemm_plan(const Plan& p) {
  Plan q = p;
  q.has_norm = q.has_ln = q.gain_in_b = false;
  q.gamma = nullptr;
  q.ln_u = q.row_ss = q.row_s = nullptr;
  q.n_ops = q.n_red = q.n_colred = 0;
  q.has_swiglu = q.has_ext = q.has_side = false;
  q.out_width = p.N;
  plan_split(&q, p.split_allowed, kMaxSplit);
  return q;
}

size_t unfused_split_offset(const Plan& p) {
  size_t bytes = unfused_col_partials_offset(p);
  if (p.n_colred > 0)
    bytes += align256(size_t((p.M + kColChunk - 1) / kColChunk) * size_t(unfused_ld(p)) * sizeof(float));
  return bytes;
}

size_t unfused_workspace_bytes(const Plan& p) {
  if (p.M == 0 || p.N == 0) return 0;
  return unfused_split_offset(p) + fused_workspace_bytes(plain_gemm_plan(p));
}

int build_plan(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
               const coda_epi_desc* d, int unfused, bool check_pointers, Plan* p) {
  return build_plan_split(A, B, M, N, K, d, unfused, check_pointers, kMaxSplit, p);
}

int build_plan_split(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                     const coda_epi_desc* d, int unfused, bool check_pointers, int max_split, Plan* p) {
  clear_error();
  if (!d || !p) {
    set_error("descriptor is NULL");
    return CODA_ERR_INVALID_ARG;
  }
  std::memset(p, 0, sizeof(*p));
  if (M < 0 || N < 0 || K < 0) {
    set_error("negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
    return CODA_ERR_INVALID_ARG;
  }
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) {
    set_error("size above 2^31-1");
    return CODA_ERR_UNSUPPORTED;
  }
  if (!valid_dtype(d->ab_dtype) || !valid_dtype(d->d_dtype)) {
    set_error("unknown dtype ab=%d d=%d", d->ab_dtype, d->d_dtype);
    return CODA_ERR_INVALID_ARG;
  }
  if (d->b_layout != CODA_B_KN && d->b_layout != CODA_B_NK) {
    set_error("unknown B layout %d", d->b_layout);
    return CODA_ERR_INVALID_ARG;
  }
  if ((d->a_layout != CODA_A_MK && d->a_layout != CODA_A_KM) || d->reserved1 != 0) {
    set_error("unknown A layout %d (or reserved1 != 0)", d->a_layout);
    return CODA_ERR_INVALID_ARG;
  }
  if (d->n_ops < 0 || d->n_ops > CODA_MAX_OPS) {
    set_error("n_ops=%d outside 0..%d", d->n_ops, CODA_MAX_OPS);
    return CODA_ERR_INVALID_ARG;
  }
  if ((d->flags & ~CODA_FLAG_NO_SPLIT_K) != 0) {
    set_error("unknown flags 0x%x", d->flags);
    return CODA_ERR_INVALID_ARG;
  }
  if (d->tile < 0 || d->tile > kNumTileCfgs) {
    set_error("tile=%d outside 0..%d", d->tile, kNumTileCfgs);
    return CODA_ERR_INVALID_ARG;
  }
  p->ab_dtype = d->ab_dtype;
  p->d_dtype = d->d_dtype;
  p->b_layout = d->b_layout;
  p->a_layout = d->a_layout;
  p->M = M;
  p->N = N;
  p->K = K;
  p->lda = d->lda;
  p->ldb = d->ldb;
  p->ldd = d->ldd;
  p->A = A;
  p->B = B;
  p->D = d->D;
  p->workspace = d->workspace;
  p->workspace_bytes = d->workspace_bytes;

  // ---- op list ----
  int64_t width = N;
  int n_red = 0, n_col = 0;
  for (int i = 0; i < d->n_ops; ++i) {
    const coda_op& o = d->ops[i];
    if (o.kind < CODA_OP_SCALE || o.kind > CODA_OP_DROPOUT) {
      set_error("op %d: unknown kind %d", i, o.kind);
      return CODA_ERR_INVALID_ARG;
    }
    if (o.reserved0 != 0) {
      set_error("op %d: reserved0 must be 0", i);
      return CODA_ERR_INVALID_ARG;
    }
    const bool ln = o.kind == CODA_OP_LN_ROWSCALE;
    const bool norm_op = ln || o.kind == CODA_OP_RMS_ROWSCALE;
    const bool bwd = o.kind == CODA_OP_RMS_BWD;
    const bool dgam = o.kind == CODA_OP_RMS_DGAMMA;
    if ((!ln && !bwd && o.in2) || (!norm_op && !bwd && !dgam && o.row_sumsq) ||
        (!ln && !bwd && o.row_sum)) {
      set_error("op %d: in2 / row_sum / row_sumsq not used by this op must be NULL", i);
      return CODA_ERR_INVALID_ARG;
    }
    if (o.kind == CODA_OP_RMS_ROWSCALE || ln) {
      const char* name = ln ? "LN_ROWSCALE" : "RMS_ROWSCALE";
      if (i != 0) {
        set_error("op %d: %s must be the first op", i, name);
        return CODA_ERR_INVALID_ARG;
      }
      if (K == 0) {
        set_error("%s needs K > 0", name);
        return CODA_ERR_INVALID_ARG;
      }
      // gamma NULL: the gain is already in B's rows (coda_fold_gain)
      const bool folded = !o.in;
      if (!folded && (!o.in || o.in_dtype != d->ab_dtype)) {
        set_error("%s needs gamma[K] in the A/B dtype", name);
        return CODA_ERR_INVALID_ARG;
      }
      if (!(std::isfinite(o.scalar) && o.scalar >= 0.0f)) {
        set_error("%s eps must be finite and >= 0", name);
        return CODA_ERR_INVALID_ARG;
      }
      if (!aligned(o.in, 16)) {
        set_error("gamma must be 16-byte aligned");
        return CODA_ERR_UNSUPPORTED;
      }
      if (ln) {
        if (!o.in2) {
          set_error("LN_ROWSCALE needs u = gamma^T B [N] in in2");
          return CODA_ERR_INVALID_ARG;
        }
        if (!aligned(o.in2, 16)) {
          set_error("LN_ROWSCALE u must be 16-byte aligned");
          return CODA_ERR_UNSUPPORTED;
        }
      }
      if (o.row_sumsq || o.row_sum) {   // given row statistics: the gain must be in B
        if (o.in) {
          set_error("%s with given row statistics needs the gain folded into B (in = NULL)", name);
          return CODA_ERR_UNSUPPORTED;
        }
        if (!o.row_sumsq || (ln && !o.row_sum)) {
          set_error("%s: given row statistics need row_sumsq%s", name, ln ? " and row_sum" : "");
          return CODA_ERR_INVALID_ARG;
        }
        if (o.row_ld < 1 || !aligned(o.row_sumsq, 4) || !aligned(o.row_sum, 4)) {
          set_error("%s row statistics: row_ld >= 1 and 4-byte alignment", name);
          return CODA_ERR_INVALID_ARG;
        }
        p->row_ss = static_cast<const float*>(o.row_sumsq);
        p->row_s = static_cast<const float*>(o.row_sum);
        p->row_ss_stride = o.row_ld;
      }
      p->has_norm = true;
      p->has_ln = ln;
      p->gain_in_b = folded;
      p->gamma = o.in;
      p->ln_u = ln ? static_cast<const float*>(o.in2) : nullptr;
      p->eps = o.scalar;
      continue;
    }
    Op& q = p->ops[p->n_ops];
    q.kind = o.kind;
    q.dtype = o.in_dtype;
    q.in = o.in;
    q.ld = o.ld;
    q.scalar = o.scalar;
    q.out = o.out;
    q.out_stride = o.out_stride;
    q.red_slot = -1;
    q.width = width;
    q.in2 = nullptr;
    q.row_s = q.row_ss = nullptr;
    q.row_ld = 0;
    q.seed = q.offset = 0;
    q.thr = 0;
    if (o.kind == CODA_OP_DROPOUT) {
      // keep when the element's 32-bit word >= floor(p * 2^32); kept values
      // are scaled by 1 / (1 - p), rounded once to fp32
      if (!(std::isfinite(o.scalar) && o.scalar >= 0.0f && o.scalar < 1.0f)) {
        set_error("op %d: DROPOUT probability must be in [0, 1)", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (o.in) {
        set_error("op %d: DROPOUT takes no input (in must be NULL)", i);
        return CODA_ERR_INVALID_ARG;
      }
      const double pd = double(o.scalar);
      q.thr = uint32_t(std::floor(pd * 4294967296.0));
      q.scalar = float(1.0 / (1.0 - pd));
      q.seed = o.seed;
      q.offset = o.offset;
    }
    if (bwd) {
      if (width == 0) {
        set_error("op %d: RMS_BWD needs width > 0", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!o.in2 || !o.row_sum || !o.row_sumsq) {
        set_error("op %d: RMS_BWD needs gamma in in2 and the row vectors row_sum (t) and row_sumsq", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!aligned(o.in2, 16)) {
        set_error("op %d: RMS_BWD gamma must be 16-byte aligned", i);
        return CODA_ERR_UNSUPPORTED;
      }
      if (o.row_ld < 1 || !aligned(o.row_sumsq, 4) || !aligned(o.row_sum, 4)) {
        set_error("op %d: RMS_BWD row vectors: row_ld >= 1 and 4-byte alignment", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!(std::isfinite(o.scalar) && o.scalar >= 0.0f)) {
        set_error("op %d: RMS_BWD eps must be finite and >= 0", i);
        return CODA_ERR_INVALID_ARG;
      }
      q.in2 = o.in2;
      q.row_s = static_cast<const float*>(o.row_sum);
      q.row_ss = static_cast<const float*>(o.row_sumsq);
      q.row_ld = o.row_ld;
    }
    if (dgam) {
      if (!o.row_sumsq || o.row_ld < 1 || !aligned(o.row_sumsq, 4)) {
        set_error("op %d: RMS_DGAMMA needs row_sumsq (4-byte aligned) and row_ld >= 1", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!(std::isfinite(o.scalar) && o.scalar >= 0.0f)) {
        set_error("op %d: RMS_DGAMMA eps must be finite and >= 0", i);
        return CODA_ERR_INVALID_ARG;
      }
      q.row_ss = static_cast<const float*>(o.row_sumsq);
      q.row_ld = o.row_ld;
    }
    if (needs_vector(o.kind) || needs_matrix(o.kind)) {
      if (!o.in) {
        set_error("op %d: input is NULL", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!valid_dtype(o.in_dtype)) {
        set_error("op %d: unknown input dtype %d", i, o.in_dtype);
        return CODA_ERR_INVALID_ARG;
      }
      if (!aligned(o.in, 16)) {
        set_error("op %d: input must be 16-byte aligned", i);
        return CODA_ERR_UNSUPPORTED;
      }
    }
    if (needs_matrix(o.kind)) {
      if (o.ld < width) {
        set_error("op %d: ld=%lld < width=%lld", i, (long long)o.ld, (long long)width);
        return CODA_ERR_INVALID_ARG;
      }
      if (o.ld % 8 != 0) {
        set_error("op %d: ld must be a multiple of 8", i);
        return CODA_ERR_UNSUPPORTED;
      }
    }
    if ((o.kind == CODA_OP_SCALE || o.kind == CODA_OP_ADD_MAT) && !std::isfinite(o.scalar)) {
      set_error("op %d: scalar must be finite", i);
      return CODA_ERR_INVALID_ARG;
    }
    if (o.kind == CODA_OP_SWIGLU_PAIR) {
      if (p->has_swiglu) {
        set_error("op %d: SWIGLU_PAIR at most once", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (width % 2 != 0) {
        set_error("op %d: SWIGLU_PAIR needs an even width (N=%lld)", i, (long long)width);
        return CODA_ERR_INVALID_ARG;
      }
      p->has_swiglu = true;
      width /= 2;
    }
    if (is_reduction(o.kind)) {
      if (n_red >= CODA_MAX_REDUCTIONS) {
        set_error("more than %d reductions", CODA_MAX_REDUCTIONS);
        return CODA_ERR_UNSUPPORTED;
      }
      if (!o.out || o.out_stride < 1) {
        set_error("op %d: reduction needs out != NULL and out_stride >= 1", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!aligned(o.out, 4)) {
        set_error("op %d: reduction output must be 4-byte aligned", i);
        return CODA_ERR_UNSUPPORTED;
      }
      q.red_slot = n_red++;
    }
    if (is_col_reduction(o.kind)) {
      if (n_col >= CODA_MAX_COL_REDUCTIONS) {
        set_error("more than %d column reductions", CODA_MAX_COL_REDUCTIONS);
        return CODA_ERR_UNSUPPORTED;
      }
      if (!o.out || o.out_stride < 1) {
        set_error("op %d: reduction needs out != NULL and out_stride >= 1", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (!aligned(o.out, 4)) {
        set_error("op %d: reduction output must be 4-byte aligned", i);
        return CODA_ERR_UNSUPPORTED;
      }
      q.red_slot = n_col++;
    }
    p->n_ops++;
  }
  p->n_red = n_red;
  p->n_colred = n_col;
  p->out_width = width;
  for (int i = 0; i < p->n_ops; ++i) {
    const int k = p->ops[i].kind;
    if (is_col_reduction(k) || k == CODA_OP_ROW_DOT || k == CODA_OP_RMS_BWD) p->has_ext = true;
  }
  for (int i = 0; i < p->n_ops; ++i) {
    const int k = p->ops[i].kind;
    if (k == CODA_OP_SWIGLU_PAIR) break;
    if ((k == CODA_OP_ADD_MAT || k == CODA_OP_MUL_DGELU_TANH) && p->ops[i].dtype == CODA_BF16) {
      p->has_side = true;
      break;
    }
  }
  if (p->has_norm && p->has_ext) {
    set_error("column reductions, ROW_DOT, RMS_BWD and RMS_DGAMMA cannot follow RMS_ROWSCALE / LN_ROWSCALE");
    return CODA_ERR_UNSUPPORTED;
  }

  // ---- shapes, leading dimensions, alignment ----
  const bool empty = (M == 0 || N == 0);
  if (empty) {
    // a no-op: only the descriptor's structure is checked
    p->grid_m = p->grid_n = 0;
    p->cfg = d->ab_dtype == CODA_F32 ? kF32Tile : kTileCfgs[0];
    p->split_s = 1;
    return CODA_OK;
  }
  if (K % 8 != 0) {
    set_error("K=%lld must be a multiple of 8", (long long)K);
    return CODA_ERR_UNSUPPORTED;
  }
  if (d->b_layout == CODA_B_KN && N % 8 != 0) {
    set_error("N=%lld must be a multiple of 8 when B is stored [K x N]", (long long)N);
    return CODA_ERR_UNSUPPORTED;
  }
  const bool akm = d->a_layout == CODA_A_KM;
  if (akm && (M % 8 != 0 || d->ab_dtype != CODA_BF16 || p->has_norm)) {
    set_error("A stored [K x M] needs M %% 8 == 0, bf16 operands and no RMS/LN_ROWSCALE");
    return CODA_ERR_UNSUPPORTED;
  }
  if (d->lda < (akm ? M : K) || d->ldb < (d->b_layout == CODA_B_KN ? N : K) || d->ldd < width) {
    set_error("leading dimension too small (lda=%lld ldb=%lld ldd=%lld)", (long long)d->lda,
              (long long)d->ldb, (long long)d->ldd);
    return CODA_ERR_INVALID_ARG;
  }
  if (d->lda > kMaxLd || d->ldb > kMaxLd) {
    set_error("lda/ldb above %lld elements", (long long)kMaxLd);
    return CODA_ERR_UNSUPPORTED;
  }
  if (d->lda % 8 || d->ldb % 8 || d->ldd % 8) {
    set_error("leading dimensions must be multiples of 8");
    return CODA_ERR_UNSUPPORTED;
  }
  if (check_pointers) {
    if ((K > 0 && (!A || !B)) || !d->D) {
      set_error("A, B or D is NULL");
      return CODA_ERR_INVALID_ARG;
    }
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(d->D, 16)) {
      set_error("A, B and D must be 16-byte aligned");
      return CODA_ERR_UNSUPPORTED;
    }
  }

  // ---- tile ----
  if (d->ab_dtype == CODA_F32) {
    p->tile = 0;
    p->cfg = kF32Tile;
  } else {
    p->tile = d->tile ? d->tile : choose_tile(M, N, K, !(d->flags & CODA_FLAG_NO_SPLIT_K));
    p->cfg = kTileCfgs[p->tile - 1];
  }
  p->grid_m = (M + p->cfg.bm - 1) / p->cfg.bm;
  p->grid_n = (N + p->cfg.bn - 1) / p->cfg.bn;
  if (p->grid_m * p->grid_n * kMaxSplit > kMaxDim) {
    set_error("too many tiles");
    return CODA_ERR_UNSUPPORTED;
  }
  p->k_steps = (K + p->cfg.bk - 1) / p->cfg.bk;
  p->split_allowed = !(d->flags & CODA_FLAG_NO_SPLIT_K);
  plan_split(p, !unfused && p->split_allowed, max_split);

  // ---- overlap ----
  if (check_pointers) {
    const size_t abs = dtype_size(d->ab_dtype), ds = dtype_size(d->d_dtype);
    Extent eD = matrix_extent(d->D, M, width, d->ldd, ds);
    Extent eA = akm ? matrix_extent(A, K, M, d->lda, abs) : matrix_extent(A, M, K, d->lda, abs);
    Extent eB = d->b_layout == CODA_B_KN ? matrix_extent(B, K, N, d->ldb, abs)
                                         : matrix_extent(B, N, K, d->ldb, abs);
    if (overlap(eD, eA) || overlap(eD, eB)) {
      set_error("D overlaps A or B");
      return CODA_ERR_INVALID_ARG;
    }
    if (p->gamma && overlap(eD, matrix_extent(p->gamma, 1, K, K, abs))) {
      set_error("D overlaps gamma");
      return CODA_ERR_INVALID_ARG;
    }
    if (p->has_ln && overlap(eD, matrix_extent(p->ln_u, 1, N, N, 4))) {
      set_error("D overlaps LN_ROWSCALE's u");
      return CODA_ERR_INVALID_ARG;
    }
    Extent outs[CODA_MAX_REDUCTIONS + CODA_MAX_COL_REDUCTIONS];
    int64_t strides[CODA_MAX_REDUCTIONS + CODA_MAX_COL_REDUCTIONS];
    int no = 0;
    for (int i = 0; i < p->n_ops; ++i) {
      const Op& q = p->ops[i];
      if (needs_vector(q.kind) || needs_matrix(q.kind)) {
        const size_t es = dtype_size(q.dtype);
        Extent e;
        if (q.kind == CODA_OP_SCALE_ROW || q.kind == CODA_OP_ADD_ROW) e = matrix_extent(q.in, 1, M, M, es);
        else if (needs_vector(q.kind)) e = matrix_extent(q.in, 1, q.width, q.width, es);
        else e = matrix_extent(q.in, M, q.width, q.ld, es);
        bool exact_alias = q.kind == CODA_OP_ADD_MAT && q.in == d->D && q.ld == d->ldd &&
                           q.dtype == d->d_dtype && q.width == width;
        if (!exact_alias && overlap(e, eD)) {
          set_error("op %d input overlaps D (only an exact in-place ADD_MAT is allowed)", i);
          return CODA_ERR_INVALID_ARG;
        }
      }
      if (q.kind == CODA_OP_RMS_DGAMMA && overlap(matrix_extent(q.row_ss, M, 1, q.row_ld, 4), eD)) {
        set_error("op %d: RMS_DGAMMA row_sumsq overlaps D", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (q.kind == CODA_OP_RMS_BWD &&
          (overlap(matrix_extent(q.in2, 1, q.width, q.width, dtype_size(q.dtype)), eD) ||
           overlap(matrix_extent(q.row_s, M, 1, q.row_ld, 4), eD) ||
           overlap(matrix_extent(q.row_ss, M, 1, q.row_ld, 4), eD))) {
        set_error("op %d: RMS_BWD gamma or row vectors overlap D", i);
        return CODA_ERR_INVALID_ARG;
      }
      if (is_reduction(q.kind) || is_col_reduction(q.kind)) {
        Extent e = is_col_reduction(q.kind) ? matrix_extent(q.out, q.width, 1, q.out_stride, 4)
                                            : matrix_extent(q.out, M, 1, q.out_stride, 4);
        if (overlap(e, eD) || overlap(e, eA) || overlap(e, eB)) {
          set_error("reduction output of op %d overlaps D, A or B", i);
          return CODA_ERR_INVALID_ARG;
        }
        for (int j = 0; j < no; ++j) {
          if (!overlap(e, outs[j])) continue;
          // interleaved columns of one [M x s] array are fine: same stride, distinct offsets
          intptr_t diff = intptr_t(e.lo) - intptr_t(outs[j].lo);
          bool interleaved = strides[j] == q.out_stride &&
                             (diff % (intptr_t)(4 * q.out_stride)) != 0;
          if (!interleaved) {
            set_error("reduction outputs overlap (op %d)", i);
            return CODA_ERR_INVALID_ARG;
          }
        }
        outs[no] = e;
        strides[no] = q.out_stride;
        ++no;
      }
    }
    // A reduction output must not overlap anything the same call reads: the
    // fused kernel and the unfused sequence read inputs at different times
    // relative to the writes, so the two paths would disagree.
    Strided ins[4 + 4 * CODA_MAX_OPS];
    int ni = 0;
    if (p->gamma) ins[ni++] = dense(matrix_extent(p->gamma, 1, K, K, abs));
    if (p->ln_u) ins[ni++] = dense(matrix_extent(p->ln_u, 1, N, N, 4));
    if (p->row_ss) ins[ni++] = column(p->row_ss, M, p->row_ss_stride);
    if (p->row_s) ins[ni++] = column(p->row_s, M, p->row_ss_stride);
    for (int i = 0; i < p->n_ops; ++i) {
      const Op& q = p->ops[i];
      if (q.in && (needs_vector(q.kind) || needs_matrix(q.kind))) {
        const size_t es = dtype_size(q.dtype);
        if (q.kind == CODA_OP_SCALE_ROW || q.kind == CODA_OP_ADD_ROW) ins[ni++] = dense(matrix_extent(q.in, 1, M, M, es));
        else if (needs_vector(q.kind)) ins[ni++] = dense(matrix_extent(q.in, 1, q.width, q.width, es));
        else ins[ni++] = dense(matrix_extent(q.in, M, q.width, q.ld, es));
      }
      if (q.in2) ins[ni++] = dense(matrix_extent(q.in2, 1, q.width, q.width, dtype_size(q.dtype)));
      if (q.row_s) ins[ni++] = column(q.row_s, M, q.row_ld);
      if (q.row_ss) ins[ni++] = column(q.row_ss, M, q.row_ld);
    }
    for (int i = 0; i < p->n_ops; ++i) {
      const Op& q = p->ops[i];
      if (!is_reduction(q.kind) && !is_col_reduction(q.kind)) continue;
      const Strided o = column(q.out, is_col_reduction(q.kind) ? q.width : M, q.out_stride);
      for (int j = 0; j < ni; ++j) {
        if (strided_overlap(o, ins[j])) {
          set_error("reduction output of op %d overlaps an input read by the same call", i);
          return CODA_ERR_INVALID_ARG;
        }
      }
    }
  }

  if (unfused && p->n_colred > 0 && (M + kColChunk - 1) / kColChunk > 65535) {
    set_error("unfused column reductions support at most %lld rows", (long long)kColChunk * 65535);
    return CODA_ERR_UNSUPPORTED;
  }

  // ---- workspace ----
  {
    size_t need = unfused ? unfused_workspace_bytes(*p) : fused_workspace_bytes(*p);
    if (need > 0 && check_pointers) {
      if (!d->workspace || d->workspace_bytes < need) {
        set_error("workspace of %zu bytes needed, %zu given", need, d->workspace_bytes);
        return CODA_ERR_WORKSPACE;
      }
      if (!aligned(d->workspace, 256)) {
        set_error("workspace must be 256-byte aligned");
        return CODA_ERR_UNSUPPORTED;
      }
    }
  }
  return CODA_OK;
}

int validate_fold_gain(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                       const void* gamma, const void* B_out, int64_t ldo) {
  clear_error();
  if (K < 0 || N < 0) {
    set_error("negative size K=%lld N=%lld", (long long)K, (long long)N);
    return CODA_ERR_INVALID_ARG;
  }
  if (K > kMaxDim || N > kMaxDim) {
    set_error("size above 2^31-1");
    return CODA_ERR_UNSUPPORTED;
  }
  if (!valid_dtype(dtype) || (b_layout != CODA_B_KN && b_layout != CODA_B_NK)) {
    set_error("unknown dtype %d or B layout %d", dtype, b_layout);
    return CODA_ERR_INVALID_ARG;
  }
  if (K == 0 || N == 0) return CODA_OK;
  if (!B || !gamma || !B_out) {
    set_error("B, gamma or B_out is NULL");
    return CODA_ERR_INVALID_ARG;
  }
  const int64_t inner = b_layout == CODA_B_KN ? N : K;
  if (ldb < inner || ldo < inner) {
    set_error("ldb=%lld or ldo=%lld below %lld", (long long)ldb, (long long)ldo, (long long)inner);
    return CODA_ERR_INVALID_ARG;
  }
  if (inner % 8 || ldb % 8 || ldo % 8) {
    set_error("the contiguous dimension and ldb, ldo must be multiples of 8");
    return CODA_ERR_UNSUPPORTED;
  }
  if (!aligned(B, 16) || !aligned(gamma, 16) || !aligned(B_out, 16)) {
    set_error("B, gamma and B_out must be 16-byte aligned");
    return CODA_ERR_UNSUPPORTED;
  }
  const size_t es = dtype_size(dtype);
  const int64_t rows = b_layout == CODA_B_KN ? K : N;
  const Extent eB = matrix_extent(B, rows, inner, ldb, es), eO = matrix_extent(B_out, rows, inner, ldo, es);
  const Extent eg = matrix_extent(gamma, 1, K, K, es);
  const bool in_place = B == B_out && ldb == ldo;
  if ((!in_place && overlap(eB, eO)) || overlap(eO, eg)) {
    set_error("B_out overlaps B (other than exactly in place) or gamma");
    return CODA_ERR_INVALID_ARG;
  }
  return CODA_OK;
}

int validate_ln_fold(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                     const void* gamma, const void* beta, const float* u, const float* c) {
  clear_error();
  if (K < 0 || N < 0) {
    set_error("negative size K=%lld N=%lld", (long long)K, (long long)N);
    return CODA_ERR_INVALID_ARG;
  }
  if (K > kMaxDim || N > kMaxDim) {
    set_error("size above 2^31-1");
    return CODA_ERR_UNSUPPORTED;
  }
  if (!valid_dtype(dtype) || (b_layout != CODA_B_KN && b_layout != CODA_B_NK)) {
    set_error("unknown dtype %d or B layout %d", dtype, b_layout);
    return CODA_ERR_INVALID_ARG;
  }
  if ((beta == nullptr) != (c == nullptr)) {
    set_error("beta and c must be both NULL or both set");
    return CODA_ERR_INVALID_ARG;
  }
  if (N == 0) return CODA_OK;
  if (!u || (K > 0 && (!B || !gamma))) {
    set_error("B, gamma or u is NULL");
    return CODA_ERR_INVALID_ARG;
  }
  if (ldb < (b_layout == CODA_B_KN ? N : K)) {
    set_error("ldb=%lld too small", (long long)ldb);
    return CODA_ERR_INVALID_ARG;
  }
  if (K % 8 || ldb % 8 || (b_layout == CODA_B_KN && N % 8)) {
    set_error("K, ldb (and N for B stored [K x N]) must be multiples of 8 (K=%lld N=%lld ldb=%lld)",
              (long long)K, (long long)N, (long long)ldb);
    return CODA_ERR_UNSUPPORTED;
  }
  if (!aligned(B, 16) || !aligned(gamma, 16) || !aligned(beta, 16) || !aligned(u, 16) || !aligned(c, 16)) {
    set_error("B, gamma, beta, u and c must be 16-byte aligned");
    return CODA_ERR_UNSUPPORTED;
  }
  const size_t es = dtype_size(dtype);
  // a NULL c / beta has no extent
  auto vec = [](const void* q, int64_t n, size_t e) { return q ? matrix_extent(q, 1, n, n, e) : Extent{0, 0}; };
  const Extent eu = vec(u, N, 4), ec = vec(c, N, 4);
  const Extent eB = b_layout == CODA_B_KN ? matrix_extent(B, K, N, ldb, es) : matrix_extent(B, N, K, ldb, es);
  const Extent eg = vec(gamma, K, es), eb = vec(beta, K, es);
  if (overlap(eu, ec) || overlap(eu, eB) || overlap(ec, eB) || overlap(eu, eg) || overlap(ec, eg) ||
      overlap(eu, eb) || overlap(ec, eb)) {
    set_error("u or c overlaps an input or each other");
    return CODA_ERR_INVALID_ARG;
  }
  return CODA_OK;
}

}  // namespace coda

extern "C" {

int coda_validate(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                  const coda_epi_desc* desc, int unfused) {
  coda::Plan p;
  return coda::build_plan(A, B, M, N, K, desc, unfused, true, &p);
}

size_t coda_workspace_size(int64_t M, int64_t N, int64_t K, const coda_epi_desc* desc, int unfused) {
  coda::Plan p;
  if (coda::build_plan(nullptr, nullptr, M, N, K, desc, unfused, false, &p) != CODA_OK) return 0;
  if (M == 0 || N == 0) return 0;
  return unfused ? coda::unfused_workspace_bytes(p) : coda::fused_workspace_bytes(p);
}

const char* coda_status_string(int status) {
  switch (status) {
    case CODA_OK: return "CODA_OK";
    case CODA_ERR_INVALID_ARG: return "CODA_ERR_INVALID_ARG";
    case CODA_ERR_UNSUPPORTED: return "CODA_ERR_UNSUPPORTED";
    case CODA_ERR_WORKSPACE: return "CODA_ERR_WORKSPACE";
    case CODA_ERR_HIP: return "CODA_ERR_HIP";
    default: return "CODA_UNKNOWN_STATUS";
  }
}

const char* coda_last_error(void) { return coda::last_error(); }

int coda_num_tile_configs(void) { return coda::kNumTileCfgs; }

int coda_selected_tile(int64_t M, int64_t N, int64_t K, const coda_epi_desc* desc) {
  coda::Plan p;
  const int st = coda::build_plan(nullptr, nullptr, M, N, K, desc, 0, false, &p);
  if (st != CODA_OK) return st;
  if (desc->ab_dtype == CODA_F32) return 0;
  return desc->tile ? desc->tile : coda::choose_tile(M, N, K, !(desc->flags & CODA_FLAG_NO_SPLIT_K));
}

int coda_tile_config(int index, int* bm, int* bn, int* bk, int* waves) {
  if (index < 1 || index > coda::kNumTileCfgs) return CODA_ERR_INVALID_ARG;
  const coda::TileCfg& c = coda::kTileCfgs[index - 1];
  if (bm) *bm = c.bm;
  if (bn) *bn = c.bn;
  if (bk) *bk = c.bk;
  if (waves) *waves = c.wm * c.wn;
  return CODA_OK;
}

}  // extern "C"
