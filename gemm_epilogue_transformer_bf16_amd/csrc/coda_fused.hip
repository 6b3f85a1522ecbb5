// Host side of the fused kernel: argument packing and dispatch to the
// compiled tile configurations.
#include "coda_fused_impl.h"
#include "coda_launch.h"

namespace coda {

// the kernel's split finalization holds one slot per part
static_assert(kMaxSplit <= dev::kMaxSplitParts, "split parts beyond the kernel's slots");

namespace {

dev::FusedArgs make_args(const Plan& p) {
  dev::FusedArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = p.A;
  a.B = p.B;
  a.D = p.D;
  a.gamma = p.gamma;
  a.ln_u = p.ln_u;
  a.row_ss = p.row_ss;
  a.row_s = p.row_s;
  a.row_ss_stride = p.row_ss_stride;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldd = p.ldd;
  a.M = (int)p.M;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.d_dtype = p.d_dtype;
  a.out_width = (int)p.out_width;
  a.n_ops = p.n_ops;
  a.n_red = p.n_red;
  a.n_colred = p.n_colred;
  a.grid_m = (int)p.grid_m;
  a.grid_n = (int)p.grid_n;
  a.eps = p.eps;
  for (int i = 0; i < p.n_ops; ++i) {
    const Op& q = p.ops[i];
    dev::DevOp& d = a.ops[i];
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
  }
  char* ws = static_cast<char*>(p.workspace);
  if (p.n_red > 0 && p.grid_n > 1) {
    a.partials = reinterpret_cast<float*>(ws + fused_partials_offset(p));
    a.counters = reinterpret_cast<unsigned*>(ws + fused_counters_offset(p));
  }
  if (p.n_colred > 0 && p.grid_m > 1) {
    a.col_partials = reinterpret_cast<float*>(ws + fused_col_partials_offset(p));
    a.col_counters = reinterpret_cast<unsigned*>(ws + fused_col_counters_offset(p));
  }
  a.full_tiles = (int)p.full_tiles;
  a.split_s = p.split_s;
  a.k_steps = (int)p.k_steps;
  if (p.split_s > 1) {
    a.split_acc = reinterpret_cast<float*>(ws + fused_split_acc_offset(p));
    a.split_ss = reinterpret_cast<float*>(ws + fused_split_ss_offset(p));
    a.split_cnt = reinterpret_cast<unsigned*>(ws + fused_split_counters_offset(p));
  }
  return a;
}

int launch_args(const Plan& p, const dev::FusedArgs& a, hipStream_t stream) {
  const int64_t nwg = p.full_tiles + p.split_tiles * p.split_s;
  const bool bkn = p.b_layout == CODA_B_KN;
  const bool akm = p.a_layout == CODA_A_KM;
  const int norm = p.has_ln      ? (p.row_ss ? dev::kNormLnGiven : p.gain_in_b ? dev::kNormLnB : dev::kNormLn)
                   : p.row_ss    ? dev::kNormRmsGiven
                   : p.gain_in_b ? dev::kNormRmsB
                   : p.has_norm  ? dev::kNormRms
                                 : dev::kNormNone;
  const bool ext = p.has_ext;
  const bool side = p.has_side;
  if (p.ab_dtype == CODA_F32) {
    return dev::launch_tile_f32(a, nwg, bkn, norm, akm, ext, side, stream);
  }
  if (norm != dev::kNormNone) {
    switch (p.tile) {
      case 1: return dev::launch_tile1_norm(a, nwg, bkn, norm, stream);
      case 2: return dev::launch_tile2_norm(a, nwg, bkn, norm, stream);
      case 3: return dev::launch_tile3_norm(a, nwg, bkn, norm, stream);
      default:
        set_error("no kernel for tile config %d", p.tile);
        return CODA_ERR_UNSUPPORTED;
    }
  }
  switch (p.tile) {
    case 1: return dev::launch_tile1(a, nwg, bkn, akm, ext, side, stream);
    case 2: return dev::launch_tile2(a, nwg, bkn, akm, ext, side, stream);
    case 3: return dev::launch_tile3(a, nwg, bkn, akm, ext, side, stream);
    default:
      set_error("no kernel for tile config %d", p.tile);
      return CODA_ERR_UNSUPPORTED;
  }
}

}  // namespace

int launch_fused(const Plan& p, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return CODA_OK;
  dev::FusedArgs a = make_args(p);
  return launch_args(p, a, stream);
}

int launch_fused_with_counters(const Plan& p, unsigned* counters, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return CODA_OK;
  dev::FusedArgs a = make_args(p);
  // the counters live in a region the caller keeps zero between calls (every
  // call leaves the counters it used at zero): row counters, then column
  // counters, then the split tiles' counters
  if (a.counters) a.counters = counters;
  if (a.col_counters) a.col_counters = counters + p.grid_m;
  if (a.split_cnt) a.split_cnt = counters + p.grid_m + p.grid_n;
  return launch_args(p, a, stream);
}

int launch_plain_gemm(const Plan& p, const void* A, int64_t lda, void* out, int64_t ldo, hipStream_t stream) {
  if (p.M == 0 || p.N == 0) return CODA_OK;
  // the fused kernel with an empty list, split like a fused call of this GEMM
  Plan q = plain_gemm_plan(p);
  q.A = A;
  q.lda = lda;
  q.D = out;
  q.ldd = ldo;
  q.workspace = static_cast<char*>(p.workspace) + unfused_split_offset(p);
  dev::FusedArgs a = make_args(q);
  return launch_args(q, a, stream);
}

}  // namespace coda
