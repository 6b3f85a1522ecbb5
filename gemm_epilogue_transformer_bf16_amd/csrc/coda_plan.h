// Host-side plan of one call: the validated, normalised form of a coda_epi_desc.
// Pure C++ (no HIP types) so that validation can be built and tested on the host alone.
#pragma once

#include <cstddef>
#include <cstdint>

#include "coda.h"

namespace coda {

// bf16 tile configurations: output tile bm x bn (rows of A x columns of B),
// K step bk, wavefronts arranged wm x wn over the tile.
// wg_per_cu: workgroups of the configuration that fit on one CU at once (LDS
// bound), used to size the split of the last, partial round of tiles.
struct TileCfg {
  int bm, bn, bk, wm, wn, wg_per_cu;
};

constexpr TileCfg kTileCfgs[] = {
    {256, 128, 64, 4, 2, 1},   // 1: 8 waves, 64x64 per wave
    {128, 128, 64, 2, 2, 2},   // 2: 4 waves, 64x64 per wave
    {256, 256, 64, 2, 4, 1},   // 3: 8 waves, 128x64 per wave
};
constexpr int kNumTileCfgs = sizeof(kTileCfgs) / sizeof(kTileCfgs[0]);

// fp32 operands use one small configuration.
constexpr TileCfg kF32Tile = {64, 64, 32, 2, 2, 4};

// Compute units of an MI355X; the split below balances the grid for this count
// (on another device the result is the same, only the balance differs).
constexpr int kNumCUs = 256;
constexpr int kMaxSplit = 4;
// main-loop rate of the 256 x 128 tile relative to the 256 x 256 one, per CU
constexpr double kTile1Speed = 0.95;
// Fewest K steps per part: the parts exchange fp32 partial tiles through
// memory, which costs about as much as 8 - 16 K steps of the main loop.
constexpr int kMinSplitSteps = 16;

struct Op {
  int kind;
  int dtype;
  const void* in;
  int64_t ld;
  float scalar;
  void* out;
  int64_t out_stride;
  int red_slot;      // index among the row (or, for COL_*, the column) reductions, -1 otherwise
  int64_t width;     // width of the running value when the op runs
  const void* in2;   // RMS_BWD: gamma [width] (dtype)
  const float* row_s;   // RMS_BWD: t per row
  const float* row_ss;  // RMS_BWD: sum of squares of x per row
  int64_t row_ld;
  uint64_t seed, offset;   // DROPOUT: the generator's key word 0 and counter word 2
  uint32_t thr;            // DROPOUT: keep when the element's 32-bit word >= thr (scalar = 1 / (1 - p))
};

struct Plan {
  int ab_dtype, d_dtype, b_layout, a_layout;
  int64_t M, N, K, lda, ldb, ldd;
  int64_t out_width;
  const void* A;
  const void* B;
  void* D;
  bool has_norm;             // a deferred row norm (RMS_ROWSCALE or LN_ROWSCALE) is op 0
  bool has_ln;               // ... and it is LN_ROWSCALE
  bool gain_in_b;            // RMS_ROWSCALE with gamma NULL: the gain is folded into B
  const void* gamma;
  const float* ln_u;         // LN_ROWSCALE: u = gamma^T B [N]
  const float* row_ss;       // given row sums of squares (stride row_ss_stride), or null
  const float* row_s;        // LN_ROWSCALE: given row sums (same stride), or null
  int64_t row_ss_stride;
  float eps;
  int n_ops;                 // ops after the norm op
  Op ops[CODA_MAX_OPS];
  int n_red;
  int n_colred;              // column reductions
  bool has_swiglu;
  bool has_ext;              // a backward-set op: column reduction, ROW_DOT, RMS_BWD or RMS_DGAMMA
  bool has_side;             // a bf16 ADD_MAT / MUL_DGELU_TANH before any SWIGLU_PAIR (read ahead)
  int tile;                  // 1-based bf16 tile config; 0 for the fp32 path
  TileCfg cfg;
  int64_t grid_m, grid_n;
  // Split of the last round: when the tiles do not fill a whole number of
  // rounds of the GPU, the last `split_tiles` tiles (in launch order) are each
  // computed by `split_s` workgroups over consecutive parts of K; the last of
  // them to finish adds the partial accumulators and runs the epilogue.
  int64_t k_steps;           // K steps of the tile configuration
  int64_t full_tiles;        // tiles computed whole
  int64_t split_tiles;       // tiles split over K
  int split_s;               // parts per split tile (1: no split)
  bool split_allowed;        // the caller did not set CODA_FLAG_NO_SPLIT_K
  void* workspace;
  size_t workspace_bytes;
};

// Validates and normalises a call.  Returns a coda_status; on error records a
// message retrievable through coda_last_error().
int build_plan(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
               const coda_epi_desc* desc, int unfused, bool check_pointers, Plan* plan);
// The same, with the split of the last round limited to max_split parts per
// tile (1: no split), e.g. to fit a fixed scratch buffer.
int build_plan_split(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                     const coda_epi_desc* desc, int unfused, bool check_pointers, int max_split, Plan* plan);

// Workspace layout of the fused path, each region 256-byte aligned: fp32 row
// reduction partials [n_red][grid_n][M], uint32 counters [grid_m]; then for
// split tiles fp32 partial accumulators [split_tiles][split_s][bm * bn], fp32
// partial row sums of squares [split_tiles][split_s][bm] (RMS op only) and
// uint32 counters [split_tiles].
size_t fused_workspace_bytes(const Plan& p);
size_t fused_partials_offset(const Plan& p);
size_t fused_counters_offset(const Plan& p);
size_t fused_split_acc_offset(const Plan& p);
size_t fused_split_ss_offset(const Plan& p);
size_t fused_split_counters_offset(const Plan& p);
// then, with column reductions over several tile rows: fp32 column partials
// [n_colred][grid_m][N] and uint32 counters [grid_n]
size_t fused_col_partials_offset(const Plan& p);
size_t fused_col_counters_offset(const Plan& p);

// Workspace layout of the unfused path: normalised A (ab dtype, [M x K]) when
// the list has the RMS op, then two [M x ldi] intermediates in d dtype, with
// ldi = N rounded up to a multiple of 8, then (column reductions) fp32 column
// partials [ceil(M / kColChunk)][ldi].
constexpr int kColChunk = 128;
size_t unfused_workspace_bytes(const Plan& p);
int64_t unfused_ld(const Plan& p);
size_t unfused_col_partials_offset(const Plan& p);
// The plain GEMM of the unfused sequence: the call's plan without a row norm
// or ops, with the split of the last round a fused call of that GEMM would
// use; its workspace (split partial tiles and counters, zero counters on
// entry and exit) sits at unfused_split_offset(p) in the unfused workspace.
Plan plain_gemm_plan(const Plan& p);
size_t unfused_split_offset(const Plan& p);

// Validates a coda_ln_fold call.  Returns a coda_status.
int validate_ln_fold(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                     const void* gamma, const void* beta, const float* u, const float* c);

// Validates a coda_fold_gain call.  Returns a coda_status.
int validate_fold_gain(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                       const void* gamma, const void* B_out, int64_t ldo);

// Automatic bf16 tile configuration (1-based) for an M x N output.
int choose_tile(int64_t M, int64_t N, int64_t K, bool split_allowed);

void set_error(const char* fmt, ...);
void clear_error();

inline size_t dtype_size(int dt) { return dt == CODA_F32 ? 4 : 2; }

}  // namespace coda
