// Host-only checks of the call validation (no GPU, no HIP runtime): every
// invalid descriptor returns its documented status.  Built with
// -fsanitize=address,undefined by tests/test_abi.py.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "coda.h"
#include "coda_plan.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, coda_last_error()); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// fake, well-aligned, non-overlapping device addresses
static const void* P(uintptr_t x) { return reinterpret_cast<const void*>(x); }
static void* Pm(uintptr_t x) { return reinterpret_cast<void*>(x); }

static coda_epi_desc base_desc(int64_t N, int64_t K) {
  coda_epi_desc d;
  std::memset(&d, 0, sizeof(d));
  d.ab_dtype = CODA_BF16;
  d.d_dtype = CODA_BF16;
  d.b_layout = CODA_B_KN;
  d.lda = K;
  d.ldb = N;
  d.ldd = N;
  d.D = Pm(0x30000000);
  // most checks below are about validation, not load balance: keep every tile
  // whole so that no workspace is needed (the split is tested on its own)
  d.flags = CODA_FLAG_NO_SPLIT_K;
  return d;
}

static coda::Plan plan_of(int64_t M, int64_t N, int64_t K, const coda_epi_desc& d, int unfused = 0) {
  coda::Plan p;
  const int st = coda::build_plan(nullptr, nullptr, M, N, K, &d, unfused, false, &p);
  if (st != CODA_OK) std::printf("build_plan failed: %s\n", coda_last_error());
  return p;
}

int main() {
  const void* A = P(0x10000000);
  const void* B = P(0x20000000);
  const int64_t M = 300, N = 520, K = 200;

  coda_epi_desc d = base_desc(N, K);
  EXPECT(coda_validate(A, B, M, N, K, &d, 0) == CODA_OK);
  EXPECT(coda_validate(A, B, M, N, K, nullptr, 0) == CODA_ERR_INVALID_ARG);
  EXPECT(coda_validate(A, B, -1, N, K, &d, 0) == CODA_ERR_INVALID_ARG);
  EXPECT(coda_validate(A, B, 0, N, K, &d, 0) == CODA_OK);   // empty is fine
  {  // K must be a multiple of 8
    coda_epi_desc e = base_desc(N, 204);
    EXPECT(coda_validate(A, B, M, N, 204, &e, 0) == CODA_ERR_UNSUPPORTED);
  }
  {  // N multiple of 8 when B is [K x N]
    coda_epi_desc e = base_desc(521, K);
    e.ldb = 528; e.ldd = 528;
    EXPECT(coda_validate(A, B, M, 521, K, &e, 0) == CODA_ERR_UNSUPPORTED);
    e.b_layout = CODA_B_NK; e.ldb = K;
    EXPECT(coda_validate(A, B, M, 521, K, &e, 0) == CODA_OK);
  }
  {  // leading dimensions
    coda_epi_desc e = d; e.lda = K - 8;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e = d; e.ldd = N + 4;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_UNSUPPORTED);
  }
  {  // misaligned pointers
    EXPECT(coda_validate(P(0x10000008), B, M, N, K, &d, 0) == CODA_ERR_UNSUPPORTED);
  }
  {  // null pointers
    EXPECT(coda_validate(nullptr, B, M, N, K, &d, 0) == CODA_ERR_INVALID_ARG);
    coda_epi_desc e = d; e.D = nullptr;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
  }
  {  // bad enums, flags, tile
    coda_epi_desc e = d; e.ab_dtype = 7;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e = d; e.b_layout = 5;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e = d; e.flags = 2;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e = d; e.tile = coda_num_tile_configs() + 1;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e = d; e.n_ops = CODA_MAX_OPS + 1;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e = d; e.n_ops = 1; e.ops[0].kind = 99;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
  }
  {  // RMS op: first, once, with gamma in the operand dtype, eps >= 0, K > 0
    coda_epi_desc e = d; e.n_ops = 1;
    e.ops[0].kind = CODA_OP_RMS_ROWSCALE; e.ops[0].in = P(0x40000000); e.ops[0].in_dtype = CODA_BF16;
    e.ops[0].scalar = 1e-6f;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    coda_epi_desc f = e; f.ops[0].in = nullptr;   // gamma NULL: the gain is folded into B
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_OK);
    {
      coda::Plan q = plan_of(M, N, K, f);
      EXPECT(q.has_norm && q.gain_in_b && !q.has_ln && q.gamma == nullptr && q.n_ops == 0);
      coda::Plan r = plan_of(M, N, K, e);
      EXPECT(r.has_norm && !r.gain_in_b);
    }
    f = e; f.ops[0].in_dtype = CODA_F32;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].scalar = -1.0f;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.n_ops = 2; f.ops[1] = f.ops[0]; f.ops[0].kind = CODA_OP_GELU_TANH; f.ops[0].in = nullptr;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // not first
    coda_epi_desc g = base_desc(N, 0); g.n_ops = 1; g.ops[0] = e.ops[0];
    EXPECT(coda_validate(A, B, M, N, 0, &g, 0) == CODA_ERR_INVALID_ARG);   // K == 0
  }
  {  // SWIGLU: even width, at most once; D width halves
    coda_epi_desc e = d; e.n_ops = 1; e.ops[0].kind = CODA_OP_SWIGLU_PAIR; e.ldd = N / 2 + 4;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    e.n_ops = 2; e.ops[1].kind = CODA_OP_SWIGLU_PAIR;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    coda_epi_desc f = base_desc(26, K); f.b_layout = CODA_B_NK; f.ldb = K; f.ldd = 32;
    f.n_ops = 2; f.ops[0].kind = CODA_OP_SWIGLU_PAIR; f.ops[1].kind = CODA_OP_SWIGLU_PAIR;
    EXPECT(coda_validate(A, B, M, 26, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f.n_ops = 1;
    EXPECT(coda_validate(A, B, M, 26, K, &f, 0) == CODA_OK);   // 26 even; 13 wide after
    coda_epi_desc h = base_desc(13 * 2 + 1, K); h.b_layout = CODA_B_NK; h.ldb = K; h.ldd = 32;
    h.n_ops = 1; h.ops[0].kind = CODA_OP_SWIGLU_PAIR;
    EXPECT(coda_validate(A, B, M, 27, K, &h, 0) == CODA_ERR_INVALID_ARG);   // odd width
  }
  {  // side inputs: non-null, aligned, ld rules
    coda_epi_desc e = d; e.n_ops = 1; e.ops[0].kind = CODA_OP_ADD_COL;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e.ops[0].in = P(0x40000004);
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_UNSUPPORTED);
    e.ops[0].in = P(0x40000000);
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    e.ops[0].kind = CODA_OP_ADD_MAT; e.ops[0].ld = N - 8;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e.ops[0].ld = N + 4;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_UNSUPPORTED);
    e.ops[0].ld = N;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
  }
  {  // aliasing: exact in-place ADD_MAT is allowed, partial overlap is not
    coda_epi_desc e = d; e.n_ops = 1; e.ops[0].kind = CODA_OP_ADD_MAT; e.ops[0].ld = N;
    e.ops[0].in = d.D; e.ops[0].in_dtype = CODA_BF16;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    e.ops[0].in = P(reinterpret_cast<uintptr_t>(d.D) + 16);
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e.ops[0].in = d.D; e.ops[0].in_dtype = CODA_F32;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    coda_epi_desc f = d; f.D = Pm(reinterpret_cast<uintptr_t>(A) + 256);
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // D overlaps A
  }
  {  // reductions: outputs, stride, interleaved columns, workspace
    coda_epi_desc e = d; e.n_ops = 2;
    e.ops[0].kind = CODA_OP_ROW_SUM; e.ops[0].out = Pm(0x50000000); e.ops[0].out_stride = 2;
    e.ops[1].kind = CODA_OP_ROW_SUMSQ; e.ops[1].out = Pm(0x50000004); e.ops[1].out_stride = 2;
    const size_t ws = coda_workspace_size(M, N, K, &e, 0);
    EXPECT(ws > 0);   // 520 columns span several tiles
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_WORKSPACE);
    e.workspace = Pm(0x60000000); e.workspace_bytes = ws - 1;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_WORKSPACE);
    e.workspace_bytes = ws;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    coda_epi_desc f = e; f.ops[1].out = Pm(0x50000000);
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // same elements
    f = e; f.ops[1].out_stride = 0;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[1].out = nullptr;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[1].out = Pm(0x50000002);
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_UNSUPPORTED);
    coda_epi_desc g = d; g.n_ops = CODA_MAX_REDUCTIONS + 1;
    for (int i = 0; i < g.n_ops; ++i) {
      g.ops[i].kind = CODA_OP_ROW_SUM; g.ops[i].out = Pm(0x50000000 + 0x100000 * i); g.ops[i].out_stride = 1;
    }
    EXPECT(coda_validate(A, B, M, N, K, &g, 0) == CODA_ERR_UNSUPPORTED);
    // unfused workspace covers normalised A and two intermediates
    coda_epi_desc u = d; u.n_ops = 1; u.ops[0].kind = CODA_OP_GELU_TANH;
    EXPECT(coda_workspace_size(M, N, K, &u, 1) >= size_t(2 * M * N * 2));
    EXPECT(coda_validate(A, B, M, N, K, &u, 1) == CODA_ERR_WORKSPACE);
  }
  {  // tile configs
    int bm = 0, bn = 0, bk = 0, w = 0;
    EXPECT(coda_num_tile_configs() >= 1);
    EXPECT(coda_tile_config(1, &bm, &bn, &bk, &w) == CODA_OK && bm > 0 && bn > 0 && bk > 0 && w > 0);
    EXPECT(coda_tile_config(0, &bm, &bn, &bk, &w) == CODA_ERR_INVALID_ARG);
  }
  {  // selected tile: explicit, automatic (by how well the grid fills rounds of 256 CUs), fp32
    coda_epi_desc e = base_desc(22016, 4096); e.flags = 0;
    EXPECT(coda_selected_tile(4096, 22016, 4096, &e) == 3);
    EXPECT(coda_selected_tile(300, 520, 200, &d) == 2);
    // 256 x 128 where it fills whole rounds and 256 x 256 does not:
    // 32 x 24 = 768 tiles (3 rounds) against 384 (1.5 rounds, 12 K steps: no split)
    EXPECT(coda_selected_tile(8192, 3072, 768, &e) == 1);
    // under one round of 256 x 256 (128 tiles): 64 x 8 = 512 tiles of 128 x 128
    // fill one round at two per CU, as well as 256 tiles of 256 x 128 do
    EXPECT(coda_selected_tile(8192, 1024, 4096, &e) == 2);
    // 31 x 8 = 248 tiles of 256 x 128: under one round
    EXPECT(coda_selected_tile(7936, 1024, 4096, &e) == 2);
    // 24 x 12 = 288 of 256 x 128 (2 rounds, 56% busy) against 48 x 12 = 576
    // of 128 x 128 (2 rounds of 512, 56%): ties go to 128 x 128
    EXPECT(coda_selected_tile(6144, 1536, 4096, &e) == 2);
    // 40 x 8 = 320 of 256 x 128 (2 rounds, 62.5%) against 79 x 8 = 632 of
    // 128 x 128 (2 rounds of 512, 61.7%); 256 x 256: 40 x 4 = 160, under a round
    EXPECT(coda_selected_tile(10112, 1024, 4096, &e) == 1);
    // 32 x 16 = 512 tiles of 256 x 256 fill two rounds
    EXPECT(coda_selected_tile(8192, 4096, 1024, &e) == 3);
    // 5.4 rounds of 256 x 256, the last one split over K (64 K steps)
    EXPECT(coda_selected_tile(4096, 22016, 4096, &e) == 3);
    // the same grid with 12 K steps, or without the split: the 256 x 128 grid
    // (10.75 rounds) fills better
    EXPECT(coda_selected_tile(4096, 22016, 768, &e) == 1);
    coda_epi_desc ns = e; ns.flags = CODA_FLAG_NO_SPLIT_K;
    EXPECT(coda_selected_tile(4096, 22016, 4096, &ns) == 1);
    e.tile = 2;
    EXPECT(coda_selected_tile(4096, 22016, 4096, &e) == 2);
    e.ab_dtype = CODA_F32; e.tile = 0;
    EXPECT(coda_selected_tile(4096, 22016, 4096, &e) == 0);
    EXPECT(coda_selected_tile(4096, 22016, 4100, &e) == CODA_ERR_UNSUPPORTED);
  }
  {  // split of the last round over K
    coda_epi_desc e = base_desc(22016, 4096); e.flags = 0; e.ldd = 11008;
    e.n_ops = 1; e.ops[0].kind = CODA_OP_SWIGLU_PAIR;
    // 16 x 86 = 1376 tiles of 256 x 256 = 5 rounds of 256 CUs + 96: split in 2
    coda::Plan p = plan_of(4096, 22016, 4096, e);
    EXPECT(p.tile == 3 && p.full_tiles == 1280 && p.split_tiles == 96 && p.split_s == 2 && p.k_steps == 64);
    const size_t ws = coda_workspace_size(4096, 22016, 4096, &e, 0);
    EXPECT(ws >= size_t(96) * 2 * 256 * 256 * 4 + 96 * 4);
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &e, 0) == CODA_ERR_WORKSPACE);
    e.workspace = Pm(0x60000000); e.workspace_bytes = ws;
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &e, 0) == CODA_OK);
    // with the RMS op the partial row sums of squares need room too
    coda_epi_desc r = e; r.n_ops = 2; r.ops[1] = r.ops[0];
    r.ops[0].kind = CODA_OP_RMS_ROWSCALE; r.ops[0].in = P(0x40000000); r.ops[0].in_dtype = CODA_BF16;
    EXPECT(coda_workspace_size(4096, 22016, 4096, &r, 0) >= ws + size_t(96) * 2 * 256 * 4);
    // the unfused sequence and CODA_FLAG_NO_SPLIT_K never split
    coda::Plan u = plan_of(4096, 22016, 4096, e, 1);
    EXPECT(u.split_s == 1 && u.split_tiles == 0 && u.full_tiles == 1376);
    coda_epi_desc n = e; n.flags = CODA_FLAG_NO_SPLIT_K;
    EXPECT(coda_workspace_size(4096, 22016, 4096, &n, 0) == 0);
    // whole rounds: 32 x 16 = 512 tiles
    coda_epi_desc w = base_desc(4096, 1024); w.flags = 0;
    coda::Plan q = plan_of(8192, 4096, 1024, w);
    EXPECT(q.split_s == 1 && q.full_tiles == 512 && coda_workspace_size(8192, 4096, 1024, &w, 0) == 0);
    // a small grid (15 tiles of 128 x 128, two per CU) takes up to 4 parts of
    // at least 16 K steps each
    coda_epi_desc sm = base_desc(N, 4096); sm.flags = 0;
    coda::Plan t = plan_of(M, N, 4096, sm);
    EXPECT(t.tile == 2 && t.full_tiles == 0 && t.split_tiles == 15 && t.split_s == 4 && t.k_steps == 64);
    coda_epi_desc k1 = base_desc(N, 2040); k1.flags = 0;   // 32 K steps: 2 parts
    EXPECT(plan_of(M, N, 2040, k1).split_s == 2);
    coda_epi_desc k2 = base_desc(N, 1984); k2.flags = 0;   // 31 K steps: too few to split
    EXPECT(plan_of(M, N, 1984, k2).split_s == 1 && coda_workspace_size(M, N, 1984, &k2, 0) == 0);
    coda_epi_desc k3 = d; k3.flags = 0;                   // K = 200
    EXPECT(plan_of(M, N, K, k3).split_s == 1);
    // fp32 operands are not split
    coda_epi_desc f = sm; f.ab_dtype = CODA_F32; f.d_dtype = CODA_F32; f.lda = 4096;
    EXPECT(plan_of(M, N, 4096, f).split_s == 1);
  }
  {  // deferred LayerNorm: first op, gamma in the A/B dtype, u in in2, never split
    coda_epi_desc e = base_desc(22016, 4096); e.flags = 0;
    e.n_ops = 2;
    e.ops[0].kind = CODA_OP_LN_ROWSCALE; e.ops[0].in = P(0x40000000); e.ops[0].in_dtype = CODA_BF16;
    e.ops[0].scalar = 1e-5f; e.ops[0].in2 = P(0x50000000);
    e.ops[1].kind = CODA_OP_GELU_TANH;
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &e, 0) == CODA_OK);
    coda::Plan p = plan_of(4096, 22016, 4096, e);
    EXPECT(p.has_norm && p.has_ln && p.n_ops == 1 && p.split_s == 1 && p.ln_u == P(0x50000000));
    EXPECT(coda_workspace_size(4096, 22016, 4096, &e, 0) == 0);
    coda_epi_desc f = e; f.ops[0].in2 = nullptr;
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].in2 = P(0x50000004);
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &f, 0) == CODA_ERR_UNSUPPORTED);
    f = e; f.ops[1].in2 = P(0x50000000);   // in2 only on LN_ROWSCALE
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[1] = e.ops[0]; f.ops[0].kind = CODA_OP_GELU_TANH; f.ops[0].in = nullptr; f.ops[0].in2 = nullptr;
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &f, 0) == CODA_ERR_INVALID_ARG);   // not first
    f = e; f.ops[0].in_dtype = CODA_F32;
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &f, 0) == CODA_ERR_INVALID_ARG);
    EXPECT(coda_validate(A, B, 4096, 22016, 0, &e, 0) == CODA_ERR_INVALID_ARG);      // K = 0
    f = e; f.D = Pm(0x50000000);                                                     // D over u
    EXPECT(coda_validate(A, B, 4096, 22016, 4096, &f, 0) == CODA_ERR_INVALID_ARG);
    EXPECT(coda_workspace_size(4096, 22016, 4096, &e, 1) >= size_t(4096) * 4096 * 2);   // unfused: normalised A
  }
  {  // column reductions: at most CODA_MAX_COL_REDUCTIONS, an output, workspace over several tile rows
    coda_epi_desc e = base_desc(N, K);
    e.n_ops = 2;
    e.ops[0].kind = CODA_OP_COL_SUM; e.ops[0].out = Pm(0x50000000); e.ops[0].out_stride = 2;
    e.ops[1].kind = CODA_OP_COL_SUMSQ; e.ops[1].out = Pm(0x50000004); e.ops[1].out_stride = 2;
    coda::Plan q = plan_of(M, N, K, e);
    EXPECT(q.n_colred == 2 && q.n_red == 0 && q.ops[0].red_slot == 0 && q.ops[1].red_slot == 1);
    // 300 rows span two or three tile rows: partials and counters are needed
    const size_t ws = coda_workspace_size(M, N, K, &e, 0);
    EXPECT(ws >= size_t(2) * size_t(q.grid_m) * size_t(N) * 4 + size_t(q.grid_n) * 4);
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_WORKSPACE);
    // overlapping outputs (same stride, same start) are rejected
    coda_epi_desc f = e; f.ops[1].out = Pm(0x50000000); f.ops[1].out_stride = 1;
    f.workspace = Pm(0x70000000); f.workspace_bytes = ws;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.n_ops = 3; f.ops[2] = f.ops[0]; f.ops[2].out = Pm(0x51000000);
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_UNSUPPORTED);   // a third column reduction
    f = e; f.ops[0].out = nullptr;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].out_stride = 0;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].out = Pm(0x30000000);                                   // over D
    f.workspace = Pm(0x70000000); f.workspace_bytes = ws;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    // one tile row: no workspace
    EXPECT(coda_workspace_size(100, N, K, &e, 0) == 0);
    // the unfused sequence keeps column partials per chunk of rows
    EXPECT(coda_workspace_size(M, N, K, &e, 1) > coda_workspace_size(M, N, K, &d, 1));
  }
  {  // the side matrix read ahead: the first bf16 ADD_MAT / MUL_DGELU_TANH before any SWIGLU_PAIR
    coda_epi_desc e = base_desc(N, K);
    e.n_ops = 1;
    e.ops[0].kind = CODA_OP_ADD_MAT; e.ops[0].in = P(0x40000000); e.ops[0].ld = N; e.ops[0].in_dtype = CODA_BF16;
    e.ops[0].scalar = 1.0f;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    coda::Plan q = plan_of(M, N, K, e);
    EXPECT(q.has_side && !q.has_ext);
    EXPECT(!coda::plain_gemm_plan(q).has_side);
    e.ops[0].in_dtype = CODA_F32; e.ops[0].ld = N;   // fp32 side matrices are read where used
    EXPECT(!plan_of(M, N, K, e).has_side);
    coda_epi_desc f = base_desc(N, K);
    f.n_ops = 2; f.ldd = 264;   // N / 2 = 260 columns, rows 16-byte aligned
    f.ops[0].kind = CODA_OP_SWIGLU_PAIR;
    f.ops[1].kind = CODA_OP_ADD_MAT; f.ops[1].in = P(0x40000000); f.ops[1].ld = 264; f.ops[1].in_dtype = CODA_BF16;
    f.ops[1].scalar = 1.0f;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_OK);
    EXPECT(!plan_of(M, N, K, f).has_side);   // after SWIGLU_PAIR
  }
  {  // the backward set does not follow a deferred row norm (fused and unfused)
    coda_epi_desc e = base_desc(N, K);
    e.n_ops = 2;
    e.ops[0].kind = CODA_OP_RMS_ROWSCALE; e.ops[0].in = P(0x40000000); e.ops[0].in_dtype = CODA_BF16;
    e.ops[1].kind = CODA_OP_COL_SUM; e.ops[1].out = Pm(0x50000000); e.ops[1].out_stride = 1;
    e.workspace = Pm(0x70000000); e.workspace_bytes = size_t(1) << 30;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_UNSUPPORTED);
    EXPECT(coda_validate(A, B, M, N, K, &e, 1) == CODA_ERR_UNSUPPORTED);
    e.ops[1].kind = CODA_OP_ROW_SUM;   // a row reduction is not in the backward set
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
  }
  {  // the RMS norm's backward: ROW_DOT is a row reduction with a matrix; RMS_BWD needs x, gamma and two row vectors
    coda_epi_desc e = base_desc(N, K);
    e.n_ops = 2;
    e.ops[0].kind = CODA_OP_ROW_DOT; e.ops[0].in = P(0x40000000); e.ops[0].ld = N; e.ops[0].in_dtype = CODA_BF16;
    e.ops[0].out = Pm(0x51000000); e.ops[0].out_stride = 2;
    e.ops[1].kind = CODA_OP_RMS_BWD; e.ops[1].in = P(0x41000000); e.ops[1].ld = N; e.ops[1].in_dtype = CODA_BF16;
    e.ops[1].in2 = P(0x42000000); e.ops[1].row_sumsq = P(0x50000000); e.ops[1].row_sum = P(0x50000004);
    e.ops[1].row_ld = 2; e.ops[1].scalar = 1e-5f;
    e.workspace = Pm(0x70000000); e.workspace_bytes = coda_workspace_size(100, N, K, &e, 0);
    coda::Plan q = plan_of(100, N, K, e);
    EXPECT(q.n_red == 1 && q.ops[0].red_slot == 0 && q.ops[1].red_slot == -1 && q.ops[1].row_ld == 2);
    EXPECT(coda_validate(A, B, 100, N, K, &e, 0) == CODA_OK);
    coda_epi_desc f = e; f.ops[1].in2 = nullptr;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // no gamma
    f = e; f.ops[1].row_sum = nullptr;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // no t
    f = e; f.ops[1].row_ld = 0;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[1].scalar = -1.0f;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // eps < 0
    f = e; f.ops[1].ld = N - 8;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // x narrower than the row
    f = e; f.ops[0].in = nullptr;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // ROW_DOT without its matrix
    f = e; f.ops[0].in2 = P(0x42000000);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // in2 only on LN_ROWSCALE / RMS_BWD
    f = e; f.ops[1].in2 = P(0x30000000);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // gamma over D
    f = e; f.ops[1].kind = 21;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // unknown kind
    // a reduction output must not overlap what the same call reads: ROW_DOT
    // writing the t column (or the sums of squares) RMS_BWD reads is rejected
    f = e; f.ops[0].out = Pm(0x50000004);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 1) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].out = Pm(0x50000000);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    // a third column of the same [M x 3] array is fine: the columns interleave
    f = e; f.ops[0].out = Pm(0x50000008); f.ops[0].out_stride = 3; f.ops[1].row_ld = 3;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_OK);
    // ... and so is a column that only starts inside another's period
    f = e; f.ops[0].out = Pm(0x50000004); f.ops[0].out_stride = 3; f.ops[1].row_ld = 3;
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    // a reduction output inside ROW_DOT's own matrix or RMS_BWD's x
    f = e; f.ops[0].out = Pm(0x40000100);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].out = Pm(0x41000100);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    // RMS_DGAMMA: a column reduction over x / r, before RMS_BWD
    f = e; f.n_ops = 3; f.ops[2] = f.ops[1]; f.ops[1] = coda_op{};
    f.ops[1].kind = CODA_OP_RMS_DGAMMA; f.ops[1].in = P(0x41000000); f.ops[1].ld = N; f.ops[1].in_dtype = CODA_BF16;
    f.ops[1].row_sumsq = P(0x50000000); f.ops[1].row_ld = 2; f.ops[1].scalar = 1e-5f;
    f.ops[1].out = Pm(0x52000000); f.ops[1].out_stride = 1;
    f.workspace_bytes = coda_workspace_size(100, N, K, &f, 0);
    coda::Plan q2 = plan_of(100, N, K, f);
    EXPECT(q2.n_colred == 1 && q2.n_red == 1 && q2.ops[1].red_slot == 0);
    EXPECT(coda_validate(A, B, 100, N, K, &f, 0) == CODA_OK);
    coda_epi_desc g2 = f; g2.ops[1].row_sumsq = nullptr;
    EXPECT(coda_validate(A, B, 100, N, K, &g2, 0) == CODA_ERR_INVALID_ARG);   // no sums of squares
    g2 = f; g2.ops[1].row_sum = P(0x50000004);
    EXPECT(coda_validate(A, B, 100, N, K, &g2, 0) == CODA_ERR_INVALID_ARG);   // row_sum is RMS_BWD's
    g2 = f; g2.ops[1].out = nullptr;
    EXPECT(coda_validate(A, B, 100, N, K, &g2, 0) == CODA_ERR_INVALID_ARG);
  }
  {  // A stored [K x M] (weight gradient): M % 8, lda >= M, bf16, no row norm
    coda_epi_desc e = base_desc(N, K); e.a_layout = CODA_A_KM; e.lda = 304;
    EXPECT(coda_validate(A, B, 304, N, K, &e, 0) == CODA_OK);
    EXPECT(coda_validate(A, B, 300, N, K, &e, 0) == CODA_ERR_UNSUPPORTED);   // M % 8
    coda_epi_desc f = e; f.lda = 296;
    EXPECT(coda_validate(A, B, 304, N, K, &f, 0) == CODA_ERR_INVALID_ARG);   // lda < M
    f = e; f.ab_dtype = CODA_F32; f.d_dtype = CODA_F32;
    EXPECT(coda_validate(A, B, 304, N, K, &f, 0) == CODA_ERR_UNSUPPORTED);
    f = e; f.n_ops = 1; f.ops[0].kind = CODA_OP_RMS_ROWSCALE; f.ops[0].in = P(0x40000000);
    f.ops[0].in_dtype = CODA_BF16;
    EXPECT(coda_validate(A, B, 304, N, K, &f, 0) == CODA_ERR_UNSUPPORTED);
    f = e; f.a_layout = 2;
    EXPECT(coda_validate(A, B, 304, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.reserved1 = 1;
    EXPECT(coda_validate(A, B, 304, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.D = Pm(0x10000000 + 2 * 304 * 8);                               // D inside A's [K x M] extent
    EXPECT(coda_validate(A, B, 304, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
  }
  {  // given row statistics: gain folded, row_sumsq (and for LN row_sum), row_ld >= 1
    coda_epi_desc e = base_desc(N, K); e.n_ops = 1;
    e.ops[0].kind = CODA_OP_RMS_ROWSCALE; e.ops[0].scalar = 1e-6f;
    e.ops[0].row_sumsq = P(0x50000004); e.ops[0].row_ld = 2;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    coda::Plan q = plan_of(M, N, K, e);
    EXPECT(q.gain_in_b && q.row_ss == P(0x50000004) && q.row_s == nullptr && q.row_ss_stride == 2);
    coda_epi_desc f = e; f.ops[0].in = P(0x40000000); f.ops[0].in_dtype = CODA_BF16;   // gain not folded
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_UNSUPPORTED);
    f = e; f.ops[0].row_ld = 0;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].row_sum = P(0x50000000);                                         // RMS takes no row sums
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    coda_epi_desc l = e; l.ops[0].kind = CODA_OP_LN_ROWSCALE; l.ops[0].in2 = P(0x60000000);
    l.ops[0].row_sum = P(0x50000000);
    EXPECT(coda_validate(A, B, M, N, K, &l, 0) == CODA_OK);
    coda::Plan r = plan_of(M, N, K, l);
    EXPECT(r.has_ln && r.gain_in_b && r.row_s == P(0x50000000) && r.row_ss == P(0x50000004));
    f = l; f.ops[0].row_sum = nullptr;                                               // LN needs both
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.n_ops = 2; f.ops[1].kind = CODA_OP_GELU_TANH; f.ops[1].row_sumsq = P(0x50000004);
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);               // only on a norm op
  }
  {  // coda_fold_gain validation
    const void* g = P(0x40000000);
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, Pm(0x70000000), 3072) == CODA_OK);
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 768, CODA_B_NK, CODA_BF16, g, Pm(0x70000000), 768) == CODA_OK);
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, Pm(0x20000000), 3072) ==
           CODA_OK);   // exactly in place
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, Pm(0x20000010), 3072) ==
           CODA_ERR_INVALID_ARG);   // overlapping, not in place
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, nullptr, Pm(0x70000000), 3072) ==
           CODA_ERR_INVALID_ARG);
    EXPECT(coda::validate_fold_gain(B, 768, 3076, 3080, CODA_B_KN, CODA_BF16, g, Pm(0x70000000), 3080) ==
           CODA_ERR_UNSUPPORTED);   // contiguous dimension not a multiple of 8
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, Pm(0x70000000), 3000) ==
           CODA_ERR_INVALID_ARG);   // ldo too small
    EXPECT(coda::validate_fold_gain(B, 768, 3072, 3072, CODA_B_KN, 7, g, Pm(0x70000000), 3072) ==
           CODA_ERR_INVALID_ARG);
    EXPECT(coda::validate_fold_gain(B, 0, 3072, 3072, CODA_B_KN, CODA_BF16, nullptr, nullptr, 3072) == CODA_OK);
  }
  {  // coda_ln_fold validation
    float* u = static_cast<float*>(Pm(0x60000000));
    float* c = static_cast<float*>(Pm(0x61000000));
    const void* g = P(0x40000000);
    const void* bt = P(0x41000000);
    EXPECT(coda::validate_ln_fold(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, bt, u, c) == CODA_OK);
    EXPECT(coda::validate_ln_fold(B, 768, 3072, 768, CODA_B_NK, CODA_BF16, g, nullptr, u, nullptr) == CODA_OK);
    EXPECT(coda::validate_ln_fold(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, bt, u, nullptr) ==
           CODA_ERR_INVALID_ARG);
    EXPECT(coda::validate_ln_fold(B, 768, 3076, 3080, CODA_B_KN, CODA_BF16, g, nullptr, u, nullptr) ==
           CODA_ERR_UNSUPPORTED);
    EXPECT(coda::validate_ln_fold(B, 768, 3072, 3000, CODA_B_KN, CODA_BF16, g, nullptr, u, nullptr) ==
           CODA_ERR_INVALID_ARG);
    EXPECT(coda::validate_ln_fold(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, bt, u,
                                  static_cast<float*>(Pm(0x60000100))) == CODA_ERR_INVALID_ARG);   // u, c overlap
    EXPECT(coda::validate_ln_fold(B, 768, 3072, 3072, CODA_B_KN, CODA_BF16, g, nullptr,
                                  static_cast<float*>(Pm(0x20000010)), nullptr) == CODA_ERR_INVALID_ARG);   // u in B
    EXPECT(coda::validate_ln_fold(B, 768, 0, 8, CODA_B_KN, CODA_BF16, g, nullptr, nullptr, nullptr) == CODA_OK);
  }
  {  // DROPOUT: 0 <= p < 1, no input; the plan holds the keep threshold and 1 / (1 - p)
    coda_epi_desc e = base_desc(N, K);
    e.n_ops = 1;
    e.ops[0].kind = CODA_OP_DROPOUT; e.ops[0].scalar = 0.5f; e.ops[0].seed = 0x1234; e.ops[0].offset = 9;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
    EXPECT(coda_validate(A, B, M, N, K, &e, 1) == CODA_ERR_WORKSPACE);   // the unfused pass needs its buffer
    e.workspace = Pm(0x70000000); e.workspace_bytes = coda_workspace_size(M, N, K, &e, 1);
    EXPECT(coda_validate(A, B, M, N, K, &e, 1) == CODA_OK);
    coda::Plan q = plan_of(M, N, K, e);
    EXPECT(q.ops[0].thr == 0x80000000u && q.ops[0].scalar == 2.0f && q.ops[0].seed == 0x1234 &&
           q.ops[0].offset == 9);
    e.ops[0].scalar = 0.0f;
    EXPECT(plan_of(M, N, K, e).ops[0].thr == 0u);
    e.ops[0].scalar = 0.25f;
    EXPECT(plan_of(M, N, K, e).ops[0].thr == 0x40000000u);
    coda_epi_desc f = e; f.ops[0].scalar = 1.0f;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].scalar = -0.1f;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
    f = e; f.ops[0].in = P(0x40000000); f.ops[0].in_dtype = CODA_BF16;
    EXPECT(coda_validate(A, B, M, N, K, &f, 0) == CODA_ERR_INVALID_ARG);
  }
  {  // a reduction output over an ADD_MAT residual the same call reads
    coda_epi_desc e = base_desc(N, K);
    e.n_ops = 2;
    e.ops[0].kind = CODA_OP_ADD_MAT; e.ops[0].in = P(0x40000000); e.ops[0].ld = N; e.ops[0].in_dtype = CODA_BF16;
    e.ops[0].scalar = 1.0f;
    e.ops[1].kind = CODA_OP_ROW_SUM; e.ops[1].out = Pm(0x40000400); e.ops[1].out_stride = 1;
    e.workspace = Pm(0x70000000); e.workspace_bytes = coda_workspace_size(M, N, K, &e, 0) + 256;
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_ERR_INVALID_ARG);
    e.ops[1].out = Pm(0x50000000);
    e.workspace_bytes = coda_workspace_size(M, N, K, &e, 0);
    EXPECT(coda_validate(A, B, M, N, K, &e, 0) == CODA_OK);
  }
  EXPECT(std::strcmp(coda_status_string(CODA_ERR_WORKSPACE), "CODA_ERR_WORKSPACE") == 0);
  if (failures == 0) std::printf("ALL OK\n");
  return failures == 0 ? 0 : 1;
}
