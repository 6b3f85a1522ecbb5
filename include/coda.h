/*
 * coda.h - C ABI of the MI355X (gfx950) fused GEMM + epilogue library.
 *
 * The operation is the GEMM-plus-epilogue program of "CODA: Rewriting
 * Transformer Blocks as GEMM-Epilogue Programs": a dense product C = A * B
 * (d9bl.com page, section 3.1, where the GEMM is C = alpha*A*B + beta*C_prev
 * and the epilogue is D = f(C)) whose output tile is transformed by an ordered
 * list of primitives while it is still on-chip (section 1 and section 3.1 of
 * the same page; the agentlenshq.com page, "CODA's approach"), before the one
 * store of D.  The primitives are the four families listed on the
 * agentlenshq.com page ("How it works"): scaling by a constant or a vector,
 * reductions over a dimension, pairwise / elementwise transforms, and
 * accumulation into a residual.  Statements run in list order, each on the
 * previous value (d9bl.com page, section 3.2, the EPILOGUE example).
 *
 * Row-wise RMS normalisation of A is expressed as the CODA_OP_RMS_ROWSCALE op:
 * the gain gamma is applied to A inside the GEMM main loop, the per-row
 * sum of squares of A is gathered from the A tiles as they stream through,
 * and the per-row factor 1/rms is applied to the accumulators in the epilogue.
 * This is the reparameterisation summarised in the "augment_me" comment on
 * the zeli.app page (a row-wise norm's per-row scale commutes past the
 * following projection) and on the agentlenshq.com page ("CODA's approach").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All matrices are row-major.  A is [M x K] with leading dimension lda
 *    (lda >= K), or, with a_layout CODA_A_KM, stored [K x M] (lda >= M).
 *    B is the logical [K x N] operand, stored either row-major [K x N]
 *    (CODA_B_KN, leading dimension ldb >= N) or row-major [N x K], i.e. the
 *    transpose of a [K x N] matrix (CODA_B_NK, ldb >= K).  D is
 *    [M x out_width] with leading dimension ldd, where out_width is N, or N/2
 *    when the list holds CODA_OP_SWIGLU_PAIR.
 *  - Every pointer is a device pointer (memory the GPU can read or write),
 *    except the descriptor itself, which is host memory read only during the
 *    call and may be reused as soon as the call returns.
 *  - The caller owns every buffer.  Buffers must stay valid until the work
 *    enqueued on `stream` has completed.  The library allocates no memory
 *    and keeps no reference to any pointer after a call returns.
 *  - `stream` is a hipStream_t passed as an opaque pointer (NULL = the
 *    default stream).  Work is enqueued asynchronously; device faults surface
 *    at the caller's next synchronisation, per HIP convention.
 *  - Validation happens before anything is enqueued: on any error code,
 *    nothing has been launched and no memory has been touched.
 *  - Shape rules: 0 <= M, N, K < 2^31; K % 8 == 0; N % 8 == 0 when B is
 *    CODA_B_KN; every matrix leading dimension is a multiple of 8 elements,
 *    and lda, ldb are at most 2^21 elements; every matrix pointer is 16-byte
 *    aligned; vector operands are 16-byte aligned.  Outside these rules a call
 *    returns CODA_ERR_UNSUPPORTED.  M == 0 or N == 0 is a no-op that returns
 *    CODA_OK.  Sizes that are not tile multiples (ragged M, N, K) are supported.
 *  - Aliasing: D may coincide exactly with the matrix of a CODA_OP_ADD_MAT op
 *    (same pointer, same dtype, same leading dimension: an in-place residual
 *    update).  Any other overlap between D and an input, between outputs,
 *    or between a reduction output and any input the same call reads (the
 *    columns of one row-major array may interleave: a reduction may write one
 *    column of a stats array whose other columns an op reads), is
 *    CODA_ERR_INVALID_ARG.
 *  - The library is stateless and reentrant, except for the workspace rule
 *    of coda_gemm_epi below.
 */
#ifndef CODA_H
#define CODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CODA_MAX_OPS 16
#define CODA_MAX_REDUCTIONS 8
#define CODA_MAX_COL_REDUCTIONS 2

/* bytes of the fixed per-GPU scratch of coda_gemm_epi_noalloc (64 MiB) */
#define CODA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* coda_epi_desc.flags */
#define CODA_FLAG_NO_SPLIT_K 1   /* coda_gemm_epi: never split the last round of
                                    tiles over K (see coda_gemm_epi)            */

typedef enum {
  CODA_OK = 0,
  CODA_ERR_INVALID_ARG = -1,  /* a null/ill-formed argument, bad op list, overlap  */
  CODA_ERR_UNSUPPORTED = -2,  /* well-formed but outside the shape/alignment rules  */
  CODA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required         */
  CODA_ERR_HIP = -4           /* the HIP runtime reported an error at launch        */
} coda_status;

typedef enum { CODA_BF16 = 0, CODA_F32 = 1 } coda_dtype;

typedef enum {
  CODA_A_MK = 0,  /* A stored row-major [M x K] (the default)                    */
  CODA_A_KM = 1   /* A stored row-major [K x M] and used transposed: the X^T of a
                     weight gradient dW = X^T dY, X being [tokens x features] and
                     tokens the contraction; bf16 only, no RMS/LN_ROWSCALE, and
                     M % 8 == 0                                                 */
} coda_a_layout;

typedef enum {
  CODA_B_KN = 0,  /* B stored row-major [K x N]                                  */
  CODA_B_NK = 1   /* B stored row-major [N x K] and used transposed (e.g. W^T)  */
} coda_b_layout;

/*
 * Epilogue primitives.  v is the fp32 running value of output element (i, j);
 * "width" is the current number of columns (N, or N/2 after SWIGLU_PAIR).
 * `in`, `ld`, `in_dtype`, `scalar`, `out`, `out_stride` are fields of coda_op.
 */
typedef enum {
  /* scaling (agentlenshq.com page, "How it works": scaling) */
  CODA_OP_SCALE = 0,          /* v *= scalar                                         */
  CODA_OP_SCALE_ROW = 1,      /* v *= in[i]          in: [M] vector                  */
  CODA_OP_SCALE_COL = 2,      /* v *= in[j]          in: [width] vector              */
  CODA_OP_RMS_ROWSCALE = 3,   /* deferred RMSNorm: in = gamma [K], scalar = eps.
                                 v *= 1/sqrt(mean_k A[i,k]^2 + eps), with A*gamma fed
                                 to the GEMM.  in = NULL: the gain is already in the
                                 rows of B (B = diag(gamma) W, see coda_fold_gain), A
                                 is fed unchanged and the row sums of squares come from
                                 the A fragments the matrix cores read.  With in = NULL
                                 and row_sumsq != NULL, the row sums of squares are
                                 inputs (sum_k A[i,k]^2 at row_sumsq[i*row_ld]), e.g.
                                 the ROW_SUMSQ output of the layer that produced A, and
                                 the main loop is the plain GEMM (a cross-layer chain).
                                 Must be the first op, at most once, and needs K > 0. */
  /* accumulation (agentlenshq.com page, "How it works": accumulation) */
  CODA_OP_ADD_COL = 4,        /* v += in[j]          (bias)                          */
  CODA_OP_ADD_ROW = 5,        /* v += in[i]                                          */
  CODA_OP_ADD_MAT = 6,        /* v += scalar * in[i*ld + j]   (beta * residual)      */
  /* pairwise / elementwise transforms (agentlenshq.com page, "How it works") */
  CODA_OP_GELU_TANH = 7,      /* v = 0.5 v (1 + tanh(sqrt(2/pi)(v + 0.044715 v^3)))  */
  CODA_OP_SILU = 8,           /* v = v * sigmoid(v)                                  */
  CODA_OP_SWIGLU_PAIR = 9,    /* out[i,j] = silu(v[i,2j]) * v[i,2j+1]; width halves,
                                 so width must be even; at most once                  */
  CODA_OP_MUL_DGELU_TANH = 10,/* v *= d/dp GELU_tanh(p), p = in[i*ld + j]             */
  /* reductions over the row (agentlenshq.com page, "How it works": reductions).
     Each writes an fp32 value per row to ((float*)out)[i*out_stride]; the value
     reduced is the running value at the op's position in the list.  At most
     CODA_MAX_REDUCTIONS per list. */
  CODA_OP_ROW_SUM = 11,
  CODA_OP_ROW_SUMSQ = 12,
  CODA_OP_ROW_MEAN = 13,
  /* deferred LayerNorm (the mean-centred row norm of the Transformer operators
     in the d9bl.com page's Fig. 4, moved past the projection as the zeli.app
     page's "augment_me" comment moves a row-wise norm's per-row factors):
     in = gamma [K] in the A/B dtype, in2 = u [N] fp32 with u[j] = sum_k
     gamma[k] B[k,j] (coda_ln_fold computes it), scalar = eps.
     v = (sum_k (A[i,k] - mu_i) gamma[k] B[k,j]) / sqrt(var_i + eps), with mu_i
     the mean of row i of A over K and var_i the mean squared deviation from it:
     the GEMM of the normalised, gained A.  The shift beta is not part of the
     op: its term beta^T B is a column vector (coda_ln_fold's c) that a later
     CODA_OP_ADD_COL adds.  in = NULL: the gain is already in the rows of B
     (coda_fold_gain), and in2 must then hold the column sums of that B
     (coda_ln_fold with gamma = 1); A is fed unchanged and its row sums and sums
     of squares come from the fragments the matrix cores read.  With in = NULL
     and row_sum, row_sumsq != NULL the row sums and sums of squares of A are
     inputs (at [i*row_ld]; e.g. the ROW_SUM / ROW_SUMSQ outputs of the layer
     that produced A) and the main loop is the plain GEMM; the variance is then
     sumsq/K - mean^2 in fp32, which loses accuracy on rows whose mean is large
     against their spread.  Must be the first op and needs K > 0; at most one
     of RMS_ROWSCALE / LN_ROWSCALE. */
  CODA_OP_LN_ROWSCALE = 14,
  /* reductions over the rows (for the backward pass: the bias gradient of a
     layer is the column sum of its output gradient).  Each writes an fp32 value
     per column j < width to ((float*)out)[j*out_stride]: the sum over all M
     rows of the running value (COL_SUM) or of its square (COL_SUMSQ) at the
     op's position.  At most CODA_MAX_COL_REDUCTIONS per list.  The backward
     set (COL_SUM, COL_SUMSQ, ROW_DOT, RMS_BWD, RMS_DGAMMA) does not share a
     list with RMS_ROWSCALE or LN_ROWSCALE: such a list is
     CODA_ERR_UNSUPPORTED (the kernels with a deferred row norm are built
     without the backward set's code). */
  CODA_OP_COL_SUM = 15,
  CODA_OP_COL_SUMSQ = 16,
  /* the RMS norm's backward (gradients are among the operators the d9bl.com
     page's Fig. 4 splits into a GEMM and an epilogue; the agentlenshq.com page,
     "How it works", has the primitives cover the backward pass too).
     ROW_DOT is a row reduction like ROW_SUM, counted among them: it writes
     sum_j v[i,j] * in[i*ld + j] over the current width, in a matrix [M x width]
     of in_dtype.  RMS_BWD takes v = dL/dY of Y = x * gamma / r (the RMS norm,
     r_i = sqrt(sum_k x[i,k]^2 / width + eps)) and makes it dL/dx:
       v = gamma[j] v / r_i - x[i,j] * t_i / (width * r_i^2)
     with in = x [M x width] (in_dtype, ld), in2 = gamma [width] (in_dtype),
     scalar = eps, row_sumsq[i*row_ld] = sum_k x[i,k]^2 and
     row_sum[i*row_ld] = t_i, both fp32.  t_i is s_i / r_i with
     s_i = sum_j gamma[j] v[i,j] x[i,j], the part of the gradient that spans
     the row.  When v = dP W^T for P = Y W, t_i = sum_l dP[i,l] P[i,l]: the
     ROW_DOT of dP against P in the epilogue of the GEMM that produced dP,
     so this op needs no pass over its own row. */
  CODA_OP_ROW_DOT = 17,
  CODA_OP_RMS_BWD = 18,
  /* the RMS norm's gain gradient, a column reduction (counted among them):
     with v = dL/dY as for RMS_BWD, writes sum_i v[i,j] * x[i,j] / r_i to
     ((float*)out)[j*out_stride], in = x [M x width] (in_dtype, ld),
     row_sumsq[i*row_ld] = sum_k x[i,k]^2 (fp32), scalar = eps.  Placed before
     RMS_BWD in the same list, it reads the same x and row statistics. */
  CODA_OP_RMS_DGAMMA = 19,
  /* dropout (the d9bl.com page, section 3.2: the dropout step of its
     EPILOGUE example): element (i, j) of the running value is
     kept with probability 1 - p and scaled by 1 / (1 - p), or set to 0; p is
     `scalar`, 0 <= p < 1.  The mask comes from the counter-based generator
     Philox-4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
     as easy as 1, 2, 3", SC 2011) with key (seed, 0) and counter
     (j / 8, i, offset, 0): j indexes the current width, and the element takes
     32-bit word j % 8 of the 256-bit block (the low half of 64-bit word
     (j % 8) / 2 when j % 8 is even, the high half when odd); it is kept when
     that word is >= floor(p * 2^32).  The mask depends on (seed, offset, i, j)
     only, so it is reproducible, needs no stored state, and a backward pass
     regenerates it; vary `offset` (or `seed`) to draw a new mask. */
  CODA_OP_DROPOUT = 20
} coda_op_kind;

typedef struct {
  int32_t kind;         /* coda_op_kind                                              */
  int32_t in_dtype;     /* coda_dtype of `in` (ignored by ops without an input)      */
  const void* in;       /* vector / matrix input (device), or NULL                   */
  int64_t ld;           /* leading dimension of a matrix input                       */
  float scalar;         /* alpha of SCALE, beta of ADD_MAT, eps of RMS_ROWSCALE      */
  int32_t reserved0;    /* must be 0                                                 */
  void* out;            /* reductions: fp32 output (device)                          */
  int64_t out_stride;   /* reductions: element stride between rows of `out`, >= 1   */
  const void* in2;      /* LN_ROWSCALE: fp32 u [N]; RMS_BWD: gamma; else NULL         */
  const void* row_sum;  /* LN_ROWSCALE: given fp32 row sums of A, or NULL; RMS_BWD: t */
  const void* row_sumsq;/* RMS/LN_ROWSCALE: given fp32 row sums of squares, or NULL;
                           RMS_BWD, RMS_DGAMMA: sum_k x[i,k]^2                       */
  int64_t row_ld;       /* element stride between rows of row_sum / row_sumsq (>= 1) */
  uint64_t seed;        /* DROPOUT: the generator's key word 0 (ignored by other ops) */
  uint64_t offset;      /* DROPOUT: counter word 2, e.g. a step count (ignored by other ops) */
} coda_op;

typedef struct {
  int32_t ab_dtype;     /* dtype of A and B: CODA_BF16 (bf16 MFMA) or CODA_F32     */
  int32_t d_dtype;      /* dtype of D                                               */
  int32_t b_layout;     /* coda_b_layout                                            */
  int32_t n_ops;        /* 0..CODA_MAX_OPS                                          */
  int64_t lda, ldb, ldd;
  void* D;              /* output (device)                                          */
  void* workspace;      /* device scratch, see coda_workspace_size                 */
  size_t workspace_bytes;
  int32_t tile;         /* 0 = automatic tile choice; k > 0 forces tile config k    */
  int32_t flags;        /* 0, or CODA_FLAG_NO_SPLIT_K; other bits must be 0         */
  int32_t a_layout;     /* coda_a_layout (0 = CODA_A_MK)                            */
  int32_t reserved1;    /* must be 0                                                 */
  coda_op ops[CODA_MAX_OPS];
} coda_epi_desc;

/*
 * coda_gemm_epi - one fused kernel: D = f(A * B) with f = desc->ops in order.
 * The GEMM runs on MFMA with fp32 accumulators.  The ops run on fp32 values
 * on-chip: each wave passes its accumulators once through its own region of
 * LDS into a row-major layout (every lane then holds runs of 8 consecutive
 * columns, so side operands and D move as whole 16-byte row chunks), and the
 * list runs there before D is written once, rounded to d_dtype
 * (round-to-nearest-even for bf16).  With CODA_OP_RMS_ROWSCALE first, the
 * GEMM operand is A*gamma rounded to ab_dtype and the row factor is applied
 * to the accumulators.  With CODA_OP_LN_ROWSCALE first and bf16 operands, the
 * GEMM operand is (A - s_i)*gamma rounded to bf16, s_i being a per-row shift
 * (a constant that leaves the norm unchanged and keeps rows whose spread is
 * small against their mean accurate): the mean of the row's first 64 stored
 * values with the gain applied in the loop, the row's first element with the
 * gain folded into B; the row mean and variance come from sums of A - s_i
 * gathered in the main loop.  LN_ROWSCALE tiles are never split over K.
 * Load balance: when the output tiles do not fill a whole number of rounds
 * of the GPU's compute units, each tile of the last, partial round is split
 * over K between up to 4 workgroups (bf16 operands only, unless flags holds
 * CODA_FLAG_NO_SPLIT_K); the last of them to finish adds the fp32 partial
 * accumulators in a fixed order and runs the epilogue, so results do not
 * depend on timing.
 * Workspace: row reductions whose row spans several output tiles combine
 * partial sums through the workspace, column reductions whose column spans
 * several tiles likewise, and so do the parts of a split tile
 * (coda_workspace_size(..., 0) bytes, 0 when neither happens).  Its counter
 * regions must be zero before the first call (a zero-filled workspace will
 * do); every call leaves them zero again.  Two calls that run concurrently
 * must not share a workspace.
 * Returns a coda_status.
 */
int coda_gemm_epi(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                  const coda_epi_desc* desc, void* stream);

/*
 * coda_gemm_epi_noalloc - coda_gemm_epi for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The same computation and results as
 * coda_gemm_epi, with the cross-workgroup scratch (row and column reduction
 * partials and counters, the split round's partial tiles) taken from a fixed
 * array of CODA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends; desc->workspace and desc->workspace_bytes
 * are ignored.  The array's first 1 MiB holds the cross-workgroup counters
 * at fixed places (zero between calls), the rest a call's partial sums and
 * tiles.  When the split of the last round would not fit, the tiles are
 * split into fewer parts, or not at all; when even the unsplit call needs
 * more scratch than the maximum (row reductions over many tile columns of a
 * very tall output), it returns CODA_ERR_WORKSPACE and launches nothing.
 * Calls no allocating routine.  Every call on one GPU shares that GPU's
 * array: calls that may run at the same time on one GPU (different streams,
 * or host threads) race and must be serialised by the caller.  The first
 * call on a device clears the array with a kernel on `stream`.
 * Returns a coda_status.
 */
int coda_gemm_epi_noalloc(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                          const coda_epi_desc* desc, void* stream);

/*
 * coda_gemm_unfused - the same computation as the framework-level sequence of
 * one kernel per operator (agentlenshq.com page, "The problem": each
 * operator launched as its own kernel, the GEMM output written to global
 * memory and read straight back): an RMS or LayerNorm normalisation pass over
 * A (when the list starts with CODA_OP_RMS_ROWSCALE or CODA_OP_LN_ROWSCALE;
 * the latter writes (A - mu) / sqrt(var + eps) * gamma), the plain GEMM with the same main
 * loop as coda_gemm_epi (split over K in its last, partial round exactly as
 * a fused call of that GEMM would be, unless flags holds
 * CODA_FLAG_NO_SPLIT_K), then one pass per remaining op.  Intermediates are
 * stored in d_dtype in the workspace (coda_workspace_size(..., 1) bytes),
 * which also holds the split's partial tiles and counters: as for
 * coda_gemm_epi, the workspace must be zero before the first call (every
 * call leaves the counters zero again) and concurrent calls must not share
 * it.  Meant as the in-run comparison for coda_gemm_epi.  Returns a
 * coda_status.
 */
int coda_gemm_unfused(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                      const coda_epi_desc* desc, void* stream);

/*
 * coda_validate - host-only check of a call: returns the status coda_gemm_epi
 * (unfused == 0) or coda_gemm_unfused (unfused != 0) would return before
 * launching, without touching the device.
 */
int coda_validate(const void* A, const void* B, int64_t M, int64_t N, int64_t K,
                  const coda_epi_desc* desc, int unfused);

/*
 * coda_workspace_size - bytes of workspace the call needs (0 when none).
 * Returns 0 for a descriptor that does not validate.
 */
size_t coda_workspace_size(int64_t M, int64_t N, int64_t K, const coda_epi_desc* desc,
                           int unfused);

/*
 * coda_fold_gain - B_out = diag(gamma) B: row k of the logical [K x N] operand
 * B scaled by gamma[k] and rounded to `dtype` (round-to-nearest-even for bf16),
 * the per-feature gain of a row norm moved into the following projection's
 * weights ((x * gamma) W = x (gamma W), the reparameterisation in the zeli.app
 * page's "augment_me" comment).  A fused call with CODA_OP_RMS_ROWSCALE and
 * in = NULL on B_out then computes what the call with in = gamma computes on
 * B.  B and B_out have the same layout (`b_layout`) with leading dimensions ldb
 * and ldo; B_out may be B itself (ldo == ldb: in place), otherwise they must
 * not overlap.  Depends on the weights alone, so a caller folds once per weight
 * set.  Shape rules: the contiguous dimension (N for CODA_B_KN, K for
 * CODA_B_NK), ldb and ldo multiples of 8; 16-byte aligned pointers.  Enqueued
 * on `stream`; nothing is launched on error.  Returns a coda_status.
 */
int coda_fold_gain(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                   const void* gamma, void* B_out, int64_t ldo, void* stream);

/*
 * coda_ln_fold - the two constant rows of the deferred LayerNorm:
 * u[j] = sum_k gamma[k] B[k,j] and, when beta is not NULL, c[j] = sum_k
 * beta[k] B[k,j], for j < N, in fp32 from exact products.  B is the logical
 * [K x N] operand in `b_layout` (ldb as for coda_gemm_epi); B, gamma and beta
 * are in `dtype` (CODA_BF16 or CODA_F32); u and c are fp32 [N] device arrays,
 * c may be NULL only together with beta.  Depends on the weights alone, so a
 * caller computes it once per weight set.  Shape rules as for coda_gemm_epi
 * (K % 8 == 0, ldb % 8 == 0, 16-byte aligned B, gamma, beta, u, c); u and c
 * must not overlap the inputs or each other.  Enqueued on `stream`; nothing is
 * launched on error.  Returns a coda_status.
 */
int coda_ln_fold(const void* B, int64_t K, int64_t N, int64_t ldb, int32_t b_layout, int32_t dtype,
                 const void* gamma, const void* beta, float* u, float* c, void* stream);

/* coda_status_string - static text for a status code. */
const char* coda_status_string(int status);

/* coda_last_error - detail of the last failing call on this host thread ("" if none). */
const char* coda_last_error(void);

/*
 * coda_num_tile_configs / coda_tile_config - the compiled bf16 tile
 * configurations, numbered 1..n, selectable through coda_epi_desc.tile.
 * coda_tile_config returns CODA_OK and fills the output tile size (bm x bn),
 * the K step (bk) and the wavefronts per workgroup, or CODA_ERR_INVALID_ARG.
 */
int coda_num_tile_configs(void);
int coda_tile_config(int index, int* bm, int* bn, int* bk, int* waves);

/*
 * coda_selected_tile - the tile configuration coda_gemm_epi would use for this
 * call: desc->tile when it is nonzero, else the automatic choice.  Returns the
 * 1-based bf16 configuration, 0 for fp32 operands (one fixed 64 x 64 tile), or
 * a negative coda_status when the descriptor does not validate.  Host-only.
 */
int coda_selected_tile(int64_t M, int64_t N, int64_t K, const coda_epi_desc* desc);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H */
