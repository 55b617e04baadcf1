/*
 * muon.h -- C ABI of the MI355X (gfx950) Muon optimizer step.
 *
 * The operation (per hidden weight matrix W with gradient G and momentum
 * buffer M), as the pages describe it:
 *   - Guide page "NanoGPT Speedrun: The Ultimate Guide to Pushing LLM Training
 *     Efficiency to Its Limits", section "Optimizer and Training Strategy
 *     Tuning": Muon is applied to hidden-layer matrix weights only; the update
 *     is orthogonalised after a Nesterov momentum step.
 *   - Overview page "The NanoGPT speedrun", paragraph "Six records account for
 *     most of the speedup" (record #3): the momentum update is orthogonalised
 *     (approximately its polar factor U V^T) by five Newton-Schulz steps.
 *
 * What muon_step computes, per matrix (rows x cols, row-major):
 *   M <- fl32(mu*M + G)                       momentum, fp32 buffer, in place
 *   U  = G + mu*M   (nesterov != 0)  or  U = M
 *   X  = U, or U^T when rows > cols           short side first (m <= n)
 *   X <- X / (||X||_F + 1e-7)
 *   T times:  A = X X^T;  B = b*A + c*A*A;  X <- a*X + B*X
 *   W <- W - lr * s * O,  O = X (or X^T back in W's orientation)
 * s is the descriptor's `scale` (<= 0 means 1).  The polynomial, the
 * normalisation and s are readings of the pages, which name the iteration but
 * not its coefficients; a, b, c and T are arguments.
 *
 * Precision.  MUON_PATH_BF16: the three products take bf16 operands (rounded
 * to nearest even) and accumulate in fp32; A and B are stored bf16; the a*X
 * term reads X for the first `x_master_iters` iterations (default 3) as a
 * (hi, lo) pair, hi = bf16(X) (the operand copy) and lo one signed byte: the
 * distance from hi to X in the integer order of fp32 bit patterns, in units
 * of 256, rounded (about 16 significant bits, relative error <= 2^-15), and as
 * the bf16 copy alone afterwards.  Matrices whose short side is
 * below 128 take the fp32 arithmetic even on this path: their A*A and B*X
 * contractions are too short for bf16 rounding errors to average out.
 * MUON_PATH_F32: everything fp32.
 *
 * Ownership.  The caller owns every device buffer: weights, gradients,
 * momentum buffers and the workspace.  The library never allocates device
 * memory.  A plan (host object) holds the layout and its device tables, which
 * live inside the caller's workspace; the workspace must stay untouched and
 * alive for the plan's lifetime.  A plan is not re-entrant: calls on one plan
 * must be ordered (one stream, or synchronised streams).  Different plans
 * with different workspaces may run concurrently.
 *
 * Streams.  `hip_stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  muon_step only enqueues work (it never waits for the device
 * unless a pointer change finds all 8 device copies of the matrix table
 * still in flight); inputs must stay alive until the stream has passed the
 * step.
 *
 * Graph capture.  A step may be enqueued into a capturing stream (HIP stream
 * capture); the graph then reads the plan's device copy of the matrix table
 * as it stood at capture time, so from then on the plan's pointers are fixed:
 * a step whose descriptors carry other pointers, during capture or after it,
 * fails with MUON_E_INVAL (make a new plan for new buffers).  Profiling must
 * be off while capturing (MUON_E_INVAL otherwise).  Replays and eager steps
 * of the same plan must be ordered like any two steps of one plan.
 *
 * Errors.  Every int-returning function returns MUON_OK (0) or a negative
 * MUON_E_* code and then sets a thread-local message readable with
 * muon_last_error().  No C++ exception crosses this ABI.  Gradient values are
 * not inspected: NaN/Inf in G propagate into M, X and W.
 */
#ifndef MUON_MI355X_H
#define MUON_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_OK 0
#define MUON_E_INVAL (-1)       /* bad argument: null pointer, size, T, non-finite scalar ... */
#define MUON_E_UNSUPPORTED (-2) /* dtype or leading dimension not supported */
#define MUON_E_MISMATCH (-3)    /* step descriptors do not match the plan */
#define MUON_E_WORKSPACE (-4)   /* workspace too small or not 256-byte aligned */
#define MUON_E_HIP (-5)         /* a HIP runtime call failed (message has its text) */

#define MUON_DTYPE_F32 0
#define MUON_DTYPE_BF16 1

#define MUON_PATH_BF16 0
#define MUON_PATH_F32 1

/* One hidden matrix.  All pointers are device pointers.  Row-major storage;
 * ld_w and ld_g are leading dimensions in elements and must equal cols (0 is
 * read as cols).  grad: MUON_DTYPE_BF16 or MUON_DTYPE_F32.  weight:
 * MUON_DTYPE_F32 or MUON_DTYPE_BF16.  momentum: always fp32, rows x cols.
 * weight must not alias grad or momentum. */
typedef struct muon_matrix_desc {
  void* weight;
  const void* grad;
  float* momentum;
  int64_t rows;
  int64_t cols;
  int64_t ld_w;
  int64_t ld_g;
  int32_t w_dtype;
  int32_t g_dtype;
  float scale;      /* per-matrix factor s of the weight step; <= 0 means 1 */
  int32_t reserved; /* must be 0 */
} muon_matrix_desc;

/* Plan options.  NULL means: MUON_PATH_BF16, x_master_iters 3, no zeroing,
 * max_T 64, 2 groups. */
typedef struct muon_options {
  int32_t path;           /* MUON_PATH_BF16 or MUON_PATH_F32 */
  int32_t x_master_iters; /* bf16 path: iterations 1..k read X in a*X as its
                             (bf16, low byte) pair; < 0 selects the default 3;
                             ignored on f32 */
  int32_t zero_momentum;  /* != 0: muon_init zeroes every momentum buffer */
  int32_t max_T;          /* largest T muon_step accepts; <= 0 selects 64 */
  int32_t groups;         /* 1: every launch on the caller's stream; 2 (or <= 0,
                             the default) to 4: that many matrix groups, each on a
                             stream of its own (see muon_plan_info.n_groups).  Two
                             measure fastest on MI355X: with 4 hardware queues per
                             process, more streams start to share queues. */
  int32_t fused;          /* != 0: a fused plan.  Every bf16 product of a step
                             (all T iterations of Gram, polynomial and update)
                             runs in one persistent launch, on the caller's stream
                             (groups is then ignored): the planner places each
                             matrix on one XCD, and the launch's blocks take the
                             tiles of their XCD in order, each waiting until the
                             tiles it reads are finished (muon_check reports a
                             wait that gave up).  Steps with T > 16 run the three
                             launches per iteration instead. */
} muon_options;

typedef struct muon_plan muon_plan;

/* Library version string, e.g. "muon-mi355x 1.0.0 (gfx950)".  Never NULL. */
const char* muon_version(void);

/* Bytes of device workspace muon_init needs for these matrices and options;
 * 0 on invalid arguments (see muon_last_error).  Host-only: no HIP call. */
size_t muon_workspace_size(const muon_matrix_desc* descs, int n, const muon_options* opts);

/* Validate the n descriptors, plan the launches and lay out the workspace
 * (device memory of ws_bytes >= muon_workspace_size(...), 256-byte aligned).
 * Uploads the plan's tables (and zeroes the momentum buffers when requested)
 * on hip_stream and waits for that stream before returning.  On success
 * *out_plan owns the host state. */
int muon_init(const muon_matrix_desc* descs, int n, const muon_options* opts,
              void* workspace, size_t ws_bytes, void* hip_stream, muon_plan** out_plan);

/* Enqueue one Muon step over every matrix of the plan on hip_stream.  Per
 * matrix group (muon_plan_info.n_groups; the first group on hip_stream itself,
 * each other one on a stream of its own, forked from and joined back into
 * hip_stream, so later work on hip_stream sees the whole step): 1 momentum launch and 1 norm launch, then 3 launches
 * per Newton-Schulz iteration (all matrices of one precision grouped in each
 * launch: 6 per iteration when the group mixes bf16 and fp32 matrices); T == 0
 * enqueues one weight-step launch instead of norm and iterations
 * (W <- W - lr*s*X0).  descs == NULL reuses the pointers the plan holds;
 * otherwise n must equal the plan's count and shapes, dtypes and scales must
 * match (pointers may differ).  Requirements: 0 <= T <= max_T,
 * 0 <= momentum <= 1, a, b, c, lr finite. */
int muon_step(muon_plan* plan, const muon_matrix_desc* descs, int n, float a, float b, float c,
              int T, float momentum, int nesterov, float lr, void* hip_stream);

/* muon_step with a polynomial of its own for every iteration: iteration t
 * (1-based) uses a = coeffs[3(t-1)], b = coeffs[3(t-1)+1], c = coeffs[3(t-1)+2].
 * The speedrun overview page ("The NanoGPT speedrun", paragraph "Reading
 * guide") names later records that tune the iteration's polynomials (Polar
 * Express); it gives no values, so the schedule is the caller's.  coeffs is a
 * host array of 3*T finite floats, read during the call (the caller may reuse
 * it on return); NULL is allowed only with T == 0. */
int muon_step_schedule(muon_plan* plan, const muon_matrix_desc* descs, int n, const float* coeffs, int T,
                       float momentum, int nesterov, float lr, void* hip_stream);

/* For callers that cannot allocate device memory (tight serving loops,
 * harnesses that forbid hipMalloc): one muon_step over
 * the n descriptors without a plan or a workspace.  The working memory (X
 * copies, A, B, partial sums, tables) is a static device array of 64 MiB
 * (MUON_SCRATCH_BYTES) that the library holds on every GPU it runs on until
 * the process ends; the call allocates nothing.  It plans on the host each
 * time, copies the tables into that array from pageable host memory on
 * hip_stream (a later call first waits for that copy to have run) and
 * enqueues the step there (groups and fused are ignored: one stream, three
 * launches per iteration).
 * That copy is not meant for stream capture: capture the planned muon_step
 * instead.
 * Arguments are those of muon_init (opts: path, x_master_iters and max_T;
 * zero_momentum must be 0) and muon_step; the stream must belong to the
 * current device.  A set whose working memory exceeds the array fails with
 * MUON_E_WORKSPACE (muon_workspace_size with fused 0 gives the need, within a
 * few KiB).
 * All calls on one GPU share its array and every call rewrites what it reads
 * before reading it, so only overlap matters: calls that can run at the same
 * time on one GPU (other streams, other host threads) race and must be
 * ordered by the caller. */
#define MUON_SCRATCH_BYTES (64u << 20)
int muon_step_scratch(const muon_matrix_desc* descs, int n, const muon_options* opts, float a, float b, float c,
                      int T, float momentum, int nesterov, float lr, void* hip_stream);

/* Free the plan's host state.  The workspace stays the caller's. */
int muon_destroy(muon_plan* plan);

/* Message of the last failed call on this thread ("" if none). */
const char* muon_last_error(void);

/* ---- introspection and measurement ---------------------------------------- */

/* Launch kinds, in the order they run within a step. */
#define MUON_KIND_MOMENTUM 0 /* momentum + Nesterov + Frobenius partial sums, writes X0 */
#define MUON_KIND_GRAM 1     /* A = X X^T (upper tiles, mirrored) */
#define MUON_KIND_POLY 2     /* B = b A + c A A (upper tiles, mirrored) */
#define MUON_KIND_UPDATE 3   /* X <- a X + B X; on the last iteration W <- W - lr s O */
#define MUON_KIND_APPLY 4    /* T == 0 only: W <- W - lr s X0 */
#define MUON_KIND_NORM 5     /* T > 0: 1 / (||U||_F + eps) per matrix from the momentum partials */
#define MUON_KIND_FUSED 6    /* fused plans: every bf16 product of the step in one launch */
#define MUON_KIND_COUNT 7

/* Host-only description of the plan these descriptors would get.  Returns
 * MUON_OK and fills the fields, or an error code.  `tiles` (optional) gets
 * the launch-ordered tile list of one kind as (matrix, tile_row, tile_col)
 * int32 triples, at most tile_cap triples; *n_tiles gets the full count. */
typedef struct muon_plan_info {
  int64_t workspace_bytes;
  int32_t n_matrices;
  int32_t tile;              /* tile edge of the fp32 Newton-Schulz products (128) */
  int32_t blocks[MUON_KIND_COUNT]; /* tile-table length of each launch kind: the grid of
                                      the momentum, norm and apply launches; the product
                                      kernels are persistent (2 blocks per CU) and
                                      stride through their table (all groups' tables,
                                      each padded to a multiple of 8) */
  int32_t x_master_iters;
  int32_t path;
  int32_t n_f32_matrices;    /* matrices whose products run in fp32 (see below) */
  int32_t n_groups;          /* matrix groups (contiguous, of equal cost) whose
                                steps run on streams of their own, forked from
                                and joined back into the caller's stream (1 to
                                4): momentum and norm have n_groups launches per
                                step, a product kind T * n_groups (times the
                                precisions present) */
  int32_t bf16_tile_rows;    /* bf16 polynomial and update products: output tile rows
                                (256); the short side of such a matrix is padded to a
                                multiple of it */
  int32_t bf16_tile_cols;    /* bf16 products: output tile columns (128); the Gram
                                product takes square tiles of this edge */
  int32_t fused;             /* 1: a fused plan (muon_options.fused); blocks[MUON_KIND_FUSED]
                                is then its queue length per iteration (all XCDs),
                                and kind MUON_KIND_FUSED lists the queue as
                                (xcd, product 1-3, matrix, tile_row, tile_col)
                                int32 quintuples, XCD by XCD, each XCD's entries
                                in the order its blocks take them */
} muon_plan_info;

int muon_describe(const muon_matrix_desc* descs, int n, const muon_options* opts,
                  muon_plan_info* info, int kind, int32_t* tiles, int tile_cap, int32_t* n_tiles);

/* Per-launch timing with HIP events (enable != 0 turns it on).  Each timed
 * launch of muon_step is issued with hipExtLaunchKernel and an event pair
 * that takes the dispatch's own start and end times, so timing adds no
 * event records to the stream; it does add host work per launch, and a step
 * with timing on must not be captured in a graph.  muon_profile_select
 * restricts the timed launches to the kinds whose bit (1 << MUON_KIND_*) is
 * set in kind_mask (default: all kinds).  muon_profile_read waits for the
 * events, adds their durations per kind into ms[MUON_KIND_COUNT] and
 * launches[MUON_KIND_COUNT] (totals since the last read), and resets the
 * totals. */
int muon_profile_enable(muon_plan* plan, int enable);
int muon_profile_select(muon_plan* plan, uint32_t kind_mask);
int muon_profile_read(muon_plan* plan, double* ms, int64_t* launches);

/* Fused plans: waits for hip_stream, then reports whether a fused launch of
 * this plan gave up a dependency wait since the last check (MUON_E_HIP with
 * the reason; that step's results are incomplete) and clears the report.
 * MUON_OK otherwise, and always for plans that are not fused.  A wait gives
 * up after the plan's poll limit (about 4 s by default), which a launch whose
 * blocks all run never reaches. */
int muon_check(muon_plan* plan, void* hip_stream);

/* Fused plans, for tests of the give-up path: polls of one dependency wait
 * before it gives up (> 0; default 1 << 24, 0.25 us apart) and a count added
 * to every wait's target (>= 0; default 0: with any larger value no wait is
 * ever met, so every block of the next fused launch gives up and returns).
 * MUON_E_INVAL for other values or a plan that is not fused. */
int muon_fused_limits(muon_plan* plan, int32_t spin_limit, int32_t dep_bias);

#ifdef __cplusplus
}
#endif

#endif /* MUON_MI355X_H */
