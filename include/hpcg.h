/*
 * hpcg.h - C ABI of the MI355X (gfx950) H-matrix-preconditioned conjugate
 * gradient solver.
 *
 * The library solves A x = b for sparse SPD A (CSR, nodes in space-filling-curve
 * order) with preconditioned CG, where the preconditioner M is a
 * weak-admissibility H-matrix approximate inverse applied every iteration
 * without ever being assembled:
 *
 *   M = blockdiag_k(U_k U_k^T)                      dense leaf blocks, L = 128
 *     + sum over tiles (l, j) of  U_{l,j} V_{l,j}^T   and its mirror V U^T
 *     + diag(g)                                     per-node gate
 *
 * Sources for the operations (cited by page title and section):
 *  - "Hierarchical Transformer Preconditioning for Interactive Physics
 *    Simulation" (arXiv 2605.13343 v1/v2), section 5 "Preconditioner
 *    Application": the diagonal stage y_k = F_k r_k as one batched product over
 *    leaves, the off-diagonal restriction / strip aggregation / coupling /
 *    prolongation chain of eqs. (2)-(5), and the CSR SpMV as the only sparse
 *    operation of the loop; section 5 "Single-graph capture": the whole
 *    iteration without host dispatch; Supplementary section 2 "Apply-path
 *    tensor layout": the partition with K - 1 unique tiles at eta = 1;
 *    Supplementary section 7: fp32 apply and vectors, fp64 scalar accumulators.
 *  - "A Neural Hierarchical-Matrix Preconditioner for Real-Time GPU Solves"
 *    (v3), section 2 "Preconditioner": leaf blocks F_k = U_k U_k^T, symmetric
 *    mirrored off-diagonal tiles.
 *
 * Partition.  n unknowns per system are cut into K = n / L leaves (L = 128,
 * K a power of two).  Tile j of level l (S = 2^l leaves per side, l = 0 ..
 * levels-1, j = 0 .. K/(2S)-1) couples row leaves [2jS, 2jS+S) with column
 * leaves [2jS+S, 2jS+2S).  Its factors are stacks of per-leaf slabs:
 * U_{l,j} stacks W_l[k] over the row leaves, V_{l,j} over the column leaves,
 * each slab L x R with R = 32, and the coupling core is the identity.
 *
 * Batching.  `batch` independent systems of equal n are solved in lockstep,
 * one launch per phase across the whole batch.  The CSR of a batch is
 * block-diagonal with global indices (system s owns rows and columns
 * [s*n, (s+1)*n)); factors and vectors carry a leading batch axis.
 *
 * Memory and ownership.  Every pointer named d_* is device memory on the
 * current HIP device; h_* pointers are host memory.  The caller owns all
 * device memory, including the workspace: the library never allocates device
 * memory and keeps only a host-side handle (plus an instantiated HIP graph and
 * a few bytes of pinned host memory for convergence polling).  hpcg_create and
 * hpcg_set_factors copy their inputs into the workspace in stream order, so the
 * caller may reuse those buffers once the stream has passed the call.  The
 * workspace must stay allocated until hpcg_destroy.
 *
 * Streams and threads.  All work is enqueued on the stream given to
 * hpcg_create.  hpcg_apply_M and hpcg_spmv are asynchronous; hpcg_solve returns
 * after its final synchronization.  A handle is not thread-safe; different
 * handles are independent.
 *
 * Errors.  Every call returns an hpcg_status; nothing throws across the ABI.
 * Arguments are validated before any launch.  HIP failures return
 * HPCG_ERR_HIP with text in hpcg_last_error.
 */
#ifndef HPCG_H
#define HPCG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hpcg_ctx* hpcg_handle;

typedef enum {
    HPCG_OK = 0,
    HPCG_ERR_INVALID_ARG = 1,   /* null pointer, bad tolerance, bad option       */
    HPCG_ERR_SHAPE = 2,         /* partition or CSR sizes not supported          */
    HPCG_ERR_HIP = 3,           /* a HIP runtime call failed                     */
    HPCG_ERR_BREAKDOWN = 4,     /* p.Ap or r.Mr not positive and finite          */
    HPCG_ERR_NOT_CONVERGED = 5, /* maxit reached before the tolerance            */
    HPCG_ERR_WORKSPACE = 6,     /* workspace too small or misaligned             */
    HPCG_ERR_STATE = 7          /* call order violated (e.g. solve before factors) */
} hpcg_status;

/* Per-system outcome of the last hpcg_solve (see hpcg_last_solve_status). */
typedef enum {
    HPCG_SYS_RUNNING = 0,
    HPCG_SYS_CONVERGED = 1,
    HPCG_SYS_NOT_CONVERGED = 2,
    HPCG_SYS_BREAKDOWN = 3
} hpcg_system_status;

typedef struct {
    int32_t n;       /* unknowns per system; n % leaf == 0, n / leaf a power of 2 */
    int32_t leaf;    /* L, must be 128                                            */
    int32_t rank;    /* R, columns of every off-diagonal slab, must be 32         */
    int32_t levels;  /* tile levels present, 0 .. min(8, log2(n / leaf)); 0 = leaves only */
    int32_t batch;   /* B >= 1 independent systems                                */
} hpcg_partition;

/* Solve engines (hpcg_set_option(HPCG_OPT_ENGINE, ...)). */
typedef enum {
    HPCG_ENGINE_AUTO = 0,       /* persistent (register-resident) when every leaf
                                   of a system gets a CU, else graph             */
    HPCG_ENGINE_GRAPH = 1,      /* per-phase kernels, unrolled iterations replayed
                                   as one hipGraph, host polls a pinned flag      */
    HPCG_ENGINE_PERSISTENT = 2  /* one launch runs the whole solve: one 512-thread
                                   workgroup per leaf with the factors in VGPRs
                                   when K <= #CUs (the values that cross
                                   workgroups travel as flagged words, two
                                   exchanges per iteration and no barrier; the
                                   SQUARED form adds one barrier among a
                                   system's workgroups; a batch with more leaves
                                   than CUs runs in groups of whole systems, one
                                   launch each), else workgroups streaming the
                                   factors (three device-wide barriers per
                                   iteration)                                     */
} hpcg_engine;

typedef enum {
    HPCG_OPT_ENGINE = 1,        /* an hpcg_engine value                          */
    HPCG_OPT_GRAPH_UNROLL = 2,  /* iterations per graph replay, 1 .. 64 (default 8) */
    HPCG_OPT_PRECISION = 4,     /* an hpcg_precision value                        */
    HPCG_OPT_APPLY_PATH = 16,   /* an hpcg_apply_path value                       */
    HPCG_OPT_FORM = 32,         /* an hpcg_form value                             */
    HPCG_OPT_FALLBACK = 64,     /* 1: an hpcg_solve in which some system breaks
                                   down (M not SPD) solves the whole batch again
                                   from x = 0 with M = diag(A)^-1 and reports
                                   that solve; 0 (default): report the breakdown */
    HPCG_OPT_POLL_LIMIT = 128,  /* register-resident engine: polls of one flagged
                                   word before the solve gives up (abort flag,
                                   hpcg_solve returns HPCG_ERR_HIP), 1 .. 2^30;
                                   0 restores the default (2^22, seconds).  A
                                   diagnostic bound: small values make a healthy
                                   solve abort, which is how its error path is
                                   tested                                         */
    HPCG_OPT_APPLY_POLL_LIMIT = 256, /* single-pass hpcg_apply_M: poll rounds of the
                                   partners' flagged words before a workgroup
                                   gives up, 1 .. 2^30; 0 restores the default
                                   (2^20, about a second).  A run-out leaves that
                                   apply's y undefined and is reported by
                                   hpcg_apply_status (or the next hpcg_solve or
                                   hpcg_estimate_spectrum); a diagnostic bound,
                                   like HPCG_OPT_POLL_LIMIT                       */
    HPCG_OPT_BLOCK_SPLIT = 512, /* block apply and block solve, where there are
                                   tile levels and a workgroup takes at most two
                                   16-column tiles: 0 = automatic (default: two
                                   workgroups per (leaf, column tile) while fewer
                                   such items than compute units), 1 = one
                                   workgroup takes the leaf stage and the
                                   restriction, 2 = each in a workgroup of its
                                   own.  Same results either way               */
    HPCG_OPT_LEAF_SPLIT = 8     /* workgroups per leaf in the apply kernels and the
                                   graph and streaming engines: 0 = automatic
                                   (default), else 1, 2, 4 or 8; a split whose LDS
                                   need exceeds a compute unit is raised to the
                                   next that fits.  A nonzero split also keeps
                                   solves off the register-resident engine (one
                                   workgroup per leaf): AUTO then runs the graph
                                   engine, PERSISTENT the streaming one          */
} hpcg_option;

/* Which preconditioner the apply and the solve use (hpcg_set_option(
 * HPCG_OPT_FORM, ...)), with H the H-matrix of the factors:
 *  DIRECT   M = H (default; "Hierarchical Transformer Preconditioning for
 *           Interactive Physics Simulation", section 5);
 *  SQUARED  M = H H, SPD whenever the symmetric H is nonsingular ("A Neural
 *           Hierarchical-Matrix Preconditioner for Real-Time GPU Solves",
 *           section 2, "SPD by construction"); two applications of H per
 *           iteration;
 *  JACOBI   M = diag(A)^-1, the fallback those pages name; needs no factors.
 * SQUARED and JACOBI solves run on the register-resident engine where it fits
 * (SQUARED with one more exchange per iteration, for the restriction of
 * w = H r), else on the graph engine (the streaming persistent engine returns
 * HPCG_ERR_SHAPE for them).  The block apply and the block solve run DIRECT
 * only (HPCG_ERR_STATE otherwise). */
typedef enum {
    HPCG_FORM_DIRECT = 0,
    HPCG_FORM_SQUARED = 1,
    HPCG_FORM_JACOBI = 2
} hpcg_form;

/* How hpcg_apply_M runs (hpcg_set_option(HPCG_OPT_APPLY_PATH, ...)).
 * STREAMING: two launches (restriction, then prolongation), any batch size;
 * the prolongation reads the level slabs a second time.  FUSED: one launch in
 * which the 512-thread workgroup of each leaf keeps U_k and its slabs in
 * registers from the restriction to the prolongation and takes its partners'
 * restrictions from flagged words, so every factor byte is read once; the
 * workgroups of one system must be resident at once, one per compute unit
 * (HPCG_ERR_SHAPE when a system has more leaves than that).  A batch with
 * more leaves than the device has compute units runs as several such
 * launches, each over as many whole systems as fit.  The wait for a partner's
 * words is bounded (HPCG_OPT_APPLY_POLL_LIMIT, about a second by default):
 * should other work hold the compute units that long, the apply gives up, its
 * output is undefined, and hpcg_apply_status reports it.
 * BRIDGE: the single pass in the pages' own format, reading the per-leaf
 * bridges U~_k, V~_k and the per-tile cores B_m as given to
 * hpcg_set_factors_bridge (O(N) factor bytes: 13.2 MB at n = 16,384 against
 * the slabs' 23.3 MB), with the coarse coupling t = B_m s in each leaf's
 * workgroup ("Hierarchical Transformer Preconditioning for Interactive Physics
 * Simulation", section 5, eqs. (2)-(5)); HPCG_ERR_STATE after
 * hpcg_set_factors, or where a system has more leaves than compute units.
 * AUTO (default): BRIDGE where the factors came in that format and it fits,
 * else FUSED where it fits, else STREAMING. */
typedef enum {
    HPCG_APPLY_AUTO = 0,
    HPCG_APPLY_STREAMING = 1,
    HPCG_APPLY_FUSED = 2,
    HPCG_APPLY_BRIDGE = 3
} hpcg_apply_path;

/* Arithmetic of the solve's vectors (hpcg_set_option(HPCG_OPT_PRECISION, ...)).
 * Factors and matrix values are fp32 and scalars and x are fp64 in both modes. */
typedef enum {
    HPCG_PREC_VEC64 = 0,        /* r, z, p, q and every accumulation in fp64 (default) */
    HPCG_PREC_VEC32 = 1         /* fp32 vectors and apply arithmetic, the plain
                                   reading of the pages' split ("Hierarchical
                                   Transformer Preconditioning for Interactive
                                   Physics Simulation", Supplementary sections 1
                                   and 7, "Mixed precision split": float32
                                   weights and apply path, float64 scalar
                                   accumulators; the vectors' type is not
                                   named).  On the grid systems it takes the
                                   fp64 count +-2.  On the tetrahedral system
                                   (P1 stiffness, 100:1 conductivity) CG is so
                                   sensitive to rounding that storing any one of
                                   r, z, p or q in fp32 costs about a quarter
                                   more iterations: the fp64 oracle with only
                                   that rounding added needs 630-641 steps
                                   against 517, and this mode takes ~671, with a
                                   true residual of ~1.03 tol.  Use VEC64 where
                                   the fp64 count matters.                     */
} hpcg_precision;

/* Bytes of device workspace hpcg_create needs for this partition and a CSR of
 * nnz_total stored entries (all systems together).  Returns 0 when the
 * partition is invalid.  The workspace must be 256-byte aligned.  The sizes
 * follow the pages' apply-path layout ("Hierarchical Transformer
 * Preconditioning for Interactive Physics Simulation", Supplementary section 2,
 * "Apply-path tensor layout", and Table 3: K leaf blocks of L x L, K - 1
 * tiles) with the per-level slabs of this library, and, for the block apply,
 * the dense leaf blocks U_k U_k^T (another L x L per leaf). */
size_t hpcg_workspace_bytes(const hpcg_partition* part, int64_t nnz_total);

/* Create a solver for one sparsity pattern and value set of A: the sparse SPD
 * matrix that the simulator hands over in CSR ("Hierarchical Transformer
 * Preconditioning for Interactive Physics Simulation", Supplementary section 1:
 * the GPU SpMV uses the generator's CSR, and the SpMV of section 5 stage (iii)
 * is the only sparse operation of the loop), with the leaf partition of
 * Supplementary section 2 (L = 128, K = n / L, weak admissibility).
 *  part        partition and batch size (validated: HPCG_ERR_SHAPE).
 *  d_row_ptr   int32 [batch*n + 1], d_row_ptr[0] == 0, nondecreasing,
 *              d_row_ptr[batch*n] == nnz_total.
 *  d_col       int32 [nnz_total] global column indices; row i of system s must
 *              only reference columns of system s.
 *  d_val       float32 [nnz_total].
 *  d_workspace at least hpcg_workspace_bytes(part, nnz_total) bytes.
 *  stream      a hipStream_t, or NULL for the null stream.
 *  out         receives the handle; untouched on error.
 * The CSR is copied into the workspace (stream-ordered), then copied back once
 * (synchronously) so the host can check the row pointer and that every column
 * index stays inside its system's block: HPCG_ERR_SHAPE otherwise. */
hpcg_status hpcg_create(const hpcg_partition* part, const int32_t* d_row_ptr,
                        const int32_t* d_col, const float* d_val, int64_t nnz_total,
                        void* d_workspace, size_t ws_bytes, void* stream,
                        hpcg_handle* out);

/* Replace the matrix values (same pattern) without rebuilding the handle, as a
 * simulator does from frame to frame ("Hierarchical Transformer
 * Preconditioning for Interactive Physics Simulation", section 1: A changes
 * every frame while the partition is reused).  d_val float32 [nnz_total], copied in stream
 * order. */
hpcg_status hpcg_set_values(hpcg_handle h, const float* d_val);

/* Load the preconditioner factors (the stand-in for the pages' network output:
 * leaf factors U_k with blocks F_k = U_k U_k^T, "A Neural Hierarchical-Matrix
 * Preconditioner for Real-Time GPU Solves", section 2 "Preconditioner";
 * rank-32 off-diagonal tiles and the diagonal gate of "Hierarchical
 * Transformer Preconditioning for Interactive Physics Simulation", section 4.4
 * "Decoder"), copied into the workspace in stream order:
 *  d_leafU  float32 [batch][K][L][L]            U_k, row-major, row = node in leaf
 *  d_tileW  float32 [batch][levels][K][L][R]    slab of leaf k at level l: a slab
 *           of U_{l,j} when (k >> l) is even, of V_{l,j} when it is odd
 *           (may be NULL when levels == 0)
 *  d_gate   float32 [batch][n]                  g, added as diag(g)
 * M is symmetric by construction; it must also be positive definite for PCG
 * (not checked here; a non-positive r.Mr is reported as HPCG_ERR_BREAKDOWN). */
hpcg_status hpcg_set_factors(hpcg_handle h, const float* d_leafU, const float* d_tileW,
                             const float* d_gate);

/* Load the preconditioner in the pages' own off-diagonal format: per-leaf
 * bridges U~_k, V~_k of L x R and one R x R core B_m per tile ("Hierarchical
 * Transformer Preconditioning for Interactive Physics Simulation", section 4.4
 * decoder heads and section 5 eqs. (2)-(5); packed width of Supplementary
 * Table 3).  Tile m of level l contributes U~_R B_m V~_C^T and its mirror.
 *  d_leafF    float32 [batch][K][L][L]   F_k (block F_k F_k^T), as d_leafU above
 *  d_bridgeU  float32 [batch][K][L][R]   U~_k
 *  d_bridgeV  float32 [batch][K][L][R]   V~_k
 *  d_cores    float32 [batch][M_H][R][R] B_m, M_H = sum over levels l of K/2^(l+1),
 *             tiles in level order, j ascending within a level
 *  d_gate     float32 [batch][n]
 * (the three off-diagonal pointers may be NULL when levels == 0).  The library
 * keeps the format as given for hpcg_apply_M (HPCG_APPLY_BRIDGE, the default
 * path after this call) and also expands it on the device into its per-level
 * slabs (W_l[k] = U~_k B_m for the row half of a tile, V~_k for the column
 * half; fp32 products), which the solve engines, the other apply paths and the
 * block calls use.  Stream-ordered. */
hpcg_status hpcg_set_factors_bridge(hpcg_handle h, const float* d_leafF, const float* d_bridgeU,
                                    const float* d_bridgeV, const float* d_cores, const float* d_gate);

/* y = M r for every system of the batch (asynchronous, stream-ordered): the
 * preconditioner application of "Hierarchical Transformer Preconditioning for
 * Interactive Physics Simulation", section 5 "Preconditioner Application",
 * stage (i) (the diagonal leaf blocks as one batched product over leaves) and
 * stage (ii) (restriction, strip aggregation, coupling and prolongation of
 * eqs. (2)-(5)), plus the diagonal gate; M is never assembled.  The form option may make it H H or
 * diag(A)^-1 instead.
 *  d_r, d_y float32 [batch*n], must not alias.
 * Returns an error only for bad arguments or a failed launch.  A single-pass
 * apply whose bounded partner wait runs out (see hpcg_apply_path) still
 * returns HPCG_OK here, since the call does not wait for the device: its y is
 * undefined and hpcg_apply_status reports it. */
hpcg_status hpcg_apply_M(hpcg_handle h, const float* d_r, float* d_y);

/* Synchronize the handle's stream and report whether any single-pass
 * hpcg_apply_M since the last report gave up a bounded wait (HPCG_ERR_HIP,
 * with text in hpcg_last_error; the record is then cleared) or not
 * (HPCG_OK).  hpcg_solve and hpcg_estimate_spectrum make the same check at
 * their final synchronization. */
hpcg_status hpcg_apply_status(hpcg_handle h);

/* y = A x for every system of the batch (asynchronous, stream-ordered): the
 * CSR SpMV of "Hierarchical Transformer Preconditioning for Interactive
 * Physics Simulation", section 5, stage (iii), the loop's only sparse
 * operation.  fp32 values and vectors,
 * entries of a row summed in stored order.
 * d_x, d_y float32 [batch*n], must not alias. */
hpcg_status hpcg_spmv(hpcg_handle h, const float* d_x, float* d_y);

/* Block products for a block of right-hand sides, e.g. the pages' probe block
 * Z of N x K_z with K_z = max(64, ceil(sqrt(N))) whose M A Z the training
 * objective needs ("Hierarchical Transformer Preconditioning for Interactive
 * Physics Simulation", project page, "Cosine Hutchinson Probe Loss" and
 * "Training Setup"; Supplementary section 3, "Probe vectors").  Every stage of
 * the apply (section 5, stages (i)-(ii), eqs. (2)-(5)) becomes a dense product
 * run on the matrix cores: fp32 products formed from fp16 pairs (each fp32
 * operand set scaled by a power of two and split into a high and a low fp16
 * part; three fp16 products per fp32 product, accumulated in fp32; about 22
 * bits per product), with the leaf stage one product with the dense leaf
 * blocks U_k U_k^T, formed at hpcg_set_factors.
 *
 * Layout: node-major, float32 [batch*n][nrhs] (the nrhs values of one node are
 * contiguous), 16-byte aligned; nrhs a multiple of 16 in [16, 1024] (pad the
 * block with zero columns otherwise: HPCG_ERR_SHAPE).  Asynchronous on the
 * handle's stream.
 *
 * hpcg_block_workspace_bytes: scratch that hpcg_apply_M_block needs for a given
 * nrhs (the per-leaf restrictions and their half sums), 0 for a bad nrhs or
 * handle.  The caller owns it; it may be reused once the stream has passed.
 *
 * hpcg_apply_M_block: Y = M R for every system and column.  d_R and d_Y must
 * not alias.  d_work may be NULL when levels == 0.
 *
 * hpcg_spmv_block: Y = A X for every system and column.  d_X and d_Y must not
 * alias. */
size_t hpcg_block_workspace_bytes(hpcg_handle h, int32_t nrhs);
hpcg_status hpcg_apply_M_block(hpcg_handle h, const float* d_R, float* d_Y, int32_t nrhs,
                               void* d_work, size_t work_bytes);
hpcg_status hpcg_spmv_block(hpcg_handle h, const float* d_X, float* d_Y, int32_t nrhs);

/* hpcg_apply_M_block without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same kernels and result as
 * hpcg_apply_M_block; the per-leaf restrictions and their half sums live in a
 * fixed scratch of 32 MiB that the library holds on every GPU it runs on until
 * the process ends (its address is looked up at hpcg_create).  Limit: 2 *
 * batch * levels * K * 32 * nrhs * 4 bytes must fit in it (e.g. n = 16,384
 * with nrhs <= 128, or n = 8,192 with nrhs <= 256); larger calls return
 * HPCG_ERR_WORKSPACE.  Allocates nothing and launches only kernels.  Every
 * call on a GPU shares that GPU's scratch and leaves it as it was written:
 * calls that overlap in time on one GPU (other streams, other handles, other
 * threads) race and must be ordered by the caller. */
hpcg_status hpcg_apply_M_block_noalloc(hpcg_handle h, const float* d_R, float* d_Y, int32_t nrhs);

/* Solve A x = b for every system with preconditioned conjugate gradients
 * ("Hierarchical Transformer Preconditioning for Interactive Physics
 * Simulation", project page, Introduction and Background, eq. (1); section 5
 * "Single-graph capture": the whole iteration, apply, SpMV, vector updates
 * and dot reductions, runs on the device without host dispatch), x_0 = 0,
 * stopping a system when its
 * recursively updated residual satisfies ||r_k||_2 <= tol * ||b||_2 (the
 * pages' ||r_k|| / ||r_0|| with r_0 = b: Supplementary section 1,
 * "Convergence criterion"), or after maxit iterations.
 *  d_b      float32 [batch*n]
 *  d_x      float64 [batch*n]  solution (written also when not converged)
 *  tol      > 0;  maxit >= 1
 *  h_iters  int32 [batch] or NULL: products q = A p done when the test passed
 *           (maxit when not converged; the iteration of the failure on breakdown)
 *  h_relres float64 [batch] or NULL: ||r||/||b|| of the recursive residual at exit
 * Scalars (dot products, norms, step sizes) and x are fp64; vectors follow
 * HPCG_OPT_PRECISION.
 * Returns HPCG_OK when every system converged, HPCG_ERR_BREAKDOWN when any
 * system broke down, else HPCG_ERR_NOT_CONVERGED when any system ran out of
 * iterations; HPCG_ERR_HIP when a bounded wait of the solve ran out, or when an
 * earlier single-pass hpcg_apply_M had (see hpcg_apply_status).  Synchronizes
 * the handle's stream before returning. */
hpcg_status hpcg_solve(hpcg_handle h, const float* d_b, double* d_x, double tol,
                       int32_t maxit, int32_t* h_iters, double* h_relres);

/* Solve to a tight tolerance with an outer iterative refinement in fp64
 * around the configured solve ("Hierarchical Transformer Preconditioning for
 * Interactive Physics Simulation", Supplementary section 7: for rtol <= 1e-10
 * the pages propose an outer refinement loop that keeps the float32 apply as
 * the inner preconditioner):
 *   x = 0;  repeat:  r = b - A x (fp64);  stop when ||r|| <= tol ||b||;
 *                    solve A d = r / ||r|| to inner_tol (engine and vector
 *                    precision as set by hpcg_set_option);  x += ||r|| d.
 *  d_b, d_x   as for hpcg_solve (x is overwritten, fp64)
 *  tol        outer tolerance on the true residual ||b - A x|| / ||b||
 *  maxit      budget of inner iterations per system, summed over the outer steps
 *  inner_tol  in (0, 1), e.g. 1e-5 with fp32 vectors
 *  max_outer  >= 1
 *  h_iters    [batch] inner iterations summed (may be NULL)
 *  h_outer    [batch] outer steps taken (may be NULL)
 *  h_relres   [batch] final true relative residual, fp64 (may be NULL)
 * Statuses as for hpcg_solve; scratch lives in the workspace.  Synchronizes
 * with the host once per outer step. */
hpcg_status hpcg_solve_refined(hpcg_handle h, const float* d_b, double* d_x, double tol, int32_t maxit,
                               double inner_tol, int32_t max_outer, int32_t* h_iters, int32_t* h_outer,
                               double* h_relres);


/* Block PCG: for every system s and column j of a block of right-hand sides,
 * an independent preconditioned CG on A_s x = b_{s,j} (x_0 = 0, stop when
 * ||r|| <= tol ||b||, the rules of hpcg_solve), run in lockstep so that each
 * application of M is one block apply on the matrix cores and each product
 * with A one block SpMV: the multi-vector form of "Hierarchical Transformer
 * Preconditioning for Interactive Physics Simulation", section 5, stages
 * (i)-(ii).  Columns share nothing but the launches; each keeps its own step
 * sizes, test and count, and a finished column stays as it was while the
 * others continue.
 *  d_B      fp32 [batch*n][nrhs], node-major (the block apply's layout), 16-byte aligned
 *  d_X      fp64 [batch*n][nrhs] out, node-major, 16-byte aligned
 *  nrhs     multiple of 16 in [16, 1024]
 *  d_work   device scratch of hpcg_block_solve_workspace_bytes(h, nrhs) bytes
 *  h_iters  [batch*nrhs] iterations per (system, column), system-major (may be NULL)
 *  h_relres [batch*nrhs] final recursive ||r|| / ||b|| (may be NULL)
 * Arithmetic: R, Z, P, Q fp32 (the block apply's), x and all scalars fp64:
 * the pages' split, so on the tetrahedral system the columns need about a
 * quarter more iterations than fp64 PCG, as HPCG_PREC_VEC32 does.  Each row
 * of A P is summed in fp64 and rounded to fp32 once, so that the true
 * residual ||b - A x|| stays with the recursive one.
 * Direct form only (HPCG_ERR_STATE otherwise).  Returns HPCG_ERR_BREAKDOWN or
 * HPCG_ERR_NOT_CONVERGED when some column ends so (x and counts still
 * written).  Records the iterations in a hipGraph, kept for repeated calls
 * with the same buffers; synchronizes with the host once per replay. */
size_t hpcg_block_solve_workspace_bytes(hpcg_handle h, int32_t nrhs);
hpcg_status hpcg_solve_block(hpcg_handle h, const float* d_B, double* d_X, int32_t nrhs, double tol, int32_t maxit,
                             void* d_work, size_t work_bytes, int32_t* h_iters, double* h_relres);

/* Measurement aid (no part of the solve): read `bytes` from d_src with one
 * launch of `workgroups` workgroups, as fast as plain 16-byte loads go, and
 * write one float per workgroup to d_sink [workgroups].  Timing it over the
 * apply's bytes gives the read ceiling that the apply's bandwidth is quoted
 * against (from the Infinity Cache when the same bytes are read back to back,
 * from HBM when the buffers cycled exceed it).  bytes a positive multiple of
 * 16, d_src 16-byte aligned; asynchronous on `stream` (a hipStream_t or
 * NULL).  Errors are reported through hpcg_last_error(NULL). */
hpcg_status hpcg_read_probe(const void* d_src, size_t bytes, float* d_sink, int32_t workgroups, void* stream);

/* Measurement aid: the in-kernel timeline of a library built with HPCG_TRACE
 * (python -m matrix_preconditioned_pcg_amd.timeline builds and reads it).
 * Kernels record the 100 MHz real-time counter at fixed points of their work
 * (slot s of workgroup w at index w * 16 + s, 4,096 workgroups); this copies
 * the first `count` entries to h_out and, if clear != 0, zeroes the table.
 * Synchronous.  The ordinary build returns HPCG_ERR_STATE. */
hpcg_status hpcg_trace_read(uint64_t* h_out, size_t count, int32_t clear);

/* Per-system hpcg_system_status values of the last hpcg_solve, int32 [batch]. */
hpcg_status hpcg_last_solve_status(hpcg_handle h, int32_t* h_status);

/* Engine and tuning options (see hpcg_option). */
hpcg_status hpcg_set_option(hpcg_handle h, int32_t option, int32_t value);

/* Extreme eigenvalues of H, the factor operator (M itself in the direct form,
 * M = H H in the squared form), whatever the form option says: the monitor of
 * lambda_min(H) that "A Neural Hierarchical-Matrix Preconditioner for
 * Real-Time GPU Solves", section 2, pairs with a Jacobi fallback.  `steps`
 * Lanczos steps (2 .. 200) on the host in fp64, with full reorthogonalization,
 * around the device apply, from a fixed pseudo-random start vector over the
 * whole batch (so the result covers every system of the batch).  Ritz values
 * lie inside the spectrum: *h_lmin <= 0 shows that H is not positive definite
 * (up to the fp32 apply's rounding); a positive value is an upper estimate of
 * lambda_min.  Requires factors.  Synchronous; uses the workspace as scratch. */
hpcg_status hpcg_estimate_spectrum(hpcg_handle h, int32_t steps, double* h_lmin, double* h_lmax);

/* 1 if the last hpcg_solve fell back to Jacobi (HPCG_OPT_FALLBACK), else 0. */
int32_t hpcg_last_fallback(hpcg_handle h);

/* Path the last hpcg_apply_M call took (an hpcg_apply_path; 0 before any). */
int32_t hpcg_last_apply_path(hpcg_handle h);

/* Engine the last hpcg_solve actually ran (an hpcg_engine value), or 0. */
int32_t hpcg_last_engine(hpcg_handle h);

/* Launch shape of the last hpcg_solve: *grid workgroups per phase launch and
 * the largest dynamic LDS a phase used, in bytes.  Either pointer may be NULL. */
hpcg_status hpcg_last_launch_info(hpcg_handle h, int32_t* grid, int32_t* lds_bytes);

/* Static text for a status code. */
const char* hpcg_status_string(hpcg_status s);

/* Text of the last error on this handle ("" when none); NULL handle gives the
 * last error of a failed hpcg_create on this thread. */
const char* hpcg_last_error(hpcg_handle h);

/* Release the handle (and its graph / pinned host memory).  Does not free the
 * caller's workspace.  NULL is ignored. */
void hpcg_destroy(hpcg_handle h);

#ifdef __cplusplus
}
#endif

#endif /* HPCG_H */
