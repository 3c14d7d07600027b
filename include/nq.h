/*
 * nq.h -- C ABI of the LB-ADMM low-rank binary factorisation library (gfx950).
 *
 * The library computes, for one linear layer, NanoQuant's Latent Binary ADMM
 * ("NanoQuant: Efficient Sub-1-Bit Quantization of Large Language Models",
 * digest at paper.rainbus.top):
 *   - section 方法步骤详情 (method steps), stage 2 step (2): precondition the
 *     target, Wt = D_out * W * D_in; run LB-ADMM; after convergence balance
 *     the magnitudes of the two factors and extract channel scales s1, s2;
 *     step (3): take signs and pack them into an integer format;
 *   - section 核心方法 (core method): each iteration (a) fixes V and solves
 *     the regularised linear system for U through a Cholesky factorisation,
 *     (b) maps the continuous U to the binary proxy Z with SVID, (c) updates
 *     the dual variable; then the same for V;
 *   - section 研究动机 (motivation): the representation
 *     W ~ s1 * U_{+-1} * V_{+-1}^T * s2.
 * The pages give names, not formulas; the formulas implemented are:
 *   G = V^T V + rho I,  U = (Wt V + rho (Z_U - Lam_U)) G^{-1},
 *   X = U + Lam_U,  Z_U = SVID_T(X) = sign(X) .* (a b^T)  with (a, b) from T
 *   alternating rank-1 least-squares steps on |X| starting at b = 1,
 *   Lam_U = X - Z_U;  then the V-half with Wt^T and the new U.
 *   Finish: c_k = sqrt(||v_k|| / ||u_k||), u_k *= c_k, v_k /= c_k;
 *   s1_i = mean_k |U_ik|, s2_j = mean_k |V_jk| (Wt space), returned divided
 *   by d_out, d_in (W space); bits = [x >= 0] of the balanced latents.
 *
 * Conventions for every entry point:
 *   - Matrices are row-major float32 with an explicit leading dimension in
 *     elements (ld >= number of columns). W is m x n = [out, in].
 *   - Pointers marked "device" must be device memory of the current HIP
 *     device, 4-byte aligned (uint32 / float). Host pointers are marked.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued on it; calls return before it finishes
 *     unless stated otherwise.
 *   - Nothing throws or aborts across this boundary; errors are status codes.
 *     Argument errors are detected before any device work is enqueued.
 *     nq_last_error_message() gives text for the last failure on the calling
 *     thread.
 *   - Outputs are owned by the caller; handles own their device workspace.
 */
#ifndef NQ_H_
#define NQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nq_status {
  NQ_OK = 0,
  NQ_ERR_INVALID_ARG = 1,           /* bad size, pointer, ld, rho, iters, flags    */
  NQ_ERR_UNSUPPORTED = 2,           /* no usable gfx950 device / shape not allowed */
  NQ_ERR_OUT_OF_MEMORY = 3,         /* device allocation failed                    */
  NQ_ERR_HIP = 4,                   /* a HIP runtime call failed, or an SVID
                                       launch's workgroups were not all resident
                                       within its wait bound (about 0.5 s)         */
  NQ_ERR_NOT_POSITIVE_DEFINITE = 5, /* a Cholesky pivot was <= 0 or not finite     */
  NQ_ERR_NONFINITE = 6,             /* NaN/Inf in the input or produced on device  */
  NQ_ERR_BAD_PRECONDITIONER = 7     /* an entry of d_out or d_in is not > 0        */
} nq_status;

/* Flags of nq_lbadmm_desc.flags. */
#define NQ_FLAG_COMPUTE_ERROR 0x1u  /* compute rel. reconstruction errors into stats     */
#define NQ_FLAG_INIT_DRAWS    0x2u  /* U0/V0 are standard-normal draws that the run
                                       scales by sigma0 (without it they are the starting
                                       latents themselves, e.g. a warm start)            */
#define NQ_FLAG_NO_BALANCE    0x4u  /* skip magnitude balancing (U, V, scales and bits
                                       then come from the raw latents)                   */
#define NQ_FLAG_SINGLE_STREAM 0x8u  /* no internal second stream: the r x r chain runs
                                       on `stream` after the right-hand-side GEMM        */
#define NQ_FLAG_PROFILE       0x10u /* record HIP events around each phase of every run
                                       (see nq_lbadmm_profile)                           */
#define NQ_FLAG_PROFILE_RHS_ONLY 0x20u /* with NQ_FLAG_PROFILE: time only
                                       NQ_PHASE_GEMM_RHS (each event pair costs a little
                                       device time; the other phases get none)           */
/* Iterative solve in place of the Cholesky factor (the gradient-descent
 * solver of the implementation blog, section 待办事项): each half takes
 * desc.solve_steps steps per row on u G = r, G = other^T other + rho I,
 * from the factor's previous value. At most one of the two; neither = the
 * exact Cholesky solve. */
#define NQ_FLAG_SOLVE_CG      0x40u /* conjugate gradients                               */
#define NQ_FLAG_SOLVE_GD      0x80u /* steepest descent, exact step along the gradient   */

/* Phases timed under NQ_FLAG_PROFILE. */
typedef enum nq_phase {
  NQ_PHASE_GEMM_RHS = 0,   /* R = Wt V + rho (Z - Lam) (one launch per half-iteration)   */
  NQ_PHASE_GEMM_SOLVE = 1, /* U = R G^-1 and U^T (one launch per half-iteration); with an
                              iterative solve: all of its steps and U^T                   */
  NQ_PHASE_CHAIN = 2,      /* Gram + Cholesky/inverse factor + L^-T L^-1 (per half); with
                              an iterative solve: the Gram and its reduction to G          */
  NQ_PHASE_SVID = 3,       /* SVID power steps + dual update (per half)                   */
  NQ_PHASE_PREP = 4,       /* preconditioning, norms, init latents, initial SVIDs         */
  NQ_PHASE_FINISH = 5,     /* balancing, scales, packing, errors                          */
  NQ_NUM_PHASES = 6
} nq_phase;

typedef struct nq_lbadmm_desc {
  int64_t m;          /* rows of W (output features), 1 .. 2^21 - 256              */
  int64_t n;          /* columns of W (input features), 1 .. 2^21 - 256            */
  int64_t r;          /* rank of the binary factors, 1 .. 2^13                     */
  float rho;          /* ADMM penalty, > 0 and finite                              */
  int32_t iters;      /* ADMM iterations (each: U-half then V-half), >= 0          */
  int32_t svid_steps; /* alternating rank-1 steps inside SVID, >= 1                */
  uint64_t seed;      /* seed of the built-in initialiser (used when U0/V0 are
                         NULL): Philox4x32-10 counter-based normals               */
  uint32_t flags;     /* NQ_FLAG_*                                                 */
  int32_t solve_steps; /* steps per half of NQ_FLAG_SOLVE_CG / _GD, 1 .. 10000;
                          must be 0 without those flags                           */
} nq_lbadmm_desc;

typedef struct nq_lbadmm_stats {
  double rel_err_wtilde; /* ||Wt - diag(s1w) S_U S_V^T diag(s2w)||_F / ||Wt||_F
                            (NaN unless NQ_FLAG_COMPUTE_ERROR)                       */
  double rel_err_w;      /* same in W space with the returned s1, s2               */
  double sumsq_wtilde;   /* ||Wt||_F^2                                              */
  double sigma0;         /* init scale (||Wt||_F^2 / (m n r))^(1/4)                 */
  int64_t potrf_info;    /* 0, or 1 + the first column whose Cholesky pivot was
                            <= 0 / not finite (over all factorisations of the run) */
  int32_t nonfinite;     /* nonzero if NaN/Inf was seen in W, the preconditioned
                            target or the final latents                            */
  int32_t bad_precond;   /* nonzero if some d_out / d_in entry was not > 0          */
  float elapsed_ms;      /* device time of the whole run (HIP events)               */
  int32_t iters_done;
  int32_t reserved;
} nq_lbadmm_stats;

typedef struct nq_lbadmm* nq_lbadmm_t;

/* Create a factorisation handle and allocate all of its device workspace on
 * the current HIP device. Sizes are rounded up internally to tile multiples
 * (256 for m and n, 128 for r); padding is zero and never visible to callers.
 * Returns NQ_ERR_INVALID_ARG for a NULL argument or a desc field out of
 * range, NQ_ERR_UNSUPPORTED when the current device is not gfx950,
 * NQ_ERR_OUT_OF_MEMORY / NQ_ERR_HIP on allocation failure (*out = NULL). */
nq_status nq_lbadmm_create(const nq_lbadmm_desc* desc, nq_lbadmm_t* out);

/* Device bytes the handle for `desc` allocates (host output). */
nq_status nq_lbadmm_workspace_bytes(const nq_lbadmm_desc* desc, size_t* bytes);

/* Run the whole per-layer path on `stream`:
 *   precondition -> init -> `iters` ADMM iterations -> balance -> scales ->
 *   sign packing (-> errors if NQ_FLAG_COMPUTE_ERROR).
 * Inputs (device): W m x n (ld ldw >= n), d_out (m), d_in (n), all > 0.
 *   U0 (m x r, ld r) and V0 (n x r, ld r): the starting latents as given, or
 *   with NQ_FLAG_INIT_DRAWS standard-normal draws that the run scales by
 *   sigma0. Both NULL: sigma0 times normals from the built-in Philox
 *   generator and desc.seed.
 *   Exactly one NULL is NQ_ERR_INVALID_ARG.
 * Outputs (device, caller-owned, contiguous):
 *   U (m x r) and V (n x r): the balanced latents;
 *   s1 (m), s2 (n): W-space scales, so W ~ diag(s1) sign(U) sign(V)^T diag(s2);
 *   U_bits (m x ceil(r/32)) and V_bits (n x ceil(r/32)) uint32 words, bit k of
 *   word w of row i = [latent(i, 32 w + k) >= 0], unused high bits zero.
 *   Any output pointer may be NULL to skip it.
 * stats (host, nullable): if non-NULL the call waits for `stream`, fills it
 *   and returns NQ_ERR_NONFINITE / NQ_ERR_BAD_PRECONDITIONER /
 *   NQ_ERR_NOT_POSITIVE_DEFINITE when the device saw such data. With
 *   stats == NULL the call is asynchronous and nq_lbadmm_query() reports.
 * The call allocates nothing. A handle is not thread-safe and must not run
 * twice concurrently; distinct handles may run concurrently on distinct
 * streams. */
nq_status nq_lbadmm_run(nq_lbadmm_t h, const float* W, int64_t ldw,
                        const float* d_out, const float* d_in,
                        const float* U0, const float* V0,
                        float* U, float* V, float* s1, float* s2,
                        uint32_t* U_bits, uint32_t* V_bits,
                        nq_lbadmm_stats* stats, void* stream);

/* Wait for the handle's last run on its stream and fill `stats` (host);
 * returns the same data-dependent status as a run with stats != NULL. */
nq_status nq_lbadmm_query(nq_lbadmm_t h, nq_lbadmm_stats* stats);

/* Copy the ADMM state left by the last run (before balancing) into caller
 * buffers (device, contiguous, each nullable): U (m x r), V (n x r), and the
 * proxies and scaled duals Z_U, Lam_U (m x r), Z_V, Lam_V (n x r).
 * Enqueued on `stream`. */
nq_status nq_lbadmm_get_state(nq_lbadmm_t h, float* U, float* V,
                              float* Z_U, float* Lam_U, float* Z_V, float* Lam_V,
                              void* stream);

/* Under NQ_FLAG_PROFILE: wait for the handle's pending work and return, per
 * nq_phase, the summed device time in ms (ms[NQ_NUM_PHASES], host) and the
 * number of timed intervals (count[NQ_NUM_PHASES], host) since the last reset;
 * reset != 0 clears the totals afterwards. Each interval is bracketed by HIP
 * events on the stream its kernels run on. Events are kept in a ring sized
 * for 8 runs; a run that would overflow it first waits for the pending ones.
 * NQ_ERR_INVALID_ARG if the handle was created without NQ_FLAG_PROFILE. */
nq_status nq_lbadmm_profile(nq_lbadmm_t h, double* ms, int64_t* count, int32_t reset);

/* Measurement of the SVID + dual update on its own (digest, section 核心方法
 * steps (b) and (c)): after a run, enqueue on `stream` `reps` (>= 1) updates
 * of factor `factor` (0 = U, 1 = V) back to back, each exactly as a
 * half-iteration makes it (X = latent + Lam, `svid_steps` rank-1 steps on
 * |X|, Lam = X - Z, P = Z - Lam, one launch), wait, and return the average
 * device time per update in ms from HIP events (*avg_ms, host). The handle's
 * duals and proxies change; the next run starts afresh from its inputs.
 * NQ_ERR_INVALID_ARG before the first run or for a bad factor / reps;
 * NQ_ERR_HIP if a launch failed or its workgroups were not co-resident. */
nq_status nq_lbadmm_time_svid(nq_lbadmm_t h, int32_t factor, int32_t reps, void* stream,
                              double* avg_ms);

/* Free the handle and its workspace (NULL is ignored). Waits for its work. */
void nq_lbadmm_destroy(nq_lbadmm_t h);

/* Pack sign bits ("方法步骤详情" step (3): signs packed to an integer format).
 * X (device) rows x cols, ld ldx >= cols; bits (device) rows x ld_words uint32,
 * ld_words >= ceil(cols/32). bit k of word w of row i = [X(i, 32 w + k) >= 0]
 * (so +0 and -0 give 1, NaN gives 0); bits beyond cols in the last word are 0;
 * words beyond ceil(cols/32) are not written. rows == 0 or cols == 0 is a
 * no-op. One kernel, no allocation. */
nq_status nq_pack_signs(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                        uint32_t* bits, int64_t ld_words, void* stream);

/* ---- applying a factorised layer ----
 * The layer is kept as W ~ diag(s1) S_U S_V^T diag(s2) (m x n; "研究动机"),
 * and applied without forming W, as the pages' binary GEMV/GEMM kernels do
 * ("技术新颖性"). */

/* Transposed sign bits: in holds rows x cols signs (rows x ld_in uint32
 * words, the layout of nq_pack_signs), out (cols x ld_out words, ld_out >=
 * ceil(rows/32)) receives the cols x rows signs of the transpose, bits past
 * `rows` in each last word zero, words past ceil(rows/32) untouched. Both on
 * the device; no allocation. Used once per layer to turn the V_bits of a run
 * (n x r) into the S_V^T bits (r x n) that nq_binary_matmul reads. */
nq_status nq_transpose_signs(const uint32_t* in, int64_t rows, int64_t cols, int64_t ld_in,
                             uint32_t* out, int64_t ld_out, void* stream);

/* Y = X W^T for W = diag(s1) S_U S_V^T diag(s2): row b of Y is
 * s1 * (S_U (S_V^T (s2 * x_b))). All pointers on the device.
 *   U_bits  m x ldu words (ldu >= ceil(r/32)): S_U, as nq_lbadmm_run returns it;
 *   Vt_bits r x ldvt words (ldvt >= ceil(n/32)): S_V^T (nq_transpose_signs of V_bits);
 *   s1 (m), s2 (n) float32; X: B x n float32, row stride ldx >= n;
 *   Y: B x m float32, row stride ldy >= m (written, not read);
 *   work: nq_binary_matmul_work_floats(B, n, r) float32 of caller scratch
 *         (partial sums of the r projections per input, then the inputs
 *         as bf16 terms), 16-byte aligned.
 * One input: two launches (lookup tables). Two or more: four (the inputs
 * split into exact bf16 terms, the matrix-core product, the same for the
 * projections). All on `stream`, no allocation, no host synchronisation.
 * Sums run in a fixed order, so results are bit-reproducible. m == 0 or
 * B == 0 is a no-op; otherwise n, r >= 1. NQ_ERR_INVALID_ARG for bad sizes
 * or strides. */
nq_status nq_binary_matmul(const uint32_t* U_bits, int64_t ldu, const uint32_t* Vt_bits,
                           int64_t ldvt, int64_t m, int64_t n, int64_t r, const float* s1,
                           const float* s2, const float* X, int64_t B, int64_t ldx, float* Y,
                           int64_t ldy, float* work, void* stream);

/* Floats of `work` that nq_binary_matmul needs for B inputs of width n and
 * rank r: 8 B r (rounded up to 64) + 3072 ceil(B / 16) ceil(max(n, r) / 128).
 * Host only; -1 for negative sizes. */
int64_t nq_binary_matmul_work_floats(int64_t B, int64_t n, int64_t r);

/* nq_binary_matmul for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. The same arguments and result (bit for bit) as
 * nq_binary_matmul without `work`: the workspace is a fixed scratch array
 * of 2^23 float32 (32 MiB) in the library, one per GPU, taken on the first
 * call on a device (the current device) and held until the process ends.
 * Limit: nq_binary_matmul_work_floats(B, n, r) <= 2^23, else
 * NQ_ERR_INVALID_ARG before any device work. Calls no allocating routine.
 * Every call on one GPU uses that GPU's one array: calls whose device work
 * overlaps (other streams, other threads) race and give wrong results; calls
 * ordered on one stream are safe. Nothing in the array needs clearing
 * between calls. */
nq_status nq_binary_matmul_noalloc(const uint32_t* U_bits, int64_t ldu, const uint32_t* Vt_bits,
                                   int64_t ldvt, int64_t m, int64_t n, int64_t r,
                                   const float* s1, const float* s2, const float* X, int64_t B,
                                   int64_t ldx, float* Y, int64_t ldy, void* stream);

/* ---- diagonal preconditioners from activation samples ----
 * The digest's first stage (方法步骤详情, stage 1) collects statistics z_in
 * and z_out of each linear layer's activations and builds robust diagonal
 * preconditioners D_in and D_out with Ledoit-Wolf shrinkage (a simplified
 * diagonal K-FAC, 前置知识). The formulas implemented (the pages give none):
 * for a sample Z (N tokens x p features), S = Z^T Z / N (uncentered),
 * m = tr(S) / p, Ledoit & Wolf's (J. Multivariate Anal. 88, 2004) intensity
 * shrinkage = min(b2bar, d2) / d2 with d2 = ||S - m I||^2 and
 * b2bar = N^-2 sum_k ||z_k z_k^T - S||^2 (||A||^2 = tr(A A^T) / p), and
 * D_jj = sqrt((1 - shrinkage) S_jj + shrinkage m). D_in comes from the
 * layer's input sample, D_out from its output-side sample; they are the
 * d_in, d_out of nq_lbadmm_run. */
typedef struct nq_lw* nq_lw_t;

/* Handle for one feature dimension p (1 .. 16384) taking chunks of at most
 * max_rows rows (1 .. 2^20, p * max_rows <= 2^30). Allocates its device
 * workspace on the current device (about 8 p^2 bytes for S in fp64, 12 p^2
 * for the Gram, 4 p max_rows for a staged chunk). NQ_ERR_INVALID_ARG for bad
 * sizes, NQ_ERR_UNSUPPORTED without a gfx950 device. */
nq_status nq_lw_create(int64_t p, int64_t max_rows, nq_lw_t* out);

/* Add the samples Z (device, rows x p floats, row stride ldz >= p; rows
 * above max_rows are taken in pieces) to the running statistics, on
 * `stream`. Asynchronous; Z must stay valid until the stream reaches the
 * call. Calls on one handle must be ordered on one stream. rows == 0 is a
 * no-op. */
nq_status nq_lw_accumulate(nq_lw_t h, const float* Z, int64_t rows, int64_t ldz, void* stream);

/* d (device, p floats) = the diagonal of D over all samples added since
 * creation or the last reset. If shrinkage (host) is non-NULL it receives
 * the intensity and the call waits for `stream`. NQ_ERR_INVALID_ARG when no
 * sample was added. The statistics are kept: more chunks may follow. */
nq_status nq_lw_finalize(nq_lw_t h, float* d, double* shrinkage, void* stream);

/* Forget the samples (no device work; the next accumulate clears). */
nq_status nq_lw_reset(nq_lw_t h);
nq_status nq_lw_destroy(nq_lw_t h);

/* ---- STE refinement of a factorised layer ----
 * The digest's stage 2 step (3) (方法步骤详情) refines the continuous latents
 * U, V and the scales s1, s2 of each layer jointly with a straight-through
 * estimator against the MSE of the quantised output, then takes the signs;
 * its reproduction settings (复现评估) use lr 1e-4 -> 1e-6 with a cosine
 * schedule, batches of 1-4 samples, 8 epochs. The formulas implemented (the
 * pages give none): for a batch X (T x n) and target Y = X W^T (T x m),
 * Yq = X diag(s2) sign(V) sign(U)^T diag(s1), loss = mean((Yq - Y)^2) over
 * T x m; sign(x >= 0) = +1 and d sign / dx taken as 1; one Adam step
 * (beta1 0.9, beta2 0.999, eps 1e-8, bias-corrected) on U, V, s1, s2 per
 * batch. The caller owns the schedule and passes each step's lr. */
typedef struct nq_ste* nq_ste_t;

/* Handle for a layer m x n of rank r and batches of up to max_tokens tokens
 * (all >= 1; m, n, max_tokens <= 2^21 - 256, r <= 2^13). Allocates every
 * buffer on the current device; steps allocate nothing. */
nq_status nq_ste_create(int64_t m, int64_t n, int64_t r, int64_t max_tokens, nq_ste_t* out);

/* Start from U (m x r), V (n x r), s1 (m), s2 (n), device, contiguous (the
 * outputs of nq_lbadmm_run); clears the Adam state. */
nq_status nq_ste_set_params(nq_ste_t h, const float* U, const float* V, const float* s1,
                            const float* s2, void* stream);

/* One step on T tokens (1 .. max_tokens): rows t of the batch are
 * X[rows[t]] and Y[rows[t]] (rows: device int32, or NULL for rows 0 .. T-1;
 * every index must be a row of X and Y: the library cannot check it);
 * X (row stride ldx >= n) and Y (ldy >= m) device float32. Computes the loss
 * of the current parameters on the batch (kept for nq_ste_last_loss) and
 * takes one Adam step with learning rate lr (finite, >= 0). Asynchronous on
 * `stream`; calls on one handle must be ordered on one stream. */
nq_status nq_ste_step(nq_ste_t h, const float* X, int64_t ldx, const float* Y, int64_t ldy,
                      const int32_t* rows, int64_t T, float lr, void* stream);

/* The loss of the last step's batch before its update (host double); waits
 * for `stream`. */
nq_status nq_ste_last_loss(nq_ste_t h, double* loss, void* stream);

/* Copy the current parameters out (device, contiguous; any may be NULL).
 * Their signs packed by nq_pack_signs are the refined binary factors. */
nq_status nq_ste_get_params(nq_ste_t h, float* U, float* V, float* s1, float* s2, void* stream);
nq_status nq_ste_destroy(nq_ste_t h);

/* ---- building blocks (the same kernels the run uses; for tests and tools) ----
 * These take caller buffers of any shape, copy into zero-padded temporaries
 * (hipMalloc, freed before the call returns), run the kernels on `stream`,
 * copy results out and wait for `stream`. They are not meant for the hot
 * path. */

/* Wt = d_out_i * (W_ij * d_in_j) in float32, the two products rounded in that
 * order ("方法步骤详情": Wt = D_out W D_in). Wt (device) m x n, ld ldwt. */
nq_status nq_op_precondition(const float* W, int64_t ldw, int64_t m, int64_t n,
                             const float* d_out, const float* d_in,
                             float* Wt, int64_t ldwt, void* stream);

/* G = A^T A + rho I for A (device) rows x cols (ld lda); G (device) cols x cols
 * (ld ldg), full symmetric ("核心方法" (a): the regularised system matrix). */
nq_status nq_op_gram(const float* A, int64_t rows, int64_t cols, int64_t lda,
                     float rho, float* G, int64_t ldg, void* stream);

/* C = A B + rho P for A rows x k (lda), B k x cols (ldb), P rows x cols (ldp,
 * nullable = 0); C rows x cols (ldc). The right-hand side of "核心方法" (a). */
nq_status nq_op_gemm_rhs(const float* A, int64_t lda, const float* B, int64_t ldb,
                         const float* P, int64_t ldp, float rho,
                         float* C, int64_t ldc,
                         int64_t rows, int64_t cols, int64_t k, void* stream);

/* C = A S^T for A rows x k (lda) and S cols x k (lds) with entries +-1: the
 * products of the STE step through the sign matrices ("方法步骤详情", stage 2
 * step (3)), on the bf16 matrix cores with A split into three exact bf16
 * terms (entries of S other than +-1 and 0 are cut to bf16). C rows x cols
 * (ldc); Ct (nullable) cols x rows (ldct) receives C^T. */
nq_status nq_op_sign_gemm(const float* A, int64_t lda, const float* S, int64_t lds,
                          float* C, int64_t ldc, float* Ct, int64_t ldct,
                          int64_t rows, int64_t cols, int64_t k, void* stream);

/* Cholesky factorisation G = L L^T of an SPD r x r matrix (lower triangle of
 * G read) and the inverse Ginv = L^-T L^-1 (full symmetric; formed, as in the
 * run, as the Gram product M^T M of M = L^-1). Ginv (device, nullable)
 * ld ldgi; L (device, nullable) ld ldl receives the factor with zeros above
 * the diagonal. *info (host) is 0 or 1 + the first failing column; the call
 * waits for `stream`. */
nq_status nq_op_cholesky_inverse(const float* G, int64_t r, int64_t ldg,
                                 float* L, int64_t ldl, float* Ginv, int64_t ldgi,
                                 int64_t* info, void* stream);

/* SVID ("核心方法" (b), "技术新颖性"): Z = sign(X) .* (a b^T) with T rank-1
 * alternating steps on |X| from b = 1. X, Z (device) rows x cols (ld ldx,
 * ldz); a (rows) and b (cols) device, nullable. */
nq_status nq_op_svid(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                     int32_t T, float* Z, int64_t ldz, float* a, float* b,
                     void* stream);

/* SVID fused with the dual update, as one half-iteration does it ("核心方法"
 * (b) and (c)): X = U + Lam, Z = SVID_T(X), Lam_out = X - Z. U and Lam
 * (device) rows x cols, ld ldi; Z and Lam_out (device) rows x cols, ld ldo;
 * a (rows), b (cols) device, nullable. Staged through padded temporaries
 * (rows to 256, cols to 128); the call waits for `stream`. NQ_ERR_HIP also
 * when the launch's workgroups were not all resident within its wait bound. */
nq_status nq_op_svid_dual(const float* U, const float* Lam, int64_t rows, int64_t cols,
                          int64_t ldi, int32_t T, float* Z, float* Lam_out, int64_t ldo,
                          float* a, float* b, void* stream);

const char* nq_status_string(nq_status s);
const char* nq_last_error_message(void);
/* Library version as major*10000 + minor*100 + patch. */
int32_t nq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NQ_H_ */
