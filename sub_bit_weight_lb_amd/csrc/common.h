// Internal declarations shared by the LB-ADMM kernels and the host driver.
// gfx950 only: wave64, fp32 MFMA (v_mfma_f32_32x32x2_f32), 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nq {

// Padded sizes: every workspace matrix is stored zero-padded to these
// multiples so that the tiled kernels need no bounds checks.
constexpr int kPadMN = 256;  // m and n (rows of Wt / Wt^T / U / V)
constexpr int kPadR = 128;   // r (rank)

inline int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

// XCD (accelerator complex die) the calling wave runs on, 0..7 on MI355X.
__device__ __forceinline__ int xcd_id() {
  return (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & 7u);  // HW_REG_XCC_ID
}

hipError_t xcd_round_robin_ok(bool* ok);

// Device-side status shared by all kernels of one run.
struct DevStats {
  double sumsq_wt;      // ||Wt||_F^2
  double sumsq_w;       // ||W||_F^2
  double sigma0;        // init scale
  double err2_wt;       // squared reconstruction error, Wt space
  double err2_w;        // squared reconstruction error, W space
  int nonfinite;        // NaN/Inf seen
  int bad_precond;      // some d <= 0
  int potrf_info;       // 0 or 1 + first failing pivot column (min over runs)
  int sync_timeout;     // an SVID launch's exchange wait ran out (workgroups not co-resident)
  // the first wait that ran out: workgroup, step, phase (0 partials, 1 b),
  // the tag expected and the tag read, the launch's epoch
  uint32_t to_wg, to_step, to_phase, to_want, to_seen, to_epoch;
  uint64_t to_start, to_now;  // the waiting workgroup's start and the expiry, 100 MHz ticks
  uint32_t to_src, to_src_prog;  // the workgroup it waited for, and its progress word then
};

// Launch layout of the pinned overlap (MI355X: 8 XCDs x 32 CUs): the chain's
// diagonal work takes the last px XCDs (px = 1 or 2), the RHS GEMM the
// others.
constexpr int kPinGrid = 256;     // workgroups of a pinned launch, 32 per XCD
constexpr int kPinXcdCus = 32;    // workgroups of a pinned launch on one XCD
constexpr int kPinMaxXcds = 2;    // at most two XCDs for the diagonal work

// ---------------------------------------------------------------- GEMM
enum GemmEpilogue : int {
  kEpiPlain = 0,   // C = A B^T
  kEpiRhs = 1,     // C = A B^T + rho P              (P ld = ldc)
  kEpiSolve = 2,   // C = A B^T; Ct = C^T when Ct is not null
};
// C = A B^T ("NT"): both operands are stored with k contiguous.
struct GemmArgs {
  const float* A; int64_t lda;   // M x K
  const float* B; int64_t ldb;   // N x K (the right factor, transposed)
  float* C; int64_t ldc;         // M x N
  const float* P;                // kEpiRhs
  float* Ct; int64_t ldct;       // kEpiSolve, optional: N x M
  float rho;
  int M, N, K;
  int yield;                     // s_sleep units per K step (0: none), to leave
                                 // issue cycles to a kernel running beside it
  int free_xcds;                 // kEpiRhs: 0, or 1-2 to run on XCDs 0 .. 7 - free_xcds
                                 // only (the others left to a pinned Cholesky
                                 // chain); part is then required
  float* part;                   // nullable: up to 256 x 256 x 128 floats of partial
                                 // tiles (gemm_part_floats)
};
// M % 256 == 0, N % 128 == 0, K % 32 == 0; every ld a multiple of 4 and every
// pointer 16-byte aligned (else hipErrorInvalidValue, nothing launched).
// With free_xcds = f, the 256 x 128 tiles go to the 32 (8 - f) workgroups of
// XCDs 0 .. 7 - f: each takes whole tiles, and the tiles left over are split
// along K into partial tiles (in part) that a second kernel adds up, with
// the epilogue, in a fixed order. With part and free_xcds = 0, a launch of
// more than 256 tiles that do not fill whole rounds of 256 runs the same way
// on all 8 XCDs; otherwise one workgroup per tile.
hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t s);
// Floats of `part` a launch of this shape with free_xcds = f needs (0 if none).
size_t gemm_part_floats(int M, int N, int K, int f);

// ---------------------------------------------------------------- Gram
// K steps (of 32) of the lower 128 x 128 tiles of a Gram product, tile
// t = I (I + 1) / 2 + J (I >= J) in that order: T steps each, or with tri
// (A upper triangular, K = rp: rows of A below row 128 I of tile row I's
// panel are zero) T - 4 I steps from step 4 I.
struct GramSteps {
  int T, tri;
  __host__ __device__ int len(int I) const { return tri ? T - 4 * I : T; }
  __host__ __device__ int first(int I) const { return tri ? 4 * I : 0; }
  // steps of the tile rows before row I
  __host__ __device__ int64_t row_start(int I) const {
    const int64_t i = I;
    return (int64_t)T * i * (i + 1) / 2 - (tri ? 4 * (i - 1) * i * (i + 1) / 3 : 0);
  }
  // steps before tile (I, J)
  __host__ __device__ int64_t tile_start(int I, int J) const {
    return row_start(I) + (int64_t)J * len(I);
  }
};
// A Gram product not yet reduced: the partial tiles `part` of a stream-K
// launch with steps gs and ranges of L steps, to be summed per tile in slot
// order, + rho on the diagonal (what launch_gram_reduce writes).
struct GramSrc {
  const float* part;
  GramSteps gs;
  int L;
  float rho;
};
// Work split of a Gram product (GramSteps over R = rp / 128 tile rows) into
// equal ranges of `steps` steps, one per workgroup (`wgs` of them); a tile's
// segments go to at most `slots` partial buffers of rp x rp.
// xcds = px > 0: the workgroups run on the last px XCDs only (two per CU),
// for a Gram that follows a chain pinned there while a GEMM holds the others.
struct GramPlan {
  int steps, wgs, slots, tri, xcds;
};
GramPlan gram_plan(int K, int rp, bool tri = false, int xcds = 0);
// Partial Gram tiles of A^T A for A (K x rp) given as At = A^T (rp x K, ld
// ldat) into part (p.slots buffers of rp x rp, ld rp; lower tiles only).
// rp % 128 == 0, K a multiple of 32; with p.tri, K == rp and A upper
// triangular (At lower triangular), whose zero K ranges are skipped.
hipError_t launch_gram_partial(const float* At, int64_t ldat, int K, int rp, const GramPlan& p,
                               float* part, hipStream_t s, hipEvent_t done = nullptr);
// G = the sum of each lower tile's segments, in slot order, + rho I (ld ldg):
// full-symmetric if `full`, else the lower triangle and the whole of each
// 64 x 64 diagonal block (what the blocked Cholesky reads). `done`
// (nullable) is recorded when the kernel completes.
hipError_t launch_gram_reduce(const float* part, int K, int rp, const GramPlan& p, float rho,
                              bool full, float* G, int64_t ldg, hipStream_t s,
                              hipEvent_t done = nullptr);

// ---------------------------------------------------------------- Cholesky / inverse
constexpr int kNB = 64;  // block size of the blocked Cholesky
// A (rp x rp, ld rp, full symmetric on entry) is used as workspace; with
// want_L its lower triangle becomes L and its upper triangle zero. The lower
// 64 x 64 tiles of M (rp x rp) become those of L^-1 (the diagonal tiles with
// zeros above their diagonal); M's other tiles are not written, and with
// zero_m M is zeroed first so that they read as zero.
// st->potrf_info gets min(1 + failing column).
// pin = px > 0: place the diagonal work on the last px XCDs (one workgroup
// per CU) and the update tiles on the others, for a run beside a GEMM with
// free_xcds = px; needs at most 32 px diagonal workgroups per launch.
// cholesky_pin_xcds gives the fewest XCDs that hold them (0: more than
// kPinMaxXcds would be needed).
int cholesky_pin_xcds(int rp, bool want_L);
// Mt (nullable): the upper block triangle of M^T (the lower blocks are never
// written and must read as zero), the operand of G^-1 = M^T M
// (launch_gram_partial with a triangular plan).
// src.part (nullable): A holds nothing yet; its tiles are the unreduced
// Gram product src, which the first launch reduces into A itself (the
// diagonal and panel workgroups sum their own tiles, the otherwise idle
// update workgroups the rest), in place of launch_gram_reduce (lower
// triangle and diagonal 64 x 64 blocks). Not with want_L.
hipError_t launch_cholesky_inverse(float* A, float* M, int rp, int r_real,
                                   DevStats* st, bool want_L, bool zero_m, hipStream_t s,
                                   int pin = 0, float* Mt = nullptr,
                                   GramSrc src = GramSrc{nullptr, GramSteps{0, 0}, 1, 0.0f});

// ---------------------------------------------------------------- SVID
// Exchange words of the persistent SVID launch (64-bit: value, tag), in a
// zero-initialised buffer of svid_sync_words(rp, G) words: part (rp / 4
// column quads x G slabs x 4), aa (G), b (rp), then two 32-bit control words
// (the epoch and the count of finished workgroups) and G progress words.
struct SvidSync {
  uint64_t* part;
  uint64_t* aa;
  uint64_t* b;
  uint32_t* ctl;
  uint32_t* prog;  // G words: per workgroup, (tag << 2) | stage of its progress
};
struct SvidWork {
  float* a;     // rows_pad: a of the last step
  float* b;     // rp: b of the last step
  SvidSync sy;
  DevStats* st; // sync_timeout is raised there
  int G;        // workgroups (svid_grid())
};
// Launch layout of one SVID update: G workgroups of TX threads (TY = 1), RS
// rows each; a thread holds NU float4 columns of RPT rows per chunk, NCH
// chunks per step (1: the slab stays in registers); a workgroup reduces NQO
// consecutive column quads (a power of two) over the slabs.
struct SvidPlan {
  int G, RS, TX, TY, NU, RPT, NCH, NQO, inst;
};
int svid_grid();  // workgroups of an SVID launch on the current device: 64, 128 or 256
size_t svid_sync_words(int rp, int G);
SvidSync svid_sync_at(uint64_t* base, int rp, int G);
bool svid_plan(int rows_pad, int rp, int G, SvidPlan* out);
int svid_nchunks(int rows_pad);  // 64-row chunks of the column-norm pass
// mode 0: init (P = Z, X zeroed: Lam = 0), mode 1: update (X <- X - Z,
// P = Z - X_new), mode 2: plain (Z written to P; X untouched). With Uadd
// (nullable, same layout as X), X is first replaced by X + Uadd. rp % 128 ==
// 0, T >= 1; one launch.
hipError_t launch_svid(float* X, float* P, int rows_pad, int rp, int r_real, int T,
                       int mode, const SvidWork& w, hipStream_t s,
                       const float* Uadd = nullptr);

// ---------------------------------------------------------------- elementwise
hipError_t launch_stats_init(DevStats* st, hipStream_t s);
hipError_t launch_check_precond(const float* d_out, int64_t m, const float* d_in, int64_t n,
                                DevStats* st, hipStream_t s);
// Wt (mp x np, ld np) and optionally WtT (np x mp, ld mp); partial sums of squares.
int precondition_nblocks(int mp, int np_);
hipError_t launch_precondition(const float* W, int64_t ldw, int64_t m, int64_t n,
                               const float* d_out, const float* d_in, float* Wt, float* WtT,
                               int mp, int np_, double* part_wt, double* part_w,
                               DevStats* st, hipStream_t s);
hipError_t launch_finalize_norms(const double* part_wt, const double* part_w, int nparts,
                                 int64_t m, int64_t n, int64_t r, DevStats* st, hipStream_t s);
// Dst (rows_pad x rp) = scale * Src (rows x r, ld lds) zero padded; scale = sigma0
// (from st) when use_sigma, else 1. Dst2 (nullable) gets the same values.
hipError_t launch_init_copy(const float* src, int64_t rows, int64_t r, int64_t lds,
                            float* dst, float* dst2, int rows_pad, int rp, bool use_sigma,
                            const DevStats* st, hipStream_t s);
// Philox4x32-10 standard normals scaled by sigma0 into dst/dst2 (rows x r real part).
hipError_t launch_init_philox(uint64_t seed, uint32_t stream_id, int64_t rows, int64_t r,
                              float* dst, float* dst2, int rows_pad, int rp,
                              const DevStats* st, hipStream_t s);
hipError_t launch_zero(float* p, size_t n, hipStream_t s);
// dst (cols x rows, ld ldd) = src^T, src rows x cols (ld lds); rows and cols
// multiples of 32.
hipError_t launch_transpose(const float* src, int64_t rows, int64_t cols, int64_t lds, float* dst,
                            int64_t ldd, hipStream_t s);
// out (rows x r, ld r) = A + B for padded A, B (ld rp).
hipError_t launch_add_compact(const float* A, const float* B, int64_t rows, int64_t r, int rp,
                              float* out, hipStream_t s);
// A[i][i] = val for from <= i < to (ld lda).
hipError_t launch_set_diag(float* A, int64_t lda, int from, int to, float val, hipStream_t s);

// ---------------------------------------------------------------- finish
// column sums of squares of F (rows_pad x rp) -> colpart (nchunks x rp)
hipError_t launch_colsumsq(const float* F, int rows_pad, int rp, float* colpart, hipStream_t s);
// c_k = sqrt(nv_k / nu_k) (1 if either is 0, or if !balance)
hipError_t launch_balance_coef(const float* partU, int nchU, const float* partV, int nchV,
                               int rp, bool balance, float* c, hipStream_t s);
// F' = F * c_k (or F / c_k when divide): writes out (rows x r, ld r, nullable),
// scale_out_i = mean_k |F'_ik| / d_i (nullable), scale_wt_i = mean_k |F'_ik|,
// bits (rows x ceil(r/32), nullable), sign8 (rows_pad x rp int8, zero padded).
hipError_t launch_apply_finish(const float* F, int64_t rows, int rows_pad, int rp, int64_t r,
                               const float* c, bool divide, const float* d,
                               float* out, float* scale_out, float* scale_wt,
                               uint32_t* bits, int8_t* sign8, DevStats* st, hipStream_t s);
// Squared errors into st->err2_wt / st->err2_w (deterministic).
int error_nparts(int mp, int np_);
// s1w/s2w: Wt-space scales (padded, zero beyond m/n); s1/s2: W-space scales (m, n).
// parts: 2 * error_nparts doubles.
hipError_t launch_error(const int8_t* SU, const int8_t* SV, int mp, int np_, int rp,
                        const float* s1w, const float* s2w, const float* Wt,
                        const float* W, int64_t ldw, int64_t m, int64_t n,
                        const float* s1, const float* s2, double* parts,
                        DevStats* st, hipStream_t s);

// ---------------------------------------------------------------- iterative solve (itsolve.hip)
// Rows x rp arrays (ld rp), rp % 4 == 0 and rp <= 8192. init: d = -g,
// delta = row sums of g^2. step (given Q = d G): alpha = delta / (d . Q)
// (0 unless d . Q > 0), u += alpha d, g += alpha Q, delta = g . g, and unless
// `last`, d = beta d - g with beta = delta_new / delta_old for conjugate
// gradients (cg), 0 for steepest descent.
hipError_t launch_itsolve_init(const float* g, float* d, float* delta, int rows, int rp,
                               hipStream_t s);
hipError_t launch_itsolve_step(const float* Q, float* d, float* u, float* g, float* delta,
                               int rows, int rp, bool cg, bool last, hipStream_t s);
// ---------------------------------------------------------------- sign products (signmm.hip)
// C (M x N, ld ldc) = A S^T for A (M x K, ld lda) and S (N x K, ld lds) whose
// entries are +-1 (stored as fp32), on the bf16 matrix cores with A split
// into three exact bf16 terms; Ct (N x M, ld ldct), if given, receives C^T.
// M, N % 128 == 0, K % 64 == 0, lds and ldct multiples of 4, A, S, Ct
// 16-byte aligned (else hipErrorInvalidValue, nothing launched).
hipError_t launch_sign_gemm(const float* A, int64_t lda, const float* S, int64_t lds, float* C,
                            int64_t ldc, float* Ct, int64_t ldct, int M, int N, int K,
                            hipStream_t s);
// ---------------------------------------------------------------- packing
hipError_t launch_pack_signs(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                             uint32_t* bits, int64_t ld_words, hipStream_t s);
// ---------------------------------------------------------------- binary layer (binmm.hip)
// out (cols x ld_out words) = the sign bits of in (rows x cols, ld_in words)
// transposed; tails of the last words zero.
hipError_t launch_transpose_bits(const uint32_t* in, int64_t rows, int64_t cols, int64_t ld_in,
                                 uint32_t* out, int64_t ld_out, hipStream_t s);
// Y (B x m, ld ldy) = s1 * ((X * s2) S_V S_U^T) from S_U bits (m x r, ld ldu
// words) and S_V^T bits (r x n, ld ldvt words); X B x n (ld ldx); work:
// binmm_work_floats(B, n, r) floats of scratch (kBinSplit B r partial
// projections, then the inputs' bf16 terms).
constexpr int kBinSplit = 8;
int64_t binmm_work_floats(int64_t B, int64_t n, int64_t r);
hipError_t launch_binary_matmul(const uint32_t* su, int64_t ldu, const uint32_t* svt,
                                int64_t ldvt, int64_t m, int64_t n, int64_t r, const float* s1,
                                const float* s2, const float* X, int64_t B, int64_t ldx,
                                float* Y, int64_t ldy, float* work, hipStream_t s);
// Floats in the fixed scratch array of binmm.hip (32 MiB per GPU): calls
// with binmm_work_floats(B, n, r) up to this fit.
constexpr int64_t kBinScratchFloats = int64_t(1) << 23;
// *out = this GPU's copy of that array (the current device's), its address
// looked up on first use on each device.
hipError_t binmm_fixed_scratch(float** out);

}  // namespace nq
