// Host driver and C ABI of the LB-ADMM library (declared in include/nq.h).
//
// One handle = one layer shape. create() allocates every workspace buffer
// once (one device allocation, zero-padded layouts); run() only enqueues
// kernels and never allocates. Each factor is kept twice, as U (m x r) and
// U^T (r x m), so that every product reads its operands k-contiguous: the
// Gram and the right-hand side read the other factor's transpose, and the
// solve writes both. Per half-iteration (run_half):
//   caller's stream: the Gram, the Cholesky + inverse (a chain of
//                    latency-bound launches), then the solve;
//   GEMM stream:     the right-hand-side GEMM, then the SVID + dual update of
//                    the factor solved by the previous half, which this half
//                    does not read.
// Events order the shared buffers: the GEMM stream starts after the Gram,
// and the solve waits for the right-hand side. The critical path (Gram,
// chain, solve) stays on one stream, with no event between its kernels.
#include "nq.h"
#include "abi.h"
#include "common.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace nq;

namespace {

thread_local std::string g_err;

nq_status fail(nq_status s, const std::string& msg) { return set_error(s, msg); }
nq_status hip_fail(hipError_t e, const char* what) { return hip_error(e, what); }

#define HIPCHK(expr) NQ_HIPCHK(expr)

constexpr uint32_t kKnownFlags = NQ_FLAG_COMPUTE_ERROR | NQ_FLAG_INIT_DRAWS |
                                  NQ_FLAG_NO_BALANCE | NQ_FLAG_SINGLE_STREAM | NQ_FLAG_PROFILE |
                                  NQ_FLAG_PROFILE_RHS_ONLY | NQ_FLAG_SOLVE_CG | NQ_FLAG_SOLVE_GD;
constexpr int kProfileRuns = 8;
constexpr int64_t kMaxMN = (1 << 21) - 256;
constexpr int64_t kMaxR = 1 << 13;
// s_sleep units per K step of the RHS GEMM beside the chain (measured best):
// 8 where chain update tiles share its CUs and the chain is about as long as
// the GEMM; 0 where the GEMM is clearly the longer side (it has nothing to
// give) or the chain keeps to two XCDs of its own.
constexpr int kRhsYield = 8;

// Whether the chain is about as long as the RHS GEMM beside it: r_p / 64
// launches of ~20 us against 2 m n r_p flops at ~105 TFLOP/s (the GEMM on 7
// XCDs). Measured: 4096 x 4096, r 2048 (chain ~640 us, GEMM ~650 us): yield
// 8 best (415 against 400 it/s at 0); 11008 x 4096, r 1536 (~480 against
// ~1320 us): yield 0 best (265.8 against 256.9 it/s).
bool chain_balances_rhs(int64_t mp, int64_t np_, int64_t rp) {
  const double chain_us = (double)(rp / 64) * 20.0;
  const double rhs_us = 2.0 * (double)mp * (double)np_ * (double)rp / 105e6;
  return chain_us >= 0.67 * rhs_us;
}

nq_status check_desc(const nq_lbadmm_desc* d) {
  if (!d) return fail(NQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->m < 1 || d->n < 1 || d->r < 1) return fail(NQ_ERR_INVALID_ARG, "m, n, r must be >= 1");
  // the tiled products address 256 rows of an operand with 32-bit byte
  // offsets (padded m and n below 2^21); an SVID workgroup reduces at most
  // 32 columns over 256 slabs
  if (d->m > kMaxMN || d->n > kMaxMN)
    return fail(NQ_ERR_INVALID_ARG, "m and n must be <= 2^21 - 256");
  if (d->r > kMaxR) return fail(NQ_ERR_INVALID_ARG, "r must be <= 2^13");
  if (!(d->rho > 0.0f) || !std::isfinite(d->rho))
    return fail(NQ_ERR_INVALID_ARG, "rho must be finite and > 0");
  if (d->iters < 0) return fail(NQ_ERR_INVALID_ARG, "iters must be >= 0");
  if (d->svid_steps < 1 || d->svid_steps > 10000)
    return fail(NQ_ERR_INVALID_ARG, "svid_steps must be in [1, 10000]");
  if (d->flags & ~kKnownFlags) return fail(NQ_ERR_INVALID_ARG, "unknown flag bits");
  const uint32_t solver = d->flags & (NQ_FLAG_SOLVE_CG | NQ_FLAG_SOLVE_GD);
  if (solver == (NQ_FLAG_SOLVE_CG | NQ_FLAG_SOLVE_GD))
    return fail(NQ_ERR_INVALID_ARG, "NQ_FLAG_SOLVE_CG and NQ_FLAG_SOLVE_GD are exclusive");
  if (solver && (d->solve_steps < 1 || d->solve_steps > 10000))
    return fail(NQ_ERR_INVALID_ARG, "solve_steps must be in [1, 10000] with an iterative solve");
  if (!solver && d->solve_steps != 0)
    return fail(NQ_ERR_INVALID_ARG, "solve_steps must be 0 without an iterative solve");
  return NQ_OK;
}

nq_status check_device(int* dev) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count < 1) {
    g_err = "no HIP device available";
    return NQ_ERR_UNSUPPORTED;
  }
  HIPCHK(hipGetDevice(dev));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, *dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(NQ_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", need gfx950");
  return NQ_OK;
}

struct Arena {
  size_t off = 0;
  template <class T>
  size_t take(size_t count) {
    const size_t o = off;
    off += round_up((int64_t)(count * sizeof(T)), 256);
    return o;
  }
};


// The side stream of a device (the RHS GEMM and the SVIDs of every handle on
// it), created with the first handle and kept until the process ends.
// HIP maps streams onto a few hardware queues (four by default), sharing
// queues round-robin once they run out; a side stream per handle made the
// seventh handle's land on its caller's queue, where it runs after the
// chain rather than beside it (that layer took 1.5x as long). Handles used
// at the same time from different caller streams share it too: their RHS
// GEMMs and SVIDs then run in the order they were enqueued.
hipError_t side_stream(int dev, hipStream_t* out) {
  static std::mutex mu;
  static std::vector<hipStream_t> streams;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0) return hipErrorInvalidDevice;
  if ((size_t)dev >= streams.size()) streams.resize(dev + 1, nullptr);
  if (!streams[dev]) {
    hipStream_t st = nullptr;
    const hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    streams[dev] = st;
  }
  *out = streams[dev];
  return hipSuccess;
}

}  // namespace

namespace nq {
nq_status set_error(nq_status s, const std::string& msg) {
  g_err = msg;
  return s;
}
nq_status hip_error(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? NQ_ERR_OUT_OF_MEMORY : NQ_ERR_HIP;
}
}  // namespace nq

struct nq_lbadmm {
  nq_lbadmm_desc d{};
  int device = 0;
  int mp = 0, np_ = 0, rp = 0;
  GramPlan gU{}, gV{};  // Gram work splits of the U-half (K = n) and V-half (K = m)
  GramPlan gI{};        // G^-1 = M^T M from M^T (triangular, K = rp)
  GramPlan gIp{};       // the same on the chain's two XCDs (pin == 2, overlap)
  char* base = nullptr;
  size_t bytes = 0;
  float *Wt, *WtT, *U, *V, *UT, *VT, *LamU, *PU, *LamV, *PV, *R, *G, *Minv, *Ginv, *gpart;
  // M^T, written by the chain (its lower blocks stay zero from creation on),
  // the operand of G^-1 = M^T M
  float* Mt;
  SvidWork svU, svV;
  double *part_wt, *part_w, *err_parts;
  float *colpartU, *colpartV, *cbal, *s1w, *s2w, *s1c, *s2c;
  int8_t *SU, *SV;
  DevStats* st;
  float* rhs_part;  // partial tiles of the split RHS and solve GEMM launches
  // iterative solve (NQ_FLAG_SOLVE_CG / _GD): gradient, direction and its
  // product with G (max(mp, np) x rp each) and the per-row g.g
  float *itG = nullptr, *itD = nullptr, *itQ = nullptr, *itDelta = nullptr;
  // gemm_s: the RHS GEMM and the SVIDs, beside the caller's stream (see
  // run_half); the device's side stream, shared by its handles
  hipStream_t gemm_s = nullptr;
  hipEvent_t ev_fork = nullptr, ev_gram = nullptr, ev_rhs = nullptr, ev_t0 = nullptr,
            ev_t1 = nullptr;
  hipStream_t last_stream = nullptr;
  bool has_run = false;
  bool stats_valid = false;  // the stats block describes the last run (not a time_svid call)
  // s_sleep units (~64 cycles each) per K step of the RHS GEMM while it runs
  // beside the chain: where chain waves share its CUs, a wave sharing a SIMD
  // with an MFMA-bound wave gets little issue time, so the RHS gives way
  // (kRhsYield) when it has slack (chain_balances_rhs); with two diagonal
  // XCDs nothing of the chain shares its CUs. NQ_RHS_YIELD overrides it.
  int rhs_yield = kRhsYield;
  // Pinned overlap: the chain's diagonal work on the last `pin` XCDs (one
  // workgroup per CU), the RHS GEMM on the others. Needs 8 x 32 CUs and at
  // most 32 diagonal workgroups per launch and XCD: pin = 1 for r_p <= 2048,
  // 2 for r_p <= 4096, 0 (unpinned) above. NQ_PIN=0 turns it off; NQ_PIN=2
  // asks for two XCDs where one would do.
  int pin = 0;
  int svid_g = 256;  // workgroups of an SVID launch (svid_grid())
  // NQ_FLAG_PROFILE: ring of (start, end) event pairs and per-phase totals
  std::vector<hipEvent_t> prof_ev;
  std::vector<int> prof_phase;  // phase of each pending pair
  size_t prof_next = 0;         // next free pair
  double prof_ms[NQ_NUM_PHASES] = {0};
  int64_t prof_cnt[NQ_NUM_PHASES] = {0};
};

namespace {

bool iterative(const nq_lbadmm* h) {
  return (h->d.flags & (NQ_FLAG_SOLVE_CG | NQ_FLAG_SOLVE_GD)) != 0;
}

// Lay out (or just size, when h->base is null) every workspace buffer.
size_t layout(nq_lbadmm* h) {
  const int64_t mp = h->mp, np_ = h->np_, rp = h->rp;
  const int64_t mx = std::max(mp, np_);
  const int gch = std::max(std::max(h->gU.slots, h->gV.slots), h->gI.slots);
  Arena a;
  size_t o_Wt = a.take<float>(mp * np_), o_WtT = a.take<float>(np_ * mp);
  size_t o_U = a.take<float>(mp * rp), o_V = a.take<float>(np_ * rp);
  size_t o_UT = a.take<float>(rp * mp), o_VT = a.take<float>(rp * np_);
  size_t o_LamU = a.take<float>(mp * rp), o_PU = a.take<float>(mp * rp);
  size_t o_LamV = a.take<float>(np_ * rp), o_PV = a.take<float>(np_ * rp);
  size_t o_R = a.take<float>(mx * rp);
  size_t o_G = a.take<float>(rp * rp), o_M = a.take<float>(rp * rp), o_Gi = a.take<float>(rp * rp);
  size_t o_Mt = a.take<float>(rp * rp);
  size_t o_gp = a.take<float>((size_t)gch * rp * rp);
  const int nchU = svid_nchunks((int)mp), nchV = svid_nchunks((int)np_);
  // SVID exchange words, sized for the largest grid (256 workgroups)
  const size_t syw = svid_sync_words((int)rp, 256);
  size_t o_sUa = a.take<float>(mp), o_sUb = a.take<float>(rp), o_sUs = a.take<uint64_t>(syw);
  size_t o_sVa = a.take<float>(np_), o_sVb = a.take<float>(rp), o_sVs = a.take<uint64_t>(syw);
  const int npre = precondition_nblocks((int)mp, (int)np_);
  size_t o_pwt = a.take<double>(npre), o_pw = a.take<double>(npre);
  size_t o_err = a.take<double>(2 * (size_t)error_nparts((int)mp, (int)np_));
  size_t o_cpU = a.take<float>((size_t)nchU * rp), o_cpV = a.take<float>((size_t)nchV * rp);
  size_t o_cb = a.take<float>(rp), o_s1w = a.take<float>(mp), o_s2w = a.take<float>(np_);
  size_t o_s1c = a.take<float>(mp), o_s2c = a.take<float>(np_);
  size_t o_SU = a.take<int8_t>(mp * rp), o_SV = a.take<int8_t>(np_ * rp);
  size_t o_st = a.take<DevStats>(1);
  // partial tiles of the split GEMM launches: the RHS GEMMs on the whole
  // chip or beside a pinned chain, and the solves (never at the same time)
  size_t part_floats = 0;
  for (int f = 0; f <= kPinMaxXcds; ++f)
    part_floats = std::max({part_floats, gemm_part_floats((int)mp, (int)rp, (int)np_, f),
                            gemm_part_floats((int)np_, (int)rp, (int)mp, f),
                            gemm_part_floats((int)mp, (int)rp, (int)rp, f),
                            gemm_part_floats((int)np_, (int)rp, (int)rp, f)});
  size_t o_rp = a.take<float>(part_floats);
  const bool it = iterative(h);
  size_t o_itG = it ? a.take<float>(mx * rp) : 0, o_itD = it ? a.take<float>(mx * rp) : 0;
  size_t o_itQ = it ? a.take<float>(mx * rp) : 0, o_itX = it ? a.take<float>(mx) : 0;
  if (h->base) {
    char* b = h->base;
    h->Wt = (float*)(b + o_Wt); h->WtT = (float*)(b + o_WtT);
    h->U = (float*)(b + o_U); h->V = (float*)(b + o_V);
    h->UT = (float*)(b + o_UT); h->VT = (float*)(b + o_VT);
    h->LamU = (float*)(b + o_LamU); h->PU = (float*)(b + o_PU);
    h->LamV = (float*)(b + o_LamV); h->PV = (float*)(b + o_PV);
    h->R = (float*)(b + o_R);
    h->G = (float*)(b + o_G); h->Minv = (float*)(b + o_M); h->Ginv = (float*)(b + o_Gi);
    h->Mt = (float*)(b + o_Mt);
    h->gpart = (float*)(b + o_gp);
    h->st = (DevStats*)(b + o_st);
    const int G = h->svid_g;
    h->svU = SvidWork{(float*)(b + o_sUa), (float*)(b + o_sUb),
                      svid_sync_at((uint64_t*)(b + o_sUs), (int)rp, G), h->st, G};
    h->svV = SvidWork{(float*)(b + o_sVa), (float*)(b + o_sVb),
                      svid_sync_at((uint64_t*)(b + o_sVs), (int)rp, G), h->st, G};
    h->part_wt = (double*)(b + o_pwt); h->part_w = (double*)(b + o_pw);
    h->err_parts = (double*)(b + o_err);
    h->colpartU = (float*)(b + o_cpU); h->colpartV = (float*)(b + o_cpV);
    h->cbal = (float*)(b + o_cb); h->s1w = (float*)(b + o_s1w); h->s2w = (float*)(b + o_s2w);
    h->s1c = (float*)(b + o_s1c); h->s2c = (float*)(b + o_s2c);
    h->SU = (int8_t*)(b + o_SU); h->SV = (int8_t*)(b + o_SV);
    h->rhs_part = (float*)(b + o_rp);
    if (it) {
      h->itG = (float*)(b + o_itG); h->itD = (float*)(b + o_itD);
      h->itQ = (float*)(b + o_itQ); h->itDelta = (float*)(b + o_itX);
    }
  }
  return a.off;
}

void plan(nq_lbadmm* h) {
  h->mp = (int)round_up(h->d.m, kPadMN);
  h->np_ = (int)round_up(h->d.n, kPadMN);
  h->rp = (int)round_up(h->d.r, kPadR);
  h->gU = gram_plan(h->np_, h->rp);  // U-half: Gram of V, K = n
  h->gV = gram_plan(h->mp, h->rp);   // V-half: Gram of U, K = m
  h->gI = gram_plan(h->rp, h->rp, true);
}

size_t pairs_per_run(const nq_lbadmm* h) { return 4 + (size_t)h->d.iters * 8; }

// Fold every pending pair into the totals (waits for the last one).
nq_status prof_harvest(nq_lbadmm* h) {
  if (h->prof_next == 0) return NQ_OK;
  for (size_t p = 0; p < h->prof_next; ++p) HIPCHK(hipEventSynchronize(h->prof_ev[2 * p + 1]));
  for (size_t p = 0; p < h->prof_next; ++p) {
    float ms = 0.0f;
    HIPCHK(hipEventElapsedTime(&ms, h->prof_ev[2 * p], h->prof_ev[2 * p + 1]));
    h->prof_ms[h->prof_phase[p]] += ms;
    h->prof_cnt[h->prof_phase[p]] += 1;
  }
  h->prof_next = 0;
  return NQ_OK;
}

// Start / end of a timed interval: returns the pair index (or -1 when off).
long prof_begin(nq_lbadmm* h, int phase, hipStream_t s) {
  if (!(h->d.flags & NQ_FLAG_PROFILE)) return -1;
  if ((h->d.flags & NQ_FLAG_PROFILE_RHS_ONLY) && phase != NQ_PHASE_GEMM_RHS) return -1;
  const size_t p = h->prof_next++;
  h->prof_phase[p] = phase;
  if (hipEventRecord(h->prof_ev[2 * p], s) != hipSuccess) return -1;
  return (long)p;
}
void prof_end(nq_lbadmm* h, long p, hipStream_t s) {
  if (p >= 0) (void)hipEventRecord(h->prof_ev[2 * p + 1], s);
}

struct Half {
  const float* Wside;  // M x K (padded, ld K)
  int M, K;            // rows of the factor being solved, rows of the other factor
  const float* otherT; // the other factor transposed, rp x K (ld K)
  float* out;          // M x rp
  float* outT;         // rp x M (ld M): out transposed
  float* Lam;          // M x rp
  float* P;            // M x rp
  const SvidWork* sv;
  GramPlan gp;
  int factor;  // 0 = U, 1 = V
};

// Z = SVID(X); Lam = X - Z; P = Z - Lam for the factor of half x.
nq_status run_svid(nq_lbadmm* h, const Half& x, hipStream_t vs) {
  long pv = prof_begin(h, NQ_PHASE_SVID, vs);
  // X = out + Lam is formed by the SVID's first step (into the Lam buffer)
  HIPCHK(launch_svid(x.Lam, x.P, x.M, h->rp, (int)h->d.r, h->d.svid_steps, 1, *x.sv, vs, x.out));
  prof_end(h, pv, vs);
  return NQ_OK;
}

// One ADMM half for the factor of x. With overlap:
//   s (the caller's stream): the critical path, in stream order: the Gram
//        G = other^T other + rho I (alone on the chip), the blocked Cholesky
//        with M = L^-1 and G^-1 = M^T M (a chain of latency-bound launches),
//        then, once R is there, the solve out = R G^-1 (and out^T);
//   gemm_s: after the Gram, R = Wside other + rho (Z - Lam), beside the
//        chain, then the SVID of the previous half (`pending`), which has
//        until the next half of its own factor (later on this stream) to
//        finish.
// Without overlap every kernel goes to s in the same order.
// The iterative form of a half (NQ_FLAG_SOLVE_CG / _GD): the Gram reduced to
// G = other^T other + rho I on s, the RHS GEMM on gemm_s beside it (on the
// whole chip: there is no chain), then on s, from the factor's current value
// u: g = u G - R (the GEMM with the RHS epilogue, rho = -1), d = -g, and
// per step the GEMM d G and the row-local step; finally out^T.
nq_status run_half_iterative(nq_lbadmm* h, const Half& x, const Half* pending, hipStream_t s,
                             bool overlap) {
  const int rp = h->rp;
  hipStream_t gs = overlap ? h->gemm_s : s;
  long pc = prof_begin(h, NQ_PHASE_CHAIN, s);
  HIPCHK(launch_gram_partial(x.otherT, x.K, x.K, rp, x.gp, h->gpart, s,
                             overlap ? h->ev_gram : nullptr));
  if (overlap) HIPCHK(hipStreamWaitEvent(h->gemm_s, h->ev_gram, 0));
  GemmArgs g{};
  g.A = x.Wside; g.lda = x.K; g.B = x.otherT; g.ldb = x.K; g.C = h->R; g.ldc = rp;
  g.P = x.P; g.rho = h->d.rho; g.M = x.M; g.N = rp; g.K = x.K;
  long pr = prof_begin(h, NQ_PHASE_GEMM_RHS, gs);
  HIPCHK(launch_gemm(g, kEpiRhs, gs));
  prof_end(h, pr, gs);
  if (overlap) HIPCHK(hipEventRecord(h->ev_rhs, gs));
  HIPCHK(launch_gram_reduce(h->gpart, x.K, rp, x.gp, h->d.rho, true, h->G, rp, s));
  prof_end(h, pc, s);
  if (overlap) HIPCHK(hipStreamWaitEvent(s, h->ev_rhs, 0));
  const bool cg = (h->d.flags & NQ_FLAG_SOLVE_CG) != 0;
  const int steps = h->d.solve_steps;
  long ps = prof_begin(h, NQ_PHASE_GEMM_SOLVE, s);
  // g = out G - R (G symmetric: its own transposed operand)
  GemmArgs r{};
  r.A = x.out; r.lda = rp; r.B = h->G; r.ldb = rp; r.C = h->itG; r.ldc = rp;
  r.P = h->R; r.rho = -1.0f; r.M = x.M; r.N = rp; r.K = rp;
  HIPCHK(launch_gemm(r, kEpiRhs, s));
  HIPCHK(launch_itsolve_init(h->itG, h->itD, h->itDelta, x.M, rp, s));
  GemmArgs q{};
  q.A = h->itD; q.lda = rp; q.B = h->G; q.ldb = rp; q.C = h->itQ; q.ldc = rp;
  q.M = x.M; q.N = rp; q.K = rp;
  for (int k = 0; k < steps; ++k) {
    HIPCHK(launch_gemm(q, kEpiPlain, s));
    HIPCHK(launch_itsolve_step(h->itQ, h->itD, x.out, h->itG, h->itDelta, x.M, rp, cg,
                               k == steps - 1, s));
  }
  HIPCHK(launch_transpose(x.out, x.M, rp, rp, x.outT, x.M, s));
  prof_end(h, ps, s);
  if (pending) {
    nq_status st = run_svid(h, *pending, overlap ? gs : s);
    if (st != NQ_OK) return st;
  }
  return NQ_OK;
}

nq_status run_half(nq_lbadmm* h, const Half& x, const Half* pending, hipStream_t s,
                   bool overlap) {
  if (iterative(h)) return run_half_iterative(h, x, pending, s, overlap);
  const int rp = h->rp;
  hipStream_t gs = overlap ? h->gemm_s : s;
  long pc = prof_begin(h, NQ_PHASE_CHAIN, s);
  // G = other^T other + rho I from other^T (rp x K)
  // ev_gram is recorded by the Gram kernel's own completion (an event record
  // of its own would put a marker, ~8 us, on s): the RHS GEMM, which does not
  // read G, starts beside the short reduction
  HIPCHK(launch_gram_partial(x.otherT, x.K, x.K, rp, x.gp, h->gpart, s,
                             overlap ? h->ev_gram : nullptr));
  if (overlap) HIPCHK(hipStreamWaitEvent(h->gemm_s, h->ev_gram, 0));
  // R = Wside other + rho (Z - Lam); Z - Lam comes from this factor's last
  // SVID, earlier on the same stream. Enqueued before the chain's launches:
  // when the host only just keeps pace with the GPU, host order is start
  // order, and the GEMM should not wait behind ~34 chain launches.
  GemmArgs g{};
  g.A = x.Wside; g.lda = x.K; g.B = x.otherT; g.ldb = x.K; g.C = h->R; g.ldc = rp;
  g.P = x.P; g.rho = h->d.rho; g.M = x.M; g.N = rp; g.K = x.K;
  g.yield = overlap ? h->rhs_yield : 0;
  g.free_xcds = overlap ? h->pin : 0;
  g.part = h->rhs_part;
  long pr = prof_begin(h, NQ_PHASE_GEMM_RHS, gs);
  HIPCHK(launch_gemm(g, kEpiRhs, gs));
  prof_end(h, pr, gs);
  if (overlap) HIPCHK(hipEventRecord(h->ev_rhs, gs));
  // M = L^-1 (and M^T); G^-1 = M^T M as a triangular Gram product of M^T
  // after the chain rather than inside it, where its 38 % of the chain's
  // update tiles would run beside the RHS GEMM. The chain's first launch
  // reduces the Gram segments into G itself (its update workgroups are
  // otherwise idle): G has no reduction launch of its own.
  HIPCHK(launch_cholesky_inverse(h->G, h->Minv, rp, (int)h->d.r, h->st, false, false,
                                 s, overlap ? h->pin : 0, h->Mt,
                                 GramSrc{h->gpart, GramSteps{x.K / 32, 0}, x.gp.steps, h->d.rho}));
  // With the chain on two XCDs of its own, G^-1's Gram stays there too: the
  // RHS GEMM on the other six is still running and is the longer side.
  const GramPlan& gi = overlap && h->pin == 2 ? h->gIp : h->gI;
  HIPCHK(launch_gram_partial(h->Mt, rp, rp, rp, gi, h->gpart, s));
  HIPCHK(launch_gram_reduce(h->gpart, rp, rp, gi, 0.0f, true, h->Ginv, rp, s));
  prof_end(h, pc, s);
  if (overlap) HIPCHK(hipStreamWaitEvent(s, h->ev_rhs, 0));
  // out = R G^-1 (G^-1 symmetric, so it is its own transposed operand),
  // outT = out^T
  GemmArgs q{};
  q.A = h->R; q.lda = rp; q.B = h->Ginv; q.ldb = rp; q.C = x.out; q.ldc = rp;
  q.Ct = x.outT; q.ldct = x.M; q.M = x.M; q.N = rp; q.K = rp;
  // leftover tiles split along K (the RHS GEMM and its fix-up, the only
  // other users of part, have ended: this stream waited for ev_rhs)
  q.part = h->rhs_part;
  long ps = prof_begin(h, NQ_PHASE_GEMM_SOLVE, s);
  HIPCHK(launch_gemm(q, kEpiSolve, s));
  prof_end(h, ps, s);
  // The SVID of the previous half, on the GEMM stream after this half's RHS
  // GEMM (stream order), where it runs beside the chain. Enqueued last: when
  // the host only just keeps pace, the solve must not wait for its ~17
  // launches to be submitted.
  if (pending) {
    nq_status st = run_svid(h, *pending, overlap ? gs : s);
    if (st != NQ_OK) return st;
  }
  return NQ_OK;
}

std::string svid_timeout_text(const DevStats& hs) {
  return "an SVID launch's workgroups were not all resident within about 0.5 s (results invalid; "
         "first expired wait: workgroup " + std::to_string(hs.to_wg) + ", step " +
         std::to_string(hs.to_step) + (hs.to_phase ? ", b" : ", partials") + ", tag wanted " +
         std::to_string(hs.to_want) + ", read " + std::to_string(hs.to_seen) + ", epoch " +
         std::to_string(hs.to_epoch) + ", waited " +
         std::to_string((long long)(hs.to_now - hs.to_start)) + " ticks from start " +
         std::to_string((unsigned long long)hs.to_start) + "; awaited workgroup " +
         std::to_string(hs.to_src) + " at tag " + std::to_string(hs.to_src_prog >> 2) +
         " stage " + std::to_string(hs.to_src_prog & 3) + ")";
}

nq_status status_from(const DevStats& hs) {
  if (hs.bad_precond) return fail(NQ_ERR_BAD_PRECONDITIONER, "an entry of d_out or d_in is not > 0");
  if (hs.nonfinite) return fail(NQ_ERR_NONFINITE, "NaN or Inf in the input or the result");
  if (hs.sync_timeout)
    return fail(NQ_ERR_HIP, svid_timeout_text(hs));
  if (hs.potrf_info != 0x7fffffff)
    return fail(NQ_ERR_NOT_POSITIVE_DEFINITE,
                "Cholesky pivot <= 0 at column " + std::to_string(hs.potrf_info - 1));
  return NQ_OK;
}

}  // namespace

extern "C" {

const char* nq_status_string(nq_status s) {
  switch (s) {
    case NQ_OK: return "NQ_OK";
    case NQ_ERR_INVALID_ARG: return "NQ_ERR_INVALID_ARG";
    case NQ_ERR_UNSUPPORTED: return "NQ_ERR_UNSUPPORTED";
    case NQ_ERR_OUT_OF_MEMORY: return "NQ_ERR_OUT_OF_MEMORY";
    case NQ_ERR_HIP: return "NQ_ERR_HIP";
    case NQ_ERR_NOT_POSITIVE_DEFINITE: return "NQ_ERR_NOT_POSITIVE_DEFINITE";
    case NQ_ERR_NONFINITE: return "NQ_ERR_NONFINITE";
    case NQ_ERR_BAD_PRECONDITIONER: return "NQ_ERR_BAD_PRECONDITIONER";
  }
  return "NQ_ERR_UNKNOWN";
}

const char* nq_last_error_message(void) { return g_err.c_str(); }

int32_t nq_version(void) { return 100; }

nq_status nq_lbadmm_workspace_bytes(const nq_lbadmm_desc* desc, size_t* bytes) {
  nq_status st = check_desc(desc);
  if (st != NQ_OK) return st;
  if (!bytes) return fail(NQ_ERR_INVALID_ARG, "bytes is NULL");
  nq_lbadmm tmp;
  tmp.d = *desc;
  plan(&tmp);
  *bytes = layout(&tmp);
  return NQ_OK;
}


nq_status nq_lbadmm_create(const nq_lbadmm_desc* desc, nq_lbadmm_t* out) {
  if (!out) return fail(NQ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  nq_status st = check_desc(desc);
  if (st != NQ_OK) return st;
  int dev = 0;
  st = check_device(&dev);
  if (st != NQ_OK) return st;
  nq_lbadmm* h = new nq_lbadmm();
  h->d = *desc;
  h->device = dev;
  h->svid_g = svid_grid();
  plan(h);
  {
    SvidPlan sp;
    if (!svid_plan(h->mp, h->rp, h->svid_g, &sp) || !svid_plan(h->np_, h->rp, h->svid_g, &sp)) {
      delete h;
      return fail(NQ_ERR_UNSUPPORTED, "no SVID launch layout for this shape");
    }
  }
  h->bytes = layout(h);
  hipError_t e = hipMalloc((void**)&h->base, h->bytes);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "hipMalloc(workspace)");
  }
  layout(h);
  {
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        ncu == kPinGrid && !iterative(h))
      h->pin = cholesky_pin_xcds((int)h->rp, false);
    if (const char* y = std::getenv("NQ_PIN")) {
      const int want = std::atoi(y);
      h->pin = want <= 0 ? 0 : h->pin ? std::max(h->pin, std::min(want, kPinMaxXcds)) : 0;
    }
    bool rr = false;
    if (h->pin && !(xcd_round_robin_ok(&rr) == hipSuccess && rr)) h->pin = 0;
  }
  h->rhs_yield = h->pin != 2 && chain_balances_rhs(h->mp, h->np_, h->rp) ? kRhsYield : 0;
  // (fewer workgroups, so longer ranges and no more partial slots than the
  // workspace holds for gI)
  h->gIp = h->pin == 2 ? gram_plan((int)h->rp, (int)h->rp, true, 2) : h->gI;
  if (h->gIp.slots > h->gI.slots) h->gIp = h->gI;
  if (const char* y = std::getenv("NQ_RHS_YIELD")) h->rhs_yield = std::max(0, std::atoi(y));
  e = side_stream(dev, &h->gemm_s);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_gram, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_rhs, hipEventDisableTiming);

  if (e == hipSuccess) e = hipEventCreate(&h->ev_t0);
  if (e == hipSuccess) e = hipEventCreate(&h->ev_t1);
  if (e == hipSuccess && (h->d.flags & NQ_FLAG_PROFILE)) {
    const size_t pairs = pairs_per_run(h) * kProfileRuns;
    h->prof_ev.assign(2 * pairs, nullptr);
    h->prof_phase.assign(pairs, 0);
    for (size_t i = 0; i < 2 * pairs && e == hipSuccess; ++i) e = hipEventCreate(&h->prof_ev[i]);
  }
  // Padding must read as zero from the start (the run rewrites every live
  // region it reads, but the finish kernels read padded rows).
  if (e == hipSuccess) e = hipMemset(h->base, 0, h->bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    nq_status s = hip_fail(e, "create");
    nq_lbadmm_destroy(h);
    return s;
  }
  *out = h;
  return NQ_OK;
}

void nq_lbadmm_destroy(nq_lbadmm_t h) {
  if (!h) return;
  int cur = 0;
  if (hipGetDevice(&cur) == hipSuccess && cur != h->device) (void)hipSetDevice(h->device);
  if (h->last_stream || h->has_run) (void)hipStreamSynchronize(h->last_stream);
  if (h->gemm_s) (void)hipStreamSynchronize(h->gemm_s);
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_gram) (void)hipEventDestroy(h->ev_gram);
  if (h->ev_rhs) (void)hipEventDestroy(h->ev_rhs);

  if (h->ev_t0) (void)hipEventDestroy(h->ev_t0);
  if (h->ev_t1) (void)hipEventDestroy(h->ev_t1);
  for (hipEvent_t ev : h->prof_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (h->base) (void)hipFree(h->base);
  if (cur != h->device) (void)hipSetDevice(cur);
  delete h;
}

nq_status nq_lbadmm_run(nq_lbadmm_t h, const float* W, int64_t ldw, const float* d_out,
                        const float* d_in, const float* U0, const float* V0, float* U, float* V,
                        float* s1, float* s2, uint32_t* U_bits, uint32_t* V_bits,
                        nq_lbadmm_stats* stats, void* stream) {
  if (!h) return fail(NQ_ERR_INVALID_ARG, "handle is NULL");
  if (!W || !d_out || !d_in) return fail(NQ_ERR_INVALID_ARG, "W, d_out and d_in are required");
  if (ldw < h->d.n) return fail(NQ_ERR_INVALID_ARG, "ldw < n");
  if ((U0 == nullptr) != (V0 == nullptr))
    return fail(NQ_ERR_INVALID_ARG, "U0 and V0 must be both given or both NULL");
  if ((h->d.flags & NQ_FLAG_INIT_DRAWS) && !U0)
    return fail(NQ_ERR_INVALID_ARG, "NQ_FLAG_INIT_DRAWS needs U0 and V0");
  int cur = 0;
  HIPCHK(hipGetDevice(&cur));
  if (cur != h->device) return fail(NQ_ERR_INVALID_ARG, "handle belongs to another device");

  hipStream_t s = (hipStream_t)stream;
  const nq_lbadmm_desc& d = h->d;
  const int mp = h->mp, np_ = h->np_, rp = h->rp;
  const bool overlap = !(d.flags & NQ_FLAG_SINGLE_STREAM);

  if ((d.flags & NQ_FLAG_PROFILE) && h->prof_next + pairs_per_run(h) > h->prof_phase.size()) {
    nq_status ps = prof_harvest(h);
    if (ps != NQ_OK) return ps;
  }
  HIPCHK(hipEventRecord(h->ev_t0, s));
  long pp = prof_begin(h, NQ_PHASE_PREP, s);
  HIPCHK(launch_stats_init(h->st, s));
  HIPCHK(launch_check_precond(d_out, d.m, d_in, d.n, h->st, s));
  HIPCHK(launch_precondition(W, ldw, d.m, d.n, d_out, d_in, h->Wt, h->WtT, mp, np_, h->part_wt,
                             h->part_w, h->st, s));
  HIPCHK(launch_finalize_norms(h->part_wt, h->part_w, precondition_nblocks(mp, np_), d.m, d.n,
                               d.r, h->st, s));
  // init: U0 (the latent) into U, and X = U0 into the Lam buffer for SVID
  if (U0) {
    const bool scale = (d.flags & NQ_FLAG_INIT_DRAWS) != 0;
    HIPCHK(launch_init_copy(U0, d.m, d.r, d.r, h->U, h->LamU, mp, rp, scale, h->st, s));
    HIPCHK(launch_init_copy(V0, d.n, d.r, d.r, h->V, h->LamV, np_, rp, scale, h->st, s));
  } else {
    HIPCHK(launch_init_philox(d.seed, 0u, d.m, d.r, h->U, h->LamU, mp, rp, h->st, s));
    HIPCHK(launch_init_philox(d.seed, 1u, d.n, d.r, h->V, h->LamV, np_, rp, h->st, s));
  }
  HIPCHK(launch_transpose(h->U, mp, rp, rp, h->UT, mp, s));
  HIPCHK(launch_transpose(h->V, np_, rp, rp, h->VT, np_, s));
  HIPCHK(launch_svid(h->LamU, h->PU, mp, rp, (int)d.r, d.svid_steps, 0, h->svU, s));
  HIPCHK(launch_svid(h->LamV, h->PV, np_, rp, (int)d.r, d.svid_steps, 0, h->svV, s));
  prof_end(h, pp, s);

  Half hu{h->Wt, mp, np_, h->VT, h->U, h->UT, h->LamU, h->PU, &h->svU, h->gU, 0};
  Half hv{h->WtT, np_, mp, h->UT, h->V, h->VT, h->LamV, h->PV, &h->svV, h->gV, 1};
  const Half* pending = nullptr;
  for (int it = 0; it < d.iters; ++it) {
    nq_status st = run_half(h, hu, pending, s, overlap);
    if (st != NQ_OK) return st;
    st = run_half(h, hv, &hu, s, overlap);
    if (st != NQ_OK) return st;
    pending = &hv;
  }
  if (overlap) {
    // join: the SVID launched by the last half on the GEMM stream
    HIPCHK(hipEventRecord(h->ev_fork, h->gemm_s));
    HIPCHK(hipStreamWaitEvent(s, h->ev_fork, 0));
  }
  if (pending) {
    nq_status st = run_svid(h, *pending, s);
    if (st != NQ_OK) return st;
  }

  // finish: balance, scales, signs, bits, errors
  long pf = prof_begin(h, NQ_PHASE_FINISH, s);
  const int nchU = svid_nchunks(mp), nchV = svid_nchunks(np_);
  HIPCHK(launch_colsumsq(h->U, mp, rp, h->colpartU, s));
  HIPCHK(launch_colsumsq(h->V, np_, rp, h->colpartV, s));
  HIPCHK(launch_balance_coef(h->colpartU, nchU, h->colpartV, nchV, rp,
                             !(d.flags & NQ_FLAG_NO_BALANCE), h->cbal, s));
  HIPCHK(launch_apply_finish(h->U, d.m, mp, rp, d.r, h->cbal, false, d_out, U, h->s1c, h->s1w,
                             U_bits, h->SU, h->st, s));
  HIPCHK(launch_apply_finish(h->V, d.n, np_, rp, d.r, h->cbal, true, d_in, V, h->s2c, h->s2w,
                             V_bits, h->SV, h->st, s));
  if (s1) HIPCHK(hipMemcpyAsync(s1, h->s1c, sizeof(float) * d.m, hipMemcpyDeviceToDevice, s));
  if (s2) HIPCHK(hipMemcpyAsync(s2, h->s2c, sizeof(float) * d.n, hipMemcpyDeviceToDevice, s));
  if (d.flags & NQ_FLAG_COMPUTE_ERROR)
    HIPCHK(launch_error(h->SU, h->SV, mp, np_, rp, h->s1w, h->s2w, h->Wt, W, ldw, d.m, d.n,
                        h->s1c, h->s2c, h->err_parts, h->st, s));
  prof_end(h, pf, s);
  HIPCHK(hipEventRecord(h->ev_t1, s));
  h->last_stream = s;
  h->has_run = true;
  h->stats_valid = true;
  if (stats) return nq_lbadmm_query(h, stats);
  return NQ_OK;
}

nq_status nq_lbadmm_profile(nq_lbadmm_t h, double* ms, int64_t* count, int32_t reset) {
  if (!h || !ms || !count) return fail(NQ_ERR_INVALID_ARG, "handle, ms and count are required");
  if (!(h->d.flags & NQ_FLAG_PROFILE))
    return fail(NQ_ERR_INVALID_ARG, "handle was created without NQ_FLAG_PROFILE");
  nq_status st = prof_harvest(h);
  if (st != NQ_OK) return st;
  for (int p = 0; p < NQ_NUM_PHASES; ++p) {
    ms[p] = h->prof_ms[p];
    count[p] = h->prof_cnt[p];
    if (reset) {
      h->prof_ms[p] = 0.0;
      h->prof_cnt[p] = 0;
    }
  }
  return NQ_OK;
}

nq_status nq_lbadmm_query(nq_lbadmm_t h, nq_lbadmm_stats* stats) {
  if (!h || !stats) return fail(NQ_ERR_INVALID_ARG, "handle and stats are required");
  if (!h->has_run) return fail(NQ_ERR_INVALID_ARG, "handle has not run");
  if (!h->stats_valid)
    return fail(NQ_ERR_INVALID_ARG, "nq_lbadmm_time_svid ran since the last run; run again");
  HIPCHK(hipEventSynchronize(h->ev_t1));
  DevStats hs;
  HIPCHK(hipMemcpy(&hs, h->st, sizeof(DevStats), hipMemcpyDeviceToHost));
  float ms = 0.0f;
  HIPCHK(hipEventElapsedTime(&ms, h->ev_t0, h->ev_t1));
  std::memset(stats, 0, sizeof(*stats));
  const bool err = (h->d.flags & NQ_FLAG_COMPUTE_ERROR) != 0;
  stats->rel_err_wtilde = err ? std::sqrt(hs.err2_wt / hs.sumsq_wt) : NAN;
  stats->rel_err_w = err ? std::sqrt(hs.err2_w / hs.sumsq_w) : NAN;
  stats->sumsq_wtilde = hs.sumsq_wt;
  stats->sigma0 = hs.sigma0;
  stats->potrf_info = hs.potrf_info == 0x7fffffff ? 0 : hs.potrf_info;
  stats->nonfinite = hs.nonfinite;
  stats->bad_precond = hs.bad_precond;
  stats->elapsed_ms = ms;
  stats->iters_done = h->d.iters;
  return status_from(hs);
}

}  // extern "C"

extern "C" nq_status nq_lbadmm_get_state(nq_lbadmm_t h, float* U, float* V, float* Z_U,
                                         float* Lam_U, float* Z_V, float* Lam_V, void* stream) {
  if (!h) return fail(NQ_ERR_INVALID_ARG, "handle is NULL");
  hipStream_t s = (hipStream_t)stream;
  const int64_t m = h->d.m, n = h->d.n, r = h->d.r, rp = h->rp;
  const size_t sp = sizeof(float) * rp, dp = sizeof(float) * r;
  if (U) HIPCHK(hipMemcpy2DAsync(U, dp, h->U, sp, dp, m, hipMemcpyDeviceToDevice, s));
  if (V) HIPCHK(hipMemcpy2DAsync(V, dp, h->V, sp, dp, n, hipMemcpyDeviceToDevice, s));
  if (Lam_U) HIPCHK(hipMemcpy2DAsync(Lam_U, dp, h->LamU, sp, dp, m, hipMemcpyDeviceToDevice, s));
  if (Lam_V) HIPCHK(hipMemcpy2DAsync(Lam_V, dp, h->LamV, sp, dp, n, hipMemcpyDeviceToDevice, s));
  if (Z_U) HIPCHK(launch_add_compact(h->PU, h->LamU, m, r, (int)rp, Z_U, s));
  if (Z_V) HIPCHK(launch_add_compact(h->PV, h->LamV, n, r, (int)rp, Z_V, s));
  return NQ_OK;
}

extern "C" nq_status nq_lbadmm_time_svid(nq_lbadmm_t h, int32_t factor, int32_t reps,
                                         void* stream, double* avg_ms) {
  if (!h || !avg_ms) return fail(NQ_ERR_INVALID_ARG, "handle and avg_ms are required");
  if (factor != 0 && factor != 1) return fail(NQ_ERR_INVALID_ARG, "factor must be 0 (U) or 1 (V)");
  if (reps < 1) return fail(NQ_ERR_INVALID_ARG, "reps must be >= 1");
  if (!h->has_run) return fail(NQ_ERR_INVALID_ARG, "handle has not run");
  hipStream_t s = (hipStream_t)stream;
  const bool u = factor == 0;
  const int rows = u ? h->mp : h->np_;
  float* lam = u ? h->LamU : h->LamV;
  float* P = u ? h->PU : h->PV;
  const float* lat = u ? h->U : h->V;
  const SvidWork& w = u ? h->svU : h->svV;
  HIPCHK(hipStreamWaitEvent(s, h->ev_t1, 0));  // after the last run
  HIPCHK(launch_stats_init(h->st, s));
  HIPCHK(hipEventRecord(h->ev_t0, s));
  for (int i = 0; i < reps; ++i)
    HIPCHK(launch_svid(lam, P, rows, h->rp, (int)h->d.r, h->d.svid_steps, 1, w, s, lat));
  HIPCHK(hipEventRecord(h->ev_t1, s));
  HIPCHK(hipEventSynchronize(h->ev_t1));
  float ms = 0.0f;
  HIPCHK(hipEventElapsedTime(&ms, h->ev_t0, h->ev_t1));
  DevStats hs;
  HIPCHK(hipMemcpy(&hs, h->st, sizeof(DevStats), hipMemcpyDeviceToHost));
  *avg_ms = (double)ms / reps;
  h->stats_valid = false;  // the stats block no longer describes a run
  if (hs.sync_timeout) return fail(NQ_ERR_HIP, svid_timeout_text(hs));
  return NQ_OK;
}
