// C ABI of the Ledoit-Wolf diagonal preconditioners (declared in
// include/nq.h; kernels in lwprec.hip). A handle holds the running second
// moment S (fp64, padded p x p), the sum of ||z||^4 and the token count for
// one feature dimension; samples are added in chunks of at most max_rows
// rows, each staged transposed so that the Gram kernel reduces over tokens.
#include <algorithm>
#include <cstring>
#include <string>

#include "abi.h"
#include "common.h"

using namespace nq;

namespace nq {
hipError_t launch_lw_stage(const float* Z, int64_t rows, int64_t p, int64_t ldz, float* Zt,
                           int64_t pp, int64_t kp, hipStream_t s);
hipError_t launch_lw_q4(const float* Z, int64_t rows, int64_t p, int64_t ldz, double* rn,
                        double* q4, hipStream_t s);
hipError_t launch_lw_accum(const float* G, double* S, int64_t n, hipStream_t s);
int lw_norm_blocks(int64_t pp);
hipError_t launch_lw_finalize(const double* S, int64_t pp, int64_t p, double N, const double* q4,
                              double* part, double* scalars, float* d, hipStream_t s);
}  // namespace nq

struct nq_lw {
  int64_t p = 0, pp = 0, kmax = 0;
  int slots = 0;
  char* base = nullptr;
  float *Zt = nullptr, *part = nullptr, *G = nullptr;
  double *S = nullptr, *rn = nullptr, *q4 = nullptr, *npart = nullptr, *scalars = nullptr;
  double N = 0.0;          // tokens added since the last reset
  bool zero_pending = true;  // S and q4 are cleared before the next chunk
};

namespace {

constexpr int64_t kMaxP = 16384;
constexpr int64_t kMaxRows = 1 << 20;
constexpr int64_t kMaxStage = int64_t(1) << 30;  // floats of the staged chunk (4 GiB)

size_t take(size_t& off, size_t bytes) {
  const size_t o = off;
  off += (bytes + 255) / 256 * 256;
  return o;
}

nq_status gfx950_device() {
  int count = 0, dev = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1)
    return set_error(NQ_ERR_UNSUPPORTED, "no HIP device available");
  NQ_HIPCHK(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  NQ_HIPCHK(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_error(NQ_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName +
                                             ", need gfx950");
  return NQ_OK;
}

}  // namespace

extern "C" {

nq_status nq_lw_create(int64_t p, int64_t max_rows, nq_lw_t* out) {
  if (!out) return set_error(NQ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (p < 1 || p > kMaxP) return set_error(NQ_ERR_INVALID_ARG, "p must be in [1, 16384]");
  if (max_rows < 1 || max_rows > kMaxRows)
    return set_error(NQ_ERR_INVALID_ARG, "max_rows must be in [1, 2^20]");
  const int64_t pp = round_up(p, kPadR), kmax = round_up(max_rows, 32);
  if (pp * kmax > kMaxStage)
    return set_error(NQ_ERR_INVALID_ARG, "p * max_rows must be <= 2^30 (the staged chunk)");
  nq_status st = gfx950_device();
  if (st != NQ_OK) return st;
  nq_lw* h = new nq_lw();
  h->p = p;
  h->pp = pp;
  h->kmax = kmax;
  for (int64_t k = 32; k <= kmax; k += 32) h->slots = std::max(h->slots, gram_plan((int)k, (int)pp).slots);
  size_t off = 0;
  const size_t o_zt = take(off, sizeof(float) * pp * kmax);
  const size_t o_part = take(off, sizeof(float) * h->slots * pp * pp);
  const size_t o_g = take(off, sizeof(float) * pp * pp);
  const size_t o_s = take(off, sizeof(double) * pp * pp);
  const size_t o_rn = take(off, sizeof(double) * kmax);
  const size_t o_q4 = take(off, sizeof(double));
  const size_t o_np = take(off, sizeof(double) * 2 * lw_norm_blocks(pp));
  const size_t o_sc = take(off, sizeof(double) * 8);
  hipError_t e = hipMalloc((void**)&h->base, off);
  if (e != hipSuccess) {
    delete h;
    return hip_error(e, "hipMalloc(Ledoit-Wolf workspace)");
  }
  char* b = h->base;
  h->Zt = (float*)(b + o_zt);
  h->part = (float*)(b + o_part);
  h->G = (float*)(b + o_g);
  h->S = (double*)(b + o_s);
  h->rn = (double*)(b + o_rn);
  h->q4 = (double*)(b + o_q4);
  h->npart = (double*)(b + o_np);
  h->scalars = (double*)(b + o_sc);
  *out = h;
  return NQ_OK;
}

nq_status nq_lw_accumulate(nq_lw_t h, const float* Z, int64_t rows, int64_t ldz, void* stream) {
  if (!h) return set_error(NQ_ERR_INVALID_ARG, "handle is NULL");
  if (rows < 0) return set_error(NQ_ERR_INVALID_ARG, "rows must be >= 0");
  if (rows == 0) return NQ_OK;
  if (!Z) return set_error(NQ_ERR_INVALID_ARG, "Z is NULL");
  if (ldz < h->p) return set_error(NQ_ERR_INVALID_ARG, "ldz < p");
  hipStream_t s = (hipStream_t)stream;
  const int64_t pp = h->pp;
  if (h->zero_pending) {
    NQ_HIPCHK(launch_zero((float*)h->S, (size_t)(2 * pp * pp), s));
    NQ_HIPCHK(launch_zero((float*)h->q4, 2, s));
    h->zero_pending = false;
  }
  for (int64_t r0 = 0; r0 < rows; r0 += h->kmax) {
    const int64_t nr = std::min(h->kmax, rows - r0);
    const int64_t kp = round_up(nr, 32);
    const float* Zc = Z + r0 * ldz;
    const GramPlan gp = gram_plan((int)kp, (int)pp);
    if (gp.slots > h->slots) return set_error(NQ_ERR_HIP, "Gram plan exceeds its workspace");
    NQ_HIPCHK(launch_lw_stage(Zc, nr, h->p, ldz, h->Zt, pp, kp, s));
    NQ_HIPCHK(launch_gram_partial(h->Zt, kp, (int)kp, (int)pp, gp, h->part, s));
    NQ_HIPCHK(launch_gram_reduce(h->part, (int)kp, (int)pp, gp, 0.0f, true, h->G, pp, s));
    NQ_HIPCHK(launch_lw_accum(h->G, h->S, pp * pp, s));
    NQ_HIPCHK(launch_lw_q4(Zc, nr, h->p, ldz, h->rn, h->q4, s));
    h->N += (double)nr;
  }
  return NQ_OK;
}

nq_status nq_lw_finalize(nq_lw_t h, float* d, double* shrinkage, void* stream) {
  if (!h) return set_error(NQ_ERR_INVALID_ARG, "handle is NULL");
  if (!d) return set_error(NQ_ERR_INVALID_ARG, "d is NULL");
  if (h->N <= 0.0 || h->zero_pending)
    return set_error(NQ_ERR_INVALID_ARG, "no samples were accumulated");
  hipStream_t s = (hipStream_t)stream;
  NQ_HIPCHK(launch_lw_finalize(h->S, h->pp, h->p, h->N, h->q4, h->npart, h->scalars, d, s));
  if (shrinkage) {
    NQ_HIPCHK(hipMemcpyAsync(shrinkage, h->scalars, sizeof(double), hipMemcpyDeviceToHost, s));
    NQ_HIPCHK(hipStreamSynchronize(s));
  }
  return NQ_OK;
}

nq_status nq_lw_reset(nq_lw_t h) {
  if (!h) return set_error(NQ_ERR_INVALID_ARG, "handle is NULL");
  h->N = 0.0;
  h->zero_pending = true;
  return NQ_OK;
}

nq_status nq_lw_destroy(nq_lw_t h) {
  if (!h) return NQ_OK;
  if (h->base) (void)hipFree(h->base);
  delete h;
  return NQ_OK;
}

}  // extern "C"
