// C ABI of the STE refinement of a factorised layer (declared in
// include/nq.h; kernels in ste.hip). A handle holds the padded parameters
// U, V, s1, s2, their Adam moments, the sign matrices and every per-batch
// buffer for batches of up to max_tokens tokens, so a step allocates
// nothing.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>

#include "abi.h"
#include "common.h"

using namespace nq;

namespace nq {
hipError_t launch_ste_signs(const float* F, int64_t rows, int64_t r, int64_t rp, int64_t rows_pad,
                            float* S, float* St, hipStream_t s);
hipError_t launch_ste_stage(const float* X, int64_t ldx, const int32_t* idx, int64_t T, int64_t n,
                            const float* s2, int64_t np_, int64_t tp, float* A, float* At,
                            hipStream_t s);
hipError_t launch_ste_loss(const float* Q, const float* Y, int64_t ldy, const int32_t* idx,
                           int64_t T, int64_t m, const float* s1, int64_t mp, int64_t tp,
                           float* dQ, float* dQt, float* ds1p, double* lossp, float* ds1,
                           double* loss, hipStream_t s);
hipError_t launch_ste_ds2(const float* dA, const float* X, int64_t ldx, const int32_t* idx,
                          int64_t T, int64_t n, int64_t np_, int64_t tp, float* ds2p, float* ds2,
                          hipStream_t s);
hipError_t launch_ste_adam(float* p, const float* g, float* m, float* v, int64_t rows,
                           int64_t cols, int64_t ld, float lr, float b1, float b2, float c1,
                           float c2, float eps, hipStream_t s);
}  // namespace nq

struct nq_ste {
  int64_t m = 0, n = 0, r = 0, tmax = 0, mp = 0, np_ = 0, rp = 0, tp = 0;
  char* base = nullptr;
  float *U, *V, *s1, *s2, *mU, *vU, *mV, *vV, *ms1, *vs1, *ms2, *vs2;
  float *SU, *SUt, *SV, *SVt, *A, *At, *P, *Pt, *Q, *dQ, *dQt, *dP, *dPt, *dA, *dU, *dV;
  float *ds1, *ds2, *ds1p, *ds2p;
  double *lossp, *loss;
  int t = 0;
  bool has_params = false;
};

namespace {

constexpr int64_t kMaxDim = (1 << 21) - 256;
constexpr float kB1 = 0.9f, kB2 = 0.999f, kEps = 1e-8f;

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

struct Carve {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(int64_t count) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += ((size_t)count * sizeof(T) + 255) / 256 * 256;
    return p;
  }
};

size_t carve(nq_ste* h) {
  Carve c{h->base};
  const int64_t mp = h->mp, np_ = h->np_, rp = h->rp, tp = h->tp;
  h->U = c.take<float>(mp * rp); h->V = c.take<float>(np_ * rp);
  h->s1 = c.take<float>(mp); h->s2 = c.take<float>(np_);
  h->mU = c.take<float>(mp * rp); h->vU = c.take<float>(mp * rp);
  h->mV = c.take<float>(np_ * rp); h->vV = c.take<float>(np_ * rp);
  h->ms1 = c.take<float>(mp); h->vs1 = c.take<float>(mp);
  h->ms2 = c.take<float>(np_); h->vs2 = c.take<float>(np_);
  h->SU = c.take<float>(mp * rp); h->SUt = c.take<float>(rp * mp);
  h->SV = c.take<float>(np_ * rp); h->SVt = c.take<float>(rp * np_);
  h->A = c.take<float>(tp * np_); h->At = c.take<float>(np_ * tp);
  h->P = c.take<float>(tp * rp); h->Pt = c.take<float>(rp * tp);
  h->Q = c.take<float>(tp * mp); h->dQ = c.take<float>(tp * mp); h->dQt = c.take<float>(mp * tp);
  h->dP = c.take<float>(tp * rp); h->dPt = c.take<float>(rp * tp);
  h->dA = c.take<float>(tp * np_);
  h->dU = c.take<float>(mp * rp); h->dV = c.take<float>(np_ * rp);
  h->ds1 = c.take<float>(mp); h->ds2 = c.take<float>(np_);
  h->ds1p = c.take<float>((tp / 32) * mp); h->ds2p = c.take<float>((tp / 32) * np_);
  h->lossp = c.take<double>((tp / 32) * (mp / 32));
  h->loss = c.take<double>(1);
  return c.off;
}

hipError_t gemm(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                int64_t M, int64_t N, int64_t K, float* Ct, int64_t ldct, hipStream_t s) {
  GemmArgs g{};
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb; g.C = C; g.ldc = ldc;
  g.Ct = Ct; g.ldct = ldct; g.M = (int)M; g.N = (int)N; g.K = (int)K;
  return launch_gemm(g, Ct ? kEpiSolve : kEpiPlain, s);
}

hipError_t stage_in(const float* src, int64_t rows, int64_t cols, int64_t lds, float* dst,
                    int64_t rows_pad, int64_t ld_pad, hipStream_t s) {
  hipError_t e = launch_zero(dst, (size_t)(rows_pad * ld_pad), s);
  if (e != hipSuccess) return e;
  return hipMemcpy2DAsync(dst, sizeof(float) * ld_pad, src, sizeof(float) * lds,
                          sizeof(float) * cols, rows, hipMemcpyDeviceToDevice, s);
}

}  // namespace

extern "C" {

nq_status nq_ste_create(int64_t m, int64_t n, int64_t r, int64_t max_tokens, nq_ste_t* out) {
  if (!out) return set_error(NQ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (m < 1 || n < 1 || r < 1 || max_tokens < 1)
    return set_error(NQ_ERR_INVALID_ARG, "m, n, r and max_tokens must be >= 1");
  if (m > kMaxDim || n > kMaxDim || max_tokens > kMaxDim)
    return set_error(NQ_ERR_INVALID_ARG, "m, n and max_tokens must be <= 2^21 - 256");
  if (r > (1 << 13)) return set_error(NQ_ERR_INVALID_ARG, "r must be <= 2^13");
  nq_status st = gfx950_device();
  if (st != NQ_OK) return st;
  nq_ste* h = new nq_ste();
  h->m = m; h->n = n; h->r = r; h->tmax = max_tokens;
  h->mp = round_up(m, kPadMN); h->np_ = round_up(n, kPadMN);
  h->rp = round_up(r, kPadR); h->tp = round_up(max_tokens, 256);
  const size_t bytes = carve(h);
  hipError_t e = hipMalloc((void**)&h->base, bytes);
  if (e != hipSuccess) {
    delete h;
    return hip_error(e, "hipMalloc(STE workspace)");
  }
  carve(h);
  *out = h;
  return NQ_OK;
}

nq_status nq_ste_set_params(nq_ste_t h, const float* U, const float* V, const float* s1,
                            const float* s2, void* stream) {
  if (!h || !U || !V || !s1 || !s2)
    return set_error(NQ_ERR_INVALID_ARG, "handle, U, V, s1 and s2 are required");
  hipStream_t s = (hipStream_t)stream;
  NQ_HIPCHK(stage_in(U, h->m, h->r, h->r, h->U, h->mp, h->rp, s));
  NQ_HIPCHK(stage_in(V, h->n, h->r, h->r, h->V, h->np_, h->rp, s));
  NQ_HIPCHK(stage_in(s1, 1, h->m, h->m, h->s1, 1, h->mp, s));
  NQ_HIPCHK(stage_in(s2, 1, h->n, h->n, h->s2, 1, h->np_, s));
  // the moments are contiguous from mU to vs2
  NQ_HIPCHK(launch_zero(h->mU, (size_t)((char*)h->SU - (char*)h->mU) / sizeof(float), s));
  NQ_HIPCHK(launch_ste_signs(h->U, h->m, h->r, h->rp, h->mp, h->SU, h->SUt, s));
  NQ_HIPCHK(launch_ste_signs(h->V, h->n, h->r, h->rp, h->np_, h->SV, h->SVt, s));
  h->t = 0;
  h->has_params = true;
  return NQ_OK;
}

nq_status nq_ste_step(nq_ste_t h, const float* X, int64_t ldx, const float* Y, int64_t ldy,
                      const int32_t* rows, int64_t T, float lr, void* stream) {
  if (!h) return set_error(NQ_ERR_INVALID_ARG, "handle is NULL");
  if (!h->has_params) return set_error(NQ_ERR_INVALID_ARG, "nq_ste_set_params has not run");
  if (!X || !Y) return set_error(NQ_ERR_INVALID_ARG, "X and Y are required");
  if (T < 1 || T > h->tmax) return set_error(NQ_ERR_INVALID_ARG, "T must be in [1, max_tokens]");
  if (ldx < h->n || ldy < h->m) return set_error(NQ_ERR_INVALID_ARG, "ldx < n or ldy < m");
  if (!(lr >= 0.0f) || !std::isfinite(lr))
    return set_error(NQ_ERR_INVALID_ARG, "lr must be finite and >= 0");
  hipStream_t s = (hipStream_t)stream;
  const int64_t mp = h->mp, np_ = h->np_, rp = h->rp, tp = round_up(T, 256);
  // forward
  NQ_HIPCHK(launch_ste_stage(X, ldx, rows, T, h->n, h->s2, np_, tp, h->A, h->At, s));
  // (the four products with a sign factor run on the bf16 matrix cores,
  // exactly: launch_sign_gemm)
  NQ_HIPCHK(launch_sign_gemm(h->A, np_, h->SVt, np_, h->P, rp, h->Pt, tp, (int)tp, (int)rp, (int)np_, s));
  NQ_HIPCHK(launch_sign_gemm(h->P, rp, h->SU, rp, h->Q, mp, nullptr, 0, (int)tp, (int)mp, (int)rp, s));
  // loss, dL/dYq, ds1, dQ
  NQ_HIPCHK(launch_ste_loss(h->Q, Y, ldy, rows, T, h->m, h->s1, mp, tp, h->dQ, h->dQt, h->ds1p,
                            h->lossp, h->ds1, h->loss, s));
  // backward through the two sign products
  NQ_HIPCHK(gemm(h->dQt, tp, h->Pt, tp, h->dU, rp, mp, rp, tp, nullptr, 0, s));
  NQ_HIPCHK(launch_sign_gemm(h->dQ, mp, h->SUt, mp, h->dP, rp, h->dPt, tp, (int)tp, (int)rp, (int)mp, s));
  NQ_HIPCHK(gemm(h->At, tp, h->dPt, tp, h->dV, rp, np_, rp, tp, nullptr, 0, s));
  NQ_HIPCHK(launch_sign_gemm(h->dP, rp, h->SV, rp, h->dA, np_, nullptr, 0, (int)tp, (int)np_, (int)rp, s));
  NQ_HIPCHK(launch_ste_ds2(h->dA, X, ldx, rows, T, h->n, np_, tp, h->ds2p, h->ds2, s));
  // Adam, then the signs of the moved latents
  h->t += 1;
  const float c1 = (float)(1.0 - std::pow((double)kB1, h->t));
  const float c2 = (float)(1.0 - std::pow((double)kB2, h->t));
  NQ_HIPCHK(launch_ste_adam(h->U, h->dU, h->mU, h->vU, h->m, h->r, rp, lr, kB1, kB2, c1, c2, kEps, s));
  NQ_HIPCHK(launch_ste_adam(h->V, h->dV, h->mV, h->vV, h->n, h->r, rp, lr, kB1, kB2, c1, c2, kEps, s));
  NQ_HIPCHK(launch_ste_adam(h->s1, h->ds1, h->ms1, h->vs1, 1, h->m, h->m, lr, kB1, kB2, c1, c2, kEps, s));
  NQ_HIPCHK(launch_ste_adam(h->s2, h->ds2, h->ms2, h->vs2, 1, h->n, h->n, lr, kB1, kB2, c1, c2, kEps, s));
  NQ_HIPCHK(launch_ste_signs(h->U, h->m, h->r, rp, mp, h->SU, h->SUt, s));
  NQ_HIPCHK(launch_ste_signs(h->V, h->n, h->r, rp, np_, h->SV, h->SVt, s));
  return NQ_OK;
}

nq_status nq_ste_last_loss(nq_ste_t h, double* loss, void* stream) {
  if (!h || !loss) return set_error(NQ_ERR_INVALID_ARG, "handle and loss are required");
  if (h->t == 0) return set_error(NQ_ERR_INVALID_ARG, "no step has run");
  hipStream_t s = (hipStream_t)stream;
  NQ_HIPCHK(hipMemcpyAsync(loss, h->loss, sizeof(double), hipMemcpyDeviceToHost, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  return NQ_OK;
}

nq_status nq_ste_get_params(nq_ste_t h, float* U, float* V, float* s1, float* s2, void* stream) {
  if (!h) return set_error(NQ_ERR_INVALID_ARG, "handle is NULL");
  if (!h->has_params) return set_error(NQ_ERR_INVALID_ARG, "nq_ste_set_params has not run");
  hipStream_t s = (hipStream_t)stream;
  const hipMemcpyKind k = hipMemcpyDeviceToDevice;
  if (U)
    NQ_HIPCHK(hipMemcpy2DAsync(U, sizeof(float) * h->r, h->U, sizeof(float) * h->rp,
                               sizeof(float) * h->r, h->m, k, s));
  if (V)
    NQ_HIPCHK(hipMemcpy2DAsync(V, sizeof(float) * h->r, h->V, sizeof(float) * h->rp,
                               sizeof(float) * h->r, h->n, k, s));
  if (s1) NQ_HIPCHK(hipMemcpyAsync(s1, h->s1, sizeof(float) * h->m, k, s));
  if (s2) NQ_HIPCHK(hipMemcpyAsync(s2, h->s2, sizeof(float) * h->n, k, s));
  return NQ_OK;
}

nq_status nq_ste_destroy(nq_ste_t h) {
  if (!h) return NQ_OK;
  if (h->base) (void)hipFree(h->base);
  delete h;
  return NQ_OK;
}

}  // extern "C"
