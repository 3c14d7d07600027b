// Building-block entry points: each runs one step of the per-layer path on
// caller buffers of any shape by staging them into zero-padded temporaries
// (the kernels themselves assume tile-multiple shapes). Synchronous; they
// allocate, so they are for tests and tools, not for the hot path.
#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

#include "abi.h"
#include "common.h"

using namespace nq;

namespace {

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
  hipError_t alloc(size_t bytes) { return hipMalloc(&p, std::max<size_t>(bytes, 256)); }
  float* f() const { return (float*)p; }
  double* d() const { return (double*)p; }
};

// dst (rows_pad x cols_pad, zero padded) <- src (rows x cols, ld lds)
hipError_t stage_in(const float* src, int64_t rows, int64_t cols, int64_t lds, float* dst,
                    int64_t rows_pad, int64_t cols_pad, hipStream_t s) {
  hipError_t e = launch_zero(dst, (size_t)(rows_pad * cols_pad), s);
  if (e != hipSuccess) return e;
  return hipMemcpy2DAsync(dst, sizeof(float) * cols_pad, src, sizeof(float) * lds,
                          sizeof(float) * cols, rows, hipMemcpyDeviceToDevice, s);
}

hipError_t stage_out(const float* src, int64_t lds, float* dst, int64_t ldd, int64_t rows,
                     int64_t cols, hipStream_t s) {
  return hipMemcpy2DAsync(dst, sizeof(float) * ldd, src, sizeof(float) * lds,
                          sizeof(float) * cols, rows, hipMemcpyDeviceToDevice, s);
}

// Argument checks shared by the two binary-layer entry points; *noop when
// there is nothing to compute.
nq_status check_binmm(const uint32_t* U_bits, int64_t ldu, const uint32_t* Vt_bits, int64_t ldvt,
                      int64_t m, int64_t n, int64_t r, const float* s1, const float* s2,
                      const float* X, int64_t B, int64_t ldx, float* Y, int64_t ldy, bool* noop) {
  if (m < 0 || n < 0 || r < 0 || B < 0)
    return set_error(NQ_ERR_INVALID_ARG, "m, n, r and B must be >= 0");
  if (m == 0 || B == 0) {
    *noop = true;
    return NQ_OK;
  }
  if (n == 0 || r == 0) return set_error(NQ_ERR_INVALID_ARG, "n and r must be >= 1 when m, B >= 1");
  if (!U_bits || !Vt_bits || !s1 || !s2 || !X || !Y)
    return set_error(NQ_ERR_INVALID_ARG, "U_bits, Vt_bits, s1, s2, X and Y are required");
  if (ldu < (r + 31) / 32) return set_error(NQ_ERR_INVALID_ARG, "ldu < ceil(r/32)");
  if (ldvt < (n + 31) / 32) return set_error(NQ_ERR_INVALID_ARG, "ldvt < ceil(n/32)");
  if (ldx < n || ldy < m) return set_error(NQ_ERR_INVALID_ARG, "ldx < n or ldy < m");
  return NQ_OK;
}

}  // namespace

extern "C" {

nq_status nq_pack_signs(const float* X, int64_t rows, int64_t cols, int64_t ldx, uint32_t* bits,
                        int64_t ld_words, void* stream) {
  if (rows < 0 || cols < 0) return set_error(NQ_ERR_INVALID_ARG, "rows and cols must be >= 0");
  if (rows == 0 || cols == 0) return NQ_OK;
  if (!X || !bits) return set_error(NQ_ERR_INVALID_ARG, "X and bits are required");
  if (ldx < cols) return set_error(NQ_ERR_INVALID_ARG, "ldx < cols");
  if (ld_words < (cols + 31) / 32) return set_error(NQ_ERR_INVALID_ARG, "ld_words < ceil(cols/32)");
  NQ_HIPCHK(launch_pack_signs(X, rows, cols, ldx, bits, ld_words, (hipStream_t)stream));
  return NQ_OK;
}

nq_status nq_transpose_signs(const uint32_t* in, int64_t rows, int64_t cols, int64_t ld_in,
                             uint32_t* out, int64_t ld_out, void* stream) {
  if (rows < 0 || cols < 0) return set_error(NQ_ERR_INVALID_ARG, "rows and cols must be >= 0");
  if (rows == 0 || cols == 0) return NQ_OK;
  if (!in || !out) return set_error(NQ_ERR_INVALID_ARG, "in and out are required");
  if (ld_in < (cols + 31) / 32) return set_error(NQ_ERR_INVALID_ARG, "ld_in < ceil(cols/32)");
  if (ld_out < (rows + 31) / 32) return set_error(NQ_ERR_INVALID_ARG, "ld_out < ceil(rows/32)");
  NQ_HIPCHK(launch_transpose_bits(in, rows, cols, ld_in, out, ld_out, (hipStream_t)stream));
  return NQ_OK;
}

int64_t nq_binary_matmul_work_floats(int64_t B, int64_t n, int64_t r) {
  if (B < 0 || n < 0 || r < 0) return -1;
  return binmm_work_floats(B, n, r);
}

nq_status nq_binary_matmul(const uint32_t* U_bits, int64_t ldu, const uint32_t* Vt_bits,
                           int64_t ldvt, int64_t m, int64_t n, int64_t r, const float* s1,
                           const float* s2, const float* X, int64_t B, int64_t ldx, float* Y,
                           int64_t ldy, float* work, void* stream) {
  bool noop = false;
  nq_status st = check_binmm(U_bits, ldu, Vt_bits, ldvt, m, n, r, s1, s2, X, B, ldx, Y, ldy, &noop);
  if (st != NQ_OK || noop) return st;
  if (!work) return set_error(NQ_ERR_INVALID_ARG, "work is required");
  if ((uintptr_t)work % 16) return set_error(NQ_ERR_INVALID_ARG, "work must be 16-byte aligned");
  NQ_HIPCHK(launch_binary_matmul(U_bits, ldu, Vt_bits, ldvt, m, n, r, s1, s2, X, B, ldx, Y, ldy,
                                 work, (hipStream_t)stream));
  return NQ_OK;
}

nq_status nq_binary_matmul_noalloc(const uint32_t* U_bits, int64_t ldu, const uint32_t* Vt_bits,
                                   int64_t ldvt, int64_t m, int64_t n, int64_t r,
                                   const float* s1, const float* s2, const float* X, int64_t B,
                                   int64_t ldx, float* Y, int64_t ldy, void* stream) {
  bool noop = false;
  nq_status st = check_binmm(U_bits, ldu, Vt_bits, ldvt, m, n, r, s1, s2, X, B, ldx, Y, ldy, &noop);
  if (st != NQ_OK || noop) return st;
  if (binmm_work_floats(B, n, r) > kBinScratchFloats)
    return set_error(NQ_ERR_INVALID_ARG,
                     "the call's workspace exceeds the fixed scratch "
                     "(nq_binary_matmul_work_floats(B, n, r) <= 2^23 for nq_binary_matmul_noalloc)");
  float* work = nullptr;
  NQ_HIPCHK(binmm_fixed_scratch(&work));
  NQ_HIPCHK(launch_binary_matmul(U_bits, ldu, Vt_bits, ldvt, m, n, r, s1, s2, X, B, ldx, Y, ldy,
                                 work, (hipStream_t)stream));
  return NQ_OK;
}

nq_status nq_op_precondition(const float* W, int64_t ldw, int64_t m, int64_t n,
                             const float* d_out, const float* d_in, float* Wt, int64_t ldwt,
                             void* stream) {
  if (m < 1 || n < 1 || ldw < n || ldwt < n || !W || !d_out || !d_in || !Wt)
    return set_error(NQ_ERR_INVALID_ARG, "bad precondition arguments");
  hipStream_t s = (hipStream_t)stream;
  const int64_t mp = round_up(m, 64), np_ = round_up(n, 64);
  DevBuf t, parts, st;
  NQ_HIPCHK(t.alloc(sizeof(float) * mp * np_));
  const int nb = precondition_nblocks((int)mp, (int)np_);
  NQ_HIPCHK(parts.alloc(sizeof(double) * 2 * nb));
  NQ_HIPCHK(st.alloc(sizeof(DevStats)));
  NQ_HIPCHK(launch_stats_init((DevStats*)st.p, s));
  NQ_HIPCHK(launch_precondition(W, ldw, m, n, d_out, d_in, t.f(), nullptr, (int)mp, (int)np_,
                                parts.d(), parts.d() + nb, (DevStats*)st.p, s));
  NQ_HIPCHK(stage_out(t.f(), np_, Wt, ldwt, m, n, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  return NQ_OK;
}

nq_status nq_op_gram(const float* A, int64_t rows, int64_t cols, int64_t lda, float rho, float* G,
                     int64_t ldg, void* stream) {
  if (rows < 1 || cols < 1 || lda < cols || ldg < cols || !A || !G)
    return set_error(NQ_ERR_INVALID_ARG, "bad gram arguments");
  hipStream_t s = (hipStream_t)stream;
  const int64_t K = round_up(rows, 32), rp = round_up(cols, 128);
  const GramPlan plan = gram_plan((int)K, (int)rp);
  DevBuf a, at, part, g;
  NQ_HIPCHK(a.alloc(sizeof(float) * K * rp));
  NQ_HIPCHK(at.alloc(sizeof(float) * rp * K));
  NQ_HIPCHK(part.alloc(sizeof(float) * plan.slots * rp * rp));
  NQ_HIPCHK(g.alloc(sizeof(float) * rp * rp));
  NQ_HIPCHK(stage_in(A, rows, cols, lda, a.f(), K, rp, s));
  NQ_HIPCHK(launch_transpose(a.f(), K, rp, rp, at.f(), K, s));
  NQ_HIPCHK(launch_gram_partial(at.f(), K, (int)K, (int)rp, plan, part.f(), s));
  NQ_HIPCHK(launch_gram_reduce(part.f(), (int)K, (int)rp, plan, rho, true, g.f(), rp, s));
  NQ_HIPCHK(stage_out(g.f(), rp, G, ldg, cols, cols, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  return NQ_OK;
}

nq_status nq_op_gemm_rhs(const float* A, int64_t lda, const float* B, int64_t ldb, const float* P,
                         int64_t ldp, float rho, float* C, int64_t ldc, int64_t rows, int64_t cols,
                         int64_t k, void* stream) {
  if (rows < 1 || cols < 1 || k < 1 || !A || !B || !C || lda < k || ldb < cols || ldc < cols ||
      (P && ldp < cols))
    return set_error(NQ_ERR_INVALID_ARG, "bad gemm arguments");
  hipStream_t s = (hipStream_t)stream;
  const int64_t Mp = round_up(rows, 256), Np = round_up(cols, 128), Kp = round_up(k, 32);
  DevBuf a, b, bt, p, c;
  NQ_HIPCHK(a.alloc(sizeof(float) * Mp * Kp));
  NQ_HIPCHK(b.alloc(sizeof(float) * Kp * Np));
  NQ_HIPCHK(bt.alloc(sizeof(float) * Np * Kp));
  NQ_HIPCHK(p.alloc(sizeof(float) * Mp * Np));
  NQ_HIPCHK(c.alloc(sizeof(float) * Mp * Np));
  NQ_HIPCHK(stage_in(A, rows, k, lda, a.f(), Mp, Kp, s));
  NQ_HIPCHK(stage_in(B, k, cols, ldb, b.f(), Kp, Np, s));
  NQ_HIPCHK(launch_transpose(b.f(), Kp, Np, Np, bt.f(), Kp, s));  // the kernel reads B^T
  if (P) NQ_HIPCHK(stage_in(P, rows, cols, ldp, p.f(), Mp, Np, s));
  else NQ_HIPCHK(launch_zero(p.f(), (size_t)(Mp * Np), s));
  GemmArgs g{};
  g.A = a.f(); g.lda = Kp; g.B = bt.f(); g.ldb = Kp; g.C = c.f(); g.ldc = Np;
  g.P = p.f(); g.rho = rho; g.M = (int)Mp; g.N = (int)Np; g.K = (int)Kp;
  // more tiles than CUs, not in whole rounds: the leftover tiles split along
  // K, as in the layer's RHS GEMM and solve
  DevBuf part;
  if (const size_t pf = gemm_part_floats((int)Mp, (int)Np, (int)Kp, 0)) {
    NQ_HIPCHK(part.alloc(sizeof(float) * pf));
    g.part = part.f();
  }
  NQ_HIPCHK(launch_gemm(g, kEpiRhs, s));
  NQ_HIPCHK(stage_out(c.f(), Np, C, ldc, rows, cols, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  return NQ_OK;
}

nq_status nq_op_sign_gemm(const float* A, int64_t lda, const float* S, int64_t lds, float* C,
                          int64_t ldc, float* Ct, int64_t ldct, int64_t rows, int64_t cols,
                          int64_t k, void* stream) {
  if (rows < 1 || cols < 1 || k < 1 || !A || !S || !C || lda < k || lds < k || ldc < cols ||
      (Ct && ldct < rows))
    return set_error(NQ_ERR_INVALID_ARG, "bad sign gemm arguments");
  if (rows > (1 << 24) || cols > (1 << 24) || k > (1 << 24))
    return set_error(NQ_ERR_INVALID_ARG, "rows, cols and k must be <= 2^24");
  hipStream_t s = (hipStream_t)stream;
  const int64_t Mp = round_up(rows, 128), Np = round_up(cols, 128), Kp = round_up(k, 64);
  DevBuf a, b, c, ct;
  NQ_HIPCHK(a.alloc(sizeof(float) * Mp * Kp));
  NQ_HIPCHK(b.alloc(sizeof(float) * Np * Kp));
  NQ_HIPCHK(c.alloc(sizeof(float) * Mp * Np));
  if (Ct) NQ_HIPCHK(ct.alloc(sizeof(float) * Np * Mp));
  NQ_HIPCHK(stage_in(A, rows, k, lda, a.f(), Mp, Kp, s));
  NQ_HIPCHK(stage_in(S, cols, k, lds, b.f(), Np, Kp, s));
  NQ_HIPCHK(launch_sign_gemm(a.f(), Kp, b.f(), Kp, c.f(), Np, Ct ? ct.f() : nullptr, Mp,
                             (int)Mp, (int)Np, (int)Kp, s));
  NQ_HIPCHK(stage_out(c.f(), Np, C, ldc, rows, cols, s));
  if (Ct) NQ_HIPCHK(stage_out(ct.f(), Mp, Ct, ldct, cols, rows, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  return NQ_OK;
}

nq_status nq_op_cholesky_inverse(const float* G, int64_t r, int64_t ldg, float* L, int64_t ldl,
                                 float* Ginv, int64_t ldgi, int64_t* info, void* stream) {
  if (r < 1 || ldg < r || !G || !info || (L && ldl < r) || (Ginv && ldgi < r))
    return set_error(NQ_ERR_INVALID_ARG, "bad cholesky arguments");
  hipStream_t s = (hipStream_t)stream;
  const int64_t rp = round_up(r, 128);
  DevBuf a, m, mt, part, gi, st;
  NQ_HIPCHK(a.alloc(sizeof(float) * rp * rp));
  NQ_HIPCHK(m.alloc(sizeof(float) * rp * rp));
  const GramPlan plan = gram_plan((int)rp, (int)rp, true);
  if (Ginv) {
    NQ_HIPCHK(mt.alloc(sizeof(float) * rp * rp));
    NQ_HIPCHK(part.alloc(sizeof(float) * plan.slots * rp * rp));
    NQ_HIPCHK(gi.alloc(sizeof(float) * rp * rp));
    // the chain writes only the upper block triangle of M^T
    NQ_HIPCHK(launch_zero(mt.f(), (size_t)rp * rp, s));
  }
  NQ_HIPCHK(st.alloc(sizeof(DevStats)));
  DevStats* dst = (DevStats*)st.p;
  NQ_HIPCHK(launch_stats_init(dst, s));
  // [G 0; 0 I]: the identity keeps the padded system positive definite
  NQ_HIPCHK(stage_in(G, r, r, ldg, a.f(), rp, rp, s));
  NQ_HIPCHK(launch_set_diag(a.f(), rp, (int)r, (int)rp, 1.0f, s));
  // m: L^-1 scratch, not returned (no zeroing needed)
  NQ_HIPCHK(launch_cholesky_inverse(a.f(), m.f(), (int)rp, (int)r, dst, true, false, s, false,
                                    Ginv ? mt.f() : nullptr));
  if (Ginv) {
    // G^-1 = M^T M, as in the ADMM loop: triangular Gram of M^T, then the
    // full-symmetric reduction with no shift
    NQ_HIPCHK(launch_gram_partial(mt.f(), rp, (int)rp, (int)rp, plan, part.f(), s));
    NQ_HIPCHK(launch_gram_reduce(part.f(), (int)rp, (int)rp, plan, 0.0f, true, gi.f(), rp, s));
    NQ_HIPCHK(stage_out(gi.f(), rp, Ginv, ldgi, r, r, s));
  }
  if (L) NQ_HIPCHK(stage_out(a.f(), rp, L, ldl, r, r, s));
  DevStats hs;
  NQ_HIPCHK(hipMemcpyAsync(&hs, dst, sizeof(hs), hipMemcpyDeviceToHost, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  *info = hs.potrf_info == 0x7fffffff ? 0 : hs.potrf_info;
  if (*info) return set_error(NQ_ERR_NOT_POSITIVE_DEFINITE, "Cholesky pivot <= 0");
  return NQ_OK;
}

nq_status nq_op_svid(const float* X, int64_t rows, int64_t cols, int64_t ldx, int32_t T, float* Z,
                     int64_t ldz, float* a, float* b, void* stream) {
  if (rows < 1 || cols < 1 || T < 1 || ldx < cols || !X || (Z && ldz < cols))
    return set_error(NQ_ERR_INVALID_ARG, "bad svid arguments");
  if (rows > (1 << 21) || cols > (1 << 13)) return set_error(NQ_ERR_INVALID_ARG, "svid shape too large");
  hipStream_t s = (hipStream_t)stream;
  const int64_t rows_pad = round_up(rows, 256), rp = round_up(cols, 128);
  DevBuf x, p, wa, wb, sync, st;
  NQ_HIPCHK(x.alloc(sizeof(float) * rows_pad * rp));
  NQ_HIPCHK(p.alloc(sizeof(float) * rows_pad * rp));
  NQ_HIPCHK(wa.alloc(sizeof(float) * rows_pad));
  NQ_HIPCHK(wb.alloc(sizeof(float) * rp));
  const int G = svid_grid();
  const size_t nw = svid_sync_words((int)rp, G);
  NQ_HIPCHK(sync.alloc(sizeof(uint64_t) * nw));
  NQ_HIPCHK(st.alloc(sizeof(DevStats)));
  NQ_HIPCHK(hipMemsetAsync(sync.p, 0, sizeof(uint64_t) * nw, s));
  NQ_HIPCHK(launch_stats_init((DevStats*)st.p, s));
  SvidWork w{wa.f(), wb.f(), svid_sync_at((uint64_t*)sync.p, (int)rp, G), (DevStats*)st.p, G};
  NQ_HIPCHK(stage_in(X, rows, cols, ldx, x.f(), rows_pad, rp, s));
  NQ_HIPCHK(launch_svid(x.f(), p.f(), (int)rows_pad, (int)rp, (int)cols, T, 2, w, s));
  if (Z) NQ_HIPCHK(stage_out(p.f(), rp, Z, ldz, rows, cols, s));
  if (a) NQ_HIPCHK(hipMemcpyAsync(a, wa.f(), sizeof(float) * rows, hipMemcpyDeviceToDevice, s));
  if (b) NQ_HIPCHK(hipMemcpyAsync(b, wb.f(), sizeof(float) * cols, hipMemcpyDeviceToDevice, s));
  DevStats hs;
  NQ_HIPCHK(hipMemcpyAsync(&hs, st.p, sizeof(hs), hipMemcpyDeviceToHost, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  if (hs.sync_timeout)
    return set_error(NQ_ERR_HIP, "the SVID launch's workgroups were not all resident within about 0.5 s "
                                 "(first expired wait: workgroup " + std::to_string(hs.to_wg) +
                                 ", step " + std::to_string(hs.to_step) + ", tag wanted " +
                                 std::to_string(hs.to_want) + ", read " +
                                 std::to_string(hs.to_seen) + ")");
  return NQ_OK;
}

nq_status nq_op_svid_dual(const float* U, const float* Lam, int64_t rows, int64_t cols,
                          int64_t ldi, int32_t T, float* Z, float* Lam_out, int64_t ldo,
                          float* a, float* b, void* stream) {
  if (rows < 1 || cols < 1 || T < 1 || ldi < cols || ldo < cols || !U || !Lam || !Z || !Lam_out)
    return set_error(NQ_ERR_INVALID_ARG, "bad svid_dual arguments");
  if (rows > (1 << 21) || cols > (1 << 13)) return set_error(NQ_ERR_INVALID_ARG, "svid shape too large");
  hipStream_t s = (hipStream_t)stream;
  const int64_t rows_pad = round_up(rows, 256), rp = round_up(cols, 128);
  DevBuf u, x, p, wa, wb, sync, st;
  NQ_HIPCHK(u.alloc(sizeof(float) * rows_pad * rp));
  NQ_HIPCHK(x.alloc(sizeof(float) * rows_pad * rp));
  NQ_HIPCHK(p.alloc(sizeof(float) * rows_pad * rp));
  NQ_HIPCHK(wa.alloc(sizeof(float) * rows_pad));
  NQ_HIPCHK(wb.alloc(sizeof(float) * rp));
  const int G = svid_grid();
  const size_t nw = svid_sync_words((int)rp, G);
  NQ_HIPCHK(sync.alloc(sizeof(uint64_t) * nw));
  NQ_HIPCHK(st.alloc(sizeof(DevStats)));
  NQ_HIPCHK(hipMemsetAsync(sync.p, 0, sizeof(uint64_t) * nw, s));
  NQ_HIPCHK(launch_stats_init((DevStats*)st.p, s));
  SvidWork w{wa.f(), wb.f(), svid_sync_at((uint64_t*)sync.p, (int)rp, G), (DevStats*)st.p, G};
  NQ_HIPCHK(stage_in(U, rows, cols, ldi, u.f(), rows_pad, rp, s));
  NQ_HIPCHK(stage_in(Lam, rows, cols, ldi, x.f(), rows_pad, rp, s));
  NQ_HIPCHK(launch_svid(x.f(), p.f(), (int)rows_pad, (int)rp, (int)cols, T, 1, w, s, u.f()));
  // Z = P + Lam_out (P = Z - Lam_out is what the update stores)
  NQ_HIPCHK(launch_add_compact(p.f(), x.f(), rows, cols, (int)rp, u.f(), s));
  NQ_HIPCHK(stage_out(u.f(), cols, Z, ldo, rows, cols, s));
  NQ_HIPCHK(stage_out(x.f(), rp, Lam_out, ldo, rows, cols, s));
  if (a) NQ_HIPCHK(hipMemcpyAsync(a, wa.f(), sizeof(float) * rows, hipMemcpyDeviceToDevice, s));
  if (b) NQ_HIPCHK(hipMemcpyAsync(b, wb.f(), sizeof(float) * cols, hipMemcpyDeviceToDevice, s));
  DevStats hs;
  NQ_HIPCHK(hipMemcpyAsync(&hs, st.p, sizeof(hs), hipMemcpyDeviceToHost, s));
  NQ_HIPCHK(hipStreamSynchronize(s));
  if (hs.sync_timeout)
    return set_error(NQ_ERR_HIP, "the SVID launch's workgroups were not all resident within about 0.5 s "
                                 "(first expired wait: workgroup " + std::to_string(hs.to_wg) +
                                 ", step " + std::to_string(hs.to_step) + ", tag wanted " +
                                 std::to_string(hs.to_want) + ", read " +
                                 std::to_string(hs.to_seen) + ")");
  return NQ_OK;
}

}  // extern "C"
