// Blocked Cholesky factorisation with the inverse factor: G = L L^T and
// M = L^-1, for the ridge-regularised system matrix G = V^T V + rho I of the
// regularised solve (NanoQuant digest, section 核心方法, step (a): the linear
// system is solved through a Cholesky factorisation; the implementation blog,
// section 待办事项, names this factorisation as where LB-ADMM spends its time).
//
// Right-looking, block size 64, two launches per block column k:
//   panel(k):  L_ik = A_ik M_kk^T for i > k (in place), and row k of the
//              inverse factor, M_kj = -M_kk S_kj for j < k;
//   update(k): trailing update A_ij -= L_ik L_jk^T (i >= j > k) and the
//              inverse partial sums S_ij += L_ik M_kj (i > k >= j); its first
//              workgroup instead updates the next diagonal tile and factors
//              it, so no launch is spent on the diagonal alone.
// Diagonal tiles: one wave factors the tile in registers (one row per lane,
// column broadcasts through LDS, no barrier per column) while a second wave
// forms L^-1 from the same broadcasts. Off-diagonal tiles: 64 x 64 x 64
// products on the 32x32x2 fp32 MFMA.
// The identity  sum_{l = j..i} L_il M_lj = delta_ij  gives
// M_ij = -M_ii sum_{l = j..i-1} L_il M_lj; the partial sums S_ij are kept in
// M's own tiles until row i of M is formed.
// Workgroups of one launch never wait for each other: every dependency
// crosses a launch boundary.
#include "common.h"
#include <climits>

namespace nq {
namespace {

constexpr int NB = kNB;   // 64
constexpr int NT = 256;
constexpr int LS = NB + 4;  // LDS row stride for MFMA tiles

// Epilogues of the 64 x 64 block product P = op(X) op(Y).
enum BlockEpi {
  kBlkAxpby,  // out = alpha P + beta out
  kBlkSymAcc  // symmetric accumulate into G^-1 (see block_mm)
};

// 64 x 64 x 64 block product on the 32x32x2 fp32 MFMA (ld = rp for all).
// op(X) = X^T if TA else X; op(Y) = Y^T if TB else Y.
// kBlkAxpby:  out = alpha P + beta out.
// kBlkSymAcc: out is tile (i, j), i >= j, of a symmetric matrix and out2 its
//   mirror tile (j, i) (out2 == out on the diagonal, where only P's lower
//   triangle is used). v = P + (beta != 0 ? out : 0) is written to out and,
//   transposed, to out2, so both halves hold the same sums and the result
//   is exactly symmetric.
template <bool TA, bool TB, BlockEpi EPI = kBlkAxpby>
__device__ void block_mm(const float* __restrict__ X, const float* __restrict__ Y, float* out,
                         int rp, float alpha, float beta, float* Xs, float* Ys,
                         float* out2 = nullptr) {
  const int tid = threadIdx.x;
  // Both operands are staged [m or n][k] with k contiguous.
  auto stage_rows = [&](const float* S, float* D) {  // operand(i, c) = S[i][c]
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + NT * q;
      const int row = idx >> 4, c4 = idx & 15;
      *(f32x4*)&D[row * LS + c4 * 4] = *(const f32x4*)&S[(int64_t)row * rp + c4 * 4];
    }
  };
  auto stage_cols = [&](const float* S, float* D) {  // operand(i, c) = S[c][i]
    const int col = tid & 63, cq = tid >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = (cq + 4 * j) * 4;
      f32x4 v = {S[(int64_t)(c0 + 0) * rp + col], S[(int64_t)(c0 + 1) * rp + col],
                 S[(int64_t)(c0 + 2) * rp + col], S[(int64_t)(c0 + 3) * rp + col]};
      *(f32x4*)&D[col * LS + c0] = v;
    }
  };
  if (TA) stage_cols(X, Xs); else stage_rows(X, Xs);
  if (TB) stage_rows(Y, Ys); else stage_cols(Y, Ys);
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  const float* xs = Xs + (wm * 32 + l32) * LS + 4 * half;
  const float* ys = Ys + (wn * 32 + l32) * LS + 4 * half;
#pragma unroll
  for (int kc = 0; kc < NB; kc += 8) {
    const f32x4 a = *(const f32x4*)&xs[kc];
    const f32x4 b = *(const f32x4*)&ys[kc];
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = wm * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
    const int col = wn * 32 + l32;
    float* o = out + (int64_t)row * rp + col;
    if (EPI == kBlkAxpby) {
      const float prev = beta != 0.0f ? *o : 0.0f;
      *o = alpha * acc[v] + beta * prev;
    } else {
      if (out2 == out && col > row) continue;  // diagonal tile: lower triangle only
      const float val = acc[v] + (beta != 0.0f ? *o : 0.0f);
      *o = val;
      out2[(int64_t)col * rp + row] = val;
    }
  }
  __syncthreads();  // Xs / Ys may be refilled by the caller's next product
}

// LDS of the diagonal-tile factorisation (aliases the product buffers of
// the update kernel, which are idle by then).
struct DiagSmem {
  float col[NB][NB];  // col[j][i]: Schur column j at row i (i >= j), published by wave 0
  float dpiv[NB];     // pivots d_j
  float rs[NB];       // 1 / sqrt(d_j)
  int ready;          // columns 0 .. ready - 1 of col are published
};

// Upper bound on the sleep iterations of the consumer wave (each s_sleep 1
// is about 64 clocks, so about 0.1 s): the producer publishes all 64
// columns within microseconds; the bound only guarantees the wait ends.
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ float bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Wait until at least n columns are published; false if the bound ran out.
__device__ __forceinline__ bool wait_ready(const DiagSmem& sm, int n) {
  int spins = 0;
  while (__hip_atomic_load(&sm.ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < n) {
    __builtin_amdgcn_s_sleep(1);
    if (++spins > kSpinLimit) return false;
  }
  return true;
}

// Diagonal tile k: A_kk = L L^T and M_kk = L^-1, written to A and M (zeros
// above the diagonal). Right-looking elimination A = Lt D Lt^T (Lt unit lower
// triangular, D the pivots), L = Lt D^1/2, L^-1 = D^-1/2 Lt^-1.
//  - Wave 0 holds the Schur complement in registers, lane i holding row i.
//    Step j broadcasts column j through LDS (uniform-address reads) and
//    updates t[c] -= (t[j] / d_j) col_j[c] for c > j. Software pipelined:
//    column j + 1 is final once its entry of step j is updated, so it is
//    published, and its reads are in flight, while the rest of step j
//    issues; the pivot comes by readlane.
//  - Wave 1 applies the same row operations to the identity in column form
//    (lane c holds column c of Lt^-1): e[i] -= col_j[i] (e[j] / d_j), i > j,
//    reading the published columns, which it waits for in groups of 8
//    through an LDS counter (bounded wait).
// Pivots <= 0 or non-finite set potrf_info (first such row, 1-based).
__device__ __forceinline__ void diag_factor(float* A, float* M, int rp, int k, int r_real,
                                            DevStats* st, DiagSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t base = (int64_t)k * NB;
  if (tid == 0) sm.ready = 0;
  __syncthreads();
  bool waited = true;
  if (wave == 0) {
    float t[NB];
#pragma unroll
    for (int c4 = 0; c4 < NB / 4; ++c4) {
      const f32x4 v = *(const f32x4*)&A[(base + lane) * rp + base + 4 * c4];
      t[4 * c4 + 0] = v[0];
      t[4 * c4 + 1] = v[1];
      t[4 * c4 + 2] = v[2];
      t[4 * c4 + 3] = v[3];
    }
    float cv[2][NB];
    sm.col[0][lane] = t[0];
    __hip_atomic_store(&sm.ready, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int c = 1; c < NB; ++c) cv[0][c] = sm.col[0][c];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int b = j & 1;
      const float d = bcast(t[j], j);
      sm.dpiv[j] = d;
      const float l = lane > j ? t[j] * __builtin_amdgcn_rcpf(d) : 0.0f;
      if (j + 1 < NB) {
        t[j + 1] = fmaf(-l, cv[b][j + 1], t[j + 1]);
        sm.col[j + 1][lane] = t[j + 1];
        __hip_atomic_store(&sm.ready, j + 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int c = j + 2; c < NB; ++c) cv[b ^ 1][c] = sm.col[j + 1][c];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = j + 2; c < NB; ++c) t[c] = fmaf(-l, cv[b][c], t[c]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // t[c] (c < lane) = Lt_ic d_c, t[lane] = d_lane; L_ic = t[c] / sqrt(d_c)
    const float di = sm.dpiv[lane];
    sm.rs[lane] = 1.0f / sqrtf(di);
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int c4 = 0; c4 < NB / 4; ++c4) {
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * c4 + q;
        v[q] = c < lane ? t[c] * sm.rs[c] : (c == lane ? sqrtf(di) : 0.0f);
      }
      *(f32x4*)&A[(base + lane) * rp + base + 4 * c4] = v;
    }
  } else if (wave == 1) {
    float e[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) e[i] = i == lane ? 1.0f : 0.0f;
    float cw[2][NB];
    float* mrow = M + base * rp + base + lane;  // row j of the tile at step j
    waited = wait_ready(sm, 9);
#pragma unroll
    for (int i = 0; i < NB; ++i) cw[0][i] = sm.col[0][i];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int b = j & 1;
      if (j + 1 < NB) {
        if ((j + 1) % 8 == 0) waited = waited && wait_ready(sm, j + 9 < NB ? j + 9 : NB);
        // The read address carries an opaque zero that depends on e[j], so
        // the compiler cannot hoist a later step's reads into this one (all
        // reads between two waits would otherwise be issued at once and
        // overflow the register file). The shift keeps 256-byte alignment
        // visible, so the reads still merge into 16-byte loads.
        int z;
        asm volatile("s_mov_b32 %0, 0" : "=s"(z) : "v"(e[j]));
        const float* cj = &sm.col[j + 1][0] + (z << 6);
#pragma unroll
        for (int i = j + 1; i < NB; ++i) cw[b ^ 1][i] = cj[i];
      }
      __builtin_amdgcn_sched_barrier(0);
      // row j of Lt^-1 is final: M_jc = e[j] / sqrt(d_j), a contiguous row store
      const float d = cw[b][j];
      *mrow = e[j] * __builtin_amdgcn_rsqf(d);
      mrow += rp;
      const float f = e[j] * __builtin_amdgcn_rcpf(d);
#pragma unroll
      for (int i = j + 1; i < NB; ++i) e[i] = fmaf(-cw[b][i], f, e[i]);
      // pin this step's updates here (no instruction): otherwise the
      // instruction selector sinks each update towards its last use and keeps
      // every broadcast value of the group of steps live
#pragma unroll
      for (int i = j + 1; i < NB; ++i) asm volatile("" : "+v"(e[i]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  if (wave == 1) {
    if (!waited && lane == 0) atomicMin(&st->potrf_info, (int)base + 1);
  } else if (wave == 0) {
    const float d = sm.dpiv[lane];
    const bool bad = !(d > 0.0f && isfinite(d)) && (int)base + lane < r_real;
    const uint64_t m = __ballot(bad);
    if (m && lane == 0) atomicMin(&st->potrf_info, (int)base + __ffsll((unsigned long long)m));
  }
}

__global__ __launch_bounds__(NT) void chol_diag0_kernel(float* A, float* M, int rp, int r_real,
                                                        DevStats* st) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ __attribute__((aligned(16))) DiagSmem dsm;
  diag_factor(A, M, rp, 0, r_real, st, dsm);
}

__global__ __launch_bounds__(NT) void chol_panel_kernel(float* A, float* M, int rp, int k) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ __attribute__((aligned(16))) float Xs[NB * LS];
  __shared__ __attribute__((aligned(16))) float Ys[NB * LS];
  const int R = rp / NB;
  const int nL = R - k - 1;
  const int b = blockIdx.x;
  const int64_t kk = (int64_t)k * NB;
  if (b < nL) {
    const int64_t i0 = (int64_t)(k + 1 + b) * NB;
    float* Aik = A + i0 * rp + kk;
    block_mm<false, true>(Aik, M + kk * rp + kk, Aik, rp, 1.0f, 0.0f, Xs, Ys);
  } else {
    const int64_t j0 = (int64_t)(b - nL) * NB;
    float* Mkj = M + kk * rp + j0;
    block_mm<false, false>(M + kk * rp + kk, Mkj, Mkj, rp, -1.0f, 0.0f, Xs, Ys);
  }
}

// Lower-triangle tile index t -> (i, j), i >= j.
__device__ __forceinline__ void tri_index(int t, int& i, int& j) {
  int ii = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
  while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
  while (ii * (ii + 1) / 2 > t) --ii;
  i = ii;
  j = t - ii * (ii + 1) / 2;
}

// Workgroups of update(k), in this order:
//   1 (if k + 1 < R): A_{k+1,k+1} -= L_{k+1,k} L_{k+1,k}^T, then factor it;
//   the other lower tiles of the trailing block: A_ij -= L_ik L_jk^T;
//   inverse partial sums: S_ij += L_ik M_kj (i > k >= j), kept in M;
//   if Ginv: Ginv_ij += M_ki^T M_kj for j <= i <= k (row k of M is final
//     once panel(k) has run; tile (i, j) starts at k = i), plus mirror.
// With k = R - 1 only the Ginv group is left (after the last panel).
__global__ __launch_bounds__(NT) void chol_update_kernel(float* A, float* M, float* Ginv, int rp,
                                                         int k, int r_real, DevStats* st) {
  __builtin_amdgcn_s_setprio(3);
  // product buffers and the diagonal-tile scratch share one LDS block
  constexpr int kProdFloats = 2 * NB * LS;
  constexpr int kDiagFloats = (int)(sizeof(DiagSmem) / sizeof(float));
  __shared__ __attribute__((aligned(16))) float lds[kProdFloats > kDiagFloats ? kProdFloats
                                                                             : kDiagFloats];
  float* Xs = lds;
  float* Ys = lds + NB * LS;
  DiagSmem& dsm = *reinterpret_cast<DiagSmem*>(lds);
  const int R = rp / NB;
  const int n = R - k - 1;
  const int64_t kk = (int64_t)k * NB;
  int b = blockIdx.x;
  if (n > 0) {
    if (b == 0) {
      const int64_t d0 = kk + NB;
      block_mm<false, true>(A + d0 * rp + kk, A + d0 * rp + kk, A + d0 * rp + d0, rp, -1.0f, 1.0f,
                            Xs, Ys);
      __threadfence_block();
      __syncthreads();
      diag_factor(A, M, rp, k + 1, r_real, st, dsm);
      return;
    }
    b -= 1;
    const int nA = n * (n + 1) / 2 - 1;  // lower tiles of the trailing block but (k+1, k+1)
    if (b < nA) {
      int ii, jj;
      tri_index(b + 1, ii, jj);
      const int64_t i0 = (int64_t)(k + 1 + ii) * NB, j0 = (int64_t)(k + 1 + jj) * NB;
      block_mm<false, true>(A + i0 * rp + kk, A + j0 * rp + kk, A + i0 * rp + j0, rp, -1.0f, 1.0f,
                            Xs, Ys);
      return;
    }
    b -= nA;
    const int nS = n * (k + 1);
    if (b < nS) {
      const int ii = b / (k + 1), jj = b % (k + 1);
      const int64_t i0 = (int64_t)(k + 1 + ii) * NB, j0 = (int64_t)jj * NB;
      block_mm<false, false>(A + i0 * rp + kk, M + kk * rp + j0, M + i0 * rp + j0, rp, 1.0f, 1.0f,
                             Xs, Ys);
      return;
    }
    b -= nS;
  }
  int ii, jj;
  tri_index(b, ii, jj);
  const int64_t i0 = (int64_t)ii * NB, j0 = (int64_t)jj * NB;
  block_mm<true, false, kBlkSymAcc>(M + kk * rp + i0, M + kk * rp + j0, Ginv + i0 * rp + j0, rp,
                                    1.0f, ii == k ? 0.0f : 1.0f, Xs, Ys, Ginv + j0 * rp + i0);
}

__global__ void zero_upper_kernel(float* A, int rp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rp * rp) return;
  const int i = (int)(idx / rp), j = (int)(idx % rp);
  if (j > i) A[idx] = 0.0f;
}

}  // namespace

hipError_t launch_cholesky_inverse(float* A, float* M, float* Ginv, int rp, int r_real,
                                   DevStats* st, bool zero_upper_L, hipStream_t s) {
  if (rp % NB) return hipErrorInvalidValue;
  const int R = rp / NB;
  hipError_t e = launch_zero(M, (size_t)rp * rp, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chol_diag0_kernel, dim3(1), dim3(NT), 0, s, A, M, rp, r_real, st);
  for (int k = 0; k < R; ++k) {
    const int np = (R - k - 1) + k;
    if (np > 0) hipLaunchKernelGGL(chol_panel_kernel, dim3(np), dim3(NT), 0, s, A, M, rp, k);
    const int n = R - k - 1;
    const int nb = (n > 0 ? 1 + (n * (n + 1) / 2 - 1) + n * (k + 1) : 0) +
                   (Ginv ? (k + 1) * (k + 2) / 2 : 0);
    if (nb > 0)
      hipLaunchKernelGGL(chol_update_kernel, dim3(nb), dim3(NT), 0, s, A, M, Ginv, rp, k, r_real,
                         st);
  }
  if (!zero_upper_L) return hipGetLastError();
  const int64_t tot = (int64_t)rp * rp;
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, A, rp);
  return hipGetLastError();
}

}  // namespace nq
