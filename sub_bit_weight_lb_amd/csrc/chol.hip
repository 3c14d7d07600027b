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
// Diagonal tiles: outer-product elimination with register-resident 4 x 4
// blocks, the same row operations applied to an identity block, giving L_kk
// and M_kk = L_kk^-1 with one barrier per column. Off-diagonal tiles: 64 x 64
// x 64 products on the 32x32x2 fp32 MFMA.
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

// out = alpha * X op(Y) + beta * out on 64 x 64 blocks (ld = rp for all).
// op(Y) = Y^T if TRANS else Y.
template <bool TRANS>
__device__ void block_mm(const float* __restrict__ X, const float* __restrict__ Y, float* out,
                         int rp, float alpha, float beta, float* Xs, float* Ys) {
  const int tid = threadIdx.x;
  // X: 64 rows x 16 float4 = 1024 float4, 4 per thread, stored as is ([p][c]).
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int idx = tid + NT * q;
    const int row = idx >> 4, c4 = idx & 15;
    *(f32x4*)&Xs[row * LS + c4 * 4] = *(const f32x4*)&X[(int64_t)row * rp + c4 * 4];
  }
  if (TRANS) {
    // B operand (k = c, n = q) = Y[q][c]: Y as is, [q][c].
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = tid + NT * q;
      const int row = idx >> 4, c4 = idx & 15;
      *(f32x4*)&Ys[row * LS + c4 * 4] = *(const f32x4*)&Y[(int64_t)row * rp + c4 * 4];
    }
  } else {
    // B operand (k = c, n = q) = Y[c][q]: transpose to [q][c] while staging.
    const int col = tid & 63, cq = tid >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c0 = (cq + 4 * j) * 4;
      f32x4 v = {Y[(int64_t)(c0 + 0) * rp + col], Y[(int64_t)(c0 + 1) * rp + col],
                 Y[(int64_t)(c0 + 2) * rp + col], Y[(int64_t)(c0 + 3) * rp + col]};
      *(f32x4*)&Ys[col * LS + c0] = v;
    }
  }
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
    const float prev = beta != 0.0f ? *o : 0.0f;
    *o = alpha * acc[v] + beta * prev;
  }
  __syncthreads();  // Xs / Ys may be refilled by the caller's next product
}

// Diagonal block: L_kk and M_kk = L_kk^-1 of the 64 x 64 block (k, k).
// Outer-product elimination on the lower triangle with the same row
// operations applied to an identity block E. Thread t holds the 4 x 4 block
// (t / 16, t % 16) of T and of E in registers. Step j needs column j of T
// (multipliers and partners T[c][j]) and row j of E; their owners publish
// them to LDS after the previous step's update, so each step costs one
// barrier. At the end L = T D^-1/2 and M = D^-1/2 E with D the pivots.
struct DiagSmem {
  float colbuf[2][NB];
  float erow[2][NB];
  float dvec[NB];
};

__device__ __forceinline__ void diag_factor(float* A, float* M, int rp, int k, int r_real,
                                            DevStats* st, DiagSmem& sm) {
  float (&colbuf)[2][NB] = sm.colbuf;
  float (&erow)[2][NB] = sm.erow;
  float (&dvec)[NB] = sm.dvec;
  const int tid = threadIdx.x;
  const int bi = tid >> 4, bj = tid & 15;
  const int64_t base = (int64_t)k * NB;
  float Tr[4][4], Er[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const f32x4 v = *(const f32x4*)&A[(base + 4 * bi + a) * rp + base + 4 * bj];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      Tr[a][b] = v[b];
      Er[a][b] = (bi == bj && a == b) ? 1.0f : 0.0f;
    }
  }
  if (bj == 0) {
#pragma unroll
    for (int a = 0; a < 4; ++a) colbuf[0][4 * bi + a] = Tr[a][0];
  }
  if (bi == 0) {
#pragma unroll
    for (int b = 0; b < 4; ++b) erow[0][4 * bj + b] = Er[0][b];
  }
  __syncthreads();
  // Outer loop over 4-wide block columns (not unrolled, to bound register
  // use), inner 4 steps unrolled so every register index is static. Rows and
  // columns <= j are masked arithmetically. The entries the next step
  // broadcasts (column j+1 of T, row j+1 of E) are updated and published
  // first; the remaining updates overlap the LDS writes.
#pragma unroll 1
  for (int J = 0; J < NB / 4; ++J) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * J + jj;
      const int buf = jj & 1;
      const float d = colbuf[buf][j];
      if (tid == 0) dvec[j] = d;
      const float inv = __builtin_amdgcn_rcpf(d);
      const f32x4 li = *(const f32x4*)&colbuf[buf][4 * bi];
      const f32x4 cj = *(const f32x4*)&colbuf[buf][4 * bj];
      const f32x4 ej = *(const f32x4*)&erow[buf][4 * bj];
      float l[4], cm[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) l[a] = (4 * bi + a > j) ? li[a] * inv : 0.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b) cm[b] = (4 * bj + b > j) ? cj[b] : 0.0f;
      const int jo = (jj + 1) & 3;               // position of j + 1 in its block
      const int nb_ = (jj == 3) ? J + 1 : J;     // block index of j + 1
      if (j + 1 < NB) {
        if (bj == nb_) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            Tr[a][jo] = fmaf(-l[a], cm[jo], Tr[a][jo]);
            colbuf[buf ^ 1][4 * bi + a] = Tr[a][jo];
          }
        }
        if (bi == nb_) {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            Er[jo][b] = fmaf(-l[jo], ej[b], Er[jo][b]);
            erow[buf ^ 1][4 * bj + b] = Er[jo][b];
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool doneT = (j + 1 < NB) && bj == nb_ && b == jo;
          const bool doneE = (j + 1 < NB) && bi == nb_ && a == jo;
          if (!doneT) Tr[a][b] = fmaf(-l[a], cm[b], Tr[a][b]);
          if (!doneE) Er[a][b] = fmaf(-l[a], ej[b], Er[a][b]);
        }
      __syncthreads();
    }
  }
  if (tid == 0) {
    for (int j = 0; j < NB; ++j) {
      const float d = dvec[j];
      if (!(d > 0.0f && isfinite(d)) && (int)base + j < r_real) {
        atomicMin(&st->potrf_info, (int)base + j + 1);
        break;
      }
    }
  }
  f32x4 lv[4], mv[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int i = 4 * bi + a;
    const float si = sqrtf(dvec[i]);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int c = 4 * bj + b;
      lv[a][b] = c <= i ? Tr[a][b] / sqrtf(dvec[c]) : 0.0f;
      mv[a][b] = c <= i ? Er[a][b] / si : 0.0f;
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    *(f32x4*)&A[(base + 4 * bi + a) * rp + base + 4 * bj] = lv[a];
    *(f32x4*)&M[(base + 4 * bi + a) * rp + base + 4 * bj] = mv[a];
  }
}

__global__ __launch_bounds__(NT) void chol_diag0_kernel(float* A, float* M, int rp, int r_real,
                                                        DevStats* st) {
  __shared__ __attribute__((aligned(16))) DiagSmem dsm;
  diag_factor(A, M, rp, 0, r_real, st, dsm);
}

__global__ __launch_bounds__(NT) void chol_panel_kernel(float* A, float* M, int rp, int k) {
  __shared__ __attribute__((aligned(16))) float Xs[NB * LS];
  __shared__ __attribute__((aligned(16))) float Ys[NB * LS];
  const int R = rp / NB;
  const int nL = R - k - 1;
  const int b = blockIdx.x;
  const int64_t kk = (int64_t)k * NB;
  if (b < nL) {
    const int64_t i0 = (int64_t)(k + 1 + b) * NB;
    float* Aik = A + i0 * rp + kk;
    block_mm<true>(Aik, M + kk * rp + kk, Aik, rp, 1.0f, 0.0f, Xs, Ys);
  } else {
    const int64_t j0 = (int64_t)(b - nL) * NB;
    float* Mkj = M + kk * rp + j0;
    block_mm<false>(M + kk * rp + kk, Mkj, Mkj, rp, -1.0f, 0.0f, Xs, Ys);
  }
}

__global__ __launch_bounds__(NT) void chol_update_kernel(float* A, float* M, int rp, int k,
                                                         int r_real, DevStats* st) {
  __shared__ __attribute__((aligned(16))) float Xs[NB * LS];
  __shared__ __attribute__((aligned(16))) float Ys[NB * LS];
  __shared__ __attribute__((aligned(16))) DiagSmem dsm;
  const int R = rp / NB;
  const int n = R - k - 1;
  const int64_t kk = (int64_t)k * NB;
  int b = blockIdx.x;
  if (b == 0) {
    // next diagonal tile: A_{k+1,k+1} -= L_{k+1,k} L_{k+1,k}^T, then factor it
    const int64_t d0 = kk + NB;
    block_mm<true>(A + d0 * rp + kk, A + d0 * rp + kk, A + d0 * rp + d0, rp, -1.0f, 1.0f, Xs, Ys);
    __threadfence_block();
    diag_factor(A, M, rp, k + 1, r_real, st, dsm);
    return;
  }
  b -= 1;
  const int nA = n * (n + 1) / 2 - 1;  // lower tiles of the trailing block but (k+1, k+1)
  if (b < nA) {
    const int t = b + 1;
    int ii = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
    while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
    while (ii * (ii + 1) / 2 > t) --ii;
    const int jj = t - ii * (ii + 1) / 2;
    const int64_t i0 = (int64_t)(k + 1 + ii) * NB, j0 = (int64_t)(k + 1 + jj) * NB;
    block_mm<true>(A + i0 * rp + kk, A + j0 * rp + kk, A + i0 * rp + j0, rp, -1.0f, 1.0f, Xs, Ys);
  } else {
    const int q = b - nA;
    const int ii = q / (k + 1), jj = q % (k + 1);
    const int64_t i0 = (int64_t)(k + 1 + ii) * NB, j0 = (int64_t)jj * NB;
    block_mm<false>(A + i0 * rp + kk, M + kk * rp + j0, M + i0 * rp + j0, rp, 1.0f, 1.0f, Xs, Ys);
  }
}

__global__ void zero_upper_kernel(float* A, int rp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rp * rp) return;
  const int i = (int)(idx / rp), j = (int)(idx % rp);
  if (j > i) A[idx] = 0.0f;
}

}  // namespace

hipError_t launch_cholesky_inverse(float* A, float* M, int rp, int r_real, DevStats* st,
                                   bool zero_upper_L, hipStream_t s) {
  if (rp % NB) return hipErrorInvalidValue;
  const int R = rp / NB;
  hipError_t e = launch_zero(M, (size_t)rp * rp, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chol_diag0_kernel, dim3(1), dim3(NT), 0, s, A, M, rp, r_real, st);
  for (int k = 0; k < R; ++k) {
    const int np = (R - k - 1) + k;
    if (np > 0) hipLaunchKernelGGL(chol_panel_kernel, dim3(np), dim3(NT), 0, s, A, M, rp, k);
    const int n = R - k - 1;
    if (n > 0) {
      const int nb = 1 + (n * (n + 1) / 2 - 1) + n * (k + 1);
      hipLaunchKernelGGL(chol_update_kernel, dim3(nb), dim3(NT), 0, s, A, M, rp, k, r_real, st);
    }
  }
  if (!zero_upper_L) return hipGetLastError();
  const int64_t tot = (int64_t)rp * rp;
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, A, rp);
  return hipGetLastError();
}

}  // namespace nq
