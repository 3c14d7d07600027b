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
// Diagonal tiles: one wave, 2 x 2 blocks of 32: two in-register
// factorisations with their inverses (readlane broadcasts) and four block
// products on the MFMA. Off-diagonal tiles: 64 x 64 x 64
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

__device__ __forceinline__ float bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---- 32 x 32 factorisation with its inverse on one wave ("half-wave" form)
// Lanes 0-31 hold rows of the Schur complement t, lanes 32-63 columns of
// E = Lt^-1 (Lt unit lower triangular, A = Lt D Lt^T). Step j broadcasts
// p_c = t[j] of lane c (readlane) and every lane applies the same
//   r[c] -= x p_c,  c > j,  x = r[j] / d_j,
// which is the elimination t[c] -= (t[j] / d_j) p_c on rows and the same
// row operation e[c] -= p_c (e[j] / d_j) on the identity. Lanes i <= j only
// touch entries right of their diagonal, which are never read. After step j
// r[j] is scaled by d_j^-1/2: lanes 0-31 then hold row i of L (c <= i),
// lanes 32-63 column i of L^-1 = D^-1/2 Lt^-1 (exact zeros above the
// diagonal).
// Broadcasts go in groups of 8 pinned into SGPRs by an empty asm (no
// instruction) before their FMAs, so they issue back to back instead of
// alternating with their consumers through one SGPR.
template <int J, int C>
__device__ __forceinline__ void hw_cols(float (&r)[32], float src, float x) {
  if constexpr (C < 32) {
    constexpr int n = (32 - C) < 8 ? (32 - C) : 8;
    float p[8];
#pragma unroll
    for (int q = 0; q < n; ++q) p[q] = bcast(src, C + q);
    if constexpr (n == 8)
      asm volatile("" : "+s"(p[0]), "+s"(p[1]), "+s"(p[2]), "+s"(p[3]), "+s"(p[4]), "+s"(p[5]),
                   "+s"(p[6]), "+s"(p[7]));
#pragma unroll
    for (int q = 0; q < n; ++q) r[C + q] = fmaf(-x, p[q], r[C + q]);
    hw_cols<J, C + n>(r, src, x);
  }
}
template <int J>
__device__ __forceinline__ void hw_steps(float (&r)[32]) {
  if constexpr (J < 32) {
    const float src = r[J];
    const float d = bcast(src, J);
    const float x = src * __builtin_amdgcn_rcpf(d);
    hw_cols<J, J + 1>(r, src, x);
    r[J] = src * __builtin_amdgcn_rsqf(d);
    hw_steps<J + 1>(r);
  }
}

// LDS of the diagonal-tile factorisation: 32 x 32 blocks that change lane
// layout between phases (aliases the product buffers of the update kernel).
struct DiagSmem {
  float Mc[32][33];  // Mc[c][i] = M11[i][c]
  float Nc[32][33];  // Nc[c][i] = M22[i][c]
  float Ls[32][33];  // L21
  float Ts[32][33];  // A22 - L21 L21^T
  float Ps[32][33];  // P = L21 M11
};

// Hand-off of LDS data between lanes of one wave: without a fence the
// compiler, which proves independence per lane, may move one lane's read of a
// value above another lane's write of it.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// 32 x 32 x 32 product on the 32x32x2 fp32 MFMA with k = 2 s + (lane / 32)
// at step s; fa(s), fb(s) return this lane's A[lane % 32][k] and
// B[k][lane % 32]. acc[v] is C[8 (v / 4) + 4 (lane / 32) + v % 4][lane % 32].
template <class FA, class FB>
__device__ __forceinline__ f32x16 mm32(FA fa, FB fb, f32x16 acc) {
#pragma unroll
  for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa(s), fb(s), acc, 0, 0, 0);
  return acc;
}

// Diagonal tile k: A_kk = L L^T and M_kk = L^-1, written to A and M (zeros
// above the diagonal), on wave 0, in 2 x 2 blocks of 32:
//   L11, M11 from A11 (half-wave factorisation);
//   L21 = A21 M11^T;  T = A22 - L21 L21^T;
//   L22, M22 from T (half-wave factorisation);
//   M21 = -M22 (L21 M11).
// The four products run on the MFMA; LDS only changes lane layouts between
// them (one wave, so LDS order is program order and no barrier is needed).
// Pivots <= 0 or non-finite set potrf_info (first such row, 1-based).
__device__ __forceinline__ void diag_factor(float* A, float* M, int rp, int k, int r_real,
                                            DevStats* st, DiagSmem& sm) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x, i = lane & 31, h = lane >> 5;
  const int64_t base = (int64_t)k * NB;
  float* A0 = A + base * rp + base;  // tile origin
  float* M0 = M + base * rp + base;
  float r[32];
  float dg = 0.0f;  // this lane's diagonal of L (lanes 0-31), block 11 then 22
  uint64_t badmask = 0;

  // A21 in the A-operand layout of the first product and A22 in the
  // accumulator layout of the second, loaded now so that their latency
  // hides behind the first factorisation
  float a21[16], a22[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) a21[s] = A0[(int64_t)(32 + i) * rp + 2 * s + h];
#pragma unroll
  for (int v = 0; v < 16; ++v)
    a22[v] = A0[(int64_t)(32 + 8 * (v >> 2) + 4 * h + (v & 3)) * rp + 32 + i];

  // ---- L11, M11
  if (h == 0) {
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      const f32x4 v = *(const f32x4*)&A0[(int64_t)i * rp + 4 * c4];
      r[4 * c4] = v[0]; r[4 * c4 + 1] = v[1]; r[4 * c4 + 2] = v[2]; r[4 * c4 + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = c == i ? 1.0f : 0.0f;
  }
  hw_steps<0>(r);
  if (h == 0) {
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * c4 + q;
        v[q] = c <= i ? r[c] : 0.0f;
        dg = c == i ? r[c] : dg;
      }
      *(f32x4*)&A0[(int64_t)i * rp + 4 * c4] = v;
      *(f32x4*)&A0[(int64_t)i * rp + 32 + 4 * c4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  } else {
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      M0[(int64_t)q * rp + i] = r[q];
      M0[(int64_t)q * rp + 32 + i] = 0.0f;
      sm.Mc[i][q] = r[q];
    }
  }
  {
    const bool bad = h == 0 && !(dg > 0.0f && isfinite(dg)) && (int)base + i < r_real;
    badmask |= (uint64_t)(uint32_t)__ballot(bad);
  }

  wave_lds_sync();  // Mc

  // ---- L21 = A21 M11^T
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  acc = mm32([&](int s) { return a21[s]; },
             [&](int s) { return sm.Mc[2 * s + h][i]; }, acc);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int iv = 8 * (v >> 2) + 4 * h + (v & 3);
    A0[(int64_t)(32 + iv) * rp + i] = acc[v];
    sm.Ls[iv][i] = acc[v];
  }

  wave_lds_sync();  // Ls

  // ---- T = A22 - L21 L21^T
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = a22[v];
  acc = mm32([&](int s) { return -sm.Ls[i][2 * s + h]; },
             [&](int s) { return sm.Ls[i][2 * s + h]; }, acc);
#pragma unroll
  for (int v = 0; v < 16; ++v) sm.Ts[8 * (v >> 2) + 4 * h + (v & 3)][i] = acc[v];

  // ---- P = L21 M11 (needs neither T nor the second factorisation)
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  acc = mm32([&](int s) { return sm.Ls[i][2 * s + h]; },
             [&](int s) { return sm.Mc[i][2 * s + h]; }, acc);
#pragma unroll
  for (int v = 0; v < 16; ++v) sm.Ps[8 * (v >> 2) + 4 * h + (v & 3)][i] = acc[v];

  wave_lds_sync();  // Ts, Ps

  // ---- L22, M22
  if (h == 0) {
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = sm.Ts[i][c];
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = c == i ? 1.0f : 0.0f;
  }
  hw_steps<0>(r);
  dg = 0.0f;
  if (h == 0) {
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = 4 * c4 + q;
        v[q] = c <= i ? r[c] : 0.0f;
        dg = c == i ? r[c] : dg;
      }
      *(f32x4*)&A0[(int64_t)(32 + i) * rp + 32 + 4 * c4] = v;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      M0[(int64_t)(32 + q) * rp + 32 + i] = r[q];
      sm.Nc[i][q] = r[q];
    }
  }
  {
    const bool bad = h == 0 && !(dg > 0.0f && isfinite(dg)) && (int)base + 32 + i < r_real;
    badmask |= (uint64_t)(uint32_t)__ballot(bad) << 32;
  }

  wave_lds_sync();  // Nc

  // ---- M21 = -M22 P
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
  acc = mm32([&](int s) { return -sm.Nc[2 * s + h][i]; },
             [&](int s) { return sm.Ps[2 * s + h][i]; }, acc);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int iv = 8 * (v >> 2) + 4 * h + (v & 3);
    M0[(int64_t)(32 + iv) * rp + i] = acc[v];
  }
  if (badmask && lane == 0)
    atomicMin(&st->potrf_info, (int)base + __ffsll((unsigned long long)badmask));
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
