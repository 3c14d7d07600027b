// Blocked Cholesky factorisation with the inverse factor: G = L L^T and
// M = L^-1 (and M^T), for the ridge-regularised system matrix
// G = V^T V + rho I of the regularised solve (NanoQuant digest, section
// 核心方法, step (a): the linear system is solved through a Cholesky
// factorisation; the implementation blog, section 待办事项, names this
// factorisation as where LB-ADMM spends its time).
//
// Right-looking, block size 64 (R = rp / 64 block columns), one launch per
// block column k (k = 0 .. R - 1; one more, k = R, only when L itself is
// wanted). Launch k holds
//   - the panel of step k: L_ik = (A_ik - L_{i,k-1} L_{k,k-1}^T) M_kk^T,
//     i > k, each tile applying the last update of step k - 1 itself;
//   - row k of the inverse: M_kj = -M_kk (S_kj + L_{k,k-1} M_{k-1,j}), j < k;
//   - M_kk itself;
//   - the rest of step k - 1: trailing update A_ij -= L_{i,k-1} L_{j,k-1}^T
//     (i >= j > k) and inverse partial sums S_ij += L_{i,k-1} M_{k-1,j}
//     (i > k, j < k);
//   - optionally L_{k-1,k-1} (only when L itself is wanted).
// Optionally M^T as well (M_kk and each inverse-row tile stored transposed),
// the operand of G^-1 = M^T M, which a triangular Gram product forms
// afterwards (G^-1 used to be accumulated here, row by row of M, as a third
// kind of update tile; the update tiles run beside the RHS GEMM, so that
// work now waits for the chain's end).
// Every workgroup that needs M_kk (panel and inverse-row tiles) factors the
// diagonal tile A_kk - L_{k,k-1} L_{k,k-1}^T itself: some 32 CUs each do
// the same 64 x 64 factorisation, and no launch is spent on the diagonal
// alone. The identity  sum_{l = j..i} L_il M_lj = delta_ij  gives
// M_ij = -M_ii sum_{l = j..i-1} L_il M_lj; the partial sums S_ij are kept in
// M's own tiles until row i of M is formed, the first term (l = j) stored
// rather than added, so M needs no zeroing beforehand. No workgroup reads a tile that
// another workgroup of the same launch writes; every dependency crosses a
// launch boundary.
// Diagonal tiles: one wave, 2 x 2 blocks of 32: two in-register
// factorisations with their inverses (readlane broadcasts) and four block
// products on the MFMA. Off-diagonal tiles: 64 x 64 x 64 products on the
// 32x32x2 fp32 MFMA.
#include "common.h"
#include <algorithm>
#include <climits>
#include <cstdlib>

namespace nq {
namespace {

constexpr int NB = kNB;     // 64
constexpr int NT = 256;
constexpr int TS = NB + 4;  // LDS row stride of a 64 x 64 tile

// Workgroups per launch. Beside a running GEMM workgroup (110.6 KB of LDS)
// a CU has room for one of these (38.5 KB), so a launch of at most one
// workgroup per CU runs in a single round; the update tiles are then
// shared out over the workgroups left after the diagonal ones. 0 = one
// workgroup per tile. NQ_CHOL_BLOCKS overrides it.
int chol_launch_cap() {
  static const int cap = [] {
    const char* e = std::getenv("NQ_CHOL_BLOCKS");
    return e ? std::max(0, std::atoi(e)) : 256;
  }();
  return cap;
}
constexpr int kCholMinUpdBlocks = 32;

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
// layout between phases.
struct DiagSmem {
  float Mc[32][33];  // Mc[c][i] = M11[i][c]
  float Nc[32][33];  // Nc[c][i] = M22[i][c]
  float Ls[32][33];  // L21
  float Ts[32][33];  // A22 - L21 L21^T
  float Ps[32][33];  // P = L21 M11
};

// LDS of one workgroup of the step kernel.
struct StepSmem {
  DiagSmem dg;
  float T[NB * TS];  // input tile of the diagonal factorisation, then M_kk
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

// ---- 64 x 64 x 64 block products, one 32 x 32 quadrant (qm, qn) per wave
// Operands are row-major tiles with leading dimension ld, in global memory
// or LDS: A(m, k) = X[m][k] (or X[k][m] if TA), B(k, n) = Y[k][n] (or
// Y[n][k] if TB). Each wave loads its MFMA fragments straight from the
// operands, all of them before the first MFMA (one load latency, no LDS
// staging, no barrier): in each group of 8 k the lane half h feeds
// k = 4 h + s to MFMA step s, so a row-major operand fragment is one 16-byte
// load. acc[v] is C[qm 32 + 8 (v / 4) + 4 h + v % 4][qn 32 + lane % 32].
template <bool TA, bool TB>
__device__ __forceinline__ f32x16 mm_quad(const float* X, int ldx, const float* Y, int ldy, int qm,
                                          int qn) {
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  const int m = qm * 32 + l32, n = qn * 32 + l32;
  f32x4 a[8], b[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int k0 = 8 * g + 4 * h;
    if (TA) {
      a[g] = f32x4{X[(int64_t)k0 * ldx + m], X[(int64_t)(k0 + 1) * ldx + m],
                   X[(int64_t)(k0 + 2) * ldx + m], X[(int64_t)(k0 + 3) * ldx + m]};
    } else {
      a[g] = *(const f32x4*)&X[(int64_t)m * ldx + k0];
    }
    if (TB) {
      b[g] = *(const f32x4*)&Y[(int64_t)n * ldy + k0];
    } else {
      b[g] = f32x4{Y[(int64_t)k0 * ldy + n], Y[(int64_t)(k0 + 1) * ldy + n],
                   Y[(int64_t)(k0 + 2) * ldy + n], Y[(int64_t)(k0 + 3) * ldy + n]};
    }
  }
  // all loads are in flight before the first MFMA (without the barrier the
  // compiler keeps two to four in flight and waits before every MFMA group)
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[g][q], b[g][q], acc, 0, 0, 0);
  return acc;
}

// The quadrant (qm, qn) of a global tile in the accumulator layout.
__device__ __forceinline__ f32x16 load_quad(const float* src, int rp, int qm, int qn) {
  f32x16 v;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int row = qm * 32 + 8 * (q >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (q & 3);
    v[q] = src[(int64_t)row * rp + qn * 32 + (threadIdx.x & 31)];
  }
  return v;
}

// Quadrant of wave w in a 4-wave product.
__device__ __forceinline__ int wave_qm() { return (threadIdx.x >> 6) & 1; }
__device__ __forceinline__ int wave_qn() { return threadIdx.x >> 7; }
__device__ __forceinline__ int qrow(int qm, int v) {
  return qm * 32 + 8 * (v >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (v & 3);
}
__device__ __forceinline__ int qcol(int qn) { return qn * 32 + (threadIdx.x & 31); }

// out = alpha * acc + prev on quadrant (qm, qn) (global, ld rp); prev is
// the quadrant's old value (load_quad, issued before the product so that its
// latency overlaps the MFMAs) or zero.
__device__ __forceinline__ void store_quad(const f32x16& acc, const f32x16& prev, float* out,
                                           int rp, float alpha, int qm, int qn) {
#pragma unroll
  for (int v = 0; v < 16; ++v) out[(int64_t)qrow(qm, v) * rp + qcol(qn)] = fmaf(alpha, acc[v], prev[v]);
}
// The transpose of quadrant (qm, qn) of a tile, v = alpha acc, into outT
// (ld rp): lane l holds column qn 32 + l % 32, rows qm 32 + 8 g + 4 (l / 32)
// + 0..3 in registers 4 g .. 4 g + 3, one float4 each.
__device__ __forceinline__ void store_quad_t(const f32x16& acc, float* outT, int rp, float alpha,
                                             int qm, int qn) {
  const int lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
  float* row = outT + (int64_t)(qn * 32 + l32) * rp + qm * 32 + 4 * h;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *(f32x4*)&row[8 * g] = f32x4{alpha * acc[4 * g], alpha * acc[4 * g + 1],
                                 alpha * acc[4 * g + 2], alpha * acc[4 * g + 3]};
}
__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int v = 0; v < 16; ++v) z[v] = 0.0f;
  return z;
}

// Quadrant (qm, qn) of the 64 x 64 tile at rows r0, columns c0 (r0 >= c0)
// of a Gram product not yet reduced, in the accumulator layout: the sum of
// its stream-K segments in slot order, + rho on the diagonal. In a diagonal
// tile the elements above the diagonal are read from their mirror below it,
// as the reduction writes them.
__device__ __forceinline__ f32x16 load_quad_gram(const GramSrc& g, int rp, int r0, int c0, int qm,
                                                 int qn) {
  const int I = r0 / 128, J = c0 / 128;
  const int64_t t0 = g.gs.tile_start(I, J);
  const int nseg = (int)((t0 + g.gs.len(I) - 1) / g.L - t0 / g.L) + 1;
  const int64_t plane = (int64_t)rp * rp;
  int64_t off[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = r0 + qrow(qm, v), col = c0 + qcol(qn);
    off[v] = row >= col ? (int64_t)row * rp + col : (int64_t)col * rp + row;
  }
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = g.part[off[v]];
  for (int c = 1; c < nseg; ++c) {
    const float* p = g.part + c * plane;
    f32x16 w;
#pragma unroll
    for (int v = 0; v < 16; ++v) w[v] = p[off[v]];
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] += w[v];
  }
  if (r0 == c0 && qm == qn) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (qrow(qm, v) == qcol(qn)) acc[v] += g.rho;
  }
  return acc;
}

// Diagonal tile: Tin (LDS, stride TS) holds the lower blocks T11, T21, T22
// of the 64 x 64 SPD tile; its factor L and M = L^-1 are formed in 2 x 2
// blocks of 32 (diag_step below: the two factorisations on wave 0, the
// block products on all four waves):
//   L11, M11 from T11 (half-wave factorisation);
//   L21 = T21 M11^T;  T22' = T22 - L21 L21^T;
//   L22, M22 from T22' (half-wave factorisation);
//   M21 = -M22 (L21 M11).
// LDS only changes lane layouts between the phases (a barrier, or a
// wavefront fence where one wave hands data between its own lanes).
// M (zeros above the diagonal) goes to M0 with leading dimension rp, or
// with M_LDS to Tin itself (stride TS; every part of the input is read
// before the part of M that replaces it is written), or nowhere if M0 is
// null. With WRITE_L, L (zeros above the diagonal) goes to L0 (ld rp).
// With st, a pivot <= 0 or non-finite sets potrf_info (first such row
// row0 + i, 1-based; rows at or past r_real are padding and not checked).
// Part 1 (wave 0): L11, M11 from T11; needs only rows 0-31, columns 0-31 of
// Tin. Sets bit i of badmask for a bad pivot in row i.
template <bool M_LDS, bool WRITE_L>
__device__ __forceinline__ void diag_part1(const float* Tin, float* M0, float* L0, int rp,
                                           int row0, int r_real, DiagSmem& sm,
                                           uint64_t& badmask, float* Mt0) {
  const int lane = threadIdx.x, i = lane & 31, h = lane >> 5;
  const int ldm = M_LDS ? TS : rp;  // M0 is Tin itself when M_LDS
  float r[32];
  float dg = 0.0f;  // this lane's diagonal of L11 (lanes 0-31)

  // ---- L11, M11
  if (h == 0) {
#pragma unroll
    for (int c4 = 0; c4 < 8; ++c4) {
      const f32x4 v = *(const f32x4*)&Tin[i * TS + 4 * c4];
      r[4 * c4] = v[0]; r[4 * c4 + 1] = v[1]; r[4 * c4 + 2] = v[2]; r[4 * c4 + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = c == i ? 1.0f : 0.0f;
  }
  wave_lds_sync();  // every lane has read its part of the input tile
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
      if (WRITE_L) {
        *(f32x4*)&L0[(int64_t)i * rp + 4 * c4] = v;
        *(f32x4*)&L0[(int64_t)i * rp + 32 + 4 * c4] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      if (M0) {
        M0[q * ldm + i] = r[q];
        M0[q * ldm + 32 + i] = 0.0f;
      }
      if (Mt0) {  // M^T, ld rp: row i of M11^T, and zeros below it in M^T
        Mt0[(int64_t)i * rp + q] = r[q];
        Mt0[(int64_t)(32 + i) * rp + q] = 0.0f;
      }
      sm.Mc[i][q] = r[q];
    }
  }
  {
    const bool bad = h == 0 && !(dg > 0.0f && isfinite(dg)) && row0 + i < r_real;
    badmask |= (uint64_t)(uint32_t)__ballot(bad);
  }
}

// 32 x 32 x 32 product split over the four waves, one 16 x 16 block
// (bi, bj) = (wave & 1, wave >> 1) each, on the 16x16x4 fp32 MFMA with
// k = 4 s + lane / 16 at step s; fa(s), fb(s) return this lane's
// A[16 bi + lane % 16][k] and B[k][16 bj + lane % 16]. c[v] is
// C[16 bi + 4 (lane / 16) + v][16 bj + lane % 16].
template <class FA, class FB>
__device__ __forceinline__ f32x4 mm16(FA fa, FB fb, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(fa(s), fb(s), c, 0, 0, 0);
  return c;
}

// Second 32 x 32 factorisation (wave 0): L22, M22 from Ts (T22 - L21 L21^T);
// L22 to L0 (WRITE_L), M22 to M0 (nullable), its columns to Nc. Sets bits
// 32 + i of badmask for a bad pivot in row 32 + i.
template <bool M_LDS, bool WRITE_L>
__device__ __forceinline__ void diag_factor2(float* M0, float* L0, int rp, int row0, int r_real,
                                             DiagSmem& sm, uint64_t& badmask, float* Mt0) {
  const int lane = threadIdx.x, i = lane & 31, h = lane >> 5;
  const int ldm = M_LDS ? TS : rp;
  float r[32];
  float dg = 0.0f;
  if (h == 0) {
#pragma unroll
    for (int c = 0; c < 32; ++c) r[c] = sm.Ts[i][c];
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
      if (WRITE_L) *(f32x4*)&L0[(int64_t)(32 + i) * rp + 32 + 4 * c4] = v;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      if (M0) M0[(32 + q) * ldm + 32 + i] = r[q];
      if (Mt0) Mt0[(int64_t)(32 + i) * rp + 32 + q] = r[q];
      sm.Nc[i][q] = r[q];
    }
  }
  const bool bad = h == 0 && !(dg > 0.0f && isfinite(dg)) && row0 + 32 + i < r_real;
  badmask |= (uint64_t)(uint32_t)__ballot(bad) << 32;
}

// Lower-triangle tile index t -> (i, j), i >= j.
__device__ __forceinline__ void tri_index(int t, int& i, int& j) {
  int ii = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
  while ((ii + 1) * (ii + 2) / 2 <= t) ++ii;
  while (ii * (ii + 1) / 2 > t) --ii;
  i = ii;
  j = t - ii * (ii + 1) / 2;
}

// The lower blocks of T = A_kk - L_{k,k-1} L_{k,k-1}^T (just A_00 for k = 0,
// summed from the Gram's segments with g), the input of the diagonal
// factorisation of step k, into sm.T: wave 0 forms T11, wave 1 T21, wave 2
// T22 (T12 is never read).
__device__ __forceinline__ void diag_input(const float* A, int rp, int k, StepSmem& sm,
                                           const GramSrc& g) {
  const int wave = threadIdx.x >> 6;
  if (wave == 3) return;
  const int qm = wave == 0 ? 0 : 1, qn = wave == 2 ? 1 : 0;
  const int64_t kk = (int64_t)k * NB;
  const float* Akk = A + kk * rp + kk;
  f32x16 t = g.part ? load_quad_gram(g, rp, 0, 0, qm, qn) : load_quad(Akk, rp, qm, qn);
  if (k > 0) {
    const float* Lk = A + kk * rp + kk - NB;  // L_{k,k-1}
    const f32x16 acc = mm_quad<false, true>(Lk, rp, Lk, rp, qm, qn);
#pragma unroll
    for (int v = 0; v < 16; ++v) t[v] -= acc[v];
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) sm.T[qrow(qm, v) * TS + qcol(qn)] = t[v];
}

// Work beside a diagonal factorisation: out += sign X op(Y) over the four
// quadrants of a 64 x 64 tile (inactive for the workgroups that only factor).
struct SideJob {
  const float* X;
  const float* Y;
  float* out;
  int rp;
  float sign;
  bool active;
  bool first;  // out holds no earlier contribution: it is overwritten
};
template <bool TB>
__device__ __forceinline__ void side_quad(const SideJob& j, int qm, int qn) {
  const f32x16 prev = j.first ? zero16() : load_quad(j.out, j.rp, qm, qn);
  const f32x16 acc = mm_quad<false, TB>(j.X, j.rp, j.Y, j.rp, qm, qn);
  store_quad(acc, prev, j.out, j.rp, j.sign, qm, qn);
}

// Diagonal tile k (input T = A_kk - L_{k,k-1} L_{k,k-1}^T) with work beside
// it, in phases separated by barriers:
//   1. wave 0 forms T11 and factors it (L11, M11); waves 1, 2 form T21, T22;
//      wave 3 does side quadrant (0, 1);
//   2. L21 = T21 M11^T (four waves);
//   3. T22 - L21 L21^T and P = L21 M11 (four waves);
//   4. wave 0 factors T22 - L21 L21^T (L22, M22); waves 1, 2, 3 do side
//      quadrants (0, 0), (1, 0), (1, 1);
//   5. M21 = -M22 P (four waves).
// Ends with a barrier (M in sm.T, when M_LDS, and the side job's result are
// then visible to all waves of the workgroup).
template <bool M_LDS, bool WRITE_L, bool TB>
__device__ __forceinline__ void diag_step(const float* A, int rp, int k, float* M0, float* L0,
                                          int r_real, DevStats* st, StepSmem& sm,
                                          const SideJob& side, float* Mt0 = nullptr,
                                          const GramSrc& gsrc = GramSrc{}) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i16 = lane & 15, g = lane >> 4;
  const int bi = wave & 1, bj = wave >> 1;
  const int row0 = k * NB;
  const int ldm = M_LDS ? TS : rp;
  DiagSmem& d = sm.dg;
  const float* Tin = sm.T;
  uint64_t bad = 0;
  // 1
  diag_input(A, rp, k, sm, gsrc);
  if (wave == 0) {
    wave_lds_sync();  // T11 was written by other lanes of this wave
    diag_part1<M_LDS, WRITE_L>(sm.T, M0, L0, rp, row0, r_real, d, bad, Mt0);
  } else if (wave == 3 && side.active) {
    side_quad<TB>(side, 0, 1);
    __threadfence_block();
  }
  __syncthreads();
  // 2. L21 = T21 M11^T  (B(k, j) = M11[j][k] = Mc[k][j])
  {
    f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
    c = mm16([&](int s_) { return Tin[(32 + 16 * bi + i16) * TS + 4 * s_ + g]; },
             [&](int s_) { return d.Mc[4 * s_ + g][16 * bj + i16]; }, c);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * bi + 4 * g + v, col = 16 * bj + i16;
      d.Ls[row][col] = c[v];
      if (WRITE_L) L0[(int64_t)(32 + row) * rp + col] = c[v];
    }
  }
  __syncthreads();
  // 3. Ts = T22 - L21 L21^T, Ps = L21 M11  (M11[k][j] = Mc[j][k])
  {
    f32x4 c;
#pragma unroll
    for (int v = 0; v < 4; ++v) c[v] = Tin[(32 + 16 * bi + 4 * g + v) * TS + 32 + 16 * bj + i16];
    c = mm16([&](int s_) { return -d.Ls[16 * bi + i16][4 * s_ + g]; },
             [&](int s_) { return d.Ls[16 * bj + i16][4 * s_ + g]; }, c);
    f32x4 q = {0.0f, 0.0f, 0.0f, 0.0f};
    q = mm16([&](int s_) { return d.Ls[16 * bi + i16][4 * s_ + g]; },
             [&](int s_) { return d.Mc[16 * bj + i16][4 * s_ + g]; }, q);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      d.Ts[16 * bi + 4 * g + v][16 * bj + i16] = c[v];
      d.Ps[16 * bi + 4 * g + v][16 * bj + i16] = q[v];
    }
  }
  __syncthreads();
  // 4
  if (wave == 0) {
    diag_factor2<M_LDS, WRITE_L>(M0, L0, rp, row0, r_real, d, bad, Mt0);
  } else if (side.active) {
    side_quad<TB>(side, wave == 1 ? 0 : 1, wave == 3 ? 1 : 0);
    __threadfence_block();
  }
  __syncthreads();
  // 5. M21 = -M22 P  (M22[i][k] = Nc[k][i])
  {
    f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
    c = mm16([&](int s_) { return -d.Nc[4 * s_ + g][16 * bi + i16]; },
             [&](int s_) { return d.Ps[4 * s_ + g][16 * bj + i16]; }, c);
    if (M0) {
#pragma unroll
      for (int v = 0; v < 4; ++v) M0[(32 + 16 * bi + 4 * g + v) * ldm + 16 * bj + i16] = c[v];
    }
    if (Mt0) {  // M21^T: rows 16 bj + i16, columns 32 + 16 bi + 4 g .. + 3
      *(f32x4*)&Mt0[(int64_t)(16 * bj + i16) * rp + 32 + 16 * bi + 4 * g] = c;
    }
  }
  if (st && wave == 0 && bad && lane == 0)
    atomicMin(&st->potrf_info, row0 + __ffsll((unsigned long long)bad));
  __syncthreads();
}

// Launch k of the factorisation (see the file header). Workgroups, in order:
//   [k < R]  1 diagonal (writes M_kk), R-1-k panel tiles, k inverse-row tiles;
//   [k >= 1] 1 with want_L (writes L_{k-1,k-1}), n(n+1)/2 trailing tiles
//            (n = R-1-k), n k partial sums.
// With pin = px > 0 (a 256-workgroup grid: 32 workgroups on each of the 8
// XCDs), the ndiag workgroups that factor a diagonal tile are on the last px
// XCDs, one per CU, and the update workgroups on the others; the rest exit.
// A GEMM that leaves those XCDs free (GemmArgs::free_xcds = px) then never
// shares a CU with the diagonal work. The XCD comes from the hardware
// register: consecutive workgroups go to consecutive XCDs, but the first
// one's XCD depends on the queue's history.
__global__ __launch_bounds__(NT) void chol_step_kernel(float* A, float* M, int rp,
                                                       int k, int r_real, int want_L,
                                                       int upd_blocks, DevStats* st, int pin,
                                                       int ndiag, int dtiles, float* Mt,
                                                       GramSrc gsrc) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ __attribute__((aligned(16))) StepSmem sm;
  const int R = rp / NB;
  const int n = R - 1 - k;
  const int64_t kk = (int64_t)k * NB;
  const int qm = wave_qm(), qn = wave_qn();
  // the first launch reduces the Gram product into A (see the launcher)
  GramSrc g = gsrc;
  if (k != 0) g.part = nullptr;
  int b = blockIdx.x;
  // update tiles [t_lo, t_hi) with stride t_step for this workgroup (pinned:
  // the workgroups of the last pin XCDs take the first dtiles after their
  // diagonal work, which runs alone on those XCDs, and the others the rest)
  int t_lo = -1, t_hi = INT_MAX, t_step = upd_blocks;
  if (pin) {
    const int x = xcd_id(), i = b >> 3, x0 = 8 - pin;
    if (x >= x0) {
      const int di = i * pin + (x - x0);
      t_lo = di;
      t_hi = dtiles;
      t_step = kPinXcdCus * pin;
      b = di < ndiag ? di : INT_MAX;
    } else {
      const int u = i * x0 + x;
      if (u >= upd_blocks) return;
      t_lo = dtiles + u;
      b = INT_MAX;
    }
  }
  // The diagonal, panel, inverse-row and L_pp workgroups; returns whether
  // this workgroup was one of them.
  auto role = [&]() -> bool {
    if (k < R) {
      if (b == 0) {  // M_kk
        diag_step<false, false, true>(A, rp, k, M + kk * rp + kk, nullptr, r_real, st, sm,
                                      SideJob{nullptr, nullptr, nullptr, rp, 0.0f, false, false},
                                      Mt ? Mt + kk * rp + kk : nullptr, g);
        return true;
      }
      b -= 1;
      if (b < n) {  // panel tile (i, k)
        const int64_t i0 = (int64_t)(k + 1 + b) * NB;
        float* Aik = A + i0 * rp + kk;
        if (g.part) {  // A_i0 from the Gram's segments (read back below, after barriers)
          const f32x16 t = load_quad_gram(g, rp, (int)i0, 0, qm, qn);
          store_quad(t, zero16(), Aik, rp, 1.0f, qm, qn);
        }
        // A_ik -= L_{i,k-1} L_{k,k-1}^T beside the factorisation
        diag_step<true, false, true>(A, rp, k, sm.T, nullptr, r_real, nullptr, sm,
                                     SideJob{Aik - NB, A + kk * rp + kk - NB, Aik, rp, -1.0f,
                                             k > 0, false},
                                     nullptr, g);
        const f32x16 acc = mm_quad<false, true>(Aik, rp, sm.T, TS, qm, qn);  // (.) M_kk^T
        __syncthreads();  // every wave has read its operands before any overwrite
        store_quad(acc, zero16(), Aik, rp, 1.0f, qm, qn);
        return true;
      }
      b -= n;
      if (b < k) {  // inverse-row tile (k, j)
        const int64_t j0 = (int64_t)b * NB;
        float* Mkj = M + kk * rp + j0;
        // S_kj += L_{k,k-1} M_{k-1,j} beside the factorisation; for j = k-1
        // this is the only term, so the tile is overwritten
        diag_step<true, false, false>(
            A, rp, k, sm.T, nullptr, r_real, nullptr, sm,
            SideJob{A + kk * rp + kk - NB, M + (kk - NB) * rp + j0, Mkj, rp, 1.0f, true,
                    b == k - 1});
        const f32x16 acc = mm_quad<false, false>(sm.T, TS, Mkj, rp, qm, qn);  // M_kk S_kj
        __syncthreads();
        store_quad(acc, zero16(), Mkj, rp, -1.0f, qm, qn);
        if (Mt) store_quad_t(acc, Mt + j0 * rp + kk, rp, -1.0f, qm, qn);
        return true;
      }
      b -= k;
    }
    if (k >= 1 && want_L) {
      if (b == 0) {  // L_pp
        const int64_t pq = (int64_t)(k - 1) * NB;
        diag_step<false, true, true>(A, rp, k - 1, nullptr, A + pq * rp + pq, r_real, nullptr,
                                     sm, SideJob{nullptr, nullptr, nullptr, rp, 0.0f, false, false});
        return true;
      }
      b -= 1;
    }
    return false;
  };
  if (role() && !pin) return;
  if (g.part) {
    // The rest of the Gram reduction: every lower 64 x 64 tile (i, j) but
    // the panel tiles (i, 0), i > 0, with the diagonal tiles in full.
    int t = pin ? t_lo : b;
    const int nred = R * (R + 1) / 2 - (R - 1);
    for (; t < nred && t < t_hi; t += t_step) {
      // t = 0: tile (0, 0); t = 1 + u: the u-th lower tile of rows and
      // columns 1 .. R-1
      int ii = 0, jj = 0;
      if (t > 0) {
        tri_index(t - 1, ii, jj);
        ++ii;
        ++jj;
      }
      const f32x16 v = load_quad_gram(g, rp, ii * NB, jj * NB, qm, qn);
      store_quad(v, zero16(), A + (int64_t)ii * NB * rp + jj * NB, rp, 1.0f, qm, qn);
    }
    return;
  }
  if (k < 1) return;
  const int p = k - 1;
  const int64_t pp = (int64_t)p * NB;
  // The update tiles of step p are spread over upd_blocks workgroups, each
  // taking every upd_blocks-th tile, so that a launch needs few enough
  // workgroups to be resident at once beside a concurrently running GEMM.
  const int nT = n > 0 ? n * (n + 1) / 2 : 0;
  const int nS = n > 0 ? n * k : 0;
  // Global tile index t over the two ranges; a workgroup takes t = first,
  // first + step, ... below t_hi. Inside the loops the row stride is re-read
  // through an empty asm, so the per-lane 64-bit fragment offsets are formed
  // per tile rather than hoisted out of the loop, where they would hold ~100
  // extra registers.
  int t = pin ? t_lo : b;
  const int eT = min(nT, t_hi);
  for (; t < eT; t += t_step) {  // trailing tile (i, j), i >= j > k
    int ld = rp;
    asm volatile("" : "+s"(ld));
    int ii, jj;
    tri_index(t, ii, jj);
    const int64_t i0 = (int64_t)(k + 1 + ii) * NB, j0 = (int64_t)(k + 1 + jj) * NB;
    const f32x16 prev = load_quad(A + i0 * ld + j0, ld, qm, qn);
    const f32x16 acc = mm_quad<false, true>(A + i0 * ld + pp, ld, A + j0 * ld + pp, ld, qm, qn);
    store_quad(acc, prev, A + i0 * ld + j0, ld, -1.0f, qm, qn);
  }
  if (t < nT) return;  // stopped by t_hi
  const int eS = min(nS, t_hi - nT);
  for (t -= nT; t < eS; t += t_step) {  // partial sum S_ij += L_ip M_pj, i > k, j < k
    int ld = rp;
    asm volatile("" : "+s"(ld));
    const int jt = t % k;
    const int64_t i0 = (int64_t)(k + 1 + t / k) * NB, j0 = (int64_t)jt * NB;
    // S_ij's first term is the one of step p = j
    const f32x16 prev = jt == p ? zero16() : load_quad(M + i0 * ld + j0, ld, qm, qn);
    const f32x16 acc = mm_quad<false, false>(A + i0 * ld + pp, ld, M + pp * ld + j0, ld, qm, qn);
    store_quad(acc, prev, M + i0 * ld + j0, ld, 1.0f, qm, qn);
  }
}

__global__ void zero_upper_kernel(float* A, int rp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rp * rp) return;
  const int i = (int)(idx / rp), j = (int)(idx % rp);
  if (j > i) A[idx] = 0.0f;
}

}  // namespace

// Update tiles per launch that the workgroups of the diagonal XCDs take
// after their diagonal work (pinned mode), measured best: with one XCD the
// first 64 (the other XCDs, beside the GEMM, take the rest); with two, all
// of them (the chain keeps to its two XCDs, the GEMM has the other six to
// itself). NQ_PIN_DIAG_TILES overrides it.
int pin_diag_tiles(int px) {
  static const int d = [] {
    const char* e = std::getenv("NQ_PIN_DIAG_TILES");
    return e ? std::max(0, std::atoi(e)) : -1;
  }();
  return d >= 0 ? d : px == 1 ? 64 : INT_MAX;
}

int cholesky_pin_xcds(int rp, bool want_L) {
  if (rp % NB) return 0;
  const int ndiag = rp / NB + (want_L ? 1 : 0);
  for (int px = 1; px <= kPinMaxXcds; ++px)
    if (ndiag <= kPinXcdCus * px) return px;
  return 0;
}

hipError_t launch_cholesky_inverse(float* A, float* M, int rp, int r_real,
                                   DevStats* st, bool want_L, bool zero_m, hipStream_t s,
                                   int pin, float* Mt, GramSrc src) {
  if (rp % NB) return hipErrorInvalidValue;
  if (src.part && (want_L || rp % 128 || src.L <= 0)) return hipErrorInvalidValue;
  if (pin < 0 || pin > kPinMaxXcds) return hipErrorInvalidValue;
  if (pin && (cholesky_pin_xcds(rp, want_L) == 0 || cholesky_pin_xcds(rp, want_L) > pin))
    return hipErrorInvalidValue;
  const int R = rp / NB;
  if (zero_m) {
    hipError_t e = launch_zero(M, (size_t)rp * rp, s);
    if (e != hipSuccess) return e;
  }
  for (int k = 0; k <= R; ++k) {
    const int n = R - 1 - k;
    int nb = k < R ? 1 + n + k : 0;  // diagonal, panel and inverse-row workgroups
    int upd = 0, upd_tiles = 0;
    // launch 0 with src: the update workgroups reduce the Gram tiles the
    // diagonal and panel ones do not (the diagonal XCDs, busy with those, take none)
    const bool red = k == 0 && src.part;
    if (k >= 1 || red) {
      nb += k >= 1 && want_L ? 1 : 0;
      const int tiles = red ? 1 + (R - 1) * R / 2 : n > 0 ? n * (n + 1) / 2 + n * k : 0;
      upd = upd_tiles = tiles;
      if (pin) {
        upd = std::min(tiles, kPinGrid - kPinXcdCus * pin);
      } else {
        const int cap = chol_launch_cap();
        if (cap > 0 && nb + upd > cap)
          upd = std::max(cap - nb, std::min(tiles, kCholMinUpdBlocks));
        upd = std::min(upd, tiles);
      }
    }
    if (nb + upd > 0)
      hipLaunchKernelGGL(chol_step_kernel, dim3(pin ? kPinGrid : nb + upd), dim3(NT), 0, s, A, M,
                         rp, k, r_real, want_L ? 1 : 0, std::max(upd, 1), st,
                         pin, nb, pin && !red ? std::min(upd_tiles, pin_diag_tiles(pin)) : 0,
                         Mt, src);
  }
  if (!want_L) return hipGetLastError();
  const int64_t tot = (int64_t)rp * rp;
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, A, rp);
  return hipGetLastError();
}

}  // namespace nq
