// Blocked Cholesky factorisation with the inverse factor: G = L L^T and
// M = L^-1, for the ridge-regularised system matrix G = V^T V + rho I of the
// regularised solve (NanoQuant digest, section 核心方法, step (a): the linear
// system is solved through a Cholesky factorisation; the implementation blog,
// section 待办事项, names this factorisation as where LB-ADMM spends its time).
//
// One persistent launch per factorisation: a tile DAG over 64 x 64 tiles
// (task kinds and their order: chol_schedule.h). Workgroups take tasks in
// list order from an atomic ticket, wait for the flags of the task's inputs,
// run the task and set its output flags. Since every input is produced by a
// task earlier in the list, which some running workgroup has already taken,
// progress never depends on more than one workgroup being resident. Each
// wait is bounded in time; on expiry the kernel records an error in the
// device stats and every workgroup leaves, so the launch always ends.
//   diagonal tiles: outer-product elimination with register-resident 4 x 4
//   blocks, the same row operations applied to an identity block, giving
//   L_kk and M_kk = L_kk^-1 with one barrier per column;
//   off-diagonal tiles: 64 x 64 x 64 products on the 32x32x2 fp32 MFMA.
// The identity  sum_{l = j..i} L_il M_lj = delta_ij  gives
// M_ij = -M_ii sum_{l = j..i-1} L_il M_lj; the partial sums S_ij are kept in
// M's own tiles until row i of M is formed.
#include "chol_schedule.h"
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

__device__ void diag_factor(float* A, float* M, int rp, int k, int r_real, DevStats* st,
                            DiagSmem& sm) {
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
  // Outer loop over 4-wide block columns, inner 4 steps unrolled so that
  // every register index is a compile-time constant. Rows <= j and columns
  // <= j are masked arithmetically instead of branching.
  for (int J = 0; J < NB / 4; ++J) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * J + jj;
      const int buf = jj & 1;  // NB / 4 steps per J is even, so parity follows jj
      const float d = colbuf[buf][j];
      if (tid == 0) {
        dvec[j] = d;
        if (!(d > 0.0f && isfinite(d)) && (int)base + j < r_real)
          atomicMin(&st->potrf_info, (int)base + j + 1);
      }
      const float inv = 1.0f / d;
      const f32x4 li = *(const f32x4*)&colbuf[buf][4 * bi];
      const f32x4 cj = *(const f32x4*)&colbuf[buf][4 * bj];
      const f32x4 ej = *(const f32x4*)&erow[buf][4 * bj];
      float l[4], cm[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) l[a] = (4 * bi + a > j) ? li[a] * inv : 0.0f;
#pragma unroll
      for (int b = 0; b < 4; ++b) cm[b] = (4 * bj + b > j) ? cj[b] : 0.0f;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          Tr[a][b] = fmaf(-l[a], cm[b], Tr[a][b]);
          Er[a][b] = fmaf(-l[a], ej[b], Er[a][b]);
        }
      // publish column j + 1 of T and row j + 1 of E for the next step
      const int nb_ = (jj == 3) ? J + 1 : J;
      if (j + 1 < NB) {
        if (bj == nb_) {
#pragma unroll
          for (int a = 0; a < 4; ++a) colbuf[buf ^ 1][4 * bi + a] = Tr[a][(jj + 1) & 3];
        }
        if (bi == nb_) {
#pragma unroll
          for (int b = 0; b < 4; ++b) erow[buf ^ 1][4 * bj + b] = Er[(jj + 1) & 3][b];
        }
      }
      __syncthreads();
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

constexpr uint64_t kVerBits = 20;           // flag = epoch << 20 | version
constexpr uint64_t kTimeoutTicks = 200000000; // wall-clock ticks (2 s at 100 MHz)

__device__ inline void acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

// Thread 0 only: wait until *f >= target; false on timeout or a recorded error.
__device__ bool wait_flag(const uint64_t* f, uint64_t target, int* err) {
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const uint64_t v = __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= target) return true;
    if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    if (wall_clock64() - t0 > kTimeoutTicks) {
      atomicOr(err, 1);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Make this workgroup's global writes visible device-wide, then set flag
// `idx` (if >= 0) to base | version.
__device__ void publish(uint64_t* flags, int idx, uint64_t base, int version) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0 && idx >= 0)
    __hip_atomic_store(flags + idx, base | (uint64_t)version, __ATOMIC_RELEASE,
                       __HIP_MEMORY_SCOPE_AGENT);
}

struct CholDagArgs {
  float* A;
  float* M;
  int rp;
  int r_real;
  DevStats* st;
  const CholDevTask* tasks;
  int ntasks;
  int* ticket;
  const uint64_t* epoch;
  uint64_t* flags;
};

__global__ __launch_bounds__(NT) void chol_dag_kernel(CholDagArgs p) {
  __shared__ __attribute__((aligned(16))) float Xs[NB * LS];
  __shared__ __attribute__((aligned(16))) float Ys[NB * LS];
  __shared__ __attribute__((aligned(16))) DiagSmem dsm;
  __shared__ int s_ticket, s_ok;
  const int tid = threadIdx.x;
  const uint64_t base = (*p.epoch) << kVerBits;
  float* A = p.A;
  float* M = p.M;
  const int rp = p.rp;
  int* err = &p.st->sched_err;
  for (;;) {
    if (tid == 0) s_ticket = atomicAdd(p.ticket, 1);
    __syncthreads();
    const int t = s_ticket;
    if (t >= p.ntasks) break;
    const CholDevTask tk = p.tasks[t];
    if (tid == 0) {
      bool ok = true;
      for (int q = 0; q < 3 && ok; ++q)
        if (tk.dep[q] >= 0) ok = wait_flag(p.flags + tk.dep[q], base | (uint64_t)tk.dver[q], err);
      s_ok = ok;
    }
    __syncthreads();
    if (!s_ok) break;
    acquire_agent();
    const int64_t i0 = (int64_t)tk.i * NB, j0 = (int64_t)tk.j * NB, k0 = (int64_t)tk.k * NB;
    switch (tk.type) {
      case kTaskDiag: {
        int o = 0;
        if (tk.k >= 1) {
          const int64_t km = k0 - NB;
          float* Lk = A + k0 * rp + km;
          // L_{k,k-1} = A_{k,k-1} M_{k-1,k-1}^T, published at once
          block_mm<true>(Lk, M + km * rp + km, Lk, rp, 1.0f, 0.0f, Xs, Ys);
          publish(p.flags, tk.out[0], base, tk.over[0]);
          acquire_agent();
          // A_kk -= L_{k,k-1} L_{k,k-1}^T
          block_mm<true>(Lk, Lk, A + k0 * rp + k0, rp, -1.0f, 1.0f, Xs, Ys);
          __threadfence();
          __syncthreads();
          acquire_agent();
          o = 1;
        }
        diag_factor(A, M, rp, tk.k, p.r_real, p.st, dsm);
        publish(p.flags, tk.out[o], base, tk.over[o]);
        if (tid == 0 && tk.out[o + 1] >= 0)
          __hip_atomic_store(p.flags + tk.out[o + 1], base | (uint64_t)tk.over[o + 1],
                             __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      case kTaskPanelL: {
        float* Aik = A + i0 * rp + k0;
        block_mm<true>(Aik, M + k0 * rp + k0, Aik, rp, 1.0f, 0.0f, Xs, Ys);
        publish(p.flags, tk.out[0], base, tk.over[0]);
        break;
      }
      case kTaskPanelM: {
        float* Mkj = M + k0 * rp + j0;
        block_mm<false>(M + k0 * rp + k0, Mkj, Mkj, rp, -1.0f, 0.0f, Xs, Ys);
        publish(p.flags, tk.out[0], base, tk.over[0]);
        break;
      }
      case kTaskUpdA: {
        block_mm<true>(A + i0 * rp + k0, A + j0 * rp + k0, A + i0 * rp + j0, rp, -1.0f, 1.0f, Xs,
                       Ys);
        publish(p.flags, tk.out[0], base, tk.over[0]);
        break;
      }
      default: {  // kTaskUpdS
        block_mm<false>(A + i0 * rp + k0, M + k0 * rp + j0, M + i0 * rp + j0, rp, 1.0f, 1.0f, Xs,
                        Ys);
        publish(p.flags, tk.out[0], base, tk.over[0]);
        break;
      }
    }
  }
}

// Ticket to 0, epoch + 1, before each factorisation (stream-ordered).
__global__ void chol_dag_prep_kernel(int* ticket, uint64_t* epoch) {
  *ticket = 0;
  *epoch = *epoch + 1;
}

__global__ void zero_upper_kernel(float* A, int rp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rp * rp) return;
  const int i = (int)(idx / rp), j = (int)(idx % rp);
  if (j > i) A[idx] = 0.0f;
}

}  // namespace

hipError_t launch_cholesky_inverse(float* A, float* M, int rp, int r_real, DevStats* st,
                                   const CholDagWork& w, bool zero_upper_L, hipStream_t s) {
  if (rp % NB || w.R != rp / NB) return hipErrorInvalidValue;
  hipError_t e = launch_zero(M, (size_t)rp * rp, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chol_dag_prep_kernel, dim3(1), dim3(1), 0, s, w.ticket, w.epoch);
  CholDagArgs a{A, M, rp, r_real, st, (const CholDevTask*)w.tasks, w.ntasks, w.ticket, w.epoch,
                w.flags};
  const int grid = w.ntasks < w.grid ? w.ntasks : w.grid;
  hipLaunchKernelGGL(chol_dag_kernel, dim3(grid), dim3(NT), 0, s, a);
  if (!zero_upper_L) return hipGetLastError();
  const int64_t tot = (int64_t)rp * rp;
  hipLaunchKernelGGL(zero_upper_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, A, rp);
  return hipGetLastError();
}

}  // namespace nq
