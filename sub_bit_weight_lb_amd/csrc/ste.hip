// STE refinement of a factorised layer (NanoQuant digest, section
// 方法步骤详情, stage 2 step (3): U, V, s1, s2 optimised jointly with a
// straight-through estimator against the MSE of the quantised output;
// section 复现评估: lr 1e-4 -> 1e-6, cosine schedule, Adam-style training).
//
// One step on a batch X (T tokens x n), target Y = X W^T (T x m):
//   A = X diag(s2) (and A^T)          ste_stage_kernel (rows gathered by index)
//   P = A S_V (and P^T)               sign GEMM (signmm.hip), C and C^T
//   Q = P S_U^T                       sign GEMM
//   E = Q diag(s1) - Y, G = 2E/(T m)  ste_loss_kernel: loss and ds1 partials,
//   dQ = G diag(s1) (and dQ^T)          dQ and dQ^T
//   dU = dQ^T P                       fp32 tiled GEMM
//   dP = dQ S_U (and dP^T)            sign GEMM, C and C^T
//   dV = A^T dP                       fp32 tiled GEMM
//   dA = dP S_V^T                     sign GEMM
//   ds2_j = sum_t dA_tj X_tj          ste_ds2_kernel (partials)
//   column partial sums -> ds1, ds2   ste_colsum_kernel (fixed order)
//   Adam on U, V, s1, s2              ste_adam_kernel
//   S_U, S_U^T, S_V, S_V^T            ste_signs_kernel (sign(x >= 0) = +1,
//                                     zero in the padding)
// The sign matrices are exact +-1 (stored in fp32): the four products with
// one run on the bf16 matrix cores with the other factor split into three
// exact bf16 terms (every product exact, fp32 accumulation), the two
// without on the fp32 matrix-core GEMM of the ADMM path. Every reduction
// runs in a fixed order.
#include "common.h"

#include <algorithm>

namespace nq {
namespace {

// S (rows_pad x rp) = sign(F) for i < rows, k < r, else 0; St = S^T
// (rp x rows_pad). 32 x 32 tiles, grid (rp / 32, rows_pad / 32).
__global__ __launch_bounds__(256) void ste_signs_kernel(const float* __restrict__ F, int64_t rows,
                                                        int64_t r, int64_t rp, int64_t rows_pad,
                                                        float* __restrict__ S,
                                                        float* __restrict__ St) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * 32, i0 = (int64_t)blockIdx.y * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t i = i0 + ty + 8 * q, k = k0 + tx;
    const float v = (i < rows && k < r) ? (F[i * rp + k] >= 0.0f ? 1.0f : -1.0f) : 0.0f;
    S[i * rp + k] = v;
    tile[ty + 8 * q][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) St[(k0 + ty + 8 * q) * rows_pad + i0 + tx] = tile[tx][ty + 8 * q];
}

// A (tp x np) = X[idx[t]] * s2 for t < T, j < n, else 0; At = A^T (np x tp)
__global__ __launch_bounds__(256) void ste_stage_kernel(const float* __restrict__ X, int64_t ldx,
                                                        const int32_t* __restrict__ idx, int64_t T,
                                                        int64_t n, const float* __restrict__ s2,
                                                        int64_t np_, int64_t tp,
                                                        float* __restrict__ A,
                                                        float* __restrict__ At) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t j0 = (int64_t)blockIdx.x * 32, t0 = (int64_t)blockIdx.y * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + ty + 8 * q, j = j0 + tx;
    float v = 0.0f;
    if (t < T && j < n) {
      const int64_t row = idx ? (int64_t)idx[t] : t;
      v = X[row * ldx + j] * s2[j];
    }
    A[t * np_ + j] = v;
    tile[ty + 8 * q][tx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) At[(j0 + ty + 8 * q) * tp + t0 + tx] = tile[tx][ty + 8 * q];
}

// Per 32 x 32 tile of Q (tp x mp): E = Q s1 - Y (0 outside T x m),
// G = inv E; dQ = G s1 into dQ (tp x mp) and dQt (mp x tp); column partial
// sums of G Q into ds1p[tile row][col]; the tile's sum of E^2 into
// lossp[tile row * (mp / 32) + tile col] (fp64). Sums over a column run
// over its 32 rows in order (8 row groups of 4, combined in group order).
__global__ __launch_bounds__(256) void ste_loss_kernel(
    const float* __restrict__ Q, const float* __restrict__ Y, int64_t ldy,
    const int32_t* __restrict__ idx, int64_t T, int64_t m, const float* __restrict__ s1,
    float inv, int64_t mp, int64_t tp, float* __restrict__ dQ, float* __restrict__ dQt,
    float* __restrict__ ds1p, double* __restrict__ lossp) {
  __shared__ float tile[32][33];
  __shared__ float cs[8][32];
  __shared__ double es[256];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t i0 = (int64_t)blockIdx.x * 32, t0 = (int64_t)blockIdx.y * 32;
  const int64_t i = i0 + tx;
  const float s = i < m ? s1[i] : 0.0f;
  float c = 0.0f;
  double e2 = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * ty + q;
    float g = 0.0f, qv = 0.0f;
    if (t < T && i < m) {
      qv = Q[t * mp + i];
      const int64_t row = idx ? (int64_t)idx[t] : t;
      const float e = qv * s - Y[row * ldy + i];
      e2 += (double)e * (double)e;
      g = inv * e;
    }
    c += g * qv;
    const float d = g * s;
    dQ[t * mp + i] = d;
    tile[4 * ty + q][tx] = d;
  }
  cs[ty][tx] = c;
  es[threadIdx.x] = e2;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) dQt[(i0 + ty + 8 * q) * tp + t0 + tx] = tile[tx][ty + 8 * q];
  if (ty == 0) {
    float a = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) a += cs[g][tx];
    ds1p[blockIdx.y * mp + i] = a;
  }
  if (threadIdx.x == 0) {
    double a = 0.0;
    for (int k = 0; k < 256; ++k) a += es[k];
    lossp[blockIdx.y * (mp / 32) + blockIdx.x] = a;
  }
}

// ds2p[tile row][j] = sum over the tile's 32 rows t < T of dA_tj X[idx t]_j
__global__ __launch_bounds__(256) void ste_ds2_kernel(const float* __restrict__ dA,
                                                      const float* __restrict__ X, int64_t ldx,
                                                      const int32_t* __restrict__ idx, int64_t T,
                                                      int64_t n, int64_t np_,
                                                      float* __restrict__ ds2p) {
  __shared__ float cs[8][32];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t j = (int64_t)blockIdx.x * 32 + tx, t0 = (int64_t)blockIdx.y * 32;
  float c = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = t0 + 4 * ty + q;
    if (t < T && j < n) {
      const int64_t row = idx ? (int64_t)idx[t] : t;
      c += dA[t * np_ + j] * X[row * ldx + j];
    }
  }
  cs[ty][tx] = c;
  __syncthreads();
  if (ty == 0) {
    float a = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) a += cs[g][tx];
    ds2p[blockIdx.y * np_ + j] = a;
  }
}

// out[c] = sum_p part[p][c] (fp64 accumulation) for 32 columns per
// workgroup: thread (c, g) sums the partials p = g, g + 8, ... in order,
// then the 8 group sums are added in group order
__global__ __launch_bounds__(256) void ste_colsum_kernel(const float* __restrict__ part,
                                                         int nparts, int64_t cols,
                                                         float* __restrict__ out) {
  __shared__ double cs[8][32];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t c = (int64_t)blockIdx.x * 32 + tx;
  double a = 0.0;
  if (c < cols)
    for (int p = ty; p < nparts; p += 8) a += part[(int64_t)p * cols + c];
  cs[ty][tx] = a;
  __syncthreads();
  if (ty == 0 && c < cols) {
    double t = 0.0;
#pragma unroll
    for (int g = 0; g < 8; ++g) t += cs[g][tx];
    out[c] = (float)t;
  }
}

// loss[0] = sum of the tile partials / count: one workgroup of 1024
// threads, thread k summing k, k + 1024, ... in order, then a fixed tree
__global__ __launch_bounds__(1024) void ste_lossum_kernel(const double* __restrict__ part,
                                                          int64_t n, double count,
                                                          double* __restrict__ loss) {
  __shared__ double red[1024];
  double a = 0.0;
  for (int64_t k = threadIdx.x; k < n; k += 1024) a += part[k];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = red[0] / count;
}

// Adam on p (rows x cols of a rows_pad x ld array; only i < rows, k < cols
// move): m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
// p -= lr (m / c1) / (sqrt(v / c2) + eps), c1 = 1 - b1^t, c2 = 1 - b2^t.
__global__ void ste_adam_kernel(float* __restrict__ p, const float* __restrict__ g,
                                float* __restrict__ mo, float* __restrict__ vo, int64_t rows,
                                int64_t cols, int64_t ld, float lr, float b1, float b2, float c1,
                                float c2, float eps) {
  const int64_t total = rows * cols;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = (q / cols) * ld + q % cols;
    const float gv = g[e];
    const float mv = b1 * mo[e] + (1.0f - b1) * gv;
    const float vv = b2 * vo[e] + (1.0f - b2) * gv * gv;
    mo[e] = mv;
    vo[e] = vv;
    p[e] -= lr * (mv / c1) / (sqrtf(vv / c2) + eps);
  }
}

unsigned grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, 16384));
}

}  // namespace

hipError_t launch_ste_signs(const float* F, int64_t rows, int64_t r, int64_t rp, int64_t rows_pad,
                            float* S, float* St, hipStream_t s) {
  if (rp % 32 || rows_pad % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ste_signs_kernel, dim3((unsigned)(rp / 32), (unsigned)(rows_pad / 32)),
                     dim3(256), 0, s, F, rows, r, rp, rows_pad, S, St);
  return hipGetLastError();
}

hipError_t launch_ste_stage(const float* X, int64_t ldx, const int32_t* idx, int64_t T, int64_t n,
                            const float* s2, int64_t np_, int64_t tp, float* A, float* At,
                            hipStream_t s) {
  if (np_ % 32 || tp % 32 || tp / 32 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ste_stage_kernel, dim3((unsigned)(np_ / 32), (unsigned)(tp / 32)), dim3(256),
                     0, s, X, ldx, idx, T, n, s2, np_, tp, A, At);
  return hipGetLastError();
}

hipError_t launch_ste_loss(const float* Q, const float* Y, int64_t ldy, const int32_t* idx,
                           int64_t T, int64_t m, const float* s1, int64_t mp, int64_t tp,
                           float* dQ, float* dQt, float* ds1p, double* lossp, float* ds1,
                           double* loss, hipStream_t s) {
  if (mp % 32 || tp % 32 || tp / 32 > 65535) return hipErrorInvalidValue;
  const float inv = (float)(2.0 / ((double)T * (double)m));
  hipLaunchKernelGGL(ste_loss_kernel, dim3((unsigned)(mp / 32), (unsigned)(tp / 32)), dim3(256),
                     0, s, Q, Y, ldy, idx, T, m, s1, inv, mp, tp, dQ, dQt, ds1p, lossp);
  hipLaunchKernelGGL(ste_colsum_kernel, dim3((unsigned)(mp / 32)), dim3(256), 0, s, ds1p,
                     (int)(tp / 32), mp, ds1);
  hipLaunchKernelGGL(ste_lossum_kernel, dim3(1), dim3(1024), 0, s, lossp, (tp / 32) * (mp / 32),
                     (double)T * (double)m, loss);
  return hipGetLastError();
}

hipError_t launch_ste_ds2(const float* dA, const float* X, int64_t ldx, const int32_t* idx,
                          int64_t T, int64_t n, int64_t np_, int64_t tp, float* ds2p, float* ds2,
                          hipStream_t s) {
  if (np_ % 32 || tp % 32 || tp / 32 > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(ste_ds2_kernel, dim3((unsigned)(np_ / 32), (unsigned)(tp / 32)), dim3(256), 0,
                     s, dA, X, ldx, idx, T, n, np_, ds2p);
  hipLaunchKernelGGL(ste_colsum_kernel, dim3((unsigned)(np_ / 32)), dim3(256), 0, s, ds2p,
                     (int)(tp / 32), np_, ds2);
  return hipGetLastError();
}

hipError_t launch_ste_adam(float* p, const float* g, float* m, float* v, int64_t rows,
                           int64_t cols, int64_t ld, float lr, float b1, float b2, float c1,
                           float c2, float eps, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(ste_adam_kernel, dim3(grid_for(rows * cols)), dim3(256), 0, s, p, g, m, v,
                     rows, cols, ld, lr, b1, b2, c1, c2, eps);
  return hipGetLastError();
}

}  // namespace nq
