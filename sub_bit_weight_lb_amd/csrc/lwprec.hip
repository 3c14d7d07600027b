// Diagonal preconditioners from activation samples with Ledoit-Wolf
// shrinkage (NanoQuant digest, section 方法步骤详情, stage 1: statistics of
// every linear layer's activations, robust diagonal preconditioners by
// Ledoit-Wolf shrinkage; section 前置知识: a simplified diagonal K-FAC
// preconditioner; O. Ledoit and M. Wolf, J. Multivariate Analysis 88 (2004)
// for the estimator).
//
// For a sample Z (N tokens x p features), S = Z^T Z / N (uncentered, as
// K-FAC's factors), m = tr(S) / p, and with ||A||^2 = tr(A A^T) / p:
//   d2    = ||S - m I||^2 = (||S||_F^2 - p m^2) / p,
//   b2bar = (1/N^2) sum_k ||z_k z_k^T - S||^2
//         = (sum_k ||z_k||^4 - N ||S||_F^2) / (N^2 p)
//     (expanding the square: sum_k z_k^T S z_k = N ||S||_F^2),
//   shrinkage = min(b2bar, d2) / d2 (0 when d2 = 0),
//   D_jj = sqrt((1 - shrinkage) S_jj + shrinkage m).
// The samples arrive in chunks of rows. Per chunk:
//   lw_stage_kernel     Z (rows x p) -> Z^T (pp x kp, zero padded), so
//                       that the Gram reads K = tokens contiguously;
//   gram_nt_kernel /    the chunk's Z^T Z (fp32 MFMA, stream-K, the same
//   gram_reduce_kernel  kernels as the ADMM Gram), full symmetric;
//   lw_accum_kernel     S += that, in fp64;
//   lw_rownorm_kernel   ||z_k||^2 per row (fp64);
//   lw_q4_kernel        q4 += sum_k ||z_k||^4 in row order (one workgroup).
// Finalize: lw_norms_kernel (tr S and ||S||_F^2, partial sums per row
// block), lw_scalar_kernel (the scalars above, one workgroup, fixed order),
// lw_diag_kernel (D). Every sum runs in a fixed order: bit-reproducible.
#include "common.h"

namespace nq {
namespace {

__device__ inline double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// fixed-order sum over a 256-thread workgroup (waves in order)
__device__ inline double block_sum_d(double v, double* red) {
  v = wave_sum_d(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const double t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

// dst (pp x kp, ld kp) = Z^T for Z rows x p (ld ldz), zero where j >= p or
// k >= rows; grid (kp / 32, pp / 32), 256 threads, 32 x 32 tiles via LDS.
__global__ __launch_bounds__(256) void lw_stage_kernel(const float* __restrict__ Z, int64_t rows,
                                                       int64_t p, int64_t ldz,
                                                       float* __restrict__ dst, int64_t kp) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * 32, j0 = (int64_t)blockIdx.y * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t k = k0 + ty + 8 * q, j = j0 + tx;
    tile[ty + 8 * q][tx] = (k < rows && j < p) ? Z[k * ldz + j] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[(j0 + ty + 8 * q) * kp + k0 + tx] = tile[tx][ty + 8 * q];
}

// rn[k] = sum_j Z_kj^2 in fp64, one wave per row, lanes over columns then a
// fixed wave tree
__global__ __launch_bounds__(256) void lw_rownorm_kernel(const float* __restrict__ Z,
                                                         int64_t rows, int64_t p, int64_t ldz,
                                                         double* __restrict__ rn) {
  const int64_t k = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (k >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* z = Z + k * ldz;
  double s = 0.0;
  for (int64_t j = lane; j < p; j += 64) {
    const double v = z[j];
    s += v * v;
  }
  s = wave_sum_d(s);
  if (lane == 0) rn[k] = s;
}

// acc[0] += sum_k rn[k]^2 (one workgroup; thread t takes rows t, t + 256, ...)
__global__ __launch_bounds__(256) void lw_q4_kernel(const double* __restrict__ rn, int64_t rows,
                                                    double* __restrict__ acc) {
  __shared__ double red[4];
  double s = 0.0;
  for (int64_t k = threadIdx.x; k < rows; k += 256) s += rn[k] * rn[k];
  s = block_sum_d(s, red);
  if (threadIdx.x == 0) acc[0] += s;
}

// S (fp64) += G (fp32), n elements
__global__ void lw_accum_kernel(const float* __restrict__ G, double* __restrict__ S, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    S[i] += (double)G[i];
}

// part[b] = (sum of S_jj, sum of S_ij^2) over rows j of block b (8 rows per
// block, 256 threads)
constexpr int kNormRows = 8;
__global__ __launch_bounds__(256) void lw_norms_kernel(const double* __restrict__ S, int64_t pp,
                                                       double* __restrict__ part) {
  __shared__ double red[4];
  double tr = 0.0, fro = 0.0;
  for (int q = 0; q < kNormRows; ++q) {
    const int64_t j = (int64_t)blockIdx.x * kNormRows + q;
    if (j >= pp) break;
    const double* row = S + j * pp;
    for (int64_t i = threadIdx.x; i < pp; i += 256) fro += row[i] * row[i];
    if (threadIdx.x == 0) tr += row[j];
  }
  fro = block_sum_d(fro, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = tr;
    part[2 * blockIdx.x + 1] = fro;
  }
}

// out = {shrinkage, m, d2, b2bar, tr S, ||S||_F^2} of the normalised S
__global__ __launch_bounds__(256) void lw_scalar_kernel(const double* __restrict__ part,
                                                        int nblk, const double* __restrict__ q4,
                                                        double N, double p,
                                                        double* __restrict__ out) {
  __shared__ double red[4];
  double tr = 0.0, fro = 0.0;
  for (int b = threadIdx.x; b < nblk; b += 256) {
    tr += part[2 * b];
    fro += part[2 * b + 1];
  }
  tr = block_sum_d(tr, red);
  fro = block_sum_d(fro, red);
  if (threadIdx.x != 0) return;
  const double trn = tr / N, fron = fro / (N * N);
  const double m = trn / p;
  double d2 = (fron - p * m * m) / p;
  if (d2 < 0.0) d2 = 0.0;
  double b2bar = (q4[0] - N * fron) / (N * N * p);
  if (b2bar < 0.0) b2bar = 0.0;
  const double b2 = b2bar < d2 ? b2bar : d2;
  out[0] = d2 > 0.0 ? b2 / d2 : 0.0;
  out[1] = m;
  out[2] = d2;
  out[3] = b2bar;
  out[4] = trn;
  out[5] = fron;
}

// d_j = sqrt((1 - s) S_jj / N + s m), j < p
__global__ void lw_diag_kernel(const double* __restrict__ S, int64_t pp, int64_t p, double N,
                               const double* __restrict__ sc, float* __restrict__ d) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= p) return;
  const double s = sc[0], m = sc[1];
  d[j] = (float)sqrt((1.0 - s) * (S[j * pp + j] / N) + s * m);
}

}  // namespace

hipError_t launch_lw_stage(const float* Z, int64_t rows, int64_t p, int64_t ldz, float* Zt,
                           int64_t pp, int64_t kp, hipStream_t s) {
  if (pp % 32 || kp % 32 || pp < p || kp < rows || kp / 32 > 0x7fffffff || pp / 32 > 65535)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lw_stage_kernel, dim3((unsigned)(kp / 32), (unsigned)(pp / 32)), dim3(256),
                     0, s, Z, rows, p, ldz, Zt, kp);
  return hipGetLastError();
}

hipError_t launch_lw_q4(const float* Z, int64_t rows, int64_t p, int64_t ldz, double* rn,
                        double* q4, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(lw_rownorm_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, Z,
                     rows, p, ldz, rn);
  hipLaunchKernelGGL(lw_q4_kernel, dim3(1), dim3(256), 0, s, rn, rows, q4);
  return hipGetLastError();
}

hipError_t launch_lw_accum(const float* G, double* S, int64_t n, hipStream_t s) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(lw_accum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, G, S, n);
  return hipGetLastError();
}

int lw_norm_blocks(int64_t pp) { return (int)((pp + kNormRows - 1) / kNormRows); }

hipError_t launch_lw_finalize(const double* S, int64_t pp, int64_t p, double N, const double* q4,
                              double* part, double* scalars, float* d, hipStream_t s) {
  const int nb = lw_norm_blocks(pp);
  hipLaunchKernelGGL(lw_norms_kernel, dim3(nb), dim3(256), 0, s, S, pp, part);
  hipLaunchKernelGGL(lw_scalar_kernel, dim3(1), dim3(256), 0, s, part, nb, q4, N, (double)p,
                     scalars);
  hipLaunchKernelGGL(lw_diag_kernel, dim3((unsigned)((p + 255) / 256)), dim3(256), 0, s, S, pp, p,
                     N, scalars, d);
  return hipGetLastError();
}

}  // namespace nq
