// Iterative solve of the step-(a) system in place of the Cholesky factor
// (NanoQuant implementation blog, section 待办事项: its author replaced the
// Cholesky solve of LB-ADMM by a gradient-descent solver, slower than
// Cholesky under CUDA, faster on another GPU).
//
// Each row u of the factor minimises 1/2 u G u^T - u r^T, G = other^T other
// + rho I (symmetric positive definite), gradient g = u G - r. From the
// factor's previous value (warm start), a fixed number of steps per row:
//   steepest descent (exact step along d = -g), or
//   conjugate gradients: alpha = (g.g) / (d G d^T), u += alpha d,
//   g += alpha d G, beta = (g'.g') / (g.g), d = -g' + beta d.
// The products d G of all rows are one GEMM per step (the same tiled kernel
// as the solve, M x rp x rp); everything else is row-local and runs here:
//   itsolve_init_kernel: d = -g, delta = g.g (g from the GEMM u G - r);
//   itsolve_step_kernel: given d G, the step above, one pass over the row.
// A row whose denominator d G d^T is not > 0 takes no step (for a positive
// definite G that means a zero gradient); padded rows and columns are zero
// and stay zero.
//
// One workgroup per row, 256 threads, each holding NV float4 of every
// array (columns 4 (tid + 256 k)); sums over a row run per thread in k
// order, then over the wave by DPP, then over the 4 waves in order, so every
// row's reductions are fixed and the results bit-reproducible. HBM-bound:
// the step reads d, d G, u, g and writes u, g, d (28 bytes per element).
#include "common.h"

namespace nq {
namespace {

constexpr int kThreads = 256;

template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}
// sum over the wave in a fixed order, returned to every lane
__device__ inline float wave_sum(float v) {
  v = dpp_add<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xf>(v);  // row_mirror: every lane of a row holds its row's sum
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31: lane 63 holds the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// sum over the workgroup (4 waves, in wave order); red holds 4 floats; two
// barriers, so consecutive calls may reuse red
__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}
__device__ inline float dot4(f32x4 a, f32x4 b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

template <int NV>
__global__ __launch_bounds__(kThreads) void itsolve_init_kernel(const float* __restrict__ g,
                                                                float* __restrict__ d,
                                                                float* __restrict__ delta,
                                                                int rp) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* gr = g + row * rp;
  float* dr = d + row * rp;
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c = 4 * (threadIdx.x + kThreads * k);
    if (c < rp) {
      const f32x4 v = *(const f32x4*)&gr[c];
      s += dot4(v, v);
      *(f32x4*)&dr[c] = -v;
    }
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) delta[row] = s;
}

template <int NV, bool CG, bool LAST>
__global__ __launch_bounds__(kThreads) void itsolve_step_kernel(
    const float* __restrict__ Q, float* __restrict__ d, float* __restrict__ u,
    float* __restrict__ g, float* __restrict__ delta, int rp) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int64_t base = row * rp;
  f32x4 dv[NV], qv[NV];
  float den = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c = 4 * (threadIdx.x + kThreads * k);
    if (c < rp) {
      dv[k] = *(const f32x4*)&d[base + c];
      qv[k] = *(const f32x4*)&Q[base + c];
    } else {
      dv[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      qv[k] = dv[k];
    }
    den += dot4(dv[k], qv[k]);
  }
  den = block_sum(den, red);
  const float gg = delta[row];
  const float alpha = den > 0.0f ? gg / den : 0.0f;
  f32x4 gv[NV];
  float gg_new = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c = 4 * (threadIdx.x + kThreads * k);
    if (c < rp) {
      f32x4 uv = *(const f32x4*)&u[base + c];
      gv[k] = *(const f32x4*)&g[base + c];
      uv += alpha * dv[k];
      gv[k] += alpha * qv[k];
      *(f32x4*)&u[base + c] = uv;
      *(f32x4*)&g[base + c] = gv[k];
    } else {
      gv[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    gg_new += dot4(gv[k], gv[k]);
  }
  gg_new = block_sum(gg_new, red);
  if (threadIdx.x == 0) delta[row] = gg_new;
  if (LAST) return;
  const float beta = (CG && den > 0.0f && gg > 0.0f) ? gg_new / gg : 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int c = 4 * (threadIdx.x + kThreads * k);
    if (c < rp) *(f32x4*)&d[base + c] = beta * dv[k] - gv[k];
  }
}

template <int NV>
hipError_t step_nv(const float* Q, float* d, float* u, float* g, float* delta, int rows, int rp,
                   bool cg, bool last, hipStream_t s) {
  const dim3 grid(rows), block(kThreads);
  if (cg) {
    if (last) hipLaunchKernelGGL((itsolve_step_kernel<NV, true, true>), grid, block, 0, s, Q, d, u, g, delta, rp);
    else hipLaunchKernelGGL((itsolve_step_kernel<NV, true, false>), grid, block, 0, s, Q, d, u, g, delta, rp);
  } else {
    if (last) hipLaunchKernelGGL((itsolve_step_kernel<NV, false, true>), grid, block, 0, s, Q, d, u, g, delta, rp);
    else hipLaunchKernelGGL((itsolve_step_kernel<NV, false, false>), grid, block, 0, s, Q, d, u, g, delta, rp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_itsolve_init(const float* g, float* d, float* delta, int rows, int rp,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rp <= 0 || rp % 4 || rp > 4 * kThreads * 8) return hipErrorInvalidValue;
  const int nv = (rp + 4 * kThreads - 1) / (4 * kThreads);
  const dim3 grid(rows), block(kThreads);
  switch (nv) {
    case 1: hipLaunchKernelGGL(itsolve_init_kernel<1>, grid, block, 0, s, g, d, delta, rp); break;
    case 2: hipLaunchKernelGGL(itsolve_init_kernel<2>, grid, block, 0, s, g, d, delta, rp); break;
    case 3:
    case 4: hipLaunchKernelGGL(itsolve_init_kernel<4>, grid, block, 0, s, g, d, delta, rp); break;
    default: hipLaunchKernelGGL(itsolve_init_kernel<8>, grid, block, 0, s, g, d, delta, rp); break;
  }
  return hipGetLastError();
}

hipError_t launch_itsolve_step(const float* Q, float* d, float* u, float* g, float* delta,
                               int rows, int rp, bool cg, bool last, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rp <= 0 || rp % 4 || rp > 4 * kThreads * 8) return hipErrorInvalidValue;
  const int nv = (rp + 4 * kThreads - 1) / (4 * kThreads);
  switch (nv) {
    case 1: return step_nv<1>(Q, d, u, g, delta, rows, rp, cg, last, s);
    case 2: return step_nv<2>(Q, d, u, g, delta, rows, rp, cg, last, s);
    case 3:
    case 4: return step_nv<4>(Q, d, u, g, delta, rows, rp, cg, last, s);
    default: return step_nv<8>(Q, d, u, g, delta, rows, rp, cg, last, s);
  }
}

}  // namespace nq
