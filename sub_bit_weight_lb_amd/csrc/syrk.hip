// Gram reduction: G = sum of each tile's K segments (stream-K partials) + rho I,
// the system matrix V^T V + rho I of the regularised solve (NanoQuant
// digest, section 核心方法 step (a)). The partial tiles (lower triangle only)
// come from gram_nt_kernel in gemm.hip; they are summed in a fixed order,
// so the result is deterministic, and written full-symmetric.
#include "common.h"

#include <hip/hip_ext.h>

namespace nq {
namespace {

// G from the partial tiles. Workgroup (q, t): rows 32 q .. 32 q + 31 of
// lower Gram tile t = I (I + 1) / 2 + J. Each thread loads its 4 float4s
// from every segment at once, sums them in slot order, and stores the strip
// into G (+ rho on the diagonal; in a diagonal tile only its lower half);
// the mirror above the diagonal (all of it if `full`, else inside the
// 64 x 64 diagonal blocks) goes through LDS as 128 rows of 32.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part,
                                                          GramSteps gs, int L, int rp, float rho,
                                                          int full, float* __restrict__ G,
                                                          int64_t ldg) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ float tile[32][129];
  const int t = blockIdx.y;
  int I = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
  while (I * (I + 1) / 2 > t) --I;
  while ((I + 1) * (I + 2) / 2 <= t) ++I;
  const int J = t - I * (I + 1) / 2;
  const int64_t t0 = gs.tile_start(I, J);
  const int nseg = (int)((t0 + gs.len(I) - 1) / L - t0 / L) + 1;
  const int64_t stride = (int64_t)rp * rp;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int r0 = I * 128 + blockIdx.x * 32, c0 = J * 128;
  const int gj = c0 + tx * 4;
  f32x4 v[4];
  {
    const float* src = part + (int64_t)(r0 + ty) * rp + gj;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = *(const f32x4*)(src + (int64_t)8 * k * rp);
    for (int c = 1; c < nseg; ++c) {
      f32x4 w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = *(const f32x4*)(src + c * stride + (int64_t)8 * k * rp);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] += w[k];
    }
  }
  const bool diag = I == J;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int gi = r0 + ty + 8 * k;
    float* dst = G + (int64_t)gi * ldg + gj;
    if (!diag) {
      *(f32x4*)dst = v[k];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (gi == gj + e) dst[e] = v[k][e] + rho;
        else if (gi > gj + e) dst[e] = v[k][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[ty + 8 * k][tx * 4 + e] = v[k][e];
  }
  // mirror: rows c0 .. c0 + 127 of G, columns r0 .. r0 + 31
  // (an off-diagonal tile has no element inside a 64 x 64 diagonal block)
  if (!full && !diag) return;
  __syncthreads();
  const int gi = r0 + tx;
#pragma unroll 4
  for (int k = 0; k < 16; ++k) {
    const int cc = ty + 8 * k, gq = c0 + cc;
    if (gi > gq && (full || (gi >> 6) == (gq >> 6))) G[(int64_t)gq * ldg + gi] = tile[tx][cc];
  }
}

}  // namespace

hipError_t launch_gram_reduce(const float* part, int K, int rp, const GramPlan& p, float rho,
                              bool full, float* G, int64_t ldg, hipStream_t s, hipEvent_t done) {
  if (rp % 128 || K % 32 || p.steps <= 0) return hipErrorInvalidValue;
  const int R = rp / 128;
  dim3 grid(4, R * (R + 1) / 2), block(256);
  // `done` is recorded by the kernel's own completion (no marker of its own
  // between this kernel and the next one on s)
  hipExtLaunchKernelGGL(gram_reduce_kernel, grid, block, 0, s, nullptr, done, 0u, part,
                        GramSteps{K / 32, p.tri}, p.steps, rp, rho, full ? 1 : 0, G, ldg);
  return hipGetLastError();
}

}  // namespace nq
