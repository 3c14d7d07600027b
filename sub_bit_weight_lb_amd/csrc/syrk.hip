// Gram reduction: G = sum of each tile's K segments (stream-K partials) + rho I,
// the system matrix V^T V + rho I of the regularised solve (NanoQuant
// digest, section 核心方法 step (a)). The partial tiles (lower triangle only)
// come from gram_nt_kernel in gemm.hip; they are summed in a fixed order,
// so the result is deterministic, and written full-symmetric.
#include "common.h"

#include <hip/hip_ext.h>

namespace nq {
namespace {

// Full symmetric G from the lower triangles of the partial tiles.
// 32 x 32 output tiles, 32 x 8 threads; upper tiles read the mirrored lower
// tile and transpose it through LDS; diagonal tiles pick per element.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part,
                                                          GramSteps gs, int L, int rp, float rho,
                                                          int full, float* __restrict__ G,
                                                          int64_t ldg) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ float tile[32][33];
  const int ti = blockIdx.y, tj = blockIdx.x;
  // without `full`, only what the blocked Cholesky reads: the lower triangle
  // and the whole of each 64 x 64 diagonal block
  if (!full && ti < tj && (ti >> 1) != (tj >> 1)) return;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t stride = (int64_t)rp * rp;
  const int si = ti >= tj ? ti : tj;  // source tile (lower triangle)
  const int sj = ti >= tj ? tj : ti;
  // segments of the 128 x 128 Gram tile holding it: workgroups w0 .. w1
  const int I = si / 4, J = sj / 4;
  const int64_t t0 = gs.tile_start(I, J);
  const int nseg = (int)((t0 + gs.len(I) - 1) / L - t0 / L) + 1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = ty + 8 * q;
    const int64_t src = (int64_t)(si * 32 + r) * rp + sj * 32 + tx;
    float acc = 0.0f;
    for (int c = 0; c < nseg; ++c) acc += part[c * stride + src];
    tile[r][tx] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = ty + 8 * q;
    float v;
    if (ti > tj) v = tile[r][tx];
    else if (ti < tj) v = tile[tx][r];
    else v = (r >= tx) ? tile[r][tx] : tile[tx][r];
    const int gi = ti * 32 + r, gj = tj * 32 + tx;
    if (gi == gj) v += rho;
    G[(int64_t)gi * ldg + gj] = v;
  }
}

}  // namespace

hipError_t launch_gram_reduce(const float* part, int K, int rp, const GramPlan& p, float rho,
                              bool full, float* G, int64_t ldg, hipStream_t s, hipEvent_t done) {
  if (rp % 128 || K % 32 || p.steps <= 0) return hipErrorInvalidValue;
  dim3 grid(rp / 32, rp / 32), block(256);
  // `done` is recorded by the kernel's own completion (no marker of its own
  // between this kernel and the next one on s)
  hipExtLaunchKernelGGL(gram_reduce_kernel, grid, block, 0, s, nullptr, done, 0u, part,
                        GramSteps{K / 32, p.tri}, p.steps, rp, rho, full ? 1 : 0, G, ldg);
  return hipGetLastError();
}

}  // namespace nq
