// Gram kernels: G = A^T A + rho I (the system matrix V^T V + rho I of the
// regularised solve, NanoQuant digest section 核心方法 step (a)), and the
// same kernel with a triangular K range for G^-1 = M^T M with M = L^-1 lower
// triangular (applying both triangular solves at once).
//
// syrk_partial: one workgroup per (lower 128 x 128 output tile, K chunk).
// 256 threads = 2 x 2 waves of 64 x 64 (2 x 2 blocks of the 32x32x2 fp32
// MFMA). Both column strips of A are staged transposed in LDS ([col][k],
// k contiguous) so every fragment is one ds_read_b128 (same K permutation as
// the GEMM). Partial tiles of all chunks are summed in a fixed order by
// gram_reduce, so the result is deterministic.
#include "common.h"

namespace nq {
namespace {

constexpr int TS = 128, BK = 16, NT = 256;
constexpr int LDS_S = BK + 4;

__global__ __launch_bounds__(NT) void syrk_partial_kernel(const float* __restrict__ A, int64_t lda,
                                                          int K, int rp, int kchunk, int tri,
                                                          float* __restrict__ part) {
  // the Gram heads the r x r chain, the critical path of an ADMM half: its
  // waves win issue arbitration against co-resident GEMM waves
  __builtin_amdgcn_s_setprio(3);
  __shared__ __attribute__((aligned(16))) float Si[2][TS * LDS_S];
  __shared__ __attribute__((aligned(16))) float Sj[2][TS * LDS_S];

  // lower-triangle tile index -> (I, J), I >= J
  const int t = blockIdx.x;
  int I = (int)((sqrtf(8.0f * t + 1.0f) - 1.0f) * 0.5f);
  while ((I + 1) * (I + 2) / 2 <= t) ++I;
  while (I * (I + 1) / 2 > t) --I;
  const int J = t - I * (I + 1) / 2;
  const int c = blockIdx.y;
  int k0 = c * kchunk;
  const int k1 = min(K, k0 + kchunk);
  if (tri) k0 = max(k0, I * TS);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int col = tid & (TS - 1), q0 = tid >> 7;

  const float* __restrict__ Ai = A + (int64_t)I * TS + col;
  const float* __restrict__ Aj = A + (int64_t)J * TS + col;
  // each thread stages column `col`, k quads q0 + 2 j of the BK-row slice
  constexpr int NQ = BK / 8;  // quads per thread
  float ri[4 * NQ], rj[4 * NQ];
  auto gload = [&](int kb) {
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t k = kb + (q0 + 2 * j) * 4 + e;
        ri[j * 4 + e] = Ai[k * lda];
        rj[j * 4 + e] = Aj[k * lda];
      }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      f32x4 vi = {ri[j * 4], ri[j * 4 + 1], ri[j * 4 + 2], ri[j * 4 + 3]};
      f32x4 vj = {rj[j * 4], rj[j * 4 + 1], rj[j * 4 + 2], rj[j * 4 + 3]};
      *(f32x4*)&Si[buf][col * LDS_S + (q0 + 2 * j) * 4] = vi;
      *(f32x4*)&Sj[buf][col * LDS_S + (q0 + 2 * j) * 4] = vj;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  const int nk = k1 > k0 ? (k1 - k0) / BK : 0;
  if (nk > 0) {
    gload(k0);
    sstore(0);
  }
  __syncthreads();
  const int ioff = (wm * 64 + l32) * LDS_S + 4 * half;
  const int joff = (wn * 64 + l32) * LDS_S + 4 * half;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(k0 + (kt + 1) * BK);
    const float* si = Si[buf] + ioff;
    const float* sj = Sj[buf] + joff;
#pragma unroll
    for (int kc = 0; kc < BK; kc += 8) {
      f32x4 af[2], bf[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = *(const f32x4*)&si[a * 32 * LDS_S + kc];
#pragma unroll
      for (int b = 0; b < 2; ++b) bf[b] = *(const f32x4*)&sj[b * 32 * LDS_S + kc];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a][s], bf[b][s], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  float* out = part + (int64_t)c * rp * rp;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = I * TS + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        const int cc = J * TS + wn * 64 + b * 32 + l32;
        out[(int64_t)row * rp + cc] = acc[a][b][v];
      }
}

// Full symmetric G from the lower triangles of the partial tiles.
// 32 x 32 output tiles, 32 x 8 threads; upper tiles read the mirrored lower
// tile and transpose it through LDS; diagonal tiles pick per element.
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part,
                                                          int nchunks, int rp, float rho,
                                                          float* __restrict__ G, int64_t ldg) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ float tile[32][33];
  const int ti = blockIdx.y, tj = blockIdx.x;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t stride = (int64_t)rp * rp;
  const int si = ti >= tj ? ti : tj;  // source tile (lower triangle)
  const int sj = ti >= tj ? tj : ti;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = ty + 8 * q;
    const int64_t src = (int64_t)(si * 32 + r) * rp + sj * 32 + tx;
    float acc = 0.0f;
    for (int c = 0; c < nchunks; ++c) acc += part[c * stride + src];
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

hipError_t launch_syrk_partial(const float* A, int64_t lda, int K, int rp, int kchunk,
                               bool tri_kstart, float* part, hipStream_t s) {
  if (rp % TS || K % BK || kchunk % BK || kchunk <= 0) return hipErrorInvalidValue;
  const int R = rp / TS;
  const int nchunks = (K + kchunk - 1) / kchunk;
  dim3 grid(R * (R + 1) / 2, nchunks), block(NT);
  hipLaunchKernelGGL(syrk_partial_kernel, grid, block, 0, s, A, lda, K, rp, kchunk,
                     tri_kstart ? 1 : 0, part);
  return hipGetLastError();
}

hipError_t launch_gram_reduce(const float* part, int nchunks, int rp, float rho, float* G,
                              int64_t ldg, hipStream_t s) {
  if (rp % 32) return hipErrorInvalidValue;
  dim3 grid(rp / 32, rp / 32), block(256);
  hipLaunchKernelGGL(gram_reduce_kernel, grid, block, 0, s, part, nchunks, rp, rho, G, ldg);
  return hipGetLastError();
}

}  // namespace nq
