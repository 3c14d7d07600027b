// fp32 MFMA GEMM C = A B (+ fused epilogue) for gfx950.
//
// Used for the right-hand side of the regularised solve, R = Wt V + rho (Z - Lam)
// (NanoQuant digest, section 核心方法, step (a)), and for applying the two
// triangular solves, U = R L^-T L^-1 = R G^-1, as one product with the
// symmetric inverse (epilogue also forms X = U + Lam for SVID, step (b)).
//
// Tiling: 256 x 128 block tile, BK = 32, 256 threads = 4 waves in a 2 x 2
// arrangement, each wave owning 128 x 64 = 4 x 2 blocks of
// v_mfma_f32_32x32x2_f32 (128 accumulators per lane). Double-buffered LDS,
// one barrier per K step, global loads of the next step issued before the
// current step's MFMAs, operand fragments of the next chunk of 8 k read from
// LDS while the current chunk's 32 MFMAs run.
//
// K ordering inside a chunk of 8: lane half h (lanes 32..63 are h = 1) feeds
// k = 4 h + s to MFMA step s = 0..3. Both tiles are stored k-contiguous in
// LDS (A as [m][k], B transposed to [n][k] while staging), so each fragment
// for 4 steps is a single ds_read_b128. Both operands use the same
// permutation, so each MFMA step still sums over a distinct pair of k.
// Row stride BK + 4 floats makes the 16-lane groups of a ds_read_b128 touch
// 64 distinct banks.
//
// Tile order: the hardware hands workgroups to the 8 XCDs round-robin, so
// workgroup b runs on XCD b % 8. Tiles are remapped so each XCD works on a
// contiguous range of row panels and shares their A rows in its own L2.
#include "common.h"

namespace nq {
namespace {

constexpr int BM = 256, BN = 128, BK = 32;
constexpr int LDS_S = BK + 4;  // row stride (floats) of both LDS tiles
constexpr int NT = 256;
constexpr int A_F4 = BM * BK / 4 / NT;   // float4 loads of A per thread (8)
constexpr int B_F1 = BK * BN / NT;       // scalar loads of B per thread (16)

template <int EPI>
__global__ __launch_bounds__(NT) void gemm_nn_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) float As[2][BM * LDS_S];
  __shared__ __attribute__((aligned(16))) float Bs[2][BN * LDS_S];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;

  const int tilesN = p.N / BN;
  const int nt = (p.M / BM) * tilesN;
  const int b = blockIdx.x;
  const int t = (nt % 8 == 0) ? (b % 8) * (nt / 8) + b / 8 : b;
  const int tm = t / tilesN, tn = t % tilesN;

  const float* __restrict__ Ag = p.A + (int64_t)tm * BM * p.lda;
  const float* __restrict__ Bg = p.B + (int64_t)tn * BN;

  // A: float4 idx = tid + NT i -> row idx / 8, k4 idx % 8.
  // B: thread owns column n = tid % 128 and k rows kq*4 .. kq*4+3 for
  //    kq = tid / 128 + 2 j (j = 0..3): four coalesced scalar row loads per
  //    quad, stored as one float4 of the transposed tile.
  f32x4 ra[A_F4];
  float rb[B_F1];
  const int bn = tid & (BN - 1), bq = tid >> 7;
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_F4; ++i) {
      const int idx = tid + NT * i;
      ra[i] = *(const f32x4*)(Ag + (int64_t)(idx >> 3) * p.lda + k0 + (idx & 7) * 4);
    }
#pragma unroll
    for (int j = 0; j < B_F1 / 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        rb[j * 4 + c] = Bg[(int64_t)(k0 + (bq + 2 * j) * 4 + c) * p.ldb + bn];
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_F4; ++i) {
      const int idx = tid + NT * i;
      *(f32x4*)&As[buf][(idx >> 3) * LDS_S + (idx & 7) * 4] = ra[i];
    }
#pragma unroll
    for (int j = 0; j < B_F1 / 4; ++j) {
      f32x4 v = {rb[j * 4 + 0], rb[j * 4 + 1], rb[j * 4 + 2], rb[j * 4 + 3]};
      *(f32x4*)&Bs[buf][bn * LDS_S + (bq + 2 * j) * 4] = v;
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

  gload(0);
  sstore(0);
  __syncthreads();

  const int a_off = (wm * 128 + l32) * LDS_S + 4 * half;
  const int b_off = (wn * 64 + l32) * LDS_S + 4 * half;
  const int nk = p.K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
    const float* as = As[buf] + a_off;
    const float* bs = Bs[buf] + b_off;
    f32x4 af[2][4], bf[2][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) af[0][mi] = *(const f32x4*)&as[mi * 32 * LDS_S];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bf[0][ni] = *(const f32x4*)&bs[ni * 32 * LDS_S];
#pragma unroll
    for (int c = 0; c < BK / 8; ++c) {
      const int cur = c & 1, nxt = cur ^ 1;
      if (c + 1 < BK / 8) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[nxt][mi] = *(const f32x4*)&as[mi * 32 * LDS_S + (c + 1) * 8];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          bf[nxt][ni] = *(const f32x4*)&bs[ni * 32 * LDS_S + (c + 1) * 8];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[cur][mi][s], bf[cur][ni][s],
                                                               acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue through LDS, one 32 x 32 block per wave at a time: the block is
  // written in the MFMA accumulator layout (lane l, register v holds row
  // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32), read back row-major as
  // float4, and combined with P / Lam by coalesced float4 accesses. This also
  // keeps the compiler from moving all 128 accumulators and their partner
  // loads into VGPRs at once. The tiles' LDS is free after the last barrier.
  constexpr int ES = 36;  // row stride of the per-wave staging block
  float* stage = &As[0][0] + wave * 32 * ES;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < 16; ++v)
        stage[(8 * (v >> 2) + 4 * half + (v & 3)) * ES + l32] = acc[mi][ni][v];
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): wave-local LDS round trip
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = 8 * t + (lane >> 3), c4 = (lane & 7) * 4;
        const f32x4 val = *(const f32x4*)&stage[r * ES + c4];
        const int row = tm * BM + wm * 128 + mi * 32 + r;
        const int col = tn * BN + wn * 64 + ni * 32 + c4;
        const int64_t idx = (int64_t)row * p.ldc + col;
        if (EPI == kEpiRhs) {
          const f32x4 pv = *(const f32x4*)&p.P[idx];
          *(f32x4*)&p.C[idx] = val + p.rho * pv;
        } else if (EPI == kEpiSolve) {
          const f32x4 xv = *(const f32x4*)&p.X[idx];
          *(f32x4*)&p.C[idx] = val;
          *(f32x4*)&p.X[idx] = val + xv;
        } else {
          *(f32x4*)&p.C[idx] = val;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.M % BM || a.N % BN || a.K % BK || a.M <= 0 || a.N <= 0 || a.K <= 0)
    return hipErrorInvalidValue;
  const int nt = (a.M / BM) * (a.N / BN);
  dim3 grid(nt), block(NT);
  switch (epi) {
    case kEpiRhs: hipLaunchKernelGGL(gemm_nn_kernel<kEpiRhs>, grid, block, 0, s, a); break;
    case kEpiSolve: hipLaunchKernelGGL(gemm_nn_kernel<kEpiSolve>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(gemm_nn_kernel<kEpiPlain>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace nq
