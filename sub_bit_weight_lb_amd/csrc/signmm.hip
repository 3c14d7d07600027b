// Products with a +-1 factor on the bf16 matrix cores, exactly: C = A S^T
// for A (M x K, fp32) and S (N x K, entries +-1 stored as fp32), both
// k-contiguous ("NT"). The STE refinement (NanoQuant digest, section
// 方法步骤详情, stage 2 step (3)) runs four such products per step: the
// forward pass through sign(V) and sign(U) and the backward pass through
// them again.
//
// +-1 is exact in bf16, and each entry a of A splits into three bf16 terms
// a = h + m + l by truncation (h = the top 16 bits of a, m the top 16 bits
// of a - h, l = a - h - m, which has at most 8 significant bits). So every
// product a s is exact as h s + m s + l s, and only the fp32 accumulation
// rounds, as in an fp32 product: three v_mfma_f32_16x16x32_bf16 cover the
// 32 k-values that eight v_mfma_f32_16x16x4_f32 would.
//
// A workgroup (256 threads, 4 waves in 2 x 2) computes a 128 x 128 tile of
// C, each wave 64 x 64 as 4 x 4 MFMA tiles. K is staged 64 at a time:
// A's fp32 rows are loaded coalesced (16 lanes per 256-byte row), split into
// the three terms and written to LDS, S's rows converted to bf16 (its top
// 16 bits), each LDS row padded to 144 bytes so that the 16 lanes reading
// one fragment column hit distinct bank groups. The next stage is loaded
// into registers while the current one multiplies. MFMA operands: A[i][k]
// from lane i + 16 (k / 8), element k % 8 (rows of A), B[k][j] the same for
// rows of S; lane l holds C[4 (l / 16) + v][l % 16], element v.
//
// Tile order is XCD-aware: workgroup b runs on XCD b % 8, and XCD x takes a
// contiguous range of tiles (row panels of A shared in its L2).
#include "common.h"

namespace nq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSm = 128, kSn = 128, kSk = 64;   // tile and K stage
constexpr int kSrow = kSk + 8;                  // bf16 per LDS row (144 bytes)

template <bool TRANS>
__global__ __launch_bounds__(256) void sign_gemm_kernel(const float* __restrict__ A, int64_t lda,
                                                        const float* __restrict__ S, int64_t lds,
                                                        float* __restrict__ C, int64_t ldc,
                                                        float* __restrict__ Ct, int64_t ldct,
                                                        int M, int N, int K) {
  __shared__ __align__(16) uint16_t as[3][kSm * kSrow];
  __shared__ __align__(16) uint16_t bs[kSn * kSrow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  // XCD-aware tile: XCD b % 8 takes tiles [x * per, (x + 1) * per)
  const int ntn = N / kSn, ntiles = (M / kSm) * ntn;
  const int b = blockIdx.x, per = (ntiles + 7) / 8;
  const int tile = (b & 7) * per + (b >> 3);
  if (tile >= ntiles) return;
  const int tm = tile / ntn, tn = tile % ntn;
  const float* Ab = A + (int64_t)tm * kSm * lda;
  const float* Sb = S + (int64_t)tn * kSn * lds;
  // staging map: thread t loads float4 c = t % 16 of rows t / 16 + 16 j
  const int sc = tid & 15, sr = tid >> 4;
  float4 ra[8], rb[8];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ra[j] = *(const float4*)(Ab + (int64_t)(sr + 16 * j) * lda + k0 + 4 * sc);
      rb[j] = *(const float4*)(Sb + (int64_t)(sr + 16 * j) * lds + k0 + 4 * sc);
    }
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  fetch(0);
  for (int k0 = 0; k0 < K; k0 += kSk) {
    __syncthreads();   // the previous stage's fragments are read
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = sr + 16 * j;
      const float x[4] = {ra[j].x, ra[j].y, ra[j].z, ra[j].w};
      uint32_t h[4], m[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = __float_as_uint(x[e]);
        const float r1 = x[e] - __uint_as_float(u & 0xffff0000u);
        const uint32_t v = __float_as_uint(r1);
        const float r2 = r1 - __uint_as_float(v & 0xffff0000u);
        h[e] = u >> 16;
        m[e] = v >> 16;
        l[e] = __float_as_uint(r2) >> 16;
      }
      const int off = row * kSrow + 4 * sc;
      *(u32x2*)&as[0][off] = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *(u32x2*)&as[1][off] = u32x2{m[0] | (m[1] << 16), m[2] | (m[3] << 16)};
      *(u32x2*)&as[2][off] = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
      const uint32_t s0 = __float_as_uint(rb[j].x) >> 16, s1 = __float_as_uint(rb[j].y) >> 16;
      const uint32_t s2 = __float_as_uint(rb[j].z) >> 16, s3 = __float_as_uint(rb[j].w) >> 16;
      *(u32x2*)&bs[off] = u32x2{s0 | (s1 << 16), s2 | (s3 << 16)};
    }
    __syncthreads();
    fetch(min(k0 + kSk, K - kSk));   // (the last stage reloads itself: no branch)
#pragma unroll
    for (int ks = 0; ks < kSk / 32; ++ks) {
      const int kof = ks * 32 + 8 * g;
      bf16x8 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)&bs[(wn * 64 + j * 16 + li) * kSrow + kof]);
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        bf16x8 af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)&as[p][(wm * 64 + i * 16 + li) * kSrow + kof]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  // lane (g, li) of tile (i, j) holds rows 4 g + v, column li
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r0 = (int64_t)tm * kSm + wm * 64 + i * 16 + 4 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = (int64_t)tn * kSn + wn * 64 + j * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) C[(r0 + v) * ldc + c] = acc[i][j][v];
      if (TRANS) *(f32x4*)&Ct[c * ldct + r0] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_sign_gemm(const float* A, int64_t lda, const float* S, int64_t lds, float* C,
                            int64_t ldc, float* Ct, int64_t ldct, int M, int N, int K,
                            hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0 || M % kSm || N % kSn || K % kSk || lda % 4 || lds % 4 ||
      (Ct && ldct % 4) || ((uintptr_t)A | (uintptr_t)S | (uintptr_t)Ct) % 16)
    return hipErrorInvalidValue;
  const int ntiles = (M / kSm) * (N / kSn);
  const int grid = (ntiles + 7) / 8 * 8;
  if (Ct)
    hipLaunchKernelGGL(sign_gemm_kernel<true>, dim3(grid), dim3(256), 0, s, A, lda, S, lds, C,
                       ldc, Ct, ldct, M, N, K);
  else
    hipLaunchKernelGGL(sign_gemm_kernel<false>, dim3(grid), dim3(256), 0, s, A, lda, S, lds, C,
                       ldc, Ct, ldct, M, N, K);
  return hipGetLastError();
}

}  // namespace nq
