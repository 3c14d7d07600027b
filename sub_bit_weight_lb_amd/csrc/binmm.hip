// Applying a low-rank binary layer from its packed signs (NanoQuant digest,
// section 研究动机: the layer is kept as W ~ diag(s1) U_{+-1} V_{+-1}^T
// diag(s2); section 技术新颖性: the authors run such layers with binary GEMV
// and GEMM kernels of their own rather than forming W).
//
//   Y = X W^T,  y_b = s1 * ( S_U ( S_V^T ( s2 * x_b ) ) )
//
// Both products are of one kind: out[row] = sum_c sign(row, c) v[c] with the
// signs packed along the row (bit = [+1], LSB first, 32 columns per word, the
// layout nq_pack_signs writes). With S_V^T packed along n (transpose_bits,
// once per layer) the first product is T = S_V^T (s2 * x) over the r rows of
// S_V^T and the second y = s1 * (S_U T) over the m rows of S_U, so one
// kernel serves both.
//
// bin_rowdot_kernel: four waves, four rows per wave. A chunk of 64 words
// (2048 columns) of v goes to LDS bit-major (the value of column 32 w + i at
// [i][w]), so lane l, which holds word l of the chunk for each of its rows,
// reads its 32 values without bank conflicts and uses each one for four
// rows. The words are fetched before the chunk of v is staged. Each lane sums
// +-v over its bits in column order, then the wave sums its lanes in a fixed
// tree: the result does not depend on timing. Bits past `cols` in a row's
// last word meet v = 0 there, so they add nothing.
#include "common.h"

namespace nq {
namespace {

constexpr int RPW = 4;   // rows per wave
constexpr int CW = 64;   // words per column chunk, one per lane

__device__ inline float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int BT>
__global__ __launch_bounds__(256) void bin_rowdot_kernel(
    const uint32_t* __restrict__ bits, int64_t ldw, int64_t rows, int64_t cols,
    const float* __restrict__ v, int64_t ldv, const float* __restrict__ pre,
    const float* __restrict__ post, float* __restrict__ out, int64_t ldo, int64_t B) {
  __shared__ float vs[BT][32][CW + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b0 = (int64_t)blockIdx.y * BT;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  const int64_t nwords = (cols + 31) / 32;
  float acc[RPW][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.0f;
  for (int64_t cw0 = 0; cw0 < nwords; cw0 += CW) {
    const int64_t w = cw0 + lane;
    uint32_t word[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      word[r] = (row0 + r < rows && w < nwords) ? bits[(row0 + r) * ldw + w] : 0u;
    __syncthreads();  // every wave is done with the previous chunk of v
    for (int e = threadIdx.x; e < BT * 32 * CW; e += 256) {
      const int b = e / (32 * CW), rem = e % (32 * CW);
      const int ww = rem / 32, i = rem % 32;
      const int64_t c = (cw0 + ww) * 32 + i;
      float x = 0.0f;
      if (b0 + b < B && c < cols) {
        x = v[(b0 + b) * ldv + c];
        if (pre) x *= pre[c];
      }
      vs[b][i][ww] = x;
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const float x = vs[b][i][lane];
#pragma unroll
        for (int r = 0; r < RPW; ++r) acc[r][b] += ((word[r] >> i) & 1u) ? x : -x;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const float s = wave_sum64(acc[r][b]);
      const int64_t row = row0 + r;
      if (lane == 0 && row < rows && b0 + b < B) out[(b0 + b) * ldo + row] = post ? s * post[row] : s;
    }
}

// out (cols x ld_out words) bit (c, i) = in bit (i, c), in holding rows x cols
// signs (rows x ld_in words). Wave (row block of 64, input word cw): lane l
// reads the word of row 64 q + l; the ballot of bit j over the lanes is
// column 32 cw + j at those 64 rows, two output words, written by lane j.
__global__ __launch_bounds__(256) void transpose_bits_kernel(const uint32_t* __restrict__ in,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ld_in,
                                                             uint32_t* __restrict__ out,
                                                             int64_t ld_out) {
  const int lane = threadIdx.x & 63;
  const int64_t nwin = (cols + 31) / 32;     // input words per row
  const int64_t nrb = (rows + 63) / 64;      // row blocks
  const int64_t nwout = (rows + 31) / 32;    // output words per row
  const int64_t total = nrb * nwin;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < total;
       t += (int64_t)gridDim.x * 4) {
    const int64_t q = t / nwin, cw = t % nwin;
    const int64_t row = q * 64 + lane;
    const uint32_t word = row < rows ? in[row * ld_in + cw] : 0u;
    uint64_t mine = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint64_t m = __ballot((word >> j) & 1u);
      mine = lane == j ? m : mine;
    }
    const int64_t c = cw * 32 + lane;
    if (lane < 32 && c < cols) {
      out[c * ld_out + 2 * q] = (uint32_t)mine;
      if (2 * q + 1 < nwout) out[c * ld_out + 2 * q + 1] = (uint32_t)(mine >> 32);
    }
  }
}

template <int BT>
void rowdot(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
            int64_t ldv, const float* pre, const float* post, float* out, int64_t ldo, int64_t B,
            hipStream_t s) {
  const dim3 grid((unsigned)((rows + 4 * RPW - 1) / (4 * RPW)), (unsigned)((B + BT - 1) / BT));
  hipLaunchKernelGGL(bin_rowdot_kernel<BT>, grid, dim3(256), 0, s, bits, ldw, rows, cols, v, ldv,
                     pre, post, out, ldo, B);
}

void rowdot_any(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
                int64_t ldv, const float* pre, const float* post, float* out, int64_t ldo,
                int64_t B, hipStream_t s) {
  if (B == 1) rowdot<1>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, B, s);
  else if (B == 2) rowdot<2>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, B, s);
  else rowdot<4>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, B, s);
}

}  // namespace

hipError_t launch_transpose_bits(const uint32_t* in, int64_t rows, int64_t cols, int64_t ld_in,
                                 uint32_t* out, int64_t ld_out, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t waves = ((rows + 63) / 64) * ((cols + 31) / 32);
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(transpose_bits_kernel, dim3((unsigned)blocks), dim3(256), 0, s, in, rows,
                     cols, ld_in, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_binary_matmul(const uint32_t* su, int64_t ldu, const uint32_t* svt,
                                int64_t ldvt, int64_t m, int64_t n, int64_t r, const float* s1,
                                const float* s2, const float* X, int64_t B, int64_t ldx,
                                float* Y, int64_t ldy, float* T, hipStream_t s) {
  if (m <= 0 || n <= 0 || r <= 0 || B <= 0) return hipSuccess;
  if ((r + 4 * RPW - 1) / (4 * RPW) > 0x7fffffff || (m + 4 * RPW - 1) / (4 * RPW) > 0x7fffffff ||
      (B + 3) / 4 > 65535)
    return hipErrorInvalidValue;
  // T = (X * s2) S_V: the r rows of S_V^T against x
  rowdot_any(svt, ldvt, r, n, X, ldx, s2, nullptr, T, r, B, s);
  // Y = s1 * (T S_U^T): the m rows of S_U against T
  rowdot_any(su, ldu, m, r, T, r, nullptr, s1, Y, ldy, B, s);
  return hipGetLastError();
}

}  // namespace nq
