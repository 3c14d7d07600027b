// Finishing kernels (NanoQuant digest, section 方法步骤详情, stage 2: after
// convergence the factor magnitudes are balanced to remove the scale
// ambiguity, channel scales s1 and s2 are extracted, and the signs are
// packed into an integer format), the reconstruction error of
// W ~ diag(s1) sign(U) sign(V)^T diag(s2) (section 研究动机), and the
// standalone sign packer.
#include "common.h"

namespace nq {
namespace {

constexpr int CB = 128;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// c_k = sqrt(||v_k|| / ||u_k||), from partial column sums of squares.
__global__ void balance_coef_kernel(const float* __restrict__ pu, int nchu,
                                    const float* __restrict__ pv, int nchv, int rp, int balance,
                                    float* __restrict__ c) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= rp) return;
  float su = 0.0f, sv = 0.0f;
  for (int q = 0; q < nchu; ++q) su += pu[(int64_t)q * rp + k];
  for (int q = 0; q < nchv; ++q) sv += pv[(int64_t)q * rp + k];
  float ck = 1.0f;
  if (balance && su > 0.0f && sv > 0.0f) ck = sqrtf(sqrtf(sv) / sqrtf(su));
  c[k] = ck;
}

// One wave per row: F' = F * c (or F / c); outputs, scales, bits via ballot,
// int8 signs (zero in the padding) for the error product.
__global__ __launch_bounds__(256) void apply_finish_kernel(
    const float* __restrict__ F, int64_t rows, int rp, int64_t r, const float* __restrict__ c,
    int divide, const float* __restrict__ d, float* __restrict__ out,
    float* __restrict__ scale_out, float* __restrict__ scale_wt, uint32_t* __restrict__ bits,
    int8_t* __restrict__ sign8, DevStats* st) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const bool row_ok = i < rows;
  const int64_t nw = (r + 31) / 32;
  float sabs = 0.0f;
  bool bad = false;
  for (int ch = 0; ch < rp / 64; ++ch) {
    const int k = ch * 64 + lane;
    const float x = F[i * rp + k];
    const float xp = divide ? x / c[k] : x * c[k];
    const bool real = row_ok && k < r;
    if (real) {
      if (out) out[i * r + k] = xp;
      sabs += fabsf(xp);
      bad |= !isfinite(xp);
    }
    const bool pos = real && xp >= 0.0f;
    const uint64_t mask = __ballot(pos);
    if (bits && row_ok && lane == 0) {
      const int64_t w0 = 2 * (int64_t)ch;
      if (w0 < nw) bits[i * nw + w0] = (uint32_t)mask;
      if (w0 + 1 < nw) bits[i * nw + w0 + 1] = (uint32_t)(mask >> 32);
    }
    sign8[i * rp + k] = real ? (xp >= 0.0f ? (int8_t)1 : (int8_t)-1) : (int8_t)0;
  }
  if (bad) atomicOr(&st->nonfinite, 1);
  sabs = wave_sum(sabs);
  if (lane == 0) {
    const float s = row_ok ? sabs / (float)r : 0.0f;
    scale_wt[i] = s;
    if (scale_out && row_ok) scale_out[i] = s / d[i];
  }
}

// Sign-product error: P = S_U S_V^T exactly with the int8 MFMA (|P| <= r, int32
// accumulate), E = s1w_i s2w_j P_ij, squared errors in Wt and W space summed
// per 128 x 128 tile in double.
// K runs in chunks of 32 (v_mfma_i32_32x32x32_i8, 16 bytes of one row per
// lane), four chunks per round: a round's 16 fragment loads all go out
// before the previous round's 16 MFMAs, so each round waits on one load
// latency at most. Lane half h of chunk u holds bytes 32 u + 16 h of the
// round's 128 for its row of S_U or S_V; both operands use the same map, so
// the products sum over every k exactly once. rp % 128 == 0.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void error_kernel(
    const int8_t* __restrict__ SU, const int8_t* __restrict__ SV, int np_, int rp,
    const float* __restrict__ s1w, const float* __restrict__ s2w, const float* __restrict__ Wt,
    const float* __restrict__ W, int64_t ldw, int64_t m, int64_t n,
    const float* __restrict__ s1, const float* __restrict__ s2, double* __restrict__ parts) {
  __shared__ double red[256];
  const int tilesN = np_ / 128;
  const int ti = blockIdx.x / tilesN, tj = blockIdx.x % tilesN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  i32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0;
  const int8_t* ua = SU + (int64_t)(ti * 128 + wm * 64 + l32) * rp + 16 * half;
  const int8_t* vb = SV + (int64_t)(tj * 128 + wn * 64 + l32) * rp + 16 * half;
  constexpr int U = 4;
  i32x4 af[U][2], bf[U][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        af[u][a] = *(const i32x4*)(ua + (int64_t)a * 32 * rp + k0 + 32 * u);
        bf[u][a] = *(const i32x4*)(vb + (int64_t)a * 32 * rp + k0 + 32 * u);
      }
  };
  load(0);
  for (int k0 = 0; k0 < rp; k0 += 32 * U) {
    i32x4 ca[U][2], cb[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        ca[u][a] = af[u][a];
        cb[u][a] = bf[u][a];
      }
    if (k0 + 32 * U < rp) load(k0 + 32 * U);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ca[u][a], cb[u][b], acc[a][b], 0, 0, 0);
  }
  double e_wt = 0.0, e_w = 0.0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = ti * 128 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        const int64_t j = tj * 128 + wn * 64 + b * 32 + l32;
        const float p = (float)acc[a][b][v];
        const float d1 = Wt[i * np_ + j] - s1w[i] * s2w[j] * p;
        e_wt += (double)d1 * (double)d1;
        if (i < m && j < n) {
          const float d2 = W[i * ldw + j] - s1[i] * s2[j] * p;
          e_w += (double)d2 * (double)d2;
        }
      }
  red[threadIdx.x] = e_wt;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) parts[2 * (int64_t)blockIdx.x] = red[0];
  __syncthreads();
  red[threadIdx.x] = e_w;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) parts[2 * (int64_t)blockIdx.x + 1] = red[0];
}

__global__ __launch_bounds__(256) void error_reduce_kernel(const double* parts, int nparts,
                                                           DevStats* st) {
  __shared__ double ra[256], rb[256];
  double a = 0.0, b = 0.0;
  for (int q = threadIdx.x; q < nparts; q += 256) {
    a += parts[2 * (int64_t)q];
    b += parts[2 * (int64_t)q + 1];
  }
  ra[threadIdx.x] = a;
  rb[threadIdx.x] = b;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      ra[threadIdx.x] += ra[threadIdx.x + o];
      rb[threadIdx.x] += rb[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    st->err2_wt = ra[0];
    st->err2_w = rb[0];
  }
}

// One wave per (row, 64-column chunk): ballot of x >= 0 gives two words.
__global__ __launch_bounds__(256) void pack_signs_kernel(const float* __restrict__ X,
                                                         int64_t rows, int64_t cols,
                                                         int64_t ldx, uint32_t* __restrict__ bits,
                                                         int64_t ld_words) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = (cols + 63) / 64;
  const int64_t nwords = (cols + 31) / 32;
  const int64_t total = rows * nch;
  for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < total;
       w += (int64_t)gridDim.x * 4) {
    const int64_t i = w / nch, ch = w % nch;
    const int64_t col = ch * 64 + lane;
    const bool pos = col < cols && X[i * ldx + col] >= 0.0f;
    const uint64_t mask = __ballot(pos);
    if (lane == 0) {
      bits[i * ld_words + 2 * ch] = (uint32_t)mask;
      if (2 * ch + 1 < nwords) bits[i * ld_words + 2 * ch + 1] = (uint32_t)(mask >> 32);
    }
  }
}

}  // namespace

hipError_t launch_balance_coef(const float* partU, int nchU, const float* partV, int nchV, int rp,
                               bool balance, float* c, hipStream_t s) {
  hipLaunchKernelGGL(balance_coef_kernel, dim3((rp + 255) / 256), dim3(256), 0, s, partU, nchU,
                     partV, nchV, rp, balance ? 1 : 0, c);
  return hipGetLastError();
}

hipError_t launch_apply_finish(const float* F, int64_t rows, int rows_pad, int rp, int64_t r,
                               const float* c, bool divide, const float* d, float* out,
                               float* scale_out, float* scale_wt, uint32_t* bits, int8_t* sign8,
                               DevStats* st, hipStream_t s) {
  if (rows_pad % 4 || rp % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(apply_finish_kernel, dim3(rows_pad / 4), dim3(256), 0, s, F, rows, rp, r, c,
                     divide ? 1 : 0, d, out, scale_out, scale_wt, bits, sign8, st);
  return hipGetLastError();
}

int error_nparts(int mp, int np_) { return (mp / 128) * (np_ / 128); }

hipError_t launch_error(const int8_t* SU, const int8_t* SV, int mp, int np_, int rp,
                        const float* s1w, const float* s2w, const float* Wt, const float* W,
                        int64_t ldw, int64_t m, int64_t n, const float* s1, const float* s2,
                        double* parts, DevStats* st, hipStream_t s) {
  if (mp % 128 || np_ % 128 || rp % 128 || rp <= 0) return hipErrorInvalidValue;
  const int nb = error_nparts(mp, np_);
  hipLaunchKernelGGL(error_kernel, dim3(nb), dim3(256), 0, s, SU, SV, np_, rp, s1w, s2w, Wt, W,
                     ldw, m, n, s1, s2, parts);
  hipLaunchKernelGGL(error_reduce_kernel, dim3(1), dim3(256), 0, s, parts, nb, st);
  return hipGetLastError();
}

hipError_t launch_pack_signs(const float* X, int64_t rows, int64_t cols, int64_t ldx,
                             uint32_t* bits, int64_t ld_words, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t waves = rows * ((cols + 63) / 64);
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_signs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, X, rows, cols,
                     ldx, bits, ld_words);
  return hipGetLastError();
}

}  // namespace nq
