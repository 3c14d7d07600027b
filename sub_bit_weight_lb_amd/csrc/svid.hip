// SVID (sign-value independent decomposition) fused with the ADMM dual
// update (NanoQuant digest, section 核心方法 steps (b) and (c), and section
// 技术新颖性, which names SVID as the operator mapping the continuous latent
// to the binary proxy).
//
//   Z = sign(X) .* (a b^T),  (a, b): T alternating rank-1 least-squares steps
//   on |X| from b = 1:  a = |X| b / (b^T b),  b = |X|^T a / (a^T a).
//   Dual: Lam = X - Z, and the right-hand side of the next solve needs
//   Z - Lam = 2 Z - X, which is stored instead of Z (one read there).
//
// HBM-bound. Per power step one fused pass: each block holds a slab of full
// rows in registers, forms a for its rows and then its rows' share of
// |X|^T a, so X is read once per step; a small reduce then forms b. In the
// ADMM update the first pass also forms X = U + Lam from the new factor and
// the dual (written over Lam), so the solve that produces U does not. For
// r beyond 16384 a row pass and a column pass replace the fused one. All
// reductions run in a fixed order, so results are bit-reproducible. Every
// kernel raises its waves' issue priority: in the ADMM loop the SVID runs
// beside the solve and the next Gram, MFMA-bound kernels whose waves would
// otherwise take most issue cycles of a shared SIMD, and the next RHS GEMM
// waits for it.
#include "common.h"

namespace nq {
namespace {

constexpr int CR = 64;    // rows per column-pass chunk
constexpr int CB = 128;   // columns per column-pass block

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__global__ void svid_init_b_kernel(float* b, float* bbpart, int rp, int r_real) {
  __builtin_amdgcn_s_setprio(3);
  const int j = blockIdx.x * CB + threadIdx.x;
  b[j] = j < r_real ? 1.0f : 0.0f;
  if (threadIdx.x == 0) {
    const int cnt = min(CB, max(0, r_real - (int)blockIdx.x * CB));
    bbpart[blockIdx.x] = (float)cnt;
  }
}

// a_i = sum_j |X_ij| b_j / bb,  bb = sum of bbpart.
__global__ __launch_bounds__(256) void svid_row_kernel(const float* __restrict__ X, int rp,
                                                       const float* __restrict__ b,
                                                       const float* __restrict__ bbpart, int nbb,
                                                       float* __restrict__ a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  float bb = 0.0f;
  for (int q = lane; q < nbb; q += 64) bb += bbpart[q];
  bb = wave_sum(bb);
  const f32x4* x4 = (const f32x4*)(X + (int64_t)i * rp);
  const f32x4* b4 = (const f32x4*)b;
  float s = 0.0f;
  for (int j = lane; j < rp / 4; j += 64) {
    const f32x4 x = x4[j], w = b4[j];
    s += fabsf(x[0]) * w[0] + fabsf(x[1]) * w[1] + fabsf(x[2]) * w[2] + fabsf(x[3]) * w[3];
  }
  s = wave_sum(s);
  if (lane == 0) a[i] = bb > 0.0f ? s / bb : 0.0f;
}

// colpart[c][j] = sum_{i in chunk c} w(X_ij, a_i); aapart[c] = sum a_i^2.
// OP 0: |X_ij| a_i (SVID); OP 1: X_ij^2 (column norms). 32 x 8 threads:
// float4 columns x row stripes of the 64-row chunk, fixed-order reduction.
template <int OP>
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ X, int rp,
                                                     int rows_pad, const float* __restrict__ a,
                                                     float* __restrict__ colpart,
                                                     float* __restrict__ aapart) {
  __shared__ f32x4 red[8][32];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int q = blockIdx.x * 32 + tx;
  const int c = blockIdx.y;
  const int i0 = c * CR, i1 = min(rows_pad, i0 + CR);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int i = i0 + ty; i < i1; i += 8) {
    const f32x4 x = ((const f32x4*)(X + (int64_t)i * rp))[q];
    if (OP == 0) {
      const float ai = a[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += fabsf(x[e]) * ai;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += x[e] * x[e];
    }
  }
  red[ty][tx] = acc;
  __syncthreads();
  if (ty == 0) {
    f32x4 t = red[0][tx];
#pragma unroll
    for (int y = 1; y < 8; ++y) t += red[y][tx];
    ((f32x4*)(colpart + (int64_t)c * rp))[q] = t;
  }
  if (OP == 0 && blockIdx.x == 0 && threadIdx.x == 0) {
    float aa = 0.0f;
    for (int i = i0; i < i1; ++i) aa += a[i] * a[i];
    aapart[c] = aa;
  }
}

// One fused power step for a slab of RS full rows held in registers:
//   a_i = sum_j |X_ij| b_j / bb          (rows of the slab, block reduction)
//   part[slab][j] = sum_{i in slab} |X_ij| a_i,  aapart[slab] = sum a_i^2
// so X is read once per step. Thread t owns float4 columns t + 256 u.
// With Uadd (first step of an update), X is first formed as X + Uadd and
// written back.
template <int RS, int NU>
__global__ __launch_bounds__(256) void svid_step_kernel(float* X, const float* __restrict__ Uadd,
                                                        int rp, const float* __restrict__ b,
                                                        const float* __restrict__ bbpart, int nbb,
                                                        float* __restrict__ a,
                                                        float* __restrict__ part,
                                                        float* __restrict__ aapart) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ float red[RS][4];
  __shared__ float arow[RS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rp4 = rp / 4;
  const int64_t i0 = (int64_t)blockIdx.x * RS;
  float bb = 0.0f;
  for (int q = lane; q < nbb; q += 64) bb += bbpart[q];
  bb = wave_sum(bb);
  f32x4 x[RS][NU];
  f32x4 bv[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int q = tid + 256 * u;
    bv[u] = q < rp4 ? ((const f32x4*)b)[q] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
#pragma unroll
  for (int r = 0; r < RS; ++r)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int q = tid + 256 * u;
      x[r][u] = q < rp4 ? ((const f32x4*)(X + (i0 + r) * rp))[q] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  if (Uadd) {
#pragma unroll
    for (int r = 0; r < RS; ++r)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int q = tid + 256 * u;
        if (q < rp4) {
          x[r][u] += ((const f32x4*)(Uadd + (i0 + r) * rp))[q];
          ((f32x4*)(X + (i0 + r) * rp))[q] = x[r][u];
        }
      }
  }
  float s[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += fabsf(x[r][u][e]) * bv[u][e];
    s[r] = wave_sum(acc);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RS; ++r) red[r][wave] = s[r];
  }
  __syncthreads();
  if (tid < RS) {
    const float tot = red[tid][0] + red[tid][1] + red[tid][2] + red[tid][3];
    const float ai = bb > 0.0f ? tot / bb : 0.0f;
    arow[tid] = ai;
    a[i0 + tid] = ai;
  }
  __syncthreads();
  float av[RS];
#pragma unroll
  for (int r = 0; r < RS; ++r) av[r] = arow[r];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int q = tid + 256 * u;
    if (q < rp4) {
      f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < RS; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] += fabsf(x[r][u][e]) * av[r];
      ((f32x4*)(part + (int64_t)blockIdx.x * rp))[q] = p;
    }
  }
  if (tid == 0) {
    float aa = 0.0f;
#pragma unroll
    for (int r = 0; r < RS; ++r) aa += av[r] * av[r];
    aapart[blockIdx.x] = aa;
  }
}

// b_j = sum_c part[c][j] / aa over nch partial rows, in two launches:
// stage 1, block (g, y): the y-th share of the partial rows for the 128
// columns of group g -> part2[y]; stage 2, block g: part2[0..NY) in order,
// aa = sum of aapart, b = sum / aa, bbpart[g] = sum b^2. Fixed order
// throughout, no inter-block communication inside a launch.
constexpr int NY = kSvidReduceRows;  // row groups of the reduce
__global__ __launch_bounds__(256) void svid_reduce1_kernel(const float* __restrict__ part, int nch,
                                                           int rp, float* __restrict__ part2) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ f32x4 red[8][32];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int q = blockIdx.x * 32 + tx;  // float4 column index
  const int y = blockIdx.y;
  const int c0 = (int)((int64_t)nch * y / NY), c1 = (int)((int64_t)nch * (y + 1) / NY);
  f32x4 p = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int c = c0 + ty; c < c1; c += 8) p += ((const f32x4*)(part + (int64_t)c * rp))[q];
  red[ty][tx] = p;
  __syncthreads();
  if (ty == 0) {
    f32x4 t = red[0][tx];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += red[k][tx];
    ((f32x4*)(part2 + (int64_t)y * rp))[q] = t;
  }
}

__global__ __launch_bounds__(256) void svid_reduce2_kernel(const float* __restrict__ part2,
                                                           const float* __restrict__ aapart,
                                                           int nch, int rp, float* __restrict__ b,
                                                           float* __restrict__ bbpart) {
  __builtin_amdgcn_s_setprio(3);
  __shared__ float fred[256];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int q = blockIdx.x * 32 + tx;
  float aa = 0.0f;
  for (int c = threadIdx.x; c < nch; c += 256) aa += aapart[c];
  fred[threadIdx.x] = aa;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) fred[threadIdx.x] += fred[threadIdx.x + o];
    __syncthreads();
  }
  const float tot = fred[0];
  __syncthreads();
  if (ty == 0) {
    f32x4 t = ((const f32x4*)part2)[q];
#pragma unroll
    for (int k = 1; k < NY; ++k) t += ((const f32x4*)(part2 + (int64_t)k * rp))[q];
    f32x4 bj;
#pragma unroll
    for (int e = 0; e < 4; ++e) bj[e] = tot > 0.0f ? t[e] / tot : 0.0f;
    ((f32x4*)b)[q] = bj;
    fred[tx] = bj[0] * bj[0] + bj[1] * bj[1] + bj[2] * bj[2] + bj[3] * bj[3];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int k = 0; k < 32; ++k) t += fred[k];
    bbpart[blockIdx.x] = t;
  }
}

// Z = sign(X) a_i b_j; mode 0: P = Z, X = 0; mode 1: X = X - Z, P = Z - X_new;
// mode 2: P = Z.
__global__ __launch_bounds__(256) void svid_final_kernel(float* __restrict__ X,
                                                         float* __restrict__ P,
                                                         const float* __restrict__ a,
                                                         const float* __restrict__ b, int rp,
                                                         int64_t n4, int mode) {
  __builtin_amdgcn_s_setprio(3);
  const int rp4 = rp / 4;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = q / rp4;
    const int j4 = (int)(q % rp4);
    const f32x4 x = ((const f32x4*)X)[q];
    const f32x4 bv = ((const f32x4*)b)[j4];
    const float ai = a[i];
    f32x4 z;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mag = ai * bv[e];
      z[e] = x[e] >= 0.0f ? mag : -mag;
    }
    if (mode == 1) {
      const f32x4 lam = x - z;
      ((f32x4*)X)[q] = lam;
      ((f32x4*)P)[q] = z - lam;
    } else {
      ((f32x4*)P)[q] = z;
      if (mode == 0) ((f32x4*)X)[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
}

}  // namespace

int svid_nchunks(int rows_pad) { return (rows_pad + CR - 1) / CR; }

namespace {
// Slab rows RS and float4s per thread NU for the fused step at this rp.
template <int RS, int NU>
void launch_step(float* X, const float* Uadd, int rows_pad, int rp, int nbb, const SvidWork& w,
                 hipStream_t s) {
  hipLaunchKernelGGL((svid_step_kernel<RS, NU>), dim3(rows_pad / RS), dim3(256), 0, s, X, Uadd,
                     rp, w.b, w.bbpart, nbb, w.a, w.colpart, w.aapart);
}
bool fused_step(float* X, const float* Uadd, int rows_pad, int rp, int nbb, const SvidWork& w,
                hipStream_t s) {
  const int nu = (rp / 4 + 255) / 256;
  if (nu <= 1) launch_step<8, 1>(X, Uadd, rows_pad, rp, nbb, w, s);
  else if (nu <= 2) launch_step<8, 2>(X, Uadd, rows_pad, rp, nbb, w, s);
  else if (nu <= 4) launch_step<4, 4>(X, Uadd, rows_pad, rp, nbb, w, s);
  else if (nu <= 8) launch_step<2, 8>(X, Uadd, rows_pad, rp, nbb, w, s);
  else if (nu <= 16) launch_step<1, 16>(X, Uadd, rows_pad, rp, nbb, w, s);
  else return false;
  return true;
}
// X += U (float4s), for the unfused path
__global__ __launch_bounds__(256) void add_into_kernel(float* __restrict__ X,
                                                       const float* __restrict__ U, int64_t n4) {
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * blockDim.x)
    ((f32x4*)X)[q] += ((const f32x4*)U)[q];
}
int fused_rows(int rp) {
  const int nu = (rp / 4 + 255) / 256;
  return nu <= 2 ? 8 : nu <= 4 ? 4 : nu <= 8 ? 2 : nu <= 16 ? 1 : 0;
}
}  // namespace

int svid_partials(int rows_pad, int rp) {
  const int rs = fused_rows(rp);
  return rs ? rows_pad / rs : svid_nchunks(rows_pad);
}

hipError_t launch_svid(float* X, float* P, int rows_pad, int rp, int r_real, int T, int mode,
                       const SvidWork& w, hipStream_t s, const float* Uadd) {
  if (rp % CB || rows_pad % 8 || T < 1) return hipErrorInvalidValue;
  const int nbb = rp / CB;
  const int nch = svid_nchunks(rows_pad);
  const int rs = fused_rows(rp);
  const int64_t n4 = (int64_t)rows_pad * rp / 4;
  const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(svid_init_b_kernel, dim3(nbb), dim3(CB), 0, s, w.b, w.bbpart, rp, r_real);
  if (Uadd && !rs) {
    hipLaunchKernelGGL(add_into_kernel, dim3(blocks), dim3(256), 0, s, X, Uadd, n4);
    Uadd = nullptr;
  }
  for (int t = 0; t < T; ++t) {
    if (rs && fused_step(X, t == 0 ? Uadd : nullptr, rows_pad, rp, nbb, w, s)) {
      hipLaunchKernelGGL(svid_reduce1_kernel, dim3(rp / 128, NY), dim3(256), 0, s, w.colpart,
                         rows_pad / rs, rp, w.part2);
      hipLaunchKernelGGL(svid_reduce2_kernel, dim3(rp / 128), dim3(256), 0, s, w.part2, w.aapart,
                         rows_pad / rs, rp, w.b, w.bbpart);
      continue;
    }
    hipLaunchKernelGGL(svid_row_kernel, dim3(rows_pad / 4), dim3(256), 0, s, X, rp, w.b,
                       w.bbpart, nbb, w.a);
    hipLaunchKernelGGL(colsum_kernel<0>, dim3(rp / 128, nch), dim3(256), 0, s, X, rp, rows_pad,
                       w.a, w.colpart, w.aapart);
    hipLaunchKernelGGL(svid_reduce1_kernel, dim3(rp / 128, NY), dim3(256), 0, s, w.colpart, nch,
                       rp, w.part2);
    hipLaunchKernelGGL(svid_reduce2_kernel, dim3(rp / 128), dim3(256), 0, s, w.part2, w.aapart,
                       nch, rp, w.b, w.bbpart);
  }
  hipLaunchKernelGGL(svid_final_kernel, dim3(blocks), dim3(256), 0, s, X, P, w.a, w.b, rp, n4,
                     mode);
  return hipGetLastError();
}

hipError_t launch_colsumsq(const float* F, int rows_pad, int rp, float* colpart, hipStream_t s) {
  if (rp % CB) return hipErrorInvalidValue;
  const int nch = svid_nchunks(rows_pad);
  hipLaunchKernelGGL(colsum_kernel<1>, dim3(rp / 128, nch), dim3(256), 0, s, F, rp, rows_pad,
                     (const float*)nullptr, colpart, (float*)nullptr);
  return hipGetLastError();
}

}  // namespace nq
