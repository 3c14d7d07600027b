// Preparation kernels: preconditioning Wt = D_out W D_in (NanoQuant digest,
// section 方法步骤详情, stage 2 step (2)), norms, the initial latents, fills.
#include "common.h"

namespace nq {
namespace {

constexpr int PT = 64;  // precondition tile (64 x 64), 256 threads

__global__ void stats_init_kernel(DevStats* st) {
  st->sumsq_wt = 0.0;
  st->sumsq_w = 0.0;
  st->sigma0 = 0.0;
  st->err2_wt = 0.0;
  st->err2_w = 0.0;
  st->nonfinite = 0;
  st->bad_precond = 0;
  st->potrf_info = 0x7fffffff;
  st->sync_timeout = 0;
  st->to_wg = st->to_step = st->to_phase = st->to_want = st->to_seen = st->to_epoch = 0;
  st->to_start = st->to_now = 0;
  st->to_src = st->to_src_prog = 0;
}

__global__ void check_precond_kernel(const float* __restrict__ d_out, int64_t m,
                                     const float* __restrict__ d_in, int64_t n, DevStats* st) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m + n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float d = i < m ? d_out[i] : d_in[i - m];
    if (!(d > 0.0f) || !isfinite(d)) atomicOr(&st->bad_precond, 1);
  }
}

__device__ inline double block_sum_d(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// One 64 x 64 tile of the padded Wt per block: Wt = d_out_i * (W_ij * d_in_j),
// the transposed tile through LDS into WtT, and fp64 partial sums of squares.
__global__ __launch_bounds__(256) void precondition_kernel(
    const float* __restrict__ W, int64_t ldw, int64_t m, int64_t n,
    const float* __restrict__ d_out, const float* __restrict__ d_in, float* __restrict__ Wt,
    float* __restrict__ WtT, int mp, int np_, double* part_wt, double* part_w, DevStats* st) {
  __shared__ float tile[PT][PT + 1];
  __shared__ double red[256];
  const int tj = blockIdx.x, ti = blockIdx.y;
  const int c = threadIdx.x & 63, r0 = threadIdx.x >> 6;
  const int64_t j = (int64_t)tj * PT + c;
  const float dj = j < n ? d_in[j] : 0.0f;
  double swt = 0.0, sw = 0.0;
  bool bad = false;
#pragma unroll 4
  for (int q = 0; q < PT / 4; ++q) {
    const int rr = r0 + 4 * q;
    const int64_t i = (int64_t)ti * PT + rr;
    float w = 0.0f, di = 0.0f;
    if (i < m && j < n) {
      w = W[i * ldw + j];
      di = d_out[i];
    }
    const float wt = __fmul_rn(__fmul_rn(w, dj), di);
    bad |= !isfinite(wt) || !isfinite(w);
    Wt[i * np_ + j] = wt;
    tile[rr][c] = wt;
    swt += (double)wt * (double)wt;
    sw += (double)w * (double)w;
  }
  if (bad) atomicOr(&st->nonfinite, 1);
  __syncthreads();
  if (WtT) {
#pragma unroll 4
    for (int q = 0; q < PT / 4; ++q) {
      const int rr = r0 + 4 * q;
      WtT[((int64_t)tj * PT + rr) * mp + (int64_t)ti * PT + c] = tile[c][rr];
    }
  }
  const double a = block_sum_d(swt, red);
  const double b = block_sum_d(sw, red);
  if (threadIdx.x == 0) {
    const int blk = blockIdx.y * gridDim.x + blockIdx.x;
    part_wt[blk] = a;
    part_w[blk] = b;
  }
}

__global__ __launch_bounds__(256) void finalize_norms_kernel(const double* part_wt,
                                                             const double* part_w, int nparts,
                                                             double mnr, DevStats* st) {
  __shared__ double red[256];
  double a = 0.0, b = 0.0;
  for (int q = threadIdx.x; q < nparts; q += 256) {
    a += part_wt[q];
    b += part_w[q];
  }
  a = block_sum_d(a, red);
  b = block_sum_d(b, red);
  if (threadIdx.x == 0) {
    st->sumsq_wt = a;
    st->sumsq_w = b;
    st->sigma0 = pow(a / mnr, 0.25);
  }
}

__global__ void init_copy_kernel(const float* __restrict__ src, int64_t rows, int64_t r,
                                 int64_t lds, float* __restrict__ dst, float* __restrict__ dst2,
                                 int rp, int64_t total, int use_sigma, const DevStats* st) {
  const float scale = use_sigma ? (float)st->sigma0 : 1.0f;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = q / rp, k = q % rp;
    const float v = (i < rows && k < r) ? scale * src[i * lds + k] : 0.0f;
    dst[q] = v;
    if (dst2) dst2[q] = v;
  }
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): 10 rounds of two 32x32->64 multiplies with the
// published multipliers and Weyl key increments.
__device__ inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

// Element e of the (rows x r) draw uses Philox block q = e / 4 with counter
// (q_lo, q_hi, stream_id, 0) and key (seed_lo, seed_hi); the block's words
// (x0, x1), (x2, x3) become two Box-Muller pairs, normal e % 4 of the four.
// Uniforms u = (x >> 8 + 0.5) / 2^24 in (0, 1); normal pair
// sqrt(-2 ln u1) (cos 2 pi u2, sin 2 pi u2), evaluated in double.
__global__ void init_philox_kernel(uint64_t seed, uint32_t stream_id, int64_t rows, int64_t r,
                                   float* __restrict__ dst, float* __restrict__ dst2, int rp,
                                   int64_t total, const DevStats* st) {
  const float scale = (float)st->sigma0;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = q / rp, k = q % rp;
    float v = 0.0f;
    if (i < rows && k < r) {
      const uint64_t e = (uint64_t)(i * r + k);
      const uint64_t blk = e >> 2;
      uint32_t c[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream_id, 0u};
      philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
      const int which = (int)(e & 3);
      const uint32_t xa = c[(which >> 1) * 2], xb = c[(which >> 1) * 2 + 1];
      const double u1 = ((double)(xa >> 8) + 0.5) * (1.0 / 16777216.0);
      const double u2 = ((double)(xb >> 8) + 0.5) * (1.0 / 16777216.0);
      const double rad = sqrt(-2.0 * log(u1));
      const double ang = 6.283185307179586 * u2;
      const double nrm = (which & 1) ? rad * sin(ang) : rad * cos(ang);
      v = scale * (float)nrm;
    }
    dst[q] = v;
    if (dst2) dst2[q] = v;
  }
}

// dst (cols x rows, ld ldd) = src^T for src (rows x cols, ld lds); 32 x 32
// tiles through LDS, rows and cols multiples of 32.
__global__ __launch_bounds__(256) void transpose_kernel(const float* __restrict__ src,
                                                        int64_t lds, float* __restrict__ dst,
                                                        int64_t ldd) {
  __shared__ float tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) tile[ty + 8 * q][tx] = src[(r0 + ty + 8 * q) * lds + c0 + tx];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[(c0 + ty + 8 * q) * ldd + r0 + tx] = tile[tx][ty + 8 * q];
}

__global__ void zero_kernel(float* p, size_t n) {
  for (size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x; q < n;
       q += (size_t)gridDim.x * blockDim.x)
    p[q] = 0.0f;
}

__global__ void add_compact_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                   int64_t rows, int64_t r, int rp, float* __restrict__ out) {
  const int64_t total = rows * r;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = q / r, k = q % r;
    out[q] = A[i * rp + k] + B[i * rp + k];
  }
}

__global__ void set_diag_kernel(float* A, int64_t lda, int from, int to, float val) {
  const int i = from + blockIdx.x * blockDim.x + threadIdx.x;
  if (i < to) A[(int64_t)i * lda + i] = val;
}

inline unsigned grid_for(int64_t total, int64_t per = 256, int64_t cap = 16384) {
  int64_t g = (total + per - 1) / per;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_stats_init(DevStats* st, hipStream_t s) {
  hipLaunchKernelGGL(stats_init_kernel, dim3(1), dim3(1), 0, s, st);
  return hipGetLastError();
}

hipError_t launch_check_precond(const float* d_out, int64_t m, const float* d_in, int64_t n,
                                DevStats* st, hipStream_t s) {
  hipLaunchKernelGGL(check_precond_kernel, dim3(grid_for(m + n, 256, 1024)), dim3(256), 0, s,
                     d_out, m, d_in, n, st);
  return hipGetLastError();
}

int precondition_nblocks(int mp, int np_) { return (mp / PT) * (np_ / PT); }

hipError_t launch_precondition(const float* W, int64_t ldw, int64_t m, int64_t n,
                               const float* d_out, const float* d_in, float* Wt, float* WtT,
                               int mp, int np_, double* part_wt, double* part_w, DevStats* st,
                               hipStream_t s) {
  if (mp % PT || np_ % PT) return hipErrorInvalidValue;
  dim3 grid(np_ / PT, mp / PT);
  hipLaunchKernelGGL(precondition_kernel, grid, dim3(256), 0, s, W, ldw, m, n, d_out, d_in, Wt,
                     WtT, mp, np_, part_wt, part_w, st);
  return hipGetLastError();
}

hipError_t launch_finalize_norms(const double* part_wt, const double* part_w, int nparts,
                                 int64_t m, int64_t n, int64_t r, DevStats* st, hipStream_t s) {
  hipLaunchKernelGGL(finalize_norms_kernel, dim3(1), dim3(256), 0, s, part_wt, part_w, nparts,
                     (double)m * (double)n * (double)r, st);
  return hipGetLastError();
}

hipError_t launch_init_copy(const float* src, int64_t rows, int64_t r, int64_t lds, float* dst,
                            float* dst2, int rows_pad, int rp, bool use_sigma,
                            const DevStats* st, hipStream_t s) {
  const int64_t total = (int64_t)rows_pad * rp;
  hipLaunchKernelGGL(init_copy_kernel, dim3(grid_for(total)), dim3(256), 0, s, src, rows, r, lds,
                     dst, dst2, rp, total, use_sigma ? 1 : 0, st);
  return hipGetLastError();
}

hipError_t launch_init_philox(uint64_t seed, uint32_t stream_id, int64_t rows, int64_t r,
                              float* dst, float* dst2, int rows_pad, int rp, const DevStats* st,
                              hipStream_t s) {
  const int64_t total = (int64_t)rows_pad * rp;
  hipLaunchKernelGGL(init_philox_kernel, dim3(grid_for(total)), dim3(256), 0, s, seed, stream_id,
                     rows, r, dst, dst2, rp, total, st);
  return hipGetLastError();
}

hipError_t launch_add_compact(const float* A, const float* B, int64_t rows, int64_t r, int rp,
                              float* out, hipStream_t s) {
  hipLaunchKernelGGL(add_compact_kernel, dim3(grid_for(rows * r)), dim3(256), 0, s, A, B, rows, r,
                     rp, out);
  return hipGetLastError();
}

hipError_t launch_set_diag(float* A, int64_t lda, int from, int to, float val, hipStream_t s) {
  if (to <= from) return hipSuccess;
  hipLaunchKernelGGL(set_diag_kernel, dim3((to - from + 255) / 256), dim3(256), 0, s, A, lda, from,
                     to, val);
  return hipGetLastError();
}

hipError_t launch_transpose(const float* src, int64_t rows, int64_t cols, int64_t lds, float* dst,
                            int64_t ldd, hipStream_t s) {
  if (rows % 32 || cols % 32 || rows <= 0 || cols <= 0 || lds < cols || ldd < rows ||
      rows / 32 > 65535)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)(cols / 32), (unsigned)(rows / 32)),
                     dim3(256), 0, s, src, lds, dst, ldd);
  return hipGetLastError();
}

hipError_t launch_zero(float* p, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for((int64_t)n)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// Whether consecutive workgroups of a 256-workgroup launch go to consecutive
// XCDs (the layout the pinned chain and the XCD-7-free GEMM rely on): one
// probe launch, checked on the host. Synchronous; called once per handle.
namespace {
__global__ void xcd_probe_kernel(int* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcd_id();
}
}  // namespace

hipError_t xcd_round_robin_ok(bool* ok) {
  *ok = false;
  int* d = nullptr;
  hipError_t e = hipMalloc((void**)&d, 256 * sizeof(int));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(xcd_probe_kernel, dim3(256), dim3(64), 0, 0, d);
  int h[256];
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost);
  (void)hipFree(d);
  if (e != hipSuccess) return e;
  bool good = true;
  for (int b = 0; b < 256; ++b) good = good && h[b] == (h[0] + b) % 8;
  *ok = good;
  return hipSuccess;
}

}  // namespace nq
