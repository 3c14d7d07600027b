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
// Up to eight inputs go through bin_rowdot_kernel (two per pass), nine or
// more through bin_mfma_kernel (below), 16 inputs per pass on the matrix
// cores. The first product's rows are long (n columns), so their words are
// split over up to kBinSplit workgroups (grid z), each writing a partial T;
// the second product sums the partials in order as it stages its input.
//
// bin_rowdot_kernel: four waves, RPW rows per wave; lane l holds word l of
// a 64-word (2048-column) chunk of each of its rows. For the chunk the
// workgroup builds, per group of 4 columns, the 16 signed sums
// +-x0 +-x1 +-x2 +-x3 in LDS, laid out [nibble index][value][word] so that
// the 64 lanes' lookups hit distinct banks. A row then costs one lookup and
// one add per 4 bits instead of a select and an add per bit. The words are
// fetched before the tables are built. Each lane adds its 8 lookups per word
// in order, then the wave sums its lanes in a fixed tree: the result does
// not depend on timing. Bits past `cols` in a row's last word meet x = 0
// there, so they add nothing.
#include "common.h"

#include <algorithm>
#include <mutex>
#include <vector>

namespace nq {
namespace {

constexpr int CW = 64;   // words per column chunk, one per lane

__device__ inline float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int BT, int RPW, int NS>
__global__ __launch_bounds__(256) void bin_rowdot_kernel(
    const uint32_t* __restrict__ bits, int64_t ldw, int64_t rows, int64_t cols,
    const float* __restrict__ v, int64_t ldv, int nsum, int64_t vstride,
    const float* __restrict__ pre, const float* __restrict__ post, float* __restrict__ out,
    int64_t ldo, int64_t ostride, int64_t wsplit, int64_t B) {
  // tab[b][j][q][w]: sum over the 4 columns 32 w + 4 j + t (t = 0..3) of
  // (bit t of q ? +x : -x), for word w of the chunk and nibble j of it
  __shared__ float tab[BT][8][16][CW];
  // the chunk's inputs, word-major with a pad so that the table builders
  // (one word per lane) read distinct banks
  __shared__ float xs[BT][CW][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b0 = (int64_t)blockIdx.y * BT;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * RPW;
  // this workgroup's words of each row: [w_lo, w_hi)
  const int64_t w_lo = (int64_t)blockIdx.z * wsplit;
  const int64_t nwords = min((cols + 31) / 32, w_lo + wsplit);
  out += (int64_t)blockIdx.z * ostride;
  float acc[RPW][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.0f;
  // table builder: word tw of the chunk, nibbles tj and tj + 1
  const int tw = threadIdx.x & 63, tj = 2 * (threadIdx.x >> 6);
  for (int64_t cw0 = w_lo; cw0 < nwords; cw0 += CW) {
    const int64_t w = cw0 + lane;
    uint32_t word[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      word[r] = (row0 + r < rows && w < nwords) ? bits[(row0 + r) * ldw + w] : 0u;
    __syncthreads();  // every wave is done with the previous chunk's tables
    // inputs of the chunk, coalesced: element e is column 32 cw0 + e, the
    // sum of nsum (<= NS) partial vectors in order; every load of a pass is
    // issued before the sums
#pragma unroll
    for (int e0 = 0; e0 < BT * 32 * CW; e0 += 256 * 4) {
      float part[4][NS];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + 256 * u + threadIdx.x;
        const int b = e / (32 * CW), k = e % (32 * CW);
        const int64_t c = cw0 * 32 + k;
        const bool ok = b0 + b < B && c < cols;
        const float* vp = v + (b0 + b) * ldv + c;
#pragma unroll
        for (int z = 0; z < NS; ++z) part[u][z] = ok && z < nsum ? vp[z * vstride] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + 256 * u + threadIdx.x;
        const int b = e / (32 * CW), k = e % (32 * CW);
        const int64_t c = cw0 * 32 + k;
        float y = part[u][0];
#pragma unroll
        for (int z = 1; z < NS; ++z)
          if (z < nsum) y += part[u][z];
        if (pre && b0 + b < B && c < cols) y *= pre[c];
        xs[b][k >> 5][k & 31] = y;
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < BT; ++b) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = tj + h;
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = xs[b][tw][4 * j + t];
        // q = 0 is -x0 - x1 - x2 - x3; setting bit t adds 2 x_t
        const float base = -x[0] - x[1] - x[2] - x[3];
        const float d0 = 2.0f * x[0], d1 = 2.0f * x[1], d2 = 2.0f * x[2], d3 = 2.0f * x[3];
        float* tq = &tab[b][j][0][tw];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          float e = base;
          if (q & 1) e += d0;
          if (q & 2) e += d1;
          if (q & 4) e += d2;
          if (q & 8) e += d3;
          tq[q * CW] = e;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        const int q = (word[r] >> (4 * j)) & 15u;
#pragma unroll
        for (int b = 0; b < BT; ++b) acc[r][b] += tab[b][j][q][lane];
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

// The same row dots for up to 16 inputs at once, on the matrix cores:
// out[b][n] = sum_k v[b][k] sign(n, k), i.e. a (B x K) x (K x N) product
// whose right operand is +-1, exact in fp32. v_mfma_f32_16x16x4f32 takes
// A[b][k] for b = lane % 16, k = lane / 16 (from the inputs staged in LDS)
// and B[k][n] for n = lane % 16 (+-1 from bit k of row n's word); lane l
// ends with out[4 (l / 16) + v][n]. Inputs are staged 256 columns at a time
// (the sum of nsum partial vectors, times pre). Two layouts:
//   SPLITW: a workgroup takes 16 rows and its four waves split each stage's
//     8 words (two each), so a wave's chain of dependent matrix steps is a
//     quarter of the row's; the waves' partial tiles are added through LDS
//     in wave order at the end (for grids that would otherwise be small);
//   otherwise: 64 rows, 16 per wave, each wave taking every word (each
//     staged input serves four times the rows; for wide grids).
// Sums run in a fixed order.
template <int NS, bool SPLITW>
__global__ __launch_bounds__(256) void bin_mfma_kernel(
    const uint32_t* __restrict__ bits, int64_t ldw, int64_t rows, int64_t cols,
    const float* __restrict__ v, int64_t ldv, int nsum, int64_t vstride,
    const float* __restrict__ pre, const float* __restrict__ post, float* __restrict__ out,
    int64_t ldo, int64_t ostride, int64_t wsplit, int64_t B) {
  constexpr int KC = 256;                 // input columns per stage
  constexpr int WPW = SPLITW ? KC / 32 / 4 : KC / 32;  // words per wave per stage
  __shared__ float zs[16][KC + 4];
  __shared__ f32x4 red[3][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b0 = (int64_t)blockIdx.y * 16;
  const int64_t n = (SPLITW ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + wave) * 16 + (lane & 15);
  const int64_t nw = (cols + 31) / 32;
  const int64_t w_lo = (int64_t)blockIdx.z * wsplit;
  const int64_t w_hi = min(nw, w_lo + wsplit);
  out += (int64_t)blockIdx.z * ostride;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const int kq = lane >> 4;               // this lane's k within a step of 4
  for (int64_t wc = w_lo; wc < w_hi; wc += KC / 32) {
    __syncthreads();  // the previous stage's inputs are consumed
    // inputs b0 .. b0 + 15, columns 32 wc .. + KC, coalesced
#pragma unroll
    for (int u = 0; u < 16 * KC / 256; ++u) {
      const int e = u * 256 + threadIdx.x;
      const int bb = e / KC, k = e % KC;
      const int64_t c = wc * 32 + k;
      const bool ok = b0 + bb < B && c < cols && wc * 32 + k < w_hi * 32;
      const float* vp = v + (b0 + bb) * ldv + c;
      float y = ok ? vp[0] : 0.0f;
#pragma unroll
      for (int z = 1; z < NS; ++z) {
        const float t = ok && z < nsum ? vp[z * vstride] : 0.0f;
        if (z < nsum) y += t;
      }
      if (ok && pre) y *= pre[c];
      zs[bb][k] = y;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < WPW; ++u) {
      const int wi = SPLITW ? WPW * wave + u : u;   // word within the stage
      const int64_t w = wc + wi;
      if (w >= w_hi) break;
      const uint32_t word = n < rows ? bits[n * ldw + w] : 0u;
      const int kb = wi * 32;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        const int k = 4 * s8 + kq;
        const float a = zs[lane & 15][kb + k];
        const float bsg = (word >> k) & 1u ? 1.0f : -1.0f;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bsg, acc, 0, 0, 0);
      }
    }
  }
  if (SPLITW) {
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) acc = ((acc + red[0][lane]) + red[1][lane]) + red[2][lane];
  }
  if ((!SPLITW || wave == 0) && n < rows) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = b0 + 4 * kq + q;
      if (b < B) out[b * ldo + n] = post ? acc[q] * post[n] : acc[q];
    }
  }
}

// part[e] = part[e] + part[e + stride] + ... (nsum slots, added in slot
// order, the order the second product's staging would add them), for the
// n = B r elements of the first slot, in place
__global__ void bin_sum_partials_kernel(float* __restrict__ part, int nsum, int64_t stride,
                                        int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    float y = part[e];
    for (int z = 1; z < nsum; ++z) y += part[e + z * stride];
    part[e] = y;
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

// One row-dot launch: `split` workgroups share each block of rows, each
// taking wsplit words (a multiple of CW) of every row and writing its own
// partial result at out + z ostride; the input is the sum of nsum partial
// vectors v + z vstride.
template <int BT, int RPW, int NS>
void rowdot(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
            int64_t ldv, int nsum, int64_t vstride, const float* pre, const float* post,
            float* out, int64_t ldo, int64_t ostride, int split, int64_t B, hipStream_t s) {
  const int64_t nw = (cols + 31) / 32;
  const int64_t wsplit = ((nw + split - 1) / split + CW - 1) / CW * CW;
  const dim3 grid((unsigned)((rows + 4 * RPW - 1) / (4 * RPW)), (unsigned)((B + BT - 1) / BT),
                  (unsigned)split);
  hipLaunchKernelGGL((bin_rowdot_kernel<BT, RPW, NS>), grid, dim3(256), 0, s, bits, ldw, rows, cols, v, ldv,
                     nsum, vstride, pre, post, out, ldo, ostride, wsplit, B);
}

template <int NS>
void rowdot_mfma(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
                 int64_t ldv, int nsum, int64_t vstride, const float* pre, const float* post,
                 float* out, int64_t ldo, int64_t ostride, int split, int64_t B, hipStream_t s) {
  const int64_t nw = (cols + 31) / 32;
  const int64_t wsplit = ((nw + split - 1) / split + 7) / 8 * 8;
  // 16-row workgroups with the words split over the waves when 64-row ones
  // would leave the chip under-filled (fewer than 512 workgroups)
  const int64_t g64 = ((rows + 63) / 64) * ((B + 15) / 16) * split;
  if (g64 < 512) {
    const dim3 grid((unsigned)((rows + 15) / 16), (unsigned)((B + 15) / 16), (unsigned)split);
    hipLaunchKernelGGL((bin_mfma_kernel<NS, true>), grid, dim3(256), 0, s, bits, ldw, rows, cols, v,
                       ldv, nsum, vstride, pre, post, out, ldo, ostride, wsplit, B);
  } else {
    const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((B + 15) / 16), (unsigned)split);
    hipLaunchKernelGGL((bin_mfma_kernel<NS, false>), grid, dim3(256), 0, s, bits, ldw, rows, cols,
                       v, ldv, nsum, vstride, pre, post, out, ldo, ostride, wsplit, B);
  }
}

template <int RPW, int NS>
void rowdot_any(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
                int64_t ldv, int nsum, int64_t vstride, const float* pre, const float* post,
                float* out, int64_t ldo, int64_t ostride, int split, int64_t B, hipStream_t s) {
  // two inputs per workgroup at most: their tables (64 KB) and inputs fill
  // most of the LDS
  if (B == 1) rowdot<1, RPW, NS>(bits, ldw, rows, cols, v, ldv, nsum, vstride, pre, post, out, ldo, ostride, split, B, s);
  else rowdot<2, RPW, NS>(bits, ldw, rows, cols, v, ldv, nsum, vstride, pre, post, out, ldo, ostride, split, B, s);
}

// rows per wave: the first product (r rows, long rows of n columns) shares
// each chunk's tables among 64 rows per workgroup and splits its columns;
// the second (m rows of r columns) keeps 16 rows per workgroup for a wide
// grid when there are one or two inputs
constexpr int kRpw1 = 16, kRpw2 = 4;

// Workgroups sharing the rows of the first product: enough for about 1024
// workgroups in all, at most kBinSplit, at most one per 64-word chunk.
int first_split(int64_t r, int64_t n, int64_t B, int rpw) {
  const int64_t wgs = ((r + 4 * rpw - 1) / (4 * rpw)) * ((B + 1) / 2);
  int64_t sp = (1024 + wgs - 1) / wgs;
  sp = std::min<int64_t>(sp, kBinSplit);
  sp = std::min<int64_t>(sp, ((n + 31) / 32 + CW - 1) / CW);
  return (int)std::max<int64_t>(sp, 1);
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
  if ((r + 4 * kRpw2 - 1) / (4 * kRpw2) > 0x7fffffff || (m + 4 * kRpw2 - 1) / (4 * kRpw2) > 0x7fffffff ||
      (B + 15) / 16 > 65535)
    return hipErrorInvalidValue;
  // T = (X * s2) S_V: the r rows of S_V^T against x, their words split over
  // sp workgroups, each writing a partial T (sp x B x r)
  if (B >= 9) {
    // nine or more inputs: the matrix-core form, 16 inputs per pass (one
    // pass costs about what four passes of two inputs through the tables
    // cost); the first product split as below, counted in 64-row blocks
    const int64_t wgs = ((r + 63) / 64) * ((B + 15) / 16);
    int64_t sp = std::min<int64_t>((1024 + wgs - 1) / wgs, kBinSplit);
    sp = std::max<int64_t>(1, std::min<int64_t>(sp, ((n + 31) / 32 + 7) / 8));
    rowdot_mfma<1>(svt, ldvt, r, n, X, ldx, 1, 0, s2, nullptr, T, r, B * r, (int)sp, B, s);
    // the partials summed once (in slot order) rather than by every row
    // block of the second product while it stages its input
    if (sp > 1) {
      const int64_t ne = B * r;
      hipLaunchKernelGGL(bin_sum_partials_kernel,
                         dim3((unsigned)std::min<int64_t>((ne + 255) / 256, 4096)), dim3(256), 0, s,
                         T, (int)sp, ne, ne);
    }
    rowdot_mfma<1>(su, ldu, m, r, T, r, 1, 0, nullptr, s1, Y, ldy, 0, 1, B, s);
    return hipGetLastError();
  }
  // (below 4096 rows and for one or two inputs, 16 rows per workgroup: 64
  // would leave most CUs idle)
  const int rpw1 = r >= 4096 || B > 2 ? kRpw1 : kRpw2;
  const int sp = first_split(r, n, B, rpw1);
  if (rpw1 == kRpw1)
    rowdot_any<kRpw1, 1>(svt, ldvt, r, n, X, ldx, 1, 0, s2, nullptr, T, r, B * r, sp, B, s);
  else
    rowdot_any<kRpw2, 1>(svt, ldvt, r, n, X, ldx, 1, 0, s2, nullptr, T, r, B * r, sp, B, s);
  // Y = s1 * (T S_U^T): the m rows of S_U against the sum of the partials
  // (more than two inputs: 64 rows per workgroup, so each table serves more
  // rows; one or two: 16, for a wider grid). With more than two inputs the
  // partials are summed once first (in slot order, as the staging would):
  // each of the m / 64 row blocks would otherwise load all of them.
  if (B > 2) {
    if (sp > 1) {
      const int64_t ne = B * r;
      hipLaunchKernelGGL(bin_sum_partials_kernel,
                         dim3((unsigned)std::min<int64_t>((ne + 255) / 256, 4096)), dim3(256), 0, s,
                         T, sp, ne, ne);
    }
    rowdot_any<kRpw1, 1>(su, ldu, m, r, T, r, 1, 0, nullptr, s1, Y, ldy, 0, 1, B, s);
  } else {
    rowdot_any<kRpw2, kBinSplit>(su, ldu, m, r, T, r, sp, B * r, nullptr, s1, Y, ldy, 0, 1, B, s);
  }
  return hipGetLastError();
}

}  // namespace nq

// ---------------------------------------------------------------- fixed scratch
// The partial projections of launch_binary_matmul for callers that cannot
// allocate: one array per GPU, held from the first use until the process
// ends. Every slot the second product reads is written by the first product
// of the same call, so nothing needs clearing between calls; two calls that
// overlap on one GPU share the array and race.
namespace nq {

static __device__ __align__(256) float scratch[kBinScratchFloats];

hipError_t binmm_fixed_scratch(float** out) {
  static std::mutex mu;
  static std::vector<float*> ptrs;
  int dev = 0, count = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= count) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs.size() < (size_t)count) ptrs.resize((size_t)count, nullptr);
  if (!ptrs[dev]) {
    // the array's name is a host-side stand-in: the device copy's address
    // comes from the runtime, once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = (float*)p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace nq
