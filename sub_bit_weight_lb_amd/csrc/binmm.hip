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
// kernel serves both. The first product's rows are long (n columns), so
// their words are split over up to kBinSplit workgroups (grid z), each
// writing a partial T, summed in slot order before the second product.
//
// One input goes through bin_rowdot_kernel (lookup tables, below); two or
// more through the bf16 matrix cores: bin_split_kernel writes the inputs as
// exact bf16 terms in the order the matrix instructions take them, and
// bin_bf16_kernel multiplies them by the signs, 16 inputs per pass.
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------- bf16 path
// The row dots for 16 inputs at once on the bf16 matrix cores, exactly: +-1
// is exact in bf16, and each input x splits into three bf16 terms
// x = h + m + l by truncation (h = the top 16 bits of x, m the top 16 bits
// of x - h, l = x - h - m, which has at most 8 significant bits), so every
// product is exact and only the fp32 accumulation rounds.
//
// v_mfma_f32_16x16x32_bf16 takes A[b][k] from lane b + 16 (k / 8), element
// k % 8, B[k][n] from lane n + 16 (k / 8), and leaves D[4 (l / 16) + v][l % 16]
// in lane l, element v. The order of k within a product is free. Words go
// in groups of four; in step s (0..3) of a group, lane group g (lanes
// 16 g .. 16 g + 15) takes word g of the group, bits 4 s + d and 4 s + d + 16
// (d = 0..3) as elements 2 d and 2 d + 1. Both bits land at 15 and 31 of
// one dword with a single shift, and (w << (15 - 4 s - d)) & 0x80008000 |
// 0x3F803F80 is the pair (-+1, -+1) in bf16: bit 1 gives -1, so the
// accumulator holds minus the row dot and is negated at the end (exact).
//
// Term layout (written by bin_split_kernel, one block of kPlaneFloats
// dwords per 16-input tile bt and word group q):
//   block (bt, q), term p (h, m, l), step s, word g, input i: four dwords,
//   dword d = bf16 pair (x[32 w + j], x[32 w + j + 16]), w = 4 q + g,
//   j = 4 s + d,
// so lane (g, i) reads its fragment of step s as one 16-byte load and a
// wave's 64 lanes read 1 KB in a row. Inputs past B or past the width are 0.
constexpr int kPlaneFloats = 3 * 4 * 4 * 16 * 4;   // dwords per (tile, word group)
constexpr uint32_t kBfOut = 0x80000000u;            // an offset past every descriptor's range
constexpr int kBufFlags = 0x00020000;               // raw buffer, 32-bit data

// planes <- the terms of v (B x cols, ld ldv): the sum of nsum (at most
// NS) partial vectors v + z vstride (added in slot order), times pre
// if given; ngw word groups per tile. One thread per dword of each term.
template <int NS>
__global__ __launch_bounds__(256) void bin_split_kernel(const float* __restrict__ v, int64_t ldv,
                                                        int64_t B, int64_t cols, int nsum,
                                                        int64_t vstride,
                                                        const float* __restrict__ pre,
                                                        uint32_t* __restrict__ planes,
                                                        int64_t ngw) {
  const int64_t total = (B + 15) / 16 * ngw * 1024;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int o = (int)(e & 1023);
    const int64_t blk = e >> 10;                  // bt * ngw + q
    const int64_t bt = blk / ngw, q = blk % ngw;
    const int d = o & 3, i = (o >> 2) & 15, g = (o >> 6) & 3, st = o >> 8;
    const int64_t b = bt * 16 + i;
    const int64_t ca = (q * 4 + g) * 32 + 4 * st + d, cb = ca + 16;
    // every load is issued before any add (clamped indices, no branches
    // around loads); the slots are then added in order
    float x[2], t[2][NS];
    bool ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t c = h ? cb : ca;
      ok[h] = b < B && c < cols;
      const float* vp = v + (ok[h] ? b * ldv + c : 0);
#pragma unroll
      for (int z = 0; z < NS; ++z) t[h][z] = vp[(z < nsum ? z : 0) * vstride];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float y = t[h][0];
#pragma unroll
      for (int z = 1; z < NS; ++z)
        if (z < nsum) y += t[h][z];
      if (pre) y *= pre[ok[h] ? (h ? cb : ca) : 0];
      x[h] = ok[h] ? y : 0.0f;
    }
    const uint32_t ua = __float_as_uint(x[0]), ub = __float_as_uint(x[1]);
    const float ra = x[0] - __uint_as_float(ua & 0xffff0000u);
    const float rb = x[1] - __uint_as_float(ub & 0xffff0000u);
    const uint32_t va = __float_as_uint(ra), vb = __float_as_uint(rb);
    const float la = ra - __uint_as_float(va & 0xffff0000u);
    const float lb = rb - __uint_as_float(vb & 0xffff0000u);
    const uint32_t wa = __float_as_uint(la), wb = __float_as_uint(lb);
    uint32_t* dst = planes + blk * kPlaneFloats + o;
    dst[0] = (ua >> 16) | (ub & 0xffff0000u);
    dst[1024] = (va >> 16) | (vb & 0xffff0000u);
    dst[2048] = (wa >> 16) | (wb & 0xffff0000u);
  }
}

// out[b][n] = post[n] * sum_k sign(n, k) x_b[k] from the terms. A workgroup
// takes RT row tiles of 16 rows of one 16-input tile and the
// word groups [q_lo, q_hi) of one slice (grid z); wave w takes groups
// q_lo + w, q_lo + w + 4, ... for all RT tiles, with the next group's terms
// and sign words in flight while it multiplies the current one (two
// register sets). The waves' partial tiles are added through LDS in wave
// order at the end. Loads go through buffer descriptors: a sign word past a
// row, or terms past the last word group, read 0, so no load needs a
// branch. Sums run in a fixed order.
template <int RT>
__global__ __launch_bounds__(256) void bin_bf16_kernel(
    const uint32_t* __restrict__ bits, int64_t ldw, int64_t rows, int64_t cols,
    const uint32_t* __restrict__ planes, int64_t ngw, const float* __restrict__ post,
    float* __restrict__ out, int64_t ldo, int64_t ostride, int64_t gsplit, int64_t B) {
  __shared__ f32x4 red[4 * RT * 64];
  // the wave index in a scalar register: the loop over word groups is
  // uniform per wave
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int64_t bt = blockIdx.y;
  const int64_t row0 = (int64_t)blockIdx.x * (16 * RT);
  const int64_t nw = (cols + 31) / 32;
  const int64_t q_lo = (int64_t)blockIdx.z * gsplit;
  const int64_t q_hi = min(ngw, q_lo + gsplit);
  out += (int64_t)blockIdx.z * ostride;
  // this tile's terms
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(planes + bt * ngw * kPlaneFloats), (short)0, (int)(ngw * kPlaneFloats * 4),
      kBufFlags);
  // rows row0 .. min(rows, row0 + 16 RT) - 1, every word of each (byte
  // offsets fit 32 bits: the host bounds the strides)
  const int64_t nr = min<int64_t>(16 * RT, rows - row0);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(bits + row0 * ldw), (short)0, (int)(((nr - 1) * ldw + nw) * 4), kBufFlags);
  const uint32_t bro = (uint32_t)(li * ldw * 4);   // this lane's row in a tile
  auto load = [&](u32x4 (&a)[3][4], uint32_t (&w)[RT], int64_t q) {
    // past the slice: offsets beyond the descriptor, the terms read 0
    const uint32_t qo = q < q_hi ? (uint32_t)(q * kPlaneFloats * 4) : kBfOut;
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        a[p][s] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, qo + (uint32_t)(((p * 4 + s) * 64 + lane) * 16), 0, 0));
    const int64_t w2 = 4 * q + g;   // this lane's word
    const uint32_t wo = (uint32_t)(w2 * 4) | (w2 < nw ? 0u : kBfOut);
#pragma unroll
    for (int t = 0; t < RT; ++t)
      w[t] = __builtin_amdgcn_raw_buffer_load_b32(br, bro + (uint32_t)(16 * t * ldw * 4) + wo, 0, 0);
  };
  // the sign masks held in registers, so that each dword of signs takes a
  // shift and one and-or
  uint32_t smask = 0x80008000u, sone = 0x3F803F80u;
  asm volatile("" : "+v"(smask), "+v"(sone));
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto mult = [&](const u32x4 (&a)[3][4], const uint32_t (&w)[RT]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 bs[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        u32x4 sg;
#pragma unroll
        for (int d = 0; d < 4; ++d) sg[d] = ((w[t] << (15 - 4 * s - d)) & smask) | sone;
        bs[t] = __builtin_bit_cast(bf16x8, sg);
      }
      // the terms in order h, m, l for every tile; consecutive products
      // are independent
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const bf16x8 ap = __builtin_bit_cast(bf16x8, a[p][s]);
#pragma unroll
        for (int t = 0; t < RT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bs[t], acc[t], 0, 0, 0);
      }
    }
  };
  // groups q0, q0 + 4, ... < q_hi: in pairs, the next group's loads issued
  // before the current group's products (no exit between a load and its
  // use, so the compiler keeps them apart), then an odd last group
  u32x4 a0[3][4], a1[3][4];
  uint32_t w0[RT], w1[RT];
  int64_t q = q_lo + wave;
  const int64_t nq = q < q_hi ? (q_hi - q + 3) / 4 : 0;
  if (nq > 0) load(a0, w0, q);
  int64_t k = 0;
  for (; k + 2 <= nq; k += 2, q += 8) {
    load(a1, w1, q + 4);
    __builtin_amdgcn_sched_barrier(0);
    mult(a0, w0);
    load(a0, w0, q + 8);
    __builtin_amdgcn_sched_barrier(0);
    mult(a1, w1);
  }
  if (k < nq) mult(a0, w0);
  // the four partial tiles, added in wave order
#pragma unroll
  for (int t = 0; t < RT; ++t) red[(wave * RT + t) * 64 + lane] = acc[t];
  __syncthreads();
  // wave w finishes tiles w, w + 4, ...
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if ((t & 3) != wave) continue;
    const f32x4 sum = ((red[(0 * RT + t) * 64 + lane] + red[(1 * RT + t) * 64 + lane]) +
                       red[(2 * RT + t) * 64 + lane]) +
                      red[(3 * RT + t) * 64 + lane];
    const int64_t n = row0 + 16 * t + li;
    if (n >= rows) continue;
    const float pn = post ? post[n] : 1.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t b = bt * 16 + 4 * g + v;
      if (b < B) out[b * ldo + n] = post ? -sum[v] * pn : -sum[v];
    }
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
// vectors v + z vstride. One input per workgroup.
template <int RPW, int NS>
void rowdot(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
            int64_t ldv, int nsum, int64_t vstride, const float* pre, const float* post,
            float* out, int64_t ldo, int64_t ostride, int split, hipStream_t s) {
  const int64_t nw = (cols + 31) / 32;
  const int64_t wsplit = ((nw + split - 1) / split + CW - 1) / CW * CW;
  const dim3 grid((unsigned)((rows + 4 * RPW - 1) / (4 * RPW)), 1u, (unsigned)split);
  hipLaunchKernelGGL((bin_rowdot_kernel<1, RPW, NS>), grid, dim3(256), 0, s, bits, ldw, rows,
                     cols, v, ldv, nsum, vstride, pre, post, out, ldo, ostride, wsplit, (int64_t)1);
}

// rows per wave of the one-input path: the first product (r rows, long rows
// of n columns) shares each chunk's tables among 64 rows per workgroup and
// splits its columns; the second (m rows of r columns) keeps 16 rows per
// workgroup for a wide grid
constexpr int kRpw1 = 16, kRpw2 = 4;

// Workgroups sharing the rows of the first product (one input): enough for
// about 1024 workgroups in all, at most kBinSplit, at most one per 64-word
// chunk.
int first_split(int64_t r, int64_t n, int rpw) {
  const int64_t wgs = (r + 4 * rpw - 1) / (4 * rpw);
  int64_t sp = (1024 + wgs - 1) / wgs;
  sp = std::min<int64_t>(sp, kBinSplit);
  sp = std::min<int64_t>(sp, ((n + 31) / 32 + CW - 1) / CW);
  return (int)std::max<int64_t>(sp, 1);
}

// The bf16 path: terms of the input, then the row dots, in workgroups of RT
// row tiles, RT as large as leaves at least kBfMinWgs workgroups (one tile
// when even that does not), at most 4: more rows per workgroup read each
// term fewer times over, more workgroups fill the chip, and 8 tiles (two
// waves per SIMD) measured slower on every layer shape tried.
constexpr int64_t kBfMinWgs = 256;

hipError_t split_terms(const float* v, int64_t ldv, int64_t B, int64_t cols, int nsum,
                       int64_t vstride, const float* pre, uint32_t* planes, hipStream_t s) {
  const int64_t ngw = (cols + 127) / 128;
  const int64_t total = (B + 15) / 16 * ngw * 1024;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  if (nsum < 1 || nsum > kBinSplit) return hipErrorInvalidValue;
  if (nsum == 1)
    hipLaunchKernelGGL(bin_split_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, v, ldv, B,
                       cols, nsum, vstride, pre, planes, ngw);
  else
    hipLaunchKernelGGL(bin_split_kernel<kBinSplit>, dim3((unsigned)blocks), dim3(256), 0, s, v,
                       ldv, B, cols, nsum, vstride, pre, planes, ngw);
  return hipGetLastError();
}

template <int RT>
void launch_bf16(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols,
                 const uint32_t* planes, const float* post, float* out, int64_t ldo,
                 int64_t ostride, int split, int64_t gsplit, int64_t B, hipStream_t s) {
  const int64_t ngw = (cols + 127) / 128;
  const dim3 grid((unsigned)((rows + 16 * RT - 1) / (16 * RT)), (unsigned)((B + 15) / 16),
                  (unsigned)split);
  hipLaunchKernelGGL((bin_bf16_kernel<RT>), grid, dim3(256), 0, s, bits, ldw, rows, cols, planes,
                     ngw, post, out, ldo, ostride, gsplit, B);
}

void rowdot_bf16(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols,
                 const uint32_t* planes, const float* post, float* out, int64_t ldo,
                 int64_t ostride, int split, int64_t B, hipStream_t s) {
  const int64_t ngw = (cols + 127) / 128;
  // word groups per slice: a multiple of 4, one per wave
  const int64_t gsplit = ((ngw + split - 1) / split + 3) / 4 * 4;
  const int64_t bt = (B + 15) / 16;
  auto wgs = [&](int rt) { return (rows + 16 * rt - 1) / (16 * rt) * bt * split; };
  if (wgs(4) >= kBfMinWgs)
    launch_bf16<4>(bits, ldw, rows, cols, planes, post, out, ldo, ostride, split, gsplit, B, s);
  else if (wgs(2) >= kBfMinWgs)
    launch_bf16<2>(bits, ldw, rows, cols, planes, post, out, ldo, ostride, split, gsplit, B, s);
  else
    launch_bf16<1>(bits, ldw, rows, cols, planes, post, out, ldo, ostride, split, gsplit, B, s);
}

}  // namespace

int64_t binmm_work_floats(int64_t B, int64_t n, int64_t r) {
  const int64_t part = (kBinSplit * B * r + 63) / 64 * 64;
  return part + (int64_t)kPlaneFloats * ((B + 15) / 16) * ((std::max(n, r) + 127) / 128);
}

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
                                float* Y, int64_t ldy, float* work, hipStream_t s) {
  if (m <= 0 || n <= 0 || r <= 0 || B <= 0) return hipSuccess;
  if ((r + 4 * kRpw2 - 1) / (4 * kRpw2) > 0x7fffffff || (m + 4 * kRpw2 - 1) / (4 * kRpw2) > 0x7fffffff ||
      (B + 15) / 16 > 65535)
    return hipErrorInvalidValue;
  float* T = work;   // kBinSplit partial projections, B x r each
  if (B >= 2) {
    // the matrix-core kernel's 32-bit byte offsets: 128 rows of signs plus
    // a row's words, and one tile's terms, stay below 2^31 bytes
    if ((129 * std::max(ldu, ldvt)) * 4 >= (int64_t(1) << 31) ||
        (int64_t)kPlaneFloats * 4 * ((std::max(n, r) + 127) / 128 + 8) >= (int64_t(1) << 31))
      return hipErrorInvalidValue;
    uint32_t* planes = (uint32_t*)(work + (kBinSplit * B * r + 63) / 64 * 64);
    // T = (X * s2) S_V: the r rows of S_V^T against x, their words split
    // over sp workgroups (enough for about 1024 in all, at most kBinSplit,
    // at least 16 words each), each writing a partial T (sp x B x r)
    const int64_t wgs = ((r + 63) / 64) * ((B + 15) / 16);
    int64_t sp = std::min<int64_t>((1024 + wgs - 1) / wgs, kBinSplit);
    sp = std::max<int64_t>(1, std::min<int64_t>(sp, ((n + 31) / 32 + 15) / 16));
    hipError_t e = split_terms(X, ldx, B, n, 1, 0, s2, planes, s);
    if (e != hipSuccess) return e;
    rowdot_bf16(svt, ldvt, r, n, planes, nullptr, T, r, B * r, (int)sp, B, s);
    // Y = s1 * (S_U T): the partials summed in slot order as they are split
    e = split_terms(T, r, B, r, (int)sp, B * r, nullptr, planes, s);
    if (e != hipSuccess) return e;
    rowdot_bf16(su, ldu, m, r, planes, s1, Y, ldy, 0, 1, B, s);
    return hipGetLastError();
  }
  // one input: the lookup tables (below 4096 rows, 16 rows per workgroup in
  // the first product: 64 would leave most CUs idle); the second product
  // adds the first's partials in slot order as it stages its input
  const int rpw1 = r >= 4096 ? kRpw1 : kRpw2;
  const int sp = first_split(r, n, rpw1);
  if (rpw1 == kRpw1)
    rowdot<kRpw1, 1>(svt, ldvt, r, n, X, ldx, 1, 0, s2, nullptr, T, r, r, sp, s);
  else
    rowdot<kRpw2, 1>(svt, ldvt, r, n, X, ldx, 1, 0, s2, nullptr, T, r, r, sp, s);
  rowdot<kRpw2, kBinSplit>(su, ldu, m, r, T, r, sp, r, nullptr, s1, Y, ldy, 0, 1, s);
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
