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

// The same row dots for up to 16 inputs at once on the bf16 matrix cores,
// exactly: +-1 is exact in bf16, and each input x is split into three bf16
// terms x = h + m + l by truncation (h = the top 16 bits of x, m the top 16
// bits of x - h, l = x - h - m, which has at most 8 significant bits), so
// every product is exact and only the fp32 accumulation rounds.
// v_mfma_f32_16x16x32_bf16 takes A[b][k] from lane b + 16 (k / 8), element
// k % 8, B[k][n] from lane n + 16 (k / 8), and leaves D[4 (l / 16) + v][l % 16]
// in lane l, element v. The order of k within a product is free, so lane
// group g (lanes 16 g .. 16 g + 15) of wave w takes word 4 g + w of the
// stage and, in step s (0..3), its bits 4 s + d and 4 s + d + 16 (d = 0..3)
// as elements 2 d and 2 d + 1. Both land at bits 15 and 31 of one dword with
// a single shift, and (w << (15 - 4 s - d)) & 0x80008000 | 0x3F803F80 is
// the pair (-+1, -+1) in bf16: bit 1 gives -1, so the accumulator holds
// minus the row dot and is negated at the end (exact). The inputs are
// staged in LDS in the same pair order: dword j (< 16) of a word holds
// (x[32 w + j], x[32 w + j + 16]) as bf16, one array per term.
//
// A workgroup takes RT row tiles of 16 rows; a stage is 16 words (512
// columns), of which each wave takes four, for all RT tiles; the waves'
// partial tiles are added through LDS in wave order at the end. The next
// stage's inputs and sign words are fetched into registers while the
// current one computes. Loads go through buffer descriptors: an element
// outside the inputs, the rows or the workgroup's words gets an offset past
// the descriptor's range and reads 0, so no load needs a branch.
// Sums run in a fixed order.
constexpr int kBfWords = 16;                   // words per stage
constexpr int kBfRow = kBfWords * 16 + 4;      // dwords per staged input row (+ pad)
constexpr uint32_t kBfOut = 0x80000000u;       // an offset past every descriptor's range
constexpr int kBufFlags = 0x00020000;          // raw buffer, 32-bit data

template <int RT, bool PRE>
__global__ __launch_bounds__(256) void bin_bf16_kernel(
    const uint32_t* __restrict__ bits, int64_t ldw, int64_t rows, int64_t cols,
    const float* __restrict__ v, int64_t ldv, const float* __restrict__ pre,
    const float* __restrict__ post, float* __restrict__ out, int64_t ldo, int64_t ostride,
    int64_t wsplit, int64_t B) {
  __shared__ __align__(16) uint32_t zs[3][16][kBfRow];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int64_t b0 = (int64_t)blockIdx.y * 16;
  const int64_t row0 = (int64_t)blockIdx.x * (16 * RT);
  const int64_t nw = (cols + 31) / 32;
  const int64_t w_lo = (int64_t)blockIdx.z * wsplit;
  const int64_t w_hi = min(nw, w_lo + wsplit);
  out += (int64_t)blockIdx.z * ostride;
  // inputs b0 .. b0 + nb - 1, columns < cols: the descriptor ends after the
  // last one (rows past nb start beyond it, as ldv >= cols)
  const int64_t nb = min<int64_t>(16, B - b0);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(v + b0 * ldv), (short)0, (int)(((nb - 1) * ldv + cols) * 4), kBufFlags);
  // rows row0 .. min(rows, row0 + 16 RT) - 1, every word of each
  const int64_t nr = min<int64_t>(16 * RT, rows - row0);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(bits + row0 * ldw), (short)0, (int)(((nr - 1) * ldw + nw) * 4), kBufFlags);
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(PRE ? pre : v), (short)0, PRE ? (int)(cols * 4) : 0, kBufFlags);
  // staging map: thread t takes pair j = t % 16 of word t / 16 for each of
  // the 16 inputs. Byte offsets are 32-bit: a valid one is below 2^31, an
  // invalid one has bit 31 set, and no sum passes 2^32 (the host bounds the
  // strides).
  const int sj = threadIdx.x & 15, sw = threadIdx.x >> 4;
  const uint32_t bro = (uint32_t)(li * ldw * 4);   // this lane's row in a tile
  float xa[16], xb[16], pa = 1.0f, pb = 1.0f;   // raw inputs and their scales
  uint32_t bw[RT];
  auto fetch = [&](int64_t wst) {
    const int64_t w = wst + sw;
    const int64_t ca = w * 32 + sj, cb = ca + 16;
    const bool okw = w < w_hi;
    const uint32_t oa = (uint32_t)(ca * 4) | (okw && ca < cols ? 0u : kBfOut);
    const uint32_t ob = (uint32_t)(cb * 4) | (okw && cb < cols ? 0u : kBfOut);
    if (PRE) {
      pa = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pr, oa, 0, 0));
      pb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pr, ob, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t ro = (uint32_t)(u * ldv * 4);
      const float ya = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, oa + ro, 0, 0));
      const float yb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(vr, ob + ro, 0, 0));
      xa[u] = ya;
      xb[u] = yb;
    }
    const int64_t w2 = wst + 4 * g + wave;   // this lane's word
    const uint32_t wo = (uint32_t)(w2 * 4) | (w2 < w_hi ? 0u : kBfOut);
#pragma unroll
    for (int t = 0; t < RT; ++t)
      bw[t] = __builtin_amdgcn_raw_buffer_load_b32(br, bro + (uint32_t)(16 * t * ldw * 4) + wo, 0, 0);
  };
  // the sign masks held in registers, so that each dword of signs takes a
  // shift and one and-or
  uint32_t smask = 0x80008000u, sone = 0x3F803F80u;
  asm volatile("" : "+v"(smask), "+v"(sone));
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (w_lo < w_hi) fetch(w_lo);
  for (int64_t wst = w_lo; wst < w_hi; wst += kBfWords) {
    __syncthreads();  // the previous stage's terms are consumed
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float xu = PRE ? xa[u] * pa : xa[u], yu = PRE ? xb[u] * pb : xb[u];
      const uint32_t ua = __float_as_uint(xu), ub = __float_as_uint(yu);
      const float ra = xu - __uint_as_float(ua & 0xffff0000u);
      const float rb = yu - __uint_as_float(ub & 0xffff0000u);
      const uint32_t va = __float_as_uint(ra), vb = __float_as_uint(rb);
      const float la = ra - __uint_as_float(va & 0xffff0000u);
      const float lb = rb - __uint_as_float(vb & 0xffff0000u);
      const uint32_t wa = __float_as_uint(la), wb = __float_as_uint(lb);
      uint32_t* z = &zs[0][u][sw * 16 + sj];
      z[0] = (ua >> 16) | (ub & 0xffff0000u);
      z[16 * kBfRow] = (va >> 16) | (vb & 0xffff0000u);
      z[32 * kBfRow] = (wa >> 16) | (wb & 0xffff0000u);
    }
    __syncthreads();
    uint32_t bc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) bc[t] = bw[t];
    if (wst + kBfWords < w_hi) fetch(wst + kBfWords);
    const int wl = 4 * g + wave;   // this lane's word in the stage
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = li * kBfRow + wl * 16 + 4 * s;
      const bf16x8 ah = __builtin_bit_cast(bf16x8, *(const u32x4*)&zs[0][0][off]);
      const bf16x8 am = __builtin_bit_cast(bf16x8, *(const u32x4*)&zs[1][0][off]);
      const bf16x8 al = __builtin_bit_cast(bf16x8, *(const u32x4*)&zs[2][0][off]);
      bf16x8 bs[RT];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        u32x4 sg;
#pragma unroll
        for (int d = 0; d < 4; ++d) sg[d] = ((bc[t] << (15 - 4 * s - d)) & smask) | sone;
        bs[t] = __builtin_bit_cast(bf16x8, sg);
      }
      // the terms in order h, m, l for every tile; consecutive products
      // are independent
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bs[t], acc[t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bs[t], acc[t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bs[t], acc[t], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with the staged terms
  f32x4* red = (f32x4*)&zs[0][0][0];   // [wave][t][lane]
#pragma unroll
  for (int t = 0; t < RT; ++t) red[(wave * RT + t) * 64 + lane] = acc[t];
  __syncthreads();
  // wave w finishes tiles w, w + 4, ...: the four partials in wave order
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    if ((t & 3) != wave) continue;
    const f32x4 a = ((red[(0 * RT + t) * 64 + lane] + red[(1 * RT + t) * 64 + lane]) +
                     red[(2 * RT + t) * 64 + lane]) +
                    red[(3 * RT + t) * 64 + lane];
    const int64_t n = row0 + 16 * t + li;
    if (n >= rows) continue;
    const float pn = post ? post[n] : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = b0 + 4 * g + q;
      if (b < B) out[b * ldo + n] = post ? -a[q] * pn : -a[q];
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

// The bf16 matrix-core row dots: workgroups of RT row tiles whose waves
// split the words, RT as large as leaves at least kBfMinWgs workgroups (one
// tile when even that does not). More rows per workgroup share each staged
// (and split) input among more tiles; more workgroups fill the chip.
constexpr int64_t kBfMinWgs = 512;

template <int RT, bool PRE>
void launch_bf16(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
                 int64_t ldv, const float* pre, const float* post, float* out, int64_t ldo,
                 int64_t ostride, int split, int64_t wsplit, int64_t B, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 16 * RT - 1) / (16 * RT)), (unsigned)((B + 15) / 16),
                  (unsigned)split);
  hipLaunchKernelGGL((bin_bf16_kernel<RT, PRE>), grid, dim3(256), 0, s, bits, ldw, rows, cols, v,
                     ldv, pre, post, out, ldo, ostride, wsplit, B);
}

template <bool PRE>
void rowdot_bf16_t(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
                   int64_t ldv, const float* pre, const float* post, float* out, int64_t ldo,
                   int64_t ostride, int split, int64_t B, hipStream_t s) {
  const int64_t nw = (cols + 31) / 32;
  const int64_t wsplit = ((nw + split - 1) / split + kBfWords - 1) / kBfWords * kBfWords;
  const int64_t bt = (B + 15) / 16;
  auto wgs = [&](int rt) { return (rows + 16 * rt - 1) / (16 * rt) * bt * split; };
  if (wgs(8) >= kBfMinWgs)
    launch_bf16<8, PRE>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, ostride, split, wsplit, B, s);
  else if (wgs(4) >= kBfMinWgs)
    launch_bf16<4, PRE>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, ostride, split, wsplit, B, s);
  else if (wgs(2) >= kBfMinWgs)
    launch_bf16<2, PRE>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, ostride, split, wsplit, B, s);
  else
    launch_bf16<1, PRE>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, ostride, split, wsplit, B, s);
}

void rowdot_bf16(const uint32_t* bits, int64_t ldw, int64_t rows, int64_t cols, const float* v,
                 int64_t ldv, const float* pre, const float* post, float* out, int64_t ldo,
                 int64_t ostride, int split, int64_t B, hipStream_t s) {
  if (pre)
    rowdot_bf16_t<true>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, ostride, split, B, s);
  else
    rowdot_bf16_t<false>(bits, ldw, rows, cols, v, ldv, pre, post, out, ldo, ostride, split, B, s);
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
      (B + 15) / 16 > 65535 || n > 0x7fffffff || r > 0x7fffffff)
    return hipErrorInvalidValue;
  // the matrix-core kernel's 32-bit byte offsets: 16 rows of an input plus
  // a stage past its width, or 128 rows of signs plus a row's words, stay
  // below 2^31 bytes
  if (B >= 9 && (16 * std::max(ldx, r) + std::max(n, r) + 1024) * 4 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  if (B >= 9 && (128 * std::max(ldu, ldvt) + std::max(ldu, ldvt)) * 4 >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  // T = (X * s2) S_V: the r rows of S_V^T against x, their words split over
  // sp workgroups, each writing a partial T (sp x B x r)
  if (B >= 9) {
    // nine or more inputs: the matrix-core form, 16 inputs per pass (one
    // pass costs about what four passes of two inputs through the tables
    // cost); the first product split as below, counted in 64-row blocks
    const int64_t wgs = ((r + 63) / 64) * ((B + 15) / 16);
    int64_t sp = std::min<int64_t>((1024 + wgs - 1) / wgs, kBinSplit);
    sp = std::max<int64_t>(1, std::min<int64_t>(sp, ((n + 31) / 32 + kBfWords - 1) / kBfWords));
    rowdot_bf16(svt, ldvt, r, n, X, ldx, s2, nullptr, T, r, B * r, (int)sp, B, s);
    // the partials summed once (in slot order) rather than by every row
    // block of the second product while it stages its input
    if (sp > 1) {
      const int64_t ne = B * r;
      hipLaunchKernelGGL(bin_sum_partials_kernel,
                         dim3((unsigned)std::min<int64_t>((ne + 255) / 256, 4096)), dim3(256), 0, s,
                         T, (int)sp, ne, ne);
    }
    rowdot_bf16(su, ldu, m, r, T, r, nullptr, s1, Y, ldy, 0, 1, B, s);
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
