// fp32 MFMA GEMMs of the regularised solve, NanoQuant digest section 核心方法
// step (a), in "NT" form: C = A B^T with both operands stored k-contiguous.
//
//   right-hand side  R = Wt V + rho (Z - Lam): A = Wt (or Wt^T for the V-half),
//                    B = V^T (or U^T), kept in HBM beside the factors;
//   solve            U = R G^-1 = R L^-T L^-1, both triangular solves as one
//                    product with the symmetric inverse (B = G^-1 = G^-T);
//                    the epilogue also writes U^T for the next half's Gram
//                    and right-hand side;
//   Gram             G = V^T V + rho I: A = B = V^T, lower 128 x 128 tiles,
//                    split over K into partial sums (gram_reduce adds them).
//
// Main loop (256 threads, 4 waves in a 2 x 2 arrangement):
// - Tile TM x 128 with TM = 256 (one workgroup per CU) or 128 (two per CU),
//   BK = 32, each wave (TM / 2) x 64 = (TM / 64) x 2 blocks of
//   v_mfma_f32_32x32x2_f32.
// - Operands go from global memory straight into LDS with
//   buffer_load_dwordx4 ... lds (no VGPR staging; the uniform part of each
//   address in an SGPR, so a copy costs no vector instruction). Two stages:
//   the copies of step k + 1 are spread over the first half of step k's
//   MFMAs (one or two after each group of 8), early enough to land before
//   the step ends. The last step is peeled, so the loop carries no branch
//   per copy.
// - LDS rows hold 32 floats as 8 slots of 16 B; row r keeps k-quad q in slot
//   q ^ ((r >> 1) & 7). Each lane's DMA fetches the quad that belongs in its
//   slot. Fragment reads are single ds_read_b128s, free of bank conflicts
//   for 16 consecutive rows.
// - K order inside a chunk of 8: lane half h (lanes 32..63 are h = 1) feeds
//   k = 4 h + s to MFMA step s = 0..3, the same for both operands.
// - Tile order is XCD-aware: workgroup b runs on XCD b % 8, and each XCD gets
//   a contiguous range of tile indices, so row and column panels are shared
//   in its L2. Indices run down bands of 4 tile rows (tile_rc), so the 32
//   tiles an XCD holds at once form a 4 x 8 block: 4 row panels and 8
//   column panels per K step instead of 2 and 16 in row-major order, a fifth
//   fewer bytes through the XCD's L2.
#include "common.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

namespace nq {
namespace {

constexpr int BK = 32;
// MFMA groups of a step after which operand copies are issued
#ifndef NQ_DMA_SLOTS
#define NQ_DMA_SLOTS 8
#endif
constexpr int TN = 128;
constexpr int NT = 256;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over `base` (raw, byte offsets, reads past 2^31 bytes
// return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
// 16 B per lane from rsrc + voff (per lane) + soff (uniform) to LDS at
// lds + 16 * lane (wave-uniform lds). The uniform part of the address stays
// in an SGPR: no vector address arithmetic per copy.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff,
                                      float* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

template <int TM>
struct Tile {
  static constexpr int MI = TM / 64;            // 32-row blocks per wave
  static constexpr int SA = TM * BK;            // floats of one A stage
  static constexpr int SST = SA + TN * BK;      // floats of one stage (A then B)
  static constexpr int NA = TM / 32, NB = TN / 32;  // DMA instructions per wave per stage
  static constexpr int DPC = (NA + NB) / 4;     // DMA instructions per chunk of 8 k
  static constexpr int LDS_FLOATS = 2 * SST;
};

// acc += A[0:TM, k0 : k0 + 32 nk] B[0:128, same]^T for the tile whose
// operand rows start at Ag and Bg. Leaves every wave past a final barrier
// with the LDS free.
template <int TM>
__device__ __forceinline__ void nt_mainloop(const float* __restrict__ Ag, int lda,
                                            const float* __restrict__ Bg, int ldb, int k0,
                                            int nk, float* lds,
                                            f32x16 (&acc)[Tile<TM>::MI][2], int yield = 0) {
  using T = Tile<TM>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;

  // DMA instruction n of this wave covers 8 rows R .. R + 7 (A for n < NA,
  // B after); lane -> row R + lane / 8, slot lane % 8. R / 2 is a multiple
  // of 4, so the swizzle of the lane's row is (4 (n & 1) + lane / 16) & 7.
  uint32_t a_lo[2], b_lo[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int q = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7);
    a_lo[par] = (uint32_t)(((lane >> 3) * lda + 4 * q) * 4);
    b_lo[par] = (uint32_t)(((lane >> 3) * ldb + 4 * q) * 4);
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(Ag), rb = make_rsrc(Bg);
  auto dma = [&](int stage, int kk, int n) {
    float* la = lds + stage * T::SST;
    if (n < T::NA) {
      const int R = (T::NA * wave + n) * 8;
      dma16(ra, a_lo[n & 1], (R * lda + kk) * 4, la + R * BK);
    } else {
      const int i = n - T::NA;
      const int R = (T::NB * wave + i) * 8;
      dma16(rb, b_lo[i & 1], (R * ldb + kk) * 4, la + T::SA + R * BK);
    }
  };
  // fragment offsets: row (wm TM/2 + l32) of A, row (wn 64 + l32) of B,
  // slot (2 c + h) ^ sw of chunk c
  const int sw = (l32 >> 1) & 7;
  int a_rd[4], b_rd[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    a_rd[c] = (wm * (TM / 2) + l32) * BK + (((2 * c + h) ^ sw) * 4);
    b_rd[c] = T::SA + (wn * 64 + l32) * BK + (((2 * c + h) ^ sw) * 4);
  }
  f32x4 af[2][T::MI], bf[2][2];
  auto frag = [&](const float* st, int c, int slot) {
#pragma unroll
    for (int mi = 0; mi < T::MI; ++mi) af[slot][mi] = *(const f32x4*)&st[a_rd[c] + mi * 32 * BK];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) bf[slot][ni] = *(const f32x4*)&st[b_rd[c] + ni * 32 * BK];
  };
#pragma unroll
  for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;
  if (nk <= 0) return;

#pragma unroll
  for (int n = 0; n < T::NA + T::NB; ++n) dma(0, k0, n);
  // Barriers are plain s_barrier: __syncthreads() adds a release fence,
  // which would also wait for the DMA of the next stage in flight. Each
  // wave waits for its own DMA (vmcnt) and LDS reads (lgkmcnt) itself.
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
  frag(lds, 0, 0);
  // One K step; the last one (MORE false) issues no DMA. The steps before
  // it are a loop without a branch per DMA.
  auto step = [&](int kt, auto more_tag) {
    constexpr bool MORE = decltype(more_tag)::value;
    const int cs = kt & 1;
    const float* st = lds + cs * T::SST;
    const int knext = k0 + (kt + 1) * BK;
#pragma unroll
    for (int c = 0; c < BK / 8; ++c) {
      const int cur = c & 1, nxt = cur ^ 1;
      if (c + 1 < BK / 8) frag(st, c + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[cur][mi][s], bf[cur][ni][s],
                                                               acc[mi][ni], 0, 0, 0);
        if constexpr (MORE) {
          // copies n in [j N / S, (j + 1) N / S) after MFMA group j = 4 c + s
          constexpr int N = T::NA + T::NB, S = NQ_DMA_SLOTS;
          const int j = 4 * c + s;
          if (j < S) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = j * N / S; n < (j + 1) * N / S; ++n) dma(cs ^ 1, knext, n);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the other stage is complete once every wave's DMA has landed; this
    // stage may be overwritten once every wave has read its fragments
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
    if constexpr (MORE) frag(lds + (cs ^ 1) * T::SST, 0, 0);
    // leave issue cycles to a co-resident kernel: ~64 cycles per unit
    for (int y = 0; y < yield; ++y) __builtin_amdgcn_s_sleep(1);
  };
  for (int kt = 0; kt + 1 < nk; ++kt) step(kt, std::true_type{});
  step(nk - 1, std::false_type{});
}

// XCD-aware tile order: workgroup b -> tile index.
__device__ __forceinline__ int xcd_tile(int b, int nt) {
  return (nt % 8 == 0) ? (b % 8) * (nt / 8) + b / 8 : b;
}

// Tile index -> (tile row, tile column) of a tilesM x tilesN grid: indices
// run down bands of kBand tile rows, column by column (the last band may be
// shorter), so any 32 consecutive indices that start on a multiple of 32
// inside a band of 16 or more columns form a kBand x 8 block. A bijection, so
// every tile is still computed exactly once and in the same way.
constexpr int kBand = 4;
__host__ __device__ inline void tile_rc(int t, int tilesM, int tilesN, int& tm, int& tn) {
  const int band = t / (kBand * tilesN);
  const int rest = tilesM - band * kBand;
  const int bh = rest < kBand ? rest : kBand;
  const int idx = t - band * kBand * tilesN;
  tm = band * kBand + idx % bh;
  tn = idx / bh;
}

// Epilogue for one 32 x 32 accumulator block through a per-wave LDS block:
// lane l, register v holds row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32;
// it is written in that layout, read back row-major as float4, and stored
// with coalesced float4 accesses (ld in floats). Returns via `store(row,
// col4, value)`.
template <class F>
__device__ __forceinline__ void stage_block(const f32x16& a, float* stage, F&& store) {
  constexpr int ES = 36;  // row stride of the per-wave staging block
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, l32 = lane & 31;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int v = 0; v < 16; ++v) stage[(8 * (v >> 2) + 4 * h + (v & 3)) * ES + l32] = a[v];
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): wave-local LDS round trip
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = 8 * t + (lane >> 3), c4 = (lane & 7) * 4;
    store(r, c4, *(const f32x4*)&stage[r * ES + c4]);
  }
  __builtin_amdgcn_wave_barrier();
}

// Work split of the 256 x 128 tiles over nwg workgroups: F whole tiles
// each, then the E tiles left over cut along K into C chunks each, q
// consecutive chunks per workgroup (workgroup w takes chunks [w q, w q + q)
// of the E C, chunk c of tile e being c - e C; the chunks of one tile that a
// workgroup holds are one K range). The largest share of a workgroup is
// F + q / C tiles; C is the smallest count (at most 64, at least one K step
// per chunk) whose share is within 2 % of the best: 32 tiles over 224
// workgroups give C = 7, q = 1; 192 tiles C = 7, q = 6 (6/7 of a tile each,
// where one workgroup per tile left 32 idle). Tile e's chunks are held by
// workgroups w0(e) = e C / q .. w1(e) = (e C + C - 1) / q, whose partial
// tiles go to slots 0 .. w1 - w0 of the tile (S slots per tile at most).
struct TileSplit {
  int F, E, C, q, S;
};
__host__ __device__ inline TileSplit tile_split(int tiles, int nwg, int ksteps) {
  TileSplit t{};
  t.F = tiles / nwg;
  t.E = tiles - t.F * nwg;
  if (t.E == 0) return t;
  const int cmax = ksteps < 64 ? ksteps : 64;
  // share(C) = F + ceil(E C / nwg) / C = (F C + q) / C, compared as fractions
  int bc = 1, bq = (t.E + nwg - 1) / nwg;
  for (int c = 2; c <= cmax; ++c) {
    const int q = (t.E * c + nwg - 1) / nwg;
    if ((int64_t)(t.F * c + q) * bc < (int64_t)(t.F * bc + bq) * c) { bc = c; bq = q; }
  }
  for (int c = 1; c <= cmax; ++c) {  // the smallest C within 2 % of the best
    const int q = (t.E * c + nwg - 1) / nwg;
    if ((int64_t)100 * (t.F * c + q) * bc <= (int64_t)102 * (t.F * bc + bq) * c) {
      bc = c;
      bq = q;
      break;
    }
  }
  t.C = bc;
  t.q = bq;
  t.S = 0;
  for (int e = 0; e < t.E; ++e) {
    const int n = (e * t.C + t.C - 1) / t.q - (e * t.C) / t.q + 1;
    t.S = n > t.S ? n : t.S;
  }
  return t;
}

// One 256 x 128 tile: K steps [ks, ke) into acc, then either the full
// epilogue (whole K) or a plain store of the partial tile to `part` (ld 128).
template <int EPI>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, int t, int ks, int ke, float* part,
                                          float* lds) {
  constexpr int TM = 256;
  using T = Tile<TM>;
  int tm, tn;
  tile_rc(t, p.M / TM, p.N / TN, tm, tn);
  f32x16 acc[T::MI][2];
  nt_mainloop<TM>(p.A + (int64_t)tm * TM * p.lda, (int)p.lda, p.B + (int64_t)tn * TN * p.ldb,
                  (int)p.ldb, ks * BK, ke - ks, lds, acc, p.yield);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int h = lane >> 5, l32 = lane & 31;
  float* stage = lds + wave * 32 * 36;
  if (part) {
#pragma unroll
    for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int r0 = wm * (TM / 2) + mi * 32, c0 = wn * 64 + ni * 32;
        stage_block(acc[mi][ni], stage, [&](int r, int c4, const f32x4& val) {
          *(f32x4*)&part[(r0 + r) * TN + c0 + c4] = val;
        });
      }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < T::MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int row0 = tm * TM + wm * (TM / 2) + mi * 32;
      const int col0 = tn * TN + wn * 64 + ni * 32;
      if (EPI == kEpiSolve && p.Ct) {
        // C^T straight from the accumulator layout: lane l holds column
        // col0 + l % 32, rows row0 + 8 g + 4 (l / 32) + 0..3 in v = 4 g ..
        float* ct = p.Ct + (int64_t)(col0 + l32) * p.ldct + row0 + 4 * h;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[mi][ni][4 * g], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2],
                           acc[mi][ni][4 * g + 3]};
          *(f32x4*)&ct[8 * g] = v;
        }
      }
      stage_block(acc[mi][ni], stage, [&](int r, int c4, const f32x4& val) {
        const int64_t idx = (int64_t)(row0 + r) * p.ldc + col0 + c4;
        if (EPI == kEpiRhs) {
          const f32x4 pv = *(const f32x4*)&p.P[idx];
          *(f32x4*)&p.C[idx] = val + p.rho * pv;
        } else {
          *(f32x4*)&p.C[idx] = val;
        }
      });
    }
}

// nx = 0: one workgroup per tile. nx > 0: 256 workgroups (32 per XCD), those
// of XCDs 0 .. nx - 1 working; each takes whole tiles, and the tiles left
// over are split along K into partial tiles that gemm_fixup_kernel adds up.
template <int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_nt_kernel(GemmArgs p, int nx, TileSplit sp) {
  __shared__ __attribute__((aligned(1024))) float lds[Tile<256>::LDS_FLOATS];
  const int tiles = (p.M / 256) * (p.N / TN);
  const int ksteps = p.K / BK;
  if (!nx) {
    gemm_tile<EPI>(p, xcd_tile(blockIdx.x, tiles), 0, ksteps, nullptr, lds);
    return;
  }
  // consecutive workgroups go to consecutive XCDs (the first one's XCD
  // depends on the queue's history): with 32 per XCD, blockIdx / 8 numbers
  // the workgroups of one XCD. XCDs nx .. 7 are left to a pinned chain.
  const int x = xcd_id(), i = blockIdx.x >> 3;
  if (x >= nx) return;
  const int per = gridDim.x / 8, nwg = nx * per, w = i * nx + x;
  bool first = true;
  for (int f = 0; f < sp.F; ++f) {
    if (!first) {  // the next tile's copies overwrite the LDS the epilogue staged in
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("s_barrier" ::: "memory");
    }
    first = false;
    gemm_tile<EPI>(p, f * nwg + x * per + i, 0, ksteps, nullptr, lds);
  }
  // this workgroup's chunks [c0, c1) of the leftover tiles, one K range per
  // tile they touch
  const int total = sp.E * sp.C;
  const int c0 = w * sp.q, c1 = c0 + sp.q < total ? c0 + sp.q : total;
  for (int c = c0; c < c1;) {
    const int e = c / sp.C, ce = (e + 1) * sp.C < c1 ? (e + 1) * sp.C : c1;
    if (!first) {
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("s_barrier" ::: "memory");
    }
    first = false;
    const int slot = w - (e * sp.C) / sp.q;
    gemm_tile<EPI>(p, sp.F * nwg + e, (c - e * sp.C) * ksteps / sp.C,
                   (ce - e * sp.C) * ksteps / sp.C,
                   p.part + ((int64_t)e * sp.S + slot) * 256 * TN, lds);
    c = ce;
  }
}

// The leftover tiles of a split launch: the sum of each tile's partial
// tiles in slot (workgroup) order, then the epilogue (+ rho P; C^T beside
// C). Block (e, y) covers rows 8 y .. 8 y + 7 of tile e.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(GemmArgs p, int nwg, TileSplit sp) {
  const int e = blockIdx.x;
  const int r = blockIdx.y * 8 + (threadIdx.x >> 5), c4 = (threadIdx.x & 31) * 4;
  int tm, tn;
  tile_rc(sp.F * nwg + e, p.M / 256, p.N / TN, tm, tn);
  const int C = (e * sp.C + sp.C - 1) / sp.q - (e * sp.C) / sp.q + 1;  // slots of tile e
  const float* src = p.part + (int64_t)e * sp.S * 256 * TN + r * TN + c4;
  const int64_t row = (int64_t)tm * 256 + r, col = (int64_t)tn * TN + c4;
  const int64_t idx = row * p.ldc + col;
  f32x4 pv = {0.0f, 0.0f, 0.0f, 0.0f};
  if (EPI == kEpiRhs) pv = *(const f32x4*)&p.P[idx];
  // every slot of a batch of 8 is loaded before any is added (a loop over a
  // run-time count would wait on each load in turn); the sum runs in slot
  // order all the same
  f32x4 sum = *(const f32x4*)src;
  for (int c0 = 1; c0 < C; c0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < C) v[j] = *(const f32x4*)(src + (int64_t)(c0 + j) * 256 * TN);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < C) sum += v[j];
  }
  if (EPI == kEpiRhs) sum += p.rho * pv;
  *(f32x4*)&p.C[idx] = sum;
  if (EPI == kEpiSolve && p.Ct) {
#pragma unroll
    for (int j = 0; j < 4; ++j) p.Ct[(col + j) * p.ldct + row] = sum[j];
  }
}

// Partial Gram tiles, stream-K: the K steps of 32 of the lower tiles (tile
// t = I (I + 1) / 2 + J, I >= J, both operands the rows I and J panels of
// At; GramSteps gives each tile's steps) are cut into ranges of L steps, one
// per workgroup, so every workgroup has the same work. A range covers the
// end of one tile and the start of the next; each segment goes to slot
// w - w0(t) of its tile, w0(t) = (steps before tile t) / L being the first
// workgroup that touches tile t.
__global__ __launch_bounds__(NT, 2) void gram_nt_kernel(const float* __restrict__ At,
                                                        int64_t ldat, int rp, GramSteps gs,
                                                        int L, int64_t S, int W, int px,
                                                        float* __restrict__ part) {
  constexpr int TM = 128;
  using T_ = Tile<TM>;
  __shared__ __attribute__((aligned(1024))) float lds[T_::LDS_FLOATS];
  int w;
  if (px) {
    // only the last px XCDs work, each on a contiguous run of ranges; the
    // workgroups that land elsewhere exit (each fits beside a GEMM
    // workgroup: 64 + 96 KB of LDS)
    const int x = xcd_id(), x0 = 8 - px;
    if (x < x0) return;
    w = (x - x0) * (int)(gridDim.x / 8) + (int)(blockIdx.x >> 3);
  } else {
    w = xcd_tile(blockIdx.x, W);
  }
  int64_t s0 = (int64_t)w * L;
  const int64_t s1 = min(S, s0 + L);
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  float* stage = lds + wave * 32 * 36;
  const int R = rp / TM;
  int I = 0;
  while (s0 < s1) {
    // tile row I holding step s0 (rows only move forward)
    while (I + 1 < R && gs.row_start(I + 1) <= s0) ++I;
    const int len = gs.len(I);
    const int64_t off = s0 - gs.row_start(I);
    const int J = (int)(off / len), ks = (int)(off % len);
    const int ke = (int)min<int64_t>(len, ks + (s1 - s0));
    const int slot = w - (int)(gs.tile_start(I, J) / L);
    f32x16 acc[T_::MI][2];
    nt_mainloop<TM>(At + (int64_t)I * TM * ldat, (int)ldat, At + (int64_t)J * TN * ldat,
                    (int)ldat, (gs.first(I) + ks) * BK, ke - ks, lds, acc);
    float* out = part + (int64_t)slot * rp * rp;
#pragma unroll
    for (int mi = 0; mi < T_::MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row0 = I * TM + wm * (TM / 2) + mi * 32;
        const int col0 = J * TN + wn * 64 + ni * 32;
        stage_block(acc[mi][ni], stage, [&](int r, int c4, const f32x4& val) {
          *(f32x4*)&out[(int64_t)(row0 + r) * rp + col0 + c4] = val;
        });
      }
    s0 += ke - ks;
    if (s0 < s1) {
      // the next segment's DMA overwrites the LDS this epilogue staged in
      __builtin_amdgcn_s_waitcnt(0xc07f);
      asm volatile("s_barrier" ::: "memory");
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Whether a whole-chip launch with a partial buffer splits its tiles (see
// launch_gemm).
bool whole_chip_split(int nt, int ksteps) {
  return (nt > kPinGrid && nt % kPinGrid) || (nt >= kPinGrid / 4 && nt < kPinGrid && ksteps >= 32);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, int epi, hipStream_t s) {
  if (a.M % 256 || a.N % TN || a.K % BK || a.M <= 0 || a.N <= 0 || a.K <= 0)
    return hipErrorInvalidValue;
  if (a.lda % 4 || a.ldb % 4 || a.ldc % 4 || a.lda < a.K || a.ldb < a.K || a.ldc < a.N ||
      !aligned16(a.A) || !aligned16(a.B) || !aligned16(a.C))
    return hipErrorInvalidValue;
  if (epi == kEpiSolve && a.Ct && (a.ldct % 4 || a.ldct < a.M || !aligned16(a.Ct)))
    return hipErrorInvalidValue;
  // operand copies address a tile's rows as 32-bit byte offsets
  if ((int64_t)256 * a.lda * 4 >= (int64_t)1 << 31 || (int64_t)TN * a.ldb * 4 >= (int64_t)1 << 31)
    return hipErrorInvalidValue;
  const int nt = (a.M / 256) * (a.N / TN);
  if (a.free_xcds && (epi != kEpiRhs || !a.part || a.free_xcds < 0 || a.free_xcds > kPinMaxXcds))
    return hipErrorInvalidValue;
  if (a.part && !aligned16(a.part)) return hipErrorInvalidValue;
  // Split launches: with free_xcds, on XCDs 0 .. 7 - free_xcds; with part
  // alone, on the whole chip when one workgroup per tile would leave CUs
  // idle: more tiles than CUs, not in whole rounds, or fewer tiles than
  // CUs but at least a quarter of them, with K long enough to cut.
  const int ksteps = a.K / BK;
  const int nx = a.free_xcds ? 8 - a.free_xcds : (a.part && whole_chip_split(nt, ksteps)) ? 8 : 0;
  const int nwg = kPinXcdCus * nx;
  const TileSplit sp = nx ? tile_split(nt, nwg, ksteps) : TileSplit{};
  dim3 grid(nx ? kPinGrid : nt), block(NT);
  switch (epi) {
    case kEpiRhs: hipLaunchKernelGGL(gemm_nt_kernel<kEpiRhs>, grid, block, 0, s, a, nx, sp); break;
    case kEpiSolve: hipLaunchKernelGGL(gemm_nt_kernel<kEpiSolve>, grid, block, 0, s, a, nx, sp); break;
    default: hipLaunchKernelGGL(gemm_nt_kernel<kEpiPlain>, grid, block, 0, s, a, nx, sp); break;
  }
  if (nx && sp.E > 0) {
    const dim3 fg(sp.E, 256 / 8);
    switch (epi) {
      case kEpiRhs: hipLaunchKernelGGL(gemm_fixup_kernel<kEpiRhs>, fg, dim3(256), 0, s, a, nwg, sp); break;
      case kEpiSolve: hipLaunchKernelGGL(gemm_fixup_kernel<kEpiSolve>, fg, dim3(256), 0, s, a, nwg, sp); break;
      default: hipLaunchKernelGGL(gemm_fixup_kernel<kEpiPlain>, fg, dim3(256), 0, s, a, nwg, sp); break;
    }
  }
  return hipGetLastError();
}

size_t gemm_part_floats(int M, int N, int K, int f) {
  if (M % 256 || N % TN || K % BK || M <= 0 || N <= 0 || K <= 0 || f < 0 || f > kPinMaxXcds)
    return 0;
  const int nt = (M / 256) * (N / TN);
  if (f == 0 && !whole_chip_split(nt, K / BK)) return 0;
  const TileSplit sp = tile_split(nt, kPinGrid - kPinXcdCus * f, K / BK);
  return (size_t)sp.E * sp.S * 256 * TN;
}

GramPlan gram_plan(int K, int rp, bool tri, int xcds) {
  GramPlan p{};
  const int R = rp / 128;
  const int T = K / BK;
  const GramSteps gs{T, tri ? 1 : 0};
  const int64_t S = gs.row_start(R);
  // two workgroups per CU (of the whole chip, or of the last xcds XCDs); a
  // tile gets at most 8 segments
  const int64_t cap = xcds > 0 ? (int64_t)2 * kPinXcdCus * xcds : 512;
  int64_t L = std::max<int64_t>((S + cap - 1) / cap, (T + 6) / 7);
  L = std::max<int64_t>(L, 1);
  p.steps = (int)L;
  p.wgs = (int)((S + L - 1) / L);
  p.slots = (int)((T + L - 1) / L) + 1;
  p.tri = tri ? 1 : 0;
  p.xcds = xcds > 0 ? std::min(xcds, kPinMaxXcds) : 0;
  return p;
}

hipError_t launch_gram_partial(const float* At, int64_t ldat, int K, int rp, const GramPlan& p,
                               float* part, hipStream_t s, hipEvent_t done) {
  if (rp % 128 || K % BK || K <= 0 || ldat % 4 || ldat < K || !aligned16(At) || p.steps <= 0)
    return hipErrorInvalidValue;
  if ((int64_t)128 * ldat * 4 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  if (p.tri && K != rp) return hipErrorInvalidValue;
  const int R = rp / 128;
  const GramSteps gs{K / BK, p.tri};
  const int64_t S = gs.row_start(R);
  // `done` is recorded by the kernel's own completion (no marker of its own
  // between this kernel and the next one on s)
  // with p.xcds: two workgroups per CU of all 8 XCDs, those of the last
  // p.xcds working (p.wgs <= 64 p.xcds)
  if (p.xcds < 0 || p.xcds > kPinMaxXcds || (p.xcds && p.wgs > 2 * kPinXcdCus * p.xcds))
    return hipErrorInvalidValue;
  const unsigned grid = p.xcds ? 2u * kPinGrid : (unsigned)p.wgs;
  hipExtLaunchKernelGGL(gram_nt_kernel, dim3(grid), dim3(NT), 0, s, nullptr, done, 0u, At, ldat,
                        rp, gs, p.steps, S, p.wgs, p.xcds, part);
  return hipGetLastError();
}

}  // namespace nq
