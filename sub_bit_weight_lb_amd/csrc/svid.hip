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
// HBM-bound: the algorithmic traffic of one update is 16 B per element (read
// the factor and Lam, write Lam and P). One persistent launch does the whole
// update. Its G workgroups (at most one per CU, 4 waves each, one per SIMD,
// so that a workgroup fits beside one of the GEMMs it runs next to in the
// ADMM loop) each own a slab of whole rows. When the slab fits in registers
// X = U + Lam is read once and stays on chip for all T steps; otherwise each
// step streams the slab again from memory (X written back by the first step).
// Per step:
//   1. a_i = sum_j |X_ij| b_j / bb for the slab's rows (DPP wave sums, then
//      the waves in order); the slab publishes its column partials
//      p_j = sum_i |X_ij| a_i as one contiguous row, and sum a_i^2;
//   2. workgroup w owns a block of 4 NQO consecutive columns: it reads that
//      block of every slab's row, sums it in slab order, b_j = sum p_j / aa,
//      and publishes b_j;
//   3. every workgroup reads all of b and forms bb = b^T b (same order
//      everywhere, so every workgroup holds the same bits).
// Exchanges go through device memory as 64-bit words (value, tag) written
// and read with relaxed device-scope atomics (coherent across the XCDs, no
// cache write-back or invalidate, which would disturb the kernels running
// beside this one). The tag, derived from a per-buffer epoch that the last
// workgroup to finish advances, names the launch, step and phase, so a reader
// simply waits until each word carries the tag it expects: no barrier, no
// flags, nothing to reset, and stale words from an earlier launch or step
// never match. A word is overwritten only after every reader of its previous
// value has published something that depends on it (which is why only
// workgroups that own columns read the slabs' words). Waits are bounded by a
// count of poll rounds (about 0.5 s, none once a wait has run out earlier in
// the run); a timeout is reported through DevStats with where it happened,
// and every workgroup still runs to its end. All sums run in a fixed order,
// so results are bit-reproducible. The waves run at the default priority and
// stream with non-temporal loads and stores: the update has a whole solve
// and Gram to finish in, and should take as little from them as it can.
//
// Every workgroup must be resident at once for the waits to end; the grid is
// at most one workgroup per CU, and the kernel does not depend on anything
// launched after it, so workgroups still queued behind other kernels start
// as those finish.
#include "common.h"

#include <algorithm>
#include <cstdlib>

namespace nq {
namespace {

constexpr int CR = 64;    // rows per chunk of the column-norm pass
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kMaxNT = 256;  // one wave per SIMD: a workgroup fits beside one of the GEMMs'
constexpr int kPollSleep = 1;      // s_sleep units (64 cycles) between polls of a wait
constexpr int kNT = 2;              // cache policy of the streaming loads and stores: nt
constexpr int kOwnRounds = 4;       // words per thread per wait of the owner's read
constexpr int kMaxKW = 32;          // columns an owner reduces (r_p <= 8192)
// Rounds a wait polls before it gives up: each round sleeps kPollSleep x 64
// cycles and waits for its loads (about 1 us), so roughly 0.5 s.
constexpr uint32_t kWaitPolls = 500000;

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over the wave by DPP moves (VALU only, no LDS round trips), in a fixed
// order; the total, read from lane 63, is returned to every lane.
template <int CTRL, int ROW_MASK>
__device__ inline float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                          0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false));
}
__device__ inline float wave_sum_dpp(float v) {
  v = dpp_add<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]: quad sums
  v = dpp_add<0x141, 0xf>(v);  // row_half_mirror: sums of 8
  v = dpp_add<0x140, 0xf>(v);  // row_mirror: sums of 16 in every lane of a row
  v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3: lane 63 has the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ inline void put_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t get_word(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline bool has_tag(uint64_t v, uint32_t tag) { return (uint32_t)(v >> 32) == tag; }
__device__ inline float word_val(uint64_t v) { return __uint_as_float((uint32_t)v); }

// Loads the tagged words k < N with bit k of `mask` set (addresses from
// addr(k)) until each carries `tag`, all loads of a round in flight together;
// false after `polls` rounds (the values are then whatever was read). The
// bound is a count of rounds, not a clock: reading the clock on every round
// from every wave stalled kernels running beside this one (a clock read is a
// scalar memory access to one chip-wide counter).
template <int N, class Addr>
__device__ inline bool wait_words(Addr addr, uint32_t mask, uint32_t tag, uint32_t polls,
                                  float* out, uint32_t* seen, int* which) {
  uint64_t v[N];
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = (mask >> k & 1u) ? get_word(addr(k)) : ((uint64_t)tag << 32);
  bool ok = true;
  for (uint32_t round = 0;; ++round) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < N; ++k) all = all && has_tag(v[k], tag);
    if (all) break;
    if (round >= polls) {
      ok = false;
#pragma unroll
      for (int k = 0; k < N; ++k)
        if (!has_tag(v[k], tag)) {
          *seen = (uint32_t)(v[k] >> 32);
          *which = k;
        }
      break;
    }
    __builtin_amdgcn_s_sleep(kPollSleep);
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (!has_tag(v[k], tag)) v[k] = get_word(addr(k));
  }
#pragma unroll
  for (int k = 0; k < N; ++k) out[k] = word_val(v[k]);
  return ok;
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 0x7fffffff,
                                           0x00020000);
}
__device__ inline f32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT));
}
// Stores keep the scalar offset at zero: the compiler then separates a
// 128-bit store from a later write of its data registers by the wait states
// the hardware needs, which it omits for a store with a register scalar
// offset (on this part such a store read data already overwritten: the dual
// update's Lam store picked up the P value, one component in a few lanes).
__device__ inline void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff + soff, 0, kNT);
}

// Fixed-order sum of one float per thread over the workgroup; every thread
// gets the same bits. sh: kMaxNT / 64 floats; one barrier before (so sh may
// be reused right after) and one after.
__device__ inline float block_sum(float v, float* sh) {
  const int nw = blockDim.x >> 6;
  v = wave_sum_dpp(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.0f;
  for (int k = 0; k < nw; ++k) t += sh[k];
  return t;
}

// The first wait of a run that ran out records where it was.
__device__ inline void note_timeout(DevStats* st, int step, int phase, uint32_t want,
                                    uint32_t seen, uint32_t epoch, uint64_t t_start, int src,
                                    const uint32_t* prog) {
  const uint64_t now = __builtin_amdgcn_s_memrealtime();
  if (atomicCAS(&st->sync_timeout, 0, 1) == 0) {
    st->to_src = (uint32_t)src;
    st->to_src_prog = __hip_atomic_load(prog + src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st->to_start = t_start;
    st->to_now = now;
    st->to_wg = blockIdx.x;
    st->to_step = (uint32_t)step;
    st->to_phase = (uint32_t)phase;
    st->to_want = want;
    st->to_seen = seen;
    st->to_epoch = epoch;
  }
}

struct SvidArgs {
  float* X;            // rows_pad x rp: Lam on entry (or the input), Lam / unchanged on exit
  const float* Uadd;   // nullable: X <- X + Uadd first
  float* P;            // rows_pad x rp
  float* a_out;        // rows_pad
  float* b_out;        // rp
  SvidSync sy;
  DevStats* st;
  int rp, r_real, T, mode;
  int G, RS, RPT, NCH, NQO;
};

// Publishes this slab's column partials and sum of a_i^2 (step tag tagP),
// reduces this workgroup's columns over all slabs into b (tag tagB), then
// reads all of b for this thread's columns and returns bb = b^T b. Every sum
// runs in a fixed order.
//
// Layout: part[s][col] is slab s's row of partials in column order, written
// whole by slab s; b[col]; aa[s]. Workgroup o owns the KW = 4 NQO
// consecutive columns from KW o (NQO a power of two), so its reads of every
// slab's block and the slabs' writes of their rows are both contiguous; LDS
// (xs: max(4 TX, G KW) floats) stages the values between the thread layout
// (thread t: float4 column t + TX u) and the word layout.
template <int NU, bool GUARD>
__device__ __forceinline__ float svid_exchange(const SvidArgs& A, const f32x4 (&pacc)[NU],
                                               float aa_w, f32x4 (&bq)[NU], const bool (&qok)[NU],
                                               uint32_t tagP, bool last, uint32_t deadline,
                                               bool& ok, float* xs, float (*red)[kMaxKW],
                                               float* sh, int step, uint32_t epoch,
                                               uint64_t t_start) {
  const int tid = threadIdx.x, NT = blockDim.x, TX = NT;
  const int lane = tid & 63, wave = tid >> 6, nw = NT >> 6;
  const int w = blockIdx.x, G = A.G, rp = A.rp;
  const int KW = 4 * A.NQO;
  const uint32_t tagB = tagP + 1u;
  f32x4* xs4 = (f32x4*)xs;

  // 1. this slab's row, one block of 4 TX columns per u, through LDS so that
  // consecutive threads write consecutive words
  uint64_t* row = A.sy.part + (int64_t)w * rp;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    xs4[tid] = pacc[u];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = 4 * TX * u + tid + NT * r;
      if (col < rp) put_tagged(row + col, xs[tid + NT * r], tagP);
    }
    __syncthreads();
  }
  if (tid == 0) {
    put_tagged(A.sy.aa + w, aa_w, tagP);
    __hip_atomic_store(A.sy.prog + w, tagP << 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // 2. owner of columns [KW w, KW w + KW): every slab's block into LDS
  // (xs[s KW + k]) with the slabs' aa, then sums in slab order. Only a
  // workgroup that owns columns reads the slabs' words: a slab overwrites them
  // in the next step only after reading every owner's b, so an owner always
  // reads them first; a workgroup with no columns would publish nothing the
  // slabs wait for, and could be overrun.
  const int c0 = KW * w;
  if (c0 < rp) {
    constexpr int NA = 2;  // aa words per thread (G <= 2 NT)
    const int total = G * KW;
    // word i = i0 + NT r + tid is column i % KW of slab i / KW; NT is a
    // multiple of KW, so the column is the same for every r and the slab
    // advances by NT / KW per round
    const int kcol = tid % KW;
    const int64_t rstride = (int64_t)(NT / KW) * rp;
    float aa_tot = 0.0f;
    for (int i0 = 0; i0 < total; i0 += kOwnRounds * NT) {
      const uint64_t* rbase = A.sy.part + (int64_t)((i0 + tid) / KW) * rp + c0 + kcol;
      uint32_t mask = 0;
#pragma unroll
      for (int r = 0; r < kOwnRounds; ++r) {
        const int i = i0 + NT * r + tid;
        if (i < total && c0 + kcol < rp) mask |= 1u << (NA + r);
      }
      if (i0 == 0) {
#pragma unroll
        for (int k = 0; k < NA; ++k)
          if (tid + NT * k < G) mask |= 1u << k;
      }
      float vv[NA + kOwnRounds];
      uint32_t seen = 0;
      int which = 0;
      const bool got = wait_words<NA + kOwnRounds>(
          [&](int k) -> const uint64_t* {
            if (k < NA) return A.sy.aa + tid + NT * k;
            return rbase + (k - NA) * rstride;
          },
          mask, tagP, ok ? deadline : 0u, vv, &seen, &which);
      if (!got)
        note_timeout(A.st, step, 0, tagP, seen, epoch, t_start,
                     which < NA ? tid + NT * which : (i0 + NT * (which - NA) + tid) / KW,
                     A.sy.prog);
      ok &= got;
#pragma unroll
      for (int r = 0; r < kOwnRounds; ++r) {
        const int i = i0 + NT * r + tid;
        if (i < total) xs[i] = (mask >> (NA + r) & 1u) ? vv[NA + r] : 0.0f;
      }
      if (i0 == 0) {
        float a2 = 0.0f;
#pragma unroll
        for (int k = 0; k < NA; ++k) a2 += (mask >> k & 1u) ? vv[k] : 0.0f;
        aa_tot = block_sum(a2, sh);
      }
    }
    __syncthreads();
    // thread (g, k): slabs g, g + NG, ... of column k; then the groups of a
    // wave by butterfly, then the waves in order
    const int NG = NT / KW, k = tid % KW, g = tid / KW;
    float part = 0.0f;
    for (int s2 = g; s2 < G; s2 += NG) part += xs[s2 * KW + k];
    for (int o = KW; o < 64; o <<= 1) part += __shfl_xor(part, o, 64);
    if (lane < KW) red[wave][lane] = part;
    __syncthreads();
    if (tid < KW && c0 + tid < rp) {
      float tot = 0.0f;
      for (int v = 0; v < nw; ++v) tot += red[v][tid];
      const float bj = aa_tot > 0.0f ? tot / aa_tot : 0.0f;
      put_tagged(A.sy.b + c0 + tid, bj, tagB);
      if (last) A.b_out[c0 + tid] = bj;
    }
  }
  if (tid == 0)
    __hip_atomic_store(A.sy.prog + w, (tagP << 2) | 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // 3. all of b for this thread's columns: per u, the block's words read by
  // consecutive threads into LDS, then each thread's float4
  float bsq = 0.0f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    uint32_t mask = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * TX * u + tid + NT * r < rp) mask |= 1u << r;
    float vv[4];
    uint32_t seen = 0;
    int which = 0;
    const bool got = wait_words<4>(
        [&](int r) { return A.sy.b + 4 * TX * u + tid + NT * r; }, mask, tagB, ok ? deadline : 0u, vv,
        &seen, &which);
    if (!got)
      note_timeout(A.st, step, 1, tagB, seen, epoch, t_start,
                   (4 * TX * u + tid + NT * which) / KW, A.sy.prog);
    ok &= got;
    __syncthreads();  // xs free
#pragma unroll
    for (int r = 0; r < 4; ++r) xs[tid + NT * r] = vv[r];
    __syncthreads();
    bq[u] = qok[u] ? xs4[tid] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) bsq += bq[u][e] * bq[u][e];
  }
  const float bbn = block_sum(bsq, sh);
  if (tid == 0)
    __hip_atomic_store(A.sy.prog + w, (tagP << 2) | 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return bbn;
}

// One SVID update. The workgroup's TX threads (TX = blockDim.x) cover its
// rows, thread t holding float4 columns q = t + TX u (u < NU); a chunk is
// RPT consecutive rows of the slab (RS = NCH chunks, the last possibly
// shorter). RES: rows_pad = G RPT and the one chunk stays in registers from
// the first step to the last. GUARD: TX NU may exceed rp / 4 (those column
// positions read as zero and are not written); otherwise every position is
// a real column.
template <int NU, int RPT, bool RES, bool GUARD>
__device__ __forceinline__ void svid_grid_body(const SvidArgs& A) {
  // dynamic: a of the slab's rows (A.RS floats, padded to a multiple of 4),
  // then the exchange's staging (max(4 TX, G KW) floats)
  extern __shared__ float dyn[];
  float* arow = dyn;
  float* xs = dyn + ((A.RS + 3) & ~3);
  __shared__ f32x4 rred[2][RPT][2];  // per-wave row sums (up to 8 waves), double-buffered by chunk
  __shared__ float red[kMaxNT / 64][kMaxKW];
  __shared__ float sh[kMaxNT / 64];
  __shared__ uint32_t sh_epoch;

  const int tid = threadIdx.x, TX = blockDim.x;
  const int nw = TX >> 6, wave = tid >> 6;
  const int w = blockIdx.x;
  const int rp = A.rp, rp4 = rp / 4;

  if (tid == 0) sh_epoch = __hip_atomic_load(&A.sy.ctl[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
  const uint32_t deadline = A.st->sync_timeout ? 0u : kWaitPolls;  // poll rounds per wait
  __syncthreads();
  const uint32_t epoch = sh_epoch;
  bool ok = true;
  if (tid == 0)
    __hip_atomic_store(A.sy.prog + w, (epoch << 2) | 3u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  bool qok[NU];
  uint32_t voff[NU];  // byte offset of the thread's column block u within a row
  f32x4 bq[NU];       // b of the thread's columns: 1 on the real ones to start
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int q = tid + TX * u;
    qok[u] = !GUARD || q < rp4;
    voff[u] = (uint32_t)(qok[u] ? q : 0) * 16u;
#pragma unroll
    for (int e = 0; e < 4; ++e) bq[u][e] = (qok[u] && 4 * q + e < A.r_real) ? 1.0f : 0.0f;
  }
  float bb = (float)A.r_real;

  const int64_t slab = (int64_t)w * A.RS * rp;
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(A.X + slab);
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(A.P + slab);
  const __amdgpu_buffer_rsrc_t rU = make_rsrc((A.Uadd ? A.Uadd : A.X) + slab);
  const bool add_u = A.Uadd != nullptr;
  const uint32_t row_bytes = (uint32_t)rp * 4u;

  f32x4 x[RPT][NU];
  float arg[RPT];  // a of the chunk's rows

  // Loads the nk rows of chunk c into x: X, or X + Uadd (written back to X
  // when `back`). With Uadd the rows go in two halves so that the Uadd values
  // need half the chunk's registers.
  auto load_rows = [&](int c, int nk, bool add, bool back) {
    const uint32_t cb = (uint32_t)(c * RPT) * row_bytes;
    if (!add) {
#pragma unroll
      for (int k = 0; k < RPT; ++k)
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          x[k][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          if (RES || k < nk) x[k][u] = bload(rX, voff[u], cb + k * row_bytes);
        }
    } else {
      constexpr int H = (RPT + 1) / 2;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 y[H][NU];
#pragma unroll
        for (int kk = 0; kk < H; ++kk) {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int k = h * H + kk;
            if (k < RPT) {
              x[k][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
              y[kk][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
              if (RES || k < nk) {
                x[k][u] = bload(rX, voff[u], cb + k * row_bytes);
                y[kk][u] = bload(rU, voff[u], cb + k * row_bytes);
              }
            }
          }
        }
#pragma unroll
        for (int kk = 0; kk < H; ++kk) {
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const int k = h * H + kk;
            if (k < RPT) {
              x[k][u] += y[kk][u];
              if (back && k < nk && qok[u]) bstore(rX, voff[u], cb + k * row_bytes, x[k][u]);
            }
          }
        }
      }
    }
    if (GUARD) {
#pragma unroll
      for (int k = 0; k < RPT; ++k)
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (!qok[u]) x[k][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  if (RES) load_rows(0, RPT, add_u, false);

  for (int t = 0; t < A.T; ++t) {
    f32x4 pacc[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) pacc[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < (RES ? 1 : A.NCH); ++c) {
      const int nk = RES ? RPT : min(RPT, A.RS - c * RPT);  // rows in this chunk
      if (!RES) load_rows(c, nk, t == 0 && add_u, true);
      // a of the chunk's rows from the current b: wave sums, then the waves
      // in order
      const int buf = c & 1;
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc += fabsf(x[k][u][e]) * bq[u][e];
        acc = wave_sum_dpp(acc);
        if ((tid & 63) == 0) ((float*)&rred[buf][k][0])[wave] = acc;
      }
      __syncthreads();
      const float inv_bb = bb > 0.0f ? 1.0f / bb : 0.0f;
#pragma unroll
      for (int k = 0; k < RPT; ++k) {
        const f32x4 lo = rred[buf][k][0], hi = rred[buf][k][1];
        float tot = lo[0];  // the waves in order; entries past nw are never read
        if (nw > 1) tot += lo[1];
        if (nw > 2) tot += lo[2];
        if (nw > 3) tot += lo[3];
        if (nw > 4) tot += hi[0];
        if (nw > 5) tot += hi[1];
        if (nw > 6) tot += hi[2];
        if (nw > 7) tot += hi[3];
        arg[k] = (RES || k < nk) ? tot * inv_bb : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < RPT; ++k)
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) pacc[u][e] += fabsf(x[k][u][e]) * arg[k];
      if (tid < RPT && (RES || tid < nk)) {
        float av = 0.0f;
#pragma unroll
        for (int k = 0; k < RPT; ++k)
          if (k == tid) av = arg[k];
        arow[c * RPT + tid] = av;
      }
    }
    __syncthreads();  // arow complete
    float aa_part = 0.0f;
    for (int i = tid; i < A.RS; i += TX) aa_part += arow[i] * arow[i];
    const float aa_w = block_sum(aa_part, sh);
    bb = svid_exchange<NU, GUARD>(A, pacc, aa_w, bq, qok, epoch + 2u * (uint32_t)t + 1u,
                                  t == A.T - 1, deadline, ok, xs, red, sh, t, epoch, t_start);
  }

  // Z = sign(X) a_i b_j with the last step's a and b; the dual update
  const int64_t arow0 = (int64_t)w * A.RS;
  for (int c = 0; c < (RES ? 1 : A.NCH); ++c) {
    const int nk = RES ? RPT : min(RPT, A.RS - c * RPT);
    const uint32_t cb = (uint32_t)(c * RPT) * row_bytes;
    if (!RES) load_rows(c, nk, false, false);
    if (tid < nk) A.a_out[arow0 + c * RPT + tid] = arow[c * RPT + tid];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      if (!RES && k >= nk) break;
      const float ai = arow[c * RPT + k];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (GUARD && !qok[u]) continue;
        f32x4 z;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float mag = ai * bq[u][e];
          z[e] = x[k][u][e] >= 0.0f ? mag : -mag;
        }
        const uint32_t so = cb + k * row_bytes;
        if (A.mode == 1) {
          const f32x4 lam = x[k][u] - z;
          bstore(rX, voff[u], so, lam);
          bstore(rP, voff[u], so, z - lam);
        } else {
          bstore(rP, voff[u], so, z);
          if (A.mode == 0) bstore(rX, voff[u], so, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
        }
      }
    }
  }

  // the last workgroup out advances the epoch for the next launch
  __syncthreads();
  if (tid == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(&A.sy.ctl[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (uint32_t)A.G - 1u) {
      __hip_atomic_store(&A.sy.ctl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&A.sy.ctl[0], epoch + 2u * (uint32_t)A.T + 2u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int NU, int RPT, bool RES, bool GUARD>
__global__ __launch_bounds__(kMaxNT) __attribute__((amdgpu_waves_per_eu(1, 2))) void svid_grid_kernel(SvidArgs A) {
  svid_grid_body<NU, RPT, RES, GUARD>(A);
}

// colpart[c][j] = sum_{i in chunk c} X_ij^2 (column norms for the balance).
// 32 x 8 threads: float4 columns x row stripes of the 64-row chunk,
// fixed-order reduction.
__global__ __launch_bounds__(256) void colsumsq_kernel(const float* __restrict__ X, int rp,
                                                       int rows_pad, float* __restrict__ colpart) {
  __shared__ f32x4 red[8][32];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  const int q = blockIdx.x * 32 + tx;
  const int c = blockIdx.y;
  const int i0 = c * CR, i1 = min(rows_pad, i0 + CR);
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
  for (int i = i0 + ty; i < i1; i += 8) {
    const f32x4 v = ((const f32x4*)(X + (int64_t)i * rp))[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += v[e] * v[e];
  }
  red[ty][tx] = acc;
  __syncthreads();
  if (ty == 0) {
    f32x4 t = red[0][tx];
#pragma unroll
    for (int y = 1; y < 8; ++y) t += red[y][tx];
    ((f32x4*)(colpart + (int64_t)c * rp))[q] = t;
  }
}

// The instances (float4 columns per thread, rows per chunk, resident,
// guarded columns).
struct Inst {
  int nu, rpt;
  bool res, guard;
};
#define NQ_SVID_INSTANCES(X)                                                              \
  X(0, 2, 16, true, false) X(1, 2, 8, true, false) X(2, 2, 4, true, false)                \
  X(3, 2, 2, true, false) X(4, 1, 16, true, false) X(5, 1, 8, true, false)                \
  X(6, 1, 4, true, false) X(7, 1, 2, true, false) X(8, 1, 1, true, false)                 \
  X(9, 1, 8, false, false) X(10, 2, 8, false, false) X(11, 3, 8, false, false)            \
  X(12, 4, 4, false, false) X(13, 6, 4, false, false) X(14, 8, 2, false, false)           \
  X(15, 1, 8, false, true) X(16, 2, 8, false, true) X(17, 4, 4, false, true)              \
  X(18, 8, 2, false, true)
#define NQ_SVID_INST(i, nu, rpt, res, gd) {nu, rpt, res, gd},
constexpr Inst kInst[] = {NQ_SVID_INSTANCES(NQ_SVID_INST)};
#undef NQ_SVID_INST
constexpr int kNumInst = sizeof(kInst) / sizeof(kInst[0]);

int grid_size() {
  static int g = -1;
  if (g < 0) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      ncu = 64;
    g = ncu >= 256 ? 256 : ncu >= 128 ? 128 : 64;  // a power of two: G divides 2 NT
  }
  return g;
}

}  // namespace

int svid_nchunks(int rows_pad) { return (rows_pad + CR - 1) / CR; }

// Chooses the instance and layout: resident first, then the fewest chunks,
// then the most workgroups and threads, exact column layouts before guarded.
bool svid_plan(int rows_pad, int rp, int Gmax, SvidPlan* out) {
  if (rp <= 0 || rp % 128 || rows_pad <= 0) return false;
  const int rp4 = rp / 4;
  bool found = false;
  SvidPlan best{};
  long best_key = 0;
  for (int ii = 0; ii < kNumInst; ++ii) {
    const Inst& in = kInst[ii];
    int TX;
    if (!in.guard) {
      if (rp4 % in.nu) continue;
      TX = rp4 / in.nu;
      if (TX % 64) continue;
    } else {
      TX = (int)round_up((rp4 + in.nu - 1) / in.nu, 64);
    }
    if (TX > kMaxNT) continue;
    for (int G = Gmax; G >= 64; G /= 2) {
      if (rows_pad % G || G > 2 * TX) continue;  // each thread reads at most two slabs' aa
      int nqo = 1;  // column quads per owner: a power of two covering rp / 4 over G owners
      while (nqo * G < rp4) nqo *= 2;
      if (4 * nqo > kMaxKW) continue;
      const int RS = rows_pad / G;
      if (RS > 8192) continue;  // a of the slab's rows in LDS (32 KB)
      if (in.res && RS != in.rpt) continue;
      const int NCH = (RS + in.rpt - 1) / in.rpt;
      // resident first, then fewer chunks, more threads, exact columns
      const long key = ((long)(in.res ? 0 : 1) << 50) | ((long)NCH << 30) |
                       (((long)(1 << 20) - (long)G * TX / 64) << 2) | (in.guard ? 1 : 0);
      if (!found || key < best_key) {
        found = true;
        best_key = key;
        best = SvidPlan{G, RS, TX, 1, in.nu, in.rpt, NCH, nqo, ii};
      }
    }
  }
  if (found) *out = best;
  return found;
}

size_t svid_sync_words(int rp, int G) { return (size_t)rp * G + G + rp + 1 + (G + 1) / 2; }

SvidSync svid_sync_at(uint64_t* base, int rp, int G) {
  SvidSync s;
  s.part = base;
  s.aa = base + (size_t)rp * G;
  s.b = s.aa + G;
  s.ctl = (uint32_t*)(s.b + rp);
  s.prog = s.ctl + 2;
  return s;
}

int svid_grid() { return grid_size(); }

hipError_t launch_svid(float* X, float* P, int rows_pad, int rp, int r_real, int T, int mode,
                       const SvidWork& w, hipStream_t s, const float* Uadd) {
  if (rp % 128 || rows_pad < 1 || T < 1) return hipErrorInvalidValue;
  SvidPlan p;
  if ((w.G != 64 && w.G != 128 && w.G != 256) || !svid_plan(rows_pad, rp, w.G, &p))
    return hipErrorInvalidValue;
  SvidArgs A{};
  A.X = X;
  A.Uadd = Uadd;
  A.P = P;
  A.a_out = w.a;
  A.b_out = w.b;
  A.sy = w.sy;
  A.st = w.st;
  A.rp = rp;
  A.r_real = r_real;
  A.T = T;
  A.mode = mode;
  A.G = p.G;
  A.RS = p.RS;
  A.RPT = p.RPT;
  A.NCH = p.NCH;
  A.NQO = p.NQO;
  const dim3 grid(p.G), block(p.TX);
  const size_t lds =
      sizeof(float) * (size_t)(((p.RS + 3) & ~3) + std::max(4 * p.TX, p.G * 4 * p.NQO));
#define NQ_SVID_CASE(i, nu, rpt, res, gd)                                                  \
  case i:                                                                               \
    hipLaunchKernelGGL((svid_grid_kernel<nu, rpt, res, gd>), grid, block, lds, s, A);   \
    break;
  switch (p.inst) {
    NQ_SVID_INSTANCES(NQ_SVID_CASE)
    default: return hipErrorInvalidValue;
  }
#undef NQ_SVID_CASE
  return hipGetLastError();
}

hipError_t launch_colsumsq(const float* F, int rows_pad, int rp, float* colpart, hipStream_t s) {
  if (rp % 128) return hipErrorInvalidValue;
  const int nch = svid_nchunks(rows_pad);
  hipLaunchKernelGGL(colsumsq_kernel, dim3(rp / 128, nch), dim3(256), 0, s, F, rp, rows_pad,
                     colpart);
  return hipGetLastError();
}

}  // namespace nq
