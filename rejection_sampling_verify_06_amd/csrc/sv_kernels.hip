// Kernels of the batched speculative-decoding verify step for gfx950.
//
// row_stats   one block per (logit row, 32 KB chunk).  The block issues its
//             chunk's 16-byte non-temporal loads first; wave 0 finds the
//             sequence that owns the row (a wave-level scan of num_draft,
//             served from cache while the chunk is in flight).  The chunk is
//             reduced in float32 to (max of the raw logits, sum of
//             exp2(x*c - round(max*c)), lowest-index argmax for greedy rows):
//             block max first, then one sum against it.  No inter-block
//             communication.
// scan        one 64-lane wave per sequence: validates the sequence, merges
//             each row's chunk partials in chunk order (lane r: row r),
//             computes p and q at the proposals, draws the Philox uniforms,
//             runs the left-to-right acceptance test (lane i: position i, the
//             stop position from a ballot) and writes everything but the
//             final token.
// tile_sums   one block per (sequence, 8192-element tile) of the row(s) at
//             the stop position: sum of the unnormalised final weights.
// select      one block per sequence: picks the tile holding t = u * Z,
//             re-reads it, prefix-sums it across the block and emits the
//             first token whose inclusive prefix exceeds t.
//
// The method (accept with probability min(1, p/q), stop at the first
// rejection, redraw from norm(max(0, p - q)) or take a bonus token from the
// next target distribution) follows "Draft Model（草稿模型）"
// (compassingai.com) section 2 and its one-step algorithm box; the one-hot
// proposal follows "5.2 Draft 模型与无模型方案" (AIInfraGuide) section 4.3;
// temperature on both rows follows the gitcode.csdn.net tutorial section 4.3.
// The path is a memory-bound streaming reduction: no matrix cores are used.
// Blocks never wait on one another: ordering comes only from kernel
// boundaries, so there are no device-scope fences (each one writes back a
// whole L2 on this chip) and no spin loops.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"

namespace sv {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;
constexpr int kWaves = kThreads / kWave;
constexpr int kNV = 8;   // 16-byte vectors per thread per 32 KB chunk
constexpr int kSample = 0, kGreedy = 1, kOnehot = 2;
constexpr int kStBadLayout = 1, kStKTooLarge = 2, kStBadMode = 4, kStBadTemp = 8, kStNoDraft = 16,
              kStBadToken = 32, kStNonfinite = 64, kStZeroResidual = 128;
constexpr float kMinTemperature = 1e-6f;
constexpr uint32_t kNaNBits = 0x7FC00000u;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// multiply/xor S-box with the key bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo_a = 0xD2511F53u * c0, hi_a = __umulhi(0xD2511F53u, c0);
    const uint32_t lo_b = 0xCD9E8D57u * c2, hi_b = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
  }
  return c0;
}

// uniform in [0, 1) on the 2^-24 grid for (sequence, position, purpose)
__device__ __forceinline__ float draw_uniform(const Params& P, uint32_t seq_id, uint32_t pos, uint32_t purpose) {
  const uint32_t w = philox_word0(pos, purpose, seq_id, 0u, P.seed_lo, P.seed_hi);
  return (float)(w >> 8) * 0x1p-24f;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float load_logit(const void* base, int64_t idx, int bf16) {
  if (bf16) return __uint_as_float(((uint32_t)((const uint16_t*)base)[idx]) << 16);
  return ((const float*)base)[idx];
}

// Merge two (max, scaled sum, argmax) triples.  s is relative to
// round(m * c); the result is relative to round(max(m, m2) * c).  The
// products are rounded on their own (the library is built without implicit
// fusion), so a partial is rescaled by exactly the reference it was summed
// against.  NaN in a sum propagates; two empty (-inf) sides add their sums.
template <bool ARG>
__device__ __forceinline__ void merge_stats(float& m, float& s, int& idx, float m2, float s2, int idx2, float c) {
  const float mn = fmaxf(m, m2);
  if (ARG) idx = (m2 > m) ? idx2 : ((m > m2) ? idx : min(idx, idx2));
  if (mn == -INFINITY) {
    s = s + s2;
  } else {
    const float mc = mn * c;
    s = s * fexp2(m * c - mc) + s2 * fexp2(m2 * c - mc);
  }
  m = mn;
}

template <bool ARG>
__device__ __forceinline__ void wave_merge(float& m, float& s, int& idx, float c) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave);
    const float s2 = __shfl_xor(s, off, kWave);
    const int i2 = ARG ? __shfl_xor(idx, off, kWave) : 0;
    merge_stats<ARG>(m, s, idx, m2, s2, i2, c);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int64_t wave_incl_scan_i64(int64_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// ---------------------------------------------------------------------------
// which sequence owns a row, with its temperature and mode.  Every wave
// works it out on its own (no LDS, no barrier): lane l takes a window of
// consecutive sequences, sums their row counts (K_s + 1 target rows or K_s
// draft rows), a wave scan gives each lane its first row, and the lane whose
// interval holds the row names the owner.  Returns -1 if no sequence owns
// the row (inconsistent num_draft: the scan kernel then reports a bad
// layout).
//
// Batches of up to 256 sequences use a 4-sequence window per lane that is
// loaded before the chunk's own loads are issued: vector loads complete in
// issue order, so the lookup then never waits for the chunk.
// ---------------------------------------------------------------------------
constexpr int kWin = 4;

struct SeqWindow {
  int k[kWin];
  float T[kWin];
  int md[kWin];
};

// Raw loads only (index clamped, no branches): nothing reads these registers
// until the chunk's loads have been issued.
__device__ __forceinline__ SeqWindow load_window(const Params& P) {
  SeqWindow w;
  const int base = (threadIdx.x & (kWave - 1)) * kWin;
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    const int s = min(base + i, P.B - 1);
    w.k[i] = P.num_draft[s];
    w.T[i] = P.temperature[s];
    w.md[i] = P.mode[s];
  }
  return w;
}

struct Owner {
  int s;       // owning sequence, -1 if none
  float T;
  int md;
  int first;   // first row of the owner's rows in this segment
  int K;       // the owner's K_s
};

// lowest lane that claims the row (a consistent layout has exactly one)
__device__ __forceinline__ Owner owner_from_lanes(int owner, float T, int md, int first, int K) {
  const unsigned long long hits = __ballot(owner >= 0);
  Owner o{-1, 1.f, kSample, 0, 0};
  if (hits == 0ull) return o;
  const int src = (int)__builtin_ctzll(hits);
  o.s = __builtin_amdgcn_readfirstlane(__shfl(owner, src, kWave));
  o.T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(__shfl(T, src, kWave))));
  o.md = __builtin_amdgcn_readfirstlane(__shfl(md, src, kWave));
  o.first = __builtin_amdgcn_readfirstlane(__shfl(first, src, kWave));
  o.K = __builtin_amdgcn_readfirstlane(__shfl(K, src, kWave));
  return o;
}

// 32-bit unsigned arithmetic (wraps instead of overflowing on a corrupt
// num_draft; a consistent layout has fewer than 2^31 rows).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ Owner owner_in_window(const SeqWindow& w, const Params& P, int plus_one, int r) {
  const int base = (threadIdx.x & (kWave - 1)) * kWin;
  uint32_t cnt[kWin];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    cnt[i] = (base + i < P.B) ? (uint32_t)w.k[i] + (uint32_t)plus_one : 0u;
    sum += cnt[i];
  }
  uint32_t start = wave_incl_scan_u32(sum) - sum;
  int owner = -1, first = 0, K = 0;
  float T = 1.f;
  int md = kSample;
  const uint32_t ur = (uint32_t)r;
#pragma unroll
  for (int i = 0; i < kWin; ++i) {
    // (ur - start) < cnt  <=>  start <= ur < start + cnt, without overflow
    if (ur - start < cnt[i]) {
      owner = base + i;
      T = w.T[i];
      md = w.md[i];
      first = (int)start;
      K = w.k[i];
    }
    start += cnt[i];
  }
  return owner_from_lanes(owner, T, md, first, K);
}

// any batch size: lane l takes sequences [l*per, (l+1)*per)
__device__ __forceinline__ Owner owner_general(const Params& P, int plus_one, int64_t r) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (P.B + kWave - 1) / kWave;
  const int lo = min(P.B, lane * per), hi = min(P.B, lo + per);
  int64_t sum = 0;
  for (int s = lo; s < hi; ++s) sum += (int64_t)P.num_draft[s] + plus_one;
  int64_t start = wave_incl_scan_i64(sum) - sum;
  int owner = -1, first = 0, K = 0;
  for (int s = lo; s < hi; ++s) {
    const int64_t cnt = (int64_t)P.num_draft[s] + plus_one;
    if (r >= start && r < start + cnt) {
      owner = s;
      first = (int)start;
      K = P.num_draft[s];
    }
    start += cnt;
  }
  const float T = (owner >= 0) ? P.temperature[owner] : 1.f;
  const int md = (owner >= 0) ? (int)P.mode[owner] : kSample;
  return owner_from_lanes(owner, T, md, first, K);
}

// ---------------------------------------------------------------------------
// thread-local statistics of a chunk
// ---------------------------------------------------------------------------

// Thread t loads vectors (u*256 + t), u < 8, of the chunk starting at c0.
// TAIL: the chunk ends at c1 before its 32 KB are up; vectors past c1 are
// loaded from the row's first 16 bytes instead (in bounds: the row has at
// least one vector) and replaced by -inf in mask_chunk.
template <bool BF16, bool TAIL>
__device__ __forceinline__ void load_chunk(const char* rowp, int c0, int c1, u32x4 (&v)[kNV]) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int ES = BF16 ? 2 : 4;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kNV; ++u) {
    const int e = c0 + (u * kThreads + t) * VEC;
    const int a = (!TAIL || e + VEC <= c1) ? e : 0;
    v[u] = __builtin_nontemporal_load((const u32x4*)(rowp + (int64_t)a * ES));
  }
}

// Replace what lies past c1 by -inf; the one vector that straddles c1 is
// rebuilt from element loads.
template <bool BF16>
__device__ __forceinline__ void mask_chunk(const char* rowp, int c0, int c1, u32x4 (&v)[kNV]) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int t = threadIdx.x;
#pragma unroll
  for (int u = 0; u < kNV; ++u) {
    const int e = c0 + (u * kThreads + t) * VEC;
    if (e + VEC > c1) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          const int e0 = e + 2 * q, e1 = e0 + 1;
          const uint32_t lo = (e0 < c1) ? (uint32_t)((const uint16_t*)rowp)[e0] : 0xFF80u;
          const uint32_t hi = (e1 < c1) ? (uint32_t)((const uint16_t*)rowp)[e1] : 0xFF80u;
          w[q] = lo | (hi << 16);
        } else {
          const int e0 = e + q;
          w[q] = (e0 < c1) ? ((const uint32_t*)rowp)[e0] : 0xFF800000u;
        }
      }
      v[u] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

// Rows that are not 16-byte aligned (or shorter than one vector): element
// e = c0 + j*256 + t, eight loads in flight per thread, each batch merged
// into the running (max, sum, argmax).
template <bool ARG>
__device__ __forceinline__ void stats_scalar(const void* row, int bf16, int c0, int c1, float c, float& m_out,
                                             float& s_out, int& i_out) {
  constexpr int NB = 8;
  float m = -INFINITY, s = 0.f;
  int idx = 0x7FFFFFFF;
  for (int b0 = c0 + (int)threadIdx.x; b0 < c1; b0 += NB * kThreads) {
    float x[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = b0 + j * kThreads;
      const float v = load_logit(row, min(e, c1 - 1), bf16);
      x[j] = (e < c1) ? v : -INFINITY;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NB; ++j) bm = fmaxf(bm, x[j]);
    int bi = 0x7FFFFFFF;
    if (ARG) {
#pragma unroll
      for (int j = NB - 1; j >= 0; --j)
        if (x[j] == bm) bi = b0 + j * kThreads;
    }
    const float bmc = (bm == -INFINITY) ? 0.f : bm * c;
    float bs = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) bs += fexp2(fmaf(x[j], c, -bmc));
    merge_stats<ARG>(m, s, idx, bm, bs, bi, c);
  }
  m_out = m;
  s_out = s;
  i_out = idx;
}

// ---------------------------------------------------------------------------
// block helpers (256 threads)
// ---------------------------------------------------------------------------

// exclusive prefix of one float per thread in thread order; *total = sum
__device__ __forceinline__ float block_excl_scan(float v, float* s_w, float* total) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  float inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) s_w[wv] = inc;
  __syncthreads();
  float before = 0.f;
  for (int w = 0; w < wv; ++w) before += s_w[w];
  float tot = 0.f;
  for (int w = 0; w < kWaves; ++w) tot += s_w[w];
  *total = tot;
  __syncthreads();
  return before + inc - v;
}

__device__ __forceinline__ float block_sum(float v, float* s_w) {
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = v;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < kWaves; ++w) tot += s_w[w];
  __syncthreads();
  return tot;
}

__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t* s_w) {
  v = wave_sum_i64(v);
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = v;
  __syncthreads();
  int64_t tot = 0;
  for (int w = 0; w < kWaves; ++w) tot += s_w[w];
  __syncthreads();
  return tot;
}

// ---------------------------------------------------------------------------
// the final draw at the stop position: tiles of 8192 elements, 256 threads
// ---------------------------------------------------------------------------
constexpr int kTileVec = kTileElems / kThreads;   // 32 elements per thread per tile

__device__ __forceinline__ float final_weight(int kind, float x, float y, int k, const SeqFinal& f) {
  const float p = fexp2(fmaf(x, f.c, -f.mct)) * f.inv_st;
  if (kind == kFinalResidual) {
    const float q = fexp2(fmaf(y, f.c, -f.mcd)) * f.inv_sd;
    return fmaxf(p - q, 0.f);
  }
  if (kind == kFinalOnehot && k == f.xhat) return 0.f;
  return p;
}

// This thread's share of the weight of tile j (coalesced: thread t owns
// elements base + (u*256 + t)*VEC .. +VEC); every load is issued before use.
// TAIL (the row's last tile): vectors past V are loaded from the row's
// first 16 bytes instead and then replaced by -inf logits (weight 0); the
// one vector that straddles V is rebuilt from element loads.
template <bool BF16, int KIND, bool TAIL>
__device__ __forceinline__ float tile_part_vec(const Params& P, const SeqFinal& f, int j) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int NV = kTileVec / VEC;
  constexpr int ES = BF16 ? 2 : 4;
  const int t = threadIdx.x;
  const int base = j * kTileElems;
  const int V = P.V;
  const char* tp = (const char*)P.tgt + (int64_t)f.trow * P.ld_t * ES;
  const char* dp = (KIND == kFinalResidual) ? (const char*)P.dft + (int64_t)f.drow * P.ld_d * ES : nullptr;
  u32x4 vt[NV], vd[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = base + (u * kThreads + t) * VEC;
    const int a = (!TAIL || e + VEC <= V) ? e : 0;
    vt[u] = __builtin_nontemporal_load((const u32x4*)(tp + (int64_t)a * ES));
    if (KIND == kFinalResidual) vd[u] = __builtin_nontemporal_load((const u32x4*)(dp + (int64_t)a * ES));
  }
  if (TAIL) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = base + (u * kThreads + t) * VEC;
      if (e + VEC > V) {
        uint32_t wt[4], wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (BF16) {
            const int e0 = e + 2 * q, e1 = e0 + 1;
            wt[q] = ((e0 < V) ? (uint32_t)((const uint16_t*)tp)[e0] : 0xFF80u) |
                    (((e1 < V) ? (uint32_t)((const uint16_t*)tp)[e1] : 0xFF80u) << 16);
            if (KIND == kFinalResidual)
              wd[q] = ((e0 < V) ? (uint32_t)((const uint16_t*)dp)[e0] : 0xFF80u) |
                      (((e1 < V) ? (uint32_t)((const uint16_t*)dp)[e1] : 0xFF80u) << 16);
          } else {
            const int e0 = e + q;
            wt[q] = (e0 < V) ? ((const uint32_t*)tp)[e0] : 0xFF800000u;
            if (KIND == kFinalResidual) wd[q] = (e0 < V) ? ((const uint32_t*)dp)[e0] : 0xFF800000u;
          }
        }
        vt[u] = u32x4{wt[0], wt[1], wt[2], wt[3]};
        if (KIND == kFinalResidual) vd[u] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      }
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = base + (u * kThreads + t) * VEC;
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      float x, y = 0.f;
      if (BF16) {
        x = (q & 1) ? bf_hi(vt[u][q >> 1]) : bf_lo(vt[u][q >> 1]);
        if (KIND == kFinalResidual) y = (q & 1) ? bf_hi(vd[u][q >> 1]) : bf_lo(vd[u][q >> 1]);
      } else {
        x = __uint_as_float(vt[u][q]);
        if (KIND == kFinalResidual) y = __uint_as_float(vd[u][q]);
      }
      acc += final_weight(KIND, x, y, e + q, f);
    }
  }
  return acc;
}

// Rows that are not 16-byte aligned, shorter than a vector, or a residual
// whose two rows differ in type: element loads clamped to V - 1, weights
// past V zeroed.
__device__ __forceinline__ float tile_part_generic(const Params& P, const SeqFinal& f, int kind, int j) {
  const int base = j * kTileElems;
  const int64_t toff = (int64_t)f.trow * P.ld_t, doff = (int64_t)f.drow * P.ld_d;
  float acc = 0.f;
  for (int u0 = 0; u0 < kTileVec; u0 += 8) {
    float x[8], y[8];
    int ee[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ee[q] = base + (u0 + q) * kThreads + (int)threadIdx.x;
      const int e = min(ee[q], P.V - 1);
      x[q] = load_logit(P.tgt, toff + e, P.t_bf16);
      y[q] = (kind == kFinalResidual) ? load_logit(P.dft, doff + e, P.d_bf16) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) acc += (ee[q] < P.V) ? final_weight(kind, x[q], y[q], ee[q], f) : 0.f;
  }
  return acc;
}

template <bool BF16, int KIND>
__device__ __forceinline__ float tile_part_k(const Params& P, const SeqFinal& f, int j) {
  if ((j + 1) * kTileElems <= P.V) return tile_part_vec<BF16, KIND, false>(P, f, j);
  return tile_part_vec<BF16, KIND, true>(P, f, j);
}

__device__ __forceinline__ float tile_part(const Params& P, const SeqFinal& f, int kind, int j) {
  const int vecmin = P.t_bf16 ? 8 : 4;
  const bool vec = P.t_vec && P.V >= vecmin && (kind != kFinalResidual || (P.d_vec && P.d_bf16 == P.t_bf16));
  if (vec) {
    if (P.t_bf16) {
      if (kind == kFinalResidual) return tile_part_k<true, kFinalResidual>(P, f, j);
      if (kind == kFinalOnehot) return tile_part_k<true, kFinalOnehot>(P, f, j);
      return tile_part_k<true, kFinalBonus>(P, f, j);
    }
    if (kind == kFinalResidual) return tile_part_k<false, kFinalResidual>(P, f, j);
    if (kind == kFinalOnehot) return tile_part_k<false, kFinalOnehot>(P, f, j);
    return tile_part_k<false, kFinalBonus>(P, f, j);
  }
  return tile_part_generic(P, f, kind, j);
}

// The weights of tile jj into LDS in element order (index e + e/32, so that
// each thread's run of 32 consecutive weights is bank-conflict free), loaded
// with the same coalesced, masked vector loads as tile_part_vec.
__device__ __forceinline__ int lds_pad(int e) { return e + (e >> 5); }
constexpr int kTileLds = kTileElems + kTileElems / 32;

template <bool BF16, int KIND, bool TAIL>
__device__ __forceinline__ void tile_weights_lds_vec(const Params& P, const SeqFinal& f, int j, float* lw) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int NV = kTileVec / VEC;
  constexpr int ES = BF16 ? 2 : 4;
  const int t = threadIdx.x;
  const int base = j * kTileElems;
  const int V = P.V;
  const char* tp = (const char*)P.tgt + (int64_t)f.trow * P.ld_t * ES;
  const char* dp = (KIND == kFinalResidual) ? (const char*)P.dft + (int64_t)f.drow * P.ld_d * ES : nullptr;
  u32x4 vt[NV], vd[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = base + (u * kThreads + t) * VEC;
    const int a = (!TAIL || e + VEC <= V) ? e : 0;
    vt[u] = __builtin_nontemporal_load((const u32x4*)(tp + (int64_t)a * ES));
    if (KIND == kFinalResidual) vd[u] = __builtin_nontemporal_load((const u32x4*)(dp + (int64_t)a * ES));
  }
  if (TAIL) {
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = base + (u * kThreads + t) * VEC;
      if (e + VEC > V) {
        uint32_t wt[4], wd[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (BF16) {
            const int e0 = e + 2 * q, e1 = e0 + 1;
            wt[q] = ((e0 < V) ? (uint32_t)((const uint16_t*)tp)[e0] : 0xFF80u) |
                    (((e1 < V) ? (uint32_t)((const uint16_t*)tp)[e1] : 0xFF80u) << 16);
            if (KIND == kFinalResidual)
              wd[q] = ((e0 < V) ? (uint32_t)((const uint16_t*)dp)[e0] : 0xFF80u) |
                      (((e1 < V) ? (uint32_t)((const uint16_t*)dp)[e1] : 0xFF80u) << 16);
          } else {
            const int e0 = e + q;
            wt[q] = (e0 < V) ? ((const uint32_t*)tp)[e0] : 0xFF800000u;
            if (KIND == kFinalResidual) wd[q] = (e0 < V) ? ((const uint32_t*)dp)[e0] : 0xFF800000u;
          }
        }
        vt[u] = u32x4{wt[0], wt[1], wt[2], wt[3]};
        if (KIND == kFinalResidual) vd[u] = u32x4{wd[0], wd[1], wd[2], wd[3]};
      }
    }
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int el = (u * kThreads + t) * VEC;    // element index within the tile
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
      float x, y = 0.f;
      if (BF16) {
        x = (q & 1) ? bf_hi(vt[u][q >> 1]) : bf_lo(vt[u][q >> 1]);
        if (KIND == kFinalResidual) y = (q & 1) ? bf_hi(vd[u][q >> 1]) : bf_lo(vd[u][q >> 1]);
      } else {
        x = __uint_as_float(vt[u][q]);
        if (KIND == kFinalResidual) y = __uint_as_float(vd[u][q]);
      }
      lw[lds_pad(el + q)] = final_weight(KIND, x, y, base + el + q, f);
    }
  }
}

// Any row alignment: element e = base + u*256 + t, loads clamped, weights past V zeroed.
__device__ __forceinline__ void tile_weights_lds_generic(const Params& P, const SeqFinal& f, int kind, int j,
                                                         float* lw) {
  const int base = j * kTileElems;
  const int64_t toff = (int64_t)f.trow * P.ld_t, doff = (int64_t)f.drow * P.ld_d;
  for (int u0 = 0; u0 < kTileVec; u0 += 8) {
    float x[8], y[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = min(base + (u0 + q) * kThreads + (int)threadIdx.x, P.V - 1);
      x[q] = load_logit(P.tgt, toff + e, P.t_bf16);
      y[q] = (kind == kFinalResidual) ? load_logit(P.dft, doff + e, P.d_bf16) : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int el = (u0 + q) * kThreads + (int)threadIdx.x;
      lw[lds_pad(el)] = (base + el < P.V) ? final_weight(kind, x[q], y[q], base + el, f) : 0.f;
    }
  }
}

template <bool BF16, int KIND>
__device__ __forceinline__ void tile_weights_lds_k(const Params& P, const SeqFinal& f, int j, float* lw) {
  if ((j + 1) * kTileElems <= P.V) tile_weights_lds_vec<BF16, KIND, false>(P, f, j, lw);
  else tile_weights_lds_vec<BF16, KIND, true>(P, f, j, lw);
}

__device__ __forceinline__ void tile_weights_lds(const Params& P, const SeqFinal& f, int kind, int j, float* lw) {
  const int vecmin = P.t_bf16 ? 8 : 4;
  const bool vec = P.t_vec && P.V >= vecmin && (kind != kFinalResidual || (P.d_vec && P.d_bf16 == P.t_bf16));
  if (vec) {
    if (P.t_bf16) {
      if (kind == kFinalResidual) tile_weights_lds_k<true, kFinalResidual>(P, f, j, lw);
      else if (kind == kFinalOnehot) tile_weights_lds_k<true, kFinalOnehot>(P, f, j, lw);
      else tile_weights_lds_k<true, kFinalBonus>(P, f, j, lw);
    } else {
      if (kind == kFinalResidual) tile_weights_lds_k<false, kFinalResidual>(P, f, j, lw);
      else if (kind == kFinalOnehot) tile_weights_lds_k<false, kFinalOnehot>(P, f, j, lw);
      else tile_weights_lds_k<false, kFinalBonus>(P, f, j, lw);
    }
  } else {
    tile_weights_lds_generic(P, f, kind, j, lw);
  }
}

// clear the outputs of a sequence that is not verified
__device__ __forceinline__ void clear_sequence(const Params& P, int s, int off_t, int off_d, int K, int st) {
  const int t = threadIdx.x;
  for (int j = t; j <= K; j += blockDim.x) P.emitted[off_t + j] = -1;
  for (int j = t; j < K; j += blockDim.x) {
    if (P.p_at) P.p_at[off_d + j] = __uint_as_float(kNaNBits);
    if (P.q_at) P.q_at[off_d + j] = __uint_as_float(kNaNBits);
  }
  if (t == 0) {
    P.accepted_len[s] = -1;
    if (P.status) P.status[s] = st;
  }
}

// Block-wide merge of the threads' (max, sum, argmax) and the partial write.
template <bool ARG>
__device__ __forceinline__ void finish_chunk(const Params& P, float m, float sum, int idx, float c) {
  __shared__ float s_m[kWaves], s_s[kWaves];
  __shared__ int s_i[kWaves];
  wave_merge<ARG>(m, sum, idx, c);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (lane == 0) {
    s_m[wv] = m;
    s_s[wv] = sum;
    s_i[wv] = idx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = s_m[0], S = s_s[0];
    int I = s_i[0];
    for (int q = 1; q < kWaves; ++q) merge_stats<true>(M, S, I, s_m[q], s_s[q], s_i[q], c);
    P.partials[blockIdx.x] = Partial{M, S, I, 0};    // block index == partial index
  }
}

__device__ __forceinline__ float row_scale(int md, float T) { return (md == kGreedy) ? kLog2e : kLog2e / T; }

// The proposed token that row `row` judges (target rows 0..K-1 and draft
// rows of a sequence), or -1 (bonus row, or an index that the host-declared
// total_draft does not cover, which only a corrupt num_draft can produce).
__device__ __forceinline__ int row_proposal(const Params& P, const Owner& own, int row, bool is_draft) {
  const int i = row - own.first;
  if (i < 0 || i >= own.K) return -1;
  const int off_d = is_draft ? own.first : own.first - own.s;
  const int idx = off_d + i;
  if (idx < 0 || idx >= P.total_draft) return -1;
  return P.tokens[idx];
}

// The logit at the proposal, taken from the chunk held in registers by the
// thread that loaded it, stored for the scan kernel (xval[row]).
template <bool BF>
__device__ __forceinline__ void record_proposal_logit(const Params& P, const float (&f)[kNV * (BF ? 8 : 4)], int c0,
                                                      int c1, int x, int64_t grow) {
  constexpr int VEC = BF ? 8 : 4;
  constexpr int N = kNV * VEC;
  if (x < c0 || x >= c1) return;
  const int o = x - c0;
  const int vi = o / VEC;
  if ((vi & (kThreads - 1)) != (int)threadIdx.x) return;
  const int k = (vi / kThreads) * VEC + o % VEC;
  // constant register indices only (a runtime index would spill f to scratch)
  float val = 0.f;
#pragma unroll
  for (int kk = 0; kk < N; ++kk)
    if (kk == k) val = f[kk];
  P.xval[grow] = val;
}

template <bool BF>
__device__ __forceinline__ void unpack_chunk(const u32x4 (&v)[kNV], float (&f)[kNV * (BF ? 8 : 4)]) {
#pragma unroll
  for (int u = 0; u < kNV; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (BF) {
        f[u * 8 + 2 * q] = bf_lo(v[u][q]);
        f[u * 8 + 2 * q + 1] = bf_hi(v[u][q]);
      } else {
        f[u * 4 + q] = __uint_as_float(v[u][q]);
      }
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, kWave));
  return v;
}

// What wave 0 of a row-statistics block hands to the other waves.
struct StatsShared {
  float m[kWaves];
  float s[kWaves];
  int i[kWaves];
  Owner own;
  int x;          // token the row judges, or -1
};

__device__ __forceinline__ void publish_owner(const Params& P, StatsShared& sh, const Owner& own, int row,
                                              bool is_draft) {
  const int x = (own.s >= 0) ? row_proposal(P, own, row, is_draft) : -1;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.own = own;
    sh.x = x;
  }
}

// A 16-byte aligned chunk (full, or the row's last when TAIL).  Every wave
// issues its share of the chunk's loads at once; wave 0 alone also looks up
// the owning sequence (its window loads go first, so the lookup overlaps the
// chunk's flight) and publishes it in LDS.  The block first agrees on the
// chunk maximum M, then every thread sums exp2(x*c - round(M*c)) against that
// common reference, so the block's partial is a plain sum (no rescaling).
template <bool BF, bool TAIL>
__device__ __forceinline__ void row_stats_vec(const Params& P, const char* rowp, int row, int c0, int c1,
                                              int plus_one, bool is_draft) {
  constexpr int VEC = BF ? 8 : 4;
  constexpr int N = kNV * VEC;
  __shared__ StatsShared sh;
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  u32x4 v[kNV];
  if (wv == 0) {
    if (P.B <= kWave * kWin) {
      const SeqWindow win = load_window(P);
      __builtin_amdgcn_sched_barrier(0);
      load_chunk<BF, TAIL>(rowp, c0, c1, v);
      __builtin_amdgcn_sched_barrier(0);
      publish_owner(P, sh, owner_in_window(win, P, plus_one, row), row, is_draft);
    } else {
      load_chunk<BF, TAIL>(rowp, c0, c1, v);
      publish_owner(P, sh, owner_general(P, plus_one, row), row, is_draft);
    }
  } else {
    load_chunk<BF, TAIL>(rowp, c0, c1, v);
  }
  if (TAIL) mask_chunk<BF>(rowp, c0, c1, v);
  float f[N];
  unpack_chunk<BF>(v, f);
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) mx = fmaxf(mx, f[k]);
  mx = wave_max(mx);
  if (lane == 0) sh.m[wv] = mx;
  __syncthreads();
  const Owner own = sh.own;
  if (own.s < 0) return;                   // the whole block: inconsistent layout
  const float M = fmaxf(fmaxf(sh.m[0], sh.m[1]), fmaxf(sh.m[2], sh.m[3]));
  const float c = row_scale(own.md, own.T);
  const float mc = (M == -INFINITY) ? 0.f : M * c;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int k = 0; k < N; k += 4) {
    a0 += fexp2(fmaf(f[k + 0], c, -mc));
    a1 += fexp2(fmaf(f[k + 1], c, -mc));
    a2 += fexp2(fmaf(f[k + 2], c, -mc));
    a3 += fexp2(fmaf(f[k + 3], c, -mc));
  }
  const float sum = wave_sum((a0 + a1) + (a2 + a3));
  int idx = 0x7FFFFFFF;
  if (own.md == kGreedy && !is_draft) {    // lowest index attaining M
#pragma unroll
    for (int k = N - 1; k >= 0; --k)
      if (f[k] == M) idx = c0 + ((k / VEC) * kThreads + t) * VEC + (k % VEC);
    idx = wave_min_i(idx);
  }
  record_proposal_logit<BF>(P, f, c0, c1, sh.x, is_draft ? (int64_t)P.n_t + row : (int64_t)row);
  if (lane == 0) {
    sh.s[wv] = sum;
    sh.i[wv] = idx;
  }
  __syncthreads();
  if (t == 0) {
    const float S = (sh.s[0] + sh.s[1]) + (sh.s[2] + sh.s[3]);
    const int I = min(min(sh.i[0], sh.i[1]), min(sh.i[2], sh.i[3]));
    P.partials[blockIdx.x] = Partial{M, S, I, 0};    // block index == partial index
  }
}

// Rows that are not 16-byte aligned, or shorter than one vector.
__device__ __forceinline__ void row_stats_scalar(const Params& P, const char* rowp, int bf, int row, int c0, int c1,
                                                 int plus_one, bool is_draft) {
  const Owner own = owner_general(P, plus_one, row);
  if (own.s < 0) return;
  const int x = row_proposal(P, own, row, is_draft);
  if (threadIdx.x == 0 && x >= c0 && x < c1)
    P.xval[is_draft ? (int64_t)P.n_t + row : (int64_t)row] = load_logit(rowp, x, bf);
  const float c = row_scale(own.md, own.T);
  float m, sum;
  int idx;
  if (own.md == kGreedy && !is_draft) {
    stats_scalar<true>(rowp, bf, c0, c1, c, m, sum, idx);
    finish_chunk<true>(P, m, sum, idx, c);
  } else {
    stats_scalar<false>(rowp, bf, c0, c1, c, m, sum, idx);
    finish_chunk<false>(P, m, sum, idx, c);
  }
}

template <bool BF>
__device__ __forceinline__ void row_stats_seg(const Params& P, const char* rowp, int vec, int row, int c0, int ce,
                                              int plus_one, bool is_draft) {
  constexpr int VEC = BF ? 8 : 4;
  const int c1 = min(P.V, c0 + ce);
  if (vec && P.V >= VEC) {
    if (c0 + ce <= P.V) row_stats_vec<BF, false>(P, rowp, row, c0, c1, plus_one, is_draft);
    else row_stats_vec<BF, true>(P, rowp, row, c0, c1, plus_one, is_draft);
  } else {
    row_stats_scalar(P, rowp, BF, row, c0, c1, plus_one, is_draft);
  }
}

template <bool TB, bool DB>
__device__ __forceinline__ void row_stats_body(const Params& P) {
  const int b = blockIdx.x;
  const int nblk_t = P.n_t * P.nch_t;
  const bool is_draft = b >= nblk_t;
  const int bb = is_draft ? b - nblk_t : b;
  const int nch = is_draft ? P.nch_d : P.nch_t;
  const int row = bb / nch;
  const int chunk = bb - row * nch;
  if (is_draft) {
    const char* rowp = (const char*)P.dft + (int64_t)row * P.ld_d * (DB ? 2 : 4);
    row_stats_seg<DB>(P, rowp, P.d_vec, row, chunk * P.ce_d, P.ce_d, 0, true);
  } else {
    const char* rowp = (const char*)P.tgt + (int64_t)row * P.ld_t * (TB ? 2 : 4);
    row_stats_seg<TB>(P, rowp, P.t_vec, row, chunk * P.ce_t, P.ce_t, 1, false);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

template <bool TB, bool DB>
__global__ void __launch_bounds__(kThreads) k_row_stats(Params P) {
  row_stats_body<TB, DB>(P);
}

// ---------------------------------------------------------------------------
// scan: one 64-lane wave per sequence, so no cross-wave barriers.  Lane r
// merges the chunk partials of row r on its own; lane i judges position i.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = kWave;
constexpr int kMergeUnroll = 16;      // chunk partials a lane has in flight at once

struct ScanShared {
  float M[2 * kMaxK + 1];   // rows 0..K: target, K+1..2K: draft
  float S[2 * kMaxK + 1];
  int I[2 * kMaxK + 1];
  int tok[kMaxK];
};

// Inconsistent num_draft: every output slot is cleared; block s clears its share.
__device__ __forceinline__ void clear_bad_layout(const Params& P, int s) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int64_t stride = (int64_t)P.B * nt;
  for (int64_t e = (int64_t)s * nt + t; e < (int64_t)P.total_draft + P.B; e += stride) P.emitted[e] = -1;
  for (int64_t e = (int64_t)s * nt + t; e < P.total_draft; e += stride) {
    if (P.p_at) P.p_at[e] = __uint_as_float(kNaNBits);
    if (P.q_at) P.q_at[e] = __uint_as_float(kNaNBits);
  }
  if (t == 0) {
    P.accepted_len[s] = -1;
    if (P.status) P.status[s] = kStBadLayout;
  }
}

// Row statistics from the row's chunk partials: M = max of the chunk maxima,
// S = sum of s_k * exp2(round(m_k*c) - round(M*c)), I = lowest index attaining
// M.  The chunks are taken in order; kMergeUnroll loads are issued before any
// is used (indices clamped into the row, surplus entries ignored).
__device__ __forceinline__ void merge_row(const Partial* pp, int nch, float c, float& M, float& S, int& I) {
  M = -INFINITY;
  S = 0.f;
  I = 0x7FFFFFFF;
  for (int k0 = 0; k0 < nch; k0 += kMergeUnroll) {
    Partial q[kMergeUnroll];
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) q[k] = pp[min(k0 + k, nch - 1)];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k)
      if (k0 + k < nch) m = fmaxf(m, q[k].m);
    // fold the running (M, S) into this group's reference
    const float mn = fmaxf(M, m);
    const float mnc = (mn == -INFINITY) ? 0.f : mn * c;
    float sum = (M == -INFINITY) ? S : S * fexp2(M * c - mnc);
    int idx = (M == mn) ? I : 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) {
      if (k0 + k < nch) {
        sum += (q[k].m == -INFINITY) ? q[k].s : q[k].s * fexp2(q[k].m * c - mnc);
        if (q[k].m == mn) idx = min(idx, q[k].idx);
      }
    }
    M = mn;
    S = sum;
    I = idx;
  }
}

// The acceptance scan of sequence s: stores every output of the sequence but
// the final token and returns what the final draw needs (kind kFinalDone when
// nothing is left).  Two dependent rounds of loads: the layout sums with the
// sequence's own inputs, then the proposals, their logits and the rows'
// partials.
__device__ __forceinline__ SeqFinal scan_sequence(const Params& P, int s, ScanShared& sh) {
  const int lane = threadIdx.x;
  SeqFinal f{};
  f.kind = kFinalDone;
  f.s = s;

  // ---- round 1: the sequence's own inputs and the layout sums ----
  const int K = P.num_draft[s];
  const int md = P.mode[s];
  const float T = P.temperature[s];
  const uint32_t seq_id = P.seq_ids[s];
  int64_t tot = 0, bef = 0, neg = 0;
#pragma unroll 4
  for (int j = lane; j < P.B; j += kScanThreads) {
    const int64_t k = P.num_draft[j];
    tot += k;
    bef += (j < s) ? k : 0;
    neg |= (k < 0);
  }
  tot = wave_sum_i64(tot);
  bef = wave_sum_i64(bef);
  neg = wave_sum_i64(neg);
  if (neg != 0 || tot != (int64_t)P.total_draft) {
    clear_bad_layout(P, s);
    return f;
  }
  const int off_d = (int)bef;
  const int off_t = off_d + s;

  int st = 0;
  if (K > P.max_k) st |= kStKTooLarge;
  if (md != kSample && md != kGreedy && md != kOnehot) st |= kStBadMode;
  if ((md == kSample || md == kOnehot) && !(isfinite(T) && T >= kMinTemperature)) st |= kStBadTemp;
  if (md == kSample && K > 0 && P.dft == nullptr) st |= kStNoDraft;
  if (st) {
    clear_sequence(P, s, off_t, off_d, K, st);
    return f;
  }
  const float c = (md == kGreedy) ? kLog2e : kLog2e / T;
  const bool sample = md == kSample;
  const int nrows = K + 1 + (sample ? K : 0);

  // ---- round 2: position `lane`'s proposal and the logits at it, then the
  // rows' chunk partials (lane r: row r); everything issued before any use ----
  int x0 = 0;
  float xt0 = 0.f, xd0 = 0.f;
  if (lane < K) {
    x0 = P.tokens[off_d + lane];
    xt0 = P.xval[off_t + lane];
    if (sample) xd0 = P.xval[(int64_t)P.n_t + off_d + lane];
  }
  int bad = 0;
  for (int r = lane; r < nrows; r += kScanThreads) {
    const bool isd = r > K;
    const Partial* pp = isd ? P.partials + (int64_t)P.n_t * P.nch_t + (int64_t)(off_d + r - K - 1) * P.nch_d
                            : P.partials + (int64_t)(off_t + r) * P.nch_t;
    float M, S;
    int I;
    merge_row(pp, isd ? P.nch_d : P.nch_t, c, M, S, I);
    sh.M[r] = M;
    sh.S[r] = S;
    sh.I[r] = I;
    bad |= !(isfinite(M) && isfinite(S) && S > 0.f);
  }
  int badtok = 0;
  if (lane < K) {
    sh.tok[lane] = x0;
    badtok = (x0 < 0 || x0 >= P.V);
  }
  for (int i = lane + kScanThreads; i < K; i += kScanThreads) {   // K > 64 only
    const int x = P.tokens[off_d + i];
    sh.tok[i] = x;
    badtok |= (x < 0 || x >= P.V);
  }
  if (__any(badtok)) {
    clear_sequence(P, s, off_t, off_d, K, kStBadToken);
    return f;
  }
  if (__any(bad)) {
    clear_sequence(P, s, off_t, off_d, K, kStNonfinite);
    return f;
  }
  __syncthreads();   // the rows' statistics and tokens, written by other lanes

  // ---- p and q at the proposals, uniforms, accept decisions ----
  int A = K;
  for (int i0 = 0; i0 < K; i0 += kScanThreads) {
    const int i = i0 + lane;
    int reject = 0;
    if (i < K) {
      const float xt = (i0 == 0) ? xt0 : P.xval[off_t + i];
      const float xd = (i0 == 0) ? xd0 : (sample ? P.xval[(int64_t)P.n_t + off_d + i] : 0.f);
      const float p = fexp2(fmaf(xt, c, -(sh.M[i] * c))) / sh.S[i];
      const float q = sample ? fexp2(fmaf(xd, c, -(sh.M[K + 1 + i] * c))) / sh.S[K + 1 + i] : 1.f;
      int acc;
      if (md == kGreedy) {
        acc = (sh.tok[i] == sh.I[i]);
      } else {
        const float u = draw_uniform(P, seq_id, (uint32_t)i, 0u);
        const float r = (md == kOnehot) ? p : (q > 0.f ? fminf(1.f, p / q) : 0.f);
        acc = u < r;
      }
      if (P.p_at) P.p_at[off_d + i] = p;
      if (P.q_at) P.q_at[off_d + i] = q;
      reject = !acc;
    }
    const unsigned long long rj = __ballot(reject);
    if (A == K && rj != 0ull) A = i0 + (int)__builtin_ctzll(rj);
  }

  // ---- emitted tokens: accepted prefix, -1 after A; greedy fills A too ----
  for (int j = lane; j <= K; j += kScanThreads) {
    if (j < A) P.emitted[off_t + j] = sh.tok[j];
    else if (j > A) P.emitted[off_t + j] = -1;
    else if (md == kGreedy) P.emitted[off_t + j] = sh.I[A];
  }
  if (lane == 0) {
    P.accepted_len[s] = A;
    if (md == kGreedy && P.status) P.status[s] = 0;
  }
  f.A = A;
  f.emit_pos = off_t + A;
  f.c = c;
  if (md != kGreedy) {
    f.trow = off_t + A;
    f.mct = sh.M[A] * c;
    f.inv_st = 1.f / sh.S[A];
    f.u = draw_uniform(P, seq_id, (uint32_t)A, 1u);
    if (A == K) {
      f.kind = kFinalBonus;
    } else if (md == kOnehot) {
      f.kind = kFinalOnehot;
      f.xhat = sh.tok[A];
    } else {
      f.kind = kFinalResidual;
      f.drow = off_d + A;
      f.mcd = sh.M[K + 1 + A] * c;
      f.inv_sd = 1.f / sh.S[K + 1 + A];
    }
  }
  return f;
}

// One wave per sequence: the acceptance scan; records the final draw.
__global__ void __launch_bounds__(kScanThreads) k_scan(Params P) {
  __shared__ ScanShared sh;
  const int s = blockIdx.x;
  const SeqFinal f = scan_sequence(P, s, sh);
  if (threadIdx.x == 0) P.fin[s] = f;
}

// grid (ntiles, B): the final weights of one tile of the row(s) at the stop
// position of sequence s.
__global__ void __launch_bounds__(kThreads) k_tile_sums(Params P) {
  __shared__ float s_w[kWaves];
  const int j = blockIdx.x, s = blockIdx.y;
  const SeqFinal f = P.fin[s];
  if (f.kind == kFinalDone) return;
  const float tot = block_sum(tile_part(P, f, f.kind, j), s_w);
  if (threadIdx.x == 0) P.tilesum[(int64_t)s * P.ntiles + j] = tot;
}

struct SelShared {
  float lw[kTileLds];          // the chosen tile's weights, element order (padded)
  float w[kWaves];
  float tiles[kMaxTiles];
  float tp;
  int jj, fallback, first, last;
};

// The residual had no mass (rounding only): the token is drawn from p at
// position A instead.  Recomputes every tile's sum of p and picks the tile.
__device__ __forceinline__ void select_fallback(const Params& P, const SeqFinal& f, SelShared& sh) {
  const int t = threadIdx.x;
  for (int q = 0; q < P.ntiles; ++q) {
    const float v = block_sum(tile_part(P, f, kFinalBonus, q), sh.w);
    if (t == 0) sh.tiles[q] = v;
  }
  __syncthreads();
  if (t == 0) {
    float Z = 0.f;
    for (int q = 0; q < P.ntiles; ++q) Z += sh.tiles[q];
    const float tt = f.u * Z;
    float cum = 0.f;
    int jj = -1;
    for (int q = 0; q < P.ntiles; ++q) {
      if (cum + sh.tiles[q] > tt) {
        jj = q;
        break;
      }
      cum += sh.tiles[q];
    }
    if (jj < 0) {
      for (int q = P.ntiles - 1; q >= 0; --q) {
        if (sh.tiles[q] > 0.f) {
          jj = q;
          break;
        }
      }
      cum = 0.f;
      for (int q = 0; q < jj; ++q) cum += sh.tiles[q];
    }
    sh.jj = jj;
    sh.tp = tt - cum;
  }
  __syncthreads();
}

// One block per sequence: the tile holding t = u * Z, then the token in it.
// Two dependent rounds of loads: the record and the tile sums together, then
// the chosen tile.
__global__ void __launch_bounds__(kThreads) k_select(Params P) {
  __shared__ SelShared sh;
  constexpr int kTPL = kMaxTiles / kWave;      // tile sums per lane of wave 0
  const int s = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1), wv = t / kWave;
  const SeqFinal f = P.fin[s];
  float tv[kTPL];
  if (wv == 0) {
#pragma unroll
    for (int k = 0; k < kTPL; ++k) {
      const int j = lane + k * kWave;
      tv[k] = (j < P.ntiles) ? P.tilesum[(int64_t)s * P.ntiles + j] : 0.f;
    }
  }
  if (f.kind == kFinalDone) return;
  if (wv == 0) {
    // prefix sums over tiles (lane-major within each group of 64), total Z
    float pre[kTPL];
    float carry = 0.f;
#pragma unroll
    for (int k = 0; k < kTPL; ++k) {
      float v = tv[k];
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
      }
      pre[k] = carry + v;
      carry += __shfl(v, kWave - 1, kWave);
    }
    const float Z = carry;
    const float tt = f.u * Z;
    // first tile whose inclusive prefix exceeds tt; else the last tile with mass
    int jj = -1, jlast = -1;
#pragma unroll
    for (int k = kTPL - 1; k >= 0; --k) {
      const unsigned long long hit = __ballot(pre[k] > tt && lane + k * kWave < P.ntiles);
      if (hit) jj = k * kWave + (int)__builtin_ctzll(hit);
      const unsigned long long pos = __ballot(tv[k] > 0.f);
      if (pos && jlast < 0) jlast = k * kWave + 63 - (int)__builtin_clzll(pos);
    }
    if (jj < 0) jj = jlast;
    // exclusive prefix of tile jj
    float before = 0.f;
#pragma unroll
    for (int k = 0; k < kTPL; ++k) {
      const float ex = pre[k] - tv[k];
      const float b = __shfl(ex, (jj < 0 ? 0 : jj) & (kWave - 1), kWave);
      if (jj >= 0 && jj / kWave == k) before = b;
    }
    if (lane == 0) {
      sh.fallback = !(Z > 0.f);
      sh.jj = jj;
      sh.tp = tt - before;
      sh.first = 0x7FFFFFFF;
      sh.last = -1;
    }
  }
  __syncthreads();
  const bool fallback = sh.fallback;
  int kind = f.kind;
  if (fallback) {
    kind = kFinalBonus;
    select_fallback(P, f, sh);
  }
  const int jj = sh.jj;
  const float tp = sh.tp;

  // re-read tile jj with coalesced loads into LDS; then thread t takes the
  // kTileVec consecutive weights starting at element t * kTileVec
  tile_weights_lds(P, f, kind, jj, sh.lw);
  __syncthreads();
  const int e0 = jj * kTileElems + t * kTileVec;
  float xv[kTileVec];
#pragma unroll
  for (int q = 0; q < kTileVec; ++q) xv[q] = sh.lw[lds_pad(t * kTileVec + q)];
  float loc = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int q = 0; q < kTileVec; ++q) {
    if (xv[q] > 0.f) last_pos = e0 + q;
    loc += xv[q];
  }
  float total;
  const float before = block_excl_scan(loc, sh.w, &total);
  // the first element (with weight) whose running prefix passes tp
  // (fully unrolled: constant register indices)
  int found = -1;
  float run = before;
#pragma unroll
  for (int q = 0; q < kTileVec; ++q) {
    run += xv[q];
    if (found < 0 && xv[q] > 0.f && run > tp) found = q;
  }
  if (found >= 0) atomicMin(&sh.first, e0 + found);   // LDS: the lowest crossing over threads wins
  if (last_pos >= 0) atomicMax(&sh.last, last_pos);
  __syncthreads();
  if (t == 0) {
    const int y = (sh.first != 0x7FFFFFFF) ? sh.first : sh.last;
    P.emitted[f.emit_pos] = y;
    if (P.status) P.status[s] = fallback ? kStZeroResidual : 0;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_row_stats(const Params& p, hipStream_t st) {
  const int64_t blocks = (int64_t)p.n_t * p.nch_t + (int64_t)p.n_d * p.nch_d;
  if (blocks <= 0) return hipSuccess;
  const dim3 g((unsigned)blocks), b(kThreads);
  if (p.t_bf16) {
    if (p.d_bf16) hipLaunchKernelGGL((k_row_stats<true, true>), g, b, 0, st, p);
    else hipLaunchKernelGGL((k_row_stats<true, false>), g, b, 0, st, p);
  } else {
    if (p.d_bf16) hipLaunchKernelGGL((k_row_stats<false, true>), g, b, 0, st, p);
    else hipLaunchKernelGGL((k_row_stats<false, false>), g, b, 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_scan(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL(k_scan, dim3(p.B), dim3(kScanThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_tile_sums(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL(k_tile_sums, dim3(p.ntiles, p.B), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_select(const Params& p, hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(p.B), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
