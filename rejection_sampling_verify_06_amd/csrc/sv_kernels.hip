// Kernels of the batched speculative-decoding verify step for gfx950.
//
// row_stats   one block per (logit row, 32 KB chunk).  The block issues its
//             chunk's 16-byte non-temporal loads first; wave 0 finds the
//             sequence that owns the row (a wave-level scan of num_draft,
//             served from cache while the chunk is in flight).  The chunk is
//             reduced in float32 to (max of the raw logits, sum of
//             exp2(x*c - round(max*c)), lowest-index argmax for greedy rows):
//             block max first, then one sum against it.  No inter-block
//             communication.  In a filtered call every block also writes
//             its chunk's 32 segment maxima (one per 8-lane group: the bound
//             of the filter's bounded selection), and one more block (the
//             first) orders the sequences by temperature and writes the list
//             of the rows the filter kernel takes, in that order.
// final       grid (nsplit, B) of 1024-thread blocks.  Wave 0 runs the
//             acceptance scan of its sequence: validates it, merges each
//             row's chunk partials in chunk order (lane r: row r), computes
//             p and q at the proposals, draws the Philox uniforms and runs
//             the left-to-right test (lane i: position i, the stop position
//             from a ballot); split 0 writes everything but the final token.
//             The block then sums the final weights over 8192-element tiles
//             of the row(s) at the stop position.  With one block per
//             sequence (batches of 128 and more) the same block picks the
//             tile holding t = u * Z, re-reads it and emits the first token
//             whose inclusive prefix exceeds t.
//             Smaller batches spread a sequence's tiles over several
//             blocks; each stores its tile sums with device-coherent stores
//             and counts itself in, and the one that arrives last reads them
//             back and runs the same search.
//
// The method (accept with probability min(1, p/q), stop at the first
// rejection, redraw from norm(max(0, p - q)) or take a bonus token from the
// next target distribution) follows "Draft Model（草稿模型）"
// (compassingai.com) section 2 and its one-step algorithm box; the one-hot
// proposal follows "5.2 Draft 模型与无模型方案" (AIInfraGuide) section 4.3;
// temperature on both rows follows the gitcode.csdn.net tutorial section 4.3.
// The path is a memory-bound streaming reduction: no matrix cores are used.
// Blocks never wait on one another and there are no device-scope fences (each
// one writes back a whole L2 on this chip) and no spin loops: row statistics
// reach the final kernel across a kernel boundary, and the split final draw
// hands its tile sums to its last-arriving block through device-coherent
// stores and loads and one counter per sequence.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"
#include "sv_wave.h"

namespace sv {

namespace {

using namespace wave;   // kWave and the DPP reductions and scans (sv_wave.h)
static_assert(kSegPerChunk * 8 == kThreads, "one segment maximum per 8-lane group of a row-stats block");

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = kThreads / kWave;
constexpr int kNV = 8;   // 16-byte vectors per thread per 32 KB chunk
constexpr int kSample = 0, kGreedy = 1, kOnehot = 2, kStrict = 3;
constexpr int64_t kMaxGridX = 65535;   // blocks per grid dimension of the row-statistics launch
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
  o.s = __builtin_amdgcn_readlane(owner, src);
  o.T = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(T), src));
  o.md = __builtin_amdgcn_readlane(md, src);
  o.first = __builtin_amdgcn_readlane(first, src);
  o.K = __builtin_amdgcn_readlane(K, src);
  return o;
}

// 32-bit unsigned arithmetic (wraps instead of overflowing on a corrupt
// num_draft; a consistent layout has fewer than 2^31 rows).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)dpp_i<kDppRowShr1>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowShr2>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowShr4>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowShr8>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowBcast15, 0xA>(0, (int)v);
  v += (uint32_t)dpp_i<kDppRowBcast31, 0xC>(0, (int)v);
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
// the final draw at the stop position A.  The row(s) at A are cut into tiles
// of 8192 elements; a 1024-thread block holds 8 elements of a tile per thread.
// ---------------------------------------------------------------------------
constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / kWave;
constexpr int kPerThread = kTileElems / kFinThreads;   // 8
// Tiles whose loads a block keeps in flight together: with a block per
// sequence on every CU, two tiles of the two residual rows (64 KB per block
// in bf16) stream fastest; a draw that reads one row keeps more tiles in
// flight, since fewer blocks have work then.
template <bool BF, int KIND>
constexpr int tile_unroll() { return KIND == kFinalResidual ? 2 : (BF ? 8 : 4); }

// Final weights up to one positive factor per sequence (the inverse CDF is
// scale-free): with e_x = exp2(x c - round(M_t c)) = S_t p(x), a residual
// weight is max(0, e_x - (S_t/S_d) e_y) = S_t max(0, p - q), formed with a
// single rounding; bonus and one-hot weights are e_x = S_t p.
__device__ __forceinline__ float final_weight(int kind, float x, float y, int k, const SeqFinal& f) {
  // tokens below a row's filter threshold weigh 0 (the threshold is -inf without a filter)
  const float ex = (x >= f.taut) ? fexp2(fmaf(x, f.c, -f.mct)) : 0.f;
  if (kind == kFinalResidual) {
    const float ey = (y >= f.taud) ? fexp2(fmaf(y, f.c, -f.mcd)) : 0.f;
    return fmaxf(fmaf(-f.rq, ey, ex), 0.f);
  }
  if (kind == kFinalOnehot && k == f.xhat) return 0.f;
  return ex;
}

struct FinShared {
  float tw[kMaxTiles][kFinWaves];   // each wave's share of each tile's sum
  float tile[kMaxTiles];            // tile sums
  float sw[kFinWaves];
  int first[kFinWaves];
  int last[kFinWaves];
  float tp;                         // remainder of u * Z inside tile jj
  int jj;
  int fallback;
  int arrived_last;                 // a split draw: this block arrived last and draws the token
};

// The final weights of the VEC elements e.. of one 16-byte vector (target
// words vt, draft words vd).
template <bool BF, int KIND>
__device__ __forceinline__ void vec_weights(const u32x4& vt, const u32x4& vd, int e, const SeqFinal& f,
                                            float (&w)[BF ? 8 : 4]) {
  constexpr int VEC = BF ? 8 : 4;
#pragma unroll
  for (int q = 0; q < VEC; ++q) {
    float x, y = 0.f;
    if (BF) {
      x = (q & 1) ? bf_hi(vt[q >> 1]) : bf_lo(vt[q >> 1]);
      if (KIND == kFinalResidual) y = (q & 1) ? bf_hi(vd[q >> 1]) : bf_lo(vd[q >> 1]);
    } else {
      x = __uint_as_float(vt[q]);
      if (KIND == kFinalResidual) y = __uint_as_float(vd[q]);
    }
    w[q] = final_weight(KIND, x, y, e + q, f);
  }
}

// The vector of elements e..e+VEC of a 16-byte aligned row: entries at or
// past V read as -inf (weight 0); a vector that straddles V is assembled
// from element loads, one wholly past V is not loaded at all.
template <bool BF>
__device__ __forceinline__ u32x4 load_vec_masked(const char* rowp, int e, int V) {
  constexpr int VEC = BF ? 8 : 4;
  constexpr int ES = BF ? 2 : 4;
  if (e + VEC <= V) return __builtin_nontemporal_load((const u32x4*)(rowp + (int64_t)e * ES));
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (BF) {
      const int e0 = e + 2 * q, e1 = e0 + 1;
      const uint32_t lo = (e0 < V) ? (uint32_t)((const uint16_t*)rowp)[e0] : 0xFF80u;
      const uint32_t hi = (e1 < V) ? (uint32_t)((const uint16_t*)rowp)[e1] : 0xFF80u;
      w[q] = lo | (hi << 16);
    } else {
      const int e0 = e + q;
      w[q] = (e0 < V) ? ((const uint32_t*)rowp)[e0] : 0xFF800000u;
    }
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Sums of the full tiles jb, jb+step, ... (< nfull) into sh.tw.  Thread t
// owns vectors (n*1024 + t), n < NV, of a tile (coalesced); the loads of
// kTileUnroll tiles are issued before any is used (indices clamped to the
// last full tile for the loads, surplus tiles skipped after).
template <bool BF, int KIND>
__device__ __forceinline__ void tiles_full_vec(const Params& P, const SeqFinal& f, int j0, int step, int nfull,
                                               FinShared& sh) {
  constexpr int kTileUnroll = tile_unroll<BF, KIND>();
  constexpr int VEC = BF ? 8 : 4;
  constexpr int NV = kPerThread / VEC;
  constexpr int ES = BF ? 2 : 4;
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const char* tp = (const char*)P.tgt + (int64_t)f.trow * P.ld_t * ES;
  const char* dp = (KIND == kFinalResidual) ? (const char*)P.dft + (int64_t)f.drow * P.ld_d * ES : tp;
  for (int jb = j0; jb < nfull; jb += kTileUnroll * step) {
    u32x4 vt[kTileUnroll][NV], vd[kTileUnroll][NV];
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) {
      const int j = min(jb + u * step, nfull - 1);
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        const int64_t e = (int64_t)j * kTileElems + (n * kFinThreads + t) * VEC;
        // plain loads: the tile the search re-reads may still be cached
        vt[u][n] = *((const u32x4*)(tp + e * ES));
        if (KIND == kFinalResidual) vd[u][n] = *((const u32x4*)(dp + e * ES));
      }
    }
#pragma unroll
    for (int u = 0; u < kTileUnroll; ++u) {
      const int j = jb + u * step;
      if (j < nfull) {
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < NV; ++n) {
          float w[VEC];
          vec_weights<BF, KIND>(vt[u][n], vd[u][n], j * kTileElems + (n * kFinThreads + t) * VEC, f, w);
#pragma unroll
          for (int q = 0; q < VEC; ++q) acc += w[q];
        }
        acc = wave_sum(acc);
        if (lane == 0) sh.tw[j][wv] = acc;
      }
    }
  }
}

// The row's last tile when it is not full (element layout as above).
template <bool BF, int KIND>
__device__ __forceinline__ void tile_tail_vec(const Params& P, const SeqFinal& f, int j, FinShared& sh) {
  constexpr int VEC = BF ? 8 : 4;
  constexpr int NV = kPerThread / VEC;
  constexpr int ES = BF ? 2 : 4;
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const char* tp = (const char*)P.tgt + (int64_t)f.trow * P.ld_t * ES;
  const char* dp = (KIND == kFinalResidual) ? (const char*)P.dft + (int64_t)f.drow * P.ld_d * ES : tp;
  float acc = 0.f;
#pragma unroll
  for (int n = 0; n < NV; ++n) {
    const int e = j * kTileElems + (n * kFinThreads + t) * VEC;
    if (e < P.V) {
      const u32x4 vt = load_vec_masked<BF>(tp, e, P.V);
      const u32x4 vd = (KIND == kFinalResidual) ? load_vec_masked<BF>(dp, e, P.V) : vt;
      float w[VEC];
      vec_weights<BF, KIND>(vt, vd, e, f, w);
#pragma unroll
      for (int q = 0; q < VEC; ++q) acc += w[q];
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) sh.tw[j][wv] = acc;
}

// Rows that are not 16-byte aligned, shorter than a vector, or a residual
// whose two rows differ in type: element loads clamped to V - 1, weights
// past V zeroed.  Thread t takes elements j*8192 + q*1024 + t.
__device__ __forceinline__ void tile_generic(const Params& P, const SeqFinal& f, int kind, int j, FinShared& sh) {
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int64_t toff = (int64_t)f.trow * P.ld_t, doff = (int64_t)f.drow * P.ld_d;
  float x[kPerThread], y[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = min(j * kTileElems + q * kFinThreads + t, P.V - 1);
    x[q] = load_logit(P.tgt, toff + e, P.t_bf16);
    y[q] = (kind == kFinalResidual) ? load_logit(P.dft, doff + e, P.d_bf16) : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int e = j * kTileElems + q * kFinThreads + t;
    acc += (e < P.V) ? final_weight(kind, x[q], y[q], e, f) : 0.f;
  }
  acc = wave_sum(acc);
  if (lane == 0) sh.tw[j][wv] = acc;
}

__device__ __forceinline__ bool final_vec_ok(const Params& P, int kind) {
  const int vecmin = P.t_bf16 ? 8 : 4;
  return P.t_vec && P.V >= vecmin && (kind != kFinalResidual || (P.d_vec && P.d_bf16 == P.t_bf16));
}

template <bool BF, int KIND>
__device__ __forceinline__ void tiles_vec(const Params& P, const SeqFinal& f, int j0, int step, FinShared& sh) {
  const int nfull = P.V / kTileElems;
  tiles_full_vec<BF, KIND>(P, f, j0, step, nfull, sh);
  const int jt = P.ntiles - 1;
  if (jt >= nfull && jt >= j0 && (jt - j0) % step == 0) tile_tail_vec<BF, KIND>(P, f, jt, sh);
}

// Per-wave sums of tiles j0, j0+step, ... of the final weights into sh.tw.
__device__ __forceinline__ void tile_sums_pass(const Params& P, const SeqFinal& f, int kind, int j0, int step,
                                               FinShared& sh) {
  if (final_vec_ok(P, kind)) {
    if (P.t_bf16) {
      if (kind == kFinalResidual) tiles_vec<true, kFinalResidual>(P, f, j0, step, sh);
      else if (kind == kFinalOnehot) tiles_vec<true, kFinalOnehot>(P, f, j0, step, sh);
      else tiles_vec<true, kFinalBonus>(P, f, j0, step, sh);
    } else {
      if (kind == kFinalResidual) tiles_vec<false, kFinalResidual>(P, f, j0, step, sh);
      else if (kind == kFinalOnehot) tiles_vec<false, kFinalOnehot>(P, f, j0, step, sh);
      else tiles_vec<false, kFinalBonus>(P, f, j0, step, sh);
    }
  } else {
    for (int j = j0; j < P.ntiles; j += step) tile_generic(P, f, kind, j, sh);
  }
}

// Tile sums from the per-wave shares (fixed order); thread j adds up tile j.
__device__ __forceinline__ float tile_total(const FinShared& sh, int j) {
  float z = 0.f;
#pragma unroll
  for (int w = 0; w < kFinWaves; ++w) z += sh.tw[j][w];
  return z;
}

// Weights of the PT consecutive elements base + t*PT .. +PT-1 (thread t).
template <bool BF, int KIND, int PT>
__device__ __forceinline__ void slice_vec(const Params& P, const SeqFinal& f, int base, float (&w)[PT]) {
  constexpr int VEC = BF ? 8 : 4;
  constexpr int NV = PT / VEC;
  constexpr int ES = BF ? 2 : 4;
  const char* tp = (const char*)P.tgt + (int64_t)f.trow * P.ld_t * ES;
  const char* dp = (KIND == kFinalResidual) ? (const char*)P.dft + (int64_t)f.drow * P.ld_d * ES : tp;
  const int e0 = base + (int)threadIdx.x * PT;
#pragma unroll
  for (int n = 0; n < NV; ++n) {
    const int e = e0 + n * VEC;
    float wv[VEC];
    if (e < P.V) {
      const u32x4 vt = load_vec_masked<BF>(tp, e, P.V);
      const u32x4 vd = (KIND == kFinalResidual) ? load_vec_masked<BF>(dp, e, P.V) : vt;
      vec_weights<BF, KIND>(vt, vd, e, f, wv);
    } else {
#pragma unroll
      for (int q = 0; q < VEC; ++q) wv[q] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < VEC; ++q) w[n * VEC + q] = wv[q];
  }
}

template <int PT>
__device__ __forceinline__ void slice_generic(const Params& P, const SeqFinal& f, int kind, int base,
                                              float (&w)[PT]) {
  const int64_t toff = (int64_t)f.trow * P.ld_t, doff = (int64_t)f.drow * P.ld_d;
  const int e0 = base + (int)threadIdx.x * PT;
  float x[PT], y[PT];
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    const int e = min(e0 + q, P.V - 1);
    x[q] = load_logit(P.tgt, toff + e, P.t_bf16);
    y[q] = (kind == kFinalResidual) ? load_logit(P.dft, doff + e, P.d_bf16) : 0.f;
  }
#pragma unroll
  for (int q = 0; q < PT; ++q) w[q] = (e0 + q < P.V) ? final_weight(kind, x[q], y[q], e0 + q, f) : 0.f;
}

template <int PT>
__device__ __forceinline__ void slice_weights(const Params& P, const SeqFinal& f, int kind, int base,
                                              float (&w)[PT]) {
  if (final_vec_ok(P, kind)) {
    if (P.t_bf16) {
      if (kind == kFinalResidual) slice_vec<true, kFinalResidual, PT>(P, f, base, w);
      else if (kind == kFinalOnehot) slice_vec<true, kFinalOnehot, PT>(P, f, base, w);
      else slice_vec<true, kFinalBonus, PT>(P, f, base, w);
    } else {
      if (kind == kFinalResidual) slice_vec<false, kFinalResidual, PT>(P, f, base, w);
      else if (kind == kFinalOnehot) slice_vec<false, kFinalOnehot, PT>(P, f, base, w);
      else slice_vec<false, kFinalBonus, PT>(P, f, base, w);
    }
  } else {
    slice_generic<PT>(P, f, kind, base, w);
  }
}

// Wave 0: prefix sums over the n unit sums in sh.tile (lane-major within each
// group of 64), total Z, the first unit whose inclusive prefix exceeds
// tt = u * Z (else the last unit with mass), and the remainder tp of tt in it.
__device__ __forceinline__ void pick_unit(const SeqFinal& f, int n, FinShared& sh) {
  constexpr int kTPL = kMaxTiles / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  float tv[kTPL], pre[kTPL];
  float carry = 0.f;
#pragma unroll
  for (int k = 0; k < kTPL; ++k) {
    const int j = lane + k * kWave;
    tv[k] = (j < n) ? sh.tile[j] : 0.f;
    const float v = wave_incl_scan_f(tv[k]);
    pre[k] = carry + v;
    carry += lane63_f(v);
  }
  const float Z = carry;
  const float tt = f.u * Z;
  int jj = -1, jlast = -1;
#pragma unroll
  for (int k = kTPL - 1; k >= 0; --k) {
    const unsigned long long hit = __ballot(pre[k] > tt && lane + k * kWave < n);
    if (hit) jj = k * kWave + (int)__builtin_ctzll(hit);
    const unsigned long long pos = __ballot(tv[k] > 0.f);
    if (pos && jlast < 0) jlast = k * kWave + 63 - (int)__builtin_clzll(pos);
  }
  if (jj < 0) jj = jlast;
  jj = min(max(jj, 0), n - 1);
  float before = 0.f;
#pragma unroll
  for (int k = 0; k < kTPL; ++k) {
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pre[k] - tv[k]), jj & (kWave - 1)));
    if (jj / kWave == k) before = b;
  }
  if (lane == 0) {
    sh.fallback = !(Z > 0.f);
    sh.jj = jj;
    sh.tp = tt - before;
  }
}

// The token of the final draw inside unit jj (elements jj*span .. +span-1,
// span = 1024*PT): thread t re-reads its PT consecutive weights, a
// block-wide exclusive prefix over the threads' sums locates the first
// element (with weight) whose running prefix passes tp; ballots pick the
// lowest such thread, and, failing one (rounding), the last element with
// weight.  Writes the token and the sequence's status.
template <int PT>
__device__ __forceinline__ void select_token(const Params& P, const SeqFinal& f, int kind, bool fallback,
                                             FinShared& sh) {
  const int t = threadIdx.x, wv = t / kWave, lane = t & (kWave - 1);
  const int jj = sh.jj;
  const float tp = sh.tp;
  const int base = jj * (kFinThreads * PT);
  float w[PT];
  slice_weights<PT>(P, f, kind, base, w);
  float loc = 0.f;
#pragma unroll
  for (int q = 0; q < PT; ++q) loc += w[q];
  const float inc = wave_incl_scan_f(loc);
  if (lane == kWave - 1) sh.sw[wv] = inc;
  __syncthreads();
  float run = inc - loc;
  for (int q = 0; q < wv; ++q) run += sh.sw[q];
  int found = -1, lastp = -1;
#pragma unroll
  for (int q = 0; q < PT; ++q) {
    run += w[q];
    if (found < 0 && w[q] > 0.f && run > tp) found = q;
    if (w[q] > 0.f) lastp = q;
  }
  const unsigned long long fm = __ballot(found >= 0);
  const unsigned long long lm = __ballot(lastp >= 0);
  const int fl = fm ? (int)__builtin_ctzll(fm) : 0;
  const int ll = lm ? 63 - (int)__builtin_clzll(lm) : 0;
  const int ff = __builtin_amdgcn_readlane(found, fl);
  const int lq = __builtin_amdgcn_readlane(lastp, ll);
  const int wbase = base + wv * kWave * PT;
  if (lane == 0) {
    sh.first[wv] = fm ? wbase + fl * PT + ff : 0x7FFFFFFF;
    sh.last[wv] = lm ? wbase + ll * PT + lq : -1;
  }
  __syncthreads();
  if (t == 0) {
    int y = 0x7FFFFFFF, z = -1;
#pragma unroll
    for (int q = 0; q < kFinWaves; ++q) {
      y = min(y, sh.first[q]);
      z = max(z, sh.last[q]);
    }
    P.emitted[f.emit_pos] = (y != 0x7FFFFFFF) ? y : z;
    if (P.status) P.status[f.s] = fallback ? kStZeroResidual : 0;
  }
}

// Residual draws, given the tile sums in sh.tile: the tile, then the token.
// A residual with no mass (rounding only) falls back to p at the stop
// position: the block recomputes every tile sum of p and picks again.
__device__ __forceinline__ void finish_draw(const Params& P, const SeqFinal& f, FinShared& sh) {
  const int t = threadIdx.x;
  if (t < kWave) pick_unit(f, P.ntiles, sh);
  __syncthreads();
  const bool fallback = sh.fallback;
  int kind = f.kind;
  if (fallback) {
    kind = kFinalBonus;
    tile_sums_pass(P, f, kind, 0, 1, sh);
    __syncthreads();
    if (t < P.ntiles) sh.tile[t] = tile_total(sh, t);
    __syncthreads();
    if (t < kWave) pick_unit(f, P.ntiles, sh);
    __syncthreads();
  }
  select_token<kPerThread>(P, f, kind, fallback, sh);
}

// Bonus and one-hot draws read one row, whose chunk sums of the weights e_x
// (S p, the scale the token search uses) follow from row_stats' partials:
// chunk k holds s_k * exp2(round(m_k c) - round(M c)) (s_k is relative to
// round(m_k c)); a one-hot draw takes e_x of the proposed token out of its
// chunk.  So the chunk holding t = u * Z is found without
// reading the row, and only that chunk (32 KB) is re-read.  Wave 0 fills
// sh.tile with the chunk sums of `kind` and picks.
__device__ __forceinline__ void pick_chunk(const Params& P, const SeqFinal& f, int kind, FinShared& sh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t sb = (int64_t)f.s * P.slots + f.A;     // target slot A
  const Partial* pp = P.partials + sb * P.nch_max;
  const bool onehot = kind == kFinalOnehot;
  const int xchunk = onehot ? f.xhat / P.ce_t : -1;
  const float xv = onehot ? P.xval[sb] : 0.f;
  const float px = (onehot && xv >= f.taut) ? fexp2(fmaf(xv, f.c, -f.mct)) : 0.f;
  for (int k = lane; k < P.nch_t; k += kWave) {
    const Partial q = pp[k];
    float z = (q.m == -INFINITY) ? 0.f : q.s * fexp2(q.m * f.c - f.mct);
    if (k == xchunk) z = fmaxf(z - px, 0.f);
    sh.tile[k] = z;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  pick_unit(f, P.nch_t, sh);
}

__device__ __forceinline__ void finish_draw_chunks(const Params& P, const SeqFinal& f, FinShared& sh) {
  const int t = threadIdx.x;
  if (t < kWave) pick_chunk(P, f, f.kind, sh);
  __syncthreads();
  const bool fallback = sh.fallback;
  int kind = f.kind;
  if (fallback) {           // one-hot residual with no mass: p itself
    kind = kFinalBonus;
    if (t < kWave) pick_chunk(P, f, kind, sh);
    __syncthreads();
  }
  // a 32 KB chunk is 16384 bf16 or 8192 float32 logits
  if (P.t_bf16) select_token<kChunkBytes / 2 / kFinThreads>(P, f, kind, fallback, sh);
  else select_token<kChunkBytes / 4 / kFinThreads>(P, f, kind, fallback, sh);
}


// clear the outputs of a sequence that is not verified (one wave)
__device__ __forceinline__ void clear_sequence(const Params& P, int s, int off_t, int off_d, int K, int st) {
  const int t = threadIdx.x & (kWave - 1);
  for (int j = t; j <= K; j += kWave) P.emitted[off_t + j] = -1;
  for (int j = t; j < K; j += kWave) {
    if (P.p_at) P.p_at[off_d + j] = __uint_as_float(kNaNBits);
    if (P.q_at) P.q_at[off_d + j] = __uint_as_float(kNaNBits);
  }
  if (t == 0) {
    P.accepted_len[s] = -1;
    if (P.status) P.status[s] = st;
  }
}

// Block-wide merge of the threads' (max, sum, argmax) and the partial write.
// xs >= 0 (a strict-mode target row judging token xs): the partial also
// carries the part of the sum from tokens below xs, summed against the
// chunk's final maximum.
template <bool ARG>
__device__ __forceinline__ void finish_chunk(const Params& P, float m, float sum, int idx, float c, int64_t pidx,
                                             const char* rowp, int bf, int c0, int c1, int xs) {
  __shared__ float s_m[kWaves], s_s[kWaves];
  __shared__ int s_i[kWaves];
  __shared__ float s_M;
  wave_merge<ARG>(m, sum, idx, c);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (lane == 0) {
    s_m[wv] = m;
    s_s[wv] = sum;
    s_i[wv] = idx;
  }
  __syncthreads();
  float M = s_m[0], S = s_s[0];
  int I = s_i[0];
  if (threadIdx.x == 0) {
    for (int q = 1; q < kWaves; ++q) merge_stats<true>(M, S, I, s_m[q], s_s[q], s_i[q], c);
    s_M = M;
  }
  float below = 0.f;
  if (xs >= c0 && xs < c1) {                 // block-uniform: the chunk holds the proposal
    __syncthreads();
    const float Mb = s_M;
    const float mc = (Mb == -INFINITY) ? 0.f : Mb * c;
    float a = 0.f;
    for (int k = c0 + (int)threadIdx.x; k < xs; k += kThreads) a += fexp2(fmaf(load_logit(rowp, k, bf), c, -mc));
    a = wave_sum(a);
    __syncthreads();                          // s_s reused
    if (lane == 0) s_s[wv] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
      below = s_s[0];
      for (int q = 1; q < kWaves; ++q) below += s_s[q];
    }
  }
  if (threadIdx.x == 0) {
    if (xs >= 0 && c1 <= xs) below = S;       // the whole chunk lies below the proposal
    if (pidx >= 0) P.partials[pidx] = Partial{M, S, I, below};
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

// The row's slot among its sequence's 2*max_k + 1: target position i at
// slot i, draft position i at slot max_k + 1 + i; -1 past them (K > max_k,
// which the scan reports).  Chunk k of slot r of sequence s keeps its
// partial at (s*slots + r)*nch_max + k, so the scan finds a sequence's rows
// without knowing its offset in the packed layout.
__device__ __forceinline__ int row_slot_base(const Params& P, const Owner& own, int row, bool is_draft) {
  const int i = row - own.first;
  int slot = -1;
  if (is_draft) {
    if (i >= 0 && i < own.K && i < P.max_k) slot = P.max_k + 1 + i;
  } else {
    if (i >= 0 && i <= own.K && i <= P.max_k) slot = i;
  }
  return slot < 0 ? -1 : own.s * P.slots + slot;    // < 4096 * 257
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

// What wave 0 of a row-statistics block hands to the other waves.
struct StatsShared {
  float m[kWaves];
  float s[kWaves];
  float b[kWaves];
  int i[kWaves];
  Owner own;
  int x;          // token the row judges, or -1
  int sb;         // the row's slot index s*slots + r, or -1
};

// Wave 0: the owner, the row's slot and proposal into LDS; chunk 0 of a
// target row also records the proposal token in the sequence's slot list.
__device__ __forceinline__ void publish_owner(const Params& P, StatsShared& sh, const Owner& own, int row,
                                              bool is_draft, int chunk) {
  const int x = (own.s >= 0) ? row_proposal(P, own, row, is_draft) : -1;
  const int sb = (own.s >= 0) ? row_slot_base(P, own, row, is_draft) : -1;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sh.own = own;
    sh.x = x;
    sh.sb = sb;
    const int i = row - own.first;
    if (chunk == 0 && !is_draft && sb >= 0 && i < own.K && i < P.max_k) P.ptok[(int64_t)own.s * P.max_k + i] = x;
  }
}

// A 16-byte aligned chunk (full, or the row's last when TAIL).  Every wave
// issues its share of the chunk's loads at once; wave 0 alone also looks up
// the owning sequence (its window loads go first, so the lookup overlaps the
// chunk's flight) and publishes it in LDS.  The block first agrees on the
// chunk maximum M, then every thread sums exp2(x*c - round(M*c)) against that
// common reference, so the block's partial is a plain sum (no rescaling).
template <bool BF, bool TAIL>
__device__ __forceinline__ void row_stats_vec(const Params& P, const char* rowp, int row, int chunk, int c0, int c1,
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
      publish_owner(P, sh, owner_in_window(win, P, plus_one, row), row, is_draft, chunk);
    } else {
      load_chunk<BF, TAIL>(rowp, c0, c1, v);
      publish_owner(P, sh, owner_general(P, plus_one, row), row, is_draft, chunk);
    }
  } else {
    load_chunk<BF, TAIL>(rowp, c0, c1, v);
  }
  if (TAIL) mask_chunk<BF>(rowp, c0, c1, v);
  float f[N];
  unpack_chunk<BF>(v, f);
  float tmx = -INFINITY;
#pragma unroll
  for (int k = 0; k < N; ++k) tmx = fmaxf(tmx, f[k]);
  const float rmx = row8_max(tmx);         // the maximum of this thread's 8-lane group
  const float mx = wave_max(rmx);
  if (lane == 0) sh.m[wv] = mx;
  __syncthreads();
  Owner own;                               // block-uniform: scalar registers
  own.s = __builtin_amdgcn_readfirstlane(sh.own.s);
  own.T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sh.own.T)));
  own.md = __builtin_amdgcn_readfirstlane(sh.own.md);
  if (own.s < 0) return;                   // the whole block: inconsistent layout
  if (P.segmax) {                          // filtered calls: the groups' maxima bound the filter
    const int sbs = __builtin_amdgcn_readfirstlane(sh.sb);
    if (sbs >= 0 && (lane & 7) == 0)
      P.segmax[((int64_t)sbs * P.nch_max + chunk) * kSegPerChunk + wv * (kWave / 8) + (lane >> 3)] = rmx;
  }
  const float M = fmaxf(fmaxf(sh.m[0], sh.m[1]), fmaxf(sh.m[2], sh.m[3]));
  const float c = row_scale(own.md, own.T);
  const float mc = (M == -INFINITY) ? 0.f : M * c;
  const int x = __builtin_amdgcn_readfirstlane(sh.x);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int k = 0; k < N; k += 4) {
    a0 += fexp2(fmaf(f[k + 0], c, -mc));
    a1 += fexp2(fmaf(f[k + 1], c, -mc));
    a2 += fexp2(fmaf(f[k + 2], c, -mc));
    a3 += fexp2(fmaf(f[k + 3], c, -mc));
  }
  const float sum = wave_sum((a0 + a1) + (a2 + a3));
  // strict-mode target row whose proposal falls in this chunk (one block per
  // such row): also the part of the sum from tokens below the proposal.  The
  // terms are recomputed against an opaque copy of mc, so the compiler cannot
  // keep the sum's terms alive for this pass (that costs registers in every
  // block).
  const bool split = own.md == kStrict && !is_draft && x >= c0 && x < c1;
  float below = 0.f;
  if (split) {
    float mc2 = mc;
    asm volatile("" : "+v"(mc2));
    const int rel = x - (c0 + t * VEC);     // element k of this thread is below x iff its offset < rel
    float bl = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int off = (k / VEC) * kThreads * VEC + (k % VEC);
      bl += (off < rel) ? fexp2(fmaf(f[k], c, -mc2)) : 0.f;
    }
    below = wave_sum(bl);
  }
  int idx = 0x7FFFFFFF;
  if (own.md == kGreedy && !is_draft) {    // lowest index attaining M
    if (mx == M) {                          // only waves that hold M search
#pragma unroll
      for (int k = N - 1; k >= 0; --k)
        if (f[k] == M) idx = c0 + ((k / VEC) * kThreads + t) * VEC + (k % VEC);
    }
    idx = wave_min_i(idx);
  }
  const int sb = __builtin_amdgcn_readfirstlane(sh.sb);
  if (sb >= 0) record_proposal_logit<BF>(P, f, c0, c1, x, sb);
  if (lane == 0) {
    sh.s[wv] = sum;
    sh.b[wv] = below;
    sh.i[wv] = idx;
  }
  __syncthreads();
  if (t == 0) {
    const float S = (sh.s[0] + sh.s[1]) + (sh.s[2] + sh.s[3]);
    const int I = min(min(sh.i[0], sh.i[1]), min(sh.i[2], sh.i[3]));
    float Bl = 0.f;
    if (split) Bl = (sh.b[0] + sh.b[1]) + (sh.b[2] + sh.b[3]);
    else if (own.md == kStrict && !is_draft && x >= 0 && c1 <= x) Bl = S;   // the whole chunk is below
    if (sb >= 0) P.partials[(int64_t)sb * P.nch_max + chunk] = Partial{M, S, I, Bl};
  }
}

// Rows that are not 16-byte aligned, or shorter than one vector.
__device__ __forceinline__ void row_stats_scalar(const Params& P, const char* rowp, int bf, int row, int chunk, int c0,
                                                 int c1, int plus_one, bool is_draft) {
  const Owner own = owner_general(P, plus_one, row);
  if (own.s < 0) return;
  const int x = row_proposal(P, own, row, is_draft);
  const int sb = row_slot_base(P, own, row, is_draft);
  if (threadIdx.x == 0 && sb >= 0) {
    if (x >= c0 && x < c1) P.xval[sb] = load_logit(rowp, x, bf);
    const int i = row - own.first;
    if (chunk == 0 && !is_draft && i < own.K && i < P.max_k) P.ptok[(int64_t)own.s * P.max_k + i] = x;
  }
  const int64_t pidx = sb < 0 ? -1 : (int64_t)sb * P.nch_max + chunk;
  const float c = row_scale(own.md, own.T);
  const int xs = (own.md == kStrict && !is_draft) ? x : -1;
  float m, sum;
  int idx;
  if (own.md == kGreedy && !is_draft) {
    stats_scalar<true>(rowp, bf, c0, c1, c, m, sum, idx);
    finish_chunk<true>(P, m, sum, idx, c, pidx, rowp, bf, c0, c1, -1);
  } else {
    stats_scalar<false>(rowp, bf, c0, c1, c, m, sum, idx);
    finish_chunk<false>(P, m, sum, idx, c, pidx, rowp, bf, c0, c1, xs);
  }
}

template <bool BF>
__device__ __forceinline__ void row_stats_seg(const Params& P, const char* rowp, int vec, int row, int chunk, int ce,
                                              int plus_one, bool is_draft) {
  constexpr int VEC = BF ? 8 : 4;
  const int c0 = chunk * ce;
  const int c1 = min(P.V, c0 + ce);
  if (vec && P.V >= VEC) {
    if (c0 + ce <= P.V) row_stats_vec<BF, false>(P, rowp, row, chunk, c0, c1, plus_one, is_draft);
    else row_stats_vec<BF, true>(P, rowp, row, chunk, c0, c1, plus_one, is_draft);
  } else {
    row_stats_scalar(P, rowp, BF, row, chunk, c0, c1, plus_one, is_draft);
  }
}

template <bool TB, bool DB>
__device__ __forceinline__ void row_stats_body(const Params& P, int b) {
  const int nblk_t = P.n_t * P.nch_t;
  const bool is_draft = b >= nblk_t;
  const int bb = is_draft ? b - nblk_t : b;
  const int nch = is_draft ? P.nch_d : P.nch_t;
  const int row = bb / nch;
  const int chunk = bb - row * nch;
  if (is_draft) {
    const char* rowp = (const char*)P.dft + (int64_t)row * P.ld_d * (DB ? 2 : 4);
    row_stats_seg<DB>(P, rowp, P.d_vec, row, chunk, P.ce_d, 0, true);
  } else {
    const char* rowp = (const char*)P.tgt + (int64_t)row * P.ld_t * (TB ? 2 : 4);
    row_stats_seg<TB>(P, rowp, P.t_vec, row, chunk, P.ce_t, 1, false);
  }
}

// The filter kernel's sequence order, written by one block of a filtered
// call's row_stats launch: top-p sequences by decreasing temperature first
// (a flatter row has a wider nucleus and takes more passes over the row), so
// that the longest rows start early instead of trailing at the end of the
// filter launch; top-k sequences next, unfiltered and greedy ones last.  A
// counting sort over 64 buckets; the order inside a bucket is whatever the
// atomics give, which changes no output (every row is filtered on its own).
constexpr int kOrderBuckets = 64;

__device__ __forceinline__ int order_bucket(const Params& P, int s) {
  const int md = P.mode[s];
  const float T = P.temperature[s];
  const int topk = P.top_k ? P.top_k[s] : 0;
  const float topp = P.top_p ? P.top_p[s] : 1.f;
  const bool use_k = topk > 0 && topk < P.V, use_p = topp < 1.f;
  if (md == kGreedy || !(use_k || use_p)) return kOrderBuckets - 1;
  if (use_k || !(T > 0.f && T < 1e30f)) return kOrderBuckets - 2;
  return max(0, kOrderBuckets - 3 - (int)fminf(T * 16.f, (float)(kOrderBuckets - 3)));
}

__device__ __forceinline__ void filter_order(const Params& P) {
  __shared__ uint32_t cnt[kOrderBuckets];
  const int t = threadIdx.x;
  if (t < kOrderBuckets) cnt[t] = 0;
  __syncthreads();
  for (int s = t; s < P.B; s += kThreads) atomicAdd(&cnt[order_bucket(P, s)], 1u);
  __syncthreads();
  if (t == 0) {
    uint32_t acc = 0;
    for (int q = 0; q < kOrderBuckets; ++q) {
      const uint32_t n = cnt[q];
      cnt[q] = acc;
      acc += n;
    }
  }
  __syncthreads();
  for (int s = t; s < P.B; s += kThreads) P.order[atomicAdd(&cnt[order_bucket(P, s)], 1u)] = s;
  __syncthreads();
  // The filter's rows in this order, as sequence slots s * slots + r: the
  // rows the filter kernel takes (target rows 0..K, then draft rows of a
  // SAMPLE sequence), none of a sequence it would skip; the count follows the
  // list (n_t + n_d entries at most: a num_draft that does not add up to
  // total_draft, which the scan reports, could ask for more).  Thread t lists
  // the sequences at order positions [i0, i1).
  __shared__ uint32_t part[kThreads];
  auto nrows = [&](int s) __attribute__((always_inline)) {
    const int K = P.num_draft[s];
    const int md = P.mode[s];
    const int topk = P.top_k ? P.top_k[s] : 0;
    const float topp = P.top_p ? P.top_p[s] : 1.f;
    const float T = P.temperature[s];
    if (K < 0 || K > P.max_k || md == kGreedy || !((topk > 0 && topk < P.V) || topp < 1.f) ||
        !(isfinite(T) && T >= kMinTemperature))
      return 0;
    return K + 1 + ((md == kSample && P.dft) ? K : 0);
  };
  const int per = (P.B + kThreads - 1) / kThreads;
  const int i0 = min(t * per, P.B), i1 = min(i0 + per, P.B);
  uint32_t n = 0;
  for (int i = i0; i < i1; ++i) n += (uint32_t)nrows(P.order[i]);
  part[t] = n;
  __syncthreads();
  if (t == 0) {
    uint32_t acc = 0;
    for (int q = 0; q < kThreads; ++q) {
      const uint32_t m = part[q];
      part[q] = acc;
      acc += m;
    }
    const uint32_t cap = (uint32_t)(P.n_t + P.n_d);
    P.flist[cap] = (int32_t)(acc < cap ? acc : cap);
  }
  __syncthreads();
  uint32_t at = part[t];
  for (int i = i0; i < i1; ++i) {
    const int s = P.order[i];
    const int k = nrows(s), K = P.num_draft[s];
    for (int j = 0; j < k; ++j)
      if (at + (uint32_t)j < (uint32_t)(P.n_t + P.n_d))
        P.flist[at + j] = s * P.slots + (j <= K ? j : P.max_k + 1 + (j - K - 1));
    at += (uint32_t)k;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// One block per (row, 32 KB chunk), numbered row-major; a grid of more than
// 65535 blocks is laid out in several rows of the y dimension (dispatch order
// is still the block number), and the few blocks past the end return at once.
template <bool TB, bool DB>
__global__ void __launch_bounds__(kThreads) k_row_stats(Params P) {
  const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t nblocks = (int64_t)P.n_t * P.nch_t + (int64_t)P.n_d * P.nch_d + P.order_block;
  if (lin >= nblocks) return;
  if (lin == 0 && P.nsplit > 1) {   // the split final blocks' arrival counters start at zero
    for (int i = threadIdx.x; i < P.B; i += kThreads) P.fincnt[i] = 0u;
  }
  int b = (int)lin;
  if (P.order_block) {            // a filtered call: block 0 lists the filter's rows
    if (b == 0) {
      filter_order(P);
      return;
    }
    --b;
  }
  row_stats_body<TB, DB>(P, b);
}

// ---------------------------------------------------------------------------
// acceptance scan: one 64-lane wave per sequence, so no barriers.  Lane r
// merges the chunk partials of row r on its own; lane i judges position i.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = kWave;
constexpr int kMergeUnroll = 8;       // chunk partials a lane has in flight at once

struct ScanShared {
  float M[2 * kMaxK + 1];   // per slot: target positions 0..K at 0..K, draft position i at max_k + 1 + i
  float S[2 * kMaxK + 1];
  float Bl[kMaxK + 1];      // target slots, strict mode: the part of S below the proposal
  int I[2 * kMaxK + 1];
  float X[2 * kMaxK + 1];   // the slot's logit at its proposal
  float Tau[2 * kMaxK + 1]; // the slot's filter threshold (-inf: no filter)
  int tok[kMaxK];
};

// Inconsistent num_draft: every output slot is cleared; the scanning wave of
// sequence s clears its share.
__device__ __forceinline__ void clear_bad_layout(const Params& P, int s) {
  const int t = threadIdx.x & (kWave - 1), nt = kWave;
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

// Row statistics from a group of chunk partials folded into a running
// (M, S, I, B): M = max of the chunk maxima, S = sum of
// s_k * exp2(round(m_k*c) - round(M*c)), I = lowest index attaining M, B the
// same sum over the chunks' below-proposal parts b_k.  Entries k >= n are
// ignored.
__device__ __forceinline__ void merge_group(const Partial (&q)[kMergeUnroll], int n, float c, float& M, float& S,
                                            int& I, float& B) {
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMergeUnroll; ++k)
    if (k < n) m = fmaxf(m, q[k].m);
  const float mn = fmaxf(M, m);
  const float mnc = (mn == -INFINITY) ? 0.f : mn * c;
  const float r0 = (M == -INFINITY) ? 1.f : fexp2(M * c - mnc);
  float sum = (M == -INFINITY) ? S : S * r0;
  float bsum = (M == -INFINITY) ? B : B * r0;
  int idx = (M == mn) ? I : 0x7FFFFFFF;
#pragma unroll
  for (int k = 0; k < kMergeUnroll; ++k) {
    if (k < n) {
      const float r = (q[k].m == -INFINITY) ? 1.f : fexp2(q[k].m * c - mnc);
      sum += (q[k].m == -INFINITY) ? q[k].s : q[k].s * r;
      bsum += (q[k].m == -INFINITY) ? q[k].b : q[k].b * r;
      if (q[k].m == mn) idx = min(idx, q[k].idx);
    }
  }
  M = mn;
  S = sum;
  I = idx;
  B = bsum;
}

// The whole row from its partials in chunk order, kMergeUnroll loads in
// flight at a time (indices clamped into the row).
__device__ __forceinline__ void merge_row(const Partial* pp, int nch, float c, float& M, float& S, int& I,
                                          float& B) {
  M = -INFINITY;
  S = 0.f;
  I = 0x7FFFFFFF;
  B = 0.f;
  for (int k0 = 0; k0 < nch; k0 += kMergeUnroll) {
    Partial q[kMergeUnroll];
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) q[k] = pp[min(k0 + k, nch - 1)];
    merge_group(q, nch - k0, c, M, S, I, B);
  }
}

// The acceptance scan of sequence s by one wave: with `write`, stores every
// output of the sequence but the final token; returns what the final draw
// needs (kind kFinalDone when nothing is left).  When a slot's chunks fit one
// lane (<= 8) or two (<= 16, then at most 32 slots), lanes own slots (one or
// two lanes per slot) and every load (the sequence's inputs, the layout sums,
// each slot's partials, proposal logit and proposal token) is issued before
// any is used: one round trip.  Otherwise lane r merges slot r in a loop.
__device__ __forceinline__ SeqFinal scan_sequence(const Params& P, int s, ScanShared& sh, bool write) {
  const int lane = threadIdx.x;
  SeqFinal f{};
  f.kind = kFinalDone;
  f.s = s;
  const int mk = P.max_k;
  const int R = P.slots;                       // 2 * max_k + 1
  const int64_t sbase = (int64_t)s * R;
  const int lps = (P.nch_max > kMergeUnroll && R <= kScanThreads / 2) ? 2 : 1;   // lanes per slot
  const bool fast = R * lps <= kScanThreads && P.nch_max <= kMergeUnroll * lps;

  const int K = P.num_draft[s];
  const int md = P.mode[s];
  const float T = P.temperature[s];
  const uint32_t seq_id = P.seq_ids[s];
  const int topk = P.top_k ? P.top_k[s] : 0;
  const float topp = P.top_p ? P.top_p[s] : 1.f;
  Partial q[kMergeUnroll];
  float xv = 0.f, tv = -INFINITY;
  int tk = 0;
  const int myslot = min(lane / lps, R - 1);
  const int part = lane % lps;                 // which 8 chunks of the slot
  const int mynch = (myslot > mk) ? P.nch_d : P.nch_t;
  const int myn = min(max(mynch - part * kMergeUnroll, 0), kMergeUnroll);
  if (fast) {
    const Partial* pp = P.partials + (sbase + myslot) * P.nch_max + part * kMergeUnroll;
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) q[k] = pp[min(k, max(myn - 1, 0))];
    xv = P.xval[sbase + myslot];
    tv = P.tau[sbase + myslot];     // meaningful only for a filtered sequence (selected below)
    tk = P.ptok[(int64_t)s * mk + min(lane, mk - 1)];
  }
  // layout sums in 32 bits: a count outside 0..kLayoutKMax cannot belong to a
  // layout of total_draft (<= 4096 * 128) rows and is flagged on its own, so
  // the in-range sums stay below 2^31
  constexpr int kLayoutKMax = 1 << 19;
  uint32_t tot = 0, bef = 0;
  int out_of_range = 0;
#pragma unroll 4
  for (int j = lane; j < P.B; j += kScanThreads) {
    const int k = P.num_draft[j];
    const bool ok = k >= 0 && k <= kLayoutKMax;
    out_of_range |= !ok;
    const uint32_t kk = ok ? (uint32_t)k : 0u;
    tot += kk;
    bef += (j < s) ? kk : 0u;
  }
  tot = wave_sum_u32(tot);
  bef = wave_sum_u32(bef);
  if (__any(out_of_range) || tot != (uint32_t)P.total_draft) {
    if (write) clear_bad_layout(P, s);
    return f;
  }
  const int off_d = (int)bef;
  const int off_t = off_d + s;

  int st = 0;
  if (K > mk) st |= kStKTooLarge;
  if (md != kSample && md != kGreedy && md != kOnehot && md != kStrict) st |= kStBadMode;
  if (md != kGreedy && !(isfinite(T) && T >= kMinTemperature)) st |= kStBadTemp;
  if (md == kSample && K > 0 && P.dft == nullptr) st |= kStNoDraft;
  if (st) {
    if (write) clear_sequence(P, s, off_t, off_d, K, st);
    return f;
  }
  const float c = (md == kGreedy) ? kLog2e : kLog2e / T;
  const bool sample = md == kSample;
  // top-k / top-p: the filter kernel rewrote this sequence's partials and thresholds
  const bool filt = md != kGreedy && ((topk > 0 && topk < P.V) || topp < 1.f);

  // ---- each used slot's statistics (lane r: slot r), the proposal tokens ----
  int bad = 0, badtok = 0;
  if (fast) {
    const int r = lane / lps;
    const bool used = (r <= K) || (sample && r > mk && r <= mk + K);
    float M = -INFINITY, S = 0.f, B = 0.f;
    int I = 0x7FFFFFFF;
    merge_group(q, myn, c, M, S, I, B);
    if (lps == 2) {         // chunks 0..7 (even lane) then 8..15 (odd lane), same order in both lanes
      const float M2 = dpp_f<kDppQuadXor1>(0.f, M);
      const float S2 = dpp_f<kDppQuadXor1>(0.f, S);
      const float B2 = dpp_f<kDppQuadXor1>(0.f, B);
      const int I2 = dpp_i<kDppQuadXor1>(0, I);
      const float Ma = part ? M2 : M, Sa = part ? S2 : S, Ba = part ? B2 : B;
      const int Ia = part ? I2 : I;
      const float Mb = part ? M : M2, Sb = part ? S : S2, Bb = part ? B : B2;
      const int Ib = part ? I : I2;
      const float mn = fmaxf(Ma, Mb);
      const float mnc = (mn == -INFINITY) ? 0.f : mn * c;
      const float ra = (Ma == -INFINITY) ? 1.f : fexp2(Ma * c - mnc);
      const float rb = (Mb == -INFINITY) ? 1.f : fexp2(Mb * c - mnc);
      M = mn;
      S = Sa * ra + Sb * rb;
      B = Ba * ra + Bb * rb;
      I = min(Ma == mn ? Ia : 0x7FFFFFFF, Mb == mn ? Ib : 0x7FFFFFFF);
    }
    if (used && part == 0 && r < R) {
      sh.M[r] = M;
      sh.S[r] = S;
      sh.I[r] = I;
      sh.X[r] = xv;
      sh.Tau[r] = filt ? tv : -INFINITY;
      if (r <= mk) sh.Bl[r] = B;
      bad = !(isfinite(M) && isfinite(S) && S > 0.f);
    }
    if (lane < K) {
      sh.tok[lane] = tk;
      badtok = (tk < 0 || tk >= P.V);
    }
  } else {
    for (int r = lane; r < R; r += kScanThreads) {
      const bool used = (r <= K) || (sample && r > mk && r <= mk + K);
      if (!used) continue;
      const int nch = (r > mk) ? P.nch_d : P.nch_t;
      float M, S, B;
      int I;
      merge_row(P.partials + (sbase + r) * P.nch_max, nch, c, M, S, I, B);
      sh.M[r] = M;
      sh.S[r] = S;
      sh.I[r] = I;
      if (r <= mk) sh.Bl[r] = B;
      sh.X[r] = P.xval[sbase + r];
      sh.Tau[r] = filt ? P.tau[sbase + r] : -INFINITY;
      bad |= !(isfinite(M) && isfinite(S) && S > 0.f);
    }
    for (int i = lane; i < K; i += kScanThreads) {
      const int x = P.ptok[(int64_t)s * mk + i];
      sh.tok[i] = x;
      badtok |= (x < 0 || x >= P.V);
    }
  }
  if (__any(badtok)) {
    if (write) clear_sequence(P, s, off_t, off_d, K, kStBadToken);
    return f;
  }
  if (__any(bad)) {
    if (write) clear_sequence(P, s, off_t, off_d, K, kStNonfinite);
    return f;
  }
  // the slots' statistics and tokens were written to LDS by other lanes of
  // this wave: keep the compiler from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // ---- p and q at the proposals, uniforms, accept decisions ----
  int A = K;
  for (int i0 = 0; i0 < K; i0 += kScanThreads) {
    const int i = i0 + lane;
    int reject = 0;
    if (i < K) {
      const int d = mk + 1 + i;
      const float p = (sh.X[i] >= sh.Tau[i]) ? fexp2(fmaf(sh.X[i], c, -(sh.M[i] * c))) / sh.S[i] : 0.f;
      const float qd =
          sample ? ((sh.X[d] >= sh.Tau[d]) ? fexp2(fmaf(sh.X[d], c, -(sh.M[d] * c))) / sh.S[d] : 0.f) : 1.f;
      int acc;
      if (md == kGreedy) {
        acc = (sh.tok[i] == sh.I[i]);
      } else if (md == kStrict) {
        // accept iff the target's own draw y ~ p_i (inverse CDF, uniform u_i)
        // lands on the proposal: t = u*S inside [B, B + e) of the proposal
        const float u = draw_uniform(P, seq_id, (uint32_t)i, 0u);
        const float e = (sh.X[i] >= sh.Tau[i]) ? fexp2(fmaf(sh.X[i], c, -(sh.M[i] * c))) : 0.f;
        const float t = u * sh.S[i];
        acc = (t >= sh.Bl[i]) && (t < sh.Bl[i] + e);
      } else {
        const float u = draw_uniform(P, seq_id, (uint32_t)i, 0u);
        const float r = (md == kOnehot) ? p : (qd > 0.f ? fminf(1.f, p / qd) : 0.f);
        acc = u < r;
      }
      if (write && P.p_at) P.p_at[off_d + i] = p;
      if (write && P.q_at) P.q_at[off_d + i] = qd;
      reject = !acc;
    }
    const unsigned long long rj = __ballot(reject);
    if (A == K && rj != 0ull) A = i0 + (int)__builtin_ctzll(rj);
  }

  // ---- emitted tokens: accepted prefix, -1 after A; greedy fills A too ----
  for (int j = lane; write && j <= K; j += kScanThreads) {
    if (j < A) P.emitted[off_t + j] = sh.tok[j];
    else if (j > A) P.emitted[off_t + j] = -1;
    else if (md == kGreedy) P.emitted[off_t + j] = sh.I[A];
  }
  if (write && lane == 0) {
    P.accepted_len[s] = A;
    if (md == kGreedy && P.status) P.status[s] = 0;
  }
  f.A = A;
  f.emit_pos = off_t + A;
  f.c = c;
  f.taut = -INFINITY;
  f.taud = -INFINITY;
  if (md != kGreedy) {
    f.trow = off_t + A;
    f.mct = sh.M[A] * c;
    f.taut = sh.Tau[A];
    if (sample && A < K) f.taud = sh.Tau[mk + 1 + A];
    f.u = draw_uniform(P, seq_id, (uint32_t)A, 1u);
    if (A == K) {
      f.kind = kFinalBonus;
    } else if (md == kOnehot) {
      f.kind = kFinalOnehot;
      f.xhat = sh.tok[A];
    } else if (md == kStrict) {
      // the emitted token is the target's own draw y (which missed the
      // proposal): the draw from p with the proposal removed, at the point
      // t' = t (below the proposal's interval) or t - e (above it), so the
      // proposal itself can never come out
      const float uA = draw_uniform(P, seq_id, (uint32_t)A, 0u);
      const float e = (sh.X[A] >= sh.Tau[A]) ? fexp2(fmaf(sh.X[A], c, -(sh.M[A] * c))) : 0.f;
      const float t = uA * sh.S[A];
      const float tr = (t < sh.Bl[A]) ? t : t - e;
      const float Zr = sh.S[A] - e;
      f.kind = kFinalOnehot;
      f.xhat = sh.tok[A];
      f.u = (Zr > 0.f) ? fminf(fmaxf(tr / Zr, 0.f), 0x1.fffffep-1f) : uA;
    } else {
      f.kind = kFinalResidual;
      f.drow = off_d + A;
      f.mcd = sh.M[mk + 1 + A] * c;
      f.rq = sh.S[A] / sh.S[mk + 1 + A];
    }
  }
  return f;
}

// Final kernel, grid (nsplit, B), 1024 threads.  Wave 0 runs the acceptance
// scan of sequence s (split 0 writes its outputs and the record); then the
// block sums the final weights of its tiles (j = split mod nsplit) of the
// row(s) at the stop position.  With one block per sequence the same block
// picks the token; otherwise the tile sums go to HBM and the last of the
// sequence's blocks to store its share picks it.
__global__ void __launch_bounds__(kFinThreads) k_final(Params P) {
  __shared__ ScanShared ssh;
  __shared__ FinShared sh;
  __shared__ SeqFinal sf;
  const int split = blockIdx.x, s = blockIdx.y;
  const int t = threadIdx.x;
  if (t < kWave) {
    const SeqFinal f = scan_sequence(P, s, ssh, split == 0);
    if (t == 0) {
      sf = f;
      if (split == 0) P.fin[s] = f;
    }
  }
  __syncthreads();
  const SeqFinal f = sf;
  if (f.kind == kFinalDone) return;
  if (f.kind != kFinalResidual) {   // bonus or one-hot: from the chunk partials
    if (split == 0) finish_draw_chunks(P, f, sh);
    return;
  }
  tile_sums_pass(P, f, f.kind, split, P.nsplit, sh);
  __syncthreads();
  if (P.nsplit == 1) {
    if (t < P.ntiles) sh.tile[t] = tile_total(sh, t);
    __syncthreads();
    finish_draw(P, f, sh);
    return;
  }
  // Split draw: wave 0 stores this block's tile sums (tiles split, split +
  // nsplit, ...) with device-coherent stores and waits until they are done,
  // then counts the block in.  The block that brings the count to nsplit
  // reads every tile sum back with device-coherent loads and draws the token.
  // No block waits for another; the counter was zeroed by row_stats.
  if (t < kWave) {
    const int64_t tb = (int64_t)s * P.ntiles;
    for (int j = split + t * P.nsplit; j < P.ntiles; j += kWave * P.nsplit)
      __hip_atomic_store(&P.tilesum[tb + j], tile_total(sh, j), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the stores are done before the count
    uint32_t old = 0;
    if (t == 0) old = __hip_atomic_fetch_add(&P.fincnt[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = __builtin_amdgcn_readfirstlane((int)old) == P.nsplit - 1;
    if (last) {
      for (int j = t; j < P.ntiles; j += kWave)
        sh.tile[j] = __hip_atomic_load(&P.tilesum[tb + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (t == 0) sh.arrived_last = last;
  }
  __syncthreads();
  if (sh.arrived_last) finish_draw(P, f, sh);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_row_stats(const Params& p, hipStream_t st, const LaunchEvents* ev) {
  const int64_t blocks = (int64_t)p.n_t * p.nch_t + (int64_t)p.n_d * p.nch_d + p.order_block;
  if (blocks <= 0) return record_empty(st, ev);
  // at most 65535 blocks per grid dimension; gy rows of gx blocks leave fewer than gy unused
  const int64_t gy = (blocks + kMaxGridX - 1) / kMaxGridX;
  const int64_t gx = (blocks + gy - 1) / gy;
  const dim3 g((unsigned)gx, (unsigned)gy), b(kThreads);
  if (p.t_bf16) {
    if (p.d_bf16) launch_timed(k_row_stats<true, true>, g, b, st, ev, p);
    else launch_timed(k_row_stats<true, false>, g, b, st, ev, p);
  } else {
    if (p.d_bf16) launch_timed(k_row_stats<false, true>, g, b, st, ev, p);
    else launch_timed(k_row_stats<false, false>, g, b, st, ev, p);
  }
  return hipGetLastError();
}

hipError_t launch_final(const Params& p, hipStream_t st, const LaunchEvents* ev) {
  launch_timed(k_final, dim3(p.nsplit, p.B), dim3(kFinThreads), st, ev, p);
  return hipGetLastError();
}

hipError_t launch_select(const Params& p, hipStream_t st, const LaunchEvents* ev) {
  (void)p;
  return record_empty(st, ev);   // the last split final block draws the token
}

}  // namespace sv
