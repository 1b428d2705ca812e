// Top-k / top-p filter of the verify rows for gfx950.
//
// The pages list top-k and nucleus rejection sampling among the
// verification strategies that keep the target's distribution ("Draft
// Model（草稿模型）", compassingai.com, 常见误读纠偏 误读 4; the
// gitcode.csdn.net tutorial, section 5.4 采样策略对比): the same filter acts
// on the target row and on the draft row, and the accept/correct rule then
// runs on the renormalised distributions.  A token is kept iff its logit is
// at least a threshold tau: top-k keeps the tokens with fewer than k
// strictly larger logits (ties at the k-th value all kept); top-p, applied
// after top-k, keeps a token iff the mass of the strictly larger tokens is
// below p (the largest logit always kept).
//
// One 512-thread block per used row of a filtered sequence, after the row
// statistics (four blocks per CU), in the order of the list that row
// statistics' first block writes (the sequences by temperature, the flattest
// rows, whose filter costs most, first).  The row maximum M comes from the row's
// chunk partials (for top-p alone, also the row's mass).  Then:
//   A. the bounded selection (no per-element atomics): a bound that every
//      kept token is at or above, from the row's segment maxima that the
//      row statistics wrote (32 per 32 KB; top-k of at most half their
//      number, and top-p alone), else from every thread's two largest
//      logits over a sample of the row (top-k) or the whole row (top-p
//      alone): the k-th largest of at most 512 segment maxima by ballots in
//      one wave, else a 2-pass radix select over the maxima; one
//      read collects the tokens at or above it into LDS (with segment
//      maxima only the segments whose maximum reaches the bound, when at
//      most 256 do); exact thresholds among them (ranks, or a sort when
//      there are many); the filtered chunk sums are the kept tokens' masses;
//   B. when the bound cannot hold (top-k above 1024, maxima short of the
//      top-p mass, more tokens than the LDS buffer) and one filter acts
//      alone: on 16-byte aligned bf16 rows the value table (a sample picks a
//      band of values around the crossing; one read counts the band's
//      tokens per value and chunk in LDS and sums the mass above it; the
//      threshold is exact among the band's values), else, or when the
//      table cannot decide, the bracket search (passes that narrow a
//      bracket of d holding the crossing, then one that collects it);
//   C. the histogram path, for what the others leave: a coarse histogram
//      of d = M*c - x*c in steps of 1/8 (log2 units; the last of 256 bins
//      also takes everything below 2^-32 of the maximum) with integer LDS
//      atomics, the bin holding the threshold, its elements compacted into
//      LDS (or refined by a fine histogram), an exact radix select over
//      their keys, and a pass for the chunk sums.
// Every path rewrites the row's chunk partials as filtered sums against
// M (and, for strict-mode target rows, the filtered part below the
// proposal), and tau is stored for the scan and the final draw.  Masses are
// exp2(x*c - M*c) in 2^-40 fixed point, summed as integers, so every result
// is independent of the order of the atomics; every decision on which
// tokens are kept is a comparison of stored values, and only the top-p
// crossing depends on sums.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"
#include "sv_wave.h"

namespace sv {

namespace {

using namespace wave;

constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / kWave;
constexpr int kHist = kFWaves / 2;             // histogram copies (one per pair of waves)
constexpr int kBins = 256;
constexpr float kBinScale = 8.f;               // bins per log2 unit below the row maximum
constexpr float kBinSpan = kBins / kBinScale;  // 32: d beyond this falls into the last bin
constexpr float kFineScale = 2048.f;           // fine bins per log2 unit inside one coarse bin
constexpr int kCap = 1024;                     // candidates held in LDS
constexpr int kUnroll = 16;                    // loads in flight per thread
constexpr int kBJ = 4;                         // thresholds of a dense bracket-search pass (8 or 16: slower, ALU-bound)
constexpr int kMaxChunks = kMaxTiles * kTileElems / (kChunkBytes / 4);   // 256
constexpr double kMassOne = 1099511627776.0;   // 2^40
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kMinTemp = 1e-6f;
constexpr int kModeSample = 0, kModeGreedy = 1, kModeStrict = 3;
constexpr int kLayoutKMax = 1 << 19;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// a block-uniform value read from LDS, moved to a scalar register
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ float uni(float v) { return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v))); }

// order-preserving 32-bit key of a float (larger float, larger key; no NaN);
// -0 and +0 get the key of +0, so equal floats have equal keys
__device__ __forceinline__ uint32_t fkey(float x) {
  uint32_t b = __float_as_uint(x);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float kval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// bf16 values in the order of their 16-bit keys: one step up or down
__device__ __forceinline__ float bf16_step(float v, int dir) {
  const uint32_t h = __float_as_uint(v) >> 16;
  uint32_t k = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
  k = (k + (uint32_t)dir) & 0xFFFFu;
  const uint32_t g = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(g << 16);
}

// true when at most one bf16 value x has dlo < fmaf(-x, c, mc) <= dhi (the
// d of every element that value holds); false also when that is not sure
__device__ __forceinline__ bool one_bf16_value(float dlo, float dhi, float c, float mc) {
  // the smallest value with d <= dhi (d does not increase with x): from an
  // estimate, a few steps each way
  float v = __uint_as_float(__float_as_uint((mc - dhi) / c) & 0xFFFF0000u);
  for (int i = 0; i < 4 && !(fmaf(-v, c, mc) <= dhi); ++i) v = bf16_step(v, 1);
  for (int i = 0; i < 4 && fmaf(-bf16_step(v, -1), c, mc) <= dhi; ++i) v = bf16_step(v, -1);
  if (!(fmaf(-v, c, mc) <= dhi) || fmaf(-bf16_step(v, -1), c, mc) <= dhi) return false;
  // one value iff the next one up is above the bracket already
  return fmaf(-bf16_step(v, 1), c, mc) <= dlo;
}

template <bool BF>
__device__ __forceinline__ float load_x(const char* rowp, int e) {
  return BF ? __uint_as_float((uint32_t)((const uint16_t*)rowp)[e] << 16) : ((const float*)rowp)[e];
}

// Every element e < V of the row once: thread t takes e = base + u*kFThreads + t,
// all kUnroll loads of a round issued before f sees any.
template <bool BF, typename F>
__device__ __forceinline__ void for_row(const char* rowp, int V, F&& f) {
  const int t = threadIdx.x;
  for (int base = 0; base < V; base += kFThreads * kUnroll) {
    float x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = base + u * kFThreads + t;
      x[u] = e < V ? load_x<BF>(rowp, e) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int e = base + u * kFThreads + t;
      if (e < V) f(x[u], e);
    }
  }
}

// coarse bin of d = M*c - x*c (correctly rounded, so monotone in x): 1/8
// log2 unit per bin; d beyond 32 (and NaN, -inf) in the last bin
__device__ __forceinline__ int coarse_bin(float d) {
  return (d < kBinSpan) ? min(kBins - 1, max(0, (int)(d * kBinScale))) : kBins - 1;
}
// fine bin inside coarse bin b: 1/2048 log2 unit per bin (monotone in d)
__device__ __forceinline__ int fine_bin(float d, int b) {
  const float f = (d - (float)b * (1.f / kBinScale)) * kFineScale;
  return (f < (float)kBins) ? max(0, (int)f) : kBins - 1;
}

// floor(e * 2^40) for e = exp2(-d) clamped to [0, 2], with integer operations only
__device__ __forceinline__ uint64_t fixed_mass_d(float d) {
  const float e = fminf(fmaxf(fexp2(-d), 0.f), 2.f);        // NaN -> 0
  const uint32_t b = __float_as_uint(e);
  const int E = (int)(b >> 23);
  const uint64_t m = (uint64_t)((b & 0x7FFFFFu) | 0x800000u);
  const int sh = E - 110;                                     // e = m * 2^(E-150); times 2^40
  if (E == 0) return 0;
  return sh >= 0 ? (m << sh) : (sh > -24 ? (m >> (-sh)) : 0);
}

struct HistBufs {
  uint32_t wc[kHist][kBins];   // per-pair histograms (coarse, then fine)
  uint64_t wm[kHist][kBins];
};
struct BoundBufs {
  uint32_t tk[kFThreads];      // the compacted kept set's keys
  int32_t ci[kCap];            // candidates' token indices
  uint64_t lsum[kWave];        // per-lane mass sums of a prefix walk
  double zl[kWave];
};

// the value table of a bf16 row: keys of S slots, then per slot the token
// counts of its chunks, 16 bits a chunk, two chunks a word
struct ValueBufs {
  uint32_t w[sizeof(HistBufs) / sizeof(uint32_t)];
};

struct FiltShared {
  union {                      // the bounded selection, the value table and the histograms run one after another
    HistBufs hb;
    BoundBufs bb;
    ValueBufs vt;
  };
  uint32_t hc[kBins];          // merged coarse histogram
  uint64_t hm[kBins];
  uint32_t fc[kBins];          // merged fine histogram
  uint64_t fm[kBins];
  alignas(16) uint32_t ck[kCap + 4];   // candidates: keys (4 spare entries for padding) and masses
  uint64_t cm[kCap];
  uint32_t rc[kBins];          // radix byte histogram
  uint64_t rm[kBins];
  uint64_t cs[kMaxChunks];     // filtered chunk sums, fixed point
  uint64_t cb[kMaxChunks];     // their parts below the proposal (strict target rows)
  uint32_t ncand, kmin_c, kmax_c;
  uint32_t tmin, nkc;          // bounded selection: smallest kept key, kept-set counter
  double mtot;                 // mass above the candidates plus theirs (selection by ranks or prefixes)
  uint32_t segb;                // bounded selection: the top-k bound from the segment maxima
  // bracket search (top-p alone): per-wave, then block sums of the masses and
  // counts at or below each threshold, and the bracket's key range
  float wfm[kFWaves][kBJ];
  uint32_t wfn[kFWaves][kBJ];
  double bm[kBJ];
  uint32_t bn[kBJ];
  uint32_t bkmin, bkmax;
  int last;                    // last non-empty bin of the latest crossing search
  uint64_t amass;
  int bin;
  uint32_t need;
  double rem;
  int ok;
  int offd;
  float M;
  double zrow;                 // the row's mass against M, 2^-40 units, from the chunk partials
  int nk, ne, ni;
  uint32_t nsegc;              // bounded selection: segments whose maximum reaches the bound (listed in hc)
  int vt_over;                 // value table: more distinct values than it takes
  uint32_t vt_n;               // value table: distinct values inserted
  uint32_t vt_tau;             // value table: the threshold key (0: none)
  uint32_t vt_na;              // value table: tokens above the band
  uint32_t vt_u16, vt_l16;     // value table: the band's keys
};

// The crossing of a 256-bin histogram, run by wave 0: bins in order
// i = 0..255 (bin i, or 255 - i when `desc`), empty bins skipped; the first
// bin where the running count reaches `need` (or the running mass reaches
// `target`).  Each lane sums 4 bins, then a walk over the 64 lane sums
// (readlane, uniform) and over the 4 bins of the crossing lane.  Writes
// sh.bin (-1 when never reached: rounding, mass mode only), sh.need or
// sh.rem (what is left inside the bin) and sh.last (the last non-empty bin).
template <bool BY_MASS>
__device__ __forceinline__ void scan_bins(FiltShared& sh, const uint32_t* hc, const uint64_t* hm, bool desc,
                                          uint32_t need, double target) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t lc = 0;
  uint64_t lm = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane * 4 + j;
    const int b = desc ? kBins - 1 - i : i;
    lc += hc[b];
    if (BY_MASS) lm += hm[b];
  }
  uint32_t acc_c = 0;
  double acc_m = 0.0;
  int cl = -1, last_l = -1;
  for (int l = 0; l < kWave; ++l) {
    const uint32_t c_l = (uint32_t)__builtin_amdgcn_readlane((int)lc, l);
    if (c_l == 0) continue;
    last_l = l;
    double m_l = 0.0;
    if (BY_MASS) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lm, l);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lm >> 32), l);
      m_l = (double)(((uint64_t)hi << 32) | lo);
      if (acc_m + m_l >= target) {
        cl = l;
        break;
      }
    } else if (acc_c + c_l >= need) {
      cl = l;
      break;
    }
    acc_c += c_l;
    acc_m += m_l;
  }
  int bin = -1, last = -1;
  const int ll = cl >= 0 ? cl : last_l;
  if (ll >= 0) {
    for (int j = 0; j < 4; ++j) {
      const int i = ll * 4 + j;
      const int b = desc ? kBins - 1 - i : i;
      const uint32_t cb = hc[b];
      if (cb == 0) continue;
      last = b;
      if (cl < 0) continue;
      if (BY_MASS) {
        const double mb = (double)hm[b];
        if (acc_m + mb >= target) {
          bin = b;
          break;
        }
        acc_m += mb;
      } else {
        if (acc_c + cb >= need) {
          bin = b;
          break;
        }
        acc_c += cb;
      }
    }
  }
  if (lane == 0) {
    sh.bin = bin;
    sh.need = need - acc_c;
    sh.rem = target - acc_m;
    sh.last = last;
  }
}

// Elements of one region of the row: coarse bin `bin`, fine bin `fine`
// (-1: any), key >= kmin.
struct Region {
  int bin, fine;
  uint32_t kmin;
};

__device__ __forceinline__ bool in_region(const Region& rg, float d, uint32_t k) {
  return coarse_bin(d) == rg.bin && (rg.fine < 0 || fine_bin(d, rg.bin) == rg.fine) && k >= rg.kmin;
}

// One slot per candidate: a ballot per wave and one LDS atomic by its first lane.
__device__ __forceinline__ uint32_t claim_slot(uint32_t* counter, bool want) {
  const unsigned long long m = __ballot(want);
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t base = 0;
  if (m) {
    const int leader = __ffsll((long long)m) - 1;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
  }
  const unsigned long long below = (lane == 0) ? 0ull : (m & (~0ull >> (kWave - lane)));
  return base + (uint32_t)__popcll(below);
}

// The key threshold inside a region, exactly: the need-th largest key
// (by count) or the key where the mass from the top first reaches `target`
// (the smallest key when it never does).  Candidates go to LDS when they
// fit; otherwise the radix passes read the row.
template <bool BF, bool BY_MASS, bool COLLECT>
__device__ __forceinline__ uint32_t select_region(FiltShared& sh, const char* rowp, int V, float c, float mc,
                                                  const Region& rg, uint32_t need, double target) {
  const int t = threadIdx.x;
  if (t == 0) {
    sh.ncand = 0;
    sh.kmin_c = 0xFFFFFFFFu;
    sh.kmax_c = 0u;
  }
  __syncthreads();
  for_row<BF>(rowp, V, [&](float x, int) {
    const float d = fmaf(-x, c, mc);
    const uint32_t k = fkey(x);
    const bool want = in_region(rg, d, k);
    const uint32_t i = claim_slot(&sh.ncand, want);
    if (want) {
      if (i < (uint32_t)kCap) {
        sh.ck[i] = k;
        if (COLLECT) sh.cm[i] = fixed_mass_d(d);
      }
      atomicMin(&sh.kmin_c, k);
      atomicMax(&sh.kmax_c, k);
    }
  });
  __syncthreads();
  const uint32_t n = sh.ncand;
  if (sh.kmin_c == sh.kmax_c) return sh.kmin_c;      // every candidate has the same key (or none)
  const bool in_lds = n <= (uint32_t)kCap;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (t < kBins) {
      sh.rc[t] = 0;
      sh.rm[t] = 0;
    }
    __syncthreads();
    if (in_lds) {
      for (uint32_t i = t; i < n; i += kFThreads) {
        const uint32_t k = sh.ck[i];
        if ((k & pmask) == prefix) {
          const int by = (k >> shift) & 0xFF;
          atomicAdd(&sh.rc[by], 1u);
          if (BY_MASS) atomicAdd(&sh.rm[by], (unsigned long long)sh.cm[i]);
        }
      }
    } else {
      for_row<BF>(rowp, V, [&](float x, int) {
        const float d = fmaf(-x, c, mc);
        const uint32_t k = fkey(x);
        if (in_region(rg, d, k) && (k & pmask) == prefix) {
          const int by = (k >> shift) & 0xFF;
          atomicAdd(&sh.rc[by], 1u);
          if (BY_MASS) atomicAdd(&sh.rm[by], (unsigned long long)fixed_mass_d(d));
        }
      });
    }
    __syncthreads();
    if (t < kWave) scan_bins<BY_MASS>(sh, sh.rc, sh.rm, true, need, target);
    __syncthreads();
    const int by = sh.bin >= 0 ? sh.bin : sh.last;
    prefix |= (uint32_t)by << shift;
    pmask |= 0xFFu << shift;
    if (BY_MASS) target = sh.rem;
    else need = sh.need;
    __syncthreads();
  }
  return prefix;
}

// Per-pair histograms of one region (coarse: fine = -2 means "bin every
// element by its coarse bin"), merged into (hc, hm).
template <bool BF, bool MASS>
__device__ __forceinline__ void histogram(FiltShared& sh, const char* rowp, int V, float c, float mc, int coarse_b,
                                          uint32_t kmin, uint32_t* hc, uint64_t* hm) {
  const int t = threadIdx.x, h = (t / kWave) >> 1;
  for (int j = t; j < kHist * kBins; j += kFThreads) {
    (&sh.hb.wc[0][0])[j] = 0;
    (&sh.hb.wm[0][0])[j] = 0;
  }
  __syncthreads();
  uint32_t lc = 0;       // the coarse last bin, in registers
  uint64_t lm = 0;
  for_row<BF>(rowp, V, [&](float x, int) {
    const float d = fmaf(-x, c, mc);
    int b = coarse_bin(d);
    if (coarse_b >= 0) {
      if (b != coarse_b || fkey(x) < kmin) return;
      b = fine_bin(d, coarse_b);
    } else if (b == kBins - 1) {
      ++lc;
      if (MASS) lm += fixed_mass_d(d);
      return;
    }
    atomicAdd(&sh.hb.wc[h][b], 1u);
    if (MASS) atomicAdd(&sh.hb.wm[h][b], (unsigned long long)fixed_mass_d(d));
  });
  if (lc) {
    atomicAdd(&sh.hb.wc[h][kBins - 1], lc);
    if (MASS) atomicAdd(&sh.hb.wm[h][kBins - 1], (unsigned long long)lm);
  }
  __syncthreads();
  if (t < kBins) {
    uint32_t cs = 0;
    uint64_t ms = 0;
    for (int w = 0; w < kHist; ++w) {
      cs += sh.hb.wc[w][t];
      if (MASS) ms += sh.hb.wm[w][t];
    }
    hc[t] = cs;
    hm[t] = ms;
  }
  __syncthreads();
}

// The threshold key inside coarse bin b (keys >= kmin): fine histogram, the
// crossing fine bin, then the exact select among its elements.  With
// `above` the mass at or above the returned key inside the bin is left in
// sh.amass (by-count selections used before a top-p step need it).
template <bool BF, bool BY_MASS, bool MASS>
__device__ __forceinline__ uint32_t select_in_bin(FiltShared& sh, const char* rowp, int V, float c, float mc, int b,
                                                  uint32_t kmin, uint32_t need, double target, bool above) {
  const int t = threadIdx.x;
  // a bin that fits the candidate buffer is selected in directly; a larger
  // one is narrowed by a fine histogram first (one more pass over the row)
  const bool fine = sh.hc[b] > (uint32_t)kCap;
  int fb = -1;
  uint32_t need2 = need;
  double rem2 = target;
  if (fine) {
    histogram<BF, MASS>(sh, rowp, V, c, mc, b, kmin, sh.fc, sh.fm);
    if (t < kWave) scan_bins<BY_MASS>(sh, sh.fc, sh.fm, false, need, target);
    __syncthreads();
    fb = sh.bin >= 0 ? sh.bin : sh.last;
    need2 = sh.need;
    rem2 = sh.rem;
    __syncthreads();
  }
  const Region rg{b, fb, kmin};
  const uint32_t key = select_region<BF, BY_MASS, MASS>(sh, rowp, V, c, mc, rg, need2, rem2);
  if (above && MASS) {
    // mass of the bin at or above the key: the fine bins before fb, plus fb's part at or above it
    if (t == 0) sh.amass = 0;
    __syncthreads();
    uint64_t part = 0;
    const uint32_t n = sh.ncand;
    if (n <= (uint32_t)kCap) {
      for (uint32_t i = t; i < n; i += kFThreads)
        if (sh.ck[i] >= key) part += sh.cm[i];
    } else {
      for_row<BF>(rowp, V, [&](float x, int) {
        const float d = fmaf(-x, c, mc);
        const uint32_t k = fkey(x);
        if (in_region(rg, d, k) && k >= key) part += fixed_mass_d(d);
      });
    }
    if (fine && t < fb) part += sh.fm[t];
    if (part) atomicAdd(&sh.amass, (unsigned long long)part);
    __syncthreads();
  }
  return key;
}

// ---- bounded selection: two reads of the row, no per-element atomics ----
//
// Each thread's largest logits are elements of the row, so the k-th largest
// of the 1024 maxima (two per thread, over the whole row or a prefix of it) is at
// most the row's k-th largest logit: every token that top-k keeps is at or
// above it.  For top-p alone, the maxima
// taken from the top until their mass reaches the target give a bound with
// the same property (everything below it has at least that much mass above
// it).  The second read collects the tokens at or above the bound into LDS;
// when they fit, the thresholds are selected exactly among them (a sort,
// then counts and fixed-point mass prefixes) and the filtered chunk sums
// are their masses.  When they do not (a bound that many tokens tie with,
// or top-k above 1024), the histogram path takes over.

constexpr int kVecPer = 4;                     // 16-byte loads in flight per thread

// the row as whole 16-byte vectors plus a few single elements: `head`
// elements before the first 16-byte boundary, `tail` after the last vector
struct RowSplit {
  int head, nvec, tail;
};
template <bool BF>
__device__ __forceinline__ RowSplit split_row(const char* rowp, int V) {
  constexpr int es = BF ? 2 : 4, epv = 16 / es;
  const int mis = (int)((uintptr_t)rowp & 15);          // a multiple of es (pointers are element-aligned)
  const int head = min(mis ? (16 - mis) / es : 0, V);
  const int nvec = (V - head) / epv;
  return {head, nvec, V - head - nvec * epv};
}

// the elements of one 16-byte vector (little-endian: element 2i in the low
// half of word i for bf16); vectors past the row are filled with NaN, which
// no comparison below accepts and fmaxf ignores
template <bool BF>
__device__ __forceinline__ float vec_elem(const uint4& w, int j) {
  const uint32_t wd = (j / (BF ? 2 : 1)) == 0 ? w.x : (j / (BF ? 2 : 1)) == 1 ? w.y : (j / (BF ? 2 : 1)) == 2 ? w.z : w.w;
  if (!BF) return __uint_as_float(wd);
  return __uint_as_float((j & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
}
constexpr uint32_t kNanFill = 0x7FC07FC0u;     // NaN as one fp32 word and as two bf16 halves
// a row-statistics segment (the 8-lane group that wrote its maximum): 8 runs
// of 8 vectors (128 bytes each), kThreads vectors apart, in a chunk of 2048
// 16-byte vectors
constexpr int kChunkVecs = kChunkBytes / 16;
constexpr int kSegRun = kThreads / kSegPerChunk;
constexpr int kSegVecs = kChunkVecs / kSegPerChunk;
constexpr int kSegRound = kFThreads * kVecPer / kSegVecs;   // segments a round of the bounded selection's read 2
static_assert(kSegRun == 8 && kSegVecs == 64 && kSegRound == 32, "the row statistics' segment layout");
// top-k from at most this many segment maxima: wave 0 holds them all (8 a
// lane) and finds the k-th largest bit by bit; from more, the radix select
constexpr int kBallotSegs = 8 * kWave;
static_assert(kBallotSegs <= kCap, "the ballot search reads the segment maxima from their copy in sh.ck");

// rounds of 16-byte vectors [vb, ve) (vb a multiple of kFThreads * kVecPer):
// f(w, v0) per round, vectors at or past ve filled with NaN
template <typename F>
__device__ __forceinline__ void for_rounds(const uint4* vp, int vb, int ve, F&& f) {
  const int t = threadIdx.x;
  for (int v0 = vb; v0 < ve; v0 += kFThreads * kVecPer) {
    uint4 w[kVecPer];
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) {
      const int vi = v0 + u * kFThreads + t;
      w[u] = vi < ve ? vp[vi] : make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
    }
    f(w, v0);
  }
}

// Rounds of 16-byte vectors [vb, ve) (vb a multiple of kFThreads * kVecPer,
// vb < ve), the first round's vectors already in w: f(w, v0) per round.
// Each round's loads are issued before the previous round is passed to f,
// and every load is issued (indices clamped into [0, ve), so the last
// round's loads are issued twice): the wait before f then covers that
// round's loads only.  f sees vectors at or past ve as NaN, and must load
// nothing from global memory itself (such a load would wait for the next
// round's too).
template <typename F>
__device__ __forceinline__ void for_rounds_pipe(const uint4* vp, uint4 (&w)[kVecPer], int vb, int ve, F&& f) {
  constexpr int kRound = kFThreads * kVecPer;
  const int t = threadIdx.x;
  const int last = ((ve - 1) / kRound) * kRound;
  for (int v0 = vb; v0 < ve; v0 += kRound) {
    uint4 nx[kVecPer];
    const int vn = min(v0 + kRound, last);
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) nx[u] = vp[min(vn + u * kFThreads + t, ve - 1)];
    if (v0 == last) {
#pragma unroll
      for (int u = 0; u < kVecPer; ++u)
        if (v0 + u * kFThreads + t >= ve) w[u] = make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
    }
    f(w, v0);
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) w[u] = nx[u];
  }
}

// element b of a round (vector b / epv, element b % epv), from the
// registers: a tree of selects over the round's 16 words held as separate
// scalars (selects between elements of one array would be folded into a
// run-time index, which places the array in memory)
template <bool BF>
__device__ __forceinline__ float round_elem(const uint4 (&w)[kVecPer], int b) {
  static_assert(kVecPer == 4, "16 words a round");
  const int wi = BF ? (b >> 1) : b;
  const bool b0 = wi & 1, b1 = wi & 2, b2 = wi & 4, b3 = wi & 8;
  const uint32_t p0 = b0 ? w[0].y : w[0].x, p1 = b0 ? w[0].w : w[0].z;
  const uint32_t p2 = b0 ? w[1].y : w[1].x, p3 = b0 ? w[1].w : w[1].z;
  const uint32_t p4 = b0 ? w[2].y : w[2].x, p5 = b0 ? w[2].w : w[2].z;
  const uint32_t p6 = b0 ? w[3].y : w[3].x, p7 = b0 ? w[3].w : w[3].z;
  const uint32_t q0 = b1 ? p1 : p0, q1 = b1 ? p3 : p2, q2 = b1 ? p5 : p4, q3 = b1 ? p7 : p6;
  const uint32_t r0 = b2 ? q1 : q0, r1 = b2 ? q3 : q2;
  const uint32_t wd = b3 ? r1 : r0;
  if (!BF) return __uint_as_float(wd);
  return __uint_as_float((b & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
}

// the head and tail elements of a row split: f(w, -1 - e) with element e as
// element 0 of w[0] and NaN everywhere else, by the first head + tail threads
template <bool BF, typename F>
__device__ __forceinline__ void for_singles(const char* rowp, const RowSplit& sp, F&& f) {
  constexpr int epv = BF ? 8 : 4;
  const int t = threadIdx.x;
  if (t < sp.head + sp.tail) {
    const int e = t < sp.head ? t : sp.head + sp.nvec * epv + (t - sp.head);
    uint4 w[kVecPer];
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) w[u] = make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
    const float x = load_x<BF>(rowp, e);
    if (BF) w[0].x = (__float_as_uint(x) >> 16) | 0x7FC00000u;   // element 0: x, element 1: NaN
    else w[0].x = __float_as_uint(x);
    f(w, -1 - e);
  }
}

// index of element j of vector u of a round (v0 >= 0), or the single element
template <bool BF>
__device__ __forceinline__ int elem_index(const RowSplit& sp, int v0, int u, int j) {
  constexpr int epv = BF ? 8 : 4;
  return v0 >= 0 ? sp.head + (v0 + u * kFThreads + (int)threadIdx.x) * epv + j : -1 - v0;
}

// bitonic sort of k[0..n2) (n2 a power of two, at most 2 * kFThreads),
// largest first, with an optional payload; every thread calls it
__device__ __forceinline__ void sort_desc(uint32_t* k, int32_t* pay, int n2) {
  const int t = threadIdx.x;
  for (int size = 2; size <= n2; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      if (t < n2 / 2) {
        const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1));
        const int l = i | j;
        const uint32_t a = k[i], b = k[l];
        const bool desc = (i & size) == 0;
        if (desc ? a < b : a > b) {
          k[i] = b;
          k[l] = a;
          if (pay) {
            const int32_t pa = pay[i];
            pay[i] = pay[l];
            pay[l] = pa;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Wave 0: over keys[0..n) sorted largest first, the fixed-point masses
// summed in order, on top of mass0 (the mass of the row above keys[0]).
// With Z = zuse (or the total of the n masses when zuse < 0) and target =
// topp * Z (0 when topp <= 0), writes sh.ne = #{i: mass strictly before i <
// target}, sh.ni = #{i: mass through i < target} and sh.mtot = mass0 + the
// n masses.
__device__ __forceinline__ void mass_prefix(FiltShared& sh, const uint32_t* keys, int n, float c, float mc,
                                            float topp, double zuse, double mass0 = 0.0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (n + kWave - 1) / kWave;
  const int lo = min(lane * per, n), hi = min(lo + per, n);
  uint64_t ls = 0;
#pragma unroll 4
  for (int i = lo; i < hi; ++i) ls += fixed_mass_d(fmaf(-kval(keys[i]), c, mc));
  sh.bb.lsum[lane] = ls;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint64_t base = 0, tot = 0;
#pragma unroll 8
  for (int l = 0; l < kWave; ++l) {
    const uint64_t v = sh.bb.lsum[l];
    base += (l < lane) ? v : 0;
    tot += v;
  }
  const double z = zuse < 0.0 ? (double)tot : zuse;
  const double target = topp > 0.f ? (double)topp * z : 0.0;
  uint32_t ne = 0, ni = 0;
  uint64_t acc = base;
#pragma unroll 4
  for (int i = lo; i < hi; ++i) {
    ne += mass0 + (double)acc < target;
    acc += fixed_mass_d(fmaf(-kval(keys[i]), c, mc));
    ni += mass0 + (double)acc < target;
  }
  ne = wave_sum_u32(ne);
  ni = wave_sum_u32(ni);
  if (lane == 0) {
    sh.ne = (int)ne;
    sh.ni = (int)ni;
    sh.mtot = mass0 + (double)tot;
  }
}

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;   // fkey(-inf)

// A lower bound of the key at a crossing among two keys per thread: the
// need-th largest (by count) or the key where the mass from the top first
// reaches `target` (by mass), taken 8 bits a pass for `passes` passes; the
// bits below are returned as zeros (so the result is at most the exact key,
// which it equals after 4 passes).  Leaves sh.bin < 0 when the first pass
// never reaches the target (mass only; the key returned is then
// meaningless).  Keys of -inf (threads without elements) are left out: by
// mass they weigh 0, and by count they could only be the answer when fewer
// than `need` finite keys exist, where the result 0 leads the caller to the
// same bound, the key of -inf; left in, they all hit one histogram bin, and
// such LDS atomics serialise.  Every thread of the block calls it.
template <bool BY_MASS>
__device__ __forceinline__ uint32_t radix_select_regs(FiltShared& sh, uint32_t ka, unsigned long long ma,
                                                      uint32_t kb, unsigned long long mb, uint32_t need,
                                                      double target, int passes) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 24 - 8 * pass;
    if (t < kBins) {
      sh.rc[t] = 0;
      sh.rm[t] = 0;
    }
    __syncthreads();
    if ((ka & pmask) == prefix && ka != kKeyNegInf) {
      const int by = (ka >> shift) & 0xFF;
      atomicAdd(&sh.rc[by], 1u);
      if (BY_MASS) atomicAdd(&sh.rm[by], ma);
    }
    if ((kb & pmask) == prefix && kb != kKeyNegInf) {
      const int by = (kb >> shift) & 0xFF;
      atomicAdd(&sh.rc[by], 1u);
      if (BY_MASS) atomicAdd(&sh.rm[by], mb);
    }
    __syncthreads();
    if (t < kWave) scan_bins<BY_MASS>(sh, sh.rc, sh.rm, true, need, target);
    __syncthreads();
    const int bin = uni(sh.bin);
    if (bin < 0) return 0u;                    // block-uniform
    prefix |= (uint32_t)bin << shift;
    pmask |= 0xFFu << shift;
    if (BY_MASS) target = sh.rem;
    else need = uni(sh.need);
    __syncthreads();
  }
  return prefix;
}

constexpr int kRankP = 512;                    // top-p alone: the most candidates selected by ranks
constexpr int kTargetCand = 160;               // top-k: tokens expected at or above the bound (C3F: 128..512 tried, 160 best)
// 16 key bits (sign, exponent, 7 mantissa bits) of the bound: within 2^-7
// of the exact maximum, for 8 barriers instead of 16
constexpr int kBoundPasses = 2;

// Exact thresholds among the n candidates in sh.ck after sorting them
// (largest first): the top-k key (the k-th), the kept set's end, then the
// top-p key from fixed-point mass prefixes.  Returns the smallest kept key.
__device__ __forceinline__ uint32_t sorted_thresholds(FiltShared& sh, int n, float c, float mc, bool use_k, int topk,
                                                      bool use_p, float topp, double mass0 = 0.0) {
  const int t = threadIdx.x;
  uint32_t key = sh.ck[0];
  int nk = n;                                  // candidates kept by top-k: keys >= the k-th largest
  if (use_k) {
    key = sh.ck[topk - 1];
    if (t == 0) sh.nk = n;
    __syncthreads();
    for (int i = topk + t; i < n; i += kFThreads)
      if (sh.ck[i] < key && sh.ck[i - 1] >= key) sh.nk = i;
    __syncthreads();
    nk = sh.nk;
  }
  if (use_p) {
    if (t < kWave) mass_prefix(sh, sh.ck, nk, c, mc, topp, use_k ? -1.0 : sh.zrow, mass0);
    __syncthreads();
    key = sh.ck[max(sh.ne - 1, 0)];           // the last token whose mass above stays below the target
  }
  return key;
}

// Exact thresholds among n <= kFThreads unsorted candidates, thread t
// holding candidate t: top-k keeps a candidate with fewer than k larger
// keys (counted over the candidates, four keys a read); top-p then runs over
// the kept set, compacted, each member summing the masses above it and the
// set's total (integers, so the order does not matter); the largest key is
// always kept.  Returns the smallest kept key.
__device__ __forceinline__ uint32_t select_by_rank(FiltShared& sh, int n, float c, float mc, bool use_k, int topk,
                                                   bool use_p, float topp, double mass0 = 0.0) {
  const int t = threadIdx.x;
  if (t < 4) sh.ck[n + t] = 0u;               // below every candidate: pads the last 4-wide read
  __syncthreads();
  const bool mine = t < n;
  const uint32_t kt = mine ? sh.ck[t] : 0u;
  bool kept = mine;
  if (use_k && mine) {
    int rank = 0;
    for (int j = 0; j < n; j += 4) {
      const uint4 q = *(const uint4*)&sh.ck[j];
      rank += (int)(q.x > kt) + (int)(q.y > kt) + (int)(q.z > kt) + (int)(q.w > kt);
    }
    kept = rank < topk;
  }
  if (!use_p) {
    if (kept) atomicMin(&sh.tmin, kt);
    __syncthreads();
    return sh.tmin;
  }
  // the kept set, compacted: keys in tk, masses in cm
  const uint32_t pos = claim_slot(&sh.nkc, kept);
  if (kept) {
    sh.bb.tk[pos] = kt;
    sh.cm[pos] = fixed_mass_d(fmaf(-kval(kt), c, mc));
  }
  __syncthreads();
  const int nk = (int)sh.nkc;
  if (t < nk) {
    const uint32_t ku = sh.bb.tk[t];
    uint64_t above = 0, tot = 0;
    for (int j = 0; j < nk; ++j) {
      const uint32_t kj = sh.bb.tk[j];
      const uint64_t mj = sh.cm[j];
      tot += mj;
      above += (kj > ku) ? mj : 0;
    }
    const double target = topp > 0.f ? (double)topp * (use_k ? (double)tot : sh.zrow) : 0.0;
    // (mass0 = 0: the set holds the row's largest logit, which is always kept)
    if ((mass0 == 0.0 && above == 0) || mass0 + (double)above < target) atomicMin(&sh.tmin, ku);
    if (t == 0) sh.mtot = mass0 + (double)tot;
  }
  __syncthreads();
  return sh.tmin;
}

// The bounded selection of one row; false (block-uniform) when the
// histogram path must run instead.  On success the filtered chunk sums are
// in sh.cs / sh.cb and the threshold key in *tau_key.
template <bool BF>
__device__ __forceinline__ bool bounded_filter(FiltShared& sh, const char* rowp, int V, int ce, float c, float mc,
                                               bool use_k, int topk, bool use_p, float topp, int xs,
                                               const float* segp, int nseg, uint32_t* tau_key) {
  constexpr int epv = BF ? 8 : 4;
  const int t = threadIdx.x;
  if (use_k && topk > 2 * kFThreads) return false;
  const RowSplit sp = split_row<BF>(rowp, V);
  const uint4* vp = (const uint4*)(rowp + (size_t)sp.head * (BF ? 2 : 4));
  constexpr int kRound = kFThreads * kVecPer;  // vectors per round
  const bool seg_lds = segp && nseg <= kCap;   // the segment maxima are in sh.ck (copied at the row's start)
  // Top-k reads only a sample here, the first nva whole vectors: the k-th
  // largest of any subset is at most the row's k-th largest, and a fraction
  // k/kTargetCand of the row leaves about kTargetCand tokens at or above the
  // bound.  Top-p alone reads every vector (a sample could miss the
  // heaviest tokens).  Either way the head and tail elements are left to
  // read 2.  With the row's segment maxima (segp: nseg maxima of disjoint
  // parts of the row, from the row statistics) nothing is read here: the
  // k-th largest of maxima of k disjoint parts is at most the row's k-th
  // largest too, and maxima whose masses reach the target bound top-p as
  // the thread maxima do.
  const int nva = segp ? 0
                  : use_k ? (int)min((int64_t)sp.nvec, max((int64_t)kRound,
                                                            ((int64_t)V * topk / kTargetCand + epv - 1) / epv))
                          : sp.nvec;

  // ---- read 1: every thread's maximum over the sample ----
  // (the first round stays in registers for read 2; with segment maxima it
  // is loaded only if read 2 reads the whole row)
  uint4 w0[kVecPer];
  auto first_round = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) {
      const int vi = u * kFThreads + t;
      w0[u] = vi < sp.nvec ? vp[vi] : make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
    }
  };
  if (!segp) first_round();
  // two maxima per thread, over its even and its odd vectors of each round
  float mxa = -INFINITY, mxb = -INFINITY;
  auto take_max = [&](const uint4(&w)[kVecPer], int) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kVecPer; ++u)
#pragma unroll
      for (int j = 0; j < epv; ++j) {
        if (u & 1) mxb = fmaxf(mxb, vec_elem<BF>(w[u], j));
        else mxa = fmaxf(mxa, vec_elem<BF>(w[u], j));
      }
  };
  if (segp) {
    // top-p alone, or more than kBallotSegs segments: every thread folds the
    // segments t, t + 1024, ... and t + 512, t + 1536, ... (maxima of
    // disjoint parts)
    if (nseg > kBallotSegs || !use_k) {
      for (int i = t; i < nseg; i += 2 * kFThreads) mxa = fmaxf(mxa, seg_lds ? __uint_as_float(sh.ck[i]) : segp[i]);
      for (int i = t + kFThreads; i < nseg; i += 2 * kFThreads)
        mxb = fmaxf(mxb, seg_lds ? __uint_as_float(sh.ck[i]) : segp[i]);
    }
  } else {
    take_max(w0, 0);
    for_rounds(vp, kRound, nva, take_max);
  }
  // ---- the bound: an exact radix select over the maxima's keys ----
  // (by count for top-k: the k-th largest maximum; by mass for top-p alone:
  // the maximum where their mass from the top reaches the target)
  if (t == 0) {
    sh.ncand = 0;
    sh.tmin = 0xFFFFFFFFu;
    sh.nkc = 0;
  }
  const uint32_t ka = fkey(mxa), kb = fkey(mxb);   // no elements: the key of -inf, mass 0
  uint32_t bound;
  if (segp && use_k && nseg <= kBallotSegs) {
    // the topk-th largest segment maximum: wave 0 holds their keys (key 0,
    // below every maximum's, where there is none) and builds, bit by bit
    // from the top, the largest key that at least topk of them reach -- a
    // ballot and a bit count per key slot and bit, no LDS atomics and no
    // barrier until the result
    if (t < kWave) {
      __builtin_amdgcn_s_setprio(3);           // the block's other waves wait for this one
      uint32_t k[kBallotSegs / kWave];
#pragma unroll
      for (int j = 0; j < kBallotSegs / kWave; ++j) {
        const int i = t + j * kWave;
        k[j] = i < nseg ? fkey(__uint_as_float(sh.ck[i])) : 0u;
      }
      uint32_t res = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = res | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < kBallotSegs / kWave; ++j) cnt += (uint32_t)__popcll(__ballot(k[j] >= cand));
        if (cnt >= (uint32_t)topk) res = cand;
      }
      if (t == 0) sh.segb = res;
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    bound = sh.segb;
  } else if (use_k) {
    bound = radix_select_regs<false>(sh, ka, 0ull, kb, 0ull, (uint32_t)topk, 0.0, kBoundPasses);
  } else {
    bound = radix_select_regs<true>(sh, ka, fixed_mass_d(fmaf(-mxa, c, mc)), kb, fixed_mass_d(fmaf(-mxb, c, mc)),
                                    0u, topp > 0.f ? (double)topp * sh.zrow : 0.0, kBoundPasses);
    if (sh.bin < 0) {                          // the maxima do not reach the target mass
      __syncthreads();
      return false;
    }
  }
  bound = max(bound, kKeyNegInf);              // keys below that of -inf are NaN patterns
  const float tf = kval(bound);

  // ---- read 2: the tokens at or above the bound ----
  // (one bit per element of a round; the rare hits are read again by index)
  auto collect = [&](const uint4(&w)[kVecPer], int v0) __attribute__((always_inline)) {
    uint64_t hit = 0;
#pragma unroll
    for (int u = 0; u < kVecPer; ++u)
#pragma unroll
      for (int j = 0; j < epv; ++j) hit |= (uint64_t)(vec_elem<BF>(w[u], j) >= tf) << (u * epv + j);
    if (__any(hit != 0)) {
      uint32_t pos = hit ? atomicAdd(&sh.ncand, (uint32_t)__popcll(hit)) : 0u;
      while (hit) {
        const int b = __builtin_ctzll(hit);
        hit &= hit - 1;
        const int e = elem_index<BF>(sp, v0, b / epv, b % epv);
        if (pos < (uint32_t)kCap) {
          sh.ck[pos] = fkey(round_elem<BF>(w, b));
          sh.bb.ci[pos] = e;
        }
        ++pos;
      }
    }
  };
  // With segment maxima only the segments whose maximum reaches the bound
  // can hold such tokens: those are read (segment g of chunk k: the vectors
  // u * 256 + 8 g + i of the chunk, u < 8, i < 8, as row statistics loads
  // them), 32 segments a round, when there are at most kBins of them.
  bool seg_read = false;
  if (segp) {
    if (t == 0) sh.nsegc = 0;
    __syncthreads();
    for (int i0 = 0; i0 < nseg; i0 += kFThreads) {   // whole waves: claim_slot
      const int i = i0 + t;
      const bool want = i < nseg && (seg_lds ? __uint_as_float(sh.ck[i]) : segp[i]) >= tf;
      const uint32_t pos = claim_slot(&sh.nsegc, want);
      if (want && pos < (uint32_t)kBins) sh.hc[pos] = (uint32_t)i;
    }
    __syncthreads();
    const int nc = uni((int)sh.nsegc);
    seg_read = nc <= kBins;
    if (seg_read) {
      auto collect_seg = [&](const uint4(&w)[kVecPer], int x0, int x1, int x2, int x3) __attribute__((always_inline)) {
        uint64_t hit = 0;
#pragma unroll
        for (int u = 0; u < kVecPer; ++u)
#pragma unroll
          for (int j = 0; j < epv; ++j) hit |= (uint64_t)(vec_elem<BF>(w[u], j) >= tf) << (u * epv + j);
        if (__any(hit != 0)) {
          uint32_t pos = hit ? atomicAdd(&sh.ncand, (uint32_t)__popcll(hit)) : 0u;
          while (hit) {
            const int b = __builtin_ctzll(hit);
            hit &= hit - 1;
            const int u = b / epv;
            const int vi = u == 0 ? x0 : u == 1 ? x1 : u == 2 ? x2 : x3;
            if (pos < (uint32_t)kCap) {
              sh.ck[pos] = fkey(round_elem<BF>(w, b));
              sh.bb.ci[pos] = sp.head + vi * epv + b % epv;
            }
            ++pos;
          }
        }
      };
      for (int r0 = 0; r0 < nc; r0 += kSegRound) {
        uint4 w[kVecPer];
        int x[kVecPer];
#pragma unroll
        for (int u = 0; u < kVecPer; ++u) {
          const int f = u * kFThreads + t;     // 32 segments of 64 vectors
          const int ci = r0 + f / kSegVecs, vs = f % kSegVecs;
          int vi = -1;
          if (ci < nc) {
            const int seg = (int)sh.hc[ci];
            vi = (seg / kSegPerChunk) * kChunkVecs + (vs / kSegRun) * kThreads + (seg % kSegPerChunk) * kSegRun +
                 vs % kSegRun;
            if (vi >= sp.nvec) vi = -1;        // past the row's whole vectors (its tail: read below)
          }
          x[u] = vi;
          w[u] = vi >= 0 ? vp[vi] : make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
        }
        collect_seg(w, x[0], x[1], x[2], x[3]);
      }
    }
  }
  if (!seg_read && sp.nvec > 0) {
    if (segp) first_round();
    for_rounds_pipe(vp, w0, 0, sp.nvec, collect);
  }
  for_singles<BF>(rowp, sp, collect);
  __syncthreads();
  const int n = uni((int)sh.ncand);
  if (n > kCap || n < 1 || (use_k && n < topk)) {
    __syncthreads();
    return false;
  }
  uint32_t key;
  if (n <= kFThreads && (use_k || n <= kRankP)) {
    key = select_by_rank(sh, n, c, mc, use_k, topk, use_p, topp);
  } else {
    int n2 = 2;
    while (n2 < n) n2 <<= 1;
    for (int i = n + t; i < n2; i += kFThreads) {
      sh.ck[i] = 0u;
      sh.bb.ci[i] = -1;
    }
    __syncthreads();
    sort_desc(sh.ck, sh.bb.ci, n2);
    key = sorted_thresholds(sh, n, c, mc, use_k, topk, use_p, topp);
  }

  // ---- filtered chunk sums from the kept candidates ----
  for (int i = t; i < n; i += kFThreads) {
    const uint32_t k = sh.ck[i];
    if (k >= key) {
      const int e = sh.bb.ci[i];
      const unsigned long long m = fixed_mass_d(fmaf(-kval(k), c, mc));
      atomicAdd(&sh.cs[e / ce], m);
      if (e < xs) atomicAdd(&sh.cb[e / ce], m);
    }
  }
  __syncthreads();
  *tau_key = key;
  return true;
}

// the row's chunk partials as filtered sums against M, and its threshold
__device__ __forceinline__ void write_partials(const FiltShared& sh, Partial* pp, int nch, float M, float tau,
                                               float* tau_out) {
  for (int k = threadIdx.x; k < nch; k += kFThreads) {
    const Partial q = pp[k];
    pp[k] = Partial{M, (float)((double)sh.cs[k] / kMassOne), q.idx, (float)((double)sh.cb[k] / kMassOne)};
  }
  if (threadIdx.x == 0) *tau_out = tau;
}

// The threshold by histograms (any top-k / top-p): the coarse histogram, the
// crossing bins, exact selects inside them.  Returns tau.
template <bool BF>
__device__ __forceinline__ float histogram_threshold(FiltShared& sh, const char* rowp, int V, float c, float mc,
                                                     bool use_k, int topk, bool use_p, float topp) {
  const int t = threadIdx.x, lane = t & (kWave - 1);
  // ---- coarse histogram (masses only when top-p needs them) ----
  if (use_p) histogram<BF, true>(sh, rowp, V, c, mc, -1, 0u, sh.hc, sh.hm);
  else histogram<BF, false>(sh, rowp, V, c, mc, -1, 0u, sh.hc, sh.hm);

  float tau = -INFINITY;
  uint32_t kkey = 0;
  int bk = kBins;
  uint64_t mass_bk = 0;          // mass of bin bk at or above the top-k key
  // ---- top-k: the k-th largest logit ----
  if (use_k) {
    if (t < kWave) scan_bins<false>(sh, sh.hc, sh.hm, false, (uint32_t)topk, 0.0);
    __syncthreads();
    bk = sh.bin >= 0 ? sh.bin : kBins - 1;
    const uint32_t need = sh.need;
    __syncthreads();
    if (use_p) {
      kkey = select_in_bin<BF, false, true>(sh, rowp, V, c, mc, bk, 0u, need, 0.0, true);
      mass_bk = sh.amass;
    } else {
      kkey = select_in_bin<BF, false, false>(sh, rowp, V, c, mc, bk, 0u, need, 0.0, false);
    }
    tau = kval(kkey);
  }
  // ---- top-p on the top-k distribution ----
  if (use_p) {
    // the top-k bin counts only its part at or above the top-k key
    if (t == 0 && use_k) {
      sh.hm[bk] = mass_bk;
      for (int b = bk + 1; b < kBins; ++b) {
        sh.hc[b] = 0;
        sh.hm[b] = 0;
      }
    }
    __syncthreads();
    if (t < kWave) {
      // Z = the mass of the kept (top-k) set, by a wave sum of lane totals
      uint64_t z = 0;
      for (int j = 0; j < 4; ++j) z += sh.hm[lane * 4 + j];
      double zt = 0.0;
      for (int l = 0; l < kWave; ++l) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)z, l);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(z >> 32), l);
        zt += (double)(((uint64_t)hi << 32) | lo);
      }
      const double target = topp > 0.f ? (double)topp * zt : 0.0;
      scan_bins<true>(sh, sh.hc, sh.hm, false, 0u, target);
    }
    __syncthreads();
    const int bp = sh.bin;
    const double rem = sh.rem;
    __syncthreads();
    if (bp >= 0) {               // -1: the crossing was never reached (rounding): keep the whole set
      const uint32_t kmin = (use_k && bp == bk) ? kkey : 0u;
      const uint32_t pkey = select_in_bin<BF, true, true>(sh, rowp, V, c, mc, bp, kmin, 0u, rem, false);
      tau = fmaxf(tau, kval(pkey));
    }
  }

  return tau;
}

// The filtered chunk sums of a row whose threshold tau is known, into sh.cs /
// sh.cb (zeroed by the caller).
template <bool BF>
__device__ __forceinline__ void chunk_pass(FiltShared& sh, const char* rowp, int V, int ce, float c, float mc,
                                           float tau, int xs) {
  const int t = threadIdx.x, lane = t & (kWave - 1);
  // ---- filtered chunk partials: per wave and chunk, float sums turned into fixed point ----
  // (explicit rounds: every lane runs every step, so the wave sums see no
  // inactive lanes; elements past V weigh 0, and the chunk of a step is the
  // same for the whole block since chunks are whole rounds of kFThreads)
  {
    float a = 0.f, bl = 0.f;
    int cur = 0;
    for (int base = 0; base < V; base += kFThreads * kUnroll) {
      float x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e = base + u * kFThreads + t;
        x[u] = e < V ? load_x<BF>(rowp, e) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e = base + u * kFThreads + t;
        const int k = (base + u * kFThreads) / ce;
        if (k != cur) {                        // block-uniform
          const float wa = wave_sum(a), wb = wave_sum(bl);
          if (lane == 0) {
            if (wa != 0.f) atomicAdd(&sh.cs[cur], (unsigned long long)((double)wa * kMassOne));
            if (wb != 0.f) atomicAdd(&sh.cb[cur], (unsigned long long)((double)wb * kMassOne));
          }
          a = 0.f;
          bl = 0.f;
          cur = k;
        }
        const float w = (e < V && x[u] >= tau) ? fexp2(fmaf(x[u], c, -mc)) : 0.f;
        a += w;
        bl += (e < xs) ? w : 0.f;
      }
    }
    const float wa = wave_sum(a), wb = wave_sum(bl);
    if (lane == 0) {
      if (wa != 0.f) atomicAdd(&sh.cs[cur], (unsigned long long)((double)wa * kMassOne));
      if (wb != 0.f) atomicAdd(&sh.cb[cur], (unsigned long long)((double)wb * kMassOne));
    }
  }
  __syncthreads();
}

// ---- bracket search (top-p alone, nuclei the maxima cannot bound) ----
//
// The crossing lies in a bracket (dlo, dhi] of d = M*c - x*c.  Each pass
// over the row splits the bracket evenly and names the part where the mass
// from the top reaches the target.  While the bracket holds more than half
// the row, a pass sums per thread, in registers, the masses and counts at
// or below kBJ thresholds; after that, the bracket's tokens are gathered
// per wave and binned into kSB bins, so the cost per element is a test and
// the binning is paid per token.  Once the bracket holds at most kCap
// tokens (or after kBracketPasses passes, or, for bf16 rows, once it can
// hold one value only), one more pass collects them into LDS and sums the
// mass above the bracket; the exact selection then runs on top of that
// mass.  A bracket of tokens that all tie is
// decided without them.  false (block-uniform): the histogram
// path must decide (a crossing past 2^-32 of the maximum, a bracket too
// large, or a float sum that put the crossing outside the bracket).
constexpr int kBracketPasses = 6;
constexpr float kCountSpan = 1024.f;           // a count bracket starts at (-1, kCountSpan] of d
constexpr int kRing = 256;                     // per-wave ring of bracket tokens (in the idle candidate masses)
constexpr int kSB = kBins;                     // bins per sparse pass (in the idle histogram buffers)
static_assert(kSB == 1 << 8, "the bracket search stops at kSB bins of 2^-21 * dhi = 2^-13 * dhi");
static_assert(kFWaves * kRing * sizeof(float) <= kCap * sizeof(uint64_t), "the rings fit in sh.cm");

// a failed bracket search leaves the chunk sums zero for the histogram path
__device__ __forceinline__ void bracket_clear(FiltShared& sh, bool chunk_sums) {
  __syncthreads();
  if (chunk_sums)
    for (int k = threadIdx.x; k < kMaxChunks; k += kFThreads) {
      sh.cs[k] = 0;
      sh.cb[k] = 0;
    }
  __syncthreads();
}

// BY_MASS: top-p alone, the crossing is where the mass from the top reaches
// p * Z.  Otherwise top-k alone (k beyond the bounded selection): the
// crossing is where the count from the top reaches k; the bracket starts at
// (-1, 1024] and the first pass splits it at 8, 32, 128 (the k-th token can
// lie far below the maximum), later passes evenly; no masses are summed
// until the collect pass.
template <bool BF, bool BY_MASS>
__device__ __forceinline__ bool bracket_search(FiltShared& sh, const char* rowp, int V, int ce, float c, float mc,
                                               int topk, float topp, int xs, uint32_t* tau_key, bool* sums) {
  constexpr int epv = BF ? 8 : 4;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  if (BY_MASS ? !(topp > 0.f) : topk < 1) return false;
  const RowSplit sp = split_row<BF>(rowp, V);
  const uint4* vp = (const uint4*)(rowp + (size_t)sp.head * (BF ? 2 : 4));
  // mass in units of the maximum's weight, or the count k
  const double target = BY_MASS ? (double)topp * sh.zrow / kMassOne : (double)topk;
  float dlo = -1.f, dhi = BY_MASS ? kBinSpan : kCountSpan;
  double alo = 0.0;                            // mass (count) of the tokens with d <= dlo
  uint32_t cnt = 0xFFFFFFFFu;
  for (int pass = 0; pass < kBracketPasses && cnt > (uint32_t)kCap; ++pass) {
    const float base = fmaxf(dlo, 0.f);
    int jq;                                    // the sub-bracket where the mass reaches the target
    double aprev;                              // mass of the bracket's tokens below it
    float nlo, nhi;                            // its bounds
    if (cnt > (uint32_t)V / 2) {
      // ---- dense pass (the first): kBJ thresholds, per-thread sums in registers ----
      const float step = (dhi - base) / kBJ;
      float D[kBJ];
#pragma unroll
      for (int q = 0; q < kBJ; ++q) D[q] = (q == kBJ - 1) ? dhi : base + (float)(q + 1) * step;
      if (!BY_MASS && pass == 0) {
        static_assert(kBJ == 4, "the first count pass's thresholds");
        D[0] = 8.f;
        D[1] = 32.f;
        D[2] = 128.f;
      }
      float m[kBJ];
      uint32_t n[kBJ];
#pragma unroll
      for (int q = 0; q < kBJ; ++q) {
        m[q] = 0.f;
        n[q] = 0;
      }
      auto acc = [&](const uint4(&w)[kVecPer], int) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kVecPer; ++u)
#pragma unroll
          for (int j = 0; j < epv; ++j) {
            const float d = fmaf(-vec_elem<BF>(w[u], j), c, mc);
            if (d > dlo && d <= dhi) {           // NaN and -inf logits never pass
              const float e = BY_MASS ? fexp2(-d) : 0.f;
#pragma unroll
              for (int q = 0; q < kBJ; ++q) {
                const bool in = d <= D[q];
                if (BY_MASS) m[q] += in ? e : 0.f;
                n[q] += in ? 1u : 0u;
              }
            }
          }
      };
      for_rounds(vp, 0, sp.nvec, acc);
      for_singles<BF>(rowp, sp, acc);
#pragma unroll
      for (int q = 0; q < kBJ; ++q) {
        const float ws = wave_sum(m[q]);
        const uint32_t ns = wave_sum_u32(n[q]);
        if (lane == 0) {
          sh.wfm[wv][q] = ws;
          sh.wfn[wv][q] = ns;
        }
      }
      __syncthreads();
      if (t < kBJ) {
        double a = 0.0;
        uint32_t b = 0;
        for (int w = 0; w < kFWaves; ++w) {
          a += (double)sh.wfm[w][t];
          b += sh.wfn[w][t];
        }
        sh.bm[t] = a;
        sh.bn[t] = b;
      }
      __syncthreads();
      jq = -1;
      for (int q = kBJ - 1; q >= 0; --q)         // the first threshold whose mass (count) reaches the target
        if (alo + (BY_MASS ? sh.bm[q] : (double)sh.bn[q]) >= target) jq = q;
      aprev = jq > 0 ? (BY_MASS ? sh.bm[jq - 1] : (double)sh.bn[jq - 1]) : 0.0;
      cnt = jq >= 0 ? sh.bn[jq] - (jq > 0 ? sh.bn[jq - 1] : 0u) : 0u;
      nlo = jq > 0 ? D[jq - 1] : dlo;
      nhi = jq >= 0 ? D[jq] : dhi;
    } else {
      // ---- sparse pass: kSB bins ----
      // The wave gathers its bracket tokens' d in a ring in LDS and bins
      // them 64 at a time, one per lane, into its wave pair's kSB bins
      // (fixed-point masses and counts, LDS atomics: order-independent).
      // The ring never holds more than 127 pending of its kRing entries;
      // within a wave, LDS accesses complete in order.
      const float step = (dhi - base) / kSB, inv = step > 0.f ? 1.f / step : 0.f;
      auto thr = [&](int q) __attribute__((always_inline)) {
        return q == kSB - 1 ? dhi : base + (float)(q + 1) * step;
      };
      for (int j = t; j < kHist * kBins; j += kFThreads) {
        (&sh.hb.wc[0][0])[j] = 0;
        (&sh.hb.wm[0][0])[j] = 0;
      }
      __syncthreads();
      uint64_t* wbm = sh.hb.wm[wv >> 1];
      uint32_t* wbn = sh.hb.wc[wv >> 1];
      // one token (d = +inf: none) into the first bin q with d <= thr(q)
      // (the estimate corrected by a step each way); its mass in units of
      // 2^-31 of the weight at d = base (every token has d > base, or
      // d >= 0 > dlo: below 2^32 units)
      auto put = [&](float d) __attribute__((always_inline)) {
        if (d <= dhi) {
          int b = (int)ceilf(fminf(fmaxf((d - base) * inv, 0.f), (float)kSB)) - 1;
          b = min(max(b, 0), kSB - 1);
          if (b < kSB - 1 && d > thr(b)) ++b;
          if (b > 0 && d <= thr(b - 1)) --b;
          if (BY_MASS) atomicAdd(&wbm[b], (unsigned long long)(uint32_t)fexp2(base - d + 31.f));
          atomicAdd(&wbn[b], 1u);
        }
      };
      float* ring = reinterpret_cast<float*>(sh.cm) + wv * kRing;
      uint32_t wr = 0, rd = 0;                 // wave-uniform: tokens written, binned
      auto gather = [&](const uint4(&w)[kVecPer], int) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kVecPer; ++u)
#pragma unroll
          for (int j = 0; j < epv; ++j) {
            const float d = fmaf(-vec_elem<BF>(w[u], j), c, mc);
            const bool in = d > dlo && d <= dhi;
            const uint64_t mask = __ballot(in);
            if (mask) {
              if (in) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                ring[(wr + below) & (kRing - 1)] = d;
              }
              wr += (uint32_t)__popcll(mask);
              if (wr - rd >= (uint32_t)kWave) {
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
                put(ring[(rd + lane) & (kRing - 1)]);
                rd += kWave;
              }
            }
          }
      };
      for_rounds(vp, 0, sp.nvec, gather);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      put(rd + lane < wr ? ring[(rd + lane) & (kRing - 1)] : INFINITY);
      for_singles<BF>(rowp, sp, [&](const uint4(&w)[kVecPer], int) __attribute__((always_inline)) {
        const float d = fmaf(-vec_elem<BF>(w[0], 0), c, mc);   // the single element
        if (d > dlo) put(d);
      });
      __syncthreads();
      if (t < kSB) {                           // block sums of the bins
        uint64_t a = 0;
        uint32_t k = 0;
        for (int h = 0; h < kHist; ++h) {
          a += sh.hb.wm[h][t];
          k += sh.hb.wc[h][t];
        }
        sh.hm[t] = a;
        sh.hc[t] = k;
      }
      __syncthreads();
      if (BY_MASS) {
        const double unit = (double)fexp2(base) * 2147483648.0;   // bin mass units per maximum's weight
        const double need = (target - alo) * unit;
        if (wv == 0) scan_bins<true>(sh, sh.hc, sh.hm, false, 0u, need);
        __syncthreads();
        aprev = (need - sh.rem) / unit;
      } else {
        const uint32_t needc = (uint32_t)(target - alo);         // tokens still to pass, >= 1
        if (wv == 0) scan_bins<false>(sh, sh.hc, sh.hm, false, needc, 0.0);
        __syncthreads();
        aprev = (double)(needc - uni(sh.need));
      }
      jq = uni(sh.bin);
      cnt = jq >= 0 ? sh.hc[jq] : 0u;
      nlo = jq > 0 ? thr(jq - 1) : dlo;
      nhi = jq >= 0 ? thr(jq) : dhi;
    }
    if (jq < 0) {                              // past dhi: beyond 2^-32 of the maximum (1024 log2 units for a count), or rounding
      __syncthreads();
      return false;
    }
    alo += aprev;
    dlo = nlo;
    dhi = nhi;
    // A bf16 bracket that can hold one value only is a tie group: narrower
    // brackets would hold the same tokens.  Nor is a bracket split further
    // once the next pass's bins would be narrower than 2^-21 * dhi (4 to 8
    // ulps of d; kSB such bins span 2^-13 * dhi): the thresholds would no
    // longer separate tokens, and the bracket holds few distinct d values.
    const bool tie = cnt > (uint32_t)kCap &&
                     ((BF && one_bf16_value(dlo, dhi, c, mc)) || !(dhi - fmaxf(dlo, 0.f) >= dhi * 0x1p-13f));
    __syncthreads();                           // the sums and bins are written again by the next pass
    if (tie) break;
  }

  // ---- collect: the bracket's tokens, the mass above it, the bracket's key range ----
  if (t == 0) {
    sh.ncand = 0;
    sh.bkmin = 0xFFFFFFFFu;
    sh.bkmax = 0u;
    sh.tmin = 0xFFFFFFFFu;                     // the selection's state
    sh.nkc = 0;
  }
  __syncthreads();
  // Without a proposal split (xs < 0) the pass also sums, per chunk, the
  // mass above the bracket (into sh.cs: always kept) and inside it (into
  // sh.cb, kept whole only when the bracket is one value).  A round of
  // vectors spans exactly one chunk's length, so it touches chunks k0 and
  // k0 + 1 only (k0 + 1 when the row does not start on 16 bytes).
  static_assert(kFThreads * kVecPer * 16 == kChunkBytes, "a round of vectors is one chunk long");
  const bool chunk_sums = xs < 0;
  float above = 0.f, inside = 0.f;
  uint32_t nabove = 0;                         // tokens above the bracket (d <= dlo)
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
  auto collect = [&](const uint4(&w)[kVecPer], int v0) __attribute__((always_inline)) {
    uint64_t hit = 0;
    float ra[2] = {0.f, 0.f}, ri[2] = {0.f, 0.f};   // this round's sums, chunks k0 and k0 + 1
    const int eb = v0 >= 0 ? sp.head + v0 * epv : -1 - v0;
    const int k0 = eb / ce;
#pragma unroll
    for (int u = 0; u < kVecPer; ++u)
#pragma unroll
      for (int j = 0; j < epv; ++j) {
        const float x = vec_elem<BF>(w[u], j);
        const float d = fmaf(-x, c, mc);
        const bool up = elem_index<BF>(sp, v0, u, j) >= (k0 + 1) * ce;
        if (d <= dlo) {
          const float e = fexp2(-d);
          above += e;
          ra[up] += e;
          ++nabove;
        } else if (d <= dhi) {
          hit |= 1ull << (u * epv + j);
          const float e = fexp2(-d);
          inside += e;
          ri[up] += e;
          const uint32_t k = fkey(x);
          kmn = min(kmn, k);
          kmx = max(kmx, k);
        }
      }
    if (chunk_sums) {
      if (v0 >= 0) {                           // every lane of the wave is here: wave sums, one atomic each
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float wa = wave_sum(ra[h]), wi = wave_sum(ri[h]);
          if (lane == 0 && k0 + h < kMaxChunks) {
            if (wa != 0.f) atomicAdd(&sh.cs[k0 + h], (unsigned long long)((double)wa * kMassOne));
            if (wi != 0.f) atomicAdd(&sh.cb[k0 + h], (unsigned long long)((double)wi * kMassOne));
          }
        }
      } else {                                 // a single element (head or tail): its own atomics
        if (ra[0] != 0.f) atomicAdd(&sh.cs[k0], (unsigned long long)((double)ra[0] * kMassOne));
        if (ri[0] != 0.f) atomicAdd(&sh.cb[k0], (unsigned long long)((double)ri[0] * kMassOne));
      }
    }
    if (__any(hit != 0)) {
      uint32_t pos = hit ? atomicAdd(&sh.ncand, (uint32_t)__popcll(hit)) : 0u;
      while (hit) {
        const int b = __builtin_ctzll(hit);
        hit &= hit - 1;
        const int e = elem_index<BF>(sp, v0, b / epv, b % epv);
        if (pos < (uint32_t)kCap) {
          sh.ck[pos] = fkey(round_elem<BF>(w, b));
          sh.bb.ci[pos] = e;
        }
        ++pos;
      }
    }
  };
  for_rounds(vp, 0, sp.nvec, collect);
  for_singles<BF>(rowp, sp, collect);
  {
    const float wa = wave_sum(above), wi = wave_sum(inside);
    const uint32_t wn = wave_sum_u32(nabove);
    const uint32_t wmn = (uint32_t)wave_min_i((int)(kmn ^ 0x80000000u)) ^ 0x80000000u;   // unsigned min
    const uint32_t wmx = (uint32_t)wave_max_i((int)(kmx ^ 0x80000000u)) ^ 0x80000000u;   // unsigned max
    if (lane == 0) {
      sh.wfm[wv][0] = wa;
      sh.wfm[wv][1] = wi;
      sh.wfn[wv][0] = wn;
      atomicMin(&sh.bkmin, wmn);
      atomicMax(&sh.bkmax, wmx);
    }
  }
  __syncthreads();
  if (t == 0) {
    double a = 0.0, b = 0.0;
    uint32_t na = 0;
    for (int w = 0; w < kFWaves; ++w) {
      a += (double)sh.wfm[w][0];
      b += (double)sh.wfm[w][1];
      na += sh.wfn[w][0];
    }
    sh.bm[0] = a * kMassOne;                   // fixed-point units from here on
    sh.bm[1] = b * kMassOne;
    sh.bn[0] = na;
  }
  __syncthreads();
  const double A = sh.bm[0], B = sh.bm[1], tgt = BY_MASS ? (double)topp * sh.zrow : 0.0;
  const int n = uni((int)sh.ncand);
  const int nab = uni((int)sh.bn[0]);
  // the float sums (the counts) must put the crossing inside the bracket
  if (n < 1 || (BY_MASS ? (A >= tgt || A + B < tgt) : (nab >= topk || nab + n < topk))) {
    bracket_clear(sh, chunk_sums);
    return false;
  }
  uint32_t key;
  const bool single = sh.bkmin == sh.bkmax;
  if (n > kCap) {
    if (!single) {                             // too many distinct values to select among
      bracket_clear(sh, chunk_sums);
      return false;
    }
    key = sh.bkmin;                            // one value: kept, since the mass above it is below the target
  } else {
    if (n <= kFThreads && (!BY_MASS || n <= kRankP)) {
      key = BY_MASS ? select_by_rank(sh, n, c, mc, false, 0, true, topp, A)
                    : select_by_rank(sh, n, c, mc, true, topk - nab, false, 0.f);
    } else {
      int n2 = 2;
      while (n2 < n) n2 <<= 1;
      for (int i = n + t; i < n2; i += kFThreads) {
        sh.ck[i] = 0u;
        sh.bb.ci[i] = -1;
      }
      __syncthreads();
      sort_desc(sh.ck, sh.bb.ci, n2);
      key = BY_MASS ? sorted_thresholds(sh, n, c, mc, false, 0, true, topp, A)
                    : sorted_thresholds(sh, n, c, mc, true, topk - nab, false, 0.f);
    }
    __syncthreads();
    // the exact sums must agree: something kept, and the crossing inside
    if (key == 0xFFFFFFFFu || (BY_MASS && !(sh.mtot >= tgt))) {
      bracket_clear(sh, chunk_sums);
      return false;
    }
  }
  *sums = chunk_sums;
  if (chunk_sums) {
    // the kept part of the bracket joins the mass above it: all of it for a
    // single value, else the kept candidates' own masses
    if (single) {
      for (int k = t; k < kMaxChunks; k += kFThreads) {
        sh.cs[k] += sh.cb[k];
        sh.cb[k] = 0;
      }
    } else {
      for (int k = t; k < kMaxChunks; k += kFThreads) sh.cb[k] = 0;
      __syncthreads();
      for (int i = t; i < n; i += kFThreads) {
        const uint32_t k = sh.ck[i];
        if (k >= key) {
          const int e = sh.bb.ci[i];
          atomicAdd(&sh.cs[e / ce], (unsigned long long)fixed_mass_d(fmaf(-kval(k), c, mc)));
        }
      }
    }
    __syncthreads();
  }
  *tau_key = key;
  return true;
}

// ---- value table and band (bf16 rows of at most kVTMaxChunks chunks) ----
//
// A bf16 row takes few distinct values where the thresholds can fall (128
// per binade), and every token of one value weighs the same: a value's
// fixed-point mass is its count times one token's, exactly.  The counts
// live in an LDS hash table keyed by the 16-bit pattern (Fibonacci hashing
// with a 24-bit multiply, linear probing, a slot claimed by
// compare-and-swap; per slot 16-bit counts per chunk, two chunks a word,
// laid out [chunk pair][slot]).  Every counted token costs LDS atomics, so
// only a band of values around the crossing is counted in full:
//   1. a sample read (the first 128 bytes of every 2 KB: 1/kVTSample of the
//      row, whole cache lines) counts each value's tokens; two binary
//      searches over the 16-bit keys, one a wave, weigh the sample's values
//      (counts for top-k, masses for top-p) and name a band [l, u] of keys
//      that should hold the crossing: top-k ranks k/kVTSample +-
//      (4 sqrt(k/kVTSample) + 2);
//      top-p the values where the tail below holds (1 - p) Z +- a quarter of
//      it (the tail: Z is known exactly, and the tail is the smaller mass to
//      estimate);
//   2. the full read sums, per chunk, the mass of the tokens above the band
//      (float, per wave, then fixed point, as the bracket search's last pass
//      does) and counts those above it; tokens in the band are counted per
//      value and chunk; tokens below are dropped;
//   3. the crossing must lie inside the band (mass or count above it below
//      the target, with the band's reaching it); the band's values, ranked
//      by wave 0 (up to 64 of them; sorted beyond), then give the threshold
//      exactly by the rules above -- top-k keeps a
//      value with fewer than k tokens strictly above it, top-p alone one
//      whose mass strictly above is below p * Z, the largest always -- and
//      its kept values join the chunk sums as counts times masses.
// -0 and +0 are two patterns with one key: for a single filter the
// threshold key is the same whichever of the two entries a crossing falls
// on, and the key comparison keeps or drops both together.  Top-p counts
// the tokens with d <= kBinSpan only (a crossing past 2^-32 of the maximum's
// weight is left to the other paths), top-k every finite token.  Rows that
// start on 16 bytes only (then a round of vectors is exactly one chunk).
// false (block-uniform), with the chunk sums zero: a table over seven
// eighths full (its read stops at the next round), or the crossing outside
// the band.
constexpr int kVTWords = (int)(sizeof(ValueBufs) / sizeof(uint32_t));
constexpr int kVTMaxChunks = 16;
constexpr int kVTMinSlots = 256;
constexpr int kVTSample = 16;                  // the sample read takes the first 128 bytes of every 2 KB
constexpr uint32_t kVTEmpty = 0xFFFFFFFFu;     // not a 16-bit pattern
constexpr uint32_t kVTGolden = 40503u;         // 2^16 / golden ratio
static_assert(kChunkBytes / 2 == 1 << 14, "a bf16 token's chunk is its index >> 14");
static_assert(kFThreads * kVecPer * 8 == 1 << 14, "a round of bf16 vectors is one chunk long");

// the slot of pattern r whose home slot h held cur != r: probe on, claiming
// an empty slot; kVTEmpty (and the overflow flag set) when the table is full
__device__ __forceinline__ uint32_t vt_probe(FiltShared& sh, uint32_t* keys, uint32_t r, uint32_t h, uint32_t cur,
                                             uint32_t smask, uint32_t limit) {
  for (uint32_t steps = 0; cur != r;) {
    if (cur == kVTEmpty) {
      const uint32_t old = atomicCAS(&keys[h], kVTEmpty, r);
      if (old == kVTEmpty) {                   // this lane claimed the slot
        if (atomicAdd(&sh.vt_n, 1u) >= limit)
          __hip_atomic_store(&sh.vt_over, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return h;
      }
      cur = old;                               // taken meanwhile: by this pattern, or another one
      continue;
    }
    if (++steps > smask) {                     // every slot taken by other patterns
      __hip_atomic_store(&sh.vt_over, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return kVTEmpty;
    }
    h = (h + 1u) & smask;
    cur = __hip_atomic_load(&keys[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  return h;
}

// the 16-bit order-preserving key of a bf16 value (-0 and +0 alike)
__device__ __forceinline__ uint32_t key16(float x) { return fkey(x) >> 16; }

// the bf16 value whose 16-bit order-preserving key is k
__device__ __forceinline__ float val16(uint32_t k) {
  return __uint_as_float(((k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu)) << 16);
}

// the smallest bf16 value x with fmaf(-x, c, mc) <= dhi (d does not increase
// with x), from an estimate and a few steps each way; NaN when not found
__device__ __forceinline__ float bf16_floor_of(float dhi, float c, float mc) {
  float v = __uint_as_float(__float_as_uint((mc - dhi) / c) & 0xFFFF0000u);
  for (int i = 0; i < 4 && !(fmaf(-v, c, mc) <= dhi); ++i) v = bf16_step(v, 1);
  for (int i = 0; i < 4 && fmaf(-bf16_step(v, -1), c, mc) <= dhi; ++i) v = bf16_step(v, -1);
  if (!(fmaf(-v, c, mc) <= dhi) || fmaf(-bf16_step(v, -1), c, mc) <= dhi) return NAN;
  return v;
}

template <bool BY_P>
__device__ __forceinline__ bool value_filter(FiltShared& sh, const char* rowp, int V, int nch, float c, float mc,
                                             int topk, float topp, uint32_t* tau_key) {
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int W = (nch + 1) >> 1;                // count words per slot
  int S = 1024, lg = 10;                       // slots: the most that fit with their counts
  while (S * (1 + W) > kVTWords) {
    S >>= 1;
    --lg;
  }
  const RowSplit sp = split_row<true>(rowp, V);
  if (nch > kVTMaxChunks || S < kVTMinSlots || sp.head != 0 || sp.nvec < kFThreads ||
      (BY_P ? !(topp > 0.f) : topk < 1))
    return false;
  // top-p counts the tokens at or above xw (d <= kBinSpan), top-k the finite ones
  const float xw = BY_P ? bf16_floor_of(kBinSpan, c, mc) : -__FLT_MAX__;
  if (!(xw == xw)) return false;               // (NaN: not found)
  const uint32_t smask = (uint32_t)S - 1u, limit = (uint32_t)(S * 7 / 8);
  uint32_t* keys = sh.vt.w;
  uint32_t* cnts = sh.vt.w + S;                // word q of slot h at cnts[q * S + h]
  const uint4* vp = (const uint4*)(rowp + (size_t)sp.head * 2);

  auto clear_table = [&]() __attribute__((always_inline)) {
    for (int i = t; i < S; i += kFThreads) keys[i] = kVTEmpty;
    for (int i = t; i < S * W; i += kFThreads) cnts[i] = 0u;
    if (t == 0) {
      sh.vt_over = 0;
      sh.vt_n = 0;
      sh.vt_na = 0;
      sh.ncand = 0;
    }
    __syncthreads();
  };
  // the slot of pattern r, inserted when new (kVTEmpty: the table is full)
  auto slot = [&](uint32_t r) __attribute__((always_inline)) {
    const uint32_t h = __builtin_amdgcn_ubfe(__umul24(r, kVTGolden), 16 - lg, lg);
    const uint32_t cur = __hip_atomic_load(&keys[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return cur == r ? h : vt_probe(sh, keys, r, h, cur, smask, limit);
  };
  auto over = [&]() __attribute__((always_inline)) {
    return uni(__hip_atomic_load(&sh.vt_over, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0;
  };

  // ---- 1. the sample: the first 128 bytes (8 vectors) of every 2 KB of the row, counts per value ----
  clear_table();
  const int ns = (sp.nvec >> 7) * 8 + min(sp.nvec & 127, 8);
  for (int s0 = 0; s0 < ns; s0 += kFThreads * kVecPer) {
    if (over()) break;
    uint4 w[kVecPer];
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) {
      const int si = s0 + u * kFThreads + t;
      w[u] = si < ns ? vp[(si >> 3) * 128 + (si & 7)] : make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
    }
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) {
      const uint32_t q[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t r = (i & 1) ? (q[i >> 1] >> 16) : (q[i >> 1] & 0xFFFFu);
        if (!(__uint_as_float(r << 16) >= xw)) continue;   // NaN and -inf too
        const uint32_t h = slot(r);
        if (h != kVTEmpty) atomicAdd(&cnts[h], 1u);
      }
    }
  }
  __syncthreads();
  if (uni(sh.vt_over)) {
    __syncthreads();
    return false;
  }

  // ---- 2. the band [l16, u16] from the sample: waves 0 and 1, a binary search over the keys each ----
  // (per slot its key and its weight -- count, or mass against the maximum -- in LDS first)
  float* wf = reinterpret_cast<float*>(sh.cm);
  for (int i = t; i < S; i += kFThreads) {
    const uint32_t r = keys[i];
    const float x = __uint_as_float(r << 16);
    sh.ck[i] = r == kVTEmpty ? 0u : key16(x);
    wf[i] = r == kVTEmpty ? 0.f : (float)cnts[i] * (BY_P ? fexp2(fmaf(x, c, -mc)) : 1.f);
  }
  __syncthreads();
  if (t < 2 * kWave) {
    // (at raised issue priority: the block's other waves wait, while the
    // CU's other blocks stream)
    __builtin_amdgcn_s_setprio(3);
    // waves 0 and 1 search for u and l, each with this lane's slots lane, lane + 64, ... in registers
    // (S <= 1024: at most 16)
    constexpr int kPer = 1024 / kWave;
    uint32_t kr[kPer];
    float wr[kPer];
    float tot = 0.f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = lane + j * kWave;
      kr[j] = i < S ? sh.ck[i] : 0u;
      wr[j] = i < S ? wf[i] : 0.f;
      tot += wr[j];
    }
    tot = wave_sum(tot);
    float tu, tl;                              // weights from the top where u and l are reached
    if (BY_P) {
      // the tail below the crossing holds (1 - p) Z; the band: a quarter of it either way
      const float zt = (float)(sh.zrow / kMassOne), tail = (1.f - topp) * zt, m = 0.25f * tail;
      tu = tot - (tail + m) / kVTSample;
      tl = (tail - m) > 0.f ? tot - (tail - m) / kVTSample : tot * 2.f + 1.f;
    } else {
      const float ks = (float)topk / kVTSample, mk = 4.f * sqrtf(ks) + 2.f;
      tu = ks - mk;
      tl = ks + mk;
    }
    // the largest key k with (weight at or above k) >= the wave's target
    const float tt = t < kWave ? tu : tl;
    uint32_t lo = 0, hi = 0xFFFFu;
    for (int it = 0; it < 16; ++it) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      float sm = 0.f;
#pragma unroll
      for (int j = 0; j < kPer; ++j) sm += kr[j] >= mid ? wr[j] : 0.f;
      sm = wave_sum(sm);
      if (sm >= tt) lo = mid; else hi = mid - 1;
    }
    if (t == 0) sh.vt_u16 = (tu > 0.f && tu <= tot) ? lo : 0xFFFFu;   // reached at once (or never): from the top
    if (t == kWave) sh.vt_l16 = tl <= tot ? lo : 0u;                 // never reached: the band runs to the bottom
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  const uint32_t u16 = uni(sh.vt_u16), l16 = uni(sh.vt_l16);
  const float xu = u16 >= 0xFFFFu ? INFINITY : val16(u16);   // above the band: x > xu
  const float xl = fmaxf(l16 == 0u ? -__FLT_MAX__ : val16(l16), xw);   // in it: xl <= x <= xu

  // ---- 3. the full read: mass (and count) above the band per chunk, the band's values per chunk ----
  clear_table();
  uint32_t na = 0;
  auto band = [&](uint32_t r, int ch) __attribute__((always_inline)) {
    const uint32_t h = slot(r);
    if (h != kVTEmpty) atomicAdd(&cnts[(ch >> 1) * S + h], 1u << ((ch & 1) << 4));
  };
  // A round's vectors.  The next round's loads are issued before this round
  // is counted; every load is issued (indices clamped into the row, so the
  // last round's is issued again), which lets the wait before the counting
  // cover this round's loads only; vectors past the row become NaN when used.
  constexpr int kRound = kFThreads * kVecPer;
  const int last_v0 = ((sp.nvec - 1) / kRound) * kRound;
  auto load_round = [&](int v0, uint4(&dst)[kVecPer]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) dst[u] = vp[min(v0 + u * kFThreads + t, sp.nvec - 1)];
  };
  uint4 w[kVecPer], nx[kVecPer];
  load_round(0, w);
  for (int v0 = 0; v0 < sp.nvec; v0 += kRound) {
    if (over()) break;
    load_round(min(v0 + kRound, last_v0), nx);
    if (v0 == last_v0) {
#pragma unroll
      for (int u = 0; u < kVecPer; ++u)
        if (v0 + u * kFThreads + t >= sp.nvec) w[u] = make_uint4(kNanFill, kNanFill, kNanFill, kNanFill);
    }
    const int k0 = (v0 * 8) >> 14;             // (the row starts on 16 bytes: the round is chunk k0 exactly)
    float ra = 0.f;
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) {
      const uint32_t q[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      uint32_t bits = 0;                       // the vector's tokens in the band
      if (BY_P) {
        // top-p: about a third of a flat row lies above its band, so every token's weight is formed
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = __uint_as_float((i & 1) ? (q[i >> 1] & 0xFFFF0000u) : (q[i >> 1] << 16));
          const bool above = x > xu;
          ra += above ? fexp2(fmaf(x, c, -mc)) : 0.f;
          bits |= (!above && x >= xl) ? (1u << i) : 0u;
        }
      } else {
        // top-k: few tokens lie above the band; their weights only, by their bits
        uint32_t abits = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = __uint_as_float((i & 1) ? (q[i >> 1] & 0xFFFF0000u) : (q[i >> 1] << 16));
          const bool above = x > xu;
          abits |= above ? (1u << i) : 0u;
          bits |= (!above && x >= xl) ? (1u << i) : 0u;
        }
        na += (uint32_t)__builtin_popcount(abits);
        while (abits) {
          const int i = __builtin_ctz(abits);
          abits &= abits - 1u;
          const uint32_t qq = (i >> 1) == 0 ? q[0] : (i >> 1) == 1 ? q[1] : (i >> 1) == 2 ? q[2] : q[3];
          ra += fexp2(fmaf(__uint_as_float((i & 1) ? (qq & 0xFFFF0000u) : (qq << 16)), c, -mc));
        }
      }
      // the sums are formed here, before the band's branch (else each test's mask is kept across it)
      asm volatile("" : "+v"(ra), "+v"(na));
      // a band token's pattern comes from the registers (a load here would wait for the next round's)
      while (bits) {
        const int i = __builtin_ctz(bits);
        bits &= bits - 1u;
        const uint32_t qq = (i >> 1) == 0 ? q[0] : (i >> 1) == 1 ? q[1] : (i >> 1) == 2 ? q[2] : q[3];
        band((i & 1) ? (qq >> 16) : (qq & 0xFFFFu), k0);
      }
      __builtin_amdgcn_sched_barrier(0);       // one vector's tests live at a time (no spilled masks)
    }
    const float wa = wave_sum(ra);               // every lane of the wave is here: a wave sum, one atomic
    if (lane == 0 && wa != 0.f) atomicAdd(&sh.cs[k0], (unsigned long long)((double)wa * kMassOne));
#pragma unroll
    for (int u = 0; u < kVecPer; ++u) w[u] = nx[u];
  }
  for_singles<true>(rowp, sp, [&](const uint4(&w)[kVecPer], int v0) __attribute__((always_inline)) {
    const int e = -1 - v0, ch = e >> 14;
    const float x = vec_elem<true>(w[0], 0);
    if (x > xu) {
      atomicAdd(&sh.cs[ch], (unsigned long long)((double)fexp2(fmaf(x, c, -mc)) * kMassOne));
      if (!BY_P) ++na;
    } else if (x >= xl) {
      band(__float_as_uint(x) >> 16, ch);
    }
  });
  if (!BY_P) {
    const uint32_t wn = wave_sum_u32(na);
    if (lane == 0 && wn) atomicAdd(&sh.vt_na, wn);
  }
  __syncthreads();
  auto fail = [&]() __attribute__((always_inline)) {
    for (int k = t; k < kMaxChunks; k += kFThreads) sh.cs[k] = 0;
    __syncthreads();
    return false;
  };
  if (uni(sh.vt_over)) return fail();

  // ---- 4. the band's values: exact weights from the top, the threshold ----
  int32_t* pay = reinterpret_cast<int32_t*>(sh.cm);
  for (int i = t; i < S; i += kFThreads) {     // whole waves: S is a multiple of 64
    const uint32_t r = keys[i];
    const uint32_t pos = claim_slot(&sh.ncand, r != kVTEmpty);
    if (r != kVTEmpty) {
      sh.ck[pos] = fkey(__uint_as_float(r << 16));
      pay[pos] = i;
    }
  }
  __syncthreads();
  const int n = uni((int)sh.ncand);
  if (n < 1) return fail();
  auto cnt_of = [&](int i) __attribute__((always_inline)) {
    const int h = pay[i];
    uint32_t a = 0;
    for (int q = 0; q < W; ++q) {
      const uint32_t v = cnts[q * S + h];
      a += (v & 0xFFFFu) + (v >> 16);
    }
    return a;
  };
  auto wgt_of = [&](int i) __attribute__((always_inline)) {
    return BY_P ? (uint64_t)cnt_of(i) * fixed_mass_d(fmaf(-kval(sh.ck[i]), c, mc)) : (uint64_t)cnt_of(i);
  };
  const double target = BY_P ? (double)topp * sh.zrow : (double)topk;
  if (n <= kWave) {
    // few values (the usual band): lane i holds value i and sums the weights of the larger ones
    if (t < kWave) {
      uint64_t a0 = 0;                         // above the band: its mass (the chunk sums so far) or its count
      if (BY_P) {
        for (int k = 0; k < nch; ++k) a0 += sh.cs[k];
      } else {
        a0 = sh.vt_na;
      }
      const bool mine = lane < n;
      const uint32_t ki = mine ? sh.ck[lane] : 0u;
      const uint64_t wi = mine ? wgt_of(lane) : 0ull;
      uint64_t before = 0, tot = 0;
      for (int l = 0; l < kWave; ++l) {
        const uint32_t kl = (uint32_t)__builtin_amdgcn_readlane((int)ki, l);
        const uint32_t vl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)wi, l);
        const uint32_t vh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(wi >> 32), l);
        const uint64_t v = ((uint64_t)vh << 32) | vl;
        before += kl > ki ? v : 0ull;
        tot += v;
      }
      const double above = (double)a0;
      const bool ok = above < target && above + (double)tot >= target;
      const bool kept = ok && mine && ((BY_P && a0 == 0 && before == 0) || above + (double)before < target);
      const uint32_t kmin = (uint32_t)wave_min_i((int)((kept ? ki : 0xFFFFFFFFu) ^ 0x80000000u)) ^ 0x80000000u;
      if (lane == 0) sh.vt_tau = kmin == 0xFFFFFFFFu ? 0u : kmin;
    }
  } else {
    int n2 = 2;
    while (n2 < n) n2 <<= 1;
    for (int i = n + t; i < n2; i += kFThreads) {
      sh.ck[i] = 0u;
      pay[i] = -1;
    }
    __syncthreads();
    sort_desc(sh.ck, pay, n2);
    if (t < kWave) {
      const int per = (n + kWave - 1) / kWave;
      const int lo = min(lane * per, n), hi = min(lo + per, n);
      uint64_t a0 = 0;
      if (BY_P) {
        for (int k = 0; k < nch; ++k) a0 += sh.cs[k];
      } else {
        a0 = sh.vt_na;
      }
      uint64_t lw = 0;
      for (int i = lo; i < hi; ++i) lw += wgt_of(i);
      uint64_t before = 0, tot = 0;
      for (int l = 0; l < kWave; ++l) {
        const uint32_t vl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lw, l);
        const uint32_t vh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lw >> 32), l);
        const uint64_t v = ((uint64_t)vh << 32) | vl;
        before += (l < lane) ? v : 0ull;
        tot += v;
      }
      const double above = (double)a0;
      uint32_t kept = 0;
      if (above < target && above + (double)tot >= target) {
        for (int i = lo; i < hi; ++i) {
          kept += ((BY_P && a0 == 0 && i == 0) || above + (double)before < target) ? 1u : 0u;
          before += wgt_of(i);
        }
      }
      const int nk = (int)wave_sum_u32(kept);
      if (lane == 0) sh.vt_tau = nk >= 1 ? sh.ck[nk - 1] : 0u;
    }
  }
  __syncthreads();
  const uint32_t tk = uni(sh.vt_tau);
  if (tk == 0u) return fail();

  // ---- the band's kept values join the chunk sums: counts times masses ----
  for (int i = t; i < S; i += kFThreads) {
    const uint32_t r = keys[i];
    if (r == kVTEmpty) continue;
    const float x = __uint_as_float(r << 16);
    if (fkey(x) < tk) continue;
    const uint64_t f = fixed_mass_d(fmaf(-x, c, mc));
    for (int q = 0; q < W; ++q) {
      const uint32_t v = cnts[q * S + i];
      if (v & 0xFFFFu) atomicAdd(&sh.cs[2 * q], (unsigned long long)((uint64_t)(v & 0xFFFFu) * f));
      if (v >> 16) atomicAdd(&sh.cs[2 * q + 1], (unsigned long long)((uint64_t)(v >> 16) * f));
    }
  }
  __syncthreads();
  *tau_key = tk;
  return true;
}

// The filter of one row (template on the row's element type).
template <bool BF>
__device__ __forceinline__ void filter_row(const Params& P, FiltShared& sh, Partial* pp, const char* rowp, int nch,
                                           int ce, float c, float mc, float M, bool use_k, int topk, bool use_p,
                                           float topp, int xs, const float* segp, float* tau_out) {
  const int t = threadIdx.x;
  const int V = P.V;
  for (int j = t; j < nch; j += kFThreads) {
    sh.cs[j] = 0;
    sh.cb[j] = 0;
  }
  uint32_t bkey;
  // top-p alone: the 1024 maxima weigh at most 1024 times the largest
  // logit's weight, so a target above that rules the bounded selection out
  const bool hopeless = use_p && !use_k && (double)topp * sh.zrow > 2.0 * kFThreads * kMassOne;
  // With segment maxima, top-p alone bounds from them (no read for the
  // bound); when they fall short of the mass, the bracket search decides.
  if (!hopeless &&
      bounded_filter<BF>(sh, rowp, V, ce, c, mc, use_k, topk, use_p, topp, xs, segp, nch * kSegPerChunk, &bkey)) {
    write_partials(sh, pp, nch, M, kval(bkey), tau_out);
    return;
  }
  if constexpr (BF) {
    if (xs < 0 && use_p != use_k &&
        (use_p ? value_filter<true>(sh, rowp, V, nch, c, mc, 0, topp, &bkey)
               : value_filter<false>(sh, rowp, V, nch, c, mc, topk, 1.f, &bkey))) {
      write_partials(sh, pp, nch, M, kval(bkey), tau_out);
      return;
    }
  }
  if (use_p != use_k) {
    bool sums = false;
    const bool found = use_p ? bracket_search<BF, true>(sh, rowp, V, ce, c, mc, 0, topp, xs, &bkey, &sums)
                             : bracket_search<BF, false>(sh, rowp, V, ce, c, mc, topk, 1.f, xs, &bkey, &sums);
    if (found) {
      if (!sums) chunk_pass<BF>(sh, rowp, V, ce, c, mc, kval(bkey), xs);
      write_partials(sh, pp, nch, M, kval(bkey), tau_out);
      return;
    }
  }
  const float tau = histogram_threshold<BF>(sh, rowp, V, c, mc, use_k, topk, use_p, topp);
  chunk_pass<BF>(sh, rowp, V, ce, c, mc, tau, xs);
  write_partials(sh, pp, nch, M, tau, tau_out);
}

}  // namespace

// The filter of sequence slot (s, r); every return is block-uniform.
__device__ __forceinline__ void filter_slot(const Params& P, FiltShared& sh, int s, int r) {
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const int mk = P.max_k;
  const int K = P.num_draft[s];
  const int md = P.mode[s];
  // everything up to the layout check depends on (s, r) only: block-uniform
  if (K < 0 || K > mk || md == kModeGreedy) return;
  const bool draft = r > mk;
  if (draft ? (md != kModeSample || P.dft == nullptr || r > mk + K) : (r > K)) return;
  const int topk = P.top_k ? P.top_k[s] : 0;
  const float topp = P.top_p ? P.top_p[s] : 1.f;
  const bool use_k = topk > 0 && topk < P.V;
  const bool use_p = topp < 1.f;
  if (!use_k && !use_p) return;
  const float T = P.temperature[s];
  if (!(isfinite(T) && T >= kMinTemp)) return;
  const float c = kLog2eF / T;

  const int nch = draft ? P.nch_d : P.nch_t;
  Partial* pp = P.partials + ((int64_t)s * P.slots + r) * P.nch_max;
  // the row's segment maxima: written by the row statistics' vector path
  // (rows of this matrix 16-byte aligned, V of a vector or more); used for
  // top-k of at most half their number, where they bound it closely, and
  // for top-p alone
  const int bf = draft ? P.d_bf16 : P.t_bf16;
  const bool vec_rows = (draft ? P.d_vec : P.t_vec) && P.V >= (bf ? 8 : 4);
  const float* segp = (P.segmax && vec_rows && (use_k ? 2 * topk <= nch * kSegPerChunk : use_p))
                          ? P.segmax + (pp - P.partials) * kSegPerChunk : nullptr;
  // wave 1 copies them to LDS (sh.ck is not used before the bound) while
  // wave 0 runs the setup below
  if (wv == 1 && segp && nch * kSegPerChunk <= kCap)
    for (int i = lane; i < nch * kSegPerChunk; i += kWave) sh.ck[i] = __float_as_uint(segp[i]);
  if (wv == 0) {
    __builtin_amdgcn_s_setprio(3);           // the block's other waves wait for this one
    // the packed layout (as the scan checks it) and this sequence's offset
    uint32_t tot = 0, bef = 0;
    int oor = 0;
    for (int j = lane; j < P.B; j += kWave) {
      const int k = P.num_draft[j];
      const bool okk = k >= 0 && k <= kLayoutKMax;
      oor |= !okk;
      const uint32_t kk = okk ? (uint32_t)k : 0u;
      tot += kk;
      bef += (j < s) ? kk : 0u;
    }
    tot = wave_sum_u32(tot);
    bef = wave_sum_u32(bef);
    const int bad = __any(oor);
    float m = -INFINITY;
    for (int k = lane; k < nch; k += kWave) m = fmaxf(m, pp[k].m);
    m = wave_max(m);
    // the row's mass against m from its partials (top-p without top-k
    // measures against it), lane sums in chunk order, then lanes in order
    double zl = 0.0;
    if (use_p && !use_k) {
      for (int k = lane; k < nch; k += kWave) {
        const Partial q = pp[k];
        if (q.m > -INFINITY) zl += (double)q.s * (double)fexp2(q.m * c - m * c);
      }
    }
    sh.bb.zl[lane] = zl;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (lane == 0) {
      double z = 0.0;
      for (int l = 0; l < kWave; ++l) z += sh.bb.zl[l];
      sh.ok = !bad && tot == (uint32_t)P.total_draft;
      sh.offd = (int)bef;
      sh.M = m;
      sh.zrow = z * kMassOne;
    }
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  if (!uni(sh.ok)) return;                   // the scan reports the layout
  const float M = uni(sh.M);
  if (!(M > -INFINITY && M < INFINITY)) return;   // an all -inf or non-finite row: the scan reports it
  if (nch > kMaxChunks) return;              // cannot happen within the context's vocabulary limit

  const int offd = uni(sh.offd);
  const int64_t row = draft ? (int64_t)offd + (r - mk - 1) : (int64_t)offd + s + r;
  const char* rowp = (const char*)(draft ? P.dft : P.tgt) + row * (draft ? P.ld_d : P.ld_t) * (bf ? 2 : 4);
  const float mc = M * c;
  const int ce = draft ? P.ce_d : P.ce_t;
  const int xs = (md == kModeStrict && !draft && r < K) ? P.ptok[(int64_t)s * mk + r] : -1;
  float* tau_out = P.tau + (int64_t)s * P.slots + r;
  if (bf)
    filter_row<true>(P, sh, pp, rowp, nch, ce, c, mc, M, use_k, topk, use_p, topp, xs, segp, tau_out);
  else
    filter_row<false>(P, sh, pp, rowp, nch, ce, c, mc, M, use_k, topk, use_p, topp, xs, segp, tau_out);
}

// One block per row of the list row_stats wrote (the filter's rows, the
// flattest first; blocks past its count return at once); four blocks per CU (8 waves
// per SIMD: at most 64 VGPRs).
__global__ void __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) k_filter(Params P) {
  __shared__ FiltShared sh;
  const int i = blockIdx.x;
  if (i >= P.flist[P.n_t + P.n_d]) return;
  const int sl = P.flist[i];
  const int s = sl / P.slots;
  filter_slot(P, sh, s, sl - s * P.slots);
}

hipError_t launch_filter(const Params& p, hipStream_t st, const LaunchEvents* ev) {
  const int rows = p.n_t + p.n_d;
  if (p.B <= 0 || (!p.top_k && !p.top_p) || rows <= 0) return record_empty(st, ev);
  launch_timed(k_filter, dim3(rows), dim3(kFThreads), st, ev, p);
  return hipGetLastError();
}

}  // namespace sv
