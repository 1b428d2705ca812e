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
// One 1024-thread block per used slot of a filtered sequence, after the row
// statistics:
//   1. the row maximum M from the row's chunk partials;
//   2. a coarse histogram of d = M*c - x*c in steps of 1/8 (log2 units; the
//      last of 256 bins also takes everything below 2^-32 of the maximum):
//      counts and masses exp2(x*c - round(M*c)) in 2^-40 fixed point, in
//      per-wave LDS copies with integer atomics (so every sum is exact and
//      the result does not depend on the order of the atomics);
//   3. the bin holding the threshold (by count from the top for top-k, by
//      mass for top-p), its elements compacted into LDS, and an exact radix
//      select over their 32-bit order-preserving keys, 8 bits a pass (a bin
//      larger than the LDS buffer is refined by passes over the row);
//   4. the row's chunk partials rewritten as filtered sums against M (and,
//      for strict-mode target rows, the filtered part below the proposal),
//      and tau stored for the scan and the final draw.
// Every decision on which tokens are kept is a comparison of stored values;
// only the top-p crossing depends on sums (exact here, in fixed point).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"
#include "sv_wave.h"

namespace sv {

namespace {

using namespace wave;

constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / kWave;
constexpr int kBins = 256;
constexpr float kBinScale = 8.f;               // bins per log2 unit below the row maximum
constexpr float kBinSpan = kBins / kBinScale;  // 32: d beyond this falls into the last bin
constexpr int kCap = 4096;                     // candidates held in LDS
constexpr double kMassOne = 1099511627776.0;   // 2^40
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kMinTemp = 1e-6f;
constexpr int kModeSample = 0, kModeGreedy = 1, kModeStrict = 3;
constexpr int kLayoutKMax = 1 << 19;

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// order-preserving 32-bit key of a float (larger float, larger key; no NaN)
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float kval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float load_x(const char* rowp, int e, int bf) {
  return bf ? __uint_as_float((uint32_t)((const uint16_t*)rowp)[e] << 16) : ((const float*)rowp)[e];
}

// coarse bin: monotone non-increasing in x (d is the correctly rounded
// M*c - x*c); NaN and -inf fall into the last bin
__device__ __forceinline__ int coarse_bin(float x, float c, float mc) {
  const float d = fmaf(-x, c, mc);
  return (d < kBinSpan) ? min(kBins - 1, max(0, (int)(d * kBinScale))) : kBins - 1;
}

__device__ __forceinline__ uint64_t fixed_mass(float x, float c, float mc) {
  const float e = fminf(fmaxf(fexp2(fmaf(x, c, -mc)), 0.f), 2.f);   // NaN -> 0
  return (uint64_t)((double)e * kMassOne);
}

struct FiltShared {
  uint32_t wc[kFWaves][kBins];
  uint64_t wm[kFWaves][kBins];
  uint32_t hc[kBins];
  uint64_t hm[kBins];
  uint32_t ck[kCap];
  uint64_t cm[kCap];
  uint32_t rc[kBins];
  uint64_t rm[kBins];
  float ra[kFWaves], rb[kFWaves];
  uint32_t ncand;
  uint32_t kcount;          // candidates of a bin at or above the top-k key
  uint64_t kmass;
  int sel_bin;
  uint32_t need;
  double rem;
  int byte;
  int ok;
  int offd;
  float M;
};

// Candidates: elements of coarse bin `bin` whose key is >= kmin.
struct Cand {
  const char* rowp;
  int bf, V;
  float c, mc;
  int bin;
  uint32_t kmin;
  bool in_lds;
  uint32_t n;
};

__device__ __forceinline__ void compact(FiltShared& sh, Cand& cd) {
  const int t = threadIdx.x;
  if (t == 0) sh.ncand = 0;
  __syncthreads();
  for (int e = t; e < cd.V; e += kFThreads) {
    const float x = load_x(cd.rowp, e, cd.bf);
    const uint32_t k = fkey(x);
    if (coarse_bin(x, cd.c, cd.mc) == cd.bin && k >= cd.kmin) {
      const uint32_t i = atomicAdd(&sh.ncand, 1u);
      if (i < (uint32_t)kCap) {
        sh.ck[i] = k;
        sh.cm[i] = fixed_mass(x, cd.c, cd.mc);
      }
    }
  }
  __syncthreads();
  cd.n = sh.ncand;
  cd.in_lds = cd.n <= (uint32_t)kCap;
}

// Radix select over the candidates from the largest key down: by count
// (the need-th largest key) or by mass (the key where the mass from the top
// first reaches `target`; the smallest candidate key when it never does).
template <bool BY_MASS>
__device__ __forceinline__ uint32_t radix_select(FiltShared& sh, const Cand& cd, uint32_t need, double target) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (t < kBins) {
      sh.rc[t] = 0;
      sh.rm[t] = 0;
    }
    __syncthreads();
    if (cd.in_lds) {
      for (uint32_t i = t; i < cd.n; i += kFThreads) {
        const uint32_t k = sh.ck[i];
        if (k >= cd.kmin && (k & pmask) == prefix) {
          const int by = (k >> shift) & 0xFF;
          atomicAdd(&sh.rc[by], 1u);
          if (BY_MASS) atomicAdd(&sh.rm[by], (unsigned long long)sh.cm[i]);
        }
      }
    } else {
      for (int e = t; e < cd.V; e += kFThreads) {
        const float x = load_x(cd.rowp, e, cd.bf);
        const uint32_t k = fkey(x);
        if (coarse_bin(x, cd.c, cd.mc) == cd.bin && k >= cd.kmin && (k & pmask) == prefix) {
          const int by = (k >> shift) & 0xFF;
          atomicAdd(&sh.rc[by], 1u);
          if (BY_MASS) atomicAdd(&sh.rm[by], (unsigned long long)fixed_mass(x, cd.c, cd.mc));
        }
      }
    }
    __syncthreads();
    if (t == 0) {
      int chosen = -1, last = 0;
      if (BY_MASS) {
        double acc = 0.0;
        for (int by = kBins - 1; by >= 0; --by) {
          if (sh.rc[by] == 0) continue;
          last = by;
          const double m = (double)sh.rm[by];
          if (acc + m >= target) {
            chosen = by;
            break;
          }
          acc += m;
        }
        sh.rem = target - acc;
      } else {
        uint32_t acc = 0;
        for (int by = kBins - 1; by >= 0; --by) {
          if (sh.rc[by] == 0) continue;
          last = by;
          if (acc + sh.rc[by] >= need) {
            chosen = by;
            break;
          }
          acc += sh.rc[by];
        }
        sh.need = need - acc;
      }
      sh.byte = chosen >= 0 ? chosen : last;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.byte << shift;
    pmask |= 0xFFu << shift;
    if (BY_MASS) target = sh.rem;
    else need = sh.need;
    __syncthreads();
  }
  return prefix;
}

}  // namespace

__global__ void __launch_bounds__(kFThreads) k_filter(Params P) {
  __shared__ FiltShared sh;
  const int r = blockIdx.x, s = blockIdx.y;
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

  const int nch = draft ? P.nch_d : P.nch_t;
  Partial* pp = P.partials + ((int64_t)s * P.slots + r) * P.nch_max;
  if (wv == 0) {
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
    if (lane == 0) {
      sh.ok = !bad && tot == (uint32_t)P.total_draft;
      sh.offd = (int)bef;
      sh.M = m;
    }
  }
  __syncthreads();
  if (!sh.ok) return;                        // the scan reports the layout
  const float M = sh.M;
  if (!(M > -INFINITY && M < INFINITY)) return;   // an all -inf or non-finite row: the scan reports it

  const int64_t row = draft ? (int64_t)sh.offd + (r - mk - 1) : (int64_t)sh.offd + s + r;
  const int bf = draft ? P.d_bf16 : P.t_bf16;
  const char* rowp = (const char*)(draft ? P.dft : P.tgt) + row * (draft ? P.ld_d : P.ld_t) * (bf ? 2 : 4);
  const int V = P.V;
  const float c = kLog2eF / T;
  const float mc = M * c;

  // ---- coarse histogram ----
  for (int j = lane; j < kBins; j += kWave) {
    sh.wc[wv][j] = 0;
    sh.wm[wv][j] = 0;
  }
  __syncthreads();
  for (int e = t; e < V; e += kFThreads) {
    const float x = load_x(rowp, e, bf);
    const int b = coarse_bin(x, c, mc);
    atomicAdd(&sh.wc[wv][b], 1u);
    atomicAdd(&sh.wm[wv][b], (unsigned long long)fixed_mass(x, c, mc));
  }
  __syncthreads();
  if (t < kBins) {
    uint32_t cs = 0;
    uint64_t ms = 0;
    for (int w = 0; w < kFWaves; ++w) {
      cs += sh.wc[w][t];
      ms += sh.wm[w][t];
    }
    sh.hc[t] = cs;
    sh.hm[t] = ms;
  }
  __syncthreads();

  Cand cd{rowp, bf, V, c, mc, 0, 0u, false, 0u};
  float tau = -INFINITY;
  uint32_t kkey = 0;
  int bk = kBins;
  // ---- top-k: the k-th largest logit ----
  if (use_k) {
    if (t == 0) {
      uint32_t cum = 0;
      int b = 0;
      for (; b < kBins - 1; ++b) {
        if (cum + sh.hc[b] >= (uint32_t)topk) break;
        cum += sh.hc[b];
      }
      sh.sel_bin = b;
      sh.need = (uint32_t)topk - cum;
    }
    __syncthreads();
    bk = sh.sel_bin;
    const uint32_t need = sh.need;
    cd.bin = bk;
    cd.kmin = 0u;
    compact(sh, cd);
    kkey = radix_select<false>(sh, cd, need, 0.0);
    tau = kval(kkey);
  }
  // ---- top-p on the top-k distribution ----
  if (use_p) {
    uint64_t Z = 0, mass_bk = 0;
    uint32_t cnt_bk = 0;
    if (use_k) {
      // mass and count of bin bk at or above the top-k key
      if (t == 0) {
        sh.kmass = 0;
        sh.kcount = 0;
      }
      __syncthreads();
      uint64_t mloc = 0;
      uint32_t cloc = 0;
      if (cd.in_lds) {
        for (uint32_t i = t; i < cd.n; i += kFThreads)
          if (sh.ck[i] >= kkey) {
            mloc += sh.cm[i];
            ++cloc;
          }
      } else {
        for (int e = t; e < V; e += kFThreads) {
          const float x = load_x(rowp, e, bf);
          if (coarse_bin(x, c, mc) == bk && fkey(x) >= kkey) {
            mloc += fixed_mass(x, c, mc);
            ++cloc;
          }
        }
      }
      if (mloc) atomicAdd(&sh.kmass, (unsigned long long)mloc);
      if (cloc) atomicAdd(&sh.kcount, cloc);
      __syncthreads();
      mass_bk = sh.kmass;
      cnt_bk = sh.kcount;
    }
    if (t == 0) {
      for (int b = 0; b < kBins; ++b) {
        if (b > bk) break;
        Z += (b == bk) ? mass_bk : sh.hm[b];
      }
      const double target = topp > 0.f ? (double)topp * (double)Z : 0.0;
      double cum = 0.0;
      int bp = -1;
      for (int b = 0; b < kBins && b <= bk; ++b) {
        const uint32_t nb = (b == bk) ? cnt_bk : sh.hc[b];
        if (nb == 0) continue;
        const double mb = (double)((b == bk) ? mass_bk : sh.hm[b]);
        if (cum + mb >= target) {
          bp = b;
          break;
        }
        cum += mb;
      }
      sh.sel_bin = bp;                  // -1: the crossing was never reached (rounding): keep everything
      sh.rem = target - cum;
    }
    __syncthreads();
    const int bp = sh.sel_bin;
    const double rem = sh.rem;
    if (bp >= 0) {
      // candidates of bin bp (at or above the top-k key when bp is the top-k bin, whose candidates
      // may already be in LDS)
      if (!(use_k && bp == bk && cd.in_lds)) {
        cd.bin = bp;
        cd.kmin = (use_k && bp == bk) ? kkey : 0u;
        compact(sh, cd);
      } else {
        cd.kmin = kkey;
      }
      const Cand cp = cd;
      const uint32_t pkey = radix_select<true>(sh, cp, 0u, rem);
      tau = fmaxf(tau, kval(pkey));
    }
  }

  // ---- filtered chunk partials ----
  const int ce = draft ? P.ce_d : P.ce_t;
  const int xs = (md == kModeStrict && !draft && r < K) ? P.ptok[(int64_t)s * mk + r] : -1;
  for (int k = 0; k < nch; ++k) {
    const int e0 = k * ce, e1 = min(V, e0 + ce);
    float a = 0.f, bl = 0.f;
    for (int e = e0 + t; e < e1; e += kFThreads) {
      const float x = load_x(rowp, e, bf);
      const float w = (x >= tau) ? fexp2(fmaf(x, c, -mc)) : 0.f;
      a += w;
      bl += (e < xs) ? w : 0.f;
    }
    a = wave_sum(a);
    bl = wave_sum(bl);
    if (lane == 0) {
      sh.ra[wv] = a;
      sh.rb[wv] = bl;
    }
    __syncthreads();
    if (t == 0) {
      float S = 0.f, Bs = 0.f;
      for (int w = 0; w < kFWaves; ++w) {
        S += sh.ra[w];
        Bs += sh.rb[w];
      }
      const Partial q = pp[k];
      pp[k] = Partial{M, S, q.idx, Bs};
    }
    __syncthreads();
  }
  if (t == 0) P.tau[(int64_t)s * P.slots + r] = tau;
}

hipError_t launch_filter(const Params& p, hipStream_t st) {
  if (p.B <= 0 || (!p.top_k && !p.top_p)) return hipSuccess;
  hipLaunchKernelGGL(k_filter, dim3(p.slots, p.B), dim3(kFThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
