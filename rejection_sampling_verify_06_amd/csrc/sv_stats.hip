// Acceptance statistics and draft-length controllers for gfx950.
//
// Statistics ("5.2 Draft 模型与无模型方案", AIInfraGuide, section 7): every
// call adds its rounds (K proposed, A accepted per sequence) to counters the
// caller keeps on the device -- rounds R, proposed D, accepted C, rounds with
// candidates, fully accepted rounds, rounds not counted, emitted tokens, and
// per position the rounds that proposed it, reached it and accepted it -- and
// a summary kernel turns them into the section's rates (C/D, 1 + C/R,
// coverage, conditional and through-position acceptance) in float64.
//
// Controllers, one per sequence, fed with (K, A) after each round:
//   window          the sliding-window rule of the gitcode.csdn.net tutorial,
//                   section 5.2 动态草稿长度策略;
//   multiplicative  the rule of that tutorial's decoder, section 4.4;
//   optimal-k       the rule of "Speculative Decoding在分布式推理中的应用"
//                   (wmrh.cn), section 三.
// The ratio each one sees is, by default, the tutorial's count of the tokens
// its verifier returns (accepted draft tokens plus the token drawn after a
// rejection, no bonus) over the proposed length, min(A + 1, K) / K (0 when
// K = 0; tutorial sections 4.3 and 4.4); or, on request, A / max(K, 1).
// Rounds with A < 0 were not verified and change nothing.  Decisions are taken in float64 in the rules'
// own order (the window mean sums its entries oldest first), so the lengths
// are exact.
//
// Counter accumulation is one block: sums over the batch use wave ballots and
// DPP reductions into registers, then a fixed-order sum of the waves' rows.
// The block is the only writer of the counters in its launch, so there are no
// atomics and the counts are exact.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"
#include "sv_wave.h"

namespace sv {

namespace {

using namespace wave;

constexpr int kStThreads = 1024;
constexpr int kStWaves = kStThreads / kWave;
constexpr int kSumThreads = 256;
constexpr int kAdWaves = 4;                       // sequences per controller block
constexpr double kBand = 0.1;                     // the rules' dead band around the target

__device__ __forceinline__ uint32_t count_of(bool pred) { return (uint32_t)__popcll(__ballot(pred)); }

// lane l of the wave holds the per-position counters of positions l and l + 64
struct PosAcc {
  uint32_t pr[2], re[2], ac[2];
};

}  // namespace

__global__ void __launch_bounds__(kStThreads) k_stats_accumulate(StatsParams P) {
  __shared__ uint32_t part[kStWaves][kStatsMaxWords];
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  const int mk = P.max_k;
  // the counters' old values are loaded now, so that their latency overlaps the batch's
  const uint64_t old = t < 8 + 3 * mk ? P.counters[t] : 0;   // 8 + 3 * max_k <= 392 < kStThreads
  uint32_t sR = 0, sD = 0, sC = 0, sCand = 0, sFull = 0, sBad = 0;
  PosAcc pa = {{0, 0}, {0, 0}, {0, 0}};
  for (int b0 = 0; b0 < P.B; b0 += kStThreads) {
    const int b = b0 + t;
    const bool in = b < P.B;
    int K = 0, A = -1;
    if (in) {
      K = P.num_draft[b];
      A = P.accepted_len[b];
    }
    const bool ok = in && A >= 0 && K >= 0 && K <= mk && A <= K;
    sR += count_of(ok);
    sCand += count_of(ok && K > 0);
    sFull += count_of(ok && K > 0 && A == K);
    sBad += count_of(in && !ok);
    sD += wave_sum_u32(ok ? (uint32_t)K : 0u);
    sC += wave_sum_u32(ok ? (uint32_t)A : 0u);
    const int kw = wave_max_i(ok ? K : 0);         // positions any round of this wave proposed
    for (int i = 0; i < kw; ++i) {
      const uint32_t pr = count_of(ok && K > i);
      const uint32_t re = count_of(ok && K > i && A >= i);
      const uint32_t ac = count_of(ok && A > i);
      const bool mine = lane == (i & (kWave - 1));
      const int m = i >= kWave;
      pa.pr[0] += (mine && !m) ? pr : 0u;
      pa.pr[1] += (mine && m) ? pr : 0u;
      pa.re[0] += (mine && !m) ? re : 0u;
      pa.re[1] += (mine && m) ? re : 0u;
      pa.ac[0] += (mine && !m) ? ac : 0u;
      pa.ac[1] += (mine && m) ? ac : 0u;
    }
  }
  // every wave writes its whole row
  if (lane < 8) {
    const uint32_t v[8] = {sR, sD, sC, sCand, sFull, sBad, sC + sR, 0u};
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) x = (lane == j) ? v[j] : x;
    part[w][lane] = x;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int i = lane + m * kWave;
    if (i < mk) {
      part[w][8 + i] = pa.pr[m];
      part[w][8 + mk + i] = pa.re[m];
      part[w][8 + 2 * mk + i] = pa.ac[m];
    }
  }
  __syncthreads();
  if (t < 8 + 3 * mk) {
    uint64_t s = old;
    for (int v = 0; v < kStWaves; ++v) s += part[v][t];
    P.counters[t] = s;
  }
}

__global__ void __launch_bounds__(kSumThreads) k_stats_summary(StatsParams P) {
  const int mk = P.max_k;
  const uint64_t* c = P.counters;
  for (int j = threadIdx.x; j < 4 + 2 * mk; j += kSumThreads) {
    uint64_t num, den;
    if (j == 0) {
      num = c[2];
      den = c[1];
    } else if (j == 1) {
      num = c[2];
      den = c[0];
    } else if (j == 2) {
      num = c[3];
      den = c[0];
    } else if (j == 3) {
      num = c[4];
      den = c[3];
    } else if (j < 4 + mk) {
      const int i = j - 4;
      num = c[8 + 2 * mk + i];
      den = c[8 + mk + i];
    } else {
      const int i = j - 4 - mk;
      num = c[8 + 2 * mk + i];
      den = c[8 + i];
    }
    double r = den ? (double)num / (double)den : __builtin_nan("");
    if (j == 1 && den) r = 1.0 + r;                  // mean acceptance length 1 + C / R
    P.summary[j] = r;
  }
}

__global__ void __launch_bounds__(kAdWaves * kWave) k_adapt(AdaptParams P) {
  __shared__ double ring[kAdWaves][kAdaptMaxWindow];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int b = blockIdx.x * kAdWaves + w;
  if (b >= P.B) return;                              // whole waves only; no block barrier below
  const int A = P.accepted_len[b], K = P.num_draft[b];
  int4* hdr = reinterpret_cast<int4*>(P.hdr) + b;
  int4 h = *hdr;                                     // length, count, head, 0
  // the whole ring is loaded with the header (lane j holds slots j, j + 64, ...),
  // so no load waits for the header; slots not in use are never used
  const int W = P.window;
  double* wb = P.win + (int64_t)b * W;
  double v[kAdaptMaxWindow / kWave];
  if (P.kind == 0) {
#pragma unroll
    for (int m = 0; m < kAdaptMaxWindow / kWave; ++m) {
      const int j = lane + m * kWave;
      v[m] = j < W ? wb[j] : 0.0;
    }
  }
  int L = h.x;
  if (A >= 0) {
    const double ratio = P.count == 0 ? (K > 0 ? (double)min(A + 1, K) / (double)K : 0.0)
                                      : (double)A / (double)max(K, 1);
    if (P.kind == 0) {
      int count = h.y, head = h.z, slot;
      if (count < W) {                               // append
        slot = head + count;
        if (slot >= W) slot -= W;
        ++count;
      } else {                                       // append and drop the oldest
        slot = head;
        head = head + 1 == W ? 0 : head + 1;
      }
      // entries in age order (age 0 oldest), the new ratio last
#pragma unroll
      for (int m = 0; m < kAdaptMaxWindow / kWave; ++m) {
        const int j = lane + m * kWave;
        int age = j - head;
        if (age < 0) age += W;
        if (j < W && age < count) ring[w][age] = j == slot ? ratio : v[m];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (count >= P.min_samples) {
        double acc = 0.0;
        for (int j = 0; j < count; ++j) acc += ring[w][j];
        const double avg = acc / (double)count;
        if (avg > P.target + kBand)
          L = min(P.max_k, L + 1);
        else if (avg < P.target - kBand)
          L = max(P.min_k, L - 1);
      }
      if (lane == 0) wb[slot] = ratio;
      h.y = count;
      h.z = head;
    } else if (P.kind == 1) {
      if (ratio > P.target + kBand)
        L = min(P.max_k, (int)((double)L * (1.0 + P.rate)));
      else if (ratio < P.target - kBand)
        L = max(P.min_k, (int)((double)L * (1.0 - P.rate)));
    } else {
      const double a = fmax(ratio, 0.01);
      const double x = a < 1.0 ? log(1.0 / (1.0 - a)) / a : INFINITY;
      const int k = x >= 16.0 ? 16 : max(2, (int)x);
      L = min(k, max(L, 2));
    }
  }
  if (lane == 0) {
    h.x = L;
    *hdr = h;
    P.next_k[b] = L;
  }
}

__global__ void __launch_bounds__(256) k_adapt_reset(AdaptParams P) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= P.B) return;
  reinterpret_cast<int4*>(P.hdr)[b] = make_int4(P.init_k, 0, 0, 0);
  P.next_k[b] = P.init_k;
}

hipError_t launch_stats_accumulate(const StatsParams& p, hipStream_t st) {
  if (p.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_stats_accumulate, dim3(1), dim3(kStThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_stats_summary(const StatsParams& p, hipStream_t st) {
  hipLaunchKernelGGL(k_stats_summary, dim3(1), dim3(kSumThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_adapt(const AdaptParams& p, hipStream_t st) {
  if (p.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_adapt, dim3((p.B + kAdWaves - 1) / kAdWaves), dim3(kAdWaves * kWave), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_adapt_reset(const AdaptParams& p, hipStream_t st) {
  if (p.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_adapt_reset, dim3((p.B + 255) / 256), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
