// N-gram (prompt-lookup) proposer for gfx950: for every sequence, the last n
// token ids of its history are looked up earlier in the same history and the
// tokens that followed the most recent occurrence become the proposal
// ("5.2 Draft 模型与无模型方案", AIInfraGuide, sections 4.1-4.3 and the lookup
// experiment of section 6).  Longer windows win over shorter ones, then the
// most recent occurrence; an occurrence must end before the tail with at
// least one token between (that token starts the proposal), and the proposal
// stops at the tail.  The proposal is deterministic: it is verified as a
// one-hot draft (spec_verify_run with SV_ONEHOT).
//
// One 1024-thread block per sequence.  Write e for the end position of a
// candidate window.  For each e the block counts how many of the last tokens
// match backwards from e (lam(e), at most max_n); window n occurs at e when
// lam(e) >= n, and is valid when e <= L - n - 2.  The block walks e downwards
// in rounds of 8192 positions staged in LDS (coalesced loads, plus the
// max_n - 1 tokens below the round), keeps per thread the highest valid e of
// every window length, and stops after the first round in which the longest
// possible window is found.  Every thread issues all its loads of a round
// before waiting for any, and the next round's loads are issued before the
// current round is searched, so one HBM latency is paid per launch rather
// than one per load; a search that stops early has then read one round it
// did not need.  The kernel is compiled for window limits of 4, 8 and 16 so
// that the per-position loops have fixed trip counts.  Integer work only.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_internal.h"
#include "sv_wave.h"

namespace sv {

namespace {

using namespace wave;

constexpr int kNgThreads = 1024;
constexpr int kNgPer = 8;                          // end positions per thread per round
constexpr int kNgSpan = kNgThreads * kNgPer;       // 8192 end positions per round
constexpr bool kNgPrefetch = true;                 // load the next round while searching this one

template <int MAXN>
struct NgShared {
  int32_t h[kNgSpan + MAXN];         // history[base - (MAXN - 1) .. base + kNgSpan - 1]
  int32_t tail[MAXN];                // tail[i] = history[L - 1 - i]
  int best[kNgThreads / kWave][MAXN + 1];
};

}  // namespace

template <int MAXN>
__global__ void __launch_bounds__(kNgThreads) k_ngram(NgramParams P) {
  __shared__ NgShared<MAXN> sh;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t / kWave;
  const int64_t lo = P.offsets[b], hi = P.offsets[b + 1];
  const bool bad = lo < 0 || hi < lo || hi > P.total_len || hi - lo > 0x7FFFFFFF;
  const int L = bad ? 0 : (int)(hi - lo);
  const int32_t* h = P.history + (bad ? 0 : lo);
  const int nmax = min(P.max_n, (L - 1) / 2);      // a valid window needs 2n + 1 <= L
  const int minn = P.min_n;

  int best[MAXN + 1];                         // highest valid end per window length (-1: none)
#pragma unroll
  for (int n = 0; n <= MAXN; ++n) best[n] = -1;

  if (nmax >= minn) {
    if (t < MAXN) sh.tail[t] = t < nmax ? h[L - 1 - t] : 0;
    const int top = L - minn - 2;                   // the highest end any window may use
    const int bottom = minn - 1;                    // a window of n tokens ends at >= n - 1
    // LDS slot j of a round holds position base - (MAXN - 1) + j; thread t
    // loads slots t + k * kNgThreads and, for t < MAXN - 1, slot kNgSpan + t.
    // All of a round's loads are issued before the first is waited for.
    int32_t v[kNgPer + 1];
    auto load_round = [&](int r_hi) {
      const int lo_pos = r_hi - kNgSpan + 1 - (MAXN - 1);
#pragma unroll
      for (int k = 0; k <= kNgPer; ++k) {
        const int pos = lo_pos + k * kNgThreads + t;
        const bool in = (k < kNgPer || t < MAXN - 1) && pos >= 0 && pos <= r_hi;
        v[k] = in ? __builtin_nontemporal_load(h + pos) : 0;
      }
    };
    load_round(top);
    for (int r_hi = top; r_hi >= bottom; r_hi -= kNgSpan) {
      const int base = r_hi - kNgSpan + 1;          // lowest end of this round (may be < 0)
      __syncthreads();                              // previous round's LDS reads are done
#pragma unroll
      for (int k = 0; k < kNgPer; ++k) sh.h[k * kNgThreads + t] = v[k];
      if (t < MAXN - 1) sh.h[kNgSpan + t] = v[kNgPer];
      __syncthreads();
      if (kNgPrefetch && r_hi - kNgSpan >= bottom) load_round(r_hi - kNgSpan);   // in flight during the search
      int hit_longest = 0;
#pragma unroll
      for (int k = 0; k < kNgPer; ++k) {
        const int e = r_hi - (k * kNgThreads + t);  // thread order: highest ends first
        const int j0 = e - base + (MAXN - 1);       // LDS slot of position e (>= MAXN - 1)
        unsigned match = 0;                         // bit i: position e - i equals tail[i]
#pragma unroll
        for (int i = 0; i < MAXN; ++i)
          match |= (unsigned)((sh.h[j0 - i] == sh.tail[i]) & (i < nmax) & (e - i >= 0)) << i;
        const int lam = e >= bottom ? __builtin_ctz(~match) : 0;   // matching run from e down
#pragma unroll
        for (int n = 1; n <= MAXN; ++n)
          if (n >= minn && n <= lam && e <= L - n - 2 && best[n] < 0) best[n] = e;
        hit_longest |= (lam >= nmax && e <= L - nmax - 2);
      }
      if (__syncthreads_or(hit_longest)) break;     // the longest window cannot be beaten
      if (!kNgPrefetch && r_hi - kNgSpan >= bottom) load_round(r_hi - kNgSpan);
    }
  }

  // block-wide highest end per window length, then the longest window with one
#pragma unroll
  for (int n = 1; n <= MAXN; ++n) {
    const int m = wave_max_i(best[n]);
    if (lane == 0) sh.best[wv][n] = m;
  }
  __syncthreads();
  int win = 0, e_best = -1;
#pragma unroll
  for (int n = 1; n <= MAXN; ++n) {
    int m = -1;
#pragma unroll
    for (int w = 0; w < kNgThreads / kWave; ++w) m = max(m, sh.best[w][n]);
    if (m >= 0) {
      win = n;
      e_best = m;
    }
  }
  // proposal: tokens e_best + 1 .. min(e_best + max_tokens, L - win - 1)
  const int count = win ? min(P.max_tokens, L - win - 1 - e_best) : 0;
  for (int j = t; j < P.max_tokens; j += kNgThreads)
    P.draft[(int64_t)b * P.max_tokens + j] = (j < count) ? h[e_best + 1 + j] : -1;
  if (t == 0) {
    P.num_draft[b] = count;
    if (P.match_n) P.match_n[b] = bad ? -1 : win;
  }
}

hipError_t launch_ngram(const NgramParams& p, hipStream_t st) {
  if (p.B <= 0) return hipSuccess;
  if (p.max_n <= 4) hipLaunchKernelGGL(k_ngram<4>, dim3(p.B), dim3(kNgThreads), 0, st, p);
  else if (p.max_n <= 8) hipLaunchKernelGGL(k_ngram<8>, dim3(p.B), dim3(kNgThreads), 0, st, p);
  else hipLaunchKernelGGL(k_ngram<kNgramMaxN>, dim3(p.B), dim3(kNgThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sv
