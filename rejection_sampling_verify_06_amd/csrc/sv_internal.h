// Internal layout shared by the host library (sv_api.cpp) and the kernels
// (sv_kernels.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

constexpr int kThreads = 256;           // row-statistics blocks: 4 waves of 64
constexpr int kChunkBytes = 32768;      // bytes of one logit row streamed by one row-stats block
constexpr int kSegPerChunk = 32;        // 8-lane groups of a row-stats block: the segments whose maxima it writes
constexpr int kTileElems = 8192;        // elements of a tile of the final draw
constexpr int kMaxK = 128;
constexpr int kMaxTiles = 256;          // => vocab <= 2,097,152
// The final kernel runs one 1024-thread block per sequence when the batch
// alone fills the chip; smaller batches split each sequence's tiles over
// about kSplitTargetBlocks / B blocks, and the last of them to store its tile
// sums draws the token.
constexpr int kFuseMinBatch = 128;
constexpr int kSplitTargetBlocks = 256;

// Row statistics of one chunk of one row: max of the raw logits m, the sum
// s = sum exp2(x*c - round(m*c)), and the lowest index attaining m.
struct Partial {
  float m;
  float s;
  int32_t idx;
  float b;        // strict-mode target rows: the part of s from tokens below the proposal; else 0
};

enum FinalKind : int32_t {
  kFinalDone = 0,         // nothing left for the final-draw kernel
  kFinalResidual = 1,     // w = max(0, p_A - q_A)
  kFinalOnehot = 2,       // w = p_A with the proposed token removed
  kFinalBonus = 3         // w = p_K
};

// What the final draw needs, written by the acceptance scan for every sequence.
struct SeqFinal {
  int32_t kind;
  int32_t A;
  int32_t trow;       // target row of position A
  int32_t drow;       // draft row of position A (kFinalResidual)
  float mct;          // round(M_t * c) of target row A
  float mcd;          // round(M_d * c) of draft row A
  float rq;           // S_t / S_d (residual weights are S_t * max(0, p - q))
  float taut;         // filter threshold of target row A (-inf: no filter); tokens below it weigh 0
  float c;
  float u;            // uniform of the final draw
  int32_t xhat;       // proposed token at A (kFinalOnehot)
  int32_t emit_pos;   // slot of the final token in emitted_tokens
  int32_t s;
  float taud;         // filter threshold of draft row A
  int32_t pad[2];
};

struct Params {
  int32_t B;
  int32_t V;
  int32_t total_draft;
  int32_t max_k;
  int32_t n_t;        // target rows = total_draft + B
  int32_t n_d;        // draft rows streamed = total_draft, or 0 without draft logits
  const void* tgt;
  int64_t ld_t;
  int32_t t_bf16;
  int32_t t_vec;      // rows 16-byte aligned: vector loads allowed
  const void* dft;
  int64_t ld_d;
  int32_t d_bf16;
  int32_t d_vec;
  const int32_t* tokens;
  const int32_t* num_draft;
  const float* temperature;   // never NULL on the device: the host substitutes
  const uint8_t* mode;        // the context's default arrays (1.0, SAMPLE, s)
  const uint32_t* seq_ids;
  uint32_t seed_lo;
  uint32_t seed_hi;
  int32_t* accepted_len;
  int32_t* emitted;
  float* p_at;
  float* q_at;
  int32_t* status;
  // scratch owned by the context, indexed by sequence slot: target position
  // i of sequence s in slot s*slots + i, draft position i in slot
  // s*slots + max_k + 1 + i
  Partial* partials;  // chunk k of slot r at r*nch_max + k
  float* segmax;      // or null: segment j of chunk k of slot r at (r*nch_max + k)*kSegPerChunk + j, the
                      // largest logit of an 8-lane group's elements (written by the vector path only)
  float* xval;        // per slot: the row's logit at its proposed token
  int32_t* ptok;      // [B * max_k]: the proposed tokens, copied by row statistics
  SeqFinal* fin;      // [B]
  float* tilesum;     // [B * ntiles]: tile sums of a split final draw
  uint32_t* fincnt;   // [B]: split final blocks of the sequence that have stored their tile sums
  int32_t nch_t;      // chunks per target row
  int32_t nch_d;      // chunks per draft row
  int32_t ce_t;       // elements per target chunk (32 KB)
  int32_t ce_d;       // elements per draft chunk (32 KB)
  int32_t ntiles;     // tiles per row for the final draw
  int32_t nsplit;     // final-kernel blocks per sequence
  int32_t slots;      // 2 * max_k + 1 slots per sequence
  int32_t nch_max;    // max(nch_t, nch_d): partials per slot
  const int32_t* top_k;   // [B] or NULL: top-k filter (<= 0 or >= V: off)
  const float* top_p;     // [B] or NULL: top-p filter (>= 1 or NaN: off)
  float* tau;             // per slot: the filter threshold (written only for filtered sequences)
  int32_t* order;         // [B]: the filter's sequence order (a permutation, costliest first)
  int32_t* flist;         // [n_t + n_d + 1]: the filter's rows in that order (slot s * slots + r), their
                          // number in the last entry (written by row_stats' order block)
  int32_t order_block;    // 1: row_stats' block 0 writes `order` (filtered calls), its other blocks shift by one
};

// N-gram proposer (sv_ngram.hip).
constexpr int kNgramMaxN = 16;          // longest lookup window

struct NgramParams {
  int32_t B;
  const int32_t* history;   // [total_len]
  const int64_t* offsets;   // [B + 1]
  int64_t total_len;
  int32_t min_n;
  int32_t max_n;
  int32_t max_tokens;
  int32_t* draft;           // [B * max_tokens]
  int32_t* num_draft;       // [B]
  int32_t* match_n;         // [B] or NULL
};

hipError_t launch_ngram(const NgramParams& p, hipStream_t st);

// Optional timing of one launch: the pair is recorded by the dispatch itself
// (hipExtLaunchKernel), so the elapsed time is the kernel's, without the gap
// that separately recorded events add.
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
  uint8_t* launched;   // set to 1 when the pair was recorded by a launch
};

template <typename K, typename... A>
inline void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t st, const LaunchEvents* ev, A... args) {
  if (ev) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev->start, ev->stop, 0, args...);
    *ev->launched = 1;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
  }
}

// a slot with no work: nothing is recorded and the slot reads 0
inline hipError_t record_empty(hipStream_t, const LaunchEvents* ev) {
  if (ev) *ev->launched = 0;
  return hipSuccess;
}

// acceptance statistics and draft-length controllers
constexpr int kStatsMaxK = kMaxK;                       // positions tracked per round
constexpr int kStatsMaxWords = 8 + 3 * kStatsMaxK;
constexpr int kAdaptMaxWindow = 256;

struct StatsParams {
  int B;
  int max_k;
  const int32_t* num_draft;
  const int32_t* accepted_len;
  uint64_t* counters;          // [8 + 3 max_k], accumulated
  double* summary;             // [4 + 2 max_k]
};

struct AdaptParams {
  int B;
  int kind;                    // 0 window, 1 multiplicative, 2 optimal-k
  int min_k, max_k;
  int window, min_samples;
  int count;                   // 0: min(A + 1, K) / K (0 for K = 0); 1: A / max(K, 1)
  double target, rate;
  const int32_t* num_draft;
  const int32_t* accepted_len;
  int32_t* hdr;                // [B][4]: length, count, head, 0
  double* win;                 // [B][window]
  int32_t* next_k;             // [B]
  int init_k;                  // reset only
};

hipError_t launch_stats_accumulate(const StatsParams& p, hipStream_t st);
hipError_t launch_stats_summary(const StatsParams& p, hipStream_t st);
hipError_t launch_adapt(const AdaptParams& p, hipStream_t st);
hipError_t launch_adapt_reset(const AdaptParams& p, hipStream_t st);

// ---- host side shared by the entry points (sv_api.cpp) ----------------------

// Sizes a verify call may use: those of a context, or of one allocation-free call.
struct Caps {
  int32_t max_batch;
  int32_t max_k;
  int64_t max_vocab;
  int64_t max_rows;    // sequence slots: max_batch * (2 * max_k + 1)
  int32_t max_nch;     // chunks per row at the smallest chunk (8192 elements)
  int32_t max_tiles;
};

// Where one call's scratch lives.
struct Scratch {
  Partial* partials;
  float* segmax;       // NULL: no room for the filters' segment maxima
  float* xval;
  float* tau;
  int32_t* order;
  int32_t* flist;
  int32_t* ptok;
  SeqFinal* fin;
  float* tilesum;
  uint32_t* fincnt;
  float* def_temperature;   // defaults for NULL temperature / mode / seq_ids: 1.0, SV_SAMPLE, s
  uint8_t* def_mode;
  uint32_t* def_seq_ids;
};

// Byte offsets of the scratch arrays for the given sizes (256-byte aligned).
struct ScratchLayout {
  size_t o_part, o_xval, o_tau, o_ptok, o_fin, o_tile, o_cnt, o_ord, o_flist, o_seg, bytes;
};

Caps caps_for(int32_t max_batch, int32_t max_k, int64_t max_vocab);
ScratchLayout scratch_layout(int32_t max_batch, int32_t max_k, int64_t max_rows, int32_t max_nch, int32_t max_tiles,
                             bool with_segmax);
Scratch scratch_at(void* base, const ScratchLayout& L, bool with_segmax);
hipError_t fill_defaults(const Scratch& v, int32_t n);
int prepare_call(const char* who, const spec_verify_args* a, const Caps& c, const Scratch& v, struct Params* out);
int launch_call(const struct Params& p, hipStream_t st, hipEvent_t* events, uint8_t* launched);
void set_err(const char* fmt, ...);
int hip_fail(const char* what, hipError_t e);
size_t align_up(size_t x, size_t a);

// The kernels of one verify step, in stream order (the select slot launches
// nothing: a split final draw finishes in its last block).
hipError_t launch_row_stats(const Params& p, hipStream_t st, const LaunchEvents* ev = nullptr);
hipError_t launch_filter(const Params& p, hipStream_t st, const LaunchEvents* ev = nullptr);
hipError_t launch_final(const Params& p, hipStream_t st, const LaunchEvents* ev = nullptr);
hipError_t launch_select(const Params& p, hipStream_t st, const LaunchEvents* ev = nullptr);

}  // namespace sv
