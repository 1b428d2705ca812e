/*
 * spec_verify.h -- C interface of the batched speculative-decoding verify step
 * (accept/reject of draft tokens plus the corrected or bonus draw) on an
 * AMD Instinct MI355X (gfx950).
 *
 * What one call computes, for every sequence s of a batch (K = K_s proposed
 * tokens x_0..x_{K-1}, target logits at K+1 positions, draft logits at K):
 *
 *   p_i = softmax(target_i / T),  q_i = softmax(draft_i / T)
 *       Both logit rows are divided by the temperature before the softmax
 *       (gitcode.csdn.net tutorial, section 4.3).
 *   scan i = 0..K-1: accept x_i iff u_i < min(1, p_i(x_i) / q_i(x_i)),
 *       stop at the first rejection
 *       ("Draft Model（草稿模型）", compassingai.com, section 2
 *       接受-拒绝准则 and the one-step algorithm box under 技术原理).
 *   on a rejection at A: draw from norm(max(0, p_A - q_A))
 *       (same page, section 2; tutorial section 3.2);
 *   if all K are accepted: draw one bonus token from p_K
 *       (same page, the one-step algorithm box).
 *   One round therefore emits between 1 and K+1 tokens.
 *
 * Modes per sequence:
 *   SV_SAMPLE  the rule above.
 *   SV_ONEHOT  deterministic proposal (N-gram / prompt lookup): q is the
 *              one-hot distribution on the proposed token, so x_i is accepted
 *              iff u_i < p_i(x_i), and a rejection draws from p_A with x_A
 *              removed ("5.2 Draft 模型与无模型方案", AIInfraGuide, section 4.3).
 *              No draft logits are read.
 *   SV_GREEDY  strict greedy: accept iff x_i is the argmax of the raw target
 *              logits (lowest index on ties); emit that argmax on a mismatch
 *              and as the bonus.  The temperature is ignored.
 *   SV_STRICT  sample match ("Speculative Decoding在分布式推理中的应用",
 *              wmrh.cn, sections 二 and 三): the target draws its own token
 *              y_i ~ p_i by the inverse CDF with u_i; x_i is accepted iff
 *              y_i = x_i, and on a mismatch y_A is emitted (it is the draw
 *              from p_A with x_A removed, at the point u_A*S minus x_A's mass
 *              when u_A lies above x_A's interval).  All K accepted: bonus
 *              from p_K as above.  Lossless; the acceptance probability is
 *              p_i(x_i).  No draft logits are read.
 *
 * Randomness: u_i and the final draw's uniform come from Philox4x32-10
 * (Salmon et al., SC'11) with key = seed and counter = (position, purpose,
 * seq_id, 0); purpose 0 for u_i at positions 0..K-1, purpose 1 for the final
 * draw at position A (SV_STRICT draws its correction with u_A, purpose 0,
 * and only its bonus with purpose 1); u = (word0 >> 8) * 2^-24.  Results are a pure function
 * of (inputs, seed, seq_ids): any call can be replayed exactly, and a batch
 * split across calls (with global seq_ids) gives the same outputs.
 *
 * Filters (top_k / top_p, optional): top-k and nucleus rejection sampling
 * keep the target's distribution ("Draft Model（草稿模型）", compassingai.com,
 * 常见误读纠偏 误读 4; gitcode.csdn.net tutorial, section 5.4): each used row
 * of a filtered SAMPLE, ONEHOT or STRICT sequence (target and draft alike)
 * keeps the tokens with logit >= tau and is renormalised before the rule
 * above; GREEDY ignores the filter.  top-k: tau is the k-th largest logit
 * (ties at it all kept).  top-p, after top-k: a token is kept iff the mass of
 * the strictly larger tokens is below p (the largest logit always kept).
 * The output then follows the filtered target distribution.  A filtered
 * call runs one more kernel (one block per used row of a filtered sequence)
 * that reads those rows again: whole, or only the parts whose maximum can
 * reach the row's threshold.
 *
 * Final draw: inverse CDF over the unnormalised weights w (residual, one-hot
 * residual or p_K): t = u * sum(w), emit the first token k whose inclusive
 * prefix sum exceeds t; tokens with w = 0 are never emitted.
 *
 * Packed ragged layout (no padding between sequences):
 *   off_d[s] = sum_{j<s} K_j            draft rows / draft_tokens / p,q at proposal
 *   off_t[s] = off_d[s] + s             target rows / emitted_tokens
 *   target row off_t[s]+i judges draft token i; row off_t[s]+K_s is the bonus row.
 *   Logit rows are ld elements apart (ld >= vocab); columns >= vocab are never read.
 *   Logits pointers are aligned to their element size (4 bytes fp32, 2 bf16).
 *
 * Arithmetic: float32 (logits are read as float32 or bfloat16 and widened
 * exactly); exp2-based online max/sum; fixed-order reductions, no float
 * atomics, so repeated calls are bitwise identical.
 *
 * Threading: a context owns device scratch memory; calls that share a context
 * must be ordered on one stream.  Use one context per concurrent stream.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify_ctx spec_verify_ctx;

/* logits element type */
enum { SV_F32 = 0, SV_BF16 = 1 };

/* per-sequence verify mode (values of args->mode[s]) */
enum { SV_SAMPLE = 0, SV_GREEDY = 1, SV_ONEHOT = 2, SV_STRICT = 3 };

/* return codes */
enum {
  SV_OK = 0,
  SV_ERR_INVALID = -1,   /* bad argument; nothing was enqueued */
  SV_ERR_NOMEM = -2,     /* device allocation failed (create / timing_enable only) */
  SV_ERR_HIP = -3,       /* a HIP call failed; see spec_verify_last_error() */
  SV_ERR_CAPACITY = -4   /* the call exceeds the sizes given to spec_verify_create */
};

/* per-sequence status bits (args->status[s]).  Any bit in 1..64 means the
 * sequence was not verified: accepted_len = -1, its emitted slots are -1 and
 * its p/q at proposal are NaN.  Bit 128 is informational. */
enum {
  SV_ST_BAD_LAYOUT = 1,        /* num_draft has a negative entry or does not sum to total_draft (set for every sequence; every output slot is cleared) */
  SV_ST_K_TOO_LARGE = 2,       /* K_s > max_k of the context */
  SV_ST_BAD_MODE = 4,          /* mode[s] not one of SV_SAMPLE, SV_GREEDY, SV_ONEHOT, SV_STRICT */
  SV_ST_BAD_TEMPERATURE = 8,   /* SAMPLE/ONEHOT/STRICT with temperature not finite or below SV_MIN_TEMPERATURE */
  SV_ST_NO_DRAFT_LOGITS = 16,  /* SAMPLE sequence with K_s > 0 but draft_logits == NULL */
  SV_ST_BAD_TOKEN = 32,        /* a proposed token outside [0, vocab) */
  SV_ST_NONFINITE = 64,        /* a used logit row holds NaN or +inf, or is entirely -inf */
  SV_ST_ZERO_RESIDUAL = 128    /* the residual had no mass (rounding only); the token was drawn from p_A instead */
};

/* smallest accepted temperature for SAMPLE/ONEHOT/STRICT (float32 1e-6) */
#define SV_MIN_TEMPERATURE 1e-6f

typedef struct spec_verify_args {
  int32_t batch;               /* B >= 0 (host value); 0 is a no-op */
  int64_t vocab;               /* V >= 1 (host value) */
  int64_t total_draft;         /* sum_s K_s (host value): sizes the grids, must match num_draft */
  int32_t target_dtype;        /* SV_F32 or SV_BF16 */
  int32_t draft_dtype;         /* SV_F32 or SV_BF16 (ignored when draft_logits == NULL) */
  const void* target_logits;   /* device, [total_draft + B][ld_target] */
  int64_t ld_target;           /* elements between target rows, >= vocab */
  const void* draft_logits;    /* device, [total_draft][ld_draft], or NULL if no SV_SAMPLE sequence has K_s > 0 */
  int64_t ld_draft;            /* elements between draft rows, >= vocab */
  const int32_t* draft_tokens; /* device, [total_draft]; may be NULL iff total_draft == 0 */
  const int32_t* num_draft;    /* device, [B], K_s */
  const float* temperature;    /* device, [B], or NULL (= 1.0 for every sequence) */
  const uint8_t* mode;         /* device, [B], or NULL (= SV_SAMPLE for every sequence) */
  const uint32_t* seq_ids;     /* device, [B], or NULL (= s): Philox counter word 2 */
  uint64_t seed;               /* Philox key */
  int32_t* accepted_len;       /* device out, [B]: accepted draft tokens A_s (0..K_s), -1 if not verified */
  int32_t* emitted_tokens;     /* device out, [total_draft + B]: seq s at off_t[s]: x_0..x_{A-1}, y, then -1 */
  float* p_at_proposal;        /* device out, [total_draft] or NULL: p_i(x_i) for every i < K_s (T = 1 for GREEDY) */
  float* q_at_proposal;        /* device out, [total_draft] or NULL: q_i(x_i); 1.0 for ONEHOT and GREEDY */
  int32_t* status;             /* device out, [B] or NULL: SV_ST_* bits */
  const int32_t* top_k;        /* device, [B], or NULL: top-k filter per sequence (<= 0 or >= vocab: off) */
  const float* top_p;          /* device, [B], or NULL: top-p filter per sequence (>= 1 or NaN: off) */
} spec_verify_args;

/* Create a context on HIP device `device` for batches of at most max_batch
 * sequences, K_s <= max_k (1..128) and vocab <= max_vocab.  Allocates the
 * context's device scratch (per-chunk partial row statistics and, for the
 * filters, 32 segment maxima per chunk; per-sequence final-draw records
 * and tile sums; defaults for NULL optional inputs): about 144 bytes per 8192
 * vocabulary entries per row slot, max_batch * (2 * max_k + 1) slots, plus
 * small per-slot and per-sequence arrays (among them the filter's list of
 * rows).  The caller owns every input and output
 * buffer.  Returns SV_OK and sets *out, or an error code (then *out = NULL). */
int spec_verify_create(spec_verify_ctx** out, int device, int32_t max_batch, int32_t max_k, int64_t max_vocab);

/* Enqueue one verify step on `hip_stream` (a hipStream_t; NULL = the null
 * stream).  Validates the host-side arguments first (SV_ERR_INVALID /
 * SV_ERR_CAPACITY: nothing is enqueued); problems that only the device can
 * see are reported per sequence through `status`.  Does not allocate, does
 * not synchronise; outputs are valid once the stream has reached this point.
 * Launches two kernels (three with top_k / top_p): row statistics (one
 * block per 32 KB of every logit row); final (per sequence: the acceptance
 * test, then the sums of the final weights over 8192-element tiles of the
 * row(s) at the stop position and the inverse-CDF search; for batches below
 * 128 a sequence's tiles are spread over several blocks, and the last of
 * them to store its tile sums does the search).  The timing slot "select"
 * is kept for the interface and reads 0. */
int spec_verify_run(spec_verify_ctx* ctx, const spec_verify_args* args, void* hip_stream);

/* ---- allocation-free call --------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as spec_verify_run, without a context.  Its scratch is one array of
 * SV_NOALLOC_SCRATCH_BYTES bytes in the library's device data, which every
 * GPU the library runs on holds until the process ends; it is laid out per
 * call for exactly the call's sizes (about 16 bytes per 32 KB chunk of each
 * of batch * (2 * max_k + 1) row slots, eight times that more with top_k /
 * top_p, plus small per-sequence arrays).  max_k (1..128) plays the part of
 * the context's max_k (K_s > max_k: status SV_ST_K_TOO_LARGE); batch <= 4096.
 * A call that would need more scratch returns SV_ERR_CAPACITY with the
 * needed size in the message; other checks and errors as spec_verify_run.
 * Runs on the calling thread's current device (hip_stream must belong to
 * it).  Allocates nothing; the first call on a device looks up the array's
 * address and writes the defaults for NULL temperature / mode / seq_ids with
 * synchronous copies, so make one call on each device before capturing a
 * graph.  All calls on one GPU share its array and it keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams or threads)
 * race and give undefined results.  No timing hooks. */
#define SV_NOALLOC_SCRATCH_BYTES 67108864
int spec_verify_run_noalloc(const spec_verify_args* args, int32_t max_k, void* hip_stream);

/* Free the context and its device memory.  NULL is accepted. */
void spec_verify_destroy(spec_verify_ctx* ctx);

/* Message of the last failing call on this thread (static storage). */
const char* spec_verify_last_error(void);

/* ---- measurement hooks ---------------------------------------------------
 * spec_verify_timing_enable(ctx, n) makes the next n calls of
 * spec_verify_run time each of its kernel slots with a pair of HIP events
 * that the dispatch itself records (hipExtLaunchKernel), so a slot's time is
 * its kernel's execution, without event gaps (n = 0 turns it off; events are
 * created here, never inside run).  spec_verify_timing_read waits for those events and
 * returns the number of recorded calls and, per slot, the summed elapsed
 * milliseconds (ms_per_kernel has SV_NUM_KERNELS entries: row statistics,
 * filter, final, select; a slot whose kernel was not launched reads 0),
 * then resets the record. */
#define SV_NUM_KERNELS 4
int spec_verify_timing_enable(spec_verify_ctx* ctx, int32_t max_calls);
int spec_verify_timing_read(spec_verify_ctx* ctx, int32_t* calls, double* ms_per_kernel);

/* ---- N-gram (prompt-lookup) proposer -------------------------------------
 * "5.2 Draft 模型与无模型方案" (AIInfraGuide), sections 4.1-4.3 and the lookup
 * experiment of section 6: for each sequence, the last n token ids of its
 * history are looked up earlier in the same history and the tokens that
 * followed become a deterministic proposal, which the target then verifies
 * as a one-hot draft (spec_verify_run with mode SV_ONEHOT).
 *
 * With history h of length L and window n, a start s is an occurrence when
 * h[s .. s+n-1] equals h[L-n .. L-1] and s + n < L - n (the occurrence ends
 * before the tail and at least one token follows it outside the tail).  The
 * chosen occurrence has the largest n in [min_n, max_n], then the largest s;
 * the proposal is h[s+n .. min(s+n+max_tokens, L-n) - 1] (never copied from
 * the tail).  No occurrence: an empty proposal.
 *
 * All pointers are device pointers owned by the caller.
 *   history        [total_len] int32 token ids; sequence b is
 *                  history[hist_offsets[b] .. hist_offsets[b+1] - 1]
 *   hist_offsets   [batch + 1] int64
 *   total_len      host value: the length of `history`; bounds every read
 *   min_n, max_n   1 <= min_n <= max_n <= SV_NGRAM_MAX_N
 *   max_tokens     1 .. SV_NGRAM_MAX_TOKENS
 *   draft_tokens   out [batch * max_tokens] int32: sequence b's proposal at
 *                  b * max_tokens, -1 after it
 *   num_draft      out [batch] int32: proposal length (0: none)
 *   match_n        out [batch] int32 or NULL: the window that matched (0:
 *                  none; -1: sequence b's offsets are out of order or outside
 *                  total_len, and nothing of it was read)
 * spec_verify_ngram_propose checks the host-side values (SV_ERR_INVALID:
 * nothing is enqueued), enqueues one kernel on `hip_stream` (one block per
 * sequence), allocates nothing and does not synchronise.  It needs no
 * context. */
#define SV_NGRAM_MAX_N 16
#define SV_NGRAM_MAX_TOKENS 128
typedef struct spec_verify_ngram_args {
  int32_t batch;
  const int32_t* history;
  const int64_t* hist_offsets;
  int64_t total_len;
  int32_t min_n;
  int32_t max_n;
  int32_t max_tokens;
  int32_t* draft_tokens;
  int32_t* num_draft;
  int32_t* match_n;
} spec_verify_ngram_args;
int spec_verify_ngram_propose(const spec_verify_ngram_args* args, void* hip_stream);

/* sizeof(spec_verify_ngram_args) as compiled into the library. */
int64_t spec_verify_ngram_args_size(void);

/* ---- acceptance statistics ------------------------------------------------
 * "5.2 Draft 模型与无模型方案" (AIInfraGuide), section 7: over R verify rounds
 * that proposed D draft tokens of which C were accepted, the draft acceptance
 * rate is C / D and the mean acceptance length 1 + C / R (a complete round
 * also commits its corrected or bonus token); candidate coverage is the
 * share of rounds that had any candidate; per position, the conditional
 * acceptance rate (among rounds that reached the position) differs from the
 * rate of being accepted all the way through it.
 *
 * A round is one sequence of one verify call: K = num_draft[s], A =
 * accepted_len[s].  spec_verify_stats_accumulate ADDS one call's rounds to
 * `stats`, device uint64 [SV_STATS_WORDS(max_k)], owned by the caller, who
 * zeroes it to start an observation window (with a fill kernel or a copy;
 * the library never clears it):
 *   [0] R rounds counted             [4] rounds with K > 0 and A = K
 *   [1] D = sum K                    [5] rounds not counted: A < 0 (not
 *   [2] C = sum A                        verified), K outside 0..max_k, A > K
 *   [3] rounds with K > 0            [6] emitted tokens sum (A + 1)   [7] 0
 *   [8 + i]            rounds with K > i                 (proposed at i)
 *   [8 + max_k + i]    rounds with K > i and A >= i      (reached i)
 *   [8 + 2 max_k + i]  rounds with A > i                 (accepted at i)
 * Counts are exact (integer sums, no atomics).  num_draft and accepted_len
 * are device int32 [batch] (for instance the verify call's own arrays, on
 * the same stream).  One block of the kernel walks the batch: meant for the
 * batch of one decode step.
 *
 * spec_verify_stats_summary writes device float64 [SV_STATS_SUMMARY_WORDS]:
 *   [0] C / D   [1] 1 + C / R   [2] [3] / R (coverage)   [3] [4] / [3]
 *   [4 + i]          conditional acceptance at i: accepted_i / reached_i
 *   [4 + max_k + i]  accepted through i:          accepted_i / proposed_i
 * NaN where the denominator is 0; each value is one correctly rounded
 * float64 division of the counts (plus 1.0 for [1]).
 * Both enqueue one kernel on `hip_stream`, allocate nothing and do not
 * synchronise; SV_ERR_INVALID (nothing enqueued) for max_k outside
 * 1..SV_STATS_MAX_K, batch < 0 or a missing buffer. */
#define SV_STATS_MAX_K 128
#define SV_STATS_WORDS(max_k) (8 + 3 * (max_k))
#define SV_STATS_SUMMARY_WORDS(max_k) (4 + 2 * (max_k))
int spec_verify_stats_accumulate(int32_t batch, int32_t max_k, const int32_t* num_draft,
                                 const int32_t* accepted_len, uint64_t* stats, void* hip_stream);
int spec_verify_stats_summary(int32_t max_k, const uint64_t* stats, double* summary, void* hip_stream);

/* ---- draft-length controllers ---------------------------------------------
 * One controller per sequence slot, fed after each round with (K, A) and
 * giving the proposal length of the next round; a round with A < 0 changes
 * nothing.  The ratio a controller sees depends on `count`:
 *   SV_ADAPT_COUNT_EMITTED (0, the pages' count)  min(A + 1, K) / K, and 0
 *       when K = 0: the tutorial's verifier returns the accepted draft
 *       tokens plus the token drawn after a rejection, without a bonus token
 *       (gitcode.csdn.net tutorial, section 4.3 验证器实现), and its decoder
 *       feeds len(accepted_tokens) / draft_len (section 4.4 完整的解码器);
 *       "Speculative Decoding在分布式推理中的应用" (wmrh.cn), section 三,
 *       counts the resampled token the same way.
 *   SV_ADAPT_COUNT_DRAFT_ONLY (1)  A / max(K, 1): accepted draft tokens only.
 * Decisions are taken in float64.
 *   SV_ADAPT_WINDOW          keep the last `window` ratios; once at least
 *       `min_samples` are held, their mean (summed oldest first) above
 *       target + 0.1 lengthens by one, below target - 0.1 shortens by one,
 *       within [min_k, max_k] (tutorial, section 5.2 动态草稿长度策略; the
 *       page's defaults are window 100, min_samples 10, target 0.7,
 *       length 5 in 1..10).
 *   SV_ADAPT_MULTIPLICATIVE  above target + 0.1 the length L becomes
 *       min(max_k, int(L (1 + rate))), below target - 0.1
 *       max(min_k, int(L (1 - rate))); int truncates (tutorial, section
 *       4.4; defaults target 0.7, rate 0.1, lengths 1..5).
 *   SV_ADAPT_OPTIMAL_K       a = max(ratio, 0.01), k* = floor(ln(1/(1-a))/a)
 *       (unbounded at a = 1), L becomes min(clamp(k*, 2, 16), max(L, 2));
 *       min_k, max_k, window and rate are not used (wmrh.cn, section 三,
 *       adapt_draft_length).
 *
 * state: device memory owned by the caller, SV_ADAPT_STATE_BYTES(batch,
 * window) bytes, 16-byte aligned: int32 [batch][4] {length, count, head, 0},
 * then float64 [batch][window] ratio rings.  spec_verify_adapt_reset sets
 * every length to init_k and empties the rings (call it first, and again
 * after changing kind, window or count); spec_verify_adapt reads num_draft and
 * accepted_len (device int32 [batch]), updates the state and writes next_k
 * (device int32 [batch]; also for unchanged lengths).  Sequence b always
 * uses slot b.  Each call enqueues one kernel on `hip_stream`, allocates
 * nothing and does not synchronise; SV_ERR_INVALID (nothing enqueued) for a
 * bad kind or count, bounds outside 1 <= min_k <= max_k <= SV_ADAPT_MAX_LENGTH,
 * window outside 1..SV_ADAPT_MAX_WINDOW or min_samples < 1 (window kind),
 * target or rate outside [0, 1], init_k outside 1..SV_ADAPT_MAX_LENGTH, or a
 * missing or misaligned buffer. */
enum { SV_ADAPT_WINDOW = 0, SV_ADAPT_MULTIPLICATIVE = 1, SV_ADAPT_OPTIMAL_K = 2 };
enum { SV_ADAPT_COUNT_EMITTED = 0, SV_ADAPT_COUNT_DRAFT_ONLY = 1 };
#define SV_ADAPT_MAX_WINDOW 256
#define SV_ADAPT_MAX_LENGTH 4096
#define SV_ADAPT_STATE_BYTES(batch, window) ((int64_t)(batch) * (16 + 8 * (int64_t)(window)))
typedef struct spec_verify_adapt_args {
  int32_t batch;
  int32_t kind;
  int32_t min_k;
  int32_t max_k;
  int32_t window;
  int32_t min_samples;
  int32_t count;               /* SV_ADAPT_COUNT_EMITTED or SV_ADAPT_COUNT_DRAFT_ONLY */
  double target;
  double rate;
  const int32_t* num_draft;
  const int32_t* accepted_len;
  void* state;
  int32_t* next_k;
} spec_verify_adapt_args;
int spec_verify_adapt_reset(const spec_verify_adapt_args* args, int32_t init_k, void* hip_stream);
int spec_verify_adapt(const spec_verify_adapt_args* args, void* hip_stream);

/* sizeof(spec_verify_adapt_args) as compiled into the library. */
int64_t spec_verify_adapt_args_size(void);

/* Library version string. */
const char* spec_verify_version(void);

/* sizeof(spec_verify_args) as compiled into the library, so that a binding
 * can check its own copy of the struct layout. */
int64_t spec_verify_args_size(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
