// Host side of the C interface declared in include/spec_verify.h: context and
// scratch ownership, argument validation, launch geometry, timing hooks.

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <vector>

#include "spec_verify.h"
#include "sv_internal.h"

namespace {

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int hip_fail(const char* what, hipError_t e) {
  set_err("%s: %s", what, hipGetErrorString(e));
  return SV_ERR_HIP;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Restores the caller's current device on scope exit.
struct DeviceGuard {
  int prev = -1;
  bool changed = false;
  hipError_t enter(int dev) {
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != dev) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return e;
      changed = true;
    }
    return hipSuccess;
  }
  ~DeviceGuard() {
    if (changed) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct spec_verify_ctx {
  int device = 0;
  int32_t max_batch = 0;
  int32_t max_k = 0;
  int64_t max_vocab = 0;
  int64_t max_rows = 0;     // sequence slots: max_batch * (2 * max_k + 1)
  int32_t max_nch = 0;      // chunks per row at the smallest chunk (8192 elements)
  int32_t max_tiles = 0;
  void* mem = nullptr;
  size_t bytes = 0;
  sv::Partial* partials = nullptr;
  float* segmax = nullptr;
  float* xval = nullptr;
  float* tau = nullptr;
  int32_t* order = nullptr;   // the filter kernel's sequence order
  int32_t* ptok = nullptr;
  sv::SeqFinal* fin = nullptr;
  float* tilesum = nullptr;
  // defaults for NULL temperature / mode / seq_ids: 1.0, SV_SAMPLE, s
  float* def_temperature = nullptr;
  uint8_t* def_mode = nullptr;
  uint32_t* def_seq_ids = nullptr;
  // timing hooks
  std::vector<hipEvent_t> events;   // a start and a stop per kernel slot of every recorded call
  std::vector<uint8_t> launched;    // per kernel slot of every recorded call: 1 when it launched
  int32_t timing_cap = 0;
  int32_t timing_used = 0;
};

extern "C" {

const char* spec_verify_last_error(void) { return g_err; }

const char* spec_verify_version(void) { return "spec_verify 0.1 (gfx950)"; }

int64_t spec_verify_args_size(void) { return (int64_t)sizeof(spec_verify_args); }

int spec_verify_create(spec_verify_ctx** out, int device, int32_t max_batch, int32_t max_k, int64_t max_vocab) {
  if (!out) {
    set_err("spec_verify_create: out is NULL");
    return SV_ERR_INVALID;
  }
  *out = nullptr;
  if (max_batch < 1 || max_batch > 4096) {
    set_err("spec_verify_create: max_batch %d outside 1..4096", max_batch);
    return SV_ERR_INVALID;
  }
  if (max_k < 1 || max_k > sv::kMaxK) {
    set_err("spec_verify_create: max_k %d outside 1..%d", max_k, sv::kMaxK);
    return SV_ERR_INVALID;
  }
  if (max_vocab < 1 || max_vocab > (int64_t)sv::kMaxTiles * sv::kTileElems) {
    set_err("spec_verify_create: max_vocab %lld outside 1..%lld", (long long)max_vocab,
            (long long)sv::kMaxTiles * sv::kTileElems);
    return SV_ERR_INVALID;
  }
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_fail("hipGetDeviceCount", e);
  if (device < 0 || device >= ndev) {
    set_err("spec_verify_create: device %d outside 0..%d", device, ndev - 1);
    return SV_ERR_INVALID;
  }
  DeviceGuard g;
  if ((e = g.enter(device)) != hipSuccess) return hip_fail("hipSetDevice", e);

  spec_verify_ctx* c = new (std::nothrow) spec_verify_ctx();
  if (!c) {
    set_err("spec_verify_create: host allocation failed");
    return SV_ERR_NOMEM;
  }
  c->device = device;
  c->max_batch = max_batch;
  c->max_k = max_k;
  c->max_vocab = max_vocab;
  c->max_rows = (int64_t)max_batch * (2 * (int64_t)max_k + 1);
  const int min_ce = sv::kChunkBytes / 4;
  c->max_nch = (int32_t)((max_vocab + min_ce - 1) / min_ce);
  c->max_tiles = (int32_t)((max_vocab + sv::kTileElems - 1) / sv::kTileElems);

  size_t off = 0;
  const size_t o_part = off;   off = align_up(off + sizeof(sv::Partial) * c->max_rows * c->max_nch, 256);
  const size_t o_xval = off;   off = align_up(off + sizeof(float) * c->max_rows, 256);
  const size_t o_tau = off;    off = align_up(off + sizeof(float) * c->max_rows, 256);
  const size_t o_ptok = off;   off = align_up(off + sizeof(int32_t) * (size_t)max_batch * max_k, 256);
  const size_t o_fin = off;    off = align_up(off + sizeof(sv::SeqFinal) * max_batch, 256);
  const size_t o_tile = off;   off = align_up(off + sizeof(float) * (size_t)max_batch * c->max_tiles, 256);
  const size_t o_dt = off;     off = align_up(off + sizeof(float) * (size_t)max_batch, 256);
  const size_t o_dm = off;     off = align_up(off + (size_t)max_batch, 256);
  const size_t o_ds = off;     off = align_up(off + sizeof(uint32_t) * (size_t)max_batch, 256);
  const size_t o_ord = off;    off = align_up(off + sizeof(int32_t) * (size_t)max_batch, 256);
  const size_t o_seg = off;    off = align_up(off + sizeof(float) * sv::kSegPerChunk * c->max_rows * c->max_nch, 256);
  c->bytes = off;
  e = hipMalloc(&c->mem, c->bytes);
  if (e != hipSuccess) {
    delete c;
    set_err("spec_verify_create: hipMalloc of %zu bytes: %s", off, hipGetErrorString(e));
    return SV_ERR_NOMEM;
  }
  e = hipMemset(c->mem, 0, c->bytes);
  if (e != hipSuccess) {
    (void)hipFree(c->mem);
    delete c;
    return hip_fail("hipMemset", e);
  }
  char* b = (char*)c->mem;
  c->partials = (sv::Partial*)(b + o_part);
  c->xval = (float*)(b + o_xval);
  c->tau = (float*)(b + o_tau);
  c->ptok = (int32_t*)(b + o_ptok);
  c->fin = (sv::SeqFinal*)(b + o_fin);
  c->tilesum = (float*)(b + o_tile);
  c->def_temperature = (float*)(b + o_dt);
  c->def_mode = (uint8_t*)(b + o_dm);
  c->def_seq_ids = (uint32_t*)(b + o_ds);
  c->order = (int32_t*)(b + o_ord);
  c->segmax = (float*)(b + o_seg);
  {
    std::vector<float> t((size_t)max_batch, 1.0f);
    std::vector<uint32_t> ids((size_t)max_batch);
    for (int32_t i = 0; i < max_batch; ++i) ids[i] = (uint32_t)i;
    // mode: the scratch is zeroed above, and 0 is SV_SAMPLE
    e = hipMemcpy(c->def_temperature, t.data(), t.size() * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(c->def_seq_ids, ids.data(), ids.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(c->mem);
      delete c;
      return hip_fail("hipMemcpy", e);
    }
  }
  *out = c;
  return SV_OK;
}

void spec_verify_destroy(spec_verify_ctx* ctx) {
  if (!ctx) return;
  DeviceGuard g;
  (void)g.enter(ctx->device);
  for (hipEvent_t ev : ctx->events) (void)hipEventDestroy(ev);
  if (ctx->mem) (void)hipFree(ctx->mem);
  delete ctx;
}

int spec_verify_run(spec_verify_ctx* ctx, const spec_verify_args* a, void* hip_stream) {
  if (!ctx || !a) {
    set_err("spec_verify_run: ctx or args is NULL");
    return SV_ERR_INVALID;
  }
  if (a->batch < 0) {
    set_err("spec_verify_run: batch %d < 0", a->batch);
    return SV_ERR_INVALID;
  }
  if (a->batch == 0) return SV_OK;
  if (a->vocab < 1 || a->vocab > 0x7FFFFFFF) {
    set_err("spec_verify_run: vocab %lld out of range", (long long)a->vocab);
    return SV_ERR_INVALID;
  }
  if (a->total_draft < 0) {
    set_err("spec_verify_run: total_draft %lld < 0", (long long)a->total_draft);
    return SV_ERR_INVALID;
  }
  if (a->target_dtype != SV_F32 && a->target_dtype != SV_BF16) {
    set_err("spec_verify_run: target_dtype %d is not SV_F32 or SV_BF16", a->target_dtype);
    return SV_ERR_INVALID;
  }
  if (a->draft_logits && a->draft_dtype != SV_F32 && a->draft_dtype != SV_BF16) {
    set_err("spec_verify_run: draft_dtype %d is not SV_F32 or SV_BF16", a->draft_dtype);
    return SV_ERR_INVALID;
  }
  if (!a->target_logits || !a->num_draft || !a->accepted_len || !a->emitted_tokens) {
    set_err("spec_verify_run: target_logits, num_draft, accepted_len and emitted_tokens are required");
    return SV_ERR_INVALID;
  }
  if (a->total_draft > 0 && !a->draft_tokens) {
    set_err("spec_verify_run: draft_tokens is NULL with total_draft > 0");
    return SV_ERR_INVALID;
  }
  if ((uintptr_t)a->target_logits % (a->target_dtype == SV_BF16 ? 2 : 4) ||
      (a->draft_logits && (uintptr_t)a->draft_logits % (a->draft_dtype == SV_BF16 ? 2 : 4))) {
    set_err("spec_verify_run: logits pointers must be aligned to their element size");
    return SV_ERR_INVALID;
  }
  if (a->ld_target < a->vocab) {
    set_err("spec_verify_run: ld_target %lld < vocab %lld", (long long)a->ld_target, (long long)a->vocab);
    return SV_ERR_INVALID;
  }
  if (a->draft_logits && a->ld_draft < a->vocab) {
    set_err("spec_verify_run: ld_draft %lld < vocab %lld", (long long)a->ld_draft, (long long)a->vocab);
    return SV_ERR_INVALID;
  }
  if (a->batch > ctx->max_batch) {
    set_err("spec_verify_run: batch %d > max_batch %d", a->batch, ctx->max_batch);
    return SV_ERR_CAPACITY;
  }
  if (a->vocab > ctx->max_vocab) {
    set_err("spec_verify_run: vocab %lld > max_vocab %lld", (long long)a->vocab, (long long)ctx->max_vocab);
    return SV_ERR_CAPACITY;
  }
  if (a->total_draft > (int64_t)ctx->max_batch * ctx->max_k) {
    set_err("spec_verify_run: total_draft %lld > max_batch * max_k = %lld", (long long)a->total_draft,
            (long long)ctx->max_batch * ctx->max_k);
    return SV_ERR_CAPACITY;
  }

  sv::Params p;
  memset(&p, 0, sizeof(p));
  p.B = a->batch;
  p.V = (int32_t)a->vocab;
  p.total_draft = (int32_t)a->total_draft;
  p.max_k = ctx->max_k;
  p.n_t = p.total_draft + p.B;
  p.n_d = a->draft_logits ? p.total_draft : 0;
  p.tgt = a->target_logits;
  p.ld_t = a->ld_target;
  p.t_bf16 = a->target_dtype == SV_BF16;
  const int es_t = p.t_bf16 ? 2 : 4;
  p.t_vec = ((uintptr_t)a->target_logits % 16 == 0) && ((a->ld_target * es_t) % 16 == 0);
  p.dft = a->draft_logits;
  p.ld_d = a->draft_logits ? a->ld_draft : 0;
  p.d_bf16 = a->draft_logits ? (a->draft_dtype == SV_BF16) : p.t_bf16;
  const int es_d = p.d_bf16 ? 2 : 4;
  p.d_vec = a->draft_logits && ((uintptr_t)a->draft_logits % 16 == 0) && ((a->ld_draft * es_d) % 16 == 0);
  p.tokens = a->draft_tokens;
  p.num_draft = a->num_draft;
  p.temperature = a->temperature ? a->temperature : ctx->def_temperature;
  p.mode = a->mode ? a->mode : ctx->def_mode;
  p.seq_ids = a->seq_ids ? a->seq_ids : ctx->def_seq_ids;
  p.seed_lo = (uint32_t)(a->seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.accepted_len = a->accepted_len;
  p.emitted = a->emitted_tokens;
  p.p_at = a->p_at_proposal;
  p.q_at = a->q_at_proposal;
  p.status = a->status;
  p.partials = ctx->partials;
  p.xval = ctx->xval;
  p.tau = ctx->tau;
  p.order = ctx->order;
  p.order_block = (a->top_k || a->top_p) ? 1 : 0;
  p.segmax = (a->top_k || a->top_p) ? ctx->segmax : nullptr;   // filter bounds from row_stats' segment maxima
  p.top_k = a->top_k;
  p.top_p = a->top_p;
  p.ptok = ctx->ptok;
  p.fin = ctx->fin;
  p.tilesum = ctx->tilesum;
  // one row-stats block streams 32 KB of a row
  p.ce_t = sv::kChunkBytes / es_t;
  p.ce_d = sv::kChunkBytes / es_d;
  p.nch_t = (p.V + p.ce_t - 1) / p.ce_t;
  p.nch_d = (p.V + p.ce_d - 1) / p.ce_d;
  p.ntiles = (p.V + sv::kTileElems - 1) / sv::kTileElems;
  p.slots = 2 * ctx->max_k + 1;
  p.nch_max = p.nch_t > p.nch_d ? p.nch_t : p.nch_d;
  p.nsplit = 1;
  if (p.B < sv::kFuseMinBatch) {
    const int want = (sv::kSplitTargetBlocks + p.B - 1) / p.B;
    p.nsplit = want < p.ntiles ? want : p.ntiles;
    if (p.nsplit < 1) p.nsplit = 1;
  }
  if ((int64_t)(p.n_t + p.n_d) > ctx->max_rows || p.nch_t > ctx->max_nch || p.nch_d > ctx->max_nch ||
      p.ntiles > ctx->max_tiles) {
    set_err("spec_verify_run: scratch capacity exceeded");
    return SV_ERR_CAPACITY;
  }

  DeviceGuard g;
  hipError_t e = g.enter(ctx->device);
  if (e != hipSuccess) return hip_fail("hipSetDevice", e);
  hipStream_t st = (hipStream_t)hip_stream;

  const bool timed = ctx->timing_used < ctx->timing_cap;
  hipEvent_t* ev = timed ? &ctx->events[(size_t)ctx->timing_used * 2 * SV_NUM_KERNELS] : nullptr;
  typedef hipError_t (*Launch)(const sv::Params&, hipStream_t, const sv::LaunchEvents*);
  static const Launch kLaunch[SV_NUM_KERNELS] = {sv::launch_row_stats, sv::launch_filter, sv::launch_final,
                                                 sv::launch_select};
  static const char* kName[SV_NUM_KERNELS] = {"row_stats", "filter", "final", "select"};
  uint8_t* launched = timed ? &ctx->launched[(size_t)ctx->timing_used * SV_NUM_KERNELS] : nullptr;
  for (int k = 0; k < SV_NUM_KERNELS; ++k) {
    const sv::LaunchEvents le{timed ? ev[2 * k] : nullptr, timed ? ev[2 * k + 1] : nullptr,
                              timed ? &launched[k] : nullptr};
    if ((e = kLaunch[k](p, st, timed ? &le : nullptr)) != hipSuccess) return hip_fail(kName[k], e);
  }
  if (timed) ctx->timing_used++;
  return SV_OK;
}

int64_t spec_verify_ngram_args_size(void) { return (int64_t)sizeof(spec_verify_ngram_args); }

int spec_verify_ngram_propose(const spec_verify_ngram_args* a, void* hip_stream) {
  if (!a) {
    set_err("spec_verify_ngram_propose: args is NULL");
    return SV_ERR_INVALID;
  }
  if (a->batch < 0) {
    set_err("spec_verify_ngram_propose: batch %d < 0", a->batch);
    return SV_ERR_INVALID;
  }
  if (a->batch == 0) return SV_OK;
  if (a->min_n < 1 || a->max_n < a->min_n || a->max_n > SV_NGRAM_MAX_N) {
    set_err("spec_verify_ngram_propose: need 1 <= min_n (%d) <= max_n (%d) <= %d", a->min_n, a->max_n,
            SV_NGRAM_MAX_N);
    return SV_ERR_INVALID;
  }
  if (a->max_tokens < 1 || a->max_tokens > SV_NGRAM_MAX_TOKENS) {
    set_err("spec_verify_ngram_propose: max_tokens %d outside 1..%d", a->max_tokens, SV_NGRAM_MAX_TOKENS);
    return SV_ERR_INVALID;
  }
  if (a->total_len < 0 || (a->total_len > 0 && !a->history) || !a->hist_offsets || !a->draft_tokens ||
      !a->num_draft) {
    set_err("spec_verify_ngram_propose: history (when total_len > 0), hist_offsets, draft_tokens and num_draft "
            "are required");
    return SV_ERR_INVALID;
  }
  static_assert(SV_NGRAM_MAX_N == sv::kNgramMaxN, "window limit");
  sv::NgramParams p;
  p.B = a->batch;
  p.history = a->history;
  p.offsets = a->hist_offsets;
  p.total_len = a->total_len;
  p.min_n = a->min_n;
  p.max_n = a->max_n;
  p.max_tokens = a->max_tokens;
  p.draft = a->draft_tokens;
  p.num_draft = a->num_draft;
  p.match_n = a->match_n;
  hipError_t e = sv::launch_ngram(p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail("ngram", e);
  return SV_OK;
}

int spec_verify_stats_accumulate(int32_t batch, int32_t max_k, const int32_t* num_draft,
                                 const int32_t* accepted_len, uint64_t* stats, void* hip_stream) {
  if (batch < 0 || max_k < 1 || max_k > SV_STATS_MAX_K) {
    set_err("spec_verify_stats_accumulate: need batch >= 0 (%d) and 1 <= max_k (%d) <= %d", batch, max_k,
            SV_STATS_MAX_K);
    return SV_ERR_INVALID;
  }
  if (!stats || (batch > 0 && (!num_draft || !accepted_len))) {
    set_err("spec_verify_stats_accumulate: stats, num_draft and accepted_len are required");
    return SV_ERR_INVALID;
  }
  static_assert(SV_STATS_MAX_K == sv::kStatsMaxK, "stats positions");
  static_assert(SV_STATS_WORDS(SV_STATS_MAX_K) == sv::kStatsMaxWords, "stats layout");
  sv::StatsParams p{};
  p.B = batch;
  p.max_k = max_k;
  p.num_draft = num_draft;
  p.accepted_len = accepted_len;
  p.counters = stats;
  hipError_t e = sv::launch_stats_accumulate(p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail("stats_accumulate", e);
  return SV_OK;
}

int spec_verify_stats_summary(int32_t max_k, const uint64_t* stats, double* summary, void* hip_stream) {
  if (max_k < 1 || max_k > SV_STATS_MAX_K || !stats || !summary) {
    set_err("spec_verify_stats_summary: need 1 <= max_k (%d) <= %d and both buffers", max_k, SV_STATS_MAX_K);
    return SV_ERR_INVALID;
  }
  sv::StatsParams p{};
  p.max_k = max_k;
  p.counters = const_cast<uint64_t*>(stats);
  p.summary = summary;
  hipError_t e = sv::launch_stats_summary(p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail("stats_summary", e);
  return SV_OK;
}

int64_t spec_verify_adapt_args_size(void) { return (int64_t)sizeof(spec_verify_adapt_args); }

static int adapt_params(const spec_verify_adapt_args* a, const char* who, sv::AdaptParams* p) {
  if (!a) {
    set_err("%s: args is NULL", who);
    return SV_ERR_INVALID;
  }
  if (a->batch < 0 || a->kind < SV_ADAPT_WINDOW || a->kind > SV_ADAPT_OPTIMAL_K ||
      (a->count != SV_ADAPT_COUNT_EMITTED && a->count != SV_ADAPT_COUNT_DRAFT_ONLY)) {
    set_err("%s: batch %d < 0, unknown kind %d or unknown count %d", who, a->batch, a->kind, a->count);
    return SV_ERR_INVALID;
  }
  if (a->kind != SV_ADAPT_OPTIMAL_K && (a->min_k < 1 || a->max_k < a->min_k || a->max_k > SV_ADAPT_MAX_LENGTH)) {
    set_err("%s: need 1 <= min_k (%d) <= max_k (%d) <= %d", who, a->min_k, a->max_k, SV_ADAPT_MAX_LENGTH);
    return SV_ERR_INVALID;
  }
  if (a->kind == SV_ADAPT_WINDOW &&
      (a->window < 1 || a->window > SV_ADAPT_MAX_WINDOW || a->min_samples < 1)) {
    set_err("%s: need 1 <= window (%d) <= %d and min_samples (%d) >= 1", who, a->window, SV_ADAPT_MAX_WINDOW,
            a->min_samples);
    return SV_ERR_INVALID;
  }
  if (!(a->target >= 0.0 && a->target <= 1.0) || !(a->rate >= 0.0 && a->rate <= 1.0)) {
    set_err("%s: need target (%g) and rate (%g) in [0, 1]", who, a->target, a->rate);
    return SV_ERR_INVALID;
  }
  if (a->batch > 0 && (!a->state || !a->next_k || ((uintptr_t)a->state & 15))) {
    set_err("%s: state (16-byte aligned) and next_k are required", who);
    return SV_ERR_INVALID;
  }
  static_assert(SV_ADAPT_MAX_WINDOW == sv::kAdaptMaxWindow, "window limit");
  p->B = a->batch;
  p->kind = a->kind;
  p->min_k = a->min_k;
  p->max_k = a->max_k;
  p->window = a->kind == SV_ADAPT_WINDOW ? a->window : 1;
  p->min_samples = a->min_samples;
  p->count = a->count;
  p->target = a->target;
  p->rate = a->rate;
  p->num_draft = a->num_draft;
  p->accepted_len = a->accepted_len;
  p->hdr = static_cast<int32_t*>(a->state);
  p->win = reinterpret_cast<double*>(static_cast<char*>(a->state) + (int64_t)a->batch * 16);
  p->next_k = a->next_k;
  return SV_OK;
}

int spec_verify_adapt_reset(const spec_verify_adapt_args* a, int32_t init_k, void* hip_stream) {
  sv::AdaptParams p{};
  int rc = adapt_params(a, "spec_verify_adapt_reset", &p);
  if (rc != SV_OK) return rc;
  if (init_k < 1 || init_k > SV_ADAPT_MAX_LENGTH) {
    set_err("spec_verify_adapt_reset: init_k %d outside 1..%d", init_k, SV_ADAPT_MAX_LENGTH);
    return SV_ERR_INVALID;
  }
  p.init_k = init_k;
  hipError_t e = sv::launch_adapt_reset(p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail("adapt_reset", e);
  return SV_OK;
}

int spec_verify_adapt(const spec_verify_adapt_args* a, void* hip_stream) {
  sv::AdaptParams p{};
  int rc = adapt_params(a, "spec_verify_adapt", &p);
  if (rc != SV_OK) return rc;
  if (a->batch > 0 && (!a->num_draft || !a->accepted_len)) {
    set_err("spec_verify_adapt: num_draft and accepted_len are required");
    return SV_ERR_INVALID;
  }
  hipError_t e = sv::launch_adapt(p, (hipStream_t)hip_stream);
  if (e != hipSuccess) return hip_fail("adapt", e);
  return SV_OK;
}

int spec_verify_timing_enable(spec_verify_ctx* ctx, int32_t max_calls) {
  if (!ctx || max_calls < 0) {
    set_err("spec_verify_timing_enable: bad arguments");
    return SV_ERR_INVALID;
  }
  DeviceGuard g;
  hipError_t e = g.enter(ctx->device);
  if (e != hipSuccess) return hip_fail("hipSetDevice", e);
  for (hipEvent_t ev : ctx->events) (void)hipEventDestroy(ev);
  ctx->events.clear();
  ctx->timing_cap = 0;
  ctx->timing_used = 0;
  if (max_calls == 0) return SV_OK;
  ctx->events.resize((size_t)max_calls * 2 * SV_NUM_KERNELS);
  ctx->launched.assign((size_t)max_calls * SV_NUM_KERNELS, 0);
  for (auto& ev : ctx->events) {
    if ((e = hipEventCreate(&ev)) != hipSuccess) {
      ctx->events.clear();
      return hip_fail("hipEventCreate", e);
    }
  }
  ctx->timing_cap = max_calls;
  return SV_OK;
}

int spec_verify_timing_read(spec_verify_ctx* ctx, int32_t* calls, double* ms_per_kernel) {
  if (!ctx || !calls || !ms_per_kernel) {
    set_err("spec_verify_timing_read: bad arguments");
    return SV_ERR_INVALID;
  }
  DeviceGuard g;
  hipError_t e = g.enter(ctx->device);
  if (e != hipSuccess) return hip_fail("hipSetDevice", e);
  for (int k = 0; k < SV_NUM_KERNELS; ++k) ms_per_kernel[k] = 0.0;
  for (int32_t i = 0; i < ctx->timing_used; ++i) {
    hipEvent_t* ev = &ctx->events[(size_t)i * 2 * SV_NUM_KERNELS];
    const uint8_t* launched = &ctx->launched[(size_t)i * SV_NUM_KERNELS];
    for (int k = 0; k < SV_NUM_KERNELS; ++k) {
      if (!launched[k]) continue;
      if ((e = hipEventSynchronize(ev[2 * k + 1])) != hipSuccess) return hip_fail("hipEventSynchronize", e);
      float ms = 0.f;
      if ((e = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1])) != hipSuccess) return hip_fail("hipEventElapsedTime", e);
      ms_per_kernel[k] += ms;
    }
  }
  *calls = ctx->timing_used;
  ctx->timing_used = 0;
  return SV_OK;
}

}  // extern "C"
