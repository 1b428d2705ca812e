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

namespace sv {

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

// 1.0, SV_SAMPLE (0) and s for the first n sequences (synchronous copies).
hipError_t fill_defaults(const Scratch& v, int32_t n) {
  std::vector<float> t((size_t)n, 1.0f);
  std::vector<uint8_t> m((size_t)n, 0);
  std::vector<uint32_t> ids((size_t)n);
  for (int32_t i = 0; i < n; ++i) ids[i] = (uint32_t)i;
  hipError_t e = hipMemcpy(v.def_temperature, t.data(), t.size() * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(v.def_mode, m.data(), m.size(), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(v.def_seq_ids, ids.data(), ids.size() * sizeof(uint32_t), hipMemcpyHostToDevice);
  return e;
}

}  // namespace sv

using sv::align_up;
using sv::hip_fail;
using sv::set_err;

namespace {

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
  sv::Caps caps;
  void* mem = nullptr;
  sv::Scratch scratch;
  // timing hooks
  std::vector<hipEvent_t> events;   // a start and a stop per kernel slot of every recorded call
  std::vector<uint8_t> launched;    // per kernel slot of every recorded call: 1 when it launched
  int32_t timing_cap = 0;
  int32_t timing_used = 0;
};

namespace sv {

ScratchLayout scratch_layout(int32_t max_batch, int32_t max_k, int64_t max_rows, int32_t max_nch, int32_t max_tiles,
                             bool with_segmax) {
  ScratchLayout L;
  size_t off = 0;
  L.o_part = off;  off = align_up(off + sizeof(Partial) * max_rows * max_nch, 256);
  L.o_xval = off;  off = align_up(off + sizeof(float) * max_rows, 256);
  L.o_tau = off;   off = align_up(off + sizeof(float) * max_rows, 256);
  L.o_ptok = off;  off = align_up(off + sizeof(int32_t) * (size_t)max_batch * max_k, 256);
  L.o_fin = off;   off = align_up(off + sizeof(SeqFinal) * max_batch, 256);
  L.o_tile = off;  off = align_up(off + sizeof(float) * (size_t)max_batch * max_tiles, 256);
  L.o_cnt = off;   off = align_up(off + sizeof(uint32_t) * (size_t)max_batch, 256);
  L.o_ord = off;   off = align_up(off + sizeof(int32_t) * (size_t)max_batch, 256);
  L.o_flist = off; off = align_up(off + sizeof(int32_t) * ((size_t)max_rows + 1), 256);
  L.o_seg = off;
  if (with_segmax) off = align_up(off + sizeof(float) * kSegPerChunk * max_rows * max_nch, 256);
  L.bytes = off;
  return L;
}

Scratch scratch_at(void* base, const ScratchLayout& L, bool with_segmax) {
  char* b = (char*)base;
  Scratch v;
  v.partials = (Partial*)(b + L.o_part);
  v.xval = (float*)(b + L.o_xval);
  v.tau = (float*)(b + L.o_tau);
  v.ptok = (int32_t*)(b + L.o_ptok);
  v.fin = (SeqFinal*)(b + L.o_fin);
  v.tilesum = (float*)(b + L.o_tile);
  v.fincnt = (uint32_t*)(b + L.o_cnt);
  v.order = (int32_t*)(b + L.o_ord);
  v.flist = (int32_t*)(b + L.o_flist);
  v.segmax = with_segmax ? (float*)(b + L.o_seg) : nullptr;
  return v;
}

Caps caps_for(int32_t max_batch, int32_t max_k, int64_t max_vocab) {
  Caps c;
  c.max_batch = max_batch;
  c.max_k = max_k;
  c.max_vocab = max_vocab;
  c.max_rows = (int64_t)max_batch * (2 * (int64_t)max_k + 1);
  const int min_ce = kChunkBytes / 4;
  c.max_nch = (int32_t)((max_vocab + min_ce - 1) / min_ce);
  c.max_tiles = (int32_t)((max_vocab + kTileElems - 1) / kTileElems);
  return c;
}

// Host-side checks of one call against the capacity `c` and the launch
// parameters; SV_OK, or an error code with the message set (nothing enqueued).
int prepare_call(const char* who, const spec_verify_args* a, const Caps& c, const Scratch& v, Params* out) {
  if (!a) {
    set_err("%s: args is NULL", who);
    return SV_ERR_INVALID;
  }
  if (a->batch < 0) {
    set_err("%s: batch %d < 0", who, a->batch);
    return SV_ERR_INVALID;
  }
  if (a->vocab < 1 || a->vocab > 0x7FFFFFFF) {
    set_err("%s: vocab %lld out of range", who, (long long)a->vocab);
    return SV_ERR_INVALID;
  }
  if (a->total_draft < 0) {
    set_err("%s: total_draft %lld < 0", who, (long long)a->total_draft);
    return SV_ERR_INVALID;
  }
  if (a->target_dtype != SV_F32 && a->target_dtype != SV_BF16) {
    set_err("%s: target_dtype %d is not SV_F32 or SV_BF16", who, a->target_dtype);
    return SV_ERR_INVALID;
  }
  if (a->draft_logits && a->draft_dtype != SV_F32 && a->draft_dtype != SV_BF16) {
    set_err("%s: draft_dtype %d is not SV_F32 or SV_BF16", who, a->draft_dtype);
    return SV_ERR_INVALID;
  }
  if (!a->target_logits || !a->num_draft || !a->accepted_len || !a->emitted_tokens) {
    set_err("%s: target_logits, num_draft, accepted_len and emitted_tokens are required", who);
    return SV_ERR_INVALID;
  }
  if (a->total_draft > 0 && !a->draft_tokens) {
    set_err("%s: draft_tokens is NULL with total_draft > 0", who);
    return SV_ERR_INVALID;
  }
  if ((uintptr_t)a->target_logits % (a->target_dtype == SV_BF16 ? 2 : 4) ||
      (a->draft_logits && (uintptr_t)a->draft_logits % (a->draft_dtype == SV_BF16 ? 2 : 4))) {
    set_err("%s: logits pointers must be aligned to their element size", who);
    return SV_ERR_INVALID;
  }
  if (a->ld_target < a->vocab) {
    set_err("%s: ld_target %lld < vocab %lld", who, (long long)a->ld_target, (long long)a->vocab);
    return SV_ERR_INVALID;
  }
  if (a->draft_logits && a->ld_draft < a->vocab) {
    set_err("%s: ld_draft %lld < vocab %lld", who, (long long)a->ld_draft, (long long)a->vocab);
    return SV_ERR_INVALID;
  }
  if (a->batch > c.max_batch) {
    set_err("%s: batch %d > max_batch %d", who, a->batch, c.max_batch);
    return SV_ERR_CAPACITY;
  }
  if (a->vocab > c.max_vocab) {
    set_err("%s: vocab %lld > max_vocab %lld", who, (long long)a->vocab, (long long)c.max_vocab);
    return SV_ERR_CAPACITY;
  }
  if (a->total_draft > (int64_t)c.max_batch * c.max_k) {
    set_err("%s: total_draft %lld > max_batch * max_k = %lld", who, (long long)a->total_draft,
            (long long)c.max_batch * c.max_k);
    return SV_ERR_CAPACITY;
  }

  Params& p = *out;
  memset(&p, 0, sizeof(p));
  p.B = a->batch;
  p.V = (int32_t)a->vocab;
  p.total_draft = (int32_t)a->total_draft;
  p.max_k = c.max_k;
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
  p.temperature = a->temperature ? a->temperature : v.def_temperature;
  p.mode = a->mode ? a->mode : v.def_mode;
  p.seq_ids = a->seq_ids ? a->seq_ids : v.def_seq_ids;
  p.seed_lo = (uint32_t)(a->seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(a->seed >> 32);
  p.accepted_len = a->accepted_len;
  p.emitted = a->emitted_tokens;
  p.p_at = a->p_at_proposal;
  p.q_at = a->q_at_proposal;
  p.status = a->status;
  p.partials = v.partials;
  p.xval = v.xval;
  p.tau = v.tau;
  p.order = v.order;
  p.flist = v.flist;
  const bool filtered = a->top_k || a->top_p;
  p.order_block = filtered ? 1 : 0;
  p.segmax = filtered ? v.segmax : nullptr;   // filter bounds from row_stats' segment maxima
  p.top_k = a->top_k;
  p.top_p = a->top_p;
  p.ptok = v.ptok;
  p.fin = v.fin;
  p.tilesum = v.tilesum;
  p.fincnt = v.fincnt;
  // one row-stats block streams 32 KB of a row
  p.ce_t = kChunkBytes / es_t;
  p.ce_d = kChunkBytes / es_d;
  p.nch_t = (p.V + p.ce_t - 1) / p.ce_t;
  p.nch_d = (p.V + p.ce_d - 1) / p.ce_d;
  p.ntiles = (p.V + kTileElems - 1) / kTileElems;
  p.slots = 2 * c.max_k + 1;
  p.nch_max = p.nch_t > p.nch_d ? p.nch_t : p.nch_d;
  p.nsplit = 1;
  if (p.B < kFuseMinBatch) {
    const int want = (kSplitTargetBlocks + p.B - 1) / p.B;
    p.nsplit = want < p.ntiles ? want : p.ntiles;
    if (p.nsplit < 1) p.nsplit = 1;
  }
  if ((int64_t)(p.n_t + p.n_d) > c.max_rows || p.nch_t > c.max_nch || p.nch_d > c.max_nch ||
      p.ntiles > c.max_tiles || (filtered && !v.segmax)) {
    set_err("%s: scratch capacity exceeded", who);
    return SV_ERR_CAPACITY;
  }
  return SV_OK;
}

// Enqueue the kernels of one step (timed when `events` is not NULL: a start
// and a stop event per kernel slot).
int launch_call(const Params& p, hipStream_t st, hipEvent_t* events, uint8_t* launched) {
  typedef hipError_t (*Launch)(const Params&, hipStream_t, const LaunchEvents*);
  static const Launch kLaunch[SV_NUM_KERNELS] = {launch_row_stats, launch_filter, launch_final, launch_select};
  static const char* kName[SV_NUM_KERNELS] = {"row_stats", "filter", "final", "select"};
  for (int k = 0; k < SV_NUM_KERNELS; ++k) {
    const LaunchEvents le{events ? events[2 * k] : nullptr, events ? events[2 * k + 1] : nullptr,
                          events ? &launched[k] : nullptr};
    hipError_t e = kLaunch[k](p, st, events ? &le : nullptr);
    if (e != hipSuccess) return hip_fail(kName[k], e);
  }
  return SV_OK;
}

}  // namespace sv

extern "C" {

const char* spec_verify_last_error(void) { return sv::g_err; }

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
  c->caps = sv::caps_for(max_batch, max_k, max_vocab);
  const sv::ScratchLayout L = sv::scratch_layout(max_batch, max_k, c->caps.max_rows, c->caps.max_nch,
                                                 c->caps.max_tiles, true);
  // defaults for NULL temperature / mode / seq_ids (1.0, SV_SAMPLE, s) after the call's scratch
  const size_t o_dt = L.bytes;
  const size_t o_dm = align_up(o_dt + sizeof(float) * (size_t)max_batch, 256);
  const size_t o_ds = align_up(o_dm + (size_t)max_batch, 256);
  const size_t bytes = align_up(o_ds + sizeof(uint32_t) * (size_t)max_batch, 256);
  e = hipMalloc(&c->mem, bytes);
  if (e != hipSuccess) {
    delete c;
    set_err("spec_verify_create: hipMalloc of %zu bytes: %s", bytes, hipGetErrorString(e));
    return SV_ERR_NOMEM;
  }
  e = hipMemset(c->mem, 0, bytes);
  if (e != hipSuccess) {
    (void)hipFree(c->mem);
    delete c;
    return hip_fail("hipMemset", e);
  }
  c->scratch = sv::scratch_at(c->mem, L, true);
  char* b = (char*)c->mem;
  c->scratch.def_temperature = (float*)(b + o_dt);
  c->scratch.def_mode = (uint8_t*)(b + o_dm);
  c->scratch.def_seq_ids = (uint32_t*)(b + o_ds);
  if ((e = sv::fill_defaults(c->scratch, max_batch)) != hipSuccess) {
    (void)hipFree(c->mem);
    delete c;
    return hip_fail("hipMemcpy", e);
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
  if (a->batch == 0) return SV_OK;
  sv::Params p;
  int rc = sv::prepare_call("spec_verify_run", a, ctx->caps, ctx->scratch, &p);
  if (rc != SV_OK) return rc;

  DeviceGuard g;
  hipError_t e = g.enter(ctx->device);
  if (e != hipSuccess) return hip_fail("hipSetDevice", e);
  const bool timed = ctx->timing_used < ctx->timing_cap;
  hipEvent_t* ev = timed ? &ctx->events[(size_t)ctx->timing_used * 2 * SV_NUM_KERNELS] : nullptr;
  uint8_t* launched = timed ? &ctx->launched[(size_t)ctx->timing_used * SV_NUM_KERNELS] : nullptr;
  rc = sv::launch_call(p, (hipStream_t)hip_stream, ev, launched);
  if (rc != SV_OK) return rc;
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
