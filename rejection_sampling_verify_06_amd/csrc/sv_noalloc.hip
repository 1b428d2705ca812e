// spec_verify_run_noalloc: the verify call for callers that cannot allocate
// device memory.  Its scratch is one file-scope device array (each GPU the
// library runs on holds its own copy until the process ends); the address of
// this GPU's copy is looked up once per device with hipGetSymbolAddress, and
// only that address is ever handed to the kernels or to copies (the array's
// name in host code is not a device address).  The kernels are the ones
// spec_verify_run launches; only where their scratch lives differs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "spec_verify.h"
#include "sv_internal.h"

namespace {

constexpr size_t kNoallocBytes = SV_NOALLOC_SCRATCH_BYTES;
constexpr int kNoallocMaxBatch = 4096;
// the defaults for NULL temperature / mode / seq_ids sit at the start of the
// array (written once per device), the call's scratch after them
constexpr size_t kDefT = 0;                                    // float [4096]
constexpr size_t kDefM = kDefT + 4 * kNoallocMaxBatch;         // uint8 [4096]
constexpr size_t kDefS = kDefM + kNoallocMaxBatch;             // uint32 [4096]
constexpr size_t kDefBytes = kDefS + 4 * kNoallocMaxBatch;     // 36 KB, 256-byte aligned
static_assert(kDefBytes % 256 == 0, "call scratch alignment");

static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_base[kMaxDevices];   // per device: the device address of `scratch`, once set up

sv::Scratch defaults_at(char* base) {
  sv::Scratch v{};
  v.def_temperature = (float*)(base + kDefT);
  v.def_mode = (uint8_t*)(base + kDefM);
  v.def_seq_ids = (uint32_t*)(base + kDefS);
  return v;
}

// The current device's copy of the array; the first call on a device looks
// it up and writes the defaults (synchronous copies).
int device_scratch(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return sv::hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) {
    sv::set_err("spec_verify_run_noalloc: device %d outside 0..%d", dev, kMaxDevices - 1);
    return SV_ERR_INVALID;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_base[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return sv::hip_fail("hipGetSymbolAddress", e != hipSuccess ? e : hipErrorUnknown);
    e = sv::fill_defaults(defaults_at((char*)ptr), kNoallocMaxBatch);
    if (e != hipSuccess) return sv::hip_fail("hipMemcpy", e);
    g_base[dev] = (char*)ptr;
  }
  *out = g_base[dev];
  return SV_OK;
}

}  // namespace

extern "C" int spec_verify_run_noalloc(const spec_verify_args* a, int32_t max_k, void* hip_stream) {
  const char* who = "spec_verify_run_noalloc";
  if (!a) {
    sv::set_err("%s: args is NULL", who);
    return SV_ERR_INVALID;
  }
  if (max_k < 1 || max_k > sv::kMaxK) {
    sv::set_err("%s: max_k %d outside 1..%d", who, max_k, sv::kMaxK);
    return SV_ERR_INVALID;
  }
  if (a->batch == 0) return SV_OK;
  if (a->batch < 0 || a->vocab < 1 || a->vocab > (int64_t)sv::kMaxTiles * sv::kTileElems) {
    sv::set_err("%s: batch %d or vocab %lld out of range", who, a->batch, (long long)a->vocab);
    return a->batch < 0 || a->vocab < 1 ? SV_ERR_INVALID : SV_ERR_CAPACITY;
  }
  if (a->batch > kNoallocMaxBatch) {
    sv::set_err("%s: batch %d > %d", who, a->batch, kNoallocMaxBatch);
    return SV_ERR_CAPACITY;
  }
  // this call's sizes: the scratch is laid out for exactly them
  const int es_t = a->target_dtype == SV_BF16 ? 2 : 4;
  const int es_d = a->draft_logits ? (a->draft_dtype == SV_BF16 ? 2 : 4) : es_t;
  const int32_t V = (int32_t)a->vocab;
  const int32_t nch_t = (V + sv::kChunkBytes / es_t - 1) / (sv::kChunkBytes / es_t);
  const int32_t nch_d = (V + sv::kChunkBytes / es_d - 1) / (sv::kChunkBytes / es_d);
  sv::Caps c;
  c.max_batch = a->batch;
  c.max_k = max_k;
  c.max_vocab = a->vocab;
  c.max_rows = (int64_t)a->batch * (2 * (int64_t)max_k + 1);
  c.max_nch = nch_t > nch_d ? nch_t : nch_d;
  c.max_tiles = (V + sv::kTileElems - 1) / sv::kTileElems;
  const bool filtered = a->top_k || a->top_p;
  const sv::ScratchLayout L = sv::scratch_layout(c.max_batch, c.max_k, c.max_rows, c.max_nch, c.max_tiles, filtered);
  if (kDefBytes + L.bytes > kNoallocBytes) {
    sv::set_err("%s: the call needs %zu bytes of scratch (batch %d, max_k %d, vocab %d%s), more than the %zu "
                "bytes reserved", who, (size_t)(kDefBytes + L.bytes), a->batch, max_k, V,
                filtered ? ", filtered" : "", kNoallocBytes);
    return SV_ERR_CAPACITY;
  }
  char* base = nullptr;
  int rc = device_scratch(&base);
  if (rc != SV_OK) return rc;
  sv::Scratch v = sv::scratch_at(base + kDefBytes, L, filtered);
  const sv::Scratch d = defaults_at(base);
  v.def_temperature = d.def_temperature;
  v.def_mode = d.def_mode;
  v.def_seq_ids = d.def_seq_ids;
  sv::Params p;
  rc = sv::prepare_call(who, a, c, v, &p);
  if (rc != SV_OK) return rc;
  return sv::launch_call(p, (hipStream_t)hip_stream, nullptr, nullptr);
}
