// dflash_verify_noalloc: the verification of dflash_verify for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation).  It needs no handle: its scratch -- the per-row
// target argmax of the greedy test, or the row statistics, accepted counts and
// per-256-id chunk sums of rejection sampling -- lives in one file-scope device
// array, whose address is resolved once per device with hipGetSymbolAddress.
// The kernels are dflash_verify's own; nothing here allocates.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dflash.h"
#include "ops.h"

namespace dfl {
namespace {

constexpr int NA_MAX_REQ = 256;
constexpr int NA_MAX_K = 31;
constexpr int NA_MAX_VOCAB = 262144;
constexpr int NA_MAX_CHUNKS = NA_MAX_VOCAB / 256;
constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// rejection: stats [n][2K+1][2] f32, acc [n] i32, chunks [2][n][chunks] f32; greedy: post [n][K+1] i32
constexpr size_t NA_STATS = align256((size_t)NA_MAX_REQ * (2 * NA_MAX_K + 1) * 2 * 4);
constexpr size_t NA_ACC = align256((size_t)NA_MAX_REQ * 4);
constexpr size_t NA_CHUNKS = align256((size_t)2 * NA_MAX_REQ * NA_MAX_CHUNKS * 4);
constexpr size_t NA_POST = align256((size_t)NA_MAX_REQ * (NA_MAX_K + 1) * 4);
constexpr size_t NA_BYTES = NA_STATS + NA_ACC + NA_CHUNKS > NA_POST ? NA_STATS + NA_ACC + NA_CHUNKS : NA_POST;

constexpr int NA_MAX_DEVICES = 64;

}  // namespace
}  // namespace dfl

// One copy per GPU the library runs on, held until the process ends.  In host
// code this name is only a stand-in for the symbol: host code uses the address
// returned by hipGetSymbolAddress for the current device, never the name.
static __device__ __align__(256) unsigned char scratch[dfl::NA_BYTES];

namespace {
std::mutex g_na_mutex;
void* g_na_ptr[dfl::NA_MAX_DEVICES] = {};

// Device address of `scratch` on the current device, resolved on the first call there.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= dfl::NA_MAX_DEVICES) return DFLASH_E_HIP;
  std::lock_guard<std::mutex> lock(g_na_mutex);
  if (!g_na_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DFLASH_E_HIP;
    g_na_ptr[dev] = ptr;
  }
  *out = g_na_ptr[dev];
  return DFLASH_OK;
}
}  // namespace

extern "C" int dflash_verify_noalloc(void* stream, int32_t n_req, int32_t K, int32_t vocab, const int32_t* slots,
                                     const int32_t* draft_ids, const float* draft_logits, const float* target_logits,
                                     float temperature, uint64_t seed, uint64_t step, int32_t* out_tokens,
                                     int32_t* out_len, int32_t* accept_len, int32_t* next_anchor) {
  using namespace dfl;
  if (n_req < 0 || K < 1 || vocab < 1) return DFLASH_E_INVALID;
  if (n_req > NA_MAX_REQ || K > NA_MAX_K || vocab > NA_MAX_VOCAB) return DFLASH_E_CAPACITY;
  if (n_req == 0) return DFLASH_OK;
  if (!draft_ids || !target_logits || !out_tokens || !out_len || !accept_len) return DFLASH_E_INVALID;
  if (!(temperature >= 0.f)) return DFLASH_E_INVALID;
  if (temperature > 0.f && (!draft_logits || !slots)) return DFLASH_E_INVALID;
  void* base = nullptr;
  int rc = scratch_for_current_device(&base);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  char* p = (char*)base;
  if (temperature == 0.f) {
    launch_verify_greedy(n_req, K, vocab, draft_ids, target_logits, (int32_t*)p, out_tokens, out_len, accept_len,
                         next_anchor, s);
  } else {
    // every scratch element these kernels read is written earlier in the same call
    launch_verify_rejection(n_req, K, vocab, slots, draft_ids, draft_logits, target_logits, 1.0f / temperature, seed,
                            step, (float*)p, (int32_t*)(p + NA_STATS), (float*)(p + NA_STATS + NA_ACC), out_tokens,
                            out_len, accept_len, next_anchor, nullptr, s);
  }
  return hipGetLastError() == hipSuccess ? DFLASH_OK : DFLASH_E_HIP;
}
