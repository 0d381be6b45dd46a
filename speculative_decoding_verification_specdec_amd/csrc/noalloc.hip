// specdec_verify_noalloc: specdec_verify with the workspace in a file-scope device array instead
// of a caller buffer, for callers that cannot allocate device memory (code under HIP-graph capture,
// tight serving loops, harnesses that forbid allocation).  Declared in include/specdec.h.
//
// The array `scratch` holds SPECDEC_NOALLOC_SCRATCH_BYTES per device for the life of the process.
// In host code its name is only a host-side stand-in, so each device's address is looked up once
// (hipGetSymbolAddress, with that device current, on the first call whose stream belongs to it)
// and only that address is handed to the kernels.  Every call on a device shares that device's array: calls that
// overlap in time on one device race (the verify kernels need no initialised workspace, so
// consecutive calls do not).
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "kernels.h"
#include "specdec.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SPECDEC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// The address of `scratch` on the device the kernels will run on -- the stream's device (the
// null stream: the current device) -- looked up on the first call there with that device made
// current for the lookup (and the caller's current device restored); null on error.
void* scratch_address(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return nullptr;
    dev = static_cast<int>(d);
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (err != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

namespace specdec {
// Host checks of a verify call's arguments other than its workspace (api.cpp).
specdec_status check_verify_args(const void* target_logits, int32_t logits_dtype,
                                 const float* draft_probs, const int32_t* proposed,
                                 const int32_t* num_draft, const float* temperature,
                                 const float* uniforms, int32_t B, int32_t K, int32_t V,
                                 const int32_t* accept_len, const int32_t* out_tokens,
                                 const float* out_probs, bool greedy_all);
}  // namespace specdec

extern "C" {

size_t specdec_noalloc_scratch_bytes(void) { return SPECDEC_NOALLOC_SCRATCH_BYTES; }

specdec_status specdec_verify_noalloc(const void* target_logits, int32_t logits_dtype,
                                      const float* draft_probs, const uint8_t* draft_onehot,
                                      const int32_t* proposed, const int32_t* num_draft,
                                      const float* temperature, const float* uniforms, int32_t B,
                                      int32_t K, int32_t V, int32_t* accept_len,
                                      int32_t* out_tokens, float* out_probs, void* stream) {
  // Every host check first -- the arguments as specdec_verify checks them, then whether the
  // workspace fits the array -- so that a refused call never touches the device.
  const specdec_status st = specdec::check_verify_args(
      target_logits, logits_dtype, draft_probs, proposed, num_draft, temperature, uniforms, B, K,
      V, accept_len, out_tokens, out_probs, false);
  if (st != SPECDEC_OK || B == 0) return st;
  if (specdec_workspace_size(B, K, V) > SPECDEC_NOALLOC_SCRATCH_BYTES) return SPECDEC_ERR_SCRATCH;
  void* ws = scratch_address(static_cast<hipStream_t>(stream));
  if (ws == nullptr) return SPECDEC_ERR_LAUNCH;
  return specdec_verify(target_logits, logits_dtype, draft_probs, draft_onehot, proposed,
                        num_draft, temperature, uniforms, B, K, V, accept_len, out_tokens,
                        out_probs, ws, SPECDEC_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
