// C ABI of the verify step (declared in include/specdec.h): host-side argument checks and
// stream-ordered launches.  Allocates nothing, keeps no state, never synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "kernels.h"
#include "specdec.h"

static_assert(SPECDEC_SMALL_V_MAX == specdec::kSmallVMax, "small-vocabulary path limit");
static_assert(SPECDEC_PATH_ONE_LAUNCH == 3 && SPECDEC_PATH_QUAD == 4,
              "path numbering shared with kernels.h");

namespace {

bool misaligned(const void* p, size_t a) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) != 0;
}

specdec_status check_sizes(int32_t B, int32_t K, int32_t V, int32_t dtype) {
  if (B < 0 || K < 0 || K > SPECDEC_MAX_K || V < 1) return SPECDEC_ERR_SHAPE;
  if (dtype != SPECDEC_F32 && dtype != SPECDEC_BF16) return SPECDEC_ERR_DTYPE;
  // B*(K+1)*V elements must be addressable with 64-bit signed offsets (always true for
  // int32 sizes); keep the chunked work count in range as well.
  // Tile counts (rows x 8192-logit chunks) are indexed with 32-bit arithmetic on the device.
  const long long rows = static_cast<long long>(B) * (K + 1);
  if (rows * specdec::num_chunks(V) >= (1LL << 31)) return SPECDEC_ERR_SHAPE;
  return SPECDEC_OK;
}

}  // namespace

namespace specdec {

specdec_status check_verify_args(const void* target_logits, int32_t logits_dtype,
                                 const float* draft_probs, const int32_t* proposed,
                                 const int32_t* num_draft, const float* temperature,
                                 const float* uniforms, int32_t B, int32_t K, int32_t V,
                                 const int32_t* accept_len, const int32_t* out_tokens,
                                 const float* out_probs, bool greedy_all) {
  specdec_status st = check_sizes(B, K, V, logits_dtype);
  if (st != SPECDEC_OK || B == 0) return st;
  if (!target_logits || !accept_len || !out_tokens) return SPECDEC_ERR_NULL;
  if (K > 0 && !proposed) return SPECDEC_ERR_NULL;
  if (!greedy_all && (!temperature || !uniforms)) return SPECDEC_ERR_NULL;
  const size_t esize = logits_dtype == SPECDEC_BF16 ? 2 : 4;
  if (misaligned(target_logits, esize) || misaligned(draft_probs, 4) ||
      misaligned(proposed, 4) || misaligned(num_draft, 4) || misaligned(temperature, 4) ||
      misaligned(uniforms, 4) || misaligned(accept_len, 4) || misaligned(out_tokens, 4) ||
      misaligned(out_probs, 4))
    return SPECDEC_ERR_ALIGN;
  return SPECDEC_OK;
}

}  // namespace specdec

namespace {

specdec_status run(const void* target_logits, int32_t logits_dtype, const float* draft_probs,
                   const uint8_t* draft_onehot, const int32_t* proposed,
                   const int32_t* num_draft, const float* temperature, const float* uniforms,
                   int32_t B, int32_t K, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                   float* out_probs, void* workspace, size_t workspace_bytes, void* stream,
                   const specdec_options* opts, bool greedy_all, bool match = false) {
  const specdec_status st = specdec::check_verify_args(
      target_logits, logits_dtype, draft_probs, proposed, num_draft, temperature, uniforms, B, K,
      V, accept_len, out_tokens, out_probs, greedy_all);
  if (st != SPECDEC_OK || B == 0) return st;
  if (!workspace) return SPECDEC_ERR_NULL;
  if (misaligned(workspace, 16)) return SPECDEC_ERR_ALIGN;
  if (workspace_bytes < specdec::workspace_bytes(B, K, V)) return SPECDEC_ERR_WORKSPACE;

  specdec::LaunchArgs a{};
  a.logits = target_logits;
  a.logits_bf16 = logits_dtype == SPECDEC_BF16;
  a.draft_probs = greedy_all ? nullptr : draft_probs;
  a.onehot = greedy_all ? nullptr : draft_onehot;
  a.proposed = proposed;
  a.num_draft = num_draft;
  a.temperature = greedy_all ? nullptr : temperature;
  a.uniforms = greedy_all ? nullptr : uniforms;
  a.B = B;
  a.K = K;
  a.V = V;
  a.greedy_all = greedy_all ? 1 : 0;
  a.match = match ? 1 : 0;
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.out_probs = out_probs;
  a.workspace = workspace;
  a.stream = static_cast<hipStream_t>(stream);
  a.hot_begin = opts ? static_cast<hipEvent_t>(opts->hot_event_begin) : nullptr;
  a.hot_end = opts ? static_cast<hipEvent_t>(opts->hot_event_end) : nullptr;
  a.draw_begin = opts ? static_cast<hipEvent_t>(opts->draw_event_begin) : nullptr;
  a.draw_end = opts ? static_cast<hipEvent_t>(opts->draw_event_end) : nullptr;
  a.path = opts ? opts->path : SPECDEC_PATH_AUTO;
  a.spin_limit = opts ? opts->spin_limit : 0;
  if (a.spin_limit < 0) return SPECDEC_ERR_SHAPE;
  if (a.path != SPECDEC_PATH_AUTO && a.path != SPECDEC_PATH_STREAMING &&
      a.path != SPECDEC_PATH_SMALL_VOCAB && a.path != SPECDEC_PATH_ONE_LAUNCH &&
      a.path != SPECDEC_PATH_QUAD)
    return SPECDEC_ERR_SHAPE;
  if (a.path == SPECDEC_PATH_SMALL_VOCAB && V > SPECDEC_SMALL_V_MAX)
    return SPECDEC_ERR_SHAPE;
  if (a.path == SPECDEC_PATH_QUAD && !specdec::quad_eligible(a)) return SPECDEC_ERR_SHAPE;
  return specdec::launch_verify(a) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

specdec_status check_ngram_sizes(int32_t B, int32_t capacity, int32_t n_min, int32_t n_max,
                                 int32_t K) {
  if (B < 0 || capacity < 1 || K < 0 || K > SPECDEC_MAX_K) return SPECDEC_ERR_SHAPE;
  if (n_min < 1 || n_max < n_min || n_max > SPECDEC_NGRAM_MAX_N) return SPECDEC_ERR_SHAPE;
  if (static_cast<long long>(B) * specdec::ngram_tiles(capacity) >= (1LL << 31))
    return SPECDEC_ERR_SHAPE;
  return SPECDEC_OK;
}

}  // namespace

extern "C" {

size_t specdec_ngram_workspace_size(int32_t B, int32_t capacity) {
  if (check_ngram_sizes(B, capacity, 1, 1, 0) != SPECDEC_OK || B == 0) return 0;
  return static_cast<size_t>(B) * specdec::ngram_tiles(capacity) * sizeof(unsigned long long);
}

specdec_status specdec_ngram_propose(const int32_t* tokens, const int32_t* lengths, int32_t B,
                                     int32_t capacity, int32_t n_min, int32_t n_max, int32_t K,
                                     int32_t* proposed, int32_t* num_draft, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const specdec_status st = check_ngram_sizes(B, capacity, n_min, n_max, K);
  if (st != SPECDEC_OK) return st;
  if (B == 0) return SPECDEC_OK;
  if (!tokens || !lengths || !num_draft || !workspace || (K > 0 && !proposed))
    return SPECDEC_ERR_NULL;
  if (misaligned(tokens, 4) || misaligned(lengths, 4) || misaligned(proposed, 4) ||
      misaligned(num_draft, 4) || misaligned(workspace, 16))
    return SPECDEC_ERR_ALIGN;
  if (workspace_bytes < specdec_ngram_workspace_size(B, capacity)) return SPECDEC_ERR_WORKSPACE;
  specdec::NgramArgs a{};
  a.tokens = tokens;
  a.lengths = lengths;
  a.B = B;
  a.capacity = capacity;
  a.n_min = n_min;
  a.n_max = n_max;
  a.K = K;
  a.proposed = proposed;
  a.num_draft = num_draft;
  a.partials = static_cast<unsigned long long*>(workspace);
  a.stream = static_cast<hipStream_t>(stream);
  return specdec::launch_ngram(a) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

size_t specdec_workspace_size(int32_t B, int32_t K, int32_t V) {
  if (check_sizes(B, K, V, SPECDEC_F32) != SPECDEC_OK || B == 0) return 0;
  return specdec::workspace_bytes(B, K, V);
}

specdec_status specdec_verify(const void* target_logits, int32_t logits_dtype,
                              const float* draft_probs, const uint8_t* draft_onehot,
                              const int32_t* proposed, const int32_t* num_draft,
                              const float* temperature, const float* uniforms, int32_t B,
                              int32_t K, int32_t V, int32_t* accept_len, int32_t* out_tokens,
                              float* out_probs, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return run(target_logits, logits_dtype, draft_probs, draft_onehot, proposed, num_draft,
             temperature, uniforms, B, K, V, accept_len, out_tokens, out_probs, workspace,
             workspace_bytes, stream, nullptr, false);
}

specdec_status specdec_verify_ex(const void* target_logits, int32_t logits_dtype,
                                 const float* draft_probs, const uint8_t* draft_onehot,
                                 const int32_t* proposed, const int32_t* num_draft,
                                 const float* temperature, const float* uniforms, int32_t B,
                                 int32_t K, int32_t V, int32_t* accept_len,
                                 int32_t* out_tokens, float* out_probs, void* workspace,
                                 size_t workspace_bytes, void* stream,
                                 const specdec_options* opts) {
  return run(target_logits, logits_dtype, draft_probs, draft_onehot, proposed, num_draft,
             temperature, uniforms, B, K, V, accept_len, out_tokens, out_probs, workspace,
             workspace_bytes, stream, opts, false);
}

specdec_status specdec_verify_greedy(const void* target_logits, int32_t logits_dtype,
                                     const int32_t* proposed, const int32_t* num_draft,
                                     int32_t B, int32_t K, int32_t V, int32_t* accept_len,
                                     int32_t* out_tokens, float* out_probs, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return run(target_logits, logits_dtype, nullptr, nullptr, proposed, num_draft, nullptr,
             nullptr, B, K, V, accept_len, out_tokens, out_probs, workspace, workspace_bytes,
             stream, nullptr, true);
}

specdec_status specdec_verify_match(const void* target_logits, int32_t logits_dtype,
                                    const int32_t* proposed, const int32_t* num_draft,
                                    const float* temperature, const float* uniforms, int32_t B,
                                    int32_t K, int32_t V, int32_t* accept_len,
                                    int32_t* out_tokens, float* out_probs, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return run(target_logits, logits_dtype, nullptr, nullptr, proposed, num_draft, temperature,
             uniforms, B, K, V, accept_len, out_tokens, out_probs, workspace, workspace_bytes,
             stream, nullptr, false, true);
}

specdec_status specdec_commit(const int32_t* accept_len, const int32_t* out_tokens, int32_t B,
                              int32_t K, int32_t* tokens, int32_t capacity, int32_t* seq_len,
                              int32_t* target_kv_len, int32_t* draft_kv_len,
                              int32_t* packed_tokens, int32_t* packed_offsets, void* stream) {
  if (B < 0 || K < 0 || K > SPECDEC_MAX_K || capacity < 1) return SPECDEC_ERR_SHAPE;
  if (static_cast<long long>(B) * (K + 1) >= (1LL << 31)) return SPECDEC_ERR_SHAPE;
  if (B > 0 && (!accept_len || !out_tokens || !seq_len)) return SPECDEC_ERR_NULL;
  if (misaligned(accept_len, 4) || misaligned(out_tokens, 4) || misaligned(tokens, 4) ||
      misaligned(seq_len, 4) || misaligned(target_kv_len, 4) || misaligned(draft_kv_len, 4) ||
      misaligned(packed_tokens, 4) || misaligned(packed_offsets, 4))
    return SPECDEC_ERR_ALIGN;
  specdec::CommitArgs a{};
  a.accept_len = accept_len;
  a.out_tokens = out_tokens;
  a.B = B;
  a.K = K;
  a.capacity = capacity;
  a.tokens = tokens;
  a.seq_len = seq_len;
  a.target_kv = target_kv_len;
  a.draft_kv = draft_kv_len;
  a.packed = packed_tokens;
  a.offsets = packed_offsets;
  a.stream = static_cast<hipStream_t>(stream);
  return specdec::launch_commit(a) == hipSuccess ? SPECDEC_OK : SPECDEC_ERR_LAUNCH;
}

const char* specdec_status_string(int32_t status) {
  switch (status) {
    case SPECDEC_OK: return "ok";
    case SPECDEC_ERR_NULL: return "a required pointer is NULL";
    case SPECDEC_ERR_SHAPE: return "invalid sizes or parameters";
    case SPECDEC_ERR_DTYPE: return "unsupported logits dtype";
    case SPECDEC_ERR_ALIGN: return "a tensor is not aligned to its element size";
    case SPECDEC_ERR_WORKSPACE: return "workspace too small";
    case SPECDEC_ERR_LAUNCH: return "kernel launch failed";
    case SPECDEC_ERR_SCRATCH:
      return "sizes need more workspace than specdec_verify_noalloc's built-in scratch";
    default: return "unknown status";
  }
}

int32_t specdec_version(void) { return 100; }

}  // extern "C"
