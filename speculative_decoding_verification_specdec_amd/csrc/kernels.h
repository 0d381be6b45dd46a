// Internal interface between the C-ABI host code (api.cpp) and the gfx950 kernels
// (kernels.hip).  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specdec {

constexpr int kThreads = 256;               // 4 x wave64 per workgroup
constexpr int kChunk = 8192;                // logits per row chunk (one workgroup tile)
constexpr int kGroup = 8;                   // consecutive tokens per thread in the draw passes
constexpr int kSeg = kThreads * kGroup;     // 2048 tokens per draw segment
constexpr int kSegPerChunk = kChunk / kSeg; // 4
constexpr unsigned kXcdBlock = 64;          // tiles per XCD block in the blocked streaming order
constexpr unsigned long long kXcdBlockMinBytes = 256ull << 20;  // streams that take it

// Per (row, 2048-token sub-chunk) partial statistics of the streaming pass.  The 16-byte
// records (also SeqState, Gather, SegSums) are 16-byte aligned so each is one vector load.
struct alignas(16) RowPartial {
  float m;      // max logit in the sub-chunk (-inf if none)
  float s;      // sum of exp2((z - m) * c) over the sub-chunk
  int32_t arg;  // lowest index attaining m (greedy rows only)
  float pre;    // match mode: the same sum over the tokens below the drafted id x_i
};

// What the draw pass must sample for one sequence.
enum SampleMode : int32_t {
  kNone = 0,            // nothing to draw (greedy, invalid, or already emitted)
  kResidual = 1,        // max(0, p_j - q_j) for a model-draft row
  kResidualOnehot = 2,  // p_j with the rejected draft x_j removed (one-hot / n-gram row)
  kBonus = 3,           // p_k (every draft accepted)
};

struct alignas(16) SeqState {
  int32_t mode;   // SampleMode
  int32_t row;    // target row j the draw is taken from
  int32_t excl;   // x_j for kResidualOnehot
  int32_t ucol;   // uniforms column of the draw (K; in match mode the mismatching position)
  float c;        // log2(e) / T
  float m;        // max of row j
  float s;        // sum_v exp2((z_j[v] - m) * c) of row j
  float pad1;
};

// One drafted slot's gathered inputs, recorded by the streaming kernel: the proposed id x_i,
// the target logit z_i[x_i] and the drafter probability q_i(x_i).
struct alignas(16) Gather {
  float z;
  float q;
  int32_t x;
  int32_t pad;
};

// Weight sums of one 2048-token draw segment.
struct alignas(16) SegSums {
  double w;       // the draw's weights
  double e;       // exp2((z - m) * c), i.e. s * p (fallback when the residual is empty)
};

inline int num_chunks(int V) { return (V + kChunk - 1) / kChunk; }

// Caller-provided device workspace of the three-launch path (no initialisation needed;
// contents are meaningless between calls).
struct Workspace {
  RowPartial* partials;  // [B*(K+1)*S*4], 4 sub-chunks per chunk
  Gather* gathers;       // [B*K]
  SeqState* states;      // [B]
  SegSums* segs;         // [B*S*kSegPerChunk]
  unsigned long long* segw;  // [B*S*kSegPerChunk*4] segment sums as marked words (in-kernel pick)
};

struct WorkspaceLayout {
  size_t partials, gathers, states, segs, segw, total;
};

// Byte layout of the three-launch path's workspace for these sizes.
WorkspaceLayout workspace_layout(int B, int K, int V);

// Per-sequence record of the one-launch path (fused.hip), in 64-bit words: the hand-off words of one
// sequence's round (see kernels.hip).  Zero between calls: every completed call puts back to zero
// every word it set, so the workspace must be zero-filled before its first use with given K, V.
struct RecordLayout {
  long long partials;  // (K+1) rows x S chunks x 4 waves x 4 words (max, sum, argmax, sum below x_i)
  long long gathers;   // K slots x 4 words (x_i, z_i[x_i], q_i(x_i), unused)
  long long segs;      // S*4 segments x 4 words (two doubles, in halves)
  long long done;      // one word per closing tile (at most 4 S)
  long long pick;      // 2 words: the drawn token and its probability
  long long words;     // record size, a multiple of 32 words (256 bytes)
};

__host__ __device__ inline RecordLayout record_layout(int K, int V) {
  const long long S = (V + kChunk - 1) / kChunk;
  RecordLayout L;
  L.partials = 0;
  L.gathers = L.partials + static_cast<long long>(K + 1) * S * 4 * 4;
  L.segs = L.gathers + static_cast<long long>(K) * 4;
  L.done = L.segs + S * kSegPerChunk * 4;
  L.pick = L.done + S * kSegPerChunk;
  L.words = (L.pick + 2 + 31) & ~31LL;
  return L;
}

// Bytes of workspace a verify call needs: enough for either streaming path.
size_t workspace_bytes(int B, int K, int V);

struct LaunchArgs {
  const void* logits;
  int logits_bf16;           // 1: bf16 bit patterns, 0: fp32
  const float* draft_probs;
  const uint8_t* onehot;
  const int32_t* proposed;
  const int32_t* num_draft;
  const float* temperature;
  const float* uniforms;
  int B, K, V;
  int greedy_all;            // 1: every row is temperature 0 (no q, T, u read)
  int match;                 // 1: sample-and-match mode (q never read)
  int32_t* accept_len;
  int32_t* out_tokens;
  float* out_probs;
  void* workspace;           // B records, zero between calls
  hipStream_t stream;
  hipEvent_t hot_begin;      // optional, recorded around the streaming (or small-vocabulary)
  hipEvent_t hot_end;        // kernel
  hipEvent_t draw_begin;     // optional, recorded around the kernels after the streaming kernel
  hipEvent_t draw_end;       // (streaming path)
  int path;                  // 0: automatic, 1: three launches, 2: small-vocabulary kernel,
                             // 3: one launch, 4: four workgroups per sequence, one launch
  int spin_limit;            // polls of the one-launch path's bounded waits (0: the default)
};

// Largest vocabulary the small-vocabulary path takes (four 4-token quads per lane of a wave).
constexpr int kSmallVMax = 1024;

// Four workgroups per sequence, one launch (quad.hip): quarter q of every row covers tokens
// [q * span, (q + 1) * span), span a whole number of 2048-token segments, at most kMaxQuadSeg.
constexpr int kMaxQuadSeg = 32;
__host__ __device__ inline int quad_span(int V) {
  return (V + 4 * kSeg - 1) / (4 * kSeg) * kSeg;
}
size_t quad_workspace_bytes(int B, int K, int V);
bool quad_eligible(const LaunchArgs& a);  // shapes, alignment, and the whole grid resident at once
hipError_t launch_quad(const LaunchArgs& a);

hipError_t launch_verify(const LaunchArgs& a);
hipError_t launch_small_verify(const LaunchArgs& a);  // small.hip; V <= kSmallVMax
hipError_t launch_one_launch(const LaunchArgs& a);    // fused.hip

// ---- n-gram drafter (ngram.hip) ----
constexpr int kNgramTile = 8192;   // candidate positions per workgroup
constexpr int kNgramMaxN = 32;     // longest suffix tried

inline int ngram_tiles(int capacity) { return (capacity + kNgramTile - 1) / kNgramTile; }

struct NgramArgs {
  const int32_t* tokens;     // [B, capacity]
  const int32_t* lengths;    // [B]
  int B, capacity, n_min, n_max, K;
  int32_t* proposed;         // [B, K] (may be null when K == 0)
  int32_t* num_draft;        // [B]
  unsigned long long* partials;  // workspace [B * ngram_tiles(capacity)]
  hipStream_t stream;
};

hipError_t launch_ngram(const NgramArgs& a);

// ---- commit: rollback and ragged compaction (commit.hip) ----
struct CommitArgs {
  const int32_t* accept_len;   // [B]
  const int32_t* out_tokens;   // [B, K+1]
  int B, K, capacity;
  int32_t* tokens;             // [B, capacity] history, or null
  int32_t* seq_len;            // [B] in/out
  int32_t* target_kv;          // [B] in/out, or null
  int32_t* draft_kv;           // [B] in/out, or null
  int32_t* packed;             // [B*(K+1)] out, or null
  int32_t* offsets;            // [B+1] out, or null
  hipStream_t stream;
};

hipError_t launch_commit(const CommitArgs& a);

// ---- acceptance telemetry and per-route draft length (telemetry.hip) ----
constexpr int kTelemetryFields = 8;
constexpr int kTelemetryBins = 64;
constexpr int kTelemetryRow = kTelemetryFields + kTelemetryBins;
constexpr int kTelemetryMaxRoutes = 64;

hipError_t launch_telemetry(const int32_t* accept_len, const int32_t* num_draft,
                            const int32_t* route, int B, int K, int n_routes,
                            long long* counters, hipStream_t stream);
hipError_t launch_apply_k(int32_t* num_draft, const int32_t* route, const int32_t* k_table,
                          int B, int n_routes, hipStream_t stream);

}  // namespace specdec
