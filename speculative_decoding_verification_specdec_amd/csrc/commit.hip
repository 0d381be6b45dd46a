// gfx950 kernel of the post-verify commit: cache rollback and ragged compaction.
//
// After the verify step each sequence keeps its A accepted drafts plus the correction or bonus
// token, so its history grows by A + 1 tokens and every cache entry past the first L + A tokens
// is dropped by moving the cache length back ("Decodificação especulativa explicada",
// gsantana.dev, section "O ciclo de rascunho e verificação": truncate the cache or move a
// pointer back, for the target and the drafter alike; "ch15 · Speculative Decoding",
// snowch.github.io, section "The build").  The emitted tokens of the whole batch are also packed
// into one ragged stream with exclusive-prefix-sum offsets, since every sequence accepts a
// different number ("Speculative decoding: el secretario...", blog.lo0.es, section "Pitfalls
// operacionales", continuous batching).
//
// One 1024-thread workgroup: thread t owns sequences [t*per, (t+1)*per); their emitted counts
// are summed and scanned across the workgroup (wave shuffles, then the 16 wave totals in LDS).
// For batches up to 4096 sequences the counts, lengths and offsets are staged in LDS and the
// tokens are copied over the flattened (sequence, slot) space, so that the copies coalesce;
// larger batches copy per sequence.  No atomics.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace specdec {
namespace {

constexpr int kCmThreads = 1024;
constexpr int kCmWaves = kCmThreads / 64;
constexpr int kCmLds = 4096;  // batches up to this size stage per-sequence data in LDS
constexpr int kCmBatch = 8;   // emitted-token slots per thread whose loads go out together

// Tokens sequence b commits: A + 1, or 0 for an invalid row / length / overflow.
__device__ __forceinline__ int emitted_count(int A, int L, int K, int capacity) {
  if (A < 0 || A > K || L < 0) return 0;
  if (static_cast<long long>(L) + A + 1 > capacity) return 0;
  return A + 1;
}

__global__ __launch_bounds__(kCmThreads) void commit_kernel(
    const int32_t* __restrict__ accept_len, const int32_t* __restrict__ out_tokens, int B, int K,
    int capacity, int32_t* __restrict__ tokens, int32_t* __restrict__ seq_len,
    int32_t* __restrict__ target_kv, int32_t* __restrict__ draft_kv,
    int32_t* __restrict__ packed, int32_t* __restrict__ offsets) {
  __shared__ int sh_wave[kCmWaves];
  __shared__ int sh_em[kCmLds], sh_base[kCmLds], sh_len[kCmLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (B + kCmThreads - 1) / kCmThreads;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  const bool staged = B <= kCmLds;  // per-sequence data fits LDS: coalesced copies below
  const int items = B * (K + 1);
  // Loads that do not depend on the scan go out first: the first batch of emitted-token slots
  // (flattened index tid + j * kCmThreads, clamped into range) and the first cache lengths.
  int32_t tok0[kCmBatch];
  int tkv0 = 0, dkv0 = 0;
  if (staged) {
#pragma unroll
    for (int j = 0; j < kCmBatch; ++j)
      tok0[j] = items > 0 ? out_tokens[min(tid + j * kCmThreads, items - 1)] : 0;
    if (tid < B) {
      if (target_kv) tkv0 = target_kv[tid];
      if (draft_kv) dkv0 = draft_kv[tid];
    }
  }
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    const int A = accept_len[b], L = seq_len[b];
    const int em = emitted_count(A, L, K, capacity);
    if (staged) {
      sh_em[b] = em;
      sh_len[b] = L;
    }
    local += em;
  }
  // Exclusive scan of the per-thread counts over the workgroup.
  int inc = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off, 64);
    if (lane >= off) inc += y;
  }
  if (lane == 63) sh_wave[wave] = inc;
  __syncthreads();
  int base = inc - local;
  for (int w = 0; w < wave; ++w) base += sh_wave[w];
  if (tid == kCmThreads - 1 && offsets) offsets[B] = base + local;
  if (staged) {
    for (int b = b0; b < b1; ++b) {
      sh_base[b] = base;
      if (offsets) offsets[b] = base;
      base += sh_em[b];
    }
    __syncthreads();
    // Token copies over the flattened (sequence, slot) space: consecutive threads take
    // consecutive slots of a row, so the reads of out_tokens and the writes of the history and
    // of the packed stream coalesce.
    // Batches of kCmBatch slots per thread, every load of a batch issued before its stores.
    for (int g0 = 0; g0 < items; g0 += kCmBatch * kCmThreads) {
      int32_t tv[kCmBatch];
      if (g0 == 0) {
#pragma unroll
        for (int j = 0; j < kCmBatch; ++j) tv[j] = tok0[j];
      } else {
#pragma unroll
        for (int j = 0; j < kCmBatch; ++j)
          tv[j] = out_tokens[min(g0 + tid + j * kCmThreads, items - 1)];
      }
#pragma unroll
      for (int j = 0; j < kCmBatch; ++j) {
        const int g = g0 + tid + j * kCmThreads;
        if (g >= items) break;
        const int b = g / (K + 1), i = g - b * (K + 1);
        if (i < sh_em[b]) {
          if (tokens) tokens[static_cast<long long>(b) * capacity + sh_len[b] + i] = tv[j];
          if (packed) packed[sh_base[b] + i] = tv[j];
        }
      }
    }
    for (int b = tid; b < B; b += kCmThreads) {
      const int em = sh_em[b];
      int tkv = tkv0, dkv = dkv0;
      if (b != tid) {
        if (target_kv) tkv = target_kv[b];
        if (draft_kv) dkv = draft_kv[b];
      }
      if (em > 0) {
        const int L = sh_len[b];
        seq_len[b] = L + em;
        if (target_kv) target_kv[b] = min(tkv, L + em - 1);
        if (draft_kv) draft_kv[b] = min(dkv, L + em - 1);
      }
    }
    return;
  }
  // Larger batches: each thread copies its own sequences.
  for (int b = b0; b < b1; ++b) {
    const int A = accept_len[b], L = seq_len[b];
    const int em = emitted_count(A, L, K, capacity);
    if (offsets) offsets[b] = base;
    if (em > 0) {
      const int32_t* src = out_tokens + static_cast<long long>(b) * (K + 1);
      int32_t* dst = tokens ? tokens + static_cast<long long>(b) * capacity + L : nullptr;
      for (int i = 0; i < em; ++i) {
        const int32_t t = src[i];
        if (dst) dst[i] = t;
        if (packed) packed[base + i] = t;
      }
      seq_len[b] = L + em;
      if (target_kv) target_kv[b] = min(target_kv[b], L + A);
      if (draft_kv) draft_kv[b] = min(draft_kv[b], L + A);
    }
    base += em;
  }
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a) {
  if (a.B == 0 && !a.offsets) return hipSuccess;  // B == 0 still writes offsets[0] = 0
  commit_kernel<<<1, kCmThreads, 0, a.stream>>>(a.accept_len, a.out_tokens, a.B, a.K,
                                                a.capacity, a.tokens, a.seq_len, a.target_kv,
                                                a.draft_kv, a.packed, a.offsets);
  return hipGetLastError();
}

}  // namespace specdec
