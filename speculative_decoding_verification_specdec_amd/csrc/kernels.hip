// gfx950 (CDNA4) kernels of the batched speculative-decoding verify step, three launches.
//
// The step (draft-then-verify with rejection sampling) is the one the three source pages
// define: "Decodificação especulativa explicada" (gsantana.dev), section "A regra de
// amostragem por rejeição"; "ch15 · Speculative Decoding" (snowch.github.io), section "Why
// the result is exactly the target model"; "Speculative decoding: el secretario que adelanta
// lo que va a decir el jefe" (blog.lo0.es), section "El mecanismo desnudo".
//
// Three kernels, enqueued back to back on the caller's stream.  They communicate only through
// the workspace across kernel boundaries: no atomics, no inter-workgroup waiting.
//   stats_kernel   one 256-thread workgroup per (8192-logit chunk, used target row).  Each wave
//       issues its 2048-token sub-chunk's 16-byte loads first, reduces the wave max, then sums
//       exp2((z - max) * log2(e)/T) against it and writes one (max, sum, lowest argmax)
//       partial per wave; chunk 0 of each drafted row also gathers x_i, z_i[x_i] and q_i(x_i).
//   accept_draw_kernel  one workgroup per (chunk of the row to draw from, sequence), or per
//       2048-token segment when the grid is smaller than the chip.  Every wave merges some rows'
//       sub-chunk partials (16 lanes per row, max-first, DPP) and wave 0 runs the sequence's accept
//       scan (lane i <-> target row i, p_i(x_i) in fp64, a 64-bit ballot finds the first rejection);
//       the chunk-0 workgroup emits every token already known (accepted drafts, greedy argmaxes) and
//       records what remains to be drawn.  Then the workgroup sums the draw's weights -- s * max(0, p
//       - q) or p without the rejected draft -- over each 2048-token segment of its chunk (fp64 DPP
//       wave sums); a plain draw of p takes those sums from the streaming kernel's partials instead,
//       and so does a one-hot residual in every segment but the rejected draft's.
//   pick_kernel  one workgroup per sequence that needs a draw: one fp64 DPP scan over the
//       segment sums finds the segment holding u * total, then a scan of that one segment in
//       ascending token order finds the first running sum above u * total.
// The sample-and-match mode uses the same three kernels (template flag): the streaming kernel
// also sums below each drafted id, the scan decides y_i == x_i from those sums, and the draw is
// a plain sample of p at the first mismatch.
// Every reduction combines in a fixed order, so results are bit-reproducible.
#include <float.h>
#include <limits.h>
#include <math.h>

#include <algorithm>

#include <hip/hip_ext.h>

#include "kernels.h"
#include "verify_dev.h"
#include "wave_ops.h"

namespace specdec {
namespace {

// Their loads, issued unconditionally so that all of them -- and the partials after them -- are
// in flight together: an absent operand (null pointer, or no drafted slot) is read from `any`, a
// valid 16-byte-aligned stand-in, and discarded by finish_scan_in.  Lane min(i, K) reads
// uniforms column i, so lane K holds column K.
struct ScanLoads {
  Gather g;
  float u;
  uint8_t oh;
};

__device__ __forceinline__ ScanLoads load_scan_in(const uint8_t* onehot, const float* uniforms,
                                                  const Gather* gathers, const void* any, int b,
                                                  int K, int lane) {
  const long long row0 = static_cast<long long>(b) * (K + 1);
  const Gather* gp = K > 0 ? gathers + static_cast<long long>(b) * K + min(lane, K - 1)
                           : static_cast<const Gather*>(any);
  const float* up = uniforms != nullptr ? uniforms + row0 + min(lane, K)
                                        : static_cast<const float*>(any);
  // Lane 0 reads the flag (the others the stand-in) and finish_scan_in broadcasts it.
  const uint8_t* op = (onehot != nullptr && lane == 0) ? onehot + b
                                                       : static_cast<const uint8_t*>(any);
  return ScanLoads{*gp, *up, *op};
}

__device__ __forceinline__ ScanIn finish_scan_in(const ScanLoads& r, const uint8_t* onehot,
                                                 const float* uniforms, int K, int lane) {
  ScanIn in;
  in.g = lane < K ? r.g : Gather{0.f, 0.f, -1, 0};
  in.u = (uniforms != nullptr && lane < K) ? r.u : 0.f;
  in.uk = uniforms != nullptr ? read_lane_f(r.u, K) : 0.f;
  in.onehot = onehot != nullptr && __builtin_amdgcn_readlane(static_cast<int>(r.oh), 0) != 0;
  return in;
}

// The scan's global writes, made after the workgroup barrier that publishes the state in LDS
// (a barrier waits for every outstanding store of the workgroup).
__device__ __forceinline__ void write_scan_out(const ScanOut& o, int b, int K,
                                               int32_t* accept_len, int32_t* out_tokens,
                                               float* out_probs, SeqState* states, int lane) {
  const long long row0 = static_cast<long long>(b) * (K + 1);
  if (lane <= K) {
    out_tokens[row0 + lane] = o.tok;
    if (out_probs) out_probs[row0 + lane] = static_cast<float>(o.num / o.den);
  }
  if (lane == 0) {
    accept_len[b] = o.A;
    states[b] = o.st;
  }
}

// Row statistics of rows 0..K of one sequence, by every wave of the workgroup: 16 lanes per
// row, wave w taking rows 4w .. 4w+3 of each 16-row pass, each lane loading up to 8 of its
// row's sub-chunk partials (l, l + 16, ...) before merging them max-first; the row's lanes then
// reduce with DPP and lane 0 of the row stores it in LDS.  Rows past k_b are merged too (their
// partials are stale) and ignored.  With `use_d` (match mode, sampled rows) the merge is the
// fp64 one of S_i and P_i.
//
// The loads are unconditional (indices clamped into the row, out-of-range values replaced
// after they arrive), and the first batch -- the whole merge while K + 1 <= 16 rows and a row
// has at most 128 partials -- is issued by prefetch_partials before the kernel reads the draft
// count and temperature, so no load waits behind a branch or a scalar load.
struct PartialBatch {
  RowPartial a[4], b[4];
};

__device__ __forceinline__ void load_partial_batch(const RowPartial* __restrict__ partials,
                                                   long long row0, int K, int nsub, int i0,
                                                   int t0, int lane, PartialBatch& p) {
  const int ri = i0 + (lane >> 4), sl = lane & 15;
  const RowPartial* P = partials + (row0 + min(ri, K)) * nsub;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    p.a[t] = P[min(sl + 16 * (t0 + t), nsub - 1)];
    p.b[t] = P[min(sl + 16 * (t0 + 4 + t), nsub - 1)];
  }
}

__device__ __forceinline__ void prefetch_partials(const RowPartial* __restrict__ partials,
                                                  long long row0, int K, int nsub, int wave,
                                                  int lane, PartialBatch& p) {
  load_partial_batch(partials, row0, K, nsub, min(4 * wave, K), 0, lane, p);
}

template <bool kMatch>
__device__ __forceinline__ void row_stats(const RowPartial* __restrict__ partials, long long row0,
                                          int K, int nsub, float c, bool use_d, int wave,
                                          int lane, const PartialBatch& batch0, Stat* sh_rows,
                                          StatD* sh_rows_d) {
  const int per_lane = (nsub + 15) / 16;
  const int sl = lane & 15;
  const RowPartial empty{-INFINITY, 0.f, INT_MAX, 0.f};
  for (int i0 = 4 * wave; i0 <= K; i0 += 4 * kWaves) {  // wave-uniform
    const int ri = i0 + (lane >> 4);
    Stat v{-INFINITY, 0.f, INT_MAX};
    StatD vd{-INFINITY, 0.0, 0.0};
    auto merge_batch = [&](PartialBatch p, int t0) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ja = sl + 16 * (t0 + t), jb = sl + 16 * (t0 + 4 + t);
        if (!(ri <= K && ja < nsub)) p.a[t] = empty;
        if (!(ri <= K && jb < nsub)) p.b[t] = empty;
      }
      if (kMatch && use_d) {
        vd = merge4_d(vd, p.a, c);
        vd = merge4_d(vd, p.b, c);
      } else {
        v = merge4(v, p.a, c);
        v = merge4(v, p.b, c);
      }
    };
    int t0 = 0;
    if (i0 == 4 * wave) {  // the prefetched batch
      merge_batch(batch0, 0);
      t0 = 8;
    }
    for (; t0 < per_lane; t0 += 8) {
      PartialBatch p;
      load_partial_batch(partials, row0, K, nsub, i0, t0, lane, p);
      merge_batch(p, t0);
    }
    if (kMatch && use_d) {
      const StatD red = row16_reduce_d(vd, c);
      if (sl == 0 && ri <= K) sh_rows_d[ri] = red;
    } else {
      const Stat red = row16_reduce_mf(v, c);
      if (sl == 0 && ri <= K) sh_rows[ri] = red;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Streaming row statistics.
// ------------------------------------------------------------------------------------------
template <typename LT, bool kVec, bool kMatch, bool kXcdBlocks>
__global__ __launch_bounds__(kThreads) void stats_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const int32_t* __restrict__ proposed, const int32_t* __restrict__ num_draft,
    const float* __restrict__ temperature, int b0, int K, int V, int S, int greedy_all,
    RowPartial* __restrict__ partials, Gather* __restrict__ gathers, u64* __restrict__ segw) {
  // Grid: x = chunk, y = row within the sequence, z = sequence (offset by b0).  Each wave
  // reduces its own 2048-token sub-chunk and writes its own partial: no LDS, no barrier.
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int s = blockIdx.x, i = blockIdx.y, b = b0 + static_cast<int>(blockIdx.z);
  if constexpr (kXcdBlocks) {
    // Workgroup l of a launch runs on XCD l mod 8.  In the plain order every XCD reads chunks of
    // every row, so each XCD touches all of the buffer's pages; here blocks of kXcdBlock
    // consecutive (sequence, row, chunk) tiles are dealt to the XCDs in turn, each XCD reading
    // runs of whole rows (an eighth of the pages).  Tiles past the last whole round of blocks
    // keep the plain order.
    const unsigned nx = gridDim.x, ny = gridDim.y, nt = nx * ny * gridDim.z;
    const unsigned lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
    const unsigned full = nt / (8 * kXcdBlock) * (8 * kXcdBlock), idx = lin >> 3;
    const unsigned t =
        lin < full ? ((idx / kXcdBlock) * 8 + (lin & 7u)) * kXcdBlock + idx % kXcdBlock : lin;
    s = static_cast<int>(t % nx);
    i = static_cast<int>((t / nx) % ny);
    b = b0 + static_cast<int>(t / (nx * ny));
  }
  if (s == 0 && i == 0 && segw != nullptr) {
    // The draw kernel's segment-sum words start from zero in every call.
    u64* w = segw + static_cast<long long>(b) * S * kSegPerChunk * 4;
    for (int j = threadIdx.x; j < S * kSegPerChunk * 4; j += kThreads) w[j] = 0;
  }
  int kb = K;
  if (num_draft != nullptr) {
    kb = num_draft[b];
    if (kb < 0 || kb > K || i > kb) return;  // padding (or an invalid count): never read
  }
  const long long r = static_cast<long long>(b) * (K + 1) + i;
  const LT* row = logits + r * V;
  const int c0 = s * kChunk + wave * kSub;
  const int n = min(kSub, V - c0);
  // The loads go out first; the row's temperature is only needed to fold them.
  float x[kPerThread];
  load_sub<LT, kVec>(row, c0, n, lane, x);
  const float T = greedy_all ? 0.f : temperature[b];
  if (s == 0 && threadIdx.x == 0 && i < kb) {
    // The accept scan's gathers for drafted slot i, recorded while the stream is in flight.
    const long long slot = static_cast<long long>(b) * K + i;
    const int xi = proposed[slot];
    Gather gi{0.f, 0.f, xi, 0};
    if (xi >= 0 && xi < V) {
      gi.z = load_logit(row, xi);
      if (draft_probs != nullptr && T != 0.f) gi.q = draft_probs[slot * V + xi];
    }
    gathers[slot] = gi;
  }
  const float c = temp_valid(T) ? temp_scale(T) : kLog2e;  // invalid rows: result unused
  // Match mode also needs, per drafted sampled row, the sum below the drafted id x_i (for other
  // rows xi = -1 and that sum is 0).
  float pre = 0.f, lane_max;
  MaxSum st;
  if constexpr (kMatch) {
    // Only the sub-chunk that holds x_i takes the masked sum (a wave-uniform branch); below
    // x_i it is the whole sum, above it 0.
    const int xi = (i < kb && T != 0.f) ? proposed[static_cast<long long>(b) * K + i] : -1;
    if (xi >= c0 && xi < c0 + n) {
      st = fold_wave<LT, kVec, true>(x, c, c0, lane, xi, lane_max, pre);
    } else {
      st = fold_wave<LT, kVec, false>(x, c, c0, lane, -1, lane_max, pre);
      pre = xi >= c0 + n ? st.s : 0.f;
    }
  } else {
    st = fold_wave<LT, kVec, false>(x, c, c0, lane, -1, lane_max, pre);
  }
  // Greedy row: the lowest token index attaining the sub-chunk max.
  const int arg = T == 0.f ? lowest_token_of<LT, kVec>(x, st.m, c0) : 0;
  (void)lane_max;
  if (lane == 0)
    partials[r * (S * kWaves) + s * kWaves + wave] = RowPartial{st.m, st.s, arg, pre};
}


// Second step, the whole workgroup (after a barrier): scan segment ps.seg of row z (draft row
// q_row for a residual, else null) in ascending token order; thread 0 writes the token and its
// probability.  `any`: a valid 16-byte-aligned stand-in address for absent loads.
template <typename LT, bool kVec>
__device__ __forceinline__ void scan_draw_segment(const LT* __restrict__ z,
                                                  const float* __restrict__ q_row, const void* any,
                                                  int V, const SeqState& st, bool force_plain,
                                                  PickLds& ps, int32_t* tok, float* prob) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int seg = ps.seg;
  const bool plain = force_plain || ps.plain != 0;
  const double t = ps.t;
  const int sc = seg / kSegPerChunk, sg = seg % kSegPerChunk;
  const int cc0 = sc * kChunk, cn = min(kChunk, V - cc0);
  const int v0 = sg * kSeg + tid * kGroup;
  const int cnt = min(kGroup, cn - v0);
  const float* qs = (st.mode == kResidual && !plain) ? q_row : nullptr;
  float zg[kGroup], qg[kGroup], w[kGroup], gw, ge;
  load_group<LT, kVec>(z, qs, any, cc0 + v0, cnt, zg, qg);
  group_weights(zg, qg, cc0 + v0, cnt, st, plain, w, gw, ge);
  const double inc = wave_inclusive_scan(static_cast<double>(gw));
  if (lane == 63) ps.wtot[wave] = inc;
  __syncthreads();
  double before = ps.base;
  for (int k = 0; k < wave; ++k) before += ps.wtot[k];
  before += inc - static_cast<double>(gw);
  int hit = -1, lastpos = -1;
  float zhit = 0.f, zlast = 0.f, run = 0.f;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    run += w[j];
    if (w[j] > 0.f) {
      lastpos = cc0 + v0 + j;
      zlast = zg[j];
      if (hit < 0 && before + static_cast<double>(run) > t) { hit = cc0 + v0 + j; zhit = zg[j]; }
    }
  }
  const unsigned long long hm = __ballot(hit >= 0);
  const unsigned long long pm = __ballot(lastpos >= 0);
  const int hl = hm ? __ffsll(static_cast<long long>(hm)) - 1 : 0;
  const int ll = pm ? 63 - __clzll(static_cast<long long>(pm)) : 0;
  // hl and ll are wave-uniform: readlane, not a cross-lane shuffle through LDS.
  const int wave_hit = hm ? __builtin_amdgcn_readlane(hit, hl) : -1;
  const float wave_zhit = read_lane_f(zhit, hl);
  const int wave_last = pm ? __builtin_amdgcn_readlane(lastpos, ll) : -1;
  const float wave_zlast = read_lane_f(zlast, ll);
  if (lane == 0) {
    ps.hit[wave] = wave_hit; ps.zhit[wave] = wave_zhit;
    ps.lastpos[wave] = wave_last; ps.zlast[wave] = wave_zlast;
  }
  __syncthreads();
  if (tid == 0) {
    int y = -1, lp = -1;
    float zy = 0.f, zl = 0.f;
    for (int k = 0; k < kWaves; ++k) {
      if (y < 0 && ps.hit[k] >= 0) { y = ps.hit[k]; zy = ps.zhit[k]; }
      if (ps.lastpos[k] >= 0) { lp = ps.lastpos[k]; zl = ps.zlast[k]; }
    }
    // Rounding left t at the very top of the segment: take its last positive token.
    if (y < 0) {
      y = lp >= 0 ? lp : cc0 + sg * kSeg;
      zy = lp >= 0 ? zl : load_logit(z, y);
    }
    const double p = exp2((static_cast<double>(zy) - static_cast<double>(st.m)) *
                          static_cast<double>(st.c)) / static_cast<double>(st.s);
    *tok = y;
    if (prob) *prob = static_cast<float>(p);
  }
  __syncthreads();
}

// Segment j's plain weight sum of row `prow`'s partials: s_j * exp2((m_j - m) * c), the partial's
// sum rescaled to the row max.
__device__ __forceinline__ double partial_seg_sum(const RowPartial* __restrict__ prow, int j,
                                                  const SeqState& st) {
  const RowPartial pj = prow[j];
  const float f = pj.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((pj.m - st.m) * st.c);
  return static_cast<double>(pj.s) * static_cast<double>(f);
}

// Segment j's sums published by a draw workgroup as four marked words (two doubles in halves);
// false if they are not all there yet.
__device__ __forceinline__ bool seg_words(const u64* __restrict__ w, double& sw, double& se) {
  const u64 w0 = load_word(w), w1 = load_word(w + 1), e0 = load_word(w + 2), e1 = load_word(w + 3);
  if (!(is_marked(w0) && is_marked(w1) && is_marked(e0) && is_marked(e1))) return false;
  sw = __longlong_as_double(static_cast<long long>((static_cast<u64>(bits_of(w1)) << 32) | bits_of(w0)));
  se = __longlong_as_double(static_cast<long long>((static_cast<u64>(bits_of(e1)) << 32) | bits_of(e0)));
  return true;
}

// Polls of the pick's bounded wait for the other draw workgroups of its sequence.
constexpr int kPickSpinLimit = 1 << 20;

// ------------------------------------------------------------------------------------------
// Accept scan + draw weight sums.  Grid: x = chunk of the row to draw from, y = sequence (offset
// by b0).  kPhase 0: every workgroup runs its sequence's accept scan (all waves merge partials,
// wave 0 decides) and the chunk-0 workgroup writes the scan's outputs and the draw state; then
// wave w sums the draw weights of 2048-token segment w of the chunk (lane l owns the 8-token
// groups l, l + 64, ... of bf16 rows, the 4-token quads of fp32 ones), in fp64.  kPhase 1: the scan only (one workgroup per sequence).  kPhase 2:
// the draw only, from the state kPhase 1 wrote.  kPhase 3: as kPhase 0, but one workgroup per
// 2048-token segment, its four waves a quarter each (grids too small to fill the chip: a
// workgroup alone pulls its bytes through one CU's few outstanding misses).
// ------------------------------------------------------------------------------------------
template <typename LT, bool kVec, bool kMatch, int kPhase>
__global__ __launch_bounds__(kThreads, 4) void accept_draw_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const uint8_t* __restrict__ onehot, const int32_t* __restrict__ proposed,
    const int32_t* __restrict__ num_draft, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, int b0, int K, int V, int S, int greedy_all,
    const RowPartial* __restrict__ partials, const Gather* __restrict__ gathers,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ out_probs, SeqState* __restrict__ states, SegSums* __restrict__ segs,
    u64* __restrict__ segw) {
  constexpr bool kFine = kPhase == 3;
  // Draw grids of at most kDrawRound workgroups (phases 0 and 3) pick in this kernel; the split
  // phases 1 and 2 leave it to the pick kernel.
  constexpr bool pick_here = kPhase == 0 || kPhase == 3;
  constexpr int kGroupsPerLane = kSeg / kGroup / 64 / (kFine ? kWaves : 1);  // scalar path
  __shared__ SeqState sh_st;
  __shared__ SegSums sh_fine[kFine ? kWaves : 1];
  __shared__ Stat sh_rows[kMaxRows];
  __shared__ StatD sh_rows_d[kMatch ? kMaxRows : 1];
  __shared__ PickLds sh_pick;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroup x of a sequence draws chunks x, x + gridDim.x, ...  Phase 0 scans and draws;
  // phase 1 only scans (one workgroup per sequence) and phase 2 only draws, reading the state
  // phase 1 wrote: for a grid of several resident rounds the per-workgroup scan would otherwise
  // be paid in every round.
  const int b = b0 + static_cast<int>(blockIdx.y);
  const bool first = blockIdx.x == 0;
  if constexpr (kPhase == 2) {
    if (tid == 0) sh_st = states[b];
    __syncthreads();
  } else {
    // The partials, the scan inputs, the draft count and the temperature all go out before
    // any of them is used (absent operands are read from a stand-in and discarded).
    const long long row0 = static_cast<long long>(b) * (K + 1);
    PartialBatch batch0;
    prefetch_partials(partials, row0, K, S * kWaves, wave, lane, batch0);
    const void* any = partials;
    const uint8_t* oh_ptr = kMatch ? nullptr : onehot;
    const ScanLoads raw = load_scan_in(oh_ptr, uniforms, gathers, any, b, K, lane);
    const int kb_ld = *(num_draft != nullptr ? num_draft + b : static_cast<const int32_t*>(any));
    const float T_ld = *((greedy_all || temperature == nullptr) ? static_cast<const float*>(any)
                                                                : temperature + b);
    const int kb = num_draft != nullptr ? kb_ld : K;
    const float T = greedy_all ? 0.f : T_ld;
    const bool use_match = kMatch && T != 0.f && kb >= 0 && kb <= K;
    // temp_scale(T) for a valid sampled row, else log2(e) (= log2(e) / 1 exactly), written as
    // one division without a branch so that nothing holds back the loads below.
    const bool scaled = kb >= 0 && kb <= K && temp_valid(T) && T != 0.f;
    const float c = kLog2e / (scaled ? T : 1.f);
    // Every wave merges some rows' partials (one round of loads for up to 16 rows), then wave 0
    // decides.
    row_stats<kMatch>(partials, row0, K, S * kWaves, c, use_match, wave, lane, batch0, sh_rows,
                      sh_rows_d);
    __syncthreads();
    ScanOut so{};
    if (wave == 0) {
      const ScanIn in = finish_scan_in(raw, oh_ptr, uniforms, K, lane);
      if (use_match)
        so = accept_sequence_match(in, kb, T, c, K, V, sh_rows_d, lane);
      else
        so = accept_sequence(in, draft_probs != nullptr, kb, T, c, K, V, sh_rows, lane);
      if (lane == 0) sh_st = so.st;
    }
    __syncthreads();
    // The chunk-0 workgroup emits the scan's outputs; the stores drain while the draw runs.
    if (wave == 0 && first)
      write_scan_out(so, b, K, accept_len, out_tokens, out_probs, states, lane);
  }
  const SeqState st = sh_st;
  if (kPhase == 1 || st.mode == kNone) return;
  const long long row = static_cast<long long>(b) * (K + 1) + st.row;
  const int nseg = S * kSegPerChunk;
  const LT* z = logits + row * V;
  const int P = (nseg + 63) / 64;  // pick: lane l owns segments [l * P, l * P + P)
  const int j0 = lane * P;
  const long long slot = static_cast<long long>(b) * (K + 1) + st.row;
  if (st.mode == kBonus) {
    // A bonus draw (plain p, also every match-mode draw) needs no pass over the row: its weight
    // sum over 2048-token segment j is the streaming kernel's partial j of that row rescaled to
    // the row max, s_j * exp2((m_j - m) * c).  Residuals are summed below exactly (a one-hot
    // residual taken from the partials would subtract e(x) from its segment's sum and cancel when
    // x dominates the row).
    const RowPartial* prow = partials + row * nseg;
    if constexpr (pick_here) {
      // The chunk-0 workgroup draws it right away.
      if (!first) return;
      if (wave == 0) {
        double lw = 0.0;
        for (int q = 0; q < P && j0 + q < nseg; ++q) lw += partial_seg_sum(prow, j0 + q, st);
        // (Sums of p, rescaled partials of a validated row: never NaN.)
        (void)find_draw_segment(lw, lw, uniforms[static_cast<long long>(b) * (K + 1) + st.ucol],
                                nseg, P, [&](int j, bool) { return partial_seg_sum(prow, j, st); },
                                sh_pick, lane);
      }
      __syncthreads();
      scan_draw_segment<LT, kVec>(z, nullptr, partials, V, st, true, sh_pick, out_tokens + slot,
                                  out_probs ? out_probs + slot : nullptr);
      return;
    }
    // Otherwise the sequence's workgroups write them in parallel (one segment per thread) for
    // the pick kernel.
    for (int j = blockIdx.x * kThreads + tid; j < nseg; j += gridDim.x * kThreads) {
      const double e = partial_seg_sum(prow, j, st);
      segs[static_cast<long long>(b) * nseg + j] = SegSums{e, e};
    }
    return;
  }
  const float* q = st.mode == kResidual
                       ? draft_probs + (static_cast<long long>(b) * K + st.row) * V
                       : nullptr;
  // Work item t: chunk t (kPhase 0, 2: wave w sums segment w) or segment t (kPhase 3: wave w
  // sums quarter w of it, the quarters added in order in LDS).
  const int nitems = kFine ? nseg : S;
  const int span = kFine ? kSeg / kWaves : kSeg;  // tokens per wave
  for (int t = blockIdx.x; t < nitems; t += gridDim.x) {
    const int s = kFine ? t / kSegPerChunk : t;
    const int seg0 = kFine ? (t % kSegPerChunk) * kSeg + wave * span : wave * kSeg;
    const int c0 = s * kChunk, n = min(kChunk, V - c0);
    double lw = 0.0, le = 0.0;
    // A one-hot residual is p itself outside the segment that holds the rejected draft x: there
    // its sums are the streaming kernel's partial rescaled to the row max, as for a bonus draw,
    // and nothing is loaded; x's own segment is summed exactly below (taking e(x) out of the
    // partial's sum could cancel when x dominates the segment).  Lane 0 of the wave (with fine
    // items, of wave 0) holds the value, so the sums below add zeros to it.
    const int seg_w = kFine ? t : s * kSegPerChunk + wave;  // the segment this wave sums into
    if (st.mode == kResidualOnehot && seg_w != st.excl / kSeg) {
      if (lane == 0 && (!kFine || wave == 0))
        lw = le = partial_seg_sum(partials + row * nseg, seg_w, st);
    } else if constexpr (kVec && sizeof(LT) == 2) {
      // bf16 rows: lane l owns the 8-token groups l, l + 64, ... of the wave's span, one 16-byte
      // target load and two 16-byte draft loads per group, all issued before any is unpacked
      // (every load 16 bytes wide: 4-token quads would load the logits 8 bytes at a time).
      constexpr int kG8 = kSeg / 8 / 64 / (kFine ? kWaves : 1);  // 4, or 1
      uint4 zr[kG8], qa[kG8], qb[kG8];
#pragma unroll
      for (int h = 0; h < kG8; ++h) {
        const int v0 = c0 + seg0 + (h * 64 + lane) * 8;
        const bool in = v0 < c0 + n;
        zr[h] = in ? plain_load(z + v0) : make_uint4(0, 0, 0, 0);
        qa[h] = (in && q != nullptr) ? plain_load(q + v0) : make_uint4(0, 0, 0, 0);
        qb[h] = (in && q != nullptr) ? plain_load(q + v0 + 4) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int h = 0; h < kG8; ++h) {
        const int v0 = seg0 + (h * 64 + lane) * 8;
        float zv[8], qv[8];
        unpack(zr[h], zv, static_cast<const uint16_t*>(nullptr));
        unpack(qa[h], qv, static_cast<const float*>(nullptr));
        unpack(qb[h], qv + 4, static_cast<const float*>(nullptr));
        const int cnt = min(8, n - v0);
        float gw = 0.f, ge = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float e = 0.f;
          const float w = k < cnt ? draw_weight(zv[k], qv[k], c0 + v0 + k, st, false, e) : 0.f;
          gw += w;
          ge += k < cnt ? e : 0.f;
        }
        lw += gw;
        le += ge;
      }
    } else if constexpr (kVec) {
      // fp32 rows: lane l owns the 4-token quads l, l + 64, ... of the wave's span: every load
      // instruction of the wave reads one contiguous span (4 logits and 4 draft probabilities,
      // 16 bytes each, per lane), and all of them go out before any is unpacked.
      constexpr int kQuads = kSeg / 4 / 64 / (kFine ? kWaves : 1);  // 8, or 2
      DrawVec<LT> zr[kQuads];
      uint4 qr[kQuads];
#pragma unroll
      for (int h = 0; h < kQuads; ++h) {
        const int v0 = c0 + seg0 + (h * 64 + lane) * 4;
        const bool in = v0 < c0 + n;
        zr[h] = in ? DrawVec<LT>::load(z + v0) : DrawVec<LT>::zero();
        qr[h] = (in && q != nullptr) ? plain_load(q + v0) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int h = 0; h < kQuads; ++h) {
        const int v0 = seg0 + (h * 64 + lane) * 4;
        float zv[4], qv[4];
        zr[h].unpack(zv);
        unpack(qr[h], qv, static_cast<const float*>(nullptr));
        const int cnt = min(4, n - v0);
        float gw = 0.f, ge = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float e = 0.f;
          const float w = k < cnt ? draw_weight(zv[k], qv[k], c0 + v0 + k, st, false, e) : 0.f;
          gw += w;
          ge += k < cnt ? e : 0.f;
        }
        lw += gw;
        le += ge;
      }
    } else {
#pragma unroll
      for (int g = 0; g < kGroupsPerLane; ++g) {
        const int v0 = seg0 + (g * 64 + lane) * kGroup;
        float zv[kGroup], qv[kGroup], w[kGroup], gw, ge;
        load_group<LT, false>(z, q, nullptr, c0 + v0, min(kGroup, n - v0), zv, qv);
        group_weights(zv, qv, c0 + v0, min(kGroup, n - v0), st, false, w, gw, ge);
        lw += gw;
        le += ge;
      }
    }
    lw = wave_total(lw);
    le = wave_total(le);
    int segi = s * kSegPerChunk + wave;  // the wave's segment (coarse items)
    if constexpr (kFine) {
      if (lane == 0) sh_fine[wave] = SegSums{lw, le};
      __syncthreads();
      SegSums tot = sh_fine[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        tot.w += sh_fine[w].w;
        tot.e += sh_fine[w].e;
      }
      lw = tot.w;
      le = tot.e;
      segi = t;
      __syncthreads();  // sh_fine is reused by the next item
    }
    if (kFine ? tid < 4 : lane < 4) {
      if constexpr (pick_here) {
        // Four marked words for the sequence's picking workgroup: the two sums in halves.
        const u64 bits = static_cast<u64>(__double_as_longlong((lane & 2) ? le : lw));
        store_word(segw + (static_cast<long long>(b) * nseg + segi) * 4 + lane,
                   marked(static_cast<uint32_t>((lane & 1) ? bits >> 32 : bits)));
      } else if (lane == 0) {
        segs[static_cast<long long>(b) * nseg + segi] = SegSums{lw, le};
      }
    }
  }
  if constexpr (!pick_here) return;
  if (!first) return;
  // The chunk-0 workgroup picks: it waits (bounded) for every segment's sums, finds the segment
  // holding u * total and scans it.
  if (wave == 0) {
    const u64* sw = segw + static_cast<long long>(b) * nseg * 4;
    double lw = 0.0, le = 0.0;
    bool got = false;
    for (int n = 0;; ++n) {
      bool mine = true;
      lw = le = 0.0;
      for (int q = 0; q < P && j0 + q < nseg; ++q) {
        double w, e;
        if (seg_words(sw + (j0 + q) * 4, w, e)) {
          lw += w;
          le += e;
        } else {
          mine = false;
        }
      }
      if (__ballot(!mine) == 0ull) { got = true; break; }
      if (n >= kPickSpinLimit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    bool drawable = false;
    if (got)
      drawable = find_draw_segment(lw, le, uniforms[static_cast<long long>(b) * (K + 1) + st.ucol],
                                   nseg, P,
                                   [&](int j, bool plain) {
                                     double w, e;
                                     seg_words(sw + j * 4, w, e);
                                     return plain ? e : w;
                                   },
                                   sh_pick, lane);
    if (lane == 0) sh_pick.flag = drawable;
  }
  __syncthreads();
  if (sh_pick.flag) {
    scan_draw_segment<LT, kVec>(z, q, partials, V, st, false, sh_pick, out_tokens + slot,
                                out_probs ? out_probs + slot : nullptr);
  } else {
    // The wait gave up (a sibling workgroup never ran), or the draft row holds a value that is
    // not a probability: the sequence is reported invalid.
    for (int i = tid; i <= K; i += kThreads) {
      out_tokens[static_cast<long long>(b) * (K + 1) + i] = -1;
      if (out_probs) out_probs[static_cast<long long>(b) * (K + 1) + i] = 0.f;
    }
    if (tid == 0) accept_len[b] = -1;
  }
}

// The pick of large draw grids (several resident rounds), one workgroup per sequence, after the
// draw kernel has written every segment's sums.
template <typename LT, bool kVec>
__global__ __launch_bounds__(kThreads) void pick_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const float* __restrict__ uniforms, int B, int K, int V, int S,
    const SeqState* __restrict__ states, const SegSums* __restrict__ all_segs,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ out_probs) {
  __shared__ PickLds ps;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nseg = S * kSegPerChunk;
  const int P = (nseg + 63) / 64;  // lane l owns the contiguous segments [l * P, l * P + P)
  const int j0 = lane * P;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const SegSums* segs = all_segs + static_cast<long long>(b) * nseg;
    // The state, the sequence's uniforms (lane i: column min(i, K)) and the lane's segment sums
    // do not depend on each other: every load goes out before any value is used.
    const SeqState st = states[b];
    const float u_lane = uniforms[static_cast<long long>(b) * (K + 1) + min(lane, K)];
    double lw = 0.0, le = 0.0;
    if (wave == 0) {
      for (int q0 = 0; q0 < P; q0 += 4) {
        SegSums sq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sq[q] = segs[min(j0 + q0 + q, nseg - 1)];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q0 + q < P && j0 + q0 + q < nseg) {
            lw += sq[q].w;
            le += sq[q].e;
          }
      }
    }
    if (st.mode == kNone) continue;
    if (wave == 0) {
      const bool ok = find_draw_segment(lw, le, read_lane_f(u_lane, st.ucol), nseg, P,
                                        [&](int j, bool plain) {
                                          return plain ? segs[j].e : segs[j].w;
                                        },
                                        ps, lane);
      if (lane == 0) ps.flag = ok;
    }
    __syncthreads();
    if (!ps.flag) {
      // The draft row holds a value that is not a probability: the sequence is invalid.
      for (int i = tid; i <= K; i += kThreads) {
        out_tokens[static_cast<long long>(b) * (K + 1) + i] = -1;
        if (out_probs) out_probs[static_cast<long long>(b) * (K + 1) + i] = 0.f;
      }
      if (tid == 0) accept_len[b] = -1;
      __syncthreads();  // ps is rewritten for the next sequence
      continue;
    }
    const long long row = static_cast<long long>(b) * (K + 1) + st.row;
    const float* q = st.mode == kResidual
                         ? draft_probs + (static_cast<long long>(b) * K + st.row) * V
                         : nullptr;
    scan_draw_segment<LT, kVec>(logits + row * V, q, all_segs, V, st, false, ps, out_tokens + row,
                                out_probs ? out_probs + row : nullptr);
  }
}

constexpr long long kMaxGrid = 1 << 20;
constexpr int kMaxZ = 65535;  // largest grid y / z extent

inline unsigned grid_for(long long work) {
  return static_cast<unsigned>(work < 1 ? 1 : (work < kMaxGrid ? work : kMaxGrid));
}

template <typename LT, int kPhase>
auto accept_draw_for(bool match, bool vec) -> decltype(&accept_draw_kernel<LT, true, true, kPhase>) {
  return match ? (vec ? accept_draw_kernel<LT, true, true, kPhase>
                      : accept_draw_kernel<LT, false, true, kPhase>)
               : (vec ? accept_draw_kernel<LT, true, false, kPhase>
                      : accept_draw_kernel<LT, false, false, kPhase>);
}

template <typename LT>
hipError_t launch_typed(const LaunchArgs& a) {
  const WorkspaceLayout L = workspace_layout(a.B, a.K, a.V);
  char* base = static_cast<char*>(a.workspace);
  Workspace ws;
  ws.partials = reinterpret_cast<RowPartial*>(base + L.partials);
  ws.gathers = reinterpret_cast<Gather*>(base + L.gathers);
  ws.states = reinterpret_cast<SeqState*>(base + L.states);
  ws.segs = reinterpret_cast<SegSums*>(base + L.segs);
  ws.segw = reinterpret_cast<u64*>(base + L.segw);
  const LT* logits = static_cast<const LT*>(a.logits);
  const int S = num_chunks(a.V);
  const bool vec_stats = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) &&
                         ((static_cast<long long>(a.V) * sizeof(LT)) % 16 == 0);
  const bool vec_draw = vec_stats && (a.V % kGroup == 0) &&
                        (a.draft_probs == nullptr ||
                         reinterpret_cast<uintptr_t>(a.draft_probs) % 16 == 0);
  hipError_t err;
  // Greedy-only calls draw nothing, and match mode only draws plain samples of p (from the
  // partials): the chunk-0 workgroups that run the scan are enough.
  // Otherwise one workgroup per chunk of the row to draw from.
  // A draw grid of more than kDrawRound workgroups (a few resident rounds: five or six 256-thread
  // workgroups per CU on 256 CUs) scans once per sequence in a separate pass instead, and a pick
  // kernel draws after it.  Smaller grids pick inside the draw kernel: the chunk-0 workgroup of a
  // sequence waits for its siblings' segment sums and draws.  That wait always ends, whatever the
  // chip holds at once: only chunk-0 workgroups wait, each for the chunks of its own sequence (the
  // next linear ids), and every XCD dispatches its share of the grid in order, so a sibling of the
  // lowest waiting chunk-0 is queued behind lower-numbered workgroups only -- none of which waits
  // except that chunk-0 itself -- and is dispatched once they finish.  (The wait is bounded all
  // the same.)
  // A draw grid smaller than the chip (up to 256 chunks) takes one workgroup per 2048-token
  // segment instead of one per chunk.
  constexpr long long kDrawRound = 1536;
  constexpr long long kFineMax = 256;
  const bool match = a.match && !a.greedy_all;
  const bool draws = !(a.greedy_all || match);
  const bool split = draws && static_cast<long long>(a.B) * S > kDrawRound;
  const bool fine = draws && static_cast<long long>(a.B) * S <= kFineMax;
  u64* segw = split ? nullptr : ws.segw;
  // The streaming kernel: grid (chunk, row within sequence, sequence), at most 65535 sequences
  // per launch.  With measurement events, the dispatches record them (first start, last end).
  auto stats_for = [&](bool xcd) {
    if (xcd)
      return match ? (vec_stats ? stats_kernel<LT, true, true, true>
                                : stats_kernel<LT, false, true, true>)
                   : (vec_stats ? stats_kernel<LT, true, false, true>
                                : stats_kernel<LT, false, false, true>);
    return match ? (vec_stats ? stats_kernel<LT, true, true, false>
                              : stats_kernel<LT, false, true, false>)
                 : (vec_stats ? stats_kernel<LT, true, false, false>
                              : stats_kernel<LT, false, false, false>);
  };
  for (int b0 = 0; b0 < a.B; b0 += kMaxZ) {
    const dim3 grid(S, a.K + 1, min(kMaxZ, a.B - b0));
    // Long streams without padding rows take the XCD-blocked tile order: measured, it gains
    // 0.5-2.5 us on 350-500 MB of logits and 7-10 us on 550-700 MB, while streams of 200 MB or
    // less lose up to about 1 us and a ragged batch (its padding rows' workgroups return at
    // once) loses 10 us on 1 GB.
    const unsigned long long tiles =
        static_cast<unsigned long long>(grid.x) * grid.y * grid.z;
    const unsigned long long bytes =
        static_cast<unsigned long long>(grid.y) * grid.z * static_cast<unsigned>(a.V) * sizeof(LT);
    const auto stats = stats_for(a.num_draft == nullptr && tiles < (1ull << 31) &&
                                 bytes >= kXcdBlockMinBytes);
    hipEvent_t ev0 = b0 == 0 ? a.hot_begin : nullptr;
    hipEvent_t ev1 = b0 + kMaxZ >= a.B ? a.hot_end : nullptr;
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(stats, grid, dim3(kThreads), 0, a.stream, ev0, ev1, 0, logits,
                            a.draft_probs, a.proposed, a.num_draft, a.temperature, b0, a.K, a.V,
                            S, a.greedy_all, ws.partials, ws.gathers, segw);
    else
      stats<<<grid, kThreads, 0, a.stream>>>(logits, a.draft_probs, a.proposed, a.num_draft,
                                             a.temperature, b0, a.K, a.V, S, a.greedy_all,
                                             ws.partials, ws.gathers, segw);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // Accept scan + draw sums: one workgroup per (chunk, sequence); greedy-only calls need just
  // the chunk-0 workgroups (no draw).  Each phase is its own kernel, so the draw-only pass does
  // not carry the scan's registers (its occupancy sets the draw's bandwidth).
  auto accept_draw = [&](int phase) {
    return phase == 0   ? accept_draw_for<LT, 0>(match, vec_draw)
           : phase == 1 ? accept_draw_for<LT, 1>(match, vec_draw)
           : phase == 2 ? accept_draw_for<LT, 2>(match, vec_draw)
                        : accept_draw_for<LT, 3>(match, vec_draw);
  };
  // With measurement events, the first dispatch below records draw_begin at its start and the
  // last one draw_end at its completion.
  const int phases[2] = {split ? 1 : (fine ? 3 : 0), 2};
  const int nphase = split ? 2 : 1;
  for (int ph = 0; ph < nphase; ++ph) {
    const int phase = phases[ph];
    const int gx = (phase == 1 || !draws) ? 1 : (phase == 3 ? S * kSegPerChunk : S);
    for (int b0 = 0; b0 < a.B; b0 += kMaxZ) {
      const dim3 grid(gx, min(kMaxZ, a.B - b0));
      hipEvent_t ev0 = (ph == 0 && b0 == 0) ? a.draw_begin : nullptr;
      hipEvent_t ev1 = (!split && b0 + kMaxZ >= a.B) ? a.draw_end : nullptr;
      if (ev0 || ev1)
        hipExtLaunchKernelGGL(accept_draw(phase), grid, dim3(kThreads), 0, a.stream, ev0, ev1, 0,
                              logits, a.draft_probs, a.onehot, a.proposed, a.num_draft,
                              a.temperature, a.uniforms, b0, a.K, a.V, S, a.greedy_all,
                              ws.partials, ws.gathers, a.accept_len, a.out_tokens, a.out_probs,
                              ws.states, ws.segs, ws.segw);
      else
        accept_draw(phase)<<<grid, kThreads, 0, a.stream>>>(
            logits, a.draft_probs, a.onehot, a.proposed, a.num_draft, a.temperature,
            a.uniforms, b0, a.K, a.V, S, a.greedy_all, ws.partials, ws.gathers, a.accept_len,
            a.out_tokens, a.out_probs, ws.states, ws.segs, ws.segw);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  if (!split) return hipSuccess;
  auto pick = vec_draw ? pick_kernel<LT, true> : pick_kernel<LT, false>;
  if (a.draw_end)
    hipExtLaunchKernelGGL(pick, dim3(grid_for(a.B)), dim3(kThreads), 0, a.stream, nullptr,
                          a.draw_end, 0, logits, a.draft_probs, a.uniforms, a.B, a.K, a.V, S,
                          ws.states, ws.segs, a.accept_len, a.out_tokens, a.out_probs);
  else
    pick<<<grid_for(a.B), kThreads, 0, a.stream>>>(logits, a.draft_probs, a.uniforms, a.B, a.K,
                                                   a.V, S, ws.states, ws.segs, a.accept_len,
                                                   a.out_tokens, a.out_probs);
  return hipGetLastError();
}

}  // namespace

WorkspaceLayout workspace_layout(int B, int K, int V) {
  auto align16 = [](size_t x) { return (x + 15) & ~static_cast<size_t>(15); };
  const size_t S = static_cast<size_t>(num_chunks(V));
  const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(K + 1);
  WorkspaceLayout L;
  size_t off = 0;
  L.partials = off;
  off = align16(off + rows * S * kWaves * sizeof(RowPartial));
  L.gathers = off;
  off = align16(off + static_cast<size_t>(B) * static_cast<size_t>(K) * sizeof(Gather));
  L.states = off;
  off = align16(off + static_cast<size_t>(B) * sizeof(SeqState));
  L.segs = off;
  off = align16(off + static_cast<size_t>(B) * S * kSegPerChunk * sizeof(SegSums));
  L.segw = off;
  off = align16(off + static_cast<size_t>(B) * S * kSegPerChunk * 4 * sizeof(unsigned long long));
  L.total = off;
  return L;
}

size_t workspace_bytes(int B, int K, int V) {
  const size_t one = static_cast<size_t>(B) * static_cast<size_t>(record_layout(K, V).words) * 8;
  return std::max({workspace_layout(B, K, V).total, one, quad_workspace_bytes(B, K, V)});
}

hipError_t launch_verify(const LaunchArgs& a) {
  if (a.path == 3) return launch_one_launch(a);
  if (a.path == 4) return quad_eligible(a) ? launch_quad(a) : hipErrorInvalidConfiguration;
  // Rows of at most kSmallVMax tokens fit one wave's registers: one kernel, a group of lanes
  // per sequence (small.hip), unless the streaming kernels are asked for.
  const bool small = a.V <= kSmallVMax && a.path != 1;
  if (small) return launch_small_verify(a);
  return a.logits_bf16 ? launch_typed<uint16_t>(a) : launch_typed<float>(a);
}

}  // namespace specdec
