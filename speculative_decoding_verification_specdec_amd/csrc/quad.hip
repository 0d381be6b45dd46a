// gfx950 (CDNA4) kernel of the batched speculative-decoding verify step in one launch, four
// workgroups per sequence: the rejection rule of "Decodificação especulativa explicada"
// (gsantana.dev), section "A regra de amostragem por rejeição"; "ch15 · Speculative Decoding"
// (snowch.github.io), section "Why the result is exactly the target model"; the inverse-CDF draw
// of the numpy listing in section "Amostragem especulativa em numpy, com prova" of the first page.
//
// Workgroup 4b + q (1024 threads, 16 waves) owns quarter q of every target row of sequence b:
// tokens [q * span, (q + 1) * span) with span a whole number of 2048-token segments.
//   1. Stream: wave w folds segments w, w + 16, ... of rows 0..k_b (the streaming kernel's
//      32-logit lane tasks: wave max first, exp2 sum, lowest argmax of greedy rows), the next
//      task's loads in flight while the current one is folded; per-segment (max, sum, argmax) in
//      LDS.  Every byte of the sequence's logits is read once, by 64 CUs' worth of workgroups at
//      B = 64 with no kernel boundary behind them.
//   2. Exchange 1, all to all: each workgroup publishes its quarter's (max, sum, argmax) of every
//      row and reads the three others', then merges the four quarters in quarter order -- the same
//      values in the same order in every workgroup, so all four run the same accept scan.
//   3. Draw sums: a residual draw sums s * max(0, p - q) (or p without x_j) over the workgroup's
//      quarter of row j, per segment, in fp64; a bonus draw takes its per-segment sums of p from
//      the stream's segment statistics.  Workgroups 1..3 publish their segment sums and finish.
//   4. Exchange 2, to workgroup 0 only: it reads the other quarters' segment sums, finds the
//      quarter, the segment and then the token holding u * total (plain p when the residual is
//      empty), and writes every output of the sequence.
//
// Hand-off words.  A value v (32 bits) travels in two 64-bit words: (tagA << 32 | v) and
// (tagB << 32 | ~v), the tags a function of the word's slot and of the sequence's epoch, a
// counter kept in the workspace that workgroup 0 advances once every sibling has read it (each
// read it before publishing its first word).  A consumer takes a value only when both tags and
// the complement match, so words left by earlier calls (older epochs) never pass, and leftover
// bytes of anything else pass with odds of 2^-96: the workspace needs no initialisation.  Each
// 64-bit store is single-copy atomic, so a word never pairs a tag with stale bits.  Waits are
// bounded (a workgroup that gives up publishes nothing more and writes nothing; workgroup 0 then
// reports the sequence invalid), and the path is taken only when every workgroup of the grid
// fits on the device at once.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <climits>

#include "kernels.h"
#include "verify_dev.h"
#include "wave_ops.h"

namespace specdec {
namespace {

constexpr int kQThreads = 1024;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQuarters = 4;
constexpr uint32_t kTagA = 0x3c6ef372u;
constexpr uint32_t kTagB = 0xa54ff53au;
constexpr int kQDefaultSpin = 1 << 20;

__device__ __forceinline__ uint32_t tag_a(uint32_t epoch, uint32_t slot) {
  return kTagA ^ epoch ^ (slot * 0x9e3779b9u);
}
__device__ __forceinline__ uint32_t tag_b(uint32_t epoch, uint32_t slot) {
  return kTagB ^ (epoch * 0x85ebca6bu) ^ (slot * 0xc2b2ae35u) ^ 0x27d4eb2fu;
}
// The value at word offset `off` of a record occupies words off and off + 1.
__device__ __forceinline__ void put_value(u64* rec, uint32_t epoch, long long off, uint32_t v) {
  const uint32_t slot = static_cast<uint32_t>(off);
  store_word(rec + off, (static_cast<u64>(tag_a(epoch, slot)) << 32) | v);
  store_word(rec + off + 1, (static_cast<u64>(tag_b(epoch, slot)) << 32) | ~v);
}
// True (and the value in v) once both words carry this epoch's tags and agree.
__device__ __forceinline__ bool get_value(const u64* rec, uint32_t epoch, long long off,
                                          uint32_t& v) {
  const uint32_t slot = static_cast<uint32_t>(off);
  const u64 w1 = load_word(rec + off), w2 = load_word(rec + off + 1);
  v = static_cast<uint32_t>(w1);
  return static_cast<uint32_t>(w1 >> 32) == tag_a(epoch, slot) &&
         static_cast<uint32_t>(w2 >> 32) == tag_b(epoch, slot) &&
         static_cast<uint32_t>(w2) == ~v;
}
// Polls one value until it is there or `spin` polls have gone by.
__device__ __forceinline__ bool wait_value(const u64* rec, uint32_t epoch, long long off,
                                           int spin, uint32_t& v) {
  for (int n = 0;; ++n) {
    if (get_value(rec, epoch, off, v)) return true;
    if (n >= spin) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// The record of one sequence, in 64-bit words: the epoch, then exchange 1 (4 quarters x (K+1)
// rows x 3 values x 2 words), then exchange 2 (quarters 1..3 x nseg segments x 4 values x 2
// words).
__host__ __device__ inline long long quad_h1(int q, int i, int K) {
  return 1 + (static_cast<long long>(q) * (K + 1) + i) * 6;
}
__host__ __device__ inline long long quad_h2(int q, int j, int K, int nseg) {
  return 1 + 4LL * (K + 1) * 6 + (static_cast<long long>(q - 1) * nseg + j) * 8;
}
__host__ __device__ inline long long quad_record_words(int K, int nseg) {
  return (quad_h2(4, 0, K, nseg) + 31) & ~31LL;
}

// Sixteen-byte raw loads of one 2048-token lane task (kPerThread logits per lane), unpacked later.
template <typename LT>
struct TaskLoads {
  static constexpr int kU = kPerThread / Vec<LT>::kPer;
  uint4 d[kU];
  __device__ __forceinline__ void issue(const LT* __restrict__ row, int c0, int n, int lane) {
    const uint4* vrow = reinterpret_cast<const uint4*>(row + c0);
    const int nvec = n / Vec<LT>::kPer;
    constexpr uint32_t ni = Vec<LT>::kNegInf;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int vi = u * 64 + lane;
      d[u] = vi < nvec ? stream_load(vrow + vi) : make_uint4(ni, ni, ni, ni);
    }
  }
  __device__ __forceinline__ void unpack_to(float (&x)[kPerThread]) const {
#pragma unroll
    for (int u = 0; u < kU; ++u) unpack(d[u], &x[u * Vec<LT>::kPer], static_cast<const LT*>(nullptr));
  }
};

// The three 16-byte loads of one lane's 8-token group of a draw row (target logits: one vector of
// bf16 or two of fp32; draft probabilities: two), issued now and unpacked later; an absent row or
// group reads `any` (a valid 16-byte-aligned address) and is zeroed when unpacked.
template <typename LT>
struct GroupLoads {
  uint4 z0, z1, q0, q1;
  __device__ __forceinline__ void issue(const LT* __restrict__ z, const float* __restrict__ q,
                                        const void* any, int v0, bool in) {
    const LT* zp = in ? z + v0 : static_cast<const LT*>(any);
    const float* qp = (in && q != nullptr) ? q + v0 : static_cast<const float*>(any);
    z0 = stream_load(zp);
    if constexpr (sizeof(LT) == 4) z1 = stream_load(zp + 4);
    q0 = stream_load(qp);
    q1 = stream_load(qp + 4);
  }
  __device__ __forceinline__ void unpack_to(bool in, bool has_q, float (&zv)[kGroup],
                                            float (&qv)[kGroup]) const {
    unpack(z0, zv, static_cast<const LT*>(nullptr));
    if constexpr (sizeof(LT) == 4) unpack(z1, zv + 4, static_cast<const LT*>(nullptr));
    unpack(q0, qv, static_cast<const float*>(nullptr));
    unpack(q1, qv + 4, static_cast<const float*>(nullptr));
#pragma unroll
    for (int k = 0; k < kGroup; ++k) {
      if (!in) zv[k] = -INFINITY;
      if (!in || !has_q) qv[k] = 0.f;
    }
  }
};

struct QuadPick {
  int hit[kQWaves], lastpos[kQWaves];
  float zhit[kQWaves], zlast[kQWaves];
  double wtot[kQWaves];
};

template <typename LT>
__global__ __launch_bounds__(kQThreads) void quad_verify_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const uint8_t* __restrict__ onehot, const int32_t* __restrict__ proposed,
    const int32_t* __restrict__ num_draft, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, int b0, int K, int V, int span, int nseg_max,
    int greedy_all, int spin, int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ out_probs, u64* __restrict__ records, long long rec_words) {
  __shared__ float sh_m[kMaxRows][kMaxQuadSeg];
  __shared__ float sh_s[kMaxRows][kMaxQuadSeg];
  __shared__ int sh_a[kMaxRows][kMaxQuadSeg];
  __shared__ Stat sh_q[kQuarters][kMaxRows];   // quarter statistics per row
  __shared__ Stat sh_rows[kMaxRows];           // full-row statistics
  __shared__ SegSums sh_seg[kQuarters][kMaxQuadSeg];
  __shared__ SeqState sh_st;
  __shared__ QuadPick sh_pick;
  __shared__ PickLds sh_ps;
  __shared__ int sh_fail, sh_draw_ok;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qq = static_cast<int>(blockIdx.x) & 3;
  const int b = b0 + static_cast<int>(blockIdx.x >> 2);
  u64* rec = records + static_cast<long long>(b) * rec_words;
  const long long row0 = static_cast<long long>(b) * (K + 1);
  const int q_lo = qq * span;
  const int q_n = max(0, min(span, V - q_lo));
  const int nseg = (q_n + kSeg - 1) / kSeg;
  const int segs_w = nseg > wave ? (nseg - wave + kQWaves - 1) / kQWaves : 0;

  // Row 0's first task goes out before anything else (row 0 always exists); then the draft
  // count, temperature, epoch and the scan inputs of wave 0.
  TaskLoads<LT> cur;
  if (segs_w > 0) {
    const int c0 = q_lo + wave * kSeg;
    cur.issue(logits + row0 * V, c0, min(kSeg, V - c0), lane);
  }
  const int kb_raw = num_draft != nullptr ? num_draft[b] : K;
  const float T = greedy_all ? 0.f : temperature[b];
  const uint32_t epoch = static_cast<uint32_t>(load_word(rec));
  const bool kb_ok = kb_raw >= 0 && kb_raw <= K;
  const int rows = kb_ok ? kb_raw + 1 : 0;
  const float c = temp_valid(T) ? temp_scale(T) : kLog2e;
  // Scan inputs (wave 0, lane i <-> slot i): the drafted id and its gathered target logit and
  // drafter probability, the uniforms, the one-hot flag.
  ScanIn in{};
  if (wave == 0) {
    const long long slot = static_cast<long long>(b) * K + lane;
    const bool drafted = lane < K && lane < rows - 1;
    const int x = drafted ? proposed[slot] : -1;
    Gather g{0.f, 0.f, x, 0};
    if (drafted && x >= 0 && x < V) {
      g.z = load_logit(logits + (row0 + lane) * V, x);
      if (draft_probs != nullptr && T != 0.f) g.q = draft_probs[slot * V + x];
    }
    in.g = lane < K ? g : Gather{0.f, 0.f, -1, 0};
    const float u = (uniforms != nullptr && lane <= K) ? uniforms[row0 + lane] : 0.f;
    in.u = lane < K ? u : 0.f;
    in.uk = uniforms != nullptr ? read_lane_f(u, K) : 0.f;
    in.onehot = onehot != nullptr && onehot[b] != 0;
  }
  if (tid == 0) sh_fail = 0;

  // 1. Stream: tasks (row i, segment wave + 16 t) in row-major order, the next one's loads in
  // flight while the current one is folded.
  const int ntask = rows * segs_w;
  for (int t = 0; t < ntask; ++t) {
    const int i = t / segs_w, j = wave + kQWaves * (t % segs_w);
    const int c0 = q_lo + j * kSeg;
    const int n = min(kSeg, V - c0);
    TaskLoads<LT> nxt;
    if (t + 1 < ntask) {
      const int i1 = (t + 1) / segs_w, j1 = wave + kQWaves * ((t + 1) % segs_w);
      const int c1 = q_lo + j1 * kSeg;
      nxt.issue(logits + (row0 + i1) * V, c1, min(kSeg, V - c1), lane);
    }
    float x[kPerThread];
    cur.unpack_to(x);
    float lane_max, pre;
    const MaxSum st = fold_wave<LT, true, false>(x, c, c0, lane, -1, lane_max, pre);
    const int arg = T == 0.f ? lowest_token_of<LT, true>(x, st.m, c0) : 0;
    (void)lane_max;
    (void)n;
    if (lane == 0) {
      sh_m[i][j] = st.m;
      sh_s[i][j] = st.s;
      sh_a[i][j] = arg;
    }
    if (t + 1 < ntask) cur = nxt;
  }
  __syncthreads();

  // 2. Quarter statistics of each row (max first, sums rescaled once), then exchange 1.
  for (int i = wave; i < rows; i += kQWaves) {
    const bool in_seg = lane < nseg;
    const float m = in_seg ? sh_m[i][lane] : -INFINITY;
    const float s = in_seg ? sh_s[i][lane] : 0.f;
    const int a = in_seg ? sh_a[i][lane] : INT_MAX;
    const float M = wave_max_f(m);
    const float f = (M == -INFINITY || m == -INFINITY) ? (M == -INFINITY ? 1.f : 0.f)
                                                       : __builtin_amdgcn_exp2f((m - M) * c);
    const float S = wave_sum_f(s * f);
    const int A = wave_min(m == M ? a : INT_MAX);
    if (lane == 0) sh_q[qq][i] = Stat{M, S, A};
  }
  __syncthreads();
  if (tid < 3 * rows) {
    const int i = tid / 3, f = tid % 3;
    const Stat s = sh_q[qq][i];
    const uint32_t v = f == 0 ? __float_as_uint(s.m) : f == 1 ? __float_as_uint(s.s)
                                                             : static_cast<uint32_t>(s.a);
    put_value(rec, epoch, quad_h1(qq, i, K) + 2 * f, v);
  }
  if (tid < 9 * rows) {
    const int k = tid / (3 * rows), r = tid % (3 * rows);
    const int q = k < qq ? k : k + 1;  // the three other quarters
    const int i = r / 3, f = r % 3;
    uint32_t v = 0;
    if (!wait_value(rec, epoch, quad_h1(q, i, K) + 2 * f, spin, v)) {
      sh_fail = 1;
    } else if (f == 0) {
      sh_q[q][i].m = __uint_as_float(v);
    } else if (f == 1) {
      sh_q[q][i].s = __uint_as_float(v);
    } else {
      sh_q[q][i].a = static_cast<int>(v);
    }
  }
  __syncthreads();
  // Every sibling has read the epoch (each before publishing): the next call takes a new one.
  if (qq == 0 && tid == 0) store_word(rec, static_cast<u64>(epoch + 1u));
  const bool failed1 = sh_fail != 0;

  // 3. Full-row statistics (quarters merged in quarter order) and the accept scan.
  if (!failed1 && tid < rows) {
    const int i = tid;
    float M = sh_q[0][i].m;
#pragma unroll
    for (int q = 1; q < kQuarters; ++q) M = fmaxf(M, sh_q[q][i].m);
    float S = 0.f;
    int A = INT_MAX;
#pragma unroll
    for (int q = 0; q < kQuarters; ++q) {
      const Stat s = sh_q[q][i];
      S += (M == -INFINITY) ? s.s
                            : (s.m == -INFINITY ? 0.f
                                                : s.s * __builtin_amdgcn_exp2f((s.m - M) * c));
      if (s.m == M) A = min(A, s.a);
    }
    sh_rows[i] = Stat{M, S, A};
  }
  __syncthreads();
  if (wave == 0 && !failed1) {
    const ScanOut so = accept_sequence(in, draft_probs != nullptr, kb_raw, T, c, K, V, sh_rows, lane);
    if (lane == 0) sh_st = so.st;
    // Workgroup 0 writes the scan's outputs; the drawn slot is left to the pick.
    if (qq == 0) {
      const bool pending = so.st.mode != kNone;
      if (lane <= K && !(pending && lane == so.A)) {
        out_tokens[row0 + lane] = so.tok;
        if (out_probs) out_probs[row0 + lane] = static_cast<float>(so.num / so.den);
      }
      if (lane == 0) accept_len[b] = so.A;
    }
  }
  if (failed1) {
    // Exchange 1 gave up: workgroup 0 reports the sequence invalid, the others stop.
    if (qq == 0) {
      for (int i = tid; i <= K; i += kQThreads) {
        out_tokens[row0 + i] = -1;
        if (out_probs) out_probs[row0 + i] = 0.f;
      }
      if (tid == 0) accept_len[b] = -1;
    }
    return;
  }
  __syncthreads();
  const SeqState st = sh_st;
  if (st.mode == kNone) return;

  // 4. Draw sums over this quarter of row j, per segment.
  const LT* z = logits + (row0 + st.row) * V;
  const float* qrow = st.mode == kResidual
                          ? draft_probs + (static_cast<long long>(b) * K + st.row) * V
                          : nullptr;
  if (st.mode == kBonus) {
    if (tid < nseg) {
      const float m = sh_m[st.row][tid];
      const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - st.m) * st.c);
      const double e = static_cast<double>(sh_s[st.row][tid]) * static_cast<double>(f);
      sh_seg[qq][tid] = SegSums{e, e};
    }
  } else {
    // Wave w sums segments w, w + 16, ... in steps of 512 tokens (lane l: the 8-token group l of
    // the step), the next step's loads in flight while the current one is weighed.
    constexpr int kStep = 64 * kGroup;
    constexpr int kSteps = kSeg / kStep;
    for (int j = wave; j < nseg; j += kQWaves) {
      const int c0 = q_lo + j * kSeg;
      const int n = min(kSeg, V - c0);
      GroupLoads<LT> cur;
      cur.issue(z, qrow, logits, c0 + lane * kGroup, lane * kGroup < n);
      double lw = 0.0, le = 0.0;
#pragma unroll
      for (int h = 0; h < kSteps; ++h) {
        const int o = h * kStep + lane * kGroup;
        GroupLoads<LT> nxt;
        if (h + 1 < kSteps) nxt.issue(z, qrow, logits, c0 + o + kStep, o + kStep < n);
        float zv[kGroup], qv[kGroup], w[kGroup], gw, ge;
        cur.unpack_to(o < n, qrow != nullptr, zv, qv);
        group_weights(zv, qv, c0 + o, min(kGroup, n - o), st, false, w, gw, ge);
        lw += gw;
        le += ge;
        if (h + 1 < kSteps) cur = nxt;
      }
      lw = wave_total(lw);
      le = wave_total(le);
      if (lane == 0) sh_seg[qq][j] = SegSums{lw, le};
    }
  }
  __syncthreads();

  // 5. Exchange 2: quarters 1..3 hand their segment sums to workgroup 0 and are done.
  if (qq != 0) {
    if (tid < 4 * nseg) {
      const int j = tid / 4, f = tid % 4;
      const SegSums s = sh_seg[qq][j];
      const u64 bits = static_cast<u64>(__double_as_longlong(f < 2 ? s.w : s.e));
      const uint32_t v = static_cast<uint32_t>((f & 1) ? bits >> 32 : bits);
      put_value(rec, epoch, quad_h2(qq, j, K, nseg_max) + 2 * f, v);
    }
    return;
  }
  {
    // Quarter q's segment count.
    const int k = tid / (4 * nseg_max), r = tid % (4 * nseg_max);
    if (k < 3) {
      const int q = k + 1;
      const int qn = max(0, min(span, V - q * span));
      const int qseg = (qn + kSeg - 1) / kSeg;
      const int j = r / 4, f = r % 4;
      if (j < qseg) {
        uint32_t lo = 0;
        if (!wait_value(rec, epoch, quad_h2(q, j, K, nseg_max) + 2 * f, spin, lo)) {
          sh_fail = 1;
        } else {
          // Halves land in the double's bit pattern through LDS (each thread one half).
          uint32_t* d = reinterpret_cast<uint32_t*>(f < 2 ? &sh_seg[q][j].w : &sh_seg[q][j].e);
          d[f & 1] = lo;
        }
      }
    }
  }
  __syncthreads();
  bool ok = sh_fail == 0;

  // 6. The pick (workgroup 0).  Segment g of the row (tokens [2048 g, 2048 g + 2048)) is segment
  // g % nseg_max of quarter g / nseg_max; segments past the row's end weigh nothing.  Wave 0 finds
  // the segment holding u * total (plain p when the residual is empty) with fp64 DPP scans, then
  // the workgroup scans that segment.
  auto seg_sum = [&](int g, bool plain) -> double {
    const int q = g / nseg_max, j = g % nseg_max;
    const int qn = max(0, min(span, V - q * span));
    if (j * kSeg >= qn) return 0.0;
    return plain ? sh_seg[q][j].e : sh_seg[q][j].w;
  };
  if (ok && wave == 0) {
    const int nseg_all = kQuarters * nseg_max;
    const int P = (nseg_all + 63) / 64;
    const int j0 = lane * P;
    double lw = 0.0, le = 0.0;
    for (int k = 0; k < P && j0 + k < nseg_all; ++k) {
      lw += seg_sum(j0 + k, false);
      le += seg_sum(j0 + k, true);
    }
    // The draw's uniform is column K (st.ucol), which wave 0 already holds from the scan inputs.
    const bool drawable = find_draw_segment(lw, le, in.uk, nseg_all, P, seg_sum, sh_ps, lane);
    if (lane == 0) sh_draw_ok = drawable;
  }
  __syncthreads();
  ok = ok && sh_draw_ok != 0;
  if (ok) {
    // Scan the segment: two tokens per thread, fp32 pair sums, fp64 scans.
    // (The segment found always has positive weight, so it lies inside the row; clamped all the
    // same so that no load can leave it.)
    const int s0 = min(sh_ps.seg, (V - 1) / kSeg) * kSeg;
    const int sn = min(kSeg, V - s0);
    const bool plain = sh_ps.plain != 0;
    const double t = sh_ps.t;
    const int v0 = s0 + 2 * tid;
    const int cnt = max(0, min(2, s0 + sn - v0));
    float zv[2] = {-INFINITY, -INFINITY}, qv[2] = {0.f, 0.f}, w[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k < cnt) {
        zv[k] = load_logit(z, v0 + k);
        if (qrow != nullptr && !plain) qv[k] = qrow[v0 + k];
      }
    }
    float gw = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float e = 0.f;
      w[k] = k < cnt ? draw_weight(zv[k], qv[k], v0 + k, st, plain, e) : 0.f;
      gw += w[k];
    }
    const double inc = wave_inclusive_scan(static_cast<double>(gw));
    if (lane == 63) sh_pick.wtot[wave] = inc;
    __syncthreads();
    double before = sh_ps.base;
    for (int k = 0; k < wave; ++k) before += sh_pick.wtot[k];
    before += inc - static_cast<double>(gw);
    int hit = -1, lastpos = -1;
    float zhit = 0.f, zlast = 0.f, run = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      run += w[k];
      if (k < cnt && w[k] > 0.f) {
        lastpos = v0 + k;
        zlast = zv[k];
        if (hit < 0 && before + static_cast<double>(run) > t) { hit = v0 + k; zhit = zv[k]; }
      }
    }
    const unsigned long long hm = __ballot(hit >= 0);
    const unsigned long long pm = __ballot(lastpos >= 0);
    const int hl = hm ? __ffsll(static_cast<long long>(hm)) - 1 : 0;
    const int ll = pm ? 63 - __clzll(static_cast<long long>(pm)) : 0;
    const int wave_hit = hm ? __builtin_amdgcn_readlane(hit, hl) : -1;
    const float wave_zhit = read_lane_f(zhit, hl);
    const int wave_last = pm ? __builtin_amdgcn_readlane(lastpos, ll) : -1;
    const float wave_zlast = read_lane_f(zlast, ll);
    if (lane == 0) {
      sh_pick.hit[wave] = wave_hit; sh_pick.zhit[wave] = wave_zhit;
      sh_pick.lastpos[wave] = wave_last; sh_pick.zlast[wave] = wave_zlast;
    }
    __syncthreads();
    if (tid == 0) {
      int y = -1, lp = -1;
      float zy = 0.f, zl = 0.f;
      for (int k = 0; k < kQWaves; ++k) {
        if (y < 0 && sh_pick.hit[k] >= 0) { y = sh_pick.hit[k]; zy = sh_pick.zhit[k]; }
        if (sh_pick.lastpos[k] >= 0) { lp = sh_pick.lastpos[k]; zl = sh_pick.zlast[k]; }
      }
      if (y < 0) {
        y = lp >= 0 ? lp : s0;
        zy = lp >= 0 ? zl : load_logit(z, y);
      }
      const double p = exp2((static_cast<double>(zy) - static_cast<double>(st.m)) *
                            static_cast<double>(st.c)) / static_cast<double>(st.s);
      out_tokens[row0 + st.row] = y;
      if (out_probs) out_probs[row0 + st.row] = static_cast<float>(p);
    }
  } else {
    // A wait gave up, or the draft row holds a value that is not a probability: the sequence is
    // reported invalid.
    for (int i = tid; i <= K; i += kQThreads) {
      out_tokens[row0 + i] = -1;
      if (out_probs) out_probs[row0 + i] = 0.f;
    }
    if (tid == 0) accept_len[b] = -1;
  }
}

template <typename LT>
int quad_capacity(hipStream_t stream) {
  // Workgroups of this kernel that the device the call runs on -- the stream's (the null stream:
  // the current device) -- holds at once; cached per device (threads that race to fill an entry
  // store the same value).  The occupancy query runs with that device current, and the caller's
  // current device is restored.
  static std::atomic<int> cache[64];
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return 0;
    dev = static_cast<int>(d);
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return 0;
  }
  if (dev < 0 || dev >= 64) return 0;
  const int known = cache[dev].load(std::memory_order_relaxed);
  if (known != 0) return known;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return 0;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return 0;
  int per_cu = 0, cus = 0;
  const bool ok =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quad_verify_kernel<LT>, kQThreads,
                                                   0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  if (cur != dev && hipSetDevice(cur) != hipSuccess) return 0;
  if (!ok) return 0;
  cache[dev].store(per_cu * cus, std::memory_order_relaxed);
  return per_cu * cus;
}

template <typename LT>
hipError_t launch_quad_typed(const LaunchArgs& a) {
  const int span = quad_span(a.V);
  const int nseg_max = (span + kSeg - 1) / kSeg;
  const long long rec_words = quad_record_words(a.K, nseg_max);
  const int spin = a.spin_limit > 0 ? a.spin_limit : kQDefaultSpin;
  // The optional hot events bracket this one kernel (its dispatch records them).
  hipExtLaunchKernelGGL(quad_verify_kernel<LT>, dim3(static_cast<unsigned>(a.B) * kQuarters),
                        dim3(kQThreads), 0, a.stream, a.hot_begin, a.hot_end, 0,
                        static_cast<const LT*>(a.logits), a.draft_probs, a.onehot, a.proposed,
                        a.num_draft, a.temperature, a.uniforms, 0, a.K, a.V, span, nseg_max,
                        a.greedy_all, spin, a.accept_len, a.out_tokens, a.out_probs,
                        static_cast<u64*>(a.workspace), rec_words);
  return hipGetLastError();
}

}  // namespace

size_t quad_workspace_bytes(int B, int K, int V) {
  const int nseg_max = (quad_span(V) + kSeg - 1) / kSeg;
  return static_cast<size_t>(B) * quad_record_words(K, nseg_max) * sizeof(u64);
}

bool quad_eligible(const LaunchArgs& a) {
  // Rows of whole 8-token groups (the draw's loads), 16-byte aligned.
  if (a.match || a.B < 1 || a.V % kGroup != 0 ||
      reinterpret_cast<uintptr_t>(a.logits) % 16 != 0 ||
      (a.draft_probs != nullptr && reinterpret_cast<uintptr_t>(a.draft_probs) % 16 != 0))
    return false;
  if ((quad_span(a.V) + kSeg - 1) / kSeg > kMaxQuadSeg) return false;
  const int cap = a.logits_bf16 ? quad_capacity<uint16_t>(a.stream) : quad_capacity<float>(a.stream);
  return static_cast<long long>(a.B) * kQuarters <= cap;
}

hipError_t launch_quad(const LaunchArgs& a) {
  return a.logits_bf16 ? launch_quad_typed<uint16_t>(a) : launch_quad_typed<float>(a);
}

}  // namespace specdec
