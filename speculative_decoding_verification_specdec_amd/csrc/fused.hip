// gfx950 (CDNA4) kernel of the batched speculative-decoding verify step in ONE launch: an
// alternative to the three launches of kernels.hip, kept selectable (SPECDEC_PATH_ONE_LAUNCH) and
// parity-tested.  On one MI355X it measured slower (batch of 64 sequences, k = 5, V = 128256:
// 42-43 us against 37 us): a hand-off between workgroups of one launch is a round trip through
// device-coherent memory that costs about 3 us while the stream keeps HBM busy, against about 1 us
// for the same loads after a kernel boundary, and each sequence's round needs four or five such
// round trips after its rows (rows -> scan -> draw -> segment sums -> pick).
//
// Workgroups: row tiles (chunk s of rows 0..K-1, as the streaming kernel) and per sequence its
// closing tiles (the chunks of row K, each also a share of the residual draw).  Every value handed
// between workgroups travels in marked 64-bit words (no counters, no fences): a producer issues
// coherent stores and goes on, a consumer polls (bounded) until every word it needs is marked.
// Each closing tile merges the round's rows itself and runs the accept scan; with a residual draw
// every closing tile sums its segments and reads all segment sums, and the tile that summed the
// segment holding u * total scans it; the first closing tile writes the known tokens and, after
// the others report, puts the record back to zero.  A zero-fill kernel runs before the launch.
//
// The rule is the one the source pages define: "Decodificação especulativa explicada"
// (gsantana.dev), section "A regra de amostragem por rejeição"; "ch15 · Speculative Decoding"
// (snowch.github.io), section "Why the result is exactly the target model"; "Speculative
// decoding: el secretario que adelanta lo que va a decir el jefe" (blog.lo0.es), section "El
// mecanismo desnudo".
#include <algorithm>

#include <hip/hip_ext.h>

#include "kernels.h"
#include "verify_dev.h"
#include "wave_ops.h"

namespace specdec {
namespace {

__global__ __launch_bounds__(kThreads) void zero_words(unsigned long long* w, long long n) {
  const long long i = (static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x) * 2;
  if (i < n) w[i] = 0;
  if (i + 1 < n) w[i + 1] = 0;
}

inline unsigned grid_for(long long items) {
  const long long g = (items + kThreads - 1) / kThreads;
  return static_cast<unsigned>(g < 1 ? 1 : g);
}

// The scan's outputs: accept_len and every output slot except a deferred one (slot A of a sampled
// valid row, drawn later, or a greedy bonus whose row statistics arrive later), which the
// sequence's finisher writes.  Coherent stores: a slot has one writer in the launch.
__device__ __forceinline__ void write_round_out(const ScanOut& o, bool deferred, int b, int K,
                                               int32_t* accept_len, int32_t* out_tokens,
                                               float* out_probs, int lane) {
  const long long row0 = static_cast<long long>(b) * (K + 1);
  if (lane <= K && !(deferred && lane == o.A)) {
    coherent_store_i(out_tokens + row0 + lane, o.tok);
    if (out_probs) coherent_store_f(out_probs + row0 + lane, static_cast<float>(o.num / o.den));
  }
  if (lane == 0) coherent_store_i(accept_len + b, o.A);
}

// ------------------------------------------------------------------------------------------
// Hand-off words.  Every value one workgroup hands to another inside the launch travels in a
// 64-bit word whose upper half is kMark: the producer issues coherent stores and goes on (no
// wait, no count), the consumer polls until every word it needs carries the mark, and the
// consumer that finishes a sequence puts every word it consumed back to zero, so a later call on
// the same workspace (same K and V) starts from zeros again.  Each 64-bit store is single-copy
// atomic, so a marked word never pairs a new mark with stale data.
// ------------------------------------------------------------------------------------------
struct KArgs {
  const void* logits;
  const float* draft_probs;
  const uint8_t* onehot;
  const int32_t* proposed;
  const int32_t* num_draft;
  const float* temperature;
  const float* uniforms;
  int b0, nb;      // this launch's sequences: b0 .. b0 + nb - 1
  int K, V, S;
  int greedy_all;
  int draws;       // 1: the call may draw residuals (every closing tile runs the round)
  int fine;        // 1: a closing tile per 2048-token segment (small grids), else per chunk
  int tasks;       // closing tiles per sequence: S, or 4 * S with `fine`
  int group;       // sequences per group of the grid layout
  int spin_limit;  // polls of a bounded wait
  u64* ws;
  RecordLayout L;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* out_probs;
};

struct Shared {
  Stat rows[kMaxRows];
  StatD rows_d[kMaxRows];
  SeqState st;
  SegSums fine[kWaves];
  int A, flag, fail;
  int seg, plain, hit[kWaves], lastpos[kWaves];
  float zhit[kWaves], zlast[kWaves];
  double t, base, wtot[kWaves];
};

__device__ __forceinline__ u64* record_of(const KArgs& a, int b) {
  return a.ws + static_cast<long long>(b) * a.L.words;
}

// Streaming part of a tile: 8192-logit chunk s of target row i of sequence b.  Each wave reduces
// its 2048-token sub-chunk (max first, then the sum of exp2((z - max) * log2(e)/T); the lowest
// argmax on greedy rows; the sum below x_i in match mode) and lanes 0..3 publish its partial
// (m, s, argmax, sum below x_i) as four marked words; chunk 0 of a drafted row also publishes x_i,
// z_i[x_i] and q_i(x_i).
template <typename LT, bool kVec, bool kMatch>
__device__ void stream_part(const KArgs& a, u64* rec, int b, int i, int s, int kb) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V, S = a.S;
  const long long r = static_cast<long long>(b) * (K + 1) + i;
  const LT* row = static_cast<const LT*>(a.logits) + r * V;
  const int c0 = s * kChunk + wave * kSub;
  const int n = min(kSub, V - c0);
  float x[kPerThread];
  load_sub<LT, kVec>(row, c0, n, lane, x);  // the loads go out first
  const float T = a.greedy_all ? 0.f : a.temperature[b];
  if (s == 0 && tid == 0 && i < kb) {
    // The accept scan's gathers for drafted slot i, recorded while the stream is in flight.
    const long long slot = static_cast<long long>(b) * K + i;
    const int xi = a.proposed[slot];
    float gz = 0.f, gq = 0.f;
    if (xi >= 0 && xi < V) {
      gz = load_logit(row, xi);
      if (a.draft_probs != nullptr && T != 0.f) gq = a.draft_probs[slot * V + xi];
    }
    u64* g = rec + a.L.gathers + static_cast<long long>(i) * 4;
    store_word(g + 0, marked(static_cast<uint32_t>(xi)));
    store_word(g + 1, marked(__float_as_uint(gz)));
    store_word(g + 2, marked(__float_as_uint(gq)));
  }
  const float c = temp_valid(T) ? temp_scale(T) : kLog2e;  // invalid rows: result unused
  float pre = 0.f, lane_max;
  MaxSum st;
  if constexpr (kMatch) {
    // Only the sub-chunk that holds x_i takes the masked sum (a wave-uniform branch); below
    // x_i it is the whole sum, above it 0.
    const int xi = (i < kb && T != 0.f) ? a.proposed[static_cast<long long>(b) * K + i] : -1;
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
  if (lane < 4) {
    const uint32_t v = lane == 0   ? __float_as_uint(st.m)
                       : lane == 1 ? __float_as_uint(st.s)
                       : lane == 2 ? static_cast<uint32_t>(arg)
                                   : __float_as_uint(pre);
    store_word(rec + a.L.partials + (static_cast<long long>(i) * S * kWaves + s * kWaves + wave) * 4 +
                   lane,
               marked(v));
  }
}

// Row statistics of rows [r0, r0 + nrows) of sequence b from their published partials: 16 lanes
// per row, 4 rows per wave and pass, each lane polling (bounded) four of its row's partials at a
// time and merging them max-first as they arrive; the row's lanes then reduce with DPP into LDS.
// Returns false in every lane of a wave if one of its partials did not arrive in time.
template <bool kMatch>
__device__ bool merge_rows(const KArgs& a, Shared& sh, const u64* rec, int r0, int nrows, float c,
                           bool use_d) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nsub = a.S * kWaves;
  const int sl = lane & 15;
  const RowPartial empty{-INFINITY, 0.f, INT_MAX, 0.f};
  bool all_in = true;
  for (int i0 = r0 + 4 * wave; i0 < r0 + nrows; i0 += 4 * kWaves) {  // wave-uniform
    const int ri = i0 + (lane >> 4);
    const bool row_in = ri < r0 + nrows;
    Stat v{-INFINITY, 0.f, INT_MAX};
    StatD vd{-INFINITY, 0.0, 0.0};
    const int per_lane = (nsub + 15) / 16;  // partials j = sl + 16 k of the row, 4 at a time
    for (int t0 = 0; t0 < per_lane; t0 += 4) {
      u64 w[4][4];
      bool got = false;
      for (int n = 0;; ++n) {
        bool mine = true;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j = sl + 16 * (t0 + t);
          const u64* q = rec + a.L.partials + (static_cast<long long>(ri) * nsub + j) * 4;
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            w[t][f] = (row_in && j < nsub) ? load_word(q + f) : marked(0);
            mine = mine && is_marked(w[t][f]);
          }
        }
        if (__ballot(!mine) == 0ull) { got = true; break; }
        if (n >= a.spin_limit) break;
        __builtin_amdgcn_s_sleep(1);
      }
      all_in = all_in && got;
      RowPartial p[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = sl + 16 * (t0 + t);
        p[t] = (got && row_in && j < nsub)
                   ? RowPartial{__uint_as_float(bits_of(w[t][0])), __uint_as_float(bits_of(w[t][1])),
                                static_cast<int>(bits_of(w[t][2])), __uint_as_float(bits_of(w[t][3]))}
                   : empty;
      }
      if (kMatch && use_d)
        vd = merge4_d(vd, p, c);
      else
        v = merge4(v, p, c);
    }
    if (kMatch && use_d) {
      const StatD red = row16_reduce_d(vd, c);
      if (sl == 0 && row_in) sh.rows_d[ri] = red;
    } else {
      const Stat red = row16_reduce_mf(v, c);
      if (sl == 0 && row_in) sh.rows[ri] = red;
    }
  }
  return all_in;
}

// Draw weights of closing tile t of sequence b: s * max(0, p - q) (one-hot rows: p without the
// rejected draft) and s * p over its 2048-token segments in fp64 -- tile t = chunk t, wave w its
// segment 4t + w; or, with `fine`, tile t = segment t, wave w a quarter of it -- published as four
// marked words per segment (the two doubles' halves).
template <typename LT, bool kVecDraw>
__device__ void draw_part(const KArgs& a, Shared& sh, u64* rec, int b, int t, const SeqState& st) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  const long long row = static_cast<long long>(b) * (K + 1) + st.row;
  const LT* z = static_cast<const LT*>(a.logits) + row * V;
  const float* q = st.mode == kResidual
                       ? a.draft_probs + (static_cast<long long>(b) * K + st.row) * V
                       : nullptr;
  const bool fine = a.fine != 0;
  const int segi = fine ? t : t * kSegPerChunk + wave;
  const int span = fine ? kSeg / kWaves : kSeg;
  const int base = segi * kSeg + (fine ? wave * span : 0);
  const int n = min(span, V - base);  // may be <= 0
  double lw = 0.0, le = 0.0;
  if constexpr (kVecDraw) {
    // Lane l owns the 4-token quads l, l + 64, ... of the wave's span: every load instruction
    // of the wave reads one contiguous span (4 logits and 4 fp32 draft probabilities per lane),
    // and all of them go out before any is unpacked.
    constexpr int kQuads = kSeg / 4 / 64;  // 8 (a whole segment per wave)
    DrawVec<LT> zr[kQuads];
    uint4 qr[kQuads];
    const int nq = span / 4 / 64;  // 8, or 2 with fine tiles
#pragma unroll
    for (int h = 0; h < kQuads; ++h) {
      const int v0 = (h * 64 + lane) * 4;
      const bool in = h < nq && v0 < n;
      zr[h] = in ? DrawVec<LT>::load(z + base + v0) : DrawVec<LT>::zero();
      qr[h] = (in && q != nullptr) ? plain_load(q + base + v0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < kQuads; ++h) {
      const int v0 = (h * 64 + lane) * 4;
      float zv[4], qv[4];
      zr[h].unpack(zv);
      unpack(qr[h], qv, static_cast<const float*>(nullptr));
      const int cnt = h < nq ? min(4, n - v0) : 0;
      float gw = 0.f, ge = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float e = 0.f;
        const float wk = k < cnt ? draw_weight(zv[k], qv[k], base + v0 + k, st, false, e) : 0.f;
        gw += wk;
        ge += k < cnt ? e : 0.f;
      }
      lw += gw;
      le += ge;
    }
  } else {
    const int groups = span / kGroup / 64;  // 4, or 1 with fine tiles
    for (int g = 0; g < groups; ++g) {
      const int v0 = (g * 64 + lane) * kGroup;
      float zv[kGroup], qv[kGroup], w[kGroup], gw, ge;
      load_group<LT, false>(z, q, nullptr, base + v0, min(kGroup, n - v0), zv, qv);
      group_weights(zv, qv, base + v0, min(kGroup, n - v0), st, false, w, gw, ge);
      lw += gw;
      le += ge;
    }
  }
  lw = wave_total(lw);
  le = wave_total(le);
  if (fine) {
    if (lane == 0) sh.fine[wave] = SegSums{lw, le};
    __syncthreads();
    if (wave == 0) {
      SegSums tot = sh.fine[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) {
        tot.w += sh.fine[w].w;
        tot.e += sh.fine[w].e;
      }
      lw = tot.w;
      le = tot.e;
    }
  }
  if ((!fine || wave == 0) && lane < 4) {
    const unsigned long long wb = static_cast<unsigned long long>(__double_as_longlong(lw));
    const unsigned long long eb = static_cast<unsigned long long>(__double_as_longlong(le));
    const unsigned long long pick = lane < 2 ? wb : eb;
    const uint32_t half = (lane & 1) ? static_cast<uint32_t>(pick >> 32) : static_cast<uint32_t>(pick);
    store_word(rec + a.L.segs + static_cast<long long>(segi) * 4 + lane, marked(half));
  }
}

// Segment weight sums for a draw: from the draw tiles' marked words (residual and plain sums), or,
// for a plain draw of p, from row j's partials rescaled to the row max: s_j * exp2((m_j - m) c).
// Polls (bounded) until the words are there; false on timeout.
__device__ __forceinline__ bool segment_sums(const KArgs& a, const u64* rec, const SeqState& st,
                                             bool from_partials, int j, double& w, double& e) {
  for (int n = 0;; ++n) {
    if (from_partials) {
      const u64* q = rec + a.L.partials +
                     (static_cast<long long>(st.row) * a.S * kWaves + j) * 4;
      const u64 wm = load_word(q), ws = load_word(q + 1);
      if (is_marked(wm) && is_marked(ws)) {
        const float m = __uint_as_float(bits_of(wm)), s = __uint_as_float(bits_of(ws));
        const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - st.m) * st.c);
        w = e = static_cast<double>(s) * static_cast<double>(f);
        return true;
      }
    } else {
      const u64* q = rec + a.L.segs + static_cast<long long>(j) * 4;
      const u64 w0 = load_word(q), w1 = load_word(q + 1), e0 = load_word(q + 2), e1 = load_word(q + 3);
      if (is_marked(w0) && is_marked(w1) && is_marked(e0) && is_marked(e1)) {
        w = __longlong_as_double(static_cast<long long>((static_cast<u64>(bits_of(w1)) << 32) | bits_of(w0)));
        e = __longlong_as_double(static_cast<long long>((static_cast<u64>(bits_of(e1)) << 32) | bits_of(e0)));
        return true;
      }
    }
    if (n >= a.spin_limit) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Inverse-CDF draw of sequence b from row st.row ("Decodificação especulativa explicada",
// section "Amostragem especulativa em numpy, com prova": the first running sum above u times the
// total, over ascending token id), first step: one fp64 DPP scan over the segment sums (wave 0)
// finds the segment holding u * total (plain p when a residual's total is not positive); the
// result is left in sh.  False (in every thread) if a segment sum did not arrive in time, or if
// the residual's total is NaN.
__device__ bool find_segment(const KArgs& a, Shared& sh, const u64* rec, int b, const SeqState& st,
                             bool from_partials) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K;
  const int nseg = a.S * kSegPerChunk;
  const int P = (nseg + 63) / 64;  // lane l owns segments [l * P, l * P + P)
  const int j0 = lane * P;
  if (wave == 0) {
    const float u_lane = a.uniforms[static_cast<long long>(b) * (K + 1) + min(lane, K)];
    double lw = 0.0, le = 0.0;
    bool got = true;
    for (int q = 0; q < P && j0 + q < nseg; ++q) {
      double w, e;
      got = segment_sums(a, rec, st, from_partials, j0 + q, w, e) && got;
      lw += w;
      le += e;
    }
    const bool all_got = __ballot(!got) == 0ull;
    const double iw = wave_inclusive_scan(lw), ie = wave_inclusive_scan(le);
    const double total_w = read_lane_d(iw, 63);
    // A NaN total (a draft row holding a value that is not a probability): nothing to draw, the
    // sequence is reported invalid.
    const bool drawable = total_w == total_w;
    const bool plain = !(total_w > 0.0);  // empty residual: draw from p itself
    const double inc = plain ? ie : iw;
    const double own = plain ? le : lw;
    const double R = read_lane_d(inc, 63);
    const double t = static_cast<double>(read_lane_f(u_lane, st.ucol)) * R;
    // The first lane whose running total passes t holds the segment; if rounding left t at the
    // very top, the last lane with positive weight does.
    const unsigned long long hit = __ballot(own > 0.0 && inc > t);
    const unsigned long long pos = __ballot(own > 0.0);
    const int hl = hit ? __ffsll(static_cast<long long>(hit)) - 1
                       : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
    if (drawable && lane == hl) {
      double run = inc - own;  // running sum before the lane's segments
      int seg = -1, lastpos = -1;
      double base_seg = 0.0, base_last = 0.0;
      for (int q = 0; q < P && j0 + q < nseg; ++q) {
        double w, e;
        segment_sums(a, rec, st, from_partials, j0 + q, w, e);  // present: read above
        const double v = plain ? e : w;
        if (v > 0.0) {
          if (run + v > t) { seg = j0 + q; base_seg = run; break; }
          lastpos = j0 + q;
          base_last = run;
        }
        run += v;
      }
      if (seg < 0) { seg = lastpos >= 0 ? lastpos : j0; base_seg = base_last; }
      sh.seg = seg; sh.plain = plain; sh.t = t; sh.base = base_seg;
    }
    if (lane == 0) sh.flag = all_got && drawable;
  }
  __syncthreads();
  return sh.flag != 0;
}

// Second step of the draw: a workgroup scan of segment sh.seg in ascending token order finds the
// first running sum above u * total; publishes the token and its probability as two marked words
// (the leader writes every output of the sequence).
template <typename LT, bool kVec>
__device__ void scan_segment(const KArgs& a, Shared& sh, u64* rec, int b, const SeqState& st,
                             bool from_partials) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, V = a.V;
  const long long row = static_cast<long long>(b) * (K + 1) + st.row;
  const int seg = sh.seg;
  const bool plain = from_partials || sh.plain != 0;
  const double t = sh.t;
  const LT* z = static_cast<const LT*>(a.logits) + row * V;
  const int sc = seg / kSegPerChunk, sg = seg % kSegPerChunk;
  const int cc0 = sc * kChunk, cn = min(kChunk, V - cc0);
  const int v0 = sg * kSeg + tid * kGroup;
  const int cnt = min(kGroup, cn - v0);
  const float* qs = (st.mode == kResidual && !plain)
                        ? a.draft_probs + (static_cast<long long>(b) * K + st.row) * V
                        : nullptr;
  float zg[kGroup], qg[kGroup], w[kGroup], gw, ge;
  load_group<LT, kVec>(z, qs, a.ws, cc0 + v0, cnt, zg, qg);
  group_weights(zg, qg, cc0 + v0, cnt, st, plain, w, gw, ge);
  const double inc = wave_inclusive_scan(static_cast<double>(gw));
  if (lane == 63) sh.wtot[wave] = inc;
  __syncthreads();
  double before = sh.base;
  for (int k = 0; k < wave; ++k) before += sh.wtot[k];
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
  const int wave_hit = hm ? __builtin_amdgcn_readlane(hit, hl) : -1;
  const float wave_zhit = read_lane_f(zhit, hl);
  const int wave_last = pm ? __builtin_amdgcn_readlane(lastpos, ll) : -1;
  const float wave_zlast = read_lane_f(zlast, ll);
  if (lane == 0) {
    sh.hit[wave] = wave_hit; sh.zhit[wave] = wave_zhit;
    sh.lastpos[wave] = wave_last; sh.zlast[wave] = wave_zlast;
  }
  __syncthreads();
  if (tid == 0) {
    int y = -1, lp = -1;
    float zy = 0.f, zl = 0.f;
    for (int k = 0; k < kWaves; ++k) {
      if (y < 0 && sh.hit[k] >= 0) { y = sh.hit[k]; zy = sh.zhit[k]; }
      if (sh.lastpos[k] >= 0) { lp = sh.lastpos[k]; zl = sh.zlast[k]; }
    }
    // Rounding left t at the very top of the segment: take its last positive token.
    if (y < 0) {
      y = lp >= 0 ? lp : cc0 + sg * kSeg;
      zy = lp >= 0 ? zl : load_logit(z, y);
    }
    const double p = exp2((static_cast<double>(zy) - static_cast<double>(st.m)) *
                          static_cast<double>(st.c)) / static_cast<double>(st.s);
    store_word(rec + a.L.pick, marked(static_cast<uint32_t>(y)));
    store_word(rec + a.L.pick + 1, marked(__float_as_uint(static_cast<float>(p))));
  }
  __syncthreads();
}

// Puts every word sequence b's round published back to zero (all of them were seen marked, so
// these stores follow the producers' in each word's order): the partials of rows 0..nrows-1, the
// gathers of kb slots, the segment sums, the closing tiles' done words and the drawn token.
__device__ void clear_record(const KArgs& a, u64* rec, int nrows, int kb, bool segs, bool done) {
  const int tid = threadIdx.x;
  const long long per_row = static_cast<long long>(a.S) * kWaves * 4;
  for (long long w = tid; w < nrows * per_row; w += kThreads) store_word(rec + a.L.partials + w, 0);
  for (int w = tid; w < kb * 4; w += kThreads) store_word(rec + a.L.gathers + w, 0);
  if (segs)
    for (long long w = tid; w < a.L.done - a.L.segs; w += kThreads) store_word(rec + a.L.segs + w, 0);
  if (done)
    for (int w = tid; w < a.tasks; w += kThreads) store_word(rec + a.L.done + w, 0);
  if (tid < 2) store_word(rec + a.L.pick + tid, 0);
}

// The round of sequence b as one closing tile sees it: every row of the round (rows 0..k_b, row K
// streamed by the closing tiles themselves) and every gather, polled and merged (16 lanes per row,
// max-first), then wave 0's accept scan (lane i <-> row i, fp64, a 64-bit ballot finds the first
// rejection).  The state goes to sh.st and A to sh.A; wave 0 keeps its output slots in `so`.
// False if a hand-off did not arrive in time.
template <bool kMatch>
__device__ bool scan_round(const KArgs& a, Shared& sh, const u64* rec, int b, int kb_raw, float T,
                           float c, bool use_match, ScanOut& so) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = a.K;
  const bool kb_ok = kb_raw >= 0 && kb_raw <= K;
  const int kb = kb_ok ? kb_raw : 0;
  const long long row0 = static_cast<long long>(b) * (K + 1);
  // Scan inputs that need no hand-off.
  const float u_lane = a.uniforms != nullptr ? a.uniforms[row0 + min(lane, K)] : 0.f;
  const int oh = (!kMatch && a.onehot != nullptr) ? a.onehot[b] : 0;
  bool in = merge_rows<kMatch>(a, sh, rec, 0, kb_ok ? kb + 1 : 0, c, use_match);
  ScanIn sin;
  sin.g = Gather{0.f, 0.f, -1, 0};
  if (wave == 0) {
    // Gathers of the drafted slots (lane i: slot i).
    const u64* g = rec + a.L.gathers + static_cast<long long>(min(lane, max(K - 1, 0))) * 4;
    bool got = false;
    for (int n = 0;; ++n) {
      u64 w0 = 0, w1 = 0, w2 = 0;
      bool mine = true;
      if (lane < kb) {
        w0 = load_word(g); w1 = load_word(g + 1); w2 = load_word(g + 2);
        mine = is_marked(w0) && is_marked(w1) && is_marked(w2);
      }
      if (__ballot(!mine) == 0ull) {
        if (lane < kb)
          sin.g = Gather{__uint_as_float(bits_of(w1)), __uint_as_float(bits_of(w2)),
                         static_cast<int>(bits_of(w0)), 0};
        got = true;
        break;
      }
      if (n >= a.spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    in = in && got;
    sin.u = (a.uniforms != nullptr && lane < K) ? u_lane : 0.f;
    sin.uk = a.uniforms != nullptr ? read_lane_f(u_lane, K) : 0.f;
    sin.onehot = oh != 0;
  }
  if (lane == 0) sh.hit[wave] = in;
  __syncthreads();
  const bool all_in = sh.hit[0] && sh.hit[1] && sh.hit[2] && sh.hit[3];
  if (wave == 0) {
    if (use_match)
      so = accept_sequence_match(sin, kb, T, c, K, a.V, sh.rows_d, lane, false);
    else
      so = accept_sequence(sin, a.draft_probs != nullptr, kb_raw, T, c, K, a.V, sh.rows, lane,
                           false);
    if (lane == 0) {
      sh.st = all_in ? so.st : SeqState{kNone, 0, 0, 0, 0.f, 0.f, 0.f, 0.f};
      sh.A = so.A;
    }
  }
  __syncthreads();
  return all_in;
}

// Closing tile t of sequence b (after it has streamed its share of row K when k_b = K).  Tile 0,
// the leader, writes every token the scan knows; with a residual draw every closing tile sums the
// weights of its segments, reads all segment sums, and the tile that summed the segment holding
// u * total scans it (its rows are still in its cache) and publishes the drawn token; a plain draw
// (bonus) is the leader's.  The leader then waits for the others' done words and writes the drawn
// token -- or, if a wait gave up, reports the sequence invalid -- and puts the record back to zero.
// Only the leader writes outputs, so a sequence reported invalid stays so.  Calls without residual
// draws run only the leader.
template <typename LT, bool kVecDraw, bool kMatch>
__device__ void close_round(const KArgs& a, Shared& sh, u64* rec, int b, int t, int kb_raw) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K;
  const bool lead = t == 0;
  if (!a.draws && !lead) return;
  const bool kb_ok = kb_raw >= 0 && kb_raw <= K;
  const int kb = kb_ok ? kb_raw : 0;
  const float T = a.greedy_all ? 0.f : a.temperature[b];
  const bool use_match = kMatch && T != 0.f && kb_ok;
  const bool scaled = kb_ok && temp_valid(T) && T != 0.f;
  const float c = kLog2e / (scaled ? T : 1.f);
  ScanOut so{};
  const bool in = scan_round<kMatch>(a, sh, rec, b, kb_raw, T, c, use_match, so);
  const SeqState st = sh.st;
  const bool residual = st.mode == kResidual || st.mode == kResidualOnehot;
  if (lead && in && wave == 0)
    write_round_out(so, st.mode != kNone, b, K, a.accept_len, a.out_tokens, a.out_probs, lane);
  bool ok = in;
  if (residual) {
    draw_part<LT, kVecDraw>(a, sh, rec, b, t, st);
    ok = find_segment(a, sh, rec, b, st, false);
    const int owner = a.fine ? sh.seg : sh.seg / kSegPerChunk;
    if (ok && owner == t) scan_segment<LT, kVecDraw>(a, sh, rec, b, st, false);
  } else if (lead && st.mode == kBonus) {
    ok = find_segment(a, sh, rec, b, st, true) && ok;
    if (ok) scan_segment<LT, kVecDraw>(a, sh, rec, b, st, true);
  }
  if (!lead) {
    if (tid == 0) store_word(rec + a.L.done + t, marked(ok ? 1u : 2u));
    return;
  }
  bool bad = !ok;
  if (a.draws) {
    // The other closing tiles report (each 1, or 2 if a wait gave up) after their last read of
    // the record.
    if (wave == 0) {
      bool fine_all = true;
      for (int u = 1 + lane; u < a.tasks; u += 64) {
        bool got = false;
        for (int n = 0;; ++n) {
          const u64 d = load_word(rec + a.L.done + u);
          if (is_marked(d)) { got = bits_of(d) == 1; break; }
          if (n >= a.spin_limit) break;
          __builtin_amdgcn_s_sleep(1);
        }
        fine_all = fine_all && got;
      }
      const bool any_bad = __ballot(!fine_all) != 0ull;
      if (lane == 0) sh.flag = any_bad;
    }
    __syncthreads();
    bad = bad || sh.flag != 0;
  }
  const long long row0 = static_cast<long long>(b) * (K + 1);
  if (!bad && (residual || st.mode == kBonus) && tid == 0) {
    // The drawn token, from whichever closing tile scanned its segment.
    bool got = false;
    u64 y = 0, p = 0;
    for (int n = 0;; ++n) {
      y = load_word(rec + a.L.pick);
      p = load_word(rec + a.L.pick + 1);
      if (is_marked(y) && is_marked(p)) { got = true; break; }
      if (n >= a.spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (got) {
      coherent_store_i(a.out_tokens + row0 + st.row, static_cast<int>(bits_of(y)));
      if (a.out_probs) coherent_store_f(a.out_probs + row0 + st.row, __uint_as_float(bits_of(p)));
    }
    sh.flag = !got;
  }
  __syncthreads();
  if (!bad && (residual || st.mode == kBonus)) bad = sh.flag != 0;
  if (bad) {
    // A wait gave up: the sequence is reported invalid (only this workgroup writes outputs).
    for (int i = tid; i <= K; i += kThreads) {
      coherent_store_i(a.out_tokens + row0 + i, -1);
      if (a.out_probs) coherent_store_f(a.out_probs + row0 + i, 0.f);
    }
    if (tid == 0) coherent_store_i(a.accept_len + b, -1);
  }
  __syncthreads();
  clear_record(a, rec, kb_ok ? kb + 1 : 0, kb, residual, a.draws != 0);
}

// Grid layout: sequences in groups of a.group; per sequence its row tiles (K*S: chunk s of rows
// 0..K-1) and its closing tiles (a.tasks: the chunks of row K, each also a share of the residual
// draw; the first is the sequence's leader).  The closing tiles of group g come after the row
// tiles of group g + 1:
//   R_0, R_1, C_0, R_2, C_1, ..., R_{n-1}, C_{n-2}, C_{n-1}.
// Only the last group may be smaller.  Workgroups are dispatched in order, so a closing tile is
// dispatched after every row tile of its sequence and its waits are short; nothing waits on a
// workgroup dispatched after it, and every wait is bounded.
struct Role {
  int close;  // 0: row tile, 1: closing tile
  int b;
  int t;      // row tile: i * S + s; closing tile: its index
};

__host__ __device__ inline Role decode_block(const KArgs& a, long long x) {
  const long long R1 = static_cast<long long>(a.K) * a.S, T = a.tasks;
  const long long G = a.group;
  const long long n = (a.nb + G - 1) / G;
  const long long last_seqs = a.nb - (n - 1) * G;
  const long long nsF = G * R1, ndF = G * T;
  auto stream = [&](long long g, long long r) {
    return Role{0, a.b0 + static_cast<int>(g * G + r / R1), static_cast<int>(r % R1)};
  };
  auto draw = [&](long long g, long long r) {
    return Role{1, a.b0 + static_cast<int>(g * G + r / T), static_cast<int>(r % T)};
  };
  const long long ns0 = (n == 1 ? last_seqs : G) * R1;
  if (x < ns0) return stream(0, x);
  x -= ns0;
  if (n == 1) return draw(0, x);
  const long long full = n - 2;  // periods [R_{j+1}, C_j] with a full R part
  if (x < full * (nsF + ndF)) {
    const long long j = x / (nsF + ndF), r = x % (nsF + ndF);
    return r < nsF ? stream(j + 1, r) : draw(j, r - nsF);
  }
  x -= full * (nsF + ndF);
  if (x < last_seqs * R1) return stream(n - 1, x);
  x -= last_seqs * R1;
  if (x < ndF) return draw(n - 2, x);
  return draw(n - 1, x - ndF);
}

template <typename LT, bool kVec, bool kVecDraw, bool kMatch>
__global__ __launch_bounds__(kThreads) void verify_kernel(const KArgs a) {
  __shared__ Shared sh;
  const Role r = decode_block(a, blockIdx.x);
  u64* rec = record_of(a, r.b);
  const int kb = a.num_draft != nullptr ? a.num_draft[r.b] : a.K;
  const bool kb_ok = kb >= 0 && kb <= a.K;
  if (!r.close) {
    const int i = r.t / a.S, s = r.t % a.S;
    // Rows past k_b (padding) are never read; nothing is read for an invalid draft count.
    if (kb_ok && i <= kb) stream_part<LT, kVec, kMatch>(a, rec, r.b, i, s, kb);
    return;
  }
  // Closing tile t streams chunk t of row K when k_b = K (with `fine`, tiles past the chunks
  // only draw).
  if (kb_ok && kb == a.K && r.t < a.S) stream_part<LT, kVec, kMatch>(a, rec, r.b, a.K, r.t, kb);
  close_round<LT, kVecDraw, kMatch>(a, sh, rec, r.b, r.t, kb);
}

// Tiles per group: about one resident round of the chip, so closing tiles start while later rows
// still stream.
constexpr long long kGroupTiles = 2048;
// A draw of at most this many 8192-token chunks in the whole call takes one closing tile per
// 2048-token segment instead (a workgroup alone pulls its bytes through one CU's few outstanding
// misses).
constexpr long long kFineMax = 256;
constexpr int kDefaultSpinLimit = 1 << 20;
constexpr long long kMaxBlocks = (1LL << 32) / kThreads - 1;

template <typename LT>
hipError_t launch_one_typed(const LaunchArgs& a) {
  const int S = num_chunks(a.V);
  const bool vec = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) &&
                   ((static_cast<long long>(a.V) * sizeof(LT)) % 16 == 0);
  const bool vec_draw = vec && (a.V % kGroup == 0) &&
                        (a.draft_probs == nullptr ||
                         reinterpret_cast<uintptr_t>(a.draft_probs) % 16 == 0);
  // Only specdec_verify (rejection rule, sampled and greedy rows) selects this path.
  const bool draws = !a.greedy_all;
  const bool fine = draws && static_cast<long long>(a.B) * S <= kFineMax;
  KArgs k{};
  k.logits = a.logits;
  k.draft_probs = a.draft_probs;
  k.onehot = a.onehot;
  k.proposed = a.proposed;
  k.num_draft = a.num_draft;
  k.temperature = a.temperature;
  k.uniforms = a.uniforms;
  k.K = a.K;
  k.V = a.V;
  k.S = S;
  k.greedy_all = a.greedy_all;
  k.draws = draws ? 1 : 0;
  k.fine = fine ? 1 : 0;
  k.tasks = fine ? S * kSegPerChunk : S;
  k.spin_limit = a.spin_limit > 0 ? a.spin_limit : kDefaultSpinLimit;
  k.ws = static_cast<u64*>(a.workspace);
  k.L = record_layout(a.K, a.V);
  k.accept_len = a.accept_len;
  k.out_tokens = a.out_tokens;
  k.out_probs = a.out_probs;
  const long long per_seq = static_cast<long long>(a.K) * S + k.tasks;
  // A launch covers whole sequences and at most kMaxBlocks workgroups (the dispatch packet's
  // grid size counts work-items in 32 bits).
  const long long per_launch = std::max(1LL, kMaxBlocks / per_seq);
  auto kern = vec ? (vec_draw ? verify_kernel<LT, true, true, false> : verify_kernel<LT, true, false, false>)
                  : verify_kernel<LT, false, false, false>;
  // The records start from zeros (a fill kernel, not a memset node, so that the call can be
  // captured in a graph): the workspace then needs no initialisation and may be shared with the
  // three-launch path.
  const long long words = static_cast<long long>(a.B) * k.L.words;
  zero_words<<<grid_for((words + 1) / 2), kThreads, 0, a.stream>>>(k.ws, words);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  for (long long b0 = 0; b0 < a.B; b0 += per_launch) {
    const long long nb = std::min(per_launch, a.B - b0);
    const long long ngroups = (per_seq * nb + kGroupTiles - 1) / kGroupTiles;
    k.b0 = static_cast<int>(b0);
    k.nb = static_cast<int>(nb);
    k.group = static_cast<int>((nb + ngroups - 1) / ngroups);
    const dim3 grid(static_cast<unsigned>(nb * per_seq));
    hipEvent_t ev0 = b0 == 0 ? a.hot_begin : nullptr;
    hipEvent_t ev1 = b0 + per_launch >= a.B ? a.hot_end : nullptr;
    if (ev0 || ev1)
      hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), 0, a.stream, ev0, ev1, 0, k);
    else
      kern<<<grid, kThreads, 0, a.stream>>>(k);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_one_launch(const LaunchArgs& a) {
  if (a.B == 0) return hipSuccess;
  return a.logits_bf16 ? launch_one_typed<uint16_t>(a) : launch_one_typed<float>(a);
}

}  // namespace specdec
