// gfx950 kernel of the verify step for small vocabularies: one wave64 per sequence.
//
// The rule is the one kernels.hip implements ("Decodificação especulativa explicada",
// gsantana.dev, section "A regra de amostragem por rejeição"; "ch15 · Speculative Decoding",
// snowch.github.io, section "Why the result is exactly the target model"; "Speculative decoding:
// el secretario...", blog.lo0.es, section "El mecanismo desnudo"): accept x_i while
// u_i * q_i(x_i) < p_i(x_i), then draw the correction from max(0, p - q) (one-hot rows: p without
// x) or the bonus from p_k, by inverse CDF over ascending token id with u[b, K].  In the
// sample-and-match mode (same page, the simpler exact scheme) slot i keeps x_i iff the draw
// from p_i with u[b, i] is x_i, decided from the row total and the sum below x_i, and the first
// mismatch (or the bonus) is a plain draw of p.
//
// When a row fits a wave's registers (V <= 1024: at most four 4-token quads per lane) one wave
// runs the whole round of its sequence.  Quad q of a row sits in lane q % 64, register q / 64, so
// every load instruction of the wave reads one contiguous span.  The wave reads rows 0..k_b once
// each (the next row's loads are in flight while the current one is reduced), reduces each
// row's max, sum and lowest argmax with DPP, takes the accept test of each drafted slot as it
// goes, keeps the row to draw from in registers, and draws: fp64 wave totals per register, the
// register whose running total passes u * total, one fp64 wave scan inside it, then the four
// tokens of the hit lane's quad.  One launch, no workspace and no inter-wave communication,
// where the streaming path would spend a 256-thread workgroup and three launches on rows of at
// most 1024 tokens.  (Eight quads per lane would need over 256 registers per lane: one wave per
// SIMD.)
#include <float.h>
#include <limits.h>
#include <math.h>

#include <hip/hip_ext.h>

#include "kernels.h"
#include "wave_ops.h"

namespace specdec {
namespace {

constexpr int kSmallWaves = 4;  // sequences per 256-thread workgroup

template <typename LT> struct QuadT;
template <> struct QuadT<uint16_t> {  // four bf16 logits: 8 bytes
  static __device__ __forceinline__ void load(const uint16_t* p, float (&o)[4]) {
    const uint2 d = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(d.x << 16); o[1] = __uint_as_float(d.x & 0xffff0000u);
    o[2] = __uint_as_float(d.y << 16); o[3] = __uint_as_float(d.y & 0xffff0000u);
  }
  static __device__ __forceinline__ float one(const uint16_t* p, int i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
};
template <> struct QuadT<float> {  // four fp32 logits: 16 bytes
  static __device__ __forceinline__ void load(const float* p, float (&o)[4]) {
    const float4 d = *reinterpret_cast<const float4*>(p);
    o[0] = d.x; o[1] = d.y; o[2] = d.z; o[3] = d.w;
  }
  static __device__ __forceinline__ float one(const float* p, int i) { return p[i]; }
};

// Row r's quads for this lane: token (j * 64 + lane) * 4 + e in z[j][e]; -inf past V.  Loads are
// unconditional (addresses clamped into the row) and masked afterwards.  kVec: V % 4 == 0 and
// the row is quad-aligned, so each quad is one load.
template <typename LT, int kQ, bool kVec>
__device__ __forceinline__ void load_row(const LT* __restrict__ row, int V, int lane,
                                         float (&z)[kQ][4]) {
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    const int v0 = (j * 64 + lane) * 4;
    if constexpr (kVec) {
      QuadT<LT>::load(row + min(v0, V - 4), z[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[j][e] = QuadT<LT>::one(row, min(v0 + e, V - 1));
    }
  }
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((j * 64 + lane) * 4 + e >= V) z[j][e] = -INFINITY;
}

template <int kQ>
__device__ __forceinline__ void load_q_row(const float* __restrict__ q, int V, int lane, bool vec,
                                           float (&w)[kQ][4]) {
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    const int v0 = (j * 64 + lane) * 4;
    if (vec) {
      QuadT<float>::load(q + min(v0, V - 4), w[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[j][e] = q[min(v0 + e, V - 1)];
    }
  }
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x124>(v));
  v = min(v, dpp_i<0x128>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

struct RowStat {
  float m;  // row max
  float s;  // sum of exp2((z - m) * c)
  int a;    // lowest token index attaining m (greedy rows)
};

// Max first, then one exp per logit against it (m * c = hi + lo split exactly, as in the
// streaming kernel), then the lowest argmax when asked.  NaN / +inf logits make s NaN and an
// all -inf row gives s = 0: both fail the caller's s > 0 check.
template <int kQ>
__device__ __forceinline__ RowStat reduce_row(const float (&z)[kQ][4], float c, bool argmax,
                                              int lane) {
  float lm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) lm = fmaxf(lm, z[j][e]);
  const float M = wave_max_f(lm);
  const float ref = (M == -INFINITY) ? 0.f : M;
  const float hi = ref * c;
  const float lo = fmaf(ref, c, -hi);
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) ls += __builtin_amdgcn_exp2f(fmaf(z[j][e], c, -hi));
  RowStat r{M, wave_sum_f(ls) * __builtin_amdgcn_exp2f(-lo), INT_MAX};
  if (argmax) {
    int a = INT_MAX;
    if (lm == M) {
#pragma unroll
      for (int j = kQ - 1; j >= 0; --j)
#pragma unroll
        for (int e = 3; e >= 0; --e)
          if (z[j][e] == M) a = (j * 64 + lane) * 4 + e;
    }
    r.a = wave_min_i(a);
  }
  return r;
}

// Match mode: the row's total S and the sum P below token x, both in fp64 from the same
// per-token exponentials as reduce_row (the row max m is given).
template <int kQ>
__device__ __forceinline__ void match_sums(const float (&z)[kQ][4], float m, float c, int x,
                                           int lane, double& S, double& P) {
  const float ref = (m == -INFINITY) ? 0.f : m;
  const float hi = ref * c;
  const float lo = fmaf(ref, c, -hi);
  float ls = 0.f, lp = 0.f;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ee = __builtin_amdgcn_exp2f(fmaf(z[j][e], c, -hi));
      ls += ee;
      lp += (j * 64 + lane) * 4 + e < x ? ee : 0.f;
    }
  const double f = static_cast<double>(__builtin_amdgcn_exp2f(-lo));
  S = wave_total(static_cast<double>(ls)) * f;
  P = wave_total(static_cast<double>(lp)) * f;
}

// Register value z[j][e] of lane l for a wave-uniform token t = (j * 64 + l) * 4 + e.
template <int kQ>
__device__ __forceinline__ float token_value(const float (&z)[kQ][4], int t) {
  const int j = t >> 8, e = t & 3, l = (t >> 2) & 63;
  float v = 0.f;
#pragma unroll
  for (int jj = 0; jj < kQ; ++jj)
#pragma unroll
    for (int ee = 0; ee < 4; ++ee)
      if (jj == j && ee == e) v = z[jj][ee];
  return read_lane_f(v, l);
}

template <typename LT, int kQ, bool kVec, bool kMatch>
__global__ __launch_bounds__(64 * kSmallWaves) void small_verify_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const uint8_t* __restrict__ onehot, const int32_t* __restrict__ proposed,
    const int32_t* __restrict__ num_draft, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, int B, int K, int V, int greedy_all, int q_vec,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ out_probs) {
  const int lane = threadIdx.x & 63;
  const int b = static_cast<int>(blockIdx.x) * kSmallWaves + static_cast<int>(threadIdx.x >> 6);
  if (b >= B) return;  // whole wave
  const long long row0 = static_cast<long long>(b) * (K + 1);
  const LT* zrow0 = logits + row0 * V;

  // Everything that does not depend on another load goes out first: row 0, the draft count,
  // the temperature, the drafted ids (lane i: slot i) and the uniforms (lane i: column i).
  float zc[kQ][4];
  load_row<LT, kQ, kVec>(zrow0, V, lane, zc);
  const int kb_raw = num_draft != nullptr ? num_draft[b] : K;
  const float T = (greedy_all || temperature == nullptr) ? 0.f : temperature[b];
  const int x_lane = (K > 0 && lane < K) ? proposed[static_cast<long long>(b) * K + lane] : -1;
  const float u_lane = (uniforms != nullptr && lane <= K) ? uniforms[row0 + lane] : 0.f;
  const bool is_oh_flag = onehot != nullptr && onehot[b] != 0;

  const bool seq_ok = kb_raw >= 0 && kb_raw <= K && temp_valid(T);
  const int kb = seq_ok ? kb_raw : 0;
  const bool greedy = T == 0.f;
  // Match mode never reads q: one-hot and model-draft rows are alike there.
  const bool is_onehot = !kMatch && !greedy && is_oh_flag;
  const bool model = !kMatch && !greedy && !is_onehot;
  const float c = seq_ok ? temp_scale(T) : kLog2e;
  // q_i(x_i) gathers (lane i < k_b of a sampled model-draft row), in flight during row 0.
  float q_lane = 0.f;
  const bool x_ok_lane = x_lane >= 0 && x_lane < V;
  if (seq_ok && model && draft_probs != nullptr && lane < kb && x_ok_lane)
    q_lane = draft_probs[(static_cast<long long>(b) * K + lane) * V + x_lane];

  bool ok = seq_ok;
  if (ok && !greedy) {
    // Used uniforms: columns < k_b and column K.
    const bool bad_u = (lane < kb || lane == K) && !(u_lane >= 0.f && u_lane < 1.f);
    if (__ballot(bad_u) != 0ull) ok = false;
    if (model && kb > 0) {
      if (draft_probs == nullptr) ok = false;
      const bool bad_q = lane < kb && x_ok_lane && !(q_lane >= 0.f && q_lane <= FLT_MAX);
      if (__ballot(bad_q) != 0ull) ok = false;
    }
  }
  if (__ballot(lane < kb && !x_ok_lane) != 0ull) ok = false;

  // Rows 0..k_b: reduce each, decide each drafted slot, keep the row to draw from.  The next
  // row's loads are in flight while the current one is reduced.  (Deeper prefetch -- groups of
  // rows in flight -- measured slower: the extra registers cost more occupancy than the round
  // trips they save.)
  int A = kb;                 // first rejected slot (k_b: every draft accepted)
  float zs[kQ][4];            // row A's logits
  RowStat sA{0.f, 0.f, INT_MAX};
  double num_lane = 0.0, den_lane = 1.0;  // lane i's output probability num / den
  for (int i = 0; i <= kb && ok; ++i) {    // wave-uniform
    float zn[kQ][4];
    if (i < kb) load_row<LT, kQ, kVec>(zrow0 + static_cast<long long>(i + 1) * V, V, lane, zn);
    const RowStat st = reduce_row<kQ>(zc, c, greedy, lane);
    if (!(st.s > 0.f)) {
      ok = false;
      break;
    }
    bool take = false;         // this row is the one to draw from
    if (i < kb && A == kb) {
      const int x = __builtin_amdgcn_readlane(x_lane, i);
      const double ex = exp2((static_cast<double>(token_value<kQ>(zc, x)) -
                              static_cast<double>(st.m)) * static_cast<double>(c));
      bool acc;
      double den = static_cast<double>(st.s);
      if (greedy) {
        acc = x == st.a;
      } else if constexpr (kMatch) {
        // y_i == x_i  <=>  P_i <= u * S_i < P_i + e(x_i)
        double S, P;
        match_sums<kQ>(zc, st.m, c, x, lane, S, P);
        const double t = static_cast<double>(read_lane_f(u_lane, i)) * S;
        acc = P <= t && t < P + ex;
        den = S;
      } else {
        const double qx = model ? static_cast<double>(read_lane_f(q_lane, i)) : 1.0;
        acc = static_cast<double>(read_lane_f(u_lane, i)) * qx * static_cast<double>(st.s) < ex;
      }
      if (acc) {
        if (lane == i) {
          num_lane = ex;
          den_lane = den;
        }
      } else {
        A = i;
        take = true;
      }
    } else if (i == kb && A == kb) {
      take = true;             // the bonus row
    }
    if (take) {
      sA = st;
#pragma unroll
      for (int j = 0; j < kQ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) zs[j][e] = zc[j][e];
    }
    if (i < kb) {
#pragma unroll
      for (int j = 0; j < kQ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) zc[j][e] = zn[j][e];
    }
  }

  int tok_lane = -1;
  float prob_lane = 0.f;
  if (ok) {
    if (lane < A) {
      tok_lane = x_lane;
      prob_lane = static_cast<float>(num_lane / den_lane);
    }
    if (greedy) {
      if (lane == A) {
        tok_lane = sA.a;       // argmax: exp2(0) / s
        prob_lane = static_cast<float>(1.0 / static_cast<double>(sA.s));
      }
    } else {
      // The draw: residual s * max(0, p - q) (model draft), p without x_A (one-hot), or p
      // (the bonus; every match-mode draw, with u[b, A] at a mismatch).
      const bool residual = !kMatch && A < kb;
      const int ucol = (kMatch && A < kb) ? A : K;
      const int excl = (residual && is_onehot) ? __builtin_amdgcn_readlane(x_lane, A) : -1;
      float qv[kQ][4];
      if (residual && model)
        load_q_row<kQ>(draft_probs + (static_cast<long long>(b) * K + A) * V, V, lane,
                       q_vec != 0, qv);
      // Weight of token v (lane-local value z, draft probability q); e returns s * p(v).
      auto weight = [&](float zv, float qq, int v, float& e) {
        e = v < V ? __builtin_amdgcn_exp2f((zv - sA.m) * c) : 0.f;
        if (residual && model) return v < V ? fmaxf(0.f, fmaf(-sA.s, qq, e)) : 0.f;
        if (residual) return v == excl ? 0.f : e;
        return e;
      };
      float gq[kQ], eq[kQ];
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        gq[j] = 0.f;
        eq[j] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float ee;
          gq[j] += weight(zs[j][e], (residual && model) ? qv[j][e] : 0.f, (j * 64 + lane) * 4 + e,
                          ee);
          eq[j] += ee;
        }
      }
      double tot_w[kQ], tot_e[kQ];
      double R = 0.0, E = 0.0;
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        tot_w[j] = wave_total(static_cast<double>(gq[j]));
        tot_e[j] = wave_total(static_cast<double>(eq[j]));
        R += tot_w[j];
        E += tot_e[j];
      }
      const bool plain = !(R > 0.0);  // empty residual: draw from p itself
      const double total = plain ? E : R;
      const double t = static_cast<double>(read_lane_f(u_lane, ucol)) * total;
      // The register (quad column) whose running total passes t; the last positive one if
      // rounding left t at the very top.
      int jh = -1, jlast = -1;
      double base = 0.0, base_last = 0.0, run = 0.0;
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const double tj = plain ? tot_e[j] : tot_w[j];
        if (tj > 0.0) {
          if (jh < 0 && run + tj > t) { jh = j; base = run; }
          jlast = j;
          base_last = run;
        }
        run += tj;
      }
      if (jh < 0) { jh = jlast >= 0 ? jlast : 0; base = base_last; }
      // Column jh's weights again (same arithmetic as the sums above).
      float g = 0.f, wq[4] = {0.f, 0.f, 0.f, 0.f}, zq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kQ; ++j)
        if (j == jh) {
          g = plain ? eq[j] : gq[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float ee;
            const float ww = weight(zs[j][e], (residual && model) ? qv[j][e] : 0.f,
                                    (j * 64 + lane) * 4 + e, ee);
            wq[e] = plain ? ee : ww;
            zq[e] = zs[j][e];
          }
        }
      const double own = static_cast<double>(g);
      const double inc = wave_inclusive_scan(own);
      const unsigned long long hit = __ballot(own > 0.0 && base + inc > t);
      const unsigned long long pos = __ballot(own > 0.0);
      const int hl = hit ? __ffsll(static_cast<long long>(hit)) - 1
                         : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
      // The hit lane walks its quad in token order.
      int y = -1, ylast = -1;
      float zy = 0.f, zlast = 0.f;
      double r = base + inc - own;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r += static_cast<double>(wq[e]);
        if (wq[e] > 0.f) {
          const int v = (jh * 64 + lane) * 4 + e;
          if (y < 0 && r > t) { y = v; zy = zq[e]; }
          ylast = v;
          zlast = zq[e];
        }
      }
      if (y < 0) { y = ylast; zy = zlast; }
      const int yt = __builtin_amdgcn_readlane(y, hl);
      const float zyt = read_lane_f(zy, hl);
      if (lane == A) {
        tok_lane = yt;
        prob_lane = static_cast<float>(
            exp2((static_cast<double>(zyt) - static_cast<double>(sA.m)) * static_cast<double>(c)) /
            static_cast<double>(sA.s));
      }
    }
  }
  if (lane <= K) {
    out_tokens[row0 + lane] = ok ? tok_lane : -1;
    if (out_probs) out_probs[row0 + lane] = ok ? prob_lane : 0.f;
  }
  if (lane == 0) accept_len[b] = ok ? A : -1;
}

template <typename LT, int kQ>
hipError_t launch_q(const LaunchArgs& a, bool vec, bool q_vec) {
  const LT* z = static_cast<const LT*>(a.logits);
  const unsigned grid = static_cast<unsigned>((a.B + kSmallWaves - 1) / kSmallWaves);
  auto k = a.match ? (vec ? small_verify_kernel<LT, kQ, true, true>
                          : small_verify_kernel<LT, kQ, false, true>)
                   : (vec ? small_verify_kernel<LT, kQ, true, false>
                          : small_verify_kernel<LT, kQ, false, false>);
  if (a.hot_begin || a.hot_end)
    hipExtLaunchKernelGGL(k, dim3(grid), dim3(64 * kSmallWaves), 0, a.stream, a.hot_begin,
                          a.hot_end, 0, z, a.draft_probs, a.onehot, a.proposed, a.num_draft,
                          a.temperature, a.uniforms, a.B, a.K, a.V, a.greedy_all, q_vec ? 1 : 0,
                          a.accept_len, a.out_tokens, a.out_probs);
  else
    k<<<grid, 64 * kSmallWaves, 0, a.stream>>>(z, a.draft_probs, a.onehot, a.proposed,
                                               a.num_draft, a.temperature, a.uniforms, a.B, a.K,
                                               a.V, a.greedy_all, q_vec ? 1 : 0, a.accept_len,
                                               a.out_tokens, a.out_probs);
  return hipGetLastError();
}

template <typename LT>
hipError_t launch_small_typed(const LaunchArgs& a) {
  const bool vec = a.V % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(a.logits) % (4 * sizeof(LT)) == 0;
  const bool q_vec = a.V % 4 == 0 && (a.draft_probs == nullptr ||
                                      reinterpret_cast<uintptr_t>(a.draft_probs) % 16 == 0);
  const int quads = (a.V + 3) / 4;  // at most 256: V <= kSmallVMax
  if (quads <= 64) return launch_q<LT, 1>(a, vec, q_vec);
  if (quads <= 128) return launch_q<LT, 2>(a, vec, q_vec);
  return launch_q<LT, 4>(a, vec, q_vec);
}

}  // namespace

hipError_t launch_small_verify(const LaunchArgs& a) {
  if (a.B == 0) return hipSuccess;
  return a.logits_bf16 ? launch_small_typed<uint16_t>(a) : launch_small_typed<float>(a);
}

}  // namespace specdec
