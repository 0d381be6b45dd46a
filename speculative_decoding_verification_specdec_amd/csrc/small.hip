// gfx950 kernel of the verify step for small vocabularies: one wave64 (or one 16-lane group of a
// wave) per sequence.
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
// When a row fits a wave's registers (V <= 1024: at most four 4-token quads per lane) a group of kG
// lanes runs the whole round of one sequence: the whole wave (kG = 64), or, when a row is at most
// 64 tokens and K < 16, each 16-lane DPP row of the wave (kG = 16: four sequences per wave), or,
// for rows of at most 32 tokens and K < 8, each half row (kG = 8: eight per wave).  Quad q of a row
// sits in group lane q % kG, register q / kG, so every load instruction reads contiguous spans. The
// group reads rows 0..k_b once each (with K < 8 and at most two quads per lane, rows 0..K all at
// once; else the next row's loads are in flight while the current one is reduced), reduces each
// row's max, sum and (in waves holding a greedy row) lowest argmax with DPP, takes the accept test
// of each drafted slot (group lane i <-> slot i; with every row in registers all slots at once,
// after the rows, z_i(x_i) gathered from memory), keeps the row to draw from in registers, and
// draws: fp64 group totals per register, the register whose running total passes u * total, one
// fp64 group scan inside it, then the four tokens of the hit lane's quad.  Every cross-lane
// operation stays within its group and sits under branches that are uniform over the group, so each
// one sees its whole group active; the loop over rows runs to the largest k_b of the wave (groups
// past their own k_b change nothing).  One launch, no workspace and no inter-wave communication,
// where the streaming path would spend a 256-thread workgroup and three launches on rows of at most
// 1024 tokens.  (Eight quads per lane would need over 256 registers per lane: one wave per SIMD.)
#include <float.h>
#include <limits.h>
#include <math.h>

#include <hip/hip_ext.h>

#include "kernels.h"
#include "wave_ops.h"

namespace specdec {
namespace {

constexpr int kSmallWaves = 4;  // waves per 256-thread workgroup

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

// Cross-lane operations within a group of kG lanes (base = its first lane).  Every lane of a
// group ends with the same value (scan_d: its inclusive prefix within the group).
//
// Groups inside one 16-lane DPP row (kG = 8: half rows, kG = 16: whole rows).  Quad permutes,
// then row_half_mirror (8) or row_ror 4 and 8 (16), leave the group's max / min / sum in every
// lane; the scan shifts with row_shr and drops what crosses into an 8-lane group from below.
template <int kG> struct Grp {
  static_assert(kG == 8 || kG == 16, "groups of 8 or 16 lanes, or the whole wave");
  template <typename T, typename F>
  static __device__ __forceinline__ T reduce(T v, F op) {
    v = op(v, dpp_x<0xB1>(v));    // quad_perm [1,0,3,2]
    v = op(v, dpp_x<0x4E>(v));    // quad_perm [2,3,0,1]
    if constexpr (kG == 8) return op(v, dpp_x<0x141>(v));  // row_half_mirror
    v = op(v, dpp_x<0x124>(v));   // row_ror:4
    return op(v, dpp_x<0x128>(v));  // row_ror:8
  }
  template <int kCtrl>
  static __device__ __forceinline__ float dpp_x(float v) { return dpp_f<kCtrl>(v); }
  template <int kCtrl>
  static __device__ __forceinline__ int dpp_x(int v) { return dpp_i<kCtrl>(v); }
  static __device__ __forceinline__ float max_f(float v) {
    return reduce(v, [](float x, float y) { return fmaxf(x, y); });
  }
  static __device__ __forceinline__ float at_f(float v, int base, int i) {
    return __shfl(v, base + i, 64);
  }
  static __device__ __forceinline__ int at_i(int v, int base, int i) {
    return __shfl(v, base + i, 64);
  }
  static __device__ __forceinline__ float sum_f(float v, int base) {
    v = reduce(v, [](float x, float y) { return x + y; });
    // row_ror pairs different partial sums in different lanes: take one lane's, so that the
    // group agrees bit for bit (the half-row mirror pairs them commutatively).
    if constexpr (kG == 16) v = at_f(v, base, 0);
    return v;
  }
  static __device__ __forceinline__ int min_i(int v) {
    return reduce(v, [](int x, int y) { return min(x, y); });
  }
  static __device__ __forceinline__ double scan_d(double v) {
    const int gl = static_cast<int>(__lane_id()) & (kG - 1);
    double t = dpp_move_d<0x111, 0xf>(v);  // row_shr:1
    v += (kG == 16 || gl >= 1) ? t : 0.0;
    t = dpp_move_d<0x112, 0xf>(v);         // row_shr:2
    v += (kG == 16 || gl >= 2) ? t : 0.0;
    t = dpp_move_d<0x114, 0xf>(v);         // row_shr:4
    v += (kG == 16 || gl >= 4) ? t : 0.0;
    if constexpr (kG == 16) v += dpp_move_d<0x118, 0xf>(v);  // row_shr:8
    return v;
  }
  static __device__ __forceinline__ double total_d(double v, int base) {
    const long long bits = __double_as_longlong(scan_d(v));
    const int lo = __shfl(static_cast<int>(bits), base + kG - 1, 64);
    const int hi = __shfl(static_cast<int>(bits >> 32), base + kG - 1, 64);
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<unsigned int>(lo));
  }
  static __device__ __forceinline__ unsigned long long bits(unsigned long long m, int base) {
    return (m >> base) & ((1ull << kG) - 1ull);
  }
};

// The whole wave.
template <> struct Grp<64> {
  static __device__ __forceinline__ float max_f(float v) { return wave_max_f(v); }
  static __device__ __forceinline__ float sum_f(float v, int) { return wave_sum_f(v); }
  static __device__ __forceinline__ int min_i(int v) {
    v = min(v, dpp_i<0xB1>(v));
    v = min(v, dpp_i<0x4E>(v));
    v = min(v, dpp_i<0x124>(v));
    v = min(v, dpp_i<0x128>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
  }
  static __device__ __forceinline__ double scan_d(double v) { return wave_inclusive_scan(v); }
  static __device__ __forceinline__ double total_d(double v, int) { return wave_total(v); }
  // Lane base + i's value (i the same in every lane of the wave).
  static __device__ __forceinline__ int at_i(int v, int, int i) {
    return __builtin_amdgcn_readlane(v, i);
  }
  static __device__ __forceinline__ float at_f(float v, int, int i) { return read_lane_f(v, i); }
  static __device__ __forceinline__ unsigned long long bits(unsigned long long m, int) {
    return m;
  }
};
// Row r's quads for this lane (group lane gl): token (j * kG + gl) * 4 + e in z[j][e]; -inf past
// V (mask_row).  Loads are unconditional (addresses clamped into the row) and masked afterwards,
// so that several rows' loads can be in flight before the first wait.  kVec: V % 4 == 0 and the
// row is quad-aligned, so each quad is one load.
template <typename LT, int kQ, int kG, bool kVec>
__device__ __forceinline__ void load_row_raw(const LT* __restrict__ row, int V, int gl,
                                             float (&z)[kQ][4]) {
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    const int v0 = (j * kG + gl) * 4;
    if constexpr (kVec) {
      QuadT<LT>::load(row + min(v0, V - 4), z[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) z[j][e] = QuadT<LT>::one(row, min(v0 + e, V - 1));
    }
  }
}

template <int kQ, int kG>
__device__ __forceinline__ void mask_row(int V, int gl, float (&z)[kQ][4]) {
  if (V == kQ * kG * 4) return;  // every lane's tokens are in the row
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((j * kG + gl) * 4 + e >= V) z[j][e] = -INFINITY;
}

template <typename LT, int kQ, int kG, bool kVec>
__device__ __forceinline__ void load_row(const LT* __restrict__ row, int V, int gl,
                                         float (&z)[kQ][4]) {
  load_row_raw<LT, kQ, kG, kVec>(row, V, gl, z);
  mask_row<kQ, kG>(V, gl, z);
}

template <int kQ, int kG>
__device__ __forceinline__ void load_q_row(const float* __restrict__ q, int V, int gl, bool vec,
                                           float (&w)[kQ][4]) {
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    const int v0 = (j * kG + gl) * 4;
    if (vec) {
      QuadT<float>::load(q + min(v0, V - 4), w[j]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[j][e] = q[min(v0 + e, V - 1)];
    }
  }
}

struct RowStat {
  float m;  // row max
  float s;  // sum of exp2((z - m) * c)
  int a;    // lowest token index attaining m (greedy rows)
};

// Max first, then one exp per logit against it (m * c = hi + lo split exactly, as in the
// streaming kernel), then the lowest argmax.  NaN / +inf logits make s NaN and an all -inf row
// gives s = 0: both fail the caller's s > 0 check.
template <int kQ, int kG>
__device__ __forceinline__ RowStat reduce_row(const float (&z)[kQ][4], float c, bool argmax,
                                              int gl, int base) {
  float lm = -INFINITY;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) lm = fmaxf(lm, z[j][e]);
  const float M = Grp<kG>::max_f(lm);
  const float ref = (M == -INFINITY) ? 0.f : M;
  const float hi = ref * c;
  const float lo = fmaf(ref, c, -hi);
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) ls += __builtin_amdgcn_exp2f(fmaf(z[j][e], c, -hi));
  RowStat r{M, Grp<kG>::sum_f(ls, base) * __builtin_amdgcn_exp2f(-lo), INT_MAX};
  if (argmax) {  // wave-uniform: some group of the wave is greedy
    int a = INT_MAX;
    if (lm == M) {
#pragma unroll
      for (int j = kQ - 1; j >= 0; --j)
#pragma unroll
        for (int e = 3; e >= 0; --e)
          if (z[j][e] == M) a = (j * kG + gl) * 4 + e;
    }
    r.a = Grp<kG>::min_i(a);
  }
  return r;
}

// Match mode: the row's total S and the sum P below token x, both in fp64 from the same
// per-token exponentials as reduce_row (the row max m is given).
template <int kQ, int kG>
__device__ __forceinline__ void match_sums(const float (&z)[kQ][4], float m, float c, int x,
                                           int gl, int base, double& S, double& P) {
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
      lp += (j * kG + gl) * 4 + e < x ? ee : 0.f;
    }
  const double f = static_cast<double>(__builtin_amdgcn_exp2f(-lo));
  S = Grp<kG>::total_d(static_cast<double>(ls), base) * f;
  P = Grp<kG>::total_d(static_cast<double>(lp), base) * f;
}

// Register value z[j][e] of group lane l for the group's token t = (j * kG + l) * 4 + e
// (0 <= t < kQ * kG * 4).
template <int kQ, int kG>
__device__ __forceinline__ float token_value(const float (&z)[kQ][4], int t, int base) {
  const int j = t / (4 * kG), e = t & 3, l = (t >> 2) & (kG - 1);
  float v = 0.f;
#pragma unroll
  for (int jj = 0; jj < kQ; ++jj)
#pragma unroll
    for (int ee = 0; ee < 4; ++ee)
      if (jj == j && ee == e) v = z[jj][ee];
  return Grp<kG>::at_f(v, base, l);
}

template <typename LT, int kQ, int kG, int kR, bool kVec, bool kMatch>
__global__ __launch_bounds__(64 * kSmallWaves) void small_verify_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const uint8_t* __restrict__ onehot, const int32_t* __restrict__ proposed,
    const int32_t* __restrict__ num_draft, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, int B, int K, int V, int greedy_all, int q_vec,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ out_tokens,
    float* __restrict__ out_probs) {
  constexpr int kPerWave = 64 / kG;
  const int lane = threadIdx.x & 63, gl = lane & (kG - 1), base = lane & ~(kG - 1);
  const long long wave_seq = (static_cast<long long>(blockIdx.x) * kSmallWaves +
                              static_cast<long long>(threadIdx.x >> 6)) * kPerWave;
  if (wave_seq >= B) return;  // whole wave
  const long long b_raw = wave_seq + lane / kG;
  const bool live = b_raw < B;             // groups past the batch compute on sequence B - 1
  const int b = live ? static_cast<int>(b_raw) : B - 1;  // and write nothing
  const long long row0 = static_cast<long long>(b) * (K + 1);
  const LT* zrow0 = logits + row0 * V;

  // Everything that does not depend on another load goes out first: row 0 (kR > 0: rows 0..K,
  // whatever k_b is), the draft count, the temperature, the drafted ids (group lane i: slot i)
  // and the uniforms (column i).
  static_assert(kR == 0 || kQ <= 2, "rows held at once only for one or two quads per lane");
  float zc[kQ][4];
  float zr[kR > 0 ? kR : 1][kQ][4];
  if constexpr (kR > 0) {
#pragma unroll
    for (int r = 0; r < kR; ++r)  // (masked where used)
      if (r <= K)
        load_row_raw<LT, kQ, kG, kVec>(zrow0 + static_cast<long long>(r) * V, V, gl, zr[r]);
  } else {
    load_row<LT, kQ, kG, kVec>(zrow0, V, gl, zc);
  }
  const int kb_raw = num_draft != nullptr ? num_draft[b] : K;
  const float T = (greedy_all || temperature == nullptr) ? 0.f : temperature[b];
  const int x_lane = (K > 0 && gl < K) ? proposed[static_cast<long long>(b) * K + gl] : -1;
  const float u_lane = (uniforms != nullptr && gl <= K) ? uniforms[row0 + gl] : 0.f;
  const bool is_oh_flag = onehot != nullptr && onehot[b] != 0;

  const bool seq_ok = kb_raw >= 0 && kb_raw <= K && temp_valid(T);
  const int kb = seq_ok ? kb_raw : 0;
  const bool greedy = T == 0.f;
  // Match mode never reads q: one-hot and model-draft rows are alike there.
  const bool is_onehot = !kMatch && !greedy && is_oh_flag;
  const bool model = !kMatch && !greedy && !is_onehot;
  const float c = seq_ok ? temp_scale(T) : kLog2e;
  // q_i(x_i) gathers (slot i < k_b of a sampled model-draft row), in flight during row 0.
  float q_lane = 0.f;
  const bool x_ok_lane = x_lane >= 0 && x_lane < V;
  if (seq_ok && model && draft_probs != nullptr && gl < kb && x_ok_lane)
    q_lane = draft_probs[(static_cast<long long>(b) * K + gl) * V + x_lane];
  // With every row in registers (kR > 0) the slots are decided together, lane i taking slot i:
  // z_i(x_i) is gathered here (row i was just loaded) instead of read out of the group's
  // registers row by row.
  float zx_lane = 0.f;
  if constexpr (kR > 0) {
    if (seq_ok && gl < kb && x_ok_lane)
      zx_lane = QuadT<LT>::one(zrow0 + static_cast<long long>(gl) * V, x_lane);
  }

  bool ok = seq_ok;
  {
    // Used uniforms: columns < k_b and column K (sampled rows); drafted ids in [0, V);
    // gathered q in [0, FLT_MAX] (sampled model-draft rows).
    const bool bad_u = !greedy && (gl < kb || gl == K) && !(u_lane >= 0.f && u_lane < 1.f);
    const bool bad_x = gl < kb && !x_ok_lane;
    const bool bad_q = model && gl < kb && x_ok_lane && !(q_lane >= 0.f && q_lane <= FLT_MAX);
    if (Grp<kG>::bits(__ballot(bad_u || bad_x || bad_q), base) != 0ull) ok = false;
    if (model && kb > 0 && draft_probs == nullptr) ok = false;
  }

  // Rows 0..k_b: reduce each, decide each drafted slot, keep the row to draw from.  With kR = 0
  // the next row's loads are in flight while the current one is reduced; with kR > 0 (K < kR)
  // every row was loaded at the start.  Rows run to the largest k_b of the wave; a group past
  // its own k_b (or invalid) changes nothing.  (In the rolling schedule, a deeper prefetch --
  // several rows in flight with per-row decisions -- measured slower: its registers cost more
  // occupancy than the round trips it saved.)
  int kb_wave = kb;
  if constexpr (kG < 64) kb_wave = -Grp<64>::min_i(-kb);  // the largest k_b of the wave
  const bool any_greedy = __ballot(greedy) != 0ull;        // rows need their argmax
  int A = kb;                 // first rejected slot (k_b: every draft accepted)
  float zs[kQ][4];            // row A's logits
#pragma unroll
  for (int j = 0; j < kQ; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) zs[j][e] = -INFINITY;
  RowStat sA{0.f, 1.f, INT_MAX};
  double num_lane = 0.0, den_lane = 1.0;  // slot gl's output probability num / den
  // The rolling schedule's step for row i: reduce it, decide slot i, and keep the row when it is
  // the one to draw from.
  auto visit = [&](int i, const float (&z)[kQ][4]) {
    const bool act = ok && i <= kb;
    const RowStat st = reduce_row<kQ, kG>(z, c, any_greedy, gl, base);
    if (act && !(st.s > 0.f)) ok = false;
    const bool decide = act && ok && i < kb && A == kb;
    const int slot = min(i, K > 0 ? K - 1 : 0);
    const int x = Grp<kG>::at_i(x_lane, base, slot);
    const int xt = min(max(x, 0), V - 1);
    const double ex = exp2_diff(token_value<kQ, kG>(z, xt, base), st.m, c);
    bool acc;
    double den = static_cast<double>(st.s);
    if (greedy) {
      acc = x == st.a;
    } else if constexpr (kMatch) {
      // y_i == x_i  <=>  P_i <= u * S_i < P_i + e(x_i)
      double S, P;
      match_sums<kQ, kG>(z, st.m, c, xt, gl, base, S, P);
      const double t = static_cast<double>(Grp<kG>::at_f(u_lane, base, slot)) * S;
      acc = P <= t && t < P + ex;
      den = S;
    } else {
      const double qx = model ? static_cast<double>(Grp<kG>::at_f(q_lane, base, slot)) : 1.0;
      acc = static_cast<double>(Grp<kG>::at_f(u_lane, base, slot)) * qx *
                static_cast<double>(st.s) < ex;
    }
    if (decide && acc && gl == i) {
      num_lane = ex;
      den_lane = den;
    }
    // This row is the one to draw from: the first rejection, or the bonus row.
    const bool take = act && ok && A == kb && ((i < kb && !acc) || i == kb);
    if (decide && !acc) A = i;
    if (take) {
      sA = st;
#pragma unroll
      for (int j = 0; j < kQ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) zs[j][e] = z[j][e];
    }
  };
  if constexpr (kR > 0) {
    // Reduce every row, row i's statistics kept by group lane i; then every drafted slot is
    // decided at once (the same tests as visit's) and the first rejection found by a ballot.
    float m_lane = 0.f, s_lane = 1.f;
    int a_lane = INT_MAX;
    double S_lane = 1.0, P_lane = 0.0;
#pragma unroll
    for (int i = 0; i < kR; ++i)
      if (i <= kb_wave) {  // wave-uniform
        mask_row<kQ, kG>(V, gl, zr[i]);
        const RowStat st = reduce_row<kQ, kG>(zr[i], c, any_greedy, gl, base);
        if (ok && i <= kb && !(st.s > 0.f)) ok = false;
        if constexpr (kMatch) {
          const int x = Grp<kG>::at_i(x_lane, base, min(i, K > 0 ? K - 1 : 0));
          double S, P;
          match_sums<kQ, kG>(zr[i], st.m, c, min(max(x, 0), V - 1), gl, base, S, P);
          if (gl == i) {
            S_lane = S;
            P_lane = P;
          }
        }
        if (gl == i) {
          m_lane = st.m;
          s_lane = st.s;
          a_lane = st.a;
        }
      }
    const double ex = exp2_diff(zx_lane, m_lane, c);
    bool acc;
    if (greedy) {
      acc = x_lane == a_lane;
    } else if constexpr (kMatch) {
      // y_i == x_i  <=>  P_i <= u * S_i < P_i + e(x_i)
      const double t = static_cast<double>(u_lane) * S_lane;
      acc = P_lane <= t && t < P_lane + ex;
    } else {
      const double qx = model ? static_cast<double>(q_lane) : 1.0;
      acc = static_cast<double>(u_lane) * qx * static_cast<double>(s_lane) < ex;
    }
    const unsigned long long rej = Grp<kG>::bits(__ballot(gl < kb && !acc), base);
    A = rej ? __ffsll(static_cast<long long>(rej)) - 1 : kb;
    num_lane = ex;
    den_lane = (kMatch && !greedy) ? S_lane : static_cast<double>(s_lane);
    // The row to draw from: the first rejection, or the bonus row k_b.
    sA = RowStat{Grp<kG>::at_f(m_lane, base, A), Grp<kG>::at_f(s_lane, base, A),
                 Grp<kG>::at_i(a_lane, base, A)};
#pragma unroll
    for (int r = 0; r < kR; ++r)
      if (r == A) {
#pragma unroll
        for (int j = 0; j < kQ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) zs[j][e] = zr[r][j][e];
      }
  } else {
    for (int i = 0; i <= kb_wave; ++i) {  // wave-uniform
      float zn[kQ][4];
      if (i < kb_wave)  // the next row of this sequence (its last one again past k_b)
        load_row<LT, kQ, kG, kVec>(zrow0 + static_cast<long long>(min(i + 1, kb)) * V, V, gl,
                                   zn);
      visit(i, zc);
      if (i < kb_wave) {
#pragma unroll
        for (int j = 0; j < kQ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) zc[j][e] = zn[j][e];
      }
    }
  }

  // The draw (sampled valid sequences; a group-uniform branch: every cross-lane operation
  // inside stays within the group): residual s * max(0, p - q) (model draft), p without x_A
  // (one-hot), or p (the bonus; every match-mode draw, with u[b, A] at a mismatch).
  int yt = -1;
  float zyt = 0.f;
  if (ok && !greedy) {
    const bool residual = !kMatch && A < kb;
    const int ucol = (kMatch && A < kb) ? A : K;
    const int xA = Grp<kG>::at_i(x_lane, base, min(A, K > 0 ? K - 1 : 0));
    const int excl = (residual && is_onehot) ? xA : -1;
    const bool need_q = residual && model;
    float qv[kQ][4];
#pragma unroll
    for (int j = 0; j < kQ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[j][e] = 0.f;
    if (need_q)  // lane-divergent load, no cross-lane operation inside
      load_q_row<kQ, kG>(draft_probs + (static_cast<long long>(b) * K + A) * V, V, gl, q_vec != 0,
                         qv);
    // Weight of token v (lane-local value z, draft probability q); e returns s * p(v).
    auto weight = [&](float zv, float qq, int v, float& e) {
      e = v < V ? __builtin_amdgcn_exp2f((zv - sA.m) * c) : 0.f;
      // A draft probability that is negative, infinite or NaN gives a NaN weight (and total):
      // the sequence is reported invalid below.
      if (residual && model)
        return v < V ? ((qq >= 0.f && qq <= __FLT_MAX__) ? fmaxf(0.f, fmaf(-sA.s, qq, e))
                                                         : __builtin_nanf(""))
                     : 0.f;
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
        gq[j] += weight(zs[j][e], qv[j][e], (j * kG + gl) * 4 + e, ee);
        eq[j] += ee;
      }
    }
    double tot_w[kQ], tot_e[kQ];
    double R = 0.0, E = 0.0;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      tot_w[j] = Grp<kG>::total_d(static_cast<double>(gq[j]), base);
      tot_e[j] = Grp<kG>::total_d(static_cast<double>(eq[j]), base);
      R += tot_w[j];
      E += tot_e[j];
    }
    if (R != R) ok = false;         // a draft row that is not a probability: invalid
    const bool plain = !(R > 0.0);  // empty residual: draw from p itself
    const double total = plain ? E : R;
    const double t = static_cast<double>(Grp<kG>::at_f(u_lane, base, ucol)) * total;
    // The register (quad column) whose running total passes t; the last positive one if
    // rounding left t at the very top.
    int jh = -1, jlast = -1;
    double run0 = 0.0, base_last = 0.0, run = 0.0;
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const double tj = plain ? tot_e[j] : tot_w[j];
      if (tj > 0.0) {
        if (jh < 0 && run + tj > t) { jh = j; run0 = run; }
        jlast = j;
        base_last = run;
      }
      run += tj;
    }
    if (jh < 0) { jh = jlast >= 0 ? jlast : 0; run0 = base_last; }
    // Column jh's weights again (same arithmetic as the sums above).
    float g = 0.f, wq[4] = {0.f, 0.f, 0.f, 0.f}, zq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kQ; ++j)
      if (j == jh) {
        g = plain ? eq[j] : gq[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float ee;
          const float ww = weight(zs[j][e], qv[j][e], (j * kG + gl) * 4 + e, ee);
          wq[e] = plain ? ee : ww;
          zq[e] = zs[j][e];
        }
      }
    const double own = static_cast<double>(g);
    const double inc = Grp<kG>::scan_d(own);
    const unsigned long long hit = Grp<kG>::bits(__ballot(own > 0.0 && run0 + inc > t), base);
    const unsigned long long pos = Grp<kG>::bits(__ballot(own > 0.0), base);
    const int hl = hit ? __ffsll(static_cast<long long>(hit)) - 1
                       : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
    // Each lane walks its quad in token order; the hit lane's result is the draw.
    int y = -1, ylast = -1;
    float zy = 0.f, zlast = 0.f;
    double r = run0 + inc - own;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r += static_cast<double>(wq[e]);
      if (wq[e] > 0.f) {
        const int v = (jh * kG + gl) * 4 + e;
        if (y < 0 && r > t) { y = v; zy = zq[e]; }
        ylast = v;
        zlast = zq[e];
      }
    }
    if (y < 0) { y = ylast; zy = zlast; }
    yt = Grp<kG>::at_i(y, base, hl);
    zyt = Grp<kG>::at_f(zy, base, hl);
  }

  int tok_lane = -1;
  float prob_lane = 0.f;
  if (ok) {
    if (gl < A) {
      tok_lane = x_lane;
      prob_lane = static_cast<float>(num_lane / den_lane);
    } else if (gl == A && greedy) {
      tok_lane = sA.a;         // argmax: exp2(0) / s
      prob_lane = static_cast<float>(1.0 / static_cast<double>(sA.s));
    } else if (gl == A) {
      tok_lane = yt;
      prob_lane = static_cast<float>(exp2_diff(zyt, sA.m, c) / static_cast<double>(sA.s));
    }
  }
  if (live && gl <= K) {
    out_tokens[row0 + gl] = ok ? tok_lane : -1;
    if (out_probs) out_probs[row0 + gl] = ok ? prob_lane : 0.f;
  }
  if (live && gl == 0) accept_len[b] = ok ? A : -1;
}

template <typename LT, int kQ, int kG, int kR = 0>
hipError_t launch_q(const LaunchArgs& a, bool vec, bool q_vec) {
  const LT* z = static_cast<const LT*>(a.logits);
  constexpr int kPerBlock = kSmallWaves * (64 / kG);  // sequences per workgroup
  const unsigned grid = static_cast<unsigned>((a.B + kPerBlock - 1) / kPerBlock);
  auto k = a.match ? (vec ? small_verify_kernel<LT, kQ, kG, kR, true, true>
                          : small_verify_kernel<LT, kQ, kG, kR, false, true>)
                   : (vec ? small_verify_kernel<LT, kQ, kG, kR, true, false>
                          : small_verify_kernel<LT, kQ, kG, kR, false, false>);
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
  // Eight, four or one sequence per wave; with K < 8 and one or two quads per lane every row
  // of a sequence is loaded at once (and its slots decided together).
  if (quads <= 8 && a.K < 8) return launch_q<LT, 1, 8, 8>(a, vec, q_vec);
  if (quads <= 16 && a.K < 8) return launch_q<LT, 1, 16, 8>(a, vec, q_vec);
  if (quads <= 16 && a.K < 16) return launch_q<LT, 1, 16>(a, vec, q_vec);
  if (quads <= 64 && a.K < 8) return launch_q<LT, 1, 64, 8>(a, vec, q_vec);
  if (quads <= 64) return launch_q<LT, 1, 64>(a, vec, q_vec);
  if (quads <= 128 && a.K < 8) return launch_q<LT, 2, 64, 8>(a, vec, q_vec);
  if (quads <= 128) return launch_q<LT, 2, 64>(a, vec, q_vec);
  return launch_q<LT, 4, 64>(a, vec, q_vec);
}

}  // namespace

hipError_t launch_small_verify(const LaunchArgs& a) {
  if (a.B == 0) return hipSuccess;
  return a.logits_bf16 ? launch_small_typed<uint16_t>(a) : launch_small_typed<float>(a);
}

}  // namespace specdec
