// Device building blocks of the streaming verify paths (kernels.hip: three launches; fused.hip:
// one launch): loads of logit rows, the streaming (max, sum, argmax) fold of a wave's sub-chunk,
// max-first merges of partial statistics, the accept scans of both rules, the draw weights, and
// relaxed device-scope accesses for data one workgroup hands to another.
//
// The rule is the one the source pages define: "Decodificação especulativa explicada"
// (gsantana.dev), section "A regra de amostragem por rejeição"; "ch15 · Speculative Decoding"
// (snowch.github.io), section "Why the result is exactly the target model"; "Speculative
// decoding: el secretario que adelanta lo que va a decir el jefe" (blog.lo0.es), section "El
// mecanismo desnudo".
#pragma once

#include <float.h>
#include <limits.h>
#include <math.h>

#include <hip/hip_runtime.h>

#include "kernels.h"
#include "wave_ops.h"

namespace specdec {

constexpr int kWaves = kThreads / 64;
constexpr int kSub = kChunk / kWaves;          // tokens per wave sub-chunk (2048)
constexpr int kPerThread = kSub / 64;          // logits per lane per sub-chunk (32)
constexpr int kMaxRows = 64;           // K + 1 <= 64 target rows per sequence

__device__ __forceinline__ float load_logit(const uint16_t* p, long long i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float load_logit(const float* p, long long i) { return p[i]; }

// 16-byte vector -> floats (bf16: shift / mask into the upper half of a binary32).
__device__ __forceinline__ void unpack(const uint4& d, float* o, const uint16_t*) {
  o[0] = __uint_as_float(d.x << 16); o[1] = __uint_as_float(d.x & 0xffff0000u);
  o[2] = __uint_as_float(d.y << 16); o[3] = __uint_as_float(d.y & 0xffff0000u);
  o[4] = __uint_as_float(d.z << 16); o[5] = __uint_as_float(d.z & 0xffff0000u);
  o[6] = __uint_as_float(d.w << 16); o[7] = __uint_as_float(d.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack(const uint4& d, float* o, const float*) {
  o[0] = __uint_as_float(d.x); o[1] = __uint_as_float(d.y);
  o[2] = __uint_as_float(d.z); o[3] = __uint_as_float(d.w);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Plain (cached) 16-byte load: the draw kernel's reads of the row to draw from, which the pick
// kernel re-reads one segment of (nontemporal loads there measured 3-6 % slower on the large
// and ragged batches).
__device__ __forceinline__ uint4 plain_load(const void* p) {
  const u32x4 t = *static_cast<const u32x4*>(p);
  return make_uint4(t.x, t.y, t.z, t.w);
}
// 16-byte streaming load: the streaming kernel reads every logit once per call, so its loads
// carry the nontemporal hint.
__device__ __forceinline__ uint4 stream_load(const void* p) {
  const u32x4 t = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ------------------------------------------------------------------------------------------
// Data handed from one workgroup to another inside the launch (partials, gathers, draw state,
// segment sums, outputs that another workgroup may overwrite) is written and read with relaxed
// device-scope atomic accesses: on gfx950 these bypass the per-XCD L2's non-coherent copies, so a
// reader on any XCD sees the value once the writer's store has been performed.  A writer waits
// for its stores to be performed (vmcnt 0) before it publishes them with a relaxed atomic count or
// flag; a reader issues its loads only after it has seen that count or flag.  No release fence is
// used: on this chip an agent-scope release writes back the whole per-XCD L2 (measured: a fence
// per workgroup of the streaming pass takes it from 16 us to 250 us or more), while the stores
// that need publishing here are already coherent.
// ------------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T coherent_load(const T* p) {
  static_assert(sizeof(T) % 8 == 0, "64-bit words");
  union {
    T t;
    unsigned long long w[sizeof(T) / 8];
  } u;
  const unsigned long long* s = reinterpret_cast<const unsigned long long*>(p);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(T) / 8); ++i)
    u.w[i] = __hip_atomic_load(s + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u.t;
}
template <typename T>
__device__ __forceinline__ void coherent_store(T* p, const T& v) {
  static_assert(sizeof(T) % 8 == 0, "64-bit words");
  union {
    T t;
    unsigned long long w[sizeof(T) / 8];
  } u;
  u.t = v;
  unsigned long long* d = reinterpret_cast<unsigned long long*>(p);
#pragma unroll
  for (int i = 0; i < static_cast<int>(sizeof(T) / 8); ++i)
    __hip_atomic_store(d + i, u.w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_i(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_f(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every store this wave issued has been performed (and keeps the compiler from
// moving memory accesses across the wait).
__device__ __forceinline__ void stores_performed() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename LT> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int kPer = 8;
  static constexpr uint32_t kNegInf = 0xff80ff80u;  // two bf16 -inf
};
template <> struct Vec<float> {
  static constexpr int kPer = 4;
  static constexpr uint32_t kNegInf = 0xff800000u;
};

// Running (max, sum of exp2((z - max) * c), lowest argmax) of a set of logits.
struct Stat {
  float m;
  float s;
  int a;
};


// ------------------------------------------------------------------------------------------
// Streaming statistics of one wave's sub-chunk.  The wave's max is reduced first and every lane
// exponentiates against it, so the sum is a plain wave sum: one exp per logit plus one, instead
// of a rescaling (m, s) merge at every reduction step.
// ------------------------------------------------------------------------------------------
struct MaxSum {
  float m;
  float s;
};

template <typename LT, bool kVec>
__device__ __forceinline__ int tok_of(int c0, int lane, int j);

// (max, sum of exp2((z - max) * c)) of the wave's logits, and with kPre the same sum over the
// tokens below `xid` (match mode).  exp2((z - m) * c) is taken as exp2(fma(z, c, -hi)) * exp2(-lo)
// with m * c = hi + lo split exactly: one fma per logit and an exponent exact up to the fma's
// rounding.  An all -inf (or NaN) sub-chunk keeps the reference at 0 so -inf maps to 0; NaN and
// +inf logits make the sum NaN, which marks the row invalid.
template <typename LT, bool kVec, bool kPre>
__device__ __forceinline__ MaxSum fold_wave(const float (&x)[kPerThread], float c, int c0,
                                           int lane, int xid, float& lane_max, float& pre) {
  float bm = x[0];
#pragma unroll
  for (int j = 1; j < kPerThread; ++j) bm = fmaxf(bm, x[j]);
  lane_max = bm;
  const float M = wave_max_f(bm);
  const float ref = (M == -INFINITY) ? 0.f : M;
  const float hi = ref * c;
  const float lo = fmaf(ref, c, -hi);
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f, p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; j += 4) {
    const float e0 = __builtin_amdgcn_exp2f(fmaf(x[j], c, -hi));
    const float e1 = __builtin_amdgcn_exp2f(fmaf(x[j + 1], c, -hi));
    const float e2 = __builtin_amdgcn_exp2f(fmaf(x[j + 2], c, -hi));
    const float e3 = __builtin_amdgcn_exp2f(fmaf(x[j + 3], c, -hi));
    s0 += e0; s1 += e1; s2 += e2; s3 += e3;
    if constexpr (kPre) {
      p0 += tok_of<LT, kVec>(c0, lane, j) < xid ? e0 : 0.f;
      p1 += tok_of<LT, kVec>(c0, lane, j + 1) < xid ? e1 : 0.f;
      p2 += tok_of<LT, kVec>(c0, lane, j + 2) < xid ? e2 : 0.f;
      p3 += tok_of<LT, kVec>(c0, lane, j + 3) < xid ? e3 : 0.f;
    }
  }
  const float f = __builtin_amdgcn_exp2f(-lo);
  if constexpr (kPre) pre = wave_sum_f((p0 + p1) + (p2 + p3)) * f;
  return MaxSum{M, wave_sum_f((s0 + s1) + (s2 + s3)) * f};
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}

// Load one lane's logits of the wave's sub-chunk [c0, c0 + n) (n <= kSub, possibly <= 0):
// 16-byte vectors u * 64 + lane (scalar path: tokens u * 64 + lane), all issued before any
// value is used.  Slots past n read as -inf.
template <typename LT, bool kVec>
__device__ __forceinline__ void load_sub(const LT* __restrict__ row, int c0, int n, int lane,
                                         float (&x)[kPerThread]) {
  if constexpr (kVec) {
    constexpr int P = Vec<LT>::kPer;
    constexpr int U = kPerThread / P;
    const uint4* vrow = reinterpret_cast<const uint4*>(row + c0);
    const int nvec = n / P;
    uint4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = u * 64 + lane;
      constexpr uint32_t ni = Vec<LT>::kNegInf;
      d[u] = vi < nvec ? stream_load(vrow + vi) : make_uint4(ni, ni, ni, ni);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) unpack(d[u], &x[u * P], static_cast<const LT*>(nullptr));
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int vi = j * 64 + lane;
      x[j] = vi < n ? load_logit(row, c0 + vi) : -INFINITY;
    }
  }
}

// The lowest token index of the wave's sub-chunk holding the value M (INT_MAX when none does),
// from one ballot per register: tokens ascend with (16-byte vector u, lane, element k) on the
// vector path and with (register j, lane) on the scalar one, so the first register group with a
// hit, its lowest hit lane and that lane's first hit element name the token.  The result is
// wave-uniform; no cross-lane reduction is needed.
template <typename LT, bool kVec>
__device__ __forceinline__ int lowest_token_of(const float (&x)[kPerThread], float M, int c0) {
  if constexpr (kVec) {
    constexpr int P = Vec<LT>::kPer;
    constexpr int U = kPerThread / P;
    for (int u = 0; u < U; ++u) {
      unsigned long long hit[P];
      unsigned long long any = 0ull;
#pragma unroll
      for (int k = 0; k < P; ++k) {
        hit[k] = __ballot(x[u * P + k] == M);
        any |= hit[k];
      }
      if (any != 0ull) {
        const int l = __ffsll(static_cast<long long>(any)) - 1;
#pragma unroll
        for (int k = 0; k < P; ++k)
          if ((hit[k] >> l) & 1ull) return c0 + (u * 64 + l) * P + k;
      }
    }
  } else {
    for (int j = 0; j < kPerThread; ++j) {
      const unsigned long long hit = __ballot(x[j] == M);
      if (hit != 0ull) return c0 + j * 64 + __ffsll(static_cast<long long>(hit)) - 1;
    }
  }
  return INT_MAX;
}

template <typename LT, bool kVec>
__device__ __forceinline__ int tok_of(int c0, int lane, int j) {
  if constexpr (kVec) {
    constexpr int P = Vec<LT>::kPer;
    return c0 + ((j / P) * 64 + lane) * P + (j % P);
  } else {
    return c0 + j * 64 + lane;
  }
}

// Max-first merges of the row partials for the accept scan: the maximum is found first and each
// sum is rescaled once against it (independent exps, no dependent chain of pairwise merges).
// The lowest index attaining the maximum is kept for greedy rows.
__device__ __forceinline__ Stat merge4(const Stat& v, const RowPartial (&p)[4], float c) {
  float M = v.m;
#pragma unroll
  for (int t = 0; t < 4; ++t) M = fmaxf(M, p[t].m);
  Stat r{M, 0.f, INT_MAX};
  if (M == -INFINITY) {  // nothing but empty sub-chunks (NaN sums stay NaN)
    r.s = v.s;
#pragma unroll
    for (int t = 0; t < 4; ++t) r.s += p[t].s;
    return r;
  }
  r.s = v.s * __builtin_amdgcn_exp2f((v.m - M) * c);
  r.a = v.m == M ? v.a : INT_MAX;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    r.s += p[t].s * __builtin_amdgcn_exp2f((p[t].m - M) * c);
    if (p[t].m == M) r.a = min(r.a, p[t].arg);
  }
  return r;
}

// The same over each 16-lane row (every lane of a row ends with its row's result).
__device__ __forceinline__ Stat row16_reduce_mf(const Stat& v, float c) {
  float M = v.m;
  M = fmaxf(M, dpp_f<0xB1>(M));
  M = fmaxf(M, dpp_f<0x4E>(M));
  M = fmaxf(M, dpp_f<0x124>(M));
  M = fmaxf(M, dpp_f<0x128>(M));
  float sum = M == -INFINITY ? v.s : v.s * __builtin_amdgcn_exp2f((v.m - M) * c);
  sum += dpp_f<0xB1>(sum);
  sum += dpp_f<0x4E>(sum);
  sum += dpp_f<0x124>(sum);
  sum += dpp_f<0x128>(sum);
  int a = v.m == M ? v.a : INT_MAX;
  a = min(a, dpp_i<0xB1>(a));
  a = min(a, dpp_i<0x4E>(a));
  a = min(a, dpp_i<0x124>(a));
  a = min(a, dpp_i<0x128>(a));
  return Stat{M, sum, a};
}

// Inputs of the accept scan that need neither the row statistics nor the temperature: the
// drafted ids with their gathered logit and q (recorded by the streaming kernel), the uniforms
// and the one-hot flag.  Lane i holds slot i.
struct ScanIn {
  Gather g;
  float u;
  float uk;
  int onehot;
};

// What an accept scan decides: the draw state (the same in every lane), the accept length and
// lane i's output slot i: its token (-1 where the draw or nothing goes) and its probability as
// num / den, divided only when the outputs are written (after the state is published).
struct ScanOut {
  SeqState st;
  int A;
  int tok;
  double num;
  double den;
};

// Accept scan of sequence b by one wave64 (lane i <-> target row i), given its raw draft count,
// temperature, exp2 scale c (temp_scale(T) for a valid sequence, else log2(e)) and the row
// statistics in LDS (an invalid count or temperature poisons the sequence).  Returns what
// remains to be drawn and the tokens already known.  The test u * q(x) < p(x) = e / s is taken
// as u * q(x) * s < e in fp64, so no division stands before the decision.  With `pending` the
// statistics of row k_b (= K) are not known yet: that row is taken as valid here (the finisher
// checks it), and a greedy bonus from it is left to the finisher.
__device__ __forceinline__ ScanOut accept_sequence(const ScanIn& in, bool have_q, int kb_raw,
                                                   float T, float c, int K, int V,
                                                   const Stat* sh_rows, int lane, bool pending = false) {
  const Gather g = in.g;
  const float u = in.u, uk = in.uk;
  const bool seq_ok = kb_raw >= 0 && kb_raw <= K && temp_valid(T);
  const int kb = seq_ok ? kb_raw : 0;
  const bool greedy = (T == 0.f);
  const bool is_onehot = !greedy && in.onehot;
  const Stat st = lane <= K ? sh_rows[lane] : Stat{-INFINITY, 0.f, INT_MAX};

  const bool drafted = lane < kb;
  const int x = g.x;
  const bool x_ok = x >= 0 && x < V;
  bool lane_ok = true;
  double ex = 0.0;  // exp2((z_i[x_i] - m_i) * c) = s_i * p_i(x_i)
  bool acc = true;
  if (lane <= kb) {
    lane_ok = (pending && lane == kb) || st.s > 0.f;  // NaN / +inf logit -> NaN; all -inf -> 0
    if (drafted) {
      if (!x_ok) {
        lane_ok = false;
      } else {
        ex = exp2((static_cast<double>(g.z) - static_cast<double>(st.m)) *
                  static_cast<double>(c));
        if (greedy) {
          acc = (x == st.a);
        } else {
          if (!(u >= 0.f && u < 1.f)) lane_ok = false;
          double qx = 1.0;  // one-hot drafter: q(x) = 1
          if (!is_onehot) {
            if (!have_q) lane_ok = false;
            else if (!(g.q >= 0.f && g.q <= FLT_MAX)) lane_ok = false;
            qx = g.q;
          }
          acc = static_cast<double>(u) * qx * static_cast<double>(st.s) < ex;
        }
      }
    }
  }
  if (!greedy && lane == 0 && !(uk >= 0.f && uk < 1.f)) lane_ok = false;
  const bool ok = seq_ok && (__ballot(!lane_ok) == 0ull);
  const unsigned long long rej = __ballot(lane < kb && !acc);
  const int A = ok ? (rej ? __ffsll(static_cast<long long>(rej)) - 1 : kb) : -1;

  SeqState out{kNone, 0, 0, 0, 0.f, 0.f, 0.f, 0.f};
  if (ok && !greedy) {  // A is wave-uniform: lane A's row is the one to draw from
    const int mode = (A == kb) ? kBonus : (is_onehot ? kResidualOnehot : kResidual);
    out = SeqState{mode, A, __builtin_amdgcn_readlane(x, A), K, c, read_lane_f(st.m, A),
                   read_lane_f(st.s, A), 0.f};
  }
  ScanOut o{out, A, -1, 0.0, 1.0};                  // a sampled slot is filled by the draw
  if (ok && lane < A) {
    o.tok = x;
    o.num = ex;
    o.den = static_cast<double>(st.s);
  } else if (ok && lane == A && greedy && !(pending && A == kb)) {
    o.tok = st.a;                                    // argmax: exp2(0) / s
    o.num = 1.0;
    o.den = static_cast<double>(st.s);
  }
  return o;
}

// ------------------------------------------------------------------------------------------
// Match mode ("Decodificação especulativa explicada", section "A regra de amostragem por
// rejeição", the simpler exact scheme): position i draws y_i from p_i with u[b, i] (the bonus
// position with u[b, K]) and the draft is kept while y_i == x_i.  The inverse-CDF draw picks x_i
// exactly when its interval [C(x_i - 1), C(x_i)) of the running sum holds t = u * total, so the
// scan decides every position from the row's total S_i, the sum P_i below x_i and x_i's own
// weight -- no pass over the row.  Only the first mismatching position (or the bonus) is then
// drawn by the draw kernels, as a plain sample of p with its own uniform column.
// ------------------------------------------------------------------------------------------
struct StatD {
  float m;
  double s;  // sum of exp2((z - m) * c)
  double p;  // the same sum below the drafted id
};

__device__ __forceinline__ StatD merge4_d(const StatD& v, const RowPartial (&p)[4], float c) {
  float M = v.m;
#pragma unroll
  for (int t = 0; t < 4; ++t) M = fmaxf(M, p[t].m);
  StatD r{M, v.s, v.p};
  if (M == -INFINITY) {
#pragma unroll
    for (int t = 0; t < 4; ++t) { r.s += p[t].s; r.p += p[t].pre; }
    return r;
  }
  const double fv = __builtin_amdgcn_exp2f((v.m - M) * c);
  r.s = v.s * fv;
  r.p = v.p * fv;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const double f = __builtin_amdgcn_exp2f((p[t].m - M) * c);
    r.s += static_cast<double>(p[t].s) * f;
    r.p += static_cast<double>(p[t].pre) * f;
  }
  return r;
}

__device__ __forceinline__ StatD row16_reduce_d(const StatD& v, float c) {
  float M = v.m;
  M = fmaxf(M, dpp_f<0xB1>(M));
  M = fmaxf(M, dpp_f<0x4E>(M));
  M = fmaxf(M, dpp_f<0x124>(M));
  M = fmaxf(M, dpp_f<0x128>(M));
  const double f = M == -INFINITY ? 1.0 : static_cast<double>(__builtin_amdgcn_exp2f((v.m - M) * c));
  double sum = v.s * f, pre = v.p * f;
  sum += dpp_move_d<0xB1, 0xf>(sum);
  pre += dpp_move_d<0xB1, 0xf>(pre);
  sum += dpp_move_d<0x4E, 0xf>(sum);
  pre += dpp_move_d<0x4E, 0xf>(pre);
  sum += dpp_move_d<0x124, 0xf>(sum);
  pre += dpp_move_d<0x124, 0xf>(pre);
  sum += dpp_move_d<0x128, 0xf>(sum);
  pre += dpp_move_d<0x128, 0xf>(pre);
  return StatD{M, sum, pre};
}

// The match-mode scan of one sampled sequence with a valid draft count (greedy and
// invalid-count sequences take the rejection-rule scan, which treats them identically).  Same
// layout and outputs as accept_sequence.
__device__ __forceinline__ ScanOut accept_sequence_match(const ScanIn& in, int kb, float T,
                                                         float c, int K, int V,
                                                         const StatD* sh_rows, int lane,
                                                         bool pending = false) {
  const Gather g = in.g;
  const float u = in.u, uk = in.uk;
  const bool seq_ok = temp_valid(T);  // T != 0 and k_b in range here
  const StatD st = lane <= K ? sh_rows[lane] : StatD{-INFINITY, 0.0, 0.0};

  const bool drafted = lane < kb;
  const int x = g.x;
  bool lane_ok = true, keep = true;
  double ex = 0.0;
  if (lane <= kb) {
    lane_ok = (pending && lane == kb) || st.s > 0.0;  // NaN / +inf logit -> NaN; all -inf -> 0
    if (drafted) {
      if (!(x >= 0 && x < V) || !(u >= 0.f && u < 1.f)) {
        lane_ok = false;
      } else {
        // y_i == x_i  <=>  P_i <= u * S_i < P_i + e(x_i)
        ex = exp2((static_cast<double>(g.z) - static_cast<double>(st.m)) *
                  static_cast<double>(c));
        const double t = static_cast<double>(u) * st.s;
        keep = st.p <= t && t < st.p + ex;
      }
    }
  }
  if (lane == 0 && !(uk >= 0.f && uk < 1.f)) lane_ok = false;
  const bool ok = seq_ok && (__ballot(!lane_ok) == 0ull);
  const unsigned long long rej = __ballot(lane < kb && !keep);
  const int A = ok ? (rej ? __ffsll(static_cast<long long>(rej)) - 1 : kb) : -1;

  SeqState out{kNone, 0, 0, 0, 0.f, 0.f, 0.f, 0.f};
  if (ok)  // a plain draw of p_A with u[b, A] (mismatch) or u[b, K] (bonus)
    out = SeqState{kBonus, A, -1, A < kb ? A : K, c, read_lane_f(st.m, A),
                   static_cast<float>(read_lane_d(st.s, A)), 0.f};
  const bool kept = ok && lane < A;                  // slot A is filled by the draw
  return ScanOut{out, A, kept ? x : -1, kept ? ex : 0.0, kept ? st.s : 1.0};
}

// ------------------------------------------------------------------------------------------
// Inverse-CDF draw ("Decodificação especulativa explicada", section "Amostragem especulativa em
// numpy, com prova": the first running sum above u times the total, over ascending token id),
// from per-segment weight sums: one fp64 DPP scan over the segment sums finds the segment holding
// u * total (plain p when the draw's total is not positive), then a workgroup scan of that one
// segment finds the token.
// ------------------------------------------------------------------------------------------
struct PickLds {
  int seg, plain, flag, hit[kWaves], lastpos[kWaves];
  float zhit[kWaves], zlast[kWaves];
  double t, base, wtot[kWaves];
};

// First step, in wave 0: lane l holds the sums (lw: the draw's weights; le: those of p) of its
// segments [l * P, l * P + P); seg_at(j, plain) gives segment j's sum again (not called when
// each lane has one segment).  Leaves the segment,
// the target u * total and the running sum before the segment in ps.  Returns false (in every
// lane) when the weights' total is NaN -- a draft row holding a value that is not a probability
// -- and the sequence is to be reported invalid.
template <typename SegAt>
__device__ __forceinline__ bool find_draw_segment(double lw, double le, float u, int nseg, int P,
                                                  SegAt seg_at, PickLds& ps, int lane) {
  const int j0 = lane * P;
  const double iw = wave_inclusive_scan(lw), ie = wave_inclusive_scan(le);
  const double total_w = read_lane_d(iw, 63);
  if (total_w != total_w) return false;
  const bool plain = !(total_w > 0.0);  // empty residual: draw from p itself
  const double inc = plain ? ie : iw;
  const double own = plain ? le : lw;
  const double R = read_lane_d(inc, 63);
  const double t = static_cast<double>(u) * R;
  // The first lane whose running total passes t holds the segment; if rounding left t at the
  // very top, the last lane with positive weight does.
  const unsigned long long hit = __ballot(own > 0.0 && inc > t);
  const unsigned long long pos = __ballot(own > 0.0);
  const int hl = hit ? __ffsll(static_cast<long long>(hit)) - 1
                     : (pos ? 63 - __clzll(static_cast<long long>(pos)) : 0);
  if (lane == hl) {
    double run = inc - own;  // running sum before the lane's segments
    int seg = -1, lastpos = -1;
    double base_seg = 0.0, base_last = 0.0;
    for (int q = 0; q < P && j0 + q < nseg; ++q) {
      // A lane with one segment holds its sum already (own = 0 + that sum, exactly).
      const double v = P == 1 ? own : seg_at(j0 + q, plain);
      if (v > 0.0) {
        if (run + v > t) { seg = j0 + q; base_seg = run; break; }
        lastpos = j0 + q;
        base_last = run;
      }
      run += v;
    }
    if (seg < 0) { seg = lastpos >= 0 ? lastpos : j0; base_seg = base_last; }
    ps.seg = seg; ps.plain = plain; ps.t = t; ps.base = base_seg;
  }
  return true;
}

// ------------------------------------------------------------------------------------------
// Draw weights of one token and of groups of tokens.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float draw_weight(float z, float q, int v, const SeqState& st,
                                             bool plain, float& e_out) {
  const float e = __builtin_amdgcn_exp2f((z - st.m) * st.c);
  e_out = e;
  if (plain || st.mode == kBonus) return e;
  if (st.mode == kResidualOnehot) return v == st.excl ? 0.f : e;
  // A draft probability that is negative, infinite or NaN makes the weight NaN, so the draw's
  // total is NaN and the pick reports the sequence invalid.
  const float w = fmaxf(0.f, fmaf(-st.s, q, e));  // s * max(0, p - q)
  return (q >= 0.f && q <= __FLT_MAX__) ? w : __builtin_nanf("");
}

// Loads of the kGroup tokens [v0, v0 + cnt) (cnt <= 0: none); -inf / 0 past cnt.  The vector
// path loads unconditionally -- from `any`, a valid 16-byte-aligned stand-in of at least 32
// bytes, when there is nothing to read -- and then selects, so the target and draft loads are
// in flight together.
template <typename LT, bool kVec>
__device__ __forceinline__ void load_group(const LT* __restrict__ z, const float* __restrict__ q,
                                           const void* any, int v0, int cnt,
                                           float (&zv)[kGroup], float (&qv)[kGroup]) {
  if constexpr (kVec) {  // cnt is kGroup or <= 0; 16-byte aligned
    const bool in = cnt > 0, inq = in && q != nullptr;
    const LT* zp = in ? z + v0 : static_cast<const LT*>(any);
    const float* qp = inq ? q + v0 : static_cast<const float*>(any);
    const uint4 z0 = stream_load(zp);
    uint4 z1 = make_uint4(0, 0, 0, 0);
    if constexpr (sizeof(LT) == 4) z1 = stream_load(zp + 4);
    const uint4 q0 = stream_load(qp), q1 = stream_load(qp + 4);
    unpack(z0, zv, static_cast<const LT*>(nullptr));
    if constexpr (sizeof(LT) == 4) unpack(z1, zv + 4, static_cast<const LT*>(nullptr));
    unpack(q0, qv, static_cast<const float*>(nullptr));
    unpack(q1, qv + 4, static_cast<const float*>(nullptr));
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (!in) zv[j] = -INFINITY;
      if (!inq) qv[j] = 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      zv[j] = j < cnt ? load_logit(z, v0 + j) : -INFINITY;
      qv[j] = (q != nullptr && j < cnt) ? q[v0 + j] : 0.f;
    }
  }
}

// Weights of one group and their sums (sequential in token order, fp32).
__device__ __forceinline__ void group_weights(const float (&zv)[kGroup], const float (&qv)[kGroup],
                                              int v0, int cnt, const SeqState& st, bool plain,
                                              float (&w)[kGroup], float& gw, float& ge) {
  gw = 0.f;
  ge = 0.f;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    float e = 0.f;
    w[j] = j < cnt ? draw_weight(zv[j], qv[j], v0 + j, st, plain, e) : 0.f;
    if (j >= cnt) e = 0.f;
    gw += w[j];
    ge += e;
  }
}


// Four consecutive logits as one cached load: 8 bytes of bf16 or 16 bytes of fp32.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <typename LT> struct DrawVec;
template <> struct DrawVec<uint16_t> {
  uint2 d;
  static __device__ __forceinline__ DrawVec load(const uint16_t* p) {
    const u32x2 t = *reinterpret_cast<const u32x2*>(p);
    return DrawVec{make_uint2(t.x, t.y)};
  }
  static __device__ __forceinline__ DrawVec zero() { return DrawVec{make_uint2(0, 0)}; }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = __uint_as_float(d.x << 16); o[1] = __uint_as_float(d.x & 0xffff0000u);
    o[2] = __uint_as_float(d.y << 16); o[3] = __uint_as_float(d.y & 0xffff0000u);
  }
};
template <> struct DrawVec<float> {
  uint4 d;
  static __device__ __forceinline__ DrawVec load(const float* p) { return DrawVec{plain_load(p)}; }
  static __device__ __forceinline__ DrawVec zero() { return DrawVec{make_uint4(0, 0, 0, 0)}; }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = __uint_as_float(d.x); o[1] = __uint_as_float(d.y);
    o[2] = __uint_as_float(d.z); o[3] = __uint_as_float(d.w);
  }
};

// Hand-off words.  A value one workgroup hands to another inside a launch travels in a 64-bit word
// whose upper half is kMark: the producer issues a coherent store and goes on, the consumer polls
// (bounded) until every word it needs carries the mark.  A 64-bit store is single-copy atomic, so
// a marked word never pairs a new mark with stale data.  Whoever consumes the words puts them back
// to zero (or a kernel that runs before the producers does).
typedef unsigned long long u64;
constexpr uint32_t kMark = 0x5ec0da7au;

__device__ __forceinline__ u64 marked(uint32_t v) { return (static_cast<u64>(kMark) << 32) | v; }
__device__ __forceinline__ bool is_marked(u64 w) { return static_cast<uint32_t>(w >> 32) == kMark; }
__device__ __forceinline__ uint32_t bits_of(u64 w) { return static_cast<uint32_t>(w); }
__device__ __forceinline__ u64 load_word(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_word(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace specdec
