// gfx950 (CDNA4) kernels of the batched speculative-decoding verify step.
//
// The step (draft-then-verify with rejection sampling) is the one the three source pages
// define: "Decodificação especulativa explicada" (gsantana.dev), section "A regra de
// amostragem por rejeição"; "ch15 · Speculative Decoding" (snowch.github.io), section "Why
// the result is exactly the target model"; "Speculative decoding: el secretario que adelanta
// lo que va a decir el jefe" (blog.lo0.es), section "El mecanismo desnudo".
//
// Four kernels, enqueued back to back on the caller's stream:
//   1. row_stats     streams every used target logit row once (the HBM-bound pass) and
//                    writes, per (row, 8192-logit chunk), the chunk max m, the sum of
//                    exp2((z - m) * log2(e)/T) and, for greedy rows, the lowest argmax.
//   2. accept        one wave64 per sequence: merges the chunk partials of its rows in chunk
//                    order, gathers p_i(x_i) (fp64) and q_i(x_i), runs the accept tests as one
//                    64-bit ballot, finds the first rejection and emits every token whose value
//                    is already known (accepted drafts, greedy argmaxes).
//   3. sample_sums   for each sequence that still needs a draw, the sum of the draw's weights
//                    (residual max(0, p - q), p without x, or p) per chunk of its one row.
//   4. sample_pick   one workgroup per sequence: picks the chunk holding u * total from the
//                    chunk sums, then scans that chunk in ascending token order (per-thread
//                    8-token groups, fp64 workgroup prefix scan) to the first running sum
//                    above u * total.
// All reductions combine in a fixed order, so results are bit-reproducible; no atomics.
#include <float.h>
#include <limits.h>
#include <math.h>

#include "kernels.h"

namespace specdec {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kTempMin = 1e-6f;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ bool temp_valid(float T) {
  return T == 0.f || (T >= kTempMin && T <= FLT_MAX);
}
// exp2 scale: log2(e)/T for sampled rows, log2(e) (softmax at T = 1) for greedy rows.
__device__ __forceinline__ float temp_scale(float T) { return T == 0.f ? kLog2e : kLog2e / T; }

__device__ __forceinline__ float load_logit(const uint16_t* p, long long i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float load_logit(const float* p, long long i) { return p[i]; }

// 16-byte vector -> floats.
__device__ __forceinline__ void unpack(const uint4& d, float (&o)[8], const uint16_t*) {
  o[0] = __uint_as_float(d.x << 16); o[1] = __uint_as_float(d.x & 0xffff0000u);
  o[2] = __uint_as_float(d.y << 16); o[3] = __uint_as_float(d.y & 0xffff0000u);
  o[4] = __uint_as_float(d.z << 16); o[5] = __uint_as_float(d.z & 0xffff0000u);
  o[6] = __uint_as_float(d.w << 16); o[7] = __uint_as_float(d.w & 0xffff0000u);
}
__device__ __forceinline__ void unpack(const uint4& d, float (&o)[4], const float*) {
  o[0] = __uint_as_float(d.x); o[1] = __uint_as_float(d.y);
  o[2] = __uint_as_float(d.z); o[3] = __uint_as_float(d.w);
}
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

__device__ __forceinline__ Stat merge(const Stat& x, const Stat& y, float c) {
  Stat r;
  r.m = fmaxf(x.m, y.m);
  if (r.m == -INFINITY) {  // both empty (or all -inf): sums are 0 (NaN stays NaN)
    r.s = x.s + y.s;
    r.a = min(x.a, y.a);
    return r;
  }
  r.s = x.s * exp2f((x.m - r.m) * c) + y.s * exp2f((y.m - r.m) * c);
  r.a = (y.m > x.m || (y.m == x.m && y.a < x.a)) ? y.a : x.a;
  return r;
}

// Fold a block of logits (in ascending index order) into the running statistics.  `idx(j)`
// gives the token index of element j; it is only evaluated for greedy rows.
template <int N, typename IdxFn>
__device__ __forceinline__ void fold_block(const float (&x)[N], float c, bool want_arg, Stat& st,
                                           IdxFn idx) {
  float bm = x[0];
#pragma unroll
  for (int j = 1; j < N; ++j) bm = fmaxf(bm, x[j]);
  if (bm > st.m) {  // strictly greater keeps the earlier (lower-index) maximum
    st.s *= exp2f((st.m - bm) * c);
    if (want_arg) {
      int a = INT_MAX;
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
        if (x[j] == bm) a = idx(j);
      st.a = a;
    }
    st.m = bm;
  }
  // A history of only -inf (or NaN) keeps the reference at 0 so -inf maps to exp2(-inf) = 0.
  const float ref = (st.m == -INFINITY) ? 0.f : st.m;
#pragma unroll
  for (int j = 0; j < N; ++j) st.s += __builtin_amdgcn_exp2f((x[j] - ref) * c);
}

__device__ __forceinline__ Stat wave_reduce(Stat v, float c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Stat o;
    o.m = __shfl_xor(v.m, off, 64);
    o.s = __shfl_xor(v.s, off, 64);
    o.a = __shfl_xor(v.a, off, 64);
    v = merge(v, o, c);
  }
  return v;
}

// ------------------------------------------------------------------------------------------
// 1. Streaming row statistics.
// ------------------------------------------------------------------------------------------
template <typename LT, bool kVec>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(
    const LT* __restrict__ logits, const int32_t* __restrict__ num_draft,
    const float* __restrict__ temperature, int B, int K, int V, int S, int greedy_all,
    RowPartial* __restrict__ partials) {
  __shared__ Stat red[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long total = static_cast<long long>(B) * (K + 1) * S;
  for (long long w = blockIdx.x; w < total; w += gridDim.x) {
    const int s = static_cast<int>(w % S);
    const long long r = w / S;
    const int b = static_cast<int>(r / (K + 1)), i = static_cast<int>(r % (K + 1));
    const int kb = num_draft ? num_draft[b] : K;
    const float T = greedy_all ? 0.f : temperature[b];
    if (kb < 0 || kb > K || i > kb || !temp_valid(T)) continue;  // padded or invalid: unread
    const bool want_arg = (T == 0.f);
    const float c = temp_scale(T);
    const LT* row = logits + r * static_cast<long long>(V);
    const int c0 = s * kChunk;
    const int n = min(kChunk, V - c0);
    Stat st{-INFINITY, 0.f, INT_MAX};
    if constexpr (kVec) {
      constexpr int P = Vec<LT>::kPer;
      constexpr int U = 4;  // 16-byte loads in flight per thread
      const uint4* vrow = reinterpret_cast<const uint4*>(row + c0);
      const int nvec = n / P;
      for (int v0 = 0; v0 < nvec; v0 += U * kThreads) {
        uint4 d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int vi = v0 + u * kThreads + tid;
          constexpr uint32_t ni = Vec<LT>::kNegInf;
          d[u] = vi < nvec ? vrow[vi] : make_uint4(ni, ni, ni, ni);
        }
        float x[U * P];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float t[P];
          unpack(d[u], t, static_cast<const LT*>(nullptr));
#pragma unroll
          for (int e = 0; e < P; ++e) x[u * P + e] = t[e];
        }
        fold_block(x, c, want_arg, st, [&](int j) {
          return c0 + (v0 + (j / P) * kThreads + tid) * P + (j % P);
        });
      }
    } else {
      constexpr int U = 8;
      for (int v0 = 0; v0 < n; v0 += U * kThreads) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int vi = v0 + u * kThreads + tid;
          x[u] = vi < n ? load_logit(row, c0 + vi) : -INFINITY;
        }
        fold_block(x, c, want_arg, st, [&](int j) { return c0 + v0 + j * kThreads + tid; });
      }
    }
    st = wave_reduce(st, c);
    if (lane == 0) red[wave] = st;
    __syncthreads();
    if (tid == 0) {
      Stat acc = red[0];
#pragma unroll
      for (int k = 1; k < kWaves; ++k) acc = merge(acc, red[k], c);
      partials[w] = RowPartial{acc.m, acc.s, acc.a, 0};
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// 2. Accept scan: one wave64 per sequence, lane i <-> target row i.
// ------------------------------------------------------------------------------------------
template <typename LT>
__global__ __launch_bounds__(64) void accept_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const uint8_t* __restrict__ onehot, const int32_t* __restrict__ proposed,
    const int32_t* __restrict__ num_draft, const float* __restrict__ temperature,
    const float* __restrict__ uniforms, int B, int K, int V, int S, int greedy_all,
    const RowPartial* __restrict__ partials, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_tokens, float* __restrict__ out_probs,
    SeqState* __restrict__ states) {
  const int lane = threadIdx.x;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const int kb = num_draft ? num_draft[b] : K;
    const float T = greedy_all ? 0.f : temperature[b];
    const bool greedy = (T == 0.f);
    bool ok = kb >= 0 && kb <= K && temp_valid(T);
    const bool is_onehot = ok && !greedy && onehot != nullptr && onehot[b] != 0;
    const float c = temp_scale(T);
    const long long row0 = static_cast<long long>(b) * (K + 1);

    // Row statistics of row `lane` (merged over chunks in chunk order).
    Stat st{-INFINITY, 0.f, INT_MAX};
    bool lane_ok = true;
    int x = -1;
    double px = 0.0;
    bool acc = true;
    if (ok && lane <= kb) {
      const RowPartial* P = partials + (row0 + lane) * S;
      st = Stat{P[0].m, P[0].s, P[0].arg};
      for (int j = 1; j < S; ++j) st = merge(st, Stat{P[j].m, P[j].s, P[j].arg}, c);
      lane_ok = st.s > 0.f;  // NaN / +inf logit -> NaN; all -inf -> 0
      if (lane < kb) {
        x = proposed[static_cast<long long>(b) * K + lane];
        if (x < 0 || x >= V) {
          lane_ok = false;
        } else {
          const double zx = load_logit(logits, (row0 + lane) * V + x);
          px = exp2((zx - static_cast<double>(st.m)) * static_cast<double>(c)) /
               static_cast<double>(st.s);
          if (greedy) {
            acc = (x == st.a);
          } else {
            const float u = uniforms[row0 + lane];
            if (!(u >= 0.f && u < 1.f)) lane_ok = false;
            double qx = 1.0;  // one-hot drafter: q(x) = 1
            if (!is_onehot) {
              if (draft_probs == nullptr) {
                lane_ok = false;
              } else {
                const float qf = draft_probs[(static_cast<long long>(b) * K + lane) * V + x];
                if (!(qf >= 0.f && qf <= FLT_MAX)) lane_ok = false;
                qx = qf;
              }
            }
            acc = static_cast<double>(u) * qx < px;
          }
        }
      }
    }
    if (ok && !greedy && lane == 0) {
      const float uk = uniforms[row0 + K];
      if (!(uk >= 0.f && uk < 1.f)) lane_ok = false;
    }
    ok = ok && (__ballot(!lane_ok) == 0ull);
    const unsigned long long rej = __ballot(lane < kb && !acc);
    const int A = ok ? (rej ? __ffsll(static_cast<long long>(rej)) - 1 : kb) : -1;

    if (lane <= K) {
      int tok = -1;
      float prob = 0.f;
      if (ok && lane < A) {
        tok = x;
        prob = static_cast<float>(px);
      } else if (ok && lane == A && greedy) {
        tok = st.a;                                    // argmax: exp2(0) / s
        prob = static_cast<float>(1.0 / static_cast<double>(st.s));
      }
      out_tokens[row0 + lane] = tok;                   // the sampled slot is filled later
      if (out_probs) out_probs[row0 + lane] = prob;
    }
    if (lane == 0) accept_len[b] = A;
    if ((!ok || greedy) && lane == 0) states[b] = SeqState{kNone, 0, 0, 0, 0.f, 0.f, 0.f, 0.f};
    if (ok && !greedy && lane == A) {
      const int mode = (A == kb) ? kBonus : (is_onehot ? kResidualOnehot : kResidual);
      states[b] = SeqState{mode, A, x, 0, c, st.m, st.s, 0.f};
    }
  }
}

// ------------------------------------------------------------------------------------------
// 3./4. Sampling passes.  Both compute a token's weight with the same code, so the chunk sums
// of pass 3 and the scan of pass 4 see identical values.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float draw_weight(float z, float q, int v, const SeqState& st,
                                             bool plain, float* e_out) {
  const float e = __builtin_amdgcn_exp2f((z - st.m) * st.c);
  *e_out = e;
  if (plain || st.mode == kBonus) return e;
  if (st.mode == kResidualOnehot) return v == st.excl ? 0.f : e;
  return fmaxf(0.f, fmaf(-st.s, q, e));  // s * max(0, p - q)
}

// Weights of the kGroup tokens [v0, v0 + cnt) (zeros past cnt).
template <typename LT, bool kVec>
__device__ __forceinline__ void load_group(const LT* __restrict__ z, const float* __restrict__ q,
                                           int v0, int cnt, const SeqState& st, bool plain,
                                           float (&w)[kGroup], float (&e)[kGroup]) {
  float zv[kGroup], qv[kGroup];
  if constexpr (kVec) {  // cnt == kGroup, 16-byte aligned
    if constexpr (sizeof(LT) == 2) {
      float t[8];
      unpack(*reinterpret_cast<const uint4*>(z + v0), t, static_cast<const LT*>(nullptr));
#pragma unroll
      for (int j = 0; j < 8; ++j) zv[j] = t[j];
    } else {
      float t0[4], t1[4];
      unpack(*reinterpret_cast<const uint4*>(z + v0), t0, static_cast<const LT*>(nullptr));
      unpack(*reinterpret_cast<const uint4*>(z + v0 + 4), t1, static_cast<const LT*>(nullptr));
#pragma unroll
      for (int j = 0; j < 4; ++j) { zv[j] = t0[j]; zv[4 + j] = t1[j]; }
    }
    if (q != nullptr) {
      float t0[4], t1[4];
      unpack(*reinterpret_cast<const uint4*>(q + v0), t0, static_cast<const float*>(nullptr));
      unpack(*reinterpret_cast<const uint4*>(q + v0 + 4), t1, static_cast<const float*>(nullptr));
#pragma unroll
      for (int j = 0; j < 4; ++j) { qv[j] = t0[j]; qv[4 + j] = t1[j]; }
    } else {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) qv[j] = 0.f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      zv[j] = j < cnt ? load_logit(z, v0 + j) : -INFINITY;
      qv[j] = (q != nullptr && j < cnt) ? q[v0 + j] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    if (j < cnt) {
      w[j] = draw_weight(zv[j], qv[j], v0 + j, st, plain, &e[j]);
    } else {
      w[j] = 0.f;
      e[j] = 0.f;
    }
  }
}

template <typename LT, bool kVec>
__global__ __launch_bounds__(kThreads) void sample_sums_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs, int B, int K, int V,
    int S, const SeqState* __restrict__ states, ChunkSums* __restrict__ sums) {
  __shared__ double redw[kWaves], rede[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long total = static_cast<long long>(B) * S;
  for (long long wi = blockIdx.x; wi < total; wi += gridDim.x) {
    const int b = static_cast<int>(wi / S), s = static_cast<int>(wi % S);
    const SeqState st = states[b];
    if (st.mode == kNone) continue;
    const long long row = static_cast<long long>(b) * (K + 1) + st.row;
    const LT* z = logits + row * V;
    const float* q = st.mode == kResidual
                         ? draft_probs + (static_cast<long long>(b) * K + st.row) * V
                         : nullptr;
    const int c0 = s * kChunk, n = min(kChunk, V - c0);
    const int ngroups = (n + kGroup - 1) / kGroup;
    double tw = 0.0, te = 0.0;
    for (int g = tid; g < ngroups; g += kThreads) {
      float w[kGroup], e[kGroup];
      load_group<LT, kVec>(z, q, c0 + g * kGroup, min(kGroup, n - g * kGroup), st, false, w, e);
      float gw = 0.f, ge = 0.f;
#pragma unroll
      for (int j = 0; j < kGroup; ++j) { gw += w[j]; ge += e[j]; }
      tw += gw;
      te += ge;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      tw += __shfl_xor(tw, off, 64);
      te += __shfl_xor(te, off, 64);
    }
    if (lane == 0) { redw[wave] = tw; rede[wave] = te; }
    __syncthreads();
    if (tid == 0) {
      double a = redw[0], c = rede[0];
#pragma unroll
      for (int k = 1; k < kWaves; ++k) { a += redw[k]; c += rede[k]; }
      sums[wi] = ChunkSums{a, c};
    }
    __syncthreads();
  }
}

template <typename LT, bool kVec>
__global__ __launch_bounds__(kThreads) void sample_pick_kernel(
    const LT* __restrict__ logits, const float* __restrict__ draft_probs,
    const float* __restrict__ uniforms, int B, int K, int V, int S,
    const SeqState* __restrict__ states, const ChunkSums* __restrict__ sums,
    int32_t* __restrict__ out_tokens, float* __restrict__ out_probs) {
  __shared__ double sh_t, sh_base;
  __shared__ int sh_chunk, sh_plain, sh_last;
  __shared__ double wtot[kWaves];
  __shared__ int wfound[kWaves], wlast[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const SeqState st = states[b];
    if (st.mode == kNone) continue;
    const long long row0 = static_cast<long long>(b) * (K + 1);
    if (tid == 0) {
      // Chunk totals in chunk order (fp64); an empty residual falls back to p itself.
      const ChunkSums* cs = sums + static_cast<long long>(b) * S;
      double R = 0.0;
      for (int s = 0; s < S; ++s) R += cs[s].w;
      const int plain = !(R > 0.0);
      if (plain) {
        R = 0.0;
        for (int s = 0; s < S; ++s) R += cs[s].e;
      }
      const double t = static_cast<double>(uniforms[row0 + K]) * R;
      double base = 0.0, base_last = 0.0;
      int chunk = -1, last = -1;
      for (int s = 0; s < S; ++s) {
        const double ws = plain ? cs[s].e : cs[s].w;
        if (ws > 0.0) {
          if (base + ws > t) { chunk = s; break; }
          last = s;
          base_last = base;
        }
        base += ws;
      }
      if (chunk < 0) { chunk = last; base = base_last; }
      if (chunk < 0) { chunk = 0; base = 0.0; }  // no positive chunk sum (cannot happen for a valid row)
      sh_t = t;
      sh_base = base;
      sh_chunk = chunk;
      sh_plain = plain;
    }
    __syncthreads();
    const double t = sh_t;
    const bool plain = sh_plain != 0;
    const int chunk = sh_chunk;
    const long long row = row0 + st.row;
    const LT* z = logits + row * V;
    const float* q = (st.mode == kResidual && !plain)
                         ? draft_probs + (static_cast<long long>(b) * K + st.row) * V
                         : nullptr;
    const int c0 = chunk * kChunk, n = min(kChunk, V - c0);
    const int ngroups = (n + kGroup - 1) / kGroup;
    double base = sh_base;
    int result = -1, last_pos = -1;
    for (int g0 = 0; g0 < ngroups; g0 += kThreads) {
      const int g = g0 + tid;
      float w[kGroup], e[kGroup];
      float gsum = 0.f;
      if (g < ngroups) {
        load_group<LT, kVec>(z, q, c0 + g * kGroup, min(kGroup, n - g * kGroup), st, plain, w, e);
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          gsum += w[j];
          if (w[j] > 0.f) last_pos = c0 + g * kGroup + j;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j) w[j] = 0.f;
      }
      // Inclusive scan of the group sums over the workgroup (fp64, ascending thread order).
      double inc = gsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(inc, off, 64);
        if (lane >= off) inc = y + inc;
      }
      double exc = __shfl_up(inc, 1, 64);
      if (lane == 0) exc = 0.0;
      if (lane == 63) wtot[wave] = inc;
      __syncthreads();
      double before = base;
      for (int k = 0; k < wave; ++k) before += wtot[k];
      before += exc;
      // First token of this group whose running sum exceeds t.
      int hit = -1;
      if (g < ngroups) {
        float run = 0.f;
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
          run += w[j];
          if (hit < 0 && w[j] > 0.f && before + static_cast<double>(run) > t)
            hit = c0 + g * kGroup + j;
        }
      }
      // Lowest hit in the workgroup.
      const unsigned long long hm = __ballot(hit >= 0);
      const int wl = hm ? __shfl(hit, __ffsll(static_cast<long long>(hm)) - 1, 64) : -1;
      if (lane == 0) wfound[wave] = wl;
      __syncthreads();
      int found = -1;
      for (int k = 0; k < kWaves; ++k)
        if (found < 0 && wfound[k] >= 0) found = wfound[k];
      double iter_total = 0.0;
      for (int k = 0; k < kWaves; ++k) iter_total += wtot[k];
      __syncthreads();
      if (found >= 0) { result = found; break; }
      base += iter_total;
    }
    if (result < 0) {
      // Rounding left u * total at the very top of the chunk: take its last positive token.
      int lp = last_pos;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) lp = max(lp, __shfl_xor(lp, off, 64));
      if (lane == 0) wlast[wave] = lp;
      __syncthreads();
      if (tid == 0) {
        int m = -1;
        for (int k = 0; k < kWaves; ++k) m = max(m, wlast[k]);
        sh_last = m;
      }
      __syncthreads();
      result = sh_last >= 0 ? sh_last : c0;
    }
    if (tid == 0) {
      const double zy = load_logit(z, result);
      const double p = exp2((zy - static_cast<double>(st.m)) * static_cast<double>(st.c)) /
                       static_cast<double>(st.s);
      out_tokens[row0 + st.row] = result;
      if (out_probs) out_probs[row0 + st.row] = static_cast<float>(p);
    }
    __syncthreads();
  }
}

constexpr long long kMaxGrid = 1 << 20;

inline unsigned grid_for(long long work) {
  return static_cast<unsigned>(work < 1 ? 1 : (work < kMaxGrid ? work : kMaxGrid));
}

template <typename LT>
hipError_t launch_typed(const LaunchArgs& a) {
  const LT* logits = static_cast<const LT*>(a.logits);
  const int S = num_chunks(a.V);
  const bool vec_stats = (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0) &&
                         ((static_cast<long long>(a.V) * sizeof(LT)) % 16 == 0);
  const bool vec_sample = vec_stats && (a.V % kGroup == 0) &&
                          (a.draft_probs == nullptr ||
                           reinterpret_cast<uintptr_t>(a.draft_probs) % 16 == 0);
  const long long rows = static_cast<long long>(a.B) * (a.K + 1);
  hipError_t err;
  if (a.hot_begin && (err = hipEventRecord(a.hot_begin, a.stream)) != hipSuccess) return err;
  if (vec_stats)
    row_stats_kernel<LT, true><<<grid_for(rows * S), kThreads, 0, a.stream>>>(
        logits, a.num_draft, a.temperature, a.B, a.K, a.V, S, a.greedy_all, a.ws.partials);
  else
    row_stats_kernel<LT, false><<<grid_for(rows * S), kThreads, 0, a.stream>>>(
        logits, a.num_draft, a.temperature, a.B, a.K, a.V, S, a.greedy_all, a.ws.partials);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.hot_end && (err = hipEventRecord(a.hot_end, a.stream)) != hipSuccess) return err;
  accept_kernel<LT><<<grid_for(a.B), 64, 0, a.stream>>>(
      logits, a.draft_probs, a.onehot, a.proposed, a.num_draft, a.temperature, a.uniforms, a.B,
      a.K, a.V, S, a.greedy_all, a.ws.partials, a.accept_len, a.out_tokens, a.out_probs,
      a.ws.states);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.greedy_all) return hipSuccess;
  if (vec_sample) {
    sample_sums_kernel<LT, true><<<grid_for(static_cast<long long>(a.B) * S), kThreads, 0,
                                  a.stream>>>(logits, a.draft_probs, a.B, a.K, a.V, S,
                                              a.ws.states, a.ws.sums);
    sample_pick_kernel<LT, true><<<grid_for(a.B), kThreads, 0, a.stream>>>(
        logits, a.draft_probs, a.uniforms, a.B, a.K, a.V, S, a.ws.states, a.ws.sums,
        a.out_tokens, a.out_probs);
  } else {
    sample_sums_kernel<LT, false><<<grid_for(static_cast<long long>(a.B) * S), kThreads, 0,
                                   a.stream>>>(logits, a.draft_probs, a.B, a.K, a.V, S,
                                               a.ws.states, a.ws.sums);
    sample_pick_kernel<LT, false><<<grid_for(a.B), kThreads, 0, a.stream>>>(
        logits, a.draft_probs, a.uniforms, a.B, a.K, a.V, S, a.ws.states, a.ws.sums,
        a.out_tokens, a.out_probs);
  }
  return hipGetLastError();
}

}  // namespace

size_t workspace_layout(int B, int K, int V, size_t* off_partials, size_t* off_states,
                        size_t* off_sums) {
  auto align16 = [](size_t x) { return (x + 15) & ~static_cast<size_t>(15); };
  const size_t S = static_cast<size_t>(num_chunks(V));
  const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(K + 1);
  size_t off = 0;
  *off_partials = off;
  off = align16(off + rows * S * sizeof(RowPartial));
  *off_states = off;
  off = align16(off + static_cast<size_t>(B) * sizeof(SeqState));
  *off_sums = off;
  off = align16(off + static_cast<size_t>(B) * S * sizeof(ChunkSums));
  return off;
}

hipError_t launch_verify(const LaunchArgs& a) {
  return a.logits_bf16 ? launch_typed<uint16_t>(a) : launch_typed<float>(a);
}

}  // namespace specdec
