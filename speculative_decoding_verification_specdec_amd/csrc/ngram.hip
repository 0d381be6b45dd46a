// gfx950 kernels of the n-gram (prompt-lookup) drafter.
//
// The drafter is the model-free one the pages describe: find where the most recent tokens of
// the sequence appeared earlier in it and propose what followed there ("Decodificação
// especulativa explicada", gsantana.dev, section "A família de rascunhos", prompt lookup; "ch15 ·
// Speculative Decoding", snowch.github.io, section "What proposes the tokens"; longest match
// first after the longest-prefix match in "Speculative decoding: el secretario...",
// blog.lo0.es, section "Las cinco familias modernas").
//
// For history h[0..L) and a follower position e in [1, L-1], let m(e) be the length of the
// longest common run h[e-j] == h[L-j], j = 1, 2, ..., capped at min(n_max, e).  The n-token
// suffix occurs at p = e - n (with at least one follower) iff m(e) >= n, so the longest suffix
// that occurs is N = max_e m(e) and its earliest occurrence ends at the smallest e with
// m(e) = N.  Both fall out of one max-reduction of the key (m(e) << 32) | (2^32 - 1 - e).
//
// No atomics, one launch whenever the rows allow 16-byte loads.  When one 8192-position tile
// covers the history capacity, ngram_match_kernel runs one 512-thread workgroup per sequence: the
// tile and a 32-token halo are staged in LDS with 16-byte loads (33 KB: four workgroups fit a CU);
// each thread first tests its 16 positions (consecutive threads on consecutive positions) for
// h[e-1] == h[L-1] with independent LDS reads, then extends only those candidates, and the
// workgroup max-reduces the keys and emits the proposal straight from LDS.  Longer histories with
// 16-byte rows take ngram_history_kernel, one 1024-thread workgroup per sequence walking the
// whole history (below).  Rows that allow only 4-byte loads keep the tiled kernel with one
// workgroup per (tile, sequence): each tile writes its key and ngram_emit_kernel (one wave per
// sequence) takes the max over tiles and copies the proposal.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace specdec {
namespace {

constexpr int kNgThreads = 512;
constexpr int kNgPer = kNgramTile / kNgThreads;  // 16 positions per thread
constexpr int kNgHalo = kNgramMaxN;              // tokens staged before the tile
constexpr int kEmitThreads = 256;                // 4 sequences per emit workgroup

__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned lo = __shfl_xor(static_cast<unsigned>(v), off, 64);
    const unsigned hi = __shfl_xor(static_cast<unsigned>(v >> 32), off, 64);
    v = max_u64(v, (static_cast<unsigned long long>(hi) << 32) | lo);
  }
  return v;
}

// The proposal for key `key` (0: none) of a valid history of length L, written by one wave:
// proposed[lane] = h[e + lane] for lane < cnt, else -1.
__device__ __forceinline__ int proposal_count(unsigned long long key, int L, int K, int& e) {
  if (key == 0ull) return 0;
  e = static_cast<int>(0xffffffffull - (key & 0xffffffffull));
  return min(K, L - e);
}

template <bool kVec>
__global__ __launch_bounds__(kNgThreads) void ngram_match_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ lengths, int capacity,
    int n_min, int n_max, int K, int ntiles, unsigned long long* __restrict__ partials,
    int32_t* __restrict__ proposed, int32_t* __restrict__ num_draft) {
  __shared__ __align__(16) int sh_tok[kNgHalo + kNgramTile];  // sh_tok[i] = h[t0 - kNgHalo + i]
  __shared__ int sh_suf[kNgramMaxN + 1];        // sh_suf[j] = h[L - j]
  __shared__ unsigned long long sh_best[kNgThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = static_cast<int>(blockIdx.x / ntiles), tile = static_cast<int>(blockIdx.x % ntiles);
  const int L = lengths[b];
  const int t0 = tile * kNgramTile;
  const bool valid = L >= 0 && L <= capacity;
  const int nmax = min(n_max, L - 1);
  // Nothing to match for an invalid length, a history too short for n_min, or a tile with no
  // follower position (e in [1, L-1]); the condition is uniform over the workgroup.
  const bool active = valid && nmax >= n_min && t0 <= L - 1;
  const int32_t* h = tokens + static_cast<long long>(b) * capacity;
  unsigned long long key = 0ull;
  if (active) {
    // Stage h[t0 - kNgHalo, t0 + kNgramTile) where it lies in [0, L); other slots are never
    // compared (every compared index e - j lies in [0, L - 2]).
    const int i0 = t0 - kNgHalo;
    if constexpr (kVec) {
      // All of the thread's 16-byte loads go out before any is stored: an out-of-range slot
      // reads h[0..3] (in the row: L >= 1 here) and is zeroed afterwards.
      constexpr int kVecs = (kNgHalo + kNgramTile) / 4;
      constexpr int kIters = (kVecs + kNgThreads - 1) / kNgThreads;
      // Each history token is read once per call (halos aside): nontemporal 16-byte loads.
      typedef int i32x4 __attribute__((ext_vector_type(4)));
      const i32x4* hv = reinterpret_cast<const i32x4*>(h);
      int4 d[kIters];
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int v = tid + it * kNgThreads;
        const int idx = i0 + 4 * v;  // a multiple of 4; idx < L <= capacity keeps idx + 3 in the row
        const bool ok = v < kVecs && idx >= 0 && idx < L;
        const i32x4 t = __builtin_nontemporal_load(hv + (ok ? idx / 4 : 0));
        d[it] = make_int4(t.x, t.y, t.z, t.w);
      }
      const int suf = h[L - min(max(tid, 1), nmax)];  // sh_suf[tid] for tid in [1, nmax]
      if (tid >= 1 && tid <= nmax) sh_suf[tid] = suf;
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int v = tid + it * kNgThreads;
        const int idx = i0 + 4 * v;
        if (v < kVecs)
          reinterpret_cast<int4*>(sh_tok)[v] =
              (idx >= 0 && idx < L) ? d[it] : make_int4(0, 0, 0, 0);
      }
    } else {
      if (tid >= 1 && tid <= nmax) sh_suf[tid] = h[L - tid];
      for (int i = tid; i < kNgHalo + kNgramTile; i += kNgThreads) {
        const int idx = i0 + i;
        sh_tok[i] = (idx >= 0 && idx < L) ? h[idx] : 0;
      }
    }
    __syncthreads();
    unsigned long long best = 0ull;
    // m(e) >= 1 needs h[e-1] == h[L-1]: one independent LDS read per position.
    const int last = sh_suf[1];
    unsigned cand = 0u;
#pragma unroll
    for (int r = 0; r < kNgPer; ++r) {
      const int e = t0 + r * kNgThreads + tid;
      if (e >= 1 && e <= L - 1 && sh_tok[kNgHalo + (e - t0) - 1] == last) cand |= 1u << r;
    }
    while (cand) {
      const int r = __ffs(cand) - 1;
      cand &= cand - 1u;
      const int e = t0 + r * kNgThreads + tid;
      const int base = kNgHalo + (e - t0);
      const int jmax = min(nmax, e);
      int J = 1;
      while (J < jmax && sh_tok[base - J - 1] == sh_suf[J + 1]) ++J;
      if (J >= n_min)
        best = max_u64(best, (static_cast<unsigned long long>(J) << 32) |
                                 (0xffffffffull - static_cast<unsigned>(e)));
    }
    best = wave_max_u64(best);
    if (lane == 0) sh_best[wave] = best;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kNgThreads / 64; ++w) key = max_u64(key, sh_best[w]);
  }
  if (ntiles > 1) {
    if (tid == 0) partials[static_cast<long long>(b) * ntiles + tile] = key;
    return;
  }
  // One tile covers the history: emit here, the proposal read from LDS (t0 = 0 and
  // [e, e + cnt) lies in [0, L), all staged).
  if (wave != 0) return;
  int e = 0;
  const int cnt = proposal_count(key, L, K, e);
  if (lane < K)
    proposed[static_cast<long long>(b) * K + lane] =
        lane < cnt ? sh_tok[kNgHalo + e + lane] : -1;
  if (lane == 0) num_draft[b] = valid ? cnt : -1;
}

__global__ __launch_bounds__(kEmitThreads) void ngram_emit_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ lengths, int B, int capacity,
    int K, int ntiles, const unsigned long long* __restrict__ partials,
    int32_t* __restrict__ proposed, int32_t* __restrict__ num_draft) {
  const int lane = threadIdx.x & 63;
  const long long bl =
      static_cast<long long>(blockIdx.x) * (kEmitThreads / 64) + (threadIdx.x >> 6);
  if (bl >= B) return;
  const int b = static_cast<int>(bl);
  // The length and the tile keys do not depend on each other: both go out before either is
  // used (the match kernel wrote every tile's key, 0 for an invalid history).
  const int L = lengths[b];
  const unsigned long long* p = partials + static_cast<long long>(b) * ntiles;
  unsigned long long key = 0ull;
  for (int t = lane; t < ntiles; t += 64) key = max_u64(key, p[t]);
  key = wave_max_u64(key);
  const bool valid = L >= 0 && L <= capacity;
  if (!valid) key = 0ull;
  int e = 0;
  const int cnt = proposal_count(key, L, K, e);
  if (lane < K) {
    const int32_t* h = tokens + static_cast<long long>(b) * capacity;
    proposed[static_cast<long long>(b) * K + lane] = lane < cnt ? h[e + lane] : -1;
  }
  if (lane == 0) num_draft[b] = valid ? cnt : -1;
}

// ------------------------------------------------------------------------------------------
// Histories longer than one tile, 16-byte rows: one 1024-thread workgroup per history.  The
// candidate positions are cut into 512-position steps dealt round-robin to the 16 waves (wave w
// takes steps w, w + 16, ...), so a round of steps is 32 KB of contiguous history and a wave's
// first step is known before the history's length is: its loads go out with the length's.  A
// wave loads each step with two 16-byte loads per lane plus the 32 tokens before it (a candidate's
// run reaches back at most kNgramMaxN - 1 tokens), the next step's loads in flight while the
// current one is staged in the wave's own LDS slot and searched.  The waves never wait for one
// another until the final max-reduction (LDS accesses of one wave complete in issue order, so a
// staged step is readable by every lane of the wave), and the tile keys never leave the
// workgroup: no per-tile records, no second launch.  A lane's candidates come in increasing
// position order within a step, and a wave's steps in increasing order, so once a lane's best run
// reaches the cap min(n_max, L - 1) none of its later candidates can win (equal runs prefer the
// earlier position) and it stops extending.  Before the reduction each wave issues the loads of
// the tokens that follow its own best match, so the proposal is at hand when the winner is known.
// ------------------------------------------------------------------------------------------
constexpr int kHistThreads = 1024;
constexpr int kHistWaves = kHistThreads / 64;
constexpr int kHistStep = 64 * 2 * 4;           // positions per wave step
constexpr int kHistSlot = kNgramMaxN + kHistStep;  // a step and the tokens before it

__global__ __launch_bounds__(kHistThreads) void ngram_history_kernel(
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ lengths, int capacity,
    int n_min, int n_max, int K, int32_t* __restrict__ proposed, int32_t* __restrict__ num_draft) {
  // slot[w][i] = h[512 s - kNgramMaxN + i] while wave w searches step s
  __shared__ __align__(16) int slot[kHistWaves][kHistSlot];
  __shared__ int sh_suf[kHistWaves][kNgramMaxN + 1];  // sh_suf[w][j] = h[L - j]
  __shared__ unsigned long long sh_best[kHistWaves];
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = static_cast<int>(blockIdx.x);
  const int32_t* h = tokens + static_cast<long long>(b) * capacity;
  const i32x4* hv = reinterpret_cast<const i32x4*>(h);  // capacity is a multiple of 4 here
  const int last_vec = capacity / 4 - 1;
  int* ws = slot[wave];
  // Lane l < 8 also loads the l-th 16-byte vector of the 32 tokens before the step.
  auto load_step = [&](int st, i32x4 (&d)[2], i32x4& halo) {
    const int v0 = st * (kHistStep / 4);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      d[j] = __builtin_nontemporal_load(hv + min(v0 + j * 64 + lane, last_vec));
    halo = hv[min(max(v0 - kNgramMaxN / 4 + (lane & 7), 0), last_vec)];
  };
  i32x4 cur[2], nxt[2] = {}, hcur, hnxt = {};
  load_step(wave, cur, hcur);
  const int L = lengths[b];
  const bool valid = L >= 0 && L <= capacity;
  const int nmax = min(n_max, L - 1);
  unsigned long long best = 0ull;
  if (valid && nmax >= n_min) {  // uniform over the workgroup; L >= 2 from here on
    const int last = h[L - 1];
    const int suf = h[L - min(max(lane, 1), nmax)];
    if (lane >= 1 && lane <= nmax) sh_suf[wave][lane] = suf;
    bool capped = false;  // this lane's best run has reached nmax
    // Candidate positions e - 1 = q in [0, L - 2]: wave w searches steps w, w + 16, ...
    for (int st = wave; st * kHistStep < L - 1; st += kHistWaves) {  // uniform over the wave
      const int q_lo = st * kHistStep, q_hi = min(q_lo + kHistStep, L - 1);
      const bool more = (st + kHistWaves) * kHistStep < L - 1;
      if (more) load_step(st + kHistWaves, nxt, hnxt);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        *reinterpret_cast<i32x4*>(&ws[kNgramMaxN + 4 * (j * 64 + lane)]) = cur[j];
      if (lane < 8) *reinterpret_cast<i32x4*>(&ws[4 * lane]) = hcur;
      unsigned cand = 0u;  // bit 4j + c: q = q_lo + 4 (j * 64 + lane) + c
      if (!capped) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q0 = q_lo + 4 * (j * 64 + lane);
          cand |= (q0 < q_hi && cur[j].x == last) ? 1u << (4 * j) : 0u;
          cand |= (q0 + 1 < q_hi && cur[j].y == last) ? 1u << (4 * j + 1) : 0u;
          cand |= (q0 + 2 < q_hi && cur[j].z == last) ? 1u << (4 * j + 2) : 0u;
          cand |= (q0 + 3 < q_hi && cur[j].w == last) ? 1u << (4 * j + 3) : 0u;
        }
      }
      __builtin_amdgcn_wave_barrier();  // the step's stores are issued before any read of it
      while (cand) {
        const int r = __ffs(cand) - 1;
        cand &= cand - 1u;
        const int i = 4 * ((r >> 2) * 64 + lane) + (r & 3);  // q - q_lo
        const int q = q_lo + i;
        const int jmax = min(nmax, q + 1);
        int J = 1;
        while (J < jmax && ws[kNgramMaxN + i - J] == sh_suf[wave][J + 1]) ++J;
        if (J >= n_min)
          best = max_u64(best, (static_cast<unsigned long long>(J) << 32) |
                                   (0xffffffffull - static_cast<unsigned>(q + 1)));
        if (J == nmax) {
          capped = true;
          break;
        }
      }
      __builtin_amdgcn_wave_barrier();  // every read of the slot precedes the next step's stores
      if (more) {
#pragma unroll
        for (int j = 0; j < 2; ++j) cur[j] = nxt[j];
        hcur = hnxt;
      }
    }
  }
  // The wave's own best and the tokens that follow it, loaded while the other waves finish.
  best = wave_max_u64(best);
  int e = 0;
  const int cnt = proposal_count(best, L, K, e);
  const int follow = lane < cnt ? h[e + lane] : -1;
  if (lane == 0) sh_best[wave] = best;
  __syncthreads();
  unsigned long long key = lane < kHistWaves ? sh_best[lane] : 0ull;
  key = wave_max_u64(key);
  // The wave holding the winning key writes the proposal (keys of different waves differ in the
  // position); wave 0 writes the empty proposal when there is none.
  if (key == 0ull ? wave != 0 : key != best) return;
  if (lane < K) proposed[static_cast<long long>(b) * K + lane] = follow;
  if (lane == 0) num_draft[b] = valid ? cnt : -1;
}

}  // namespace

hipError_t launch_ngram(const NgramArgs& a) {
  if (a.B == 0) return hipSuccess;
  const int ntiles = ngram_tiles(a.capacity);
  const bool vec = (reinterpret_cast<uintptr_t>(a.tokens) % 16 == 0) && (a.capacity % 4 == 0);
  if (vec && ntiles > 1) {
    ngram_history_kernel<<<static_cast<unsigned>(a.B), kHistThreads, 0, a.stream>>>(
        a.tokens, a.lengths, a.capacity, a.n_min, a.n_max, a.K, a.proposed, a.num_draft);
    return hipGetLastError();
  }
  const unsigned grid1 = static_cast<unsigned>(static_cast<long long>(a.B) * ntiles);
  if (vec)
    ngram_match_kernel<true><<<grid1, kNgThreads, 0, a.stream>>>(
        a.tokens, a.lengths, a.capacity, a.n_min, a.n_max, a.K, ntiles, a.partials, a.proposed,
        a.num_draft);
  else
    ngram_match_kernel<false><<<grid1, kNgThreads, 0, a.stream>>>(
        a.tokens, a.lengths, a.capacity, a.n_min, a.n_max, a.K, ntiles, a.partials, a.proposed,
        a.num_draft);
  if (ntiles == 1) return hipGetLastError();
  const unsigned grid2 = static_cast<unsigned>((a.B + kEmitThreads / 64 - 1) / (kEmitThreads / 64));
  ngram_emit_kernel<<<grid2, kEmitThreads, 0, a.stream>>>(a.tokens, a.lengths, a.B, a.capacity,
                                                        a.K, ntiles, a.partials, a.proposed,
                                                        a.num_draft);
  return hipGetLastError();
}

}  // namespace specdec
