// gfx950 kernels of the acceptance telemetry and of the per-route draft-length plan.
//
// The pages' operational advice is to record the acceptance rate per route and to pick the
// draft length from it ("Decodificação especulativa explicada", gsantana.dev, sections "Quanto
// mais rápido: a matemática" and "Checagem de realidade em produção"; "Speculative decoding: el
// secretario...", blog.lo0.es, section "Pitfalls operacionales").  The device side only counts
// (telemetry_kernel) and applies a chosen length (apply_k_kernel); the choice itself is host
// arithmetic (telemetry.cpp).
//
// telemetry_kernel: one 1024-thread workgroup accumulates every sequence of the batch into
// per-route counters in LDS (integer atomics, so the totals do not depend on the order), then
// adds them to the caller's int64 counters.  A wave whose counted lanes share one route sums
// the seven scalar fields with shuffles first and issues one LDS atomic per field.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace specdec {
namespace {

constexpr int kTmThreads = 1024;

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(kTmThreads) void telemetry_kernel(
    const int32_t* __restrict__ accept_len, const int32_t* __restrict__ num_draft,
    const int32_t* __restrict__ route, int B, int K, int n_routes,
    long long* __restrict__ counters) {
  extern __shared__ unsigned long long sh[];  // [n_routes][kTelemetryRow]
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = n_routes * kTelemetryRow;
  for (int i = tid; i < n; i += kTmThreads) sh[i] = 0ull;
  __syncthreads();
  // The caller's counters are read now (after the barrier, which would wait for them), while
  // the batch is counted.
  constexpr int kPre = 5;
  static_assert(kTelemetryMaxRoutes * kTelemetryRow <= kPre * kTmThreads, "counter prefetch");
  long long cpre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) cpre[j] = counters[min(tid + j * kTmThreads, n - 1)];
  for (int b0 = 0; b0 < B; b0 += kTmThreads) {
    const int b = b0 + tid;
    // The three per-sequence loads go out together (index clamped into the batch).
    const int bc = min(b, B - 1);
    const int r_ld = route ? route[bc] : 0;
    const int A_ld = accept_len[bc];
    const int k_ld = num_draft ? num_draft[bc] : K;
    int r = -1, A = 0, k = 0;
    bool counted = false, valid = false;
    if (b < B) {
      r = r_ld;
      if (r >= 0 && r < n_routes) {
        counted = true;
        A = A_ld;
        k = k_ld;
        valid = A >= 0 && k >= 0 && k <= K && A <= k;
      }
    }
    const int f[7] = {valid ? 1 : 0,       valid ? k : 0,
                      valid ? A : 0,       valid ? A + 1 : 0,
                      valid && A == k,     valid && A < k,
                      counted && !valid};
    const unsigned long long cm = __ballot(counted);
    const int r0 = cm ? __shfl(r, __ffsll(static_cast<long long>(cm)) - 1, 64) : -1;
    const bool same = __all(!counted || r == r0);
    if (same) {
      if (cm) {
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          const int v = wave_sum_i(f[i]);
          if (lane == 0 && v) atomicAdd(&sh[r0 * kTelemetryRow + i], static_cast<unsigned long long>(v));
        }
      }
    } else if (counted) {
#pragma unroll
      for (int i = 0; i < 7; ++i)
        if (f[i]) atomicAdd(&sh[r * kTelemetryRow + i], static_cast<unsigned long long>(f[i]));
    }
    if (valid) atomicAdd(&sh[r * kTelemetryRow + kTelemetryFields + A], 1ull);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int i = tid + j * kTmThreads;
    if (i < n) counters[i] = cpre[j] + static_cast<long long>(sh[i]);
  }
}

__global__ __launch_bounds__(256) void apply_k_kernel(int32_t* __restrict__ num_draft,
                                                      const int32_t* __restrict__ route,
                                                      const int32_t* __restrict__ k_table,
                                                      int B, int n_routes) {
  const long long bl = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (bl >= B) return;
  const int b = static_cast<int>(bl);
  // The route and the draft count are read together; the table read waits only for the route.
  const int r = route ? route[b] : 0;
  const int nd = num_draft[b];
  if (r < 0 || r >= n_routes || nd < 0) return;
  num_draft[b] = min(nd, max(0, k_table[r]));
}

}  // namespace

hipError_t launch_telemetry(const int32_t* accept_len, const int32_t* num_draft,
                            const int32_t* route, int B, int K, int n_routes,
                            long long* counters, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const size_t lds = static_cast<size_t>(n_routes) * kTelemetryRow * sizeof(unsigned long long);
  telemetry_kernel<<<1, kTmThreads, lds, stream>>>(accept_len, num_draft, route, B, K, n_routes,
                                                   counters);
  return hipGetLastError();
}

hipError_t launch_apply_k(int32_t* num_draft, const int32_t* route, const int32_t* k_table,
                          int B, int n_routes, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  apply_k_kernel<<<(B + 255) / 256, 256, 0, stream>>>(num_draft, route, k_table, B, n_routes);
  return hipGetLastError();
}

}  // namespace specdec
