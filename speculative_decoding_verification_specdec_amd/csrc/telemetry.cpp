// C ABI of the acceptance telemetry and of the per-route draft-length plan (declared in
// include/specdec.h).  The counting runs on the device (telemetry.hip); estimating the
// acceptance rate and choosing k are a few host flops on the counters:
//   E[tokens per target pass] = (1 - a^(k+1)) / (1 - a)   and
//   speedup = E / (k c + 1)
// ("Decodificação especulativa explicada", gsantana.dev, section "Quanto mais rápido: a
// matemática"; "Speculative decoding: el secretario...", blog.lo0.es, section "La matemática
// que importa: techo y speedup").
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "specdec.h"

namespace {

bool misaligned(const void* p, size_t a) {
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) != 0;
}

}  // namespace

extern "C" {

specdec_status specdec_telemetry_update(const int32_t* accept_len, const int32_t* num_draft,
                                        const int32_t* route, int32_t B, int32_t K,
                                        int32_t n_routes, int64_t* counters, void* stream) {
  if (B < 0 || K < 0 || K > SPECDEC_MAX_K || n_routes < 1 ||
      n_routes > SPECDEC_TELEMETRY_MAX_ROUTES)
    return SPECDEC_ERR_SHAPE;
  if (B == 0) return SPECDEC_OK;
  if (!accept_len || !counters) return SPECDEC_ERR_NULL;
  if (misaligned(accept_len, 4) || misaligned(num_draft, 4) || misaligned(route, 4) ||
      misaligned(counters, 8))
    return SPECDEC_ERR_ALIGN;
  return specdec::launch_telemetry(accept_len, num_draft, route, B, K, n_routes,
                                   reinterpret_cast<long long*>(counters),
                                   static_cast<hipStream_t>(stream)) == hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

specdec_status specdec_apply_k(int32_t* num_draft, const int32_t* route, const int32_t* k_table,
                               int32_t B, int32_t n_routes, void* stream) {
  if (B < 0 || n_routes < 1) return SPECDEC_ERR_SHAPE;
  if (B == 0) return SPECDEC_OK;
  if (!num_draft || !k_table) return SPECDEC_ERR_NULL;
  if (misaligned(num_draft, 4) || misaligned(route, 4) || misaligned(k_table, 4))
    return SPECDEC_ERR_ALIGN;
  return specdec::launch_apply_k(num_draft, route, k_table, B, n_routes,
                                 static_cast<hipStream_t>(stream)) == hipSuccess
             ? SPECDEC_OK
             : SPECDEC_ERR_LAUNCH;
}

double specdec_alpha_estimate(const int64_t* route_counters) {
  if (!route_counters) return NAN;
  const double acc = static_cast<double>(route_counters[2]);
  const double rej = static_cast<double>(route_counters[5]);
  return acc + rej > 0.0 ? acc / (acc + rej) : NAN;
}

double specdec_expected_tokens(double alpha, int32_t k) {
  if (!(alpha >= 0.0 && alpha <= 1.0) || k < 0) return NAN;
  if (alpha == 1.0) return static_cast<double>(k) + 1.0;
  return (1.0 - pow(alpha, static_cast<double>(k) + 1.0)) / (1.0 - alpha);
}

double specdec_speedup(double alpha, int32_t k, double c) {
  if (!(c >= 0.0) || !isfinite(c)) return NAN;
  return specdec_expected_tokens(alpha, k) / (static_cast<double>(k) * c + 1.0);
}

int32_t specdec_choose_k(double alpha, double c, int32_t k_min, int32_t k_max) {
  if (k_min < 0 || k_max < k_min || k_max > SPECDEC_MAX_K) return -1;
  if (!(alpha >= 0.0 && alpha <= 1.0) || !(c >= 0.0) || !isfinite(c)) return -1;
  int32_t best_k = k_min;
  double best = -INFINITY;
  for (int32_t k = k_min; k <= k_max; ++k) {
    const double s = specdec_speedup(alpha, k, c);
    if (s > best) {
      best = s;
      best_k = k;
    }
  }
  return best_k;
}

specdec_status specdec_plan_k(const int64_t* counters, int32_t n_routes, double c, int32_t k_min,
                              int32_t k_max, int32_t k_default, int32_t* k_table) {
  if (n_routes < 1 || k_min < 0 || k_max < k_min || k_max > SPECDEC_MAX_K || k_default < 0 ||
      k_default > SPECDEC_MAX_K || !(c >= 0.0) || !isfinite(c))
    return SPECDEC_ERR_SHAPE;
  if (!counters || !k_table) return SPECDEC_ERR_NULL;
  for (int32_t r = 0; r < n_routes; ++r) {
    const double a = specdec_alpha_estimate(counters + static_cast<size_t>(r) * SPECDEC_TELEMETRY_ROW);
    k_table[r] = isnan(a) ? k_default : specdec_choose_k(a, c, k_min, k_max);
  }
  return SPECDEC_OK;
}

}  // extern "C"
