// Device building blocks shared by the gfx950 verify kernels: the temperature rules, wave64 DPP
// reductions and scans within one wavefront (no LDS round trips) with uniform lane reads, and the
// probability weight 2^((z - m) * c) of one token in double precision.
#pragma once

#include <float.h>
#include <math.h>

#include <hip/hip_runtime.h>

namespace specdec {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kTempMin = 1e-6f;  // smallest non-zero temperature (SPECDEC_TEMPERATURE_MIN)

// A temperature is 0 (greedy) or a finite value of at least kTempMin.
__device__ __forceinline__ bool temp_valid(float T) {
  return T == 0.f || (T >= kTempMin && T <= FLT_MAX);
}
// exp2 scale: log2(e)/T for sampled rows, log2(e) (softmax at T = 1) for greedy rows.
__device__ __forceinline__ float temp_scale(float T) { return T == 0.f ? kLog2e : kLog2e / T; }

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float read_lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Max over the wave (every lane gets it): 16-lane rows by DPP, then the four row results.
// fmaxf ignores NaN; a NaN logit poisons the sum instead.
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  return fmaxf(fmaxf(read_lane_f(v, 0), read_lane_f(v, 16)),
               fmaxf(read_lane_f(v, 32), read_lane_f(v, 48)));
}

// Sum over the wave in a fixed order (every lane gets it).
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  return (read_lane_f(v, 0) + read_lane_f(v, 16)) + (read_lane_f(v, 32) + read_lane_f(v, 48));
}

// fp64 wave scans with DPP moves of both 32-bit halves (no LDS round trips): row_shr 1, 2, 4, 8
// within each 16-lane row, then row_bcast 15 / 31 carry the row totals across rows.  Lanes whose
// DPP source lies outside the row read 0, so the additions are the textbook inclusive scan.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ double dpp_move_d(double v) {
  const long long bits = __double_as_longlong(v);
  const int lo =
      __builtin_amdgcn_update_dpp(0, static_cast<int>(bits), kCtrl, kRowMask, 0xf, false);
  const int hi =
      __builtin_amdgcn_update_dpp(0, static_cast<int>(bits >> 32), kCtrl, kRowMask, 0xf, false);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

__device__ __forceinline__ double wave_inclusive_scan(double v) {
  v += dpp_move_d<0x111, 0xf>(v);  // row_shr:1
  v += dpp_move_d<0x112, 0xf>(v);  // row_shr:2
  v += dpp_move_d<0x114, 0xf>(v);  // row_shr:4
  v += dpp_move_d<0x118, 0xf>(v);  // row_shr:8
  v += dpp_move_d<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_move_d<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Lane l's value, read by every lane (uniform).
__device__ __forceinline__ double read_lane_d(double v, int l) {
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(bits), l);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(bits >> 32), l);
  return __longlong_as_double((static_cast<long long>(hi) << 32) |
                              static_cast<unsigned int>(lo));
}

// Sum over the wave, the same in every lane.
__device__ __forceinline__ double wave_total(double v) {
  return read_lane_d(wave_inclusive_scan(v), 63);
}

template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xf, 0xf, false);
}

// 2^((z - m) * c) for one token, as a double good to a few parts in 1e7: the exponent r in fp64 (z
// - m is exact there), split as r = rh + rl with rh = (float)r, then 2^rh from the hardware exp2
// (about 1 ulp) times 2^rl = 1 + rl ln 2 (|rl| <= ulp(rh) / 2, so the next term is below 1e-14).
// The accept tests and the emitted probabilities need no more (the sums it is compared with are
// built from fp32 terms), and this costs a dozen instructions where a full fp64 exp2 costs about
// fifty, on the path from the row statistics to the decisions.  Exponents at or below -120 (2^r
// within reach of fp32's subnormals, or -inf logits) take the fp64 exp2.
__device__ __forceinline__ double exp2_diff(float z, float m, float c) {
  const double r = (static_cast<double>(z) - static_cast<double>(m)) * static_cast<double>(c);
  const float rh = static_cast<float>(r);
  if (!(rh > -120.f)) return exp2(r);
  const double rl = r - static_cast<double>(rh);
  return static_cast<double>(__builtin_amdgcn_exp2f(rh)) * fma(rl, 0x1.62e42fefa39efp-1, 1.0);
}

}  // namespace specdec
