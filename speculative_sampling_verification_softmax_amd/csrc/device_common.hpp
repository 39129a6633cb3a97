// device_common.hpp -- small device helpers shared by the verify kernels:
// logit loads, wave64/block reductions and scans, and an fp64 exponential.
//
// Compiled with -ffp-contract=off: every floating-point expression rounds
// exactly as written (fused multiply-adds only where fma()/fmaf() is called),
// so two evaluations of the same expression on the same inputs always give
// the same bits.  The residual kernel relies on that to re-derive one chunk's
// prefix sums identically.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

constexpr int kWave = 64;

enum : int { kF32 = 0, kBF16 = 1 };

template <int DT> struct Elt;
template <> struct Elt<kF32> { using T = float; static constexpr int bytes = 4; };
template <> struct Elt<kBF16> { using T = uint16_t; static constexpr int bytes = 2; };

// Exact widening of stored logits to fp32 (bf16 is the upper half of a binary32).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ float logit_f32(const void* base, int64_t i) {
  if constexpr (DT == kF32) {
    return static_cast<const float*>(base)[i];
  } else {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
  }
}

// A row defines a distribution iff its max is finite and its sum is not NaN.
__device__ __forceinline__ bool row_ok(float m, float s) {
  return !__builtin_isnan(s) && __builtin_isfinite(m);
}

// ---------------------------------------------------------------- wave64 ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = v + __shfl_xor(v, o, kWave);
  return v;
}

// Inclusive prefix sum across the 64 lanes (Hillis-Steele order, fixed).
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    double o = __shfl_up(v, d, kWave);
    if (lane >= d) v = v + o;
  }
  return v;
}

// ---------------------------------------------------------------- block ops
// `red` must hold at least BLOCK/64 entries of the reduced type.
template <int BLOCK>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < BLOCK / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <int BLOCK>
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int i = 1; i < BLOCK / kWave; ++i) r = r + red[i];
  return r;
}

// ---------------------------------------------------------------- fp64 exp
// exp(d) for d <= 0 with relative error below 1e-13, in the form
//   d * 64/ln2 = y = k + r,  k = rint(y), |r| <= 1/2,
//   exp(d) = 2^(k>>6) * 2^((k&63)/64) * 2^(r/64),
// with 2^(j/64) from a 64-entry table (tab, filled by fill_exp2_table) and
// 2^(r/64) = exp(r ln2/64) by its degree-4 Taylor polynomial
// (|r ln2/64| <= 0.0055, truncation error <= 4e-14).  Callers pass y, the
// argument already multiplied by 64/ln2.  Results below ~2^-1060 flush to 0.
struct Exp64 {
  static constexpr double kLn2 = 0.693147180559945309417232121458176568;
  static constexpr double kScale = 64.0 / kLn2;   // 64 / ln 2
  static constexpr double c1 = kLn2 / 64.0;
  static constexpr double c2 = c1 * c1 / 2.0;
  static constexpr double c3 = c1 * c1 * c1 / 6.0;
  static constexpr double c4 = c1 * c1 * c1 * c1 / 24.0;
};

__device__ __forceinline__ void fill_exp2_table(double* tab) {
  for (int j = threadIdx.x; j < 64; j += blockDim.x) tab[j] = exp2(static_cast<double>(j) / 64.0);
}

__device__ __forceinline__ double exp64_scaled(double y, const double* tab) {
  if (!(y > -67900.0)) return 0.0;  // also -inf
  const double k = rint(y);
  const double r = y - k;
  const int ki = static_cast<int>(k);
  double p = fma(r, Exp64::c4, Exp64::c3);
  p = fma(r, p, Exp64::c2);
  p = fma(r, p, Exp64::c1);
  p = fma(r, p, 1.0);
  return ldexp(tab[ki & 63] * p, ki >> 6);
}

}  // namespace spec
