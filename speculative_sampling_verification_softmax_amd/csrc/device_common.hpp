// device_common.hpp -- small device helpers shared by the verify kernels:
// logit loads, wave64/block reductions and scans, and an fp64 exponential.
//
// Compiled with -ffp-contract=off: every floating-point expression rounds
// exactly as written (fused multiply-adds only where fma()/fmaf() is called),
// so two evaluations of the same expression on the same inputs always give
// the same bits.  The residual draw relies on that to re-derive one chunk's
// weights identically.
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

// The 16 bytes at a 16-byte aligned address as fp32 values (8 bf16 or 4 fp32).
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float (&x)[16 / Elt<DT>::bytes]) {
  if constexpr (DT == kBF16) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  } else {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
}

// E = 16/elt consecutive logits starting at x0 (a multiple of E); positions at
// or past V read as -inf.  One 16-byte load when the row start is 16-byte
// aligned and the group is whole, element loads otherwise.
template <int DT>
__device__ __forceinline__ void load_group(const void* row, int64_t x0, int V, bool aligned,
                                           float (&z)[16 / Elt<DT>::bytes]) {
  constexpr int E = 16 / Elt<DT>::bytes;
  if (aligned && x0 + E <= V) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const char*>(row) +
                                                    x0 * Elt<DT>::bytes);
    unpack16<DT>(v, z);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      z[e] = (x0 + e < V) ? logit_f32<DT>(row, x0 + e) : -__builtin_huge_valf();
  }
}

// A row defines a distribution iff its max is finite and its sum is not NaN.
__device__ __forceinline__ bool row_ok(float m, float s) {
  return !__builtin_isnan(s) && __builtin_isfinite(m);
}

// ---------------------------------------------------------------- wave64 ops
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// A value known to be the same in every lane (read from LDS or from one
// address), moved to a scalar register so that the compiler treats it, and
// everything derived from it, as uniform.
__device__ __forceinline__ unsigned uniform(unsigned v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Butterfly sum: every lane ends with the same bits (a+b == b+a exactly).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = v + __shfl_xor(v, o, kWave);
  return v;
}

// Sum over the 64 lanes without the LDS crossbar: an inclusive scan inside
// each row of 16 lanes with DPP row shifts (lanes shifted in from outside the
// row read 0), then the four row totals (lanes 15, 31, 47, 63) added in
// order.  Fixed order; every lane gets the same bits.
__device__ __forceinline__ double dpp_row_shr(double v, int ctrl_n) {
  const int lo = __double2loint(v), hi = __double2hiint(v);
  int rlo, rhi;
  switch (ctrl_n) {  // dpp_ctrl must be a constant: row_shr:n is 0x110 + n
    case 1:
      rlo = __builtin_amdgcn_update_dpp(0, lo, 0x111, 0xf, 0xf, true);
      rhi = __builtin_amdgcn_update_dpp(0, hi, 0x111, 0xf, 0xf, true);
      break;
    case 2:
      rlo = __builtin_amdgcn_update_dpp(0, lo, 0x112, 0xf, 0xf, true);
      rhi = __builtin_amdgcn_update_dpp(0, hi, 0x112, 0xf, 0xf, true);
      break;
    case 4:
      rlo = __builtin_amdgcn_update_dpp(0, lo, 0x114, 0xf, 0xf, true);
      rhi = __builtin_amdgcn_update_dpp(0, hi, 0x114, 0xf, 0xf, true);
      break;
    default:
      rlo = __builtin_amdgcn_update_dpp(0, lo, 0x118, 0xf, 0xf, true);
      rhi = __builtin_amdgcn_update_dpp(0, hi, 0x118, 0xf, 0xf, true);
      break;
  }
  return __hiloint2double(rhi, rlo);
}

// The inclusive scan inside each row of 16 lanes: lanes 15, 31, 47 and 63
// end with their row's total.
__device__ __forceinline__ double wave_scan_rows(double v) {
  v = v + dpp_row_shr(v, 1);
  v = v + dpp_row_shr(v, 2);
  v = v + dpp_row_shr(v, 4);
  v = v + dpp_row_shr(v, 8);
  return v;
}

// The four row totals added in order (every lane gets the same bits).
__device__ __forceinline__ double sum_row_totals(double r0, double r1, double r2, double r3) {
  return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ double wave_sum_rows(double v) {
  v = wave_scan_rows(v);
  auto lane_val = [&](int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
  };
  return sum_row_totals(lane_val(15), lane_val(31), lane_val(47), lane_val(63));
}

// Inclusive prefix sum across the 64 lanes (Hillis-Steele order, fixed),
// through the LDS crossbar.
__device__ __forceinline__ double wave_incl_scan_shfl(double v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    double o = __shfl_up(v, d, kWave);
    if (lane >= d) v = v + o;
  }
  return v;
}

// A DPP move of a double (both halves with the same control); lanes of rows
// outside row_mask, and lanes without a source, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_mov(double v) {
  const int lo = __double2loint(v), hi = __double2hiint(v);
  return __hiloint2double(__builtin_amdgcn_update_dpp(0, hi, CTRL, ROW_MASK, 0xf, true),
                          __builtin_amdgcn_update_dpp(0, lo, CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum across the 64 lanes in DPP moves only: the in-row
// scans, then the total of row 0 added to row 1 and of row 2 to row 3
// (row_bcast:15), then the total of rows 0-1 added to rows 2 and 3
// (row_bcast:31).  Fixed order.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v = wave_scan_rows(v);
  v = v + dpp_mov<0x142, 0xA>(v);
  v = v + dpp_mov<0x143, 0xC>(v);
  return v;
}

// The value of lane i-1 (0 in lane 0): DPP wave_shr:1.
__device__ __forceinline__ double wave_shr1(double v) { return dpp_mov<0x138, 0xF>(v); }

// The value of a double in lane l (l wave-uniform).
__device__ __forceinline__ double readlane_d(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}

// ---------------------------------------------------------------- block ops
// `red` must hold at least BLOCK/64 entries of the reduced type.  The result
// is returned to every thread.
template <int BLOCK>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < BLOCK / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <int BLOCK>
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int i = 1; i < BLOCK / kWave; ++i) r = r + red[i];
  return r;
}

// ---------------------------------------------------------------- fp64 exp
// exp(d) for d <= 0 with relative error below 2e-13, in the form
//   d * 256/ln2 = y = k + r,  k = rint(y), |r| <= 1/2,
//   exp(d) = 2^(k>>8) * 2^((k&255)/256) * 2^(r/256),
// with 2^(j/256) from a 256-entry table (tab, filled by fill_exp2_table) and
// 2^(r/256) = exp(r ln2/256) by its degree-3 Taylor polynomial
// (|r ln2/256| <= 0.00136, truncation error <= 1.5e-13).  Callers pass y, the
// argument already multiplied by 256/ln2.
struct Exp64 {
  static constexpr int kTab = 256;
  static constexpr double kLn2 = 0.693147180559945309417232121458176568;
  static constexpr double kScale = 256.0 / kLn2;
  static constexpr double c1 = kLn2 / 256.0;
  // Adding 1.5*2^52 rounds a double of magnitude below 2^51 to an integer k
  // (to nearest, ties to even) and leaves k in the low 32 bits of the sum.
  static constexpr double kRound = 6755399441055744.0;
  // y is clamped here: 2^(-300000/256) = 2^-1172 underflows to exactly 0, so
  // -inf (and NaN, which fmax drops) give 0 without a select.
  static constexpr double kFloor = -300000.0;
};

// Threads first .. blockDim.x-1 fill the table.
__device__ __forceinline__ void fill_exp2_table(double* tab, int first = 0) {
  for (int j = static_cast<int>(threadIdx.x) - first; j < Exp64::kTab;
       j += static_cast<int>(blockDim.x) - first)
    tab[j] = exp2(static_cast<double>(j) / Exp64::kTab);
}

__device__ __forceinline__ double exp64_scaled(double y, const double* tab) {
  const double yc = fmax(y, Exp64::kFloor);
  const double kb = yc + Exp64::kRound;
  const int ki = __double2loint(kb);
  const double x = (yc - (kb - Exp64::kRound)) * Exp64::c1;  // r ln2/256
  // 1 + x + x^2/2 + x^3/6; only the 1/6 is not an inline constant
  double p = fma(x, 1.0 / 6.0, 0.5);
  p = fma(x, p, 1.0);
  p = fma(x, p, 1.0);
  return ldexp(tab[ki & 255] * p, ki >> 8);
}

// ------------------------------------------------- cross-workgroup handoff
// Values handed from one workgroup to another inside one launch (possibly on
// another XCD, whose L2 is not coherent with this one) move through
// device-scope relaxed atomic loads and stores: on gfx950 these are ordinary
// vector loads/stores with the sc1 bit, which go to the device-coherent
// level instead of a possibly stale or dirty XCD L2 line.  A publisher makes
// its sc1 stores complete (store_complete: s_waitcnt on the wave's memory
// counter) before the workgroup barrier and the counter/flag update that
// announces them; a consumer reads the flag, then the data, both with sc1.
// This avoids device-scope fences, which write back and invalidate the whole
// L2 of the XCD each time.
__device__ __forceinline__ unsigned atomic_add_dev(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned atomic_load_dev(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_dev(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads of an array written by other workgroups of the same launch, as
// buffer loads with the sc1 bit: unlike the atomic loads above they carry no
// ordering, so the compiler issues a thread's loads together.  `base` must be
// uniform across the wave (it goes into a scalar buffer resource) and the
// array no longer than 2^31 bytes.  Src<false, T> is the plain-pointer view
// with the same interface.
constexpr int kBufWord3Dev = 0x00020000;  // untyped dword access (gfx9 family)
constexpr int kAuxSc1 = 16;               // cache-policy bit sc1

template <bool XB, typename T>
struct Src;

template <typename T>
struct Src<false, T> {
  const T* p;
  __device__ __forceinline__ Src(const T* base, int64_t) : p(base) {}
  __device__ __forceinline__ T operator[](int64_t i) const { return p[i]; }
};

template <typename T>
struct Src<true, T> {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte elements");
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ Src(const T* base, int64_t n)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), static_cast<short>(0),
                                            static_cast<int>(n * static_cast<int64_t>(sizeof(T))),
                                            kBufWord3Dev)) {}
  __device__ __forceinline__ T operator[](int64_t i) const {
    const int off = static_cast<int>(i * static_cast<int64_t>(sizeof(T)));
    if constexpr (sizeof(T) == 4) {
      const unsigned w = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAuxSc1);
      return __builtin_bit_cast(T, w);
    } else {
      const auto w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kAuxSc1);
      const unsigned long long v =
          static_cast<unsigned long long>(w[0]) | (static_cast<unsigned long long>(w[1]) << 32);
      return __builtin_bit_cast(T, v);
    }
  }
};

// Wait until this wave's outstanding memory operations have completed.
__device__ __forceinline__ void store_complete() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// Loads and stores of handed-off values.  XB = false gives plain accesses
// (single-workgroup or single-kernel use); XB = true the sc1 form above.
template <bool XB>
__device__ __forceinline__ float ld(const float* p) {
  if constexpr (XB) {
    return __uint_as_float(
        __hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT));
  } else {
    return *p;
  }
}
template <bool XB>
__device__ __forceinline__ double ld(const double* p) {
  if constexpr (XB) {
    return __longlong_as_double(static_cast<long long>(
        __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT)));
  } else {
    return *p;
  }
}
template <bool XB>
__device__ __forceinline__ int ld(const int* p) {
  if constexpr (XB) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    return *p;
  }
}
template <bool XB>
__device__ __forceinline__ void st(float* p, float v) {
  if constexpr (XB) {
    __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = v;
  }
}
template <bool XB>
__device__ __forceinline__ void st(double* p, double v) {
  if constexpr (XB) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       static_cast<unsigned long long>(__double_as_longlong(v)),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = v;
  }
}
template <bool XB>
__device__ __forceinline__ void st(int* p, int v) {
  if constexpr (XB) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *p = v;
  }
}

}  // namespace spec
