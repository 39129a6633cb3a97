// spec_softmax.hip -- host side of the C ABI declared in include/spec_softmax.h:
// argument validation, launch configuration and launches on the caller's
// stream.  No allocation, no synchronisation, no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "spec_softmax.h"
#include "kernels.hpp"

namespace {

using spec::kBF16;
using spec::kF32;

#ifndef SPEC_STATS_BLOCK
#define SPEC_STATS_BLOCK 1024
#endif
#ifndef SPEC_STATS_VPG_BF16
#define SPEC_STATS_VPG_BF16 4
#endif
#ifndef SPEC_STATS_VPG_F32
#define SPEC_STATS_VPG_F32 8
#endif
#ifndef SPEC_FILTER_VPG_BF16
#define SPEC_FILTER_VPG_BF16 4
#endif
#ifndef SPEC_FILTER_VPG_F32
#define SPEC_FILTER_VPG_F32 4
#endif
#ifndef SPEC_FUSED_VPG_BF16
#define SPEC_FUSED_VPG_BF16 4
#endif
#ifndef SPEC_FUSED_VPG_F32
#define SPEC_FUSED_VPG_F32 4
#endif
constexpr int kStatsBlock = SPEC_STATS_BLOCK;
constexpr int kResidBlock = 1024;
constexpr int kFusedBlock = 256;
constexpr int kFusedNW = kFusedBlock / spec::kWave;
// Dynamic LDS of the fused kernel: one double per chunk of a row.
constexpr size_t kFusedMaxDynLds = static_cast<size_t>(SPEC_MAX_V / 64 / 4) * sizeof(double);
// Dynamic LDS of a draw workgroup (the bf16 exponential tables when they fit
// too, then the fast-path arrays).  The static part is ~2.3 KB; a gfx950
// workgroup may hold 160 KB, and a draw workgroup has its CU alone.
constexpr size_t kResidFastLds = 152 * 1024;
constexpr size_t kDrawDynLds = 152 * 1024;

// Dynamic LDS of the residual / sample kernels: the fast-path arrays (or the
// slow path's nch doubles), preceded by `rows` bf16 exponential tables when
// they fit.
struct DrawLds {
  int fast, etab;
  size_t bytes;
};

DrawLds draw_lds(int nch, int dtype, int rows) {
  DrawLds d{};
  const size_t fast_lds = spec::draw_fast_lds(nch);
  d.fast = fast_lds <= kResidFastLds ? 1 : 0;
  const size_t work = d.fast ? fast_lds : static_cast<size_t>(nch) * sizeof(double);
  const size_t tables = static_cast<size_t>(rows) * spec::kETab * sizeof(double);
  d.etab = (dtype == SPEC_DTYPE_BF16 && work + tables <= kDrawDynLds) ? 1 : 0;
  d.bytes = work + (d.etab ? tables : 0);
  return d;
}

int elt_bytes(int dtype) { return dtype == SPEC_DTYPE_F32 ? 4 : 2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by all entry points.  Returns SPEC_OK or SPEC_ERR_INVALID_ARG.
int check_common(const void* tgt, const void* dft, int dtype, int B, int K, int V, float T) {
  if (tgt == nullptr || dft == nullptr) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_ERR_INVALID_ARG;
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return SPEC_ERR_INVALID_ARG;
  if (!std::isfinite(T) || !(T > 0.0f)) return SPEC_ERR_INVALID_ARG;
  const int eb = elt_bytes(dtype);
  if (!aligned(tgt, eb) || !aligned(dft, eb)) return SPEC_ERR_INVALID_ARG;
  // B*(K+1)*V*eb must fit comfortably in int64 and the row count in a grid.
  const double bytes = static_cast<double>(B) * (K + 1) * static_cast<double>(V) * eb;
  if (bytes > 4.0e18) return SPEC_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * (2 * K + 1) > 0x7fffffffLL) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

int chunk_tokens(int dtype) { return spec::kWave * (16 / elt_bytes(dtype)); }
int num_chunks(int V, int dtype) { return (V + chunk_tokens(dtype) - 1) / chunk_tokens(dtype); }
size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Workspace layout of spec_verify_fused (offsets in bytes from the base).
struct FusedLayout {
  size_t ctl, stat_word, ready, slices_done, rec, sq_part, sp_part, A, Bv, unc_n, unc_idx, total;
  int nch, S;
};

FusedLayout fused_layout(int B, int K, int V, int dtype) {
  FusedLayout L{};
  L.nch = num_chunks(V, dtype);
  const int cps = kFusedNW * spec::kFusedCPW;
  L.S = (L.nch + cps - 1) / cps;
  const size_t b = static_cast<size_t>(B);
  const size_t rows = b * (2 * static_cast<size_t>(K) + 1);
  size_t off = 0;
  // flags first: zero after every completed call, and a later call with
  // B' <= B and K' <= K finds all of its own flags inside that region
  L.ctl = off;         off = round256(off + spec::kCtlWords * sizeof(unsigned));
  L.stat_word = off;   off = round256(off + rows * sizeof(unsigned long long));
  L.ready = off;       off = round256(off + b * sizeof(unsigned));
  L.slices_done = off; off = round256(off + b * sizeof(unsigned));
  // written before they are read within each call
  L.rec = off;         off = round256(off + b * 8 * sizeof(int));
  L.sq_part = off;     off = round256(off + b * L.S * sizeof(double));
  L.sp_part = off;     off = round256(off + b * L.S * sizeof(double));
  L.A = off;           off = round256(off + b * L.nch * sizeof(double));
  L.Bv = off;          off = round256(off + b * L.nch * sizeof(double));
  L.unc_n = off;       off = round256(off + b * L.nch * sizeof(int));
  L.unc_idx = off;     off = round256(off + b * L.nch * spec::kUncMax * sizeof(int));
  L.total = off;
  return L;
}

// Item order of the fused kernel: group g holds 2K+1 ROW items if g < B, one
// SCAN item if D1 <= g < B+D1 and S SLICE items if D2 <= g < B+D2.  Groups
// are cut into segments of constant size; segments without items are
// dropped.  Returns the total item count.
int64_t fused_order(int B, int K, int S, int D1, int D2, spec::FusedArgs& a) {
  int64_t bp[6] = {0, D1, D2, B, static_cast<int64_t>(B) + D1, static_cast<int64_t>(B) + D2};
  for (int i = 1; i < 6; ++i)  // insertion sort
    for (int j = i; j > 0 && bp[j - 1] > bp[j]; --j) {
      const int64_t t = bp[j]; bp[j] = bp[j - 1]; bp[j - 1] = t;
    }
  const int64_t end = static_cast<int64_t>(B) + D2;
  int nseg = 0;
  int64_t items = 0;
  for (int i = 0; i < 6; ++i) {
    const int64_t g0 = bp[i], g1 = (i + 1 < 6) ? bp[i + 1] : end;
    if (g1 <= g0 || g0 >= end) continue;
    const int64_t size = (g0 < B ? 2 * K + 1 : 0) + (g0 >= D1 && g0 < B + D1 ? 1 : 0) +
                         (g0 >= D2 && g0 < B + D2 ? S : 0);
    if (size == 0) continue;
    a.seg_g0[nseg] = static_cast<int>(g0);
    a.seg_size[nseg] = static_cast<int>(size);
    a.seg_item0[nseg] = static_cast<unsigned>(items);
    items += size * (g1 - g0);
    ++nseg;
  }
  a.nseg = nseg;
  return items;
}

// Persistent grid size of the fused kernel on the current device: as many
// workgroups as can be resident at once.  Cached per device.
template <int DT>
int fused_grid() {
  static std::mutex mu;
  static int cache[2][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  int& g = cache[DT][dev];
  if (g == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    constexpr int VPG = DT == kBF16 ? SPEC_FUSED_VPG_BF16 : SPEC_FUSED_VPG_F32;
    // dynamic LDS: nch doubles; sized here for the largest row (SPEC_MAX_V fp32)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, spec::fused_kernel<kFusedBlock, DT, VPG>, kFusedBlock,
            kFusedMaxDynLds) != hipSuccess)
      return 0;
    g = cus * (per_cu > 0 ? per_cu : 1);
  }
  return g;
}

int launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

}  // namespace

extern "C" {

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG: return "SPEC_ERR_INVALID_ARG: invalid argument";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED: unsupported configuration";
    case SPEC_ERR_LAUNCH: return "SPEC_ERR_LAUNCH: kernel launch failed";
    default: return "unknown status";
  }
}

int spec_softmax_stats(const void* target_logits, const void* draft_logits, int dtype, int B,
                       int K, int V, float temperature, float* target_stats, float* draft_stats,
                       void* stream) {
  int rc = check_common(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (target_stats == nullptr || draft_stats == nullptr) return SPEC_ERR_INVALID_ARG;
  if (!aligned(target_stats, 4) || !aligned(draft_stats, 4)) return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n_tgt = static_cast<int64_t>(B) * (K + 1);
  const int64_t rows = n_tgt + static_cast<int64_t>(B) * K;
  const float c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(rows)), block(kStatsBlock);
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, kBF16, SPEC_STATS_VPG_BF16>), grid, block, 0, s,
                       target_logits, draft_logits, n_tgt, V, c2, target_stats, draft_stats);
  } else {
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, kF32, SPEC_STATS_VPG_F32>), grid, block, 0, s,
                       target_logits, draft_logits, n_tgt, V, c2, target_stats, draft_stats);
  }
  return launched();
}

int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, const float* uniforms, const float* target_stats,
                const float* draft_stats, int B, int K, int V, float temperature,
                int32_t* num_accepted, int32_t* out_tokens, float* probs, void* stream) {
  int rc = check_common(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !uniforms || !target_stats || !draft_stats || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(uniforms, 4) || !aligned(target_stats, 4) ||
      !aligned(draft_stats, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) ||
      !aligned(probs, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double invT = 1.0 / static_cast<double>(temperature);
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(B)), block(spec::kWave);
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::verify_kernel<kBF16>), grid, block, 0, s, target_logits,
                       draft_logits, draft_tokens, uniforms, target_stats, draft_stats, K, V,
                       invT, num_accepted, out_tokens, probs);
  } else {
    hipLaunchKernelGGL((spec::verify_kernel<kF32>), grid, block, 0, s, target_logits,
                       draft_logits, draft_tokens, uniforms, target_stats, draft_stats, K, V,
                       invT, num_accepted, out_tokens, probs);
  }
  return launched();
}

int spec_residual_sample(const void* target_logits, const void* draft_logits, int dtype,
                         const float* uniforms, const float* target_stats,
                         const float* draft_stats, const int32_t* num_accepted, int B, int K,
                         int V, float temperature, int32_t* out_tokens, int32_t* num_emitted,
                         void* stream) {
  int rc = check_common(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!uniforms || !target_stats || !draft_stats || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned(uniforms, 4) || !aligned(target_stats, 4) || !aligned(draft_stats, 4) ||
      !aligned(num_accepted, 4) || !aligned(out_tokens, 4) || !aligned(num_emitted, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double yscale = (1.0 / static_cast<double>(temperature)) * spec::Exp64::kScale;
  const DrawLds d = draw_lds(num_chunks(V, dtype), dtype, 2);
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(B)), block(kResidBlock);
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::residual_kernel<kResidBlock, kBF16>), grid, block, d.bytes, s,
                       target_logits, draft_logits, uniforms, target_stats, draft_stats,
                       num_accepted, K, V, yscale, d.fast, d.etab, out_tokens, num_emitted);
  } else {
    hipLaunchKernelGGL((spec::residual_kernel<kResidBlock, kF32>), grid, block, d.bytes, s,
                       target_logits, draft_logits, uniforms, target_stats, draft_stats,
                       num_accepted, K, V, yscale, d.fast, d.etab, out_tokens, num_emitted);
  }
  return launched();
}

int spec_verify_sample(const void* target_logits, const void* draft_logits, int dtype,
                       const int32_t* draft_tokens, const float* uniforms,
                       const float* target_stats, const float* draft_stats, int B, int K, int V,
                       float temperature, int32_t* num_accepted, int32_t* out_tokens,
                       float* probs, int32_t* num_emitted, void* stream) {
  int rc = check_common(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !uniforms || !target_stats || !draft_stats || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(uniforms, 4) || !aligned(target_stats, 4) ||
      !aligned(draft_stats, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) ||
      !aligned(probs, 4) || !aligned(num_emitted, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const double invT = 1.0 / static_cast<double>(temperature);
  const double yscale = invT * spec::Exp64::kScale;
  const DrawLds d = draw_lds(num_chunks(V, dtype), dtype, 2);
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(B)), block(kResidBlock);
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::verify_draw_kernel<kResidBlock, kBF16>), grid, block, d.bytes, s,
                       target_logits, draft_logits, draft_tokens, uniforms, target_stats,
                       draft_stats, K, V, invT, yscale, d.fast, d.etab, num_accepted, out_tokens,
                       probs, num_emitted);
  } else {
    hipLaunchKernelGGL((spec::verify_draw_kernel<kResidBlock, kF32>), grid, block, d.bytes, s,
                       target_logits, draft_logits, draft_tokens, uniforms, target_stats,
                       draft_stats, K, V, invT, yscale, d.fast, d.etab, num_accepted, out_tokens,
                       probs, num_emitted);
  }
  return launched();
}

int spec_greedy_verify(const void* target_logits, int dtype, const int32_t* draft_tokens, int B,
                       int K, int V, int32_t* target_argmax, int32_t* num_accepted,
                       int32_t* out_tokens, int32_t* num_emitted, void* stream) {
  // the target rows alone are checked; T plays no part in an argmax
  int rc = check_common(target_logits, target_logits, dtype, B, K, V, 1.0f);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !target_argmax || !num_accepted || !out_tokens) return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(target_argmax, 4) || !aligned(num_accepted, 4) ||
      !aligned(out_tokens, 4) || !aligned(num_emitted, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = static_cast<int64_t>(B) * (K + 1);
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::argmax_kernel<kStatsBlock, kBF16, SPEC_STATS_VPG_BF16>),
                       dim3(static_cast<unsigned>(rows)), dim3(kStatsBlock), 0, s, target_logits,
                       V, target_argmax);
  } else {
    hipLaunchKernelGGL((spec::argmax_kernel<kStatsBlock, kF32, SPEC_STATS_VPG_F32>),
                       dim3(static_cast<unsigned>(rows)), dim3(kStatsBlock), 0, s, target_logits,
                       V, target_argmax);
  }
  rc = launched();
  if (rc != SPEC_OK) return rc;
  hipLaunchKernelGGL(spec::greedy_scan_kernel, dim3(static_cast<unsigned>(B)), dim3(spec::kWave), 0,
                     s, target_argmax, draft_tokens, K, V, num_accepted, out_tokens, num_emitted);
  return launched();
}

int spec_sample(const void* logits, int dtype, int R, int V, float temperature,
                const float* uniforms, float* row_stats, int32_t* tokens, void* stream) {
  if (R < 1 || static_cast<int64_t>(R) * 2 > 0x7fffffffLL) return SPEC_ERR_INVALID_ARG;
  // the row checks of the verify calls, with the R rows as a batch of target rows
  int rc = check_common(logits, logits, dtype, R, 1, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!uniforms || !row_stats || !tokens) return SPEC_ERR_INVALID_ARG;
  if (!aligned(uniforms, 4) || !aligned(row_stats, 4) || !aligned(tokens, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  const double yscale = (1.0 / static_cast<double>(temperature)) * spec::Exp64::kScale;
  const DrawLds d = draw_lds(num_chunks(V, dtype), dtype, 1);
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, kBF16, SPEC_STATS_VPG_BF16>), dim3(R),
                       dim3(kStatsBlock), 0, s, logits, logits, static_cast<int64_t>(R), V, c2,
                       row_stats, row_stats);
  } else {
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, kF32, SPEC_STATS_VPG_F32>), dim3(R),
                       dim3(kStatsBlock), 0, s, logits, logits, static_cast<int64_t>(R), V, c2,
                       row_stats, row_stats);
  }
  rc = launched();
  if (rc != SPEC_OK) return rc;
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::sample_kernel<kResidBlock, kBF16>), dim3(R), dim3(kResidBlock),
                       d.bytes, s, logits, row_stats, uniforms, V, yscale, d.fast, d.etab, tokens);
  } else {
    hipLaunchKernelGGL((spec::sample_kernel<kResidBlock, kF32>), dim3(R), dim3(kResidBlock),
                       d.bytes, s, logits, row_stats, uniforms, V, yscale, d.fast, d.etab, tokens);
  }
  return launched();
}

int spec_filter(const void* logits, int dtype, int R, int V, float temperature, int top_k,
                float top_p, float* thresholds, float* row_stats, void* filtered, void* stream) {
  if (R < 1) return SPEC_ERR_INVALID_ARG;
  int rc = check_common(logits, logits, dtype, R, 1, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!thresholds || !aligned(thresholds, 4) || !aligned(row_stats, 4)) return SPEC_ERR_INVALID_ARG;
  if (top_k < 0 || !(top_p > 0.0f) || std::isnan(top_p)) return SPEC_ERR_INVALID_ARG;
  const int eb = elt_bytes(dtype);
  if (filtered != nullptr && filtered != logits) {
    if (!aligned(filtered, eb)) return SPEC_ERR_INVALID_ARG;
    const uintptr_t a = reinterpret_cast<uintptr_t>(logits), b = reinterpret_cast<uintptr_t>(filtered);
    const uintptr_t n = static_cast<uintptr_t>(R) * static_cast<uintptr_t>(V) * eb;
    if (a < b + n && b < a + n) return SPEC_ERR_INVALID_ARG;  // partial overlap
  }
  const int k = top_k >= V ? 0 : top_k;
  const float p = top_p >= 1.0f ? 1.0f : top_p;
  const float c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  const double yscale = (1.0 / static_cast<double>(temperature)) * spec::Exp64::kScale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::filter_kernel<kStatsBlock, kBF16, SPEC_FILTER_VPG_BF16>), dim3(R),
                       dim3(kStatsBlock), 0, s, logits, filtered, V, c2, yscale, k, p,
                       thresholds, row_stats);
  } else {
    hipLaunchKernelGGL((spec::filter_kernel<kStatsBlock, kF32, SPEC_FILTER_VPG_F32>), dim3(R),
                       dim3(kStatsBlock), 0, s, logits, filtered, V, c2, yscale, k, p,
                       thresholds, row_stats);
  }
  return launched();
}

size_t spec_verify_workspace_size(int B, int K, int V, int dtype) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return 0;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return 0;
  return fused_layout(B, K, V, dtype).total;
}

int spec_verify_fused(const void* target_logits, const void* draft_logits, int dtype,
                      const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                      float temperature, float* target_stats, float* draft_stats,
                      int32_t* num_accepted, int32_t* out_tokens, float* probs,
                      int32_t* num_emitted, void* workspace, size_t workspace_bytes,
                      void* stream) {
  int rc = check_common(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !uniforms || !target_stats || !draft_stats || !num_accepted ||
      !out_tokens || !workspace)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(uniforms, 4) || !aligned(target_stats, 4) ||
      !aligned(draft_stats, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) ||
      !aligned(probs, 4) || !aligned(num_emitted, 4) || !aligned(workspace, 256))
    return SPEC_ERR_INVALID_ARG;
  const FusedLayout L = fused_layout(B, K, V, dtype);
  if (workspace_bytes < L.total) return SPEC_ERR_INVALID_ARG;
  const int grid_max = dtype == SPEC_DTYPE_BF16 ? fused_grid<kBF16>() : fused_grid<kF32>();
  if (grid_max <= 0) return SPEC_ERR_LAUNCH;

  char* ws = static_cast<char*>(workspace);
  spec::FusedArgs a{};
  a.tgt = target_logits;
  a.dft = draft_logits;
  a.tokens = draft_tokens;
  a.uni = uniforms;
  a.tstats = target_stats;
  a.dstats = draft_stats;
  a.num_accepted = num_accepted;
  a.out_tokens = out_tokens;
  a.probs = probs;
  a.num_emitted = num_emitted;
  a.ctl = reinterpret_cast<unsigned*>(ws + L.ctl);
  a.stat_word = reinterpret_cast<unsigned long long*>(ws + L.stat_word);
  a.ready = reinterpret_cast<unsigned*>(ws + L.ready);
  a.slices_done = reinterpret_cast<unsigned*>(ws + L.slices_done);
  a.rec = reinterpret_cast<int*>(ws + L.rec);
  a.sq_part = reinterpret_cast<double*>(ws + L.sq_part);
  a.sp_part = reinterpret_cast<double*>(ws + L.sp_part);
  a.A = reinterpret_cast<double*>(ws + L.A);
  a.Bv = reinterpret_cast<double*>(ws + L.Bv);
  a.unc_n = reinterpret_cast<int*>(ws + L.unc_n);
  a.unc_idx = reinterpret_cast<int*>(ws + L.unc_idx);
  a.B = B;
  a.K = K;
  a.V = V;
  a.S = L.S;
  a.nch = L.nch;
  // A sequence's scan follows its rows by about one grid's worth of rows, so
  // that the rows are done when the scan is taken; its slices follow the scan.
  a.D1 = (grid_max + 2 * K) / (2 * K + 1) + 2;
  a.D2 = a.D1 + 2;
  const int64_t items = fused_order(B, K, L.S, a.D1, a.D2, a);
  if (items != static_cast<int64_t>(B) * (2 * K + 2 + L.S) || items >= 0xffffffffLL)
    return SPEC_ERR_INVALID_ARG;
  a.total_items = static_cast<unsigned>(items);
  const int grid = static_cast<int>(items < grid_max ? items : grid_max);
  a.c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  a.invT = 1.0 / static_cast<double>(temperature);
  a.yscale = a.invT * spec::Exp64::kScale;
  const size_t lds = static_cast<size_t>(L.nch) * sizeof(double);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::fused_kernel<kFusedBlock, kBF16, SPEC_FUSED_VPG_BF16>),
                       dim3(grid), dim3(kFusedBlock), lds, s, a);
  } else {
    hipLaunchKernelGGL((spec::fused_kernel<kFusedBlock, kF32, SPEC_FUSED_VPG_F32>),
                       dim3(grid), dim3(kFusedBlock), lds, s, a);
  }
  return launched();
}

}  // extern "C"
