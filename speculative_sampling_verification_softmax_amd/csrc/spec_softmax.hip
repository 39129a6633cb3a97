// spec_softmax.hip -- host side of the C ABI declared in include/spec_softmax.h:
// argument validation, launch configuration and launches on the caller's
// stream.  No allocation, no synchronisation, no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "spec_softmax.h"
#include "kernels.hpp"

namespace {

using spec::kBF16;
using spec::kF32;

constexpr int kStatsBlock = 256;
constexpr int kResidBlock = 512;

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
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, kBF16, 4>), grid, block, 0, s,
                       target_logits, draft_logits, n_tgt, V, c2, target_stats, draft_stats);
  } else {
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, kF32, 8>), grid, block, 0, s,
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
  const double invT = 1.0 / static_cast<double>(temperature);
  const int E = 16 / elt_bytes(dtype);
  const int nch = (V + 64 * E - 1) / (64 * E);
  const size_t lds = static_cast<size_t>(nch) * sizeof(double);
  (void)hipGetLastError();
  const dim3 grid(static_cast<unsigned>(B)), block(kResidBlock);
  if (dtype == SPEC_DTYPE_BF16) {
    hipLaunchKernelGGL((spec::residual_kernel<kResidBlock, kBF16>), grid, block, lds, s,
                       target_logits, draft_logits, uniforms, target_stats, draft_stats,
                       num_accepted, K, V, invT, out_tokens, num_emitted);
  } else {
    hipLaunchKernelGGL((spec::residual_kernel<kResidBlock, kF32>), grid, block, lds, s,
                       target_logits, draft_logits, uniforms, target_stats, draft_stats,
                       num_accepted, K, V, invT, out_tokens, num_emitted);
  }
  return launched();
}

}  // extern "C"
