// spec_softmax.hip -- host side of the C ABI declared in include/spec_softmax.h:
// argument validation, launch configuration and launches on the caller's
// stream.  No allocation, no synchronisation, no state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
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
// 512 threads: two filter workgroups share a CU, so one row's selects overlap
// another row's streaming
#ifndef SPEC_FILTER_BLOCK
#define SPEC_FILTER_BLOCK 512
#endif
#ifndef SPEC_FILTER_VPG_F32
#define SPEC_FILTER_VPG_F32 4
#endif
constexpr int kStatsBlock = SPEC_STATS_BLOCK;
constexpr int kResidBlock = 1024;
// The split final draw of spec_verify_step: block size, the largest batch it
// is used for (past 64 sequences the at most floor(256/B) parts per sequence
// save less than their hand-off costs: one 1024-thread workgroup per sequence
// draws as fast or faster), the most workgroups it launches and the most
// parts per sequence.
constexpr int kSplitDrawBlock = 512;
constexpr int kSplitDrawMaxB = 64;
constexpr int kStepDrawWGs = 256;
constexpr int kMaxParts = 64;
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

// The most workgroups of 1024 threads one launch may have (gridDim.x *
// blockDim.x must stay below 2^32): the row, sequence and row-of-R limit of
// every entry point (SPEC_MAX_ROWS in the header).
constexpr int64_t kMaxGroups = 0xffffffffLL / 1024;
static_assert(kMaxGroups == SPEC_MAX_ROWS, "header limit");

// Checks shared by all entry points.  Returns SPEC_OK or SPEC_ERR_INVALID_ARG.
// rows: the number of logit rows one workgroup each (B*(2K+1) for the verify
// calls, R for the per-row calls).
int check_common(const void* tgt, const void* dft, int dtype, int B, int K, int V, float T,
                 int64_t rows) {
  if (tgt == nullptr || dft == nullptr) return SPEC_ERR_INVALID_ARG;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return SPEC_ERR_INVALID_ARG;
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return SPEC_ERR_INVALID_ARG;
  if (!std::isfinite(T) || !(T > 0.0f)) return SPEC_ERR_INVALID_ARG;
  const int eb = elt_bytes(dtype);
  if (!aligned(tgt, eb) || !aligned(dft, eb)) return SPEC_ERR_INVALID_ARG;
  if (rows < 1 || rows > kMaxGroups) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

int check_verify(const void* tgt, const void* dft, int dtype, int B, int K, int V, float T) {
  const int64_t rows = (B < 1 || K < 1) ? 0 : static_cast<int64_t>(B) * (2 * K + 1);
  return check_common(tgt, dft, dtype, B, K, V, T, rows);
}

int check_rows(const void* logits, int dtype, int R, int V, float T) {
  return check_common(logits, logits, dtype, R, 1, V, T, R);
}

int chunk_tokens(int dtype) { return spec::kWave * (16 / elt_bytes(dtype)); }
int num_chunks(int V, int dtype) { return (V + chunk_tokens(dtype) - 1) / chunk_tokens(dtype); }
size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Every launch here has one workgroup per row, per sequence or per part of
// one; gridDim.x * blockDim.x must stay below 2^32.
bool grid_fits(int64_t groups, int block) {
  return groups >= 1 && groups * block <= static_cast<int64_t>(0xffffffffLL);
}

// Dynamic LDS of a split-draw workgroup: the shared bf16 table, the finish's
// max(ni, nch) doubles and the part's own item records.
size_t split_draw_lds(int ni, int nch, int Pd, int dtype) {
  return (dtype == SPEC_DTYPE_BF16 ? spec::kETab * sizeof(double) : 0) +
         static_cast<size_t>(std::max(ni, nch)) * sizeof(double) +
         spec::lds_items_bytes((ni + Pd - 1) / Pd);
}
constexpr size_t kSplitDrawMaxLds = 120 * 1024;

// Parts per sequence of the split draw and the workspace layout of
// spec_verify_step (offsets in bytes from the base).  Functions of the shape
// only, so that spec_verify_step_workspace_size needs no device.
struct StepLayout {
  int Pd, nch, ni;
  size_t parts_done, items, total;
};

StepLayout step_layout(int B, int K, int V, int dtype) {
  (void)K;
  StepLayout L{};
  L.nch = num_chunks(V, dtype);
  L.ni = (L.nch + spec::kDrawG - 1) / spec::kDrawG;
  L.Pd = 1;
  if (B <= kSplitDrawMaxB) {
    // As many parts as leave half the CUs busy, or one item per wave of a
    // part (8 waves) when that is more; at most one workgroup per CU
    // (measured: past 128 workgroups, parts of fewer than 8 items cost more
    // in scans, tables and records than their shorter sweeps save).
    const int per_wave = (L.ni + kSplitDrawBlock / spec::kWave - 1) / (kSplitDrawBlock / spec::kWave);
    const int want = std::max(kStepDrawWGs / 2 / B, per_wave);
    L.Pd = std::max(1, std::min(std::min(L.ni, kMaxParts), std::min(kStepDrawWGs / B, want)));
    // a part's item records must fit its LDS next to the table and W
    while (L.Pd < L.ni && split_draw_lds(L.ni, L.nch, L.Pd, dtype) > kSplitDrawMaxLds) ++L.Pd;
  }
  const size_t b = static_cast<size_t>(B);
  size_t off = 0;
  // counters first: zero before the first call, zero again after each
  L.parts_done = off; off = round256(off + b * sizeof(unsigned));
  L.items = off;
  if (L.Pd > 1) off = round256(off + b * L.ni * spec::kItemRec * sizeof(double));
  L.total = off;
  return L;
}

int launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

// The row-stats launch every verify path uses (so that all of them get the
// same bits): one workgroup per row.  Past 512 rows, 512-thread workgroups,
// four per CU: between 512 and 1024 rows they all run in one round of the
// device's 256 CUs instead of two rounds of latency-bound rows, and for more
// bf16 rows the last, partly filled round is a smaller share of the launch
// (measured ~1 % faster at B=256 K=8 V=128256 than 1024 threads).  fp32 rows
// past 1024 keep 1024 threads (their 72 VGPRs would allow only three
// 512-thread workgroups per CU); at most 512 rows also keep 1024, the row's
// latency being what counts there.
template <int DT>
void launch_stats_dt(const void* tgt, const void* dft, int64_t n_tgt, int64_t rows, int V, float c2,
                     float* tstats, float* dstats, hipStream_t s) {
  constexpr int VPG = DT == kBF16 ? SPEC_STATS_VPG_BF16 : SPEC_STATS_VPG_F32;
  const dim3 grid(static_cast<unsigned>(rows));
  if (rows > 512 && (rows <= 1024 || DT == kBF16))
    hipLaunchKernelGGL((spec::stats_kernel<512, DT, VPG>), grid, dim3(512), 0, s, tgt, dft, n_tgt,
                       V, c2, tstats, dstats);
  else
    hipLaunchKernelGGL((spec::stats_kernel<kStatsBlock, DT, VPG>), grid, dim3(kStatsBlock), 0, s,
                       tgt, dft, n_tgt, V, c2, tstats, dstats);
}

// ------------------------------------------------- no-allocation scratch
// The device memory of spec_verify_step_noalloc: one file-scope array, of
// which every GPU the library runs on holds its own copy until the process
// ends.  In host code the name `scratch` stands for the symbol only; the
// copy's device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is ever used (kernel arguments,
// the clearing below).
constexpr size_t kScratchBytes = SPEC_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(1024) void zero_scratch_kernel(uint4* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// This device's scratch address, set up by the first call on the device:
// the symbol's address, then the whole array cleared by a fill kernel on
// the caller's stream, ahead of the call's own kernels (the counters must
// start at zero; every completed call leaves them zero again).  nullptr on
// failure.
void* scratch_for_current_device(hipStream_t s) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    (void)hipGetLastError();
    hipLaunchKernelGGL(zero_scratch_kernel, dim3(256), dim3(1024), 0, s, static_cast<uint4*>(p),
                       kScratchBytes / sizeof(uint4));
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

// The two launches of spec_verify_step on an already checked call: row
// stats, then the accept scan and final draw (split over Pd workgroups per
// sequence when there are few sequences), with the counters and records in
// `ws` laid out as L says.
template <int DT>
int launch_step_dt(const void* tgt, const void* dft, const int32_t* tokens, const float* uni,
                   int B, int K, int V, float T, float* tstats, float* dstats, int32_t* nacc,
                   int32_t* out, float* probs, int32_t* nemit, char* ws, const StepLayout& L,
                   hipStream_t s) {
  const int64_t n_tgt = static_cast<int64_t>(B) * (K + 1);
  const int64_t rows = n_tgt + static_cast<int64_t>(B) * K;
  const double invT = 1.0 / static_cast<double>(T);
  const double yscale = invT * spec::Exp64::kScale;
  const float c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(T));
  (void)hipGetLastError();
  launch_stats_dt<DT>(tgt, dft, n_tgt, rows, V, c2, tstats, dstats, s);
  int rc = launched();
  if (rc != SPEC_OK) return rc;
  if (L.Pd > 1) {
    spec::SplitDraw a{};
    a.tgt = tgt;
    a.dft = dft;
    a.tokens = tokens;
    a.uni = uni;
    a.tstats = tstats;
    a.dstats = dstats;
    a.num_accepted = nacc;
    a.out_tokens = out;
    a.probs = probs;
    a.num_emitted = nemit;
    a.parts_done = reinterpret_cast<unsigned*>(ws + L.parts_done);
    a.items = reinterpret_cast<double*>(ws + L.items);
    a.K = K;
    a.V = V;
    a.P = L.Pd;
    a.ni = L.ni;
    a.nch = L.nch;
    a.etab = DT == kBF16 ? 1 : 0;
    a.invT = invT;
    a.yscale = yscale;
    const size_t lds = split_draw_lds(L.ni, L.nch, L.Pd, DT == kBF16 ? SPEC_DTYPE_BF16 : SPEC_DTYPE_F32);
    if (!grid_fits(static_cast<int64_t>(B) * L.Pd, kSplitDrawBlock)) return SPEC_ERR_INVALID_ARG;
    hipLaunchKernelGGL((spec::verify_draw_split_kernel<kSplitDrawBlock, DT>),
                       dim3(static_cast<unsigned>(B * L.Pd)), dim3(kSplitDrawBlock), lds, s, a);
  } else {
    const DrawLds d = draw_lds(L.nch, DT == kBF16 ? SPEC_DTYPE_BF16 : SPEC_DTYPE_F32, 2);
    hipLaunchKernelGGL((spec::verify_draw_kernel<kResidBlock, DT>), dim3(static_cast<unsigned>(B)),
                       dim3(kResidBlock), d.bytes, s, tgt, dft, tokens, uni, tstats, dstats, K, V,
                       invT, yscale, d.fast, d.etab, nacc, out, probs, nemit);
  }
  return launched();
}

int launch_step(const void* tgt, const void* dft, int dtype, const int32_t* tokens,
                const float* uni, int B, int K, int V, float T, float* tstats, float* dstats,
                int32_t* nacc, int32_t* out, float* probs, int32_t* nemit, char* ws,
                const StepLayout& L, hipStream_t s) {
  if (dtype == SPEC_DTYPE_BF16)
    return launch_step_dt<kBF16>(tgt, dft, tokens, uni, B, K, V, T, tstats, dstats, nacc, out,
                                 probs, nemit, ws, L, s);
  return launch_step_dt<kF32>(tgt, dft, tokens, uni, B, K, V, T, tstats, dstats, nacc, out, probs,
                              nemit, ws, L, s);
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
  int rc = check_verify(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (target_stats == nullptr || draft_stats == nullptr) return SPEC_ERR_INVALID_ARG;
  if (!aligned(target_stats, 4) || !aligned(draft_stats, 4)) return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t n_tgt = static_cast<int64_t>(B) * (K + 1);
  const int64_t rows = n_tgt + static_cast<int64_t>(B) * K;
  const float c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16)
    launch_stats_dt<kBF16>(target_logits, draft_logits, n_tgt, rows, V, c2, target_stats,
                           draft_stats, s);
  else
    launch_stats_dt<kF32>(target_logits, draft_logits, n_tgt, rows, V, c2, target_stats,
                          draft_stats, s);
  return launched();
}

int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, const float* uniforms, const float* target_stats,
                const float* draft_stats, int B, int K, int V, float temperature,
                int32_t* num_accepted, int32_t* out_tokens, float* probs, void* stream) {
  int rc = check_verify(target_logits, draft_logits, dtype, B, K, V, temperature);
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
  int rc = check_verify(target_logits, draft_logits, dtype, B, K, V, temperature);
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
  int rc = check_verify(target_logits, draft_logits, dtype, B, K, V, temperature);
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
  int rc = check_verify(target_logits, target_logits, dtype, B, K, V, 1.0f);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !target_argmax || !num_accepted || !out_tokens) return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(target_argmax, 4) || !aligned(num_accepted, 4) ||
      !aligned(out_tokens, 4) || !aligned(num_emitted, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = static_cast<int64_t>(B) * (K + 1);
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16) {
    // bf16 rows in 512-thread workgroups, four per CU: the rows' last round
    // leaves fewer slots idle (measured ~1 % faster at B=256 K=8, ~4 % at
    // B=64 K=4 V=32000 than 1024 threads)
    hipLaunchKernelGGL((spec::argmax_kernel<512, kBF16, SPEC_STATS_VPG_BF16>),
                       dim3(static_cast<unsigned>(rows)), dim3(512), 0, s, target_logits,
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
  int rc = check_rows(logits, dtype, R, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!uniforms || !row_stats || !tokens) return SPEC_ERR_INVALID_ARG;
  if (!aligned(uniforms, 4) || !aligned(row_stats, 4) || !aligned(tokens, 4))
    return SPEC_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float c2 = static_cast<float>(1.4426950408889634074 / static_cast<double>(temperature));
  const double yscale = (1.0 / static_cast<double>(temperature)) * spec::Exp64::kScale;
  const DrawLds d = draw_lds(num_chunks(V, dtype), dtype, 1);
  (void)hipGetLastError();
  if (dtype == SPEC_DTYPE_BF16 && d.fast && d.etab) {
    // one read per row: the statistics come out of the draw's own sweep
    // 512 threads (78 VGPRs, ~52 KB of LDS): three rows share a CU, so one
    // row's table fill and finish overlap the others' sweeps
    hipLaunchKernelGGL((spec::sample_onepass_kernel<512>), dim3(R), dim3(512), d.bytes, s, logits,
                       uniforms, V, yscale, row_stats, tokens);
    return launched();
  }
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
  int rc = check_rows(logits, dtype, R, V, temperature);
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
  if (dtype == SPEC_DTYPE_BF16)
    hipLaunchKernelGGL((spec::filter_kernel<SPEC_FILTER_BLOCK, kBF16, SPEC_FILTER_VPG_BF16>),
                       dim3(R), dim3(SPEC_FILTER_BLOCK), 0, s, logits, filtered, V, c2, yscale, k,
                       p, thresholds, row_stats);
  else
    hipLaunchKernelGGL((spec::filter_kernel<SPEC_FILTER_BLOCK, kF32, SPEC_FILTER_VPG_F32>),
                       dim3(R), dim3(SPEC_FILTER_BLOCK), 0, s, logits, filtered, V, c2, yscale, k,
                       p, thresholds, row_stats);
  return launched();
}

size_t spec_verify_step_workspace_size(int B, int K, int V, int dtype) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return 0;
  if (dtype != SPEC_DTYPE_F32 && dtype != SPEC_DTYPE_BF16) return 0;
  if (static_cast<int64_t>(B) * (2 * K + 1) > kMaxGroups) return 0;
  return step_layout(B, K, V, dtype).total;
}

int spec_verify_step(const void* target_logits, const void* draft_logits, int dtype,
                     const int32_t* draft_tokens, const float* uniforms, int B, int K, int V,
                     float temperature, float* target_stats, float* draft_stats,
                     int32_t* num_accepted, int32_t* out_tokens, float* probs,
                     int32_t* num_emitted, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int rc = check_verify(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !uniforms || !target_stats || !draft_stats || !num_accepted ||
      !out_tokens || !workspace)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(uniforms, 4) || !aligned(target_stats, 4) ||
      !aligned(draft_stats, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) ||
      !aligned(probs, 4) || !aligned(num_emitted, 4) || !aligned(workspace, 256))
    return SPEC_ERR_INVALID_ARG;
  const StepLayout L = step_layout(B, K, V, dtype);
  if (workspace_bytes < L.total) return SPEC_ERR_INVALID_ARG;
  return launch_step(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V,
                     temperature, target_stats, draft_stats, num_accepted, out_tokens, probs,
                     num_emitted, static_cast<char*>(workspace), L,
                     static_cast<hipStream_t>(stream));
}

int spec_verify_step_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* draft_tokens, const float* uniforms, int B, int K,
                             int V, float temperature, float* target_stats, float* draft_stats,
                             int32_t* num_accepted, int32_t* out_tokens, float* probs,
                             int32_t* num_emitted, void* stream) {
  int rc = check_verify(target_logits, draft_logits, dtype, B, K, V, temperature);
  if (rc != SPEC_OK) return rc;
  if (!draft_tokens || !uniforms || !target_stats || !draft_stats || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned(draft_tokens, 4) || !aligned(uniforms, 4) || !aligned(target_stats, 4) ||
      !aligned(draft_stats, 4) || !aligned(num_accepted, 4) || !aligned(out_tokens, 4) ||
      !aligned(probs, 4) || !aligned(num_emitted, 4))
    return SPEC_ERR_INVALID_ARG;
  const StepLayout L = step_layout(B, K, V, dtype);
  if (L.total > kScratchBytes) return SPEC_ERR_UNSUPPORTED;  // past the static scratch
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = scratch_for_current_device(s);
  if (ws == nullptr) return SPEC_ERR_LAUNCH;
  return launch_step(target_logits, draft_logits, dtype, draft_tokens, uniforms, B, K, V,
                     temperature, target_stats, draft_stats, num_accepted, out_tokens, probs,
                     num_emitted, static_cast<char*>(ws), L, s);
}

#ifdef SPEC_PHASE_STAMPS
// Measurement builds only (libspec_phases.so): copy the phase stamps the
// kernels recorded to host memory -- which 0: stats_kernel's [8192][2], 1:
// the draw kernels' [8192][8], both uint64 -- or zero them.  Synchronous;
// call them with no launch of this library in flight.
int spec_phase_stamps(void* host, size_t bytes, int which) {
  const size_t have = which == 0 ? sizeof(spec::stamps_rows) : sizeof(spec::stamps_draw);
  if (host == nullptr || (which != 0 && which != 1) || bytes > have) return SPEC_ERR_INVALID_ARG;
  const hipError_t e =
      which == 0 ? hipMemcpyFromSymbol(host, HIP_SYMBOL(spec::stamps_rows), bytes, 0,
                                       hipMemcpyDeviceToHost)
                 : hipMemcpyFromSymbol(host, HIP_SYMBOL(spec::stamps_draw), bytes, 0,
                                       hipMemcpyDeviceToHost);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

int spec_phase_clear(void) {
  static unsigned long long zr[spec::kStampWGs][2];  // zero (static storage)
  static unsigned long long zd[spec::kStampWGs][8];
  if (hipMemcpyToSymbol(HIP_SYMBOL(spec::stamps_rows), zr, sizeof(zr), 0,
                        hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(spec::stamps_draw), zd, sizeof(zd), 0,
                        hipMemcpyHostToDevice) != hipSuccess)
    return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}
#endif

}  // extern "C"
