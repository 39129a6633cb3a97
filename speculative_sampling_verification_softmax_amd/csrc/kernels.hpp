// kernels.hpp -- the verify kernels for gfx950 and the device functions they
// share.
//
//   stats_kernel     one workgroup per logit row: max m and s = sum exp((z-m)/T)
//   verify_kernel    one wave per sequence: q, p at the drafted tokens, accept
//                    tests, first rejection
//   residual_kernel  one workgroup per sequence: residual (or bonus) weights on
//                    the row(s) at the first rejection and the inverse-CDF draw
//
// What is computed: wikillm.com card for arXiv 2302.01318, Method
// ("Modified rejection sampling", paper sec. 4.2; "Algorithm: Speculative
// Sampling (SpS)", alg. 2 steps 2-4; "Decoding transforms") and Pitfalls.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace spec {

// ============================================================= phase stamps
//
// Measurement builds only (-DSPEC_PHASE_STAMPS, libspec_phases.so): thread 0
// of workgroup g < kStampWGs records the device's 100 MHz real-time counter
// as it passes phase k, in stamps_rows[g][k] (stats_kernel: 0 start, 1 end)
// or stamps_draw[g][k] (the draw kernels' phases, listed where they are
// taken).  Every launch overwrites its workgroups' entries.  A time taken
// early and stored late (SPEC_STAMP_NOW, SPEC_STAMP_AT) stays in scalar
// registers meanwhile, so the streaming loop keeps its vector registers.  In
// the library the macros expand to nothing.
#ifdef SPEC_PHASE_STAMPS
constexpr int kStampWGs = 8192;
__device__ unsigned long long stamps_rows[kStampWGs][2];
__device__ unsigned long long stamps_draw[kStampWGs][8];
#define SPEC_STAMP_NOW() __builtin_amdgcn_s_memrealtime()
#define SPEC_STAMP_AT(arr, k, t)                            \
  do {                                                      \
    if (threadIdx.x == 0 && blockIdx.x < ::spec::kStampWGs) \
      ::spec::arr[blockIdx.x][k] = (t);                     \
  } while (0)
#define SPEC_STAMP(arr, k) SPEC_STAMP_AT(arr, k, SPEC_STAMP_NOW())
#else
#define SPEC_STAMP_NOW() 0ull
#define SPEC_STAMP_AT(arr, k, t) ((void)(t))
#define SPEC_STAMP(arr, k) ((void)0)
#endif

// ================================================================ row stats
//
// HBM-bound streaming reduction of one row.  The row is split into an
// unaligned head, a body of 16-byte vectors (8 bf16 or 4 fp32 per load, fully
// coalesced across the wave) and a tail.  Each thread takes groups of VPG
// vectors; the next group's loads are issued before the current group is
// reduced.
//
// Per thread the sum is kept against an integer shift k = rint(max * c2)
// (c2 = log2(e)/T): every term is exp2(fma(x, c2, -k)), one fused multiply-add
// (x*c2 is exact inside it, one rounding) and one exp2, and when the max grows
// the running fp64 sum is rescaled by an exact power of two.  The group's
// terms are summed in fp32, the running sum in fp64.  At the end the thread
// sums are brought to the row's shift k_r by exact powers of two, summed in
// fp64 and multiplied by 2^(k_r - m*c2) (|k_r - m*c2| <= 1/2, m*c2 exact in
// fp64), giving s = sum exp2((x - m) * c2).  Relative error of s: a few 1e-7.
//
// Rows whose max has |m*c2| >= 2^22 (logits beyond ~2.9e6*T) cannot use an
// fp32 integer shift; their s comes from a second pass that takes the
// difference x - m first (row_stats_wide).

constexpr float kShiftMax = 4194304.f;  // 2^22

struct RowAcc {
  float m = -__builtin_huge_valf();  // max of the values seen
  float k = -kShiftMax;              // integer shift, rint(m*c2) clamped to +-2^22
  double s = 0.0;                    // sum of exp2(x*c2 - k)
};

template <int N>
__device__ __forceinline__ float group_max(const float (&x)[N]) {
  float g = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) g = fmaxf(g, x[i]);
  return g;
}

// Sum of exp2(fma(x, c2, -k)) over the group, pairwise.
template <int N>
__device__ __forceinline__ float group_exp_sum(const float (&x)[N], float c2, float k) {
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = __builtin_amdgcn_exp2f(fmaf(x[i], c2, -k));
#pragma unroll
  for (int w = 1; w < N; w *= 2)
#pragma unroll
    for (int i = 0; i + w < N; i += 2 * w) t[i] = t[i] + t[i + w];
  return t[0];
}

template <int N>
__device__ __forceinline__ void fold(RowAcc& a, const float (&x)[N], float c2) {
  const float mn = fmaxf(a.m, group_max(x));
  // -inf (nothing finite seen) and very negative maxima clamp to -2^22: the
  // terms are then 0 or negligible against any row whose max is in range.
  const float kn = rintf(__builtin_amdgcn_fmed3f(mn * c2, -kShiftMax, kShiftMax));
  const float gs = group_exp_sum(x, c2, kn);
  a.s = ldexp(a.s, static_cast<int>(a.k - kn)) + static_cast<double>(gs);
  a.m = mn;
  a.k = kn;
}

// The old-style accumulator for rows with huge logits: terms exp2((x - m)*c2)
// with the difference taken first, the running sum rescaled when m grows.
struct WideAcc {
  float m = -__builtin_huge_valf();
  double s = 0.0;
};

template <int N>
__device__ __forceinline__ void fold_wide(WideAcc& a, const float (&x)[N], float c2) {
  const float mn = fmaxf(a.m, group_max(x));
  const float ms = (mn == -__builtin_huge_valf()) ? 0.f : mn;
  float gs = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) gs = gs + __builtin_amdgcn_exp2f((x[i] - ms) * c2);
  const float scale = (mn == a.m) ? 1.f : __builtin_amdgcn_exp2f((a.m - ms) * c2);
  a.s = fma(a.s, static_cast<double>(scale), static_cast<double>(gs));
  a.m = mn;
}

// Geometry of one row: head elements before the first 16-byte boundary, nvec
// whole vectors, then the tail.
template <int DT>
struct RowGeom {
  int head, nvec, tail0;
  __device__ __forceinline__ RowGeom(const char* row, int V) {
    constexpr int EB = Elt<DT>::bytes;
    const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
    head = static_cast<int>(((16 - (addr & 15)) & 15) / EB);
    if (head > V) head = V;
    nvec = (V - head) / (16 / EB);
    tail0 = head + nvec * (16 / EB);
  }
};

// Second pass for rows with |m*c2| >= 2^22 (block-uniform; rare).
template <int BLOCK, int DT>
__device__ __noinline__ double row_stats_wide(const char* row, int V, float c2, float m,
                                              float* red_f, double* red_d) {
  constexpr int EPV = 16 / Elt<DT>::bytes;
  const int tid = threadIdx.x;
  const RowGeom<DT> G(row, V);
  WideAcc acc;
  for (int i = tid; i < G.head; i += BLOCK) {
    float x[1] = {logit_f32<DT>(row, i)};
    fold_wide(acc, x, c2);
  }
  for (int i = G.tail0 + tid; i < V; i += BLOCK) {
    float x[1] = {logit_f32<DT>(row, i)};
    fold_wide(acc, x, c2);
  }
  const uint4* vp = reinterpret_cast<const uint4*>(row + static_cast<int64_t>(G.head) *
                                                             Elt<DT>::bytes);
  for (int i = tid; i < G.nvec; i += BLOCK) {
    float x[EPV];
    unpack16<DT>(vp[i], x);
    fold_wide(acc, x, c2);
  }
  const float scale = (acc.m == m) ? 1.f : __builtin_amdgcn_exp2f((acc.m - m) * c2);
  return block_sum<BLOCK>(acc.s * static_cast<double>(scale), red_d);
}

// VPG vectors of a row body at vector indices i0 + u*BLOCK, u < VPG, as fp32.
// The body is addressed through a buffer resource: the per-thread offset is
// a fixed VGPR and the group offset a scalar, so the loads cost no vector
// address arithmetic.
// Cache policy of a buffer load: default, or non-temporal for data that is
// read once (the streamed rows of the single-pass kernels: keeping them out
// of the caches' way lets the stream run at ~7 TB/s instead of ~6.2 TB/s).
constexpr int kLoadDefault = 0;
constexpr int kLoadStream = 2;  // nt

template <int BLOCK, int DT, int VPG, int AUX>
__device__ __forceinline__ void body_load(__amdgpu_buffer_rsrc_t rs, int vo, int i0,
                                          uint4 (&v)[VPG]) {
#pragma unroll
  for (int u = 0; u < VPG; ++u) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, (i0 + u * BLOCK) * 16, AUX);
    v[u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int DT, int VPG>
__device__ __forceinline__ void body_unpack(const uint4 (&v)[VPG],
                                            float (&x)[VPG * (16 / Elt<DT>::bytes)]) {
  constexpr int EPV = 16 / Elt<DT>::bytes;
#pragma unroll
  for (int u = 0; u < VPG; ++u) {
    float xu[EPV];
    unpack16<DT>(v[u], xu);
#pragma unroll
    for (int e = 0; e < EPV; ++e) x[u * EPV + e] = xu[e];
  }
}

// Word 3 of a raw buffer resource on gfx9-family parts (untyped dword access).
constexpr int kBufWord3 = 0x00020000;

// Streams a row body of nvec 16-byte vectors (body 16-byte aligned) through
// the block in groups: thread tid's group `it` holds vectors
// it*BLOCK*VPG + tid + u*BLOCK, u < VPG, unpacked to fp32 in x[u*EPV + e].
// The next group's loads are issued before f(x, i0) reduces the current one
// (i0 = the group's first vector index for this thread); the last, partial
// group reads vectors past nvec as -inf.  `body` must be uniform.
template <int BLOCK, int DT, int VPG, int AUX = kLoadDefault, typename F>
__device__ __forceinline__ void stream_body(const char* body, int nvec, F f) {
  constexpr int EPV = 16 / Elt<DT>::bytes;
  constexpr int STEP = BLOCK * VPG;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(body), static_cast<short>(0), nvec * 16, kBufWord3);
  const int vo = tid * 16;
  const int nfull = nvec / STEP;
  if (nfull > 0) {
    uint4 v[VPG];
    body_load<BLOCK, DT, VPG, AUX>(rs, vo, 0, v);
    for (int it = 1; it < nfull; ++it) {
      float x[VPG * EPV];
      body_unpack<DT, VPG>(v, x);
      body_load<BLOCK, DT, VPG, AUX>(rs, vo, it * STEP, v);  // next group in flight
      f(x, (it - 1) * STEP + tid);
    }
    float x[VPG * EPV];
    body_unpack<DT, VPG>(v, x);
    f(x, (nfull - 1) * STEP + tid);
  }
  if (nfull * STEP < nvec) {  // one partial group: vectors past nvec read as -inf
    const int i0 = nfull * STEP + tid;
    // every load issued before any is used (one round trip, not VPG): a lane
    // whose vector lies past nvec loads the row's last vector instead (its
    // offset entirely in the range-checked vector operand) and drops it
    uint4 v[VPG];
#pragma unroll
    for (int u = 0; u < VPG; ++u) {
      const int vi = min(i0 + u * BLOCK, nvec - 1);
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, vi * 16, 0, AUX);
      v[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    float x[VPG * EPV];
#pragma unroll
    for (int u = 0; u < VPG; ++u) {
      float xu[EPV];
      unpack16<DT>(v[u], xu);
      const bool in = i0 + u * BLOCK < nvec;
#pragma unroll
      for (int e = 0; e < EPV; ++e) x[u * EPV + e] = in ? xu[e] : -__builtin_huge_valf();
    }
    f(x, i0);
  }
}

// {m, s} of one row, returned to every thread of the block.  A row with no
// finite maximum gets s = NaN (NaN logits already make s NaN).  `row` must be
// uniform across the block.
template <int BLOCK, int DT, int VPG, int AUX = kLoadStream>
__device__ __forceinline__ void row_stats(const char* row, int V, float c2, float* red_f,
                                          double* red_d, float& m_out, float& s_out) {
  constexpr int EPV = 16 / Elt<DT>::bytes;
  constexpr int STEP = BLOCK * VPG;
  const int tid = threadIdx.x;
  const RowGeom<DT> G(row, V);

  RowAcc acc;
  if (tid < G.head) {
    float x[1] = {logit_f32<DT>(row, tid)};
    fold(acc, x, c2);
  }
  if (tid < V - G.tail0) {
    float x[1] = {logit_f32<DT>(row, G.tail0 + tid)};
    fold(acc, x, c2);
  }
  const char* body = row + static_cast<int64_t>(G.head) * Elt<DT>::bytes;
  stream_body<BLOCK, DT, VPG, AUX>(body, G.nvec,
                                   [&](const float(&x)[VPG * EPV], int) { fold(acc, x, c2); });

  const float m = block_max<BLOCK>(acc.m, red_f);
  float sf;
  if (!__builtin_isfinite(m)) {
    sf = __builtin_nanf("");
  } else if (fabsf(m * c2) < kShiftMax) {
    const float kr = rintf(m * c2);
    const double s = block_sum<BLOCK>(ldexp(acc.s, static_cast<int>(acc.k - kr)), red_d);
    const double t = static_cast<double>(kr) - static_cast<double>(m) * static_cast<double>(c2);
    sf = static_cast<float>(s * exp2(t));
  } else {
    sf = static_cast<float>(row_stats_wide<BLOCK, DT>(row, V, c2, m, red_f, red_d));
  }
  m_out = m;
  s_out = sf;
}

template <int BLOCK, int DT, int VPG>
__global__ __launch_bounds__(BLOCK) void stats_kernel(const void* __restrict__ tgt,
                                                      const void* __restrict__ dft,
                                                      int64_t n_tgt_rows, int V, float c2,
                                                      float* __restrict__ tstats,
                                                      float* __restrict__ dstats) {
  __shared__ float red_f[BLOCK / kWave];
  __shared__ double red_d[BLOCK / kWave];
  [[maybe_unused]] const unsigned long long t_start = SPEC_STAMP_NOW();
  int64_t r = blockIdx.x;
  const char* row;
  float* out;
  if (r < n_tgt_rows) {
    row = static_cast<const char*>(tgt) + r * static_cast<int64_t>(V) * Elt<DT>::bytes;
    out = tstats + 2 * r;
  } else {
    r -= n_tgt_rows;
    row = static_cast<const char*>(dft) + r * static_cast<int64_t>(V) * Elt<DT>::bytes;
    out = dstats + 2 * r;
  }
  float m, s;
  row_stats<BLOCK, DT, VPG>(row, V, c2, red_f, red_d, m, s);
  if (threadIdx.x == 0) {
    out[0] = m;
    out[1] = s;
  }
  SPEC_STAMP_AT(stamps_rows, 0, t_start);
  SPEC_STAMP(stamps_rows, 1);
}

// =================================================================== verify
//
// One wave per sequence; lane t runs accept test t.  q_t(x_t) and p_t(x_t)
// are formed in fp64 from the stored logit and the row stats, and the test
// is u < min(1, q/p) written as (u < 1) && (u*p < q), which also covers
// p = 0 (accept iff q > 0).  The first rejection is the lowest set bit of
// the wave's reject ballot.  Must be called by all 64 lanes of one wave.
// XB: the stats come from other workgroups of the same launch (handoff loads,
// see device_common.hpp).

template <int DT, bool XB>
__device__ int verify_seq(int64_t b, const void* tgt, const void* dft, const int32_t* tokens,
                           const float* uni, const float* ts_b, const float* ds_b, int K,
                           int V, double invT, int32_t* num_accepted, int32_t* out_tokens,
                           float* probs, bool skip_final, bool write = true) {
  // ts_b: this sequence's target stats [K+1][2]; ds_b: its draft stats [K][2].
  // skip_final: leave out_tokens[b][n] to the final draw (written elsewhere).
  // write: store num_accepted, out_tokens and probs (false: only return n).
  const int t = lane_id();
  const int64_t K1 = K + 1;
  bool valid = true;
  bool reject = false;
  double q = 0.0, p = 0.0;
  if (t < K) {
    const int x = tokens[b * K + t];
    const int64_t rq = b * K1 + t, rp = b * K + t;
    const float mq = ld<XB>(&ts_b[2 * t]), sq = ld<XB>(&ts_b[2 * t + 1]);
    const float mp = ld<XB>(&ds_b[2 * t]), sp = ld<XB>(&ds_b[2 * t + 1]);
    valid = row_ok(mq, sq) && row_ok(mp, sp) && x >= 0 && x < V;
    if (valid) {
      const double zq = logit_f32<DT>(tgt, rq * V + x);
      const double zp = logit_f32<DT>(dft, rp * V + x);
      q = exp((zq - static_cast<double>(mq)) * invT) / static_cast<double>(sq);
      p = exp((zp - static_cast<double>(mp)) * invT) / static_cast<double>(sp);
      const double u = uni[b * K1 + t];
      reject = !((u < 1.0) && (u * p < q));
    }
  }
  if (t == 0)  // the bonus row is part of the sequence too
    valid = valid && row_ok(ld<XB>(&ts_b[2 * K]), ld<XB>(&ts_b[2 * K + 1]));
  const bool all_valid = __all(valid);
  const unsigned long long rej = __ballot(reject);
  const int n = !all_valid ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : K);
  if (!write) return n;
  if (t == 0) num_accepted[b] = n;
  for (int pos = t; pos <= K; pos += kWave)
    if (!(skip_final && pos == n)) out_tokens[b * K1 + pos] = (pos < n) ? tokens[b * K + pos] : -1;
  if (probs != nullptr && t < K) {
    const float nan = __builtin_nanf("");
    probs[2 * (b * K + t)] = all_valid ? static_cast<float>(q) : nan;
    probs[2 * (b * K + t) + 1] = all_valid ? static_cast<float>(p) : nan;
  }
  return n;
}

template <int DT>
__global__ __launch_bounds__(kWave) void verify_kernel(
    const void* __restrict__ tgt, const void* __restrict__ dft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uni,
    const float* __restrict__ tstats, const float* __restrict__ dstats, int K, int V,
    double invT, int32_t* __restrict__ num_accepted, int32_t* __restrict__ out_tokens,
    float* __restrict__ probs) {
  const int64_t b = blockIdx.x;
  (void)verify_seq<DT, false>(b, tgt, dft, tokens, uni, tstats + 2 * b * (K + 1),
                              dstats + 2 * b * K, K, V, invT, num_accepted, out_tokens, probs,
                              false);
}

// ================================================================= residual
//
// Weights at position n = num_accepted[b] (all fp64, e(x) = exp((z(x)-m)/T)):
//   residual  w(x) = max(0, e_q(x)/S_q - e_p(x)/S_p)
//   fallback  w(x) = e_q(x) when the residual has no mass
//   bonus     w(x) = e_q(x) on row K
// (the draw is invariant to a common scale, so bonus/fallback weights stay
// unnormalised) and x* = min{x : sum_{y<=x} w(y) > u * sum_y w(y)}.
//
// The row is cut into chunks of 64*E tokens (E per lane, contiguous per lane,
// lanes contiguous); one wave owns a chunk at a time and loads the next one
// while it computes the current one.
//
// For a residual every e_q is taken times the draft row's fp32 normaliser
// s~_p from the stats and every e_p times s~_q (the factors cq, cp of
// DrawRows; per-row tables hold the products), so that e_q >= e_p reads as
// q >= p up to the stats' rounding.  With the table both rows share, e is
// exp(z/T) with no maximum and no factor, and the balance moves into the
// sign test's constants instead (rho of DrawRows).  Either way the draw is
// unchanged: q = e_q/S_q with S_q the sum of the same values.
//
// Fast path, one sweep over the row(s): every token's e_q, e_p (fp64 table
// exponential) go into the normalisers S_q, S_p; the sign of the residual is
// decided with a relative margin kDelta: e_q >= (1+kDelta) rho e_p is
// certainly positive, e_q <= (1-kDelta) rho e_p certainly not.
// Tokens clearly positive add e_q and e_p to the chunk's sums A_c, B_c;
// tokens clearly negative add nothing; the few inside the margin are recorded
// (up to kUncMax per chunk) and resolved once S_q, S_p are exact.  Then
// W_c = A_c/S_q - B_c/S_p (+ the resolved tokens).  If the exact ratio
// S_q/S_p falls outside rho by more than kDelta/4, a chunk records more
// uncertain tokens than it can hold, or the residual has no mass, the draw
// takes the exact slow path instead: normalisers first, then every chunk's
// weights, two sweeps.
//
// Draw: running prefix over chunk totals in chunk order (wave 0), the first
// chunk whose inclusive prefix exceeds u*S_w, then that chunk's weights are
// re-derived token by token with the exact definition, and the first lane and
// token whose cumulative weight exceeds the target are chosen.  A token of
// weight 0 is never chosen; if rounding leaves no crossing, the last token of
// positive weight is chosen, as the oracle does.

enum : int { kModeResidual = 0, kModeBonus = 1 };
constexpr int kUncMax = 2;
constexpr double kDelta = 1.0 / 65536.0;
constexpr int kDrawG = 2;  // chunks per item of the fast sweep

// Dynamic LDS of the fast sweep for a row of nch chunks: per item, the
// finish's total W, then four row totals of each of A, Bv, Lq, Lp, unc_n,
// kUncMax unc_q and kUncMax unc_p (LdsItems).
constexpr size_t draw_fast_lds(int nch) {
  return static_cast<size_t>((nch + kDrawG - 1) / kDrawG) *
         (17 * sizeof(double) + (1 + 2 * kUncMax) * sizeof(int));
}

// -(1 + kDelta) and -(1 - kDelta) (their low words are 0) as wave-uniform
// registers, so that fma(e_p, k, e_q) is one v_fma_f64 (a literal operand
// would make it a copy and a v_fmac).
static_assert(-(1.0 + kDelta) == -1.0000152587890625 && -(1.0 - kDelta) == -0.9999847412109375,
              "the high words below encode -(1 +- 2^-16)");
__device__ __forceinline__ double uniform_margin(bool upper) {
  unsigned h;
  if (upper)
    asm("s_mov_b32 %0, 0xbff00010" : "=s"(h));
  else
    asm("s_mov_b32 %0, 0xbfefffe0" : "=s"(h));
  return __hiloint2double(static_cast<int>(h), 0);
}

struct DrawRows {
  const void* qrow;
  const void* prow;
  int V;
  int mode;
  bool aligned;       // both rows start on 16-byte boundaries
  double yscale;      // (1/T) * 256/ln2
  double mq, mp;      // row maxima (exact stored logits)
  double cq, cp;      // factors on e_q and e_p: s~_p and s~_q for a residual, else 1
  const double* et;   // bf16 exponential table of the q row in LDS, or null
  const double* etp;  // ... of the p row (the same table when the rows share one)
  // the sign test's constants -(1 + kDelta) * rho, -(1 - kDelta) * rho, and rho,
  // the ratio e_q / e_p takes at q = p up to the fp32 normalisers (1 when the
  // factors cq, cp already balance the two rows)
  double k_hi, k_lo, rho;
};

// The rows at position n of sequence b and their stats.  Returns false when a
// row there defines no distribution.
template <int DT>
__device__ __forceinline__ bool make_draw_rows(int64_t b, int n, int K, int V, const void* tgt,
                                               const void* dft, float mq, float sq, float mp,
                                               float sp, double yscale, DrawRows& R) {
  constexpr int EB = Elt<DT>::bytes;
  const bool resid = n < K;
  const int64_t rq = b * (K + 1) + n, rp = resid ? b * K + n : 0;
  R.qrow = static_cast<const char*>(tgt) + rq * static_cast<int64_t>(V) * EB;
  R.prow = static_cast<const char*>(dft) + rp * static_cast<int64_t>(V) * EB;
  R.V = V;
  R.mode = resid ? kModeResidual : kModeBonus;
  R.aligned =
      ((reinterpret_cast<uintptr_t>(R.qrow) | reinterpret_cast<uintptr_t>(R.prow)) & 15) == 0;
  R.yscale = yscale;
  R.mq = mq;
  R.mp = resid ? mp : 0.0;
  R.cq = resid ? sp : 1.0;
  R.cp = resid ? sq : 1.0;
  R.et = nullptr;
  R.etp = nullptr;
  R.k_hi = uniform_margin(true);
  R.k_lo = uniform_margin(false);
  R.rho = 1.0;
  return row_ok(mq, sq) && (!resid || row_ok(mp, sp));
}

// e(x) of one token: exp((z - m)/T) = 2^((z - m) * yscale * ln2/256).  The
// difference is taken first: it is exact (or correctly rounded) whatever the
// magnitude of the logits, so the maximum gets exactly exp(0) = 1.
__device__ __forceinline__ double tok_exp(float z, double yscale, double m, const double* tab) {
  return exp64_scaled((static_cast<double>(z) - m) * yscale, tab);
}

// e of a token of the q row (P false) or the p row of R, times its factor.
template <bool P>
__device__ __forceinline__ double row_tok_exp(const DrawRows& R, float z, const double* tab) {
  return tok_exp(z, R.yscale, P ? R.mp : R.mq, tab) * (P ? R.cp : R.cq);
}

// bf16 rows hold few distinct values: every z with 2^-7 <= |z| < 2^6 is one
// of 2 * 13 * 128 codes.  A workgroup that draws from a row can fill a table
// of row_tok_exp over those codes once (kETab doubles per row: a block of
// kETabSign entries per sign, the codes in order and then 0s) and look tokens
// up instead of evaluating the exponential; other values are computed.  Every
// use of a code's value (sweep, uncertain tokens, in-chunk draw, slow path)
// goes through the same lookup, so each code has one value.  With
// t = |code| - kETabLo (unsigned), a code's entry is sign * kETabSign +
// min(t, kETabN): every code outside the table, -inf included, lands on a 0.
constexpr unsigned kETabLo = 120u << 7;  // bf16 bits of 2^-7, sign cleared
constexpr unsigned kETabN = 13u << 7;    // codes per sign: exponents 2^-7 .. 2^5
constexpr unsigned kETabSign = 2048;     // entries per sign block (a power of two)
constexpr int kETab = 2 * static_cast<int>(kETabSign);  // doubles per row

// Fills the tables of `rows` rows (1 or 2: the q row of R, then its p row)
// at et, kETab doubles apart: row by row (m stays wave-uniform), the kETabN
// codes of each sign block spread evenly over the workgroup, then each
// block's 0 (entries past it are never read).
template <int BLOCK>
__device__ __forceinline__ void fill_row_exp_tables(double* et, int rows, const DrawRows& R,
                                                    const double* tab) {
  constexpr unsigned NC = 2 * kETabN;        // codes per row
  constexpr int J = (NC + BLOCK - 1) / BLOCK;  // entries per thread and row
  // all of a thread's entries of a row at once: independent exponentials
  for (int r = 0; r < rows; ++r) {
    double v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const unsigned k = threadIdx.x + j * BLOCK;
      const unsigned sg = k >= kETabN ? 1u : 0u, i = k - sg * kETabN;
      const float z = __uint_as_float(((kETabLo + i) | (sg << 15)) << 16);
      v[j] = r == 0 ? row_tok_exp<false>(R, z, tab) : row_tok_exp<true>(R, z, tab);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const unsigned k = threadIdx.x + j * BLOCK;
      const unsigned sg = k >= kETabN ? 1u : 0u, i = k - sg * kETabN;
      if (k < NC) et[r * kETab + sg * kETabSign + i] = v[j];
    }
  }
  if (threadIdx.x < 2 * rows)
    et[(threadIdx.x >> 1) * kETab + (threadIdx.x & 1) * kETabSign + kETabN] = 0.0;
}

// The table both rows of a draw can share: exp(z/T) over the codes, no row
// maximum (so it can be filled before the drawn rows are known), by threads
// first .. blockDim.x-1, with 1/T = yscale * ln2/256 formed the same way
// wherever it is filled.  Usable for rows whose maxima have |m|/T <= 300
// (draw_rows_share_table): then no entry a row looks up overflows, the row's
// own maximum stays a normal double, and only entries more than ~400 nats
// below it (weights below 1e-170 of the row's top) can lose precision.
constexpr double kSharedTableMax = 300.0;
template <int BLOCK>
__device__ __forceinline__ void fill_shared_exp_table(double* et, double yscale, int first) {
  constexpr int NC = 2 * static_cast<int>(kETabN);
  constexpr int J = (NC + (BLOCK - kWave) - 1) / (BLOCK - kWave);
  const int nt = BLOCK - first, t0 = static_cast<int>(threadIdx.x) - first;
  const double invT = yscale / Exp64::kScale;
  double v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {  // independent exponentials
    const int k = t0 + j * nt;
    const int sg = k >= static_cast<int>(kETabN) ? 1 : 0, i = k - sg * static_cast<int>(kETabN);
    const float z = __uint_as_float(((kETabLo + i) | (static_cast<unsigned>(sg) << 15)) << 16);
    v[j] = k < NC ? exp(static_cast<double>(z) * invT) : 0.0;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = t0 + j * nt;
    const int sg = k >= static_cast<int>(kETabN) ? 1 : 0, i = k - sg * static_cast<int>(kETabN);
    if (k < NC) et[sg * static_cast<int>(kETabSign) + i] = v[j];
  }
  if (t0 >= 0 && t0 < 2) et[t0 * static_cast<int>(kETabSign) + static_cast<int>(kETabN)] = 0.0;
}

// Whether the rows of R may share the table above.
__device__ __forceinline__ bool draw_rows_share_table(const DrawRows& R) {
  const double invT = R.yscale / Exp64::kScale;
  return fabs(R.mq) * invT <= kSharedTableMax &&
         (R.mode != kModeResidual || fabs(R.mp) * invT <= kSharedTableMax);
}

// Switch R to the shared table at et: e_q = exp(z_q/T), e_p = exp(z_p/T)
// (no maxima, no factors), with the sign test's balance
// rho = exp((m_q - m_p)/T) * s~_q / s~_p -- the ratio e_q / e_p takes where
// q = p up to the fp32 normalisers.  The draw's weights e_q/S_q - e_p/S_p
// do not depend on these scales.
__device__ __forceinline__ void use_shared_table(DrawRows& R, const double* et) {
  const double invT = R.yscale / Exp64::kScale;
  const double rho =
      R.mode == kModeResidual ? exp((R.mq - R.mp) * invT) * (R.cp / R.cq) : 1.0;
  R.rho = rho;
  R.k_hi = uniform_margin(true) * rho;
  R.k_lo = uniform_margin(false) * rho;
  R.mq = 0.0;
  R.mp = 0.0;
  R.cq = 1.0;
  R.cp = 1.0;
  R.et = et;
  R.etp = et;
}

// Table entry of bf16 code b, and whether b needs the computed exponential
// (outside the table and not infinite; a row that is drawn from has a finite
// maximum, so its only infinite logits are -inf).
__device__ __forceinline__ int etab_index(unsigned b) {
  const unsigned t = (b & 0x7FFFu) - kETabLo;
  return static_cast<int>((b >> 15) * kETabSign + min(t, kETabN));
}
__device__ __forceinline__ bool etab_other(unsigned b) {
  return (b & 0x7FFFu) - kETabLo >= kETabN && (b & 0x7FFFu) != 0x7F80u;
}

// e(x) of a token of the q row (P false) or the p row (P true) of R.  With
// the tables (ET), every lane reads one entry, and a wave computes the
// exponential only when one of its lanes holds a code outside the table.
template <int DT, bool ET, bool P>
__device__ __forceinline__ double row_exp(const DrawRows& R, float z, const double* tab) {
  if constexpr (DT == kBF16 && ET) {
    const unsigned b = __float_as_uint(z) >> 16;
    double e = (P ? R.etp : R.et)[etab_index(b)];
    const bool other = etab_other(b);
    if (__builtin_amdgcn_ballot_w64(other) != 0ull) {
      if (other) e = row_tok_exp<P>(R, z, tab);
    }
    return e;
  }
  return row_tok_exp<P>(R, z, tab);
}

// row_exp for H tokens of one row at once: the table reads are issued
// together, then one wave-level test covers all H for the computed codes.
template <int DT, bool ET, bool P, int H>
__device__ __forceinline__ void row_exp_n(const DrawRows& R, const float* z, const double* tab,
                                          double (&e)[H]) {
  if constexpr (DT == kBF16 && ET) {
    bool other[H];
    bool any = false;
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const unsigned b = __float_as_uint(z[k]) >> 16;
      e[k] = (P ? R.etp : R.et)[etab_index(b)];
      other[k] = etab_other(b);
      any = any || other[k];
    }
    if (__builtin_amdgcn_ballot_w64(any) != 0ull) {
#pragma unroll
      for (int k = 0; k < H; ++k)
        if (other[k]) e[k] = row_tok_exp<P>(R, z[k], tab);
    }
  } else {
#pragma unroll
    for (int k = 0; k < H; ++k) e[k] = row_tok_exp<P>(R, z[k], tab);
  }
}

// The same lookups from the raw words of a bf16 row (two codes per word, the
// lower token id in the low half), with the index arithmetic done on both
// halves at once in 16-bit lanes.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

static_assert(kETabSign == 1u << 11 && kETabN < kETabSign, "sign bit 15 -> entry bit 11");

// base + 8 * (low or high 16 bits of x), one v_mad_u32_u16 each (its op_sel
// picks the half; the compiler otherwise extracts, shifts and adds).
__device__ __forceinline__ unsigned lds_entry_lo(unsigned x, unsigned base) {
  unsigned r;
  asm("v_mad_u32_u16 %0, %1, 8, %2" : "=v"(r) : "v"(x), "s"(base));
  return r;
}
__device__ __forceinline__ unsigned lds_entry_hi(unsigned x, unsigned base) {
  unsigned r;
  asm("v_mad_u32_u16 %0, %1, 8, %2 op_sel:[1,0,0,0]" : "=v"(r) : "v"(x), "s"(base));
  return r;
}

// LDS addresses (table base + 8 * entry) of the two codes of w.  mx keeps
// per half the largest clamped offset seen: kETabN there means a code outside
// the table (-inf included).
__device__ __forceinline__ void etab_addresses(unsigned w, unsigned base, unsigned& a0,
                                               unsigned& a1, u16x2& mx) {
  const u16x2 mag = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  const u16x2 t = mag - static_cast<u16x2>(static_cast<unsigned short>(kETabLo));
  const u16x2 tc = __builtin_elementwise_min(t, static_cast<u16x2>(static_cast<unsigned short>(kETabN)));
  mx = __builtin_elementwise_max(mx, tc);
  // each half's sign bit (15) moves to bit 11: + kETabSign for a negative code
  const unsigned idx = __builtin_bit_cast(unsigned, tc) | ((w >> 4) & 0x08000800u);
  a0 = lds_entry_lo(idx, base);
  a1 = lds_entry_hi(idx, base);
}

// Nonzero when a code of w is neither in the table nor infinite.
__device__ __forceinline__ unsigned etab_other_word(unsigned w) {
  const u16x2 mag = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  const u16x2 t = mag - static_cast<u16x2>(static_cast<unsigned short>(kETabLo));
  const u16x2 out = __builtin_elementwise_sub_sat(
      t, static_cast<u16x2>(static_cast<unsigned short>(kETabN - 1)));
  const u16x2 ninf = mag ^ static_cast<u16x2>(static_cast<unsigned short>(0x7F80u));  // 0 iff +-inf
  return __builtin_bit_cast(unsigned, __builtin_elementwise_min(out, ninf));
}

// The 8 bf16 codes of z (stored values, -inf past V) as 4 words.
__device__ __forceinline__ uint4 pack_bf16_words(const float (&z)[8]) {
  unsigned w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = (__float_as_uint(z[2 * k + 1]) & 0xFFFF0000u) | (__float_as_uint(z[2 * k]) >> 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// e of the 2*NW codes in words w[0..NW) of the q row (P false) or p row.
template <bool P, int NW>
__device__ __forceinline__ void row_exp_words(const DrawRows& R, const unsigned (&w)[NW],
                                              const double* tab, double (&e)[2 * NW]) {
  typedef const __attribute__((address_space(3))) double* LdsDouble;
  const LdsDouble et = (LdsDouble)(P ? R.etp : R.et);  // the tables live in LDS
  const unsigned base = static_cast<unsigned>(reinterpret_cast<uintptr_t>(et));
  unsigned a[2 * NW];
  u16x2 mx = static_cast<u16x2>(static_cast<unsigned short>(0));
#pragma unroll
  for (int k = 0; k < NW; ++k) etab_addresses(w[k], base, a[2 * k], a[2 * k + 1], mx);
#pragma unroll
  for (int k = 0; k < 2 * NW; ++k) e[k] = *(LdsDouble)(static_cast<uintptr_t>(a[k]));
  // 0 iff every code was in the table
  const unsigned out = __builtin_bit_cast(
      unsigned, __builtin_elementwise_sub_sat(
                    mx, static_cast<u16x2>(static_cast<unsigned short>(kETabN - 1))));
  // A code outside the table is rare in a plain row; -inf (a filtered row)
  // reads its 0 correctly, so only finite codes outside it are computed.
  if (__builtin_amdgcn_ballot_w64(out != 0u) != 0ull) {
    unsigned other = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) other |= etab_other_word(w[k]);
    if (__builtin_amdgcn_ballot_w64(other != 0u) != 0ull) {
#pragma unroll
      for (int k = 0; k < 2 * NW; ++k) {
        const unsigned b = (w[k / 2] >> (16 * (k % 2))) & 0xFFFFu;
        if (etab_other(b)) e[k] = row_tok_exp<P>(R, __uint_as_float(b << 16), tab);
      }
    }
  }
}

// Raw 16-byte groups of one lane for one chunk (q row, and p row for a residual).
struct RawChunk {
  uint4 q, p;
};

// Whether chunk c lies whole inside aligned rows.  32-bit arithmetic (chunks
// past the row's end are never asked about, and V <= 2^20), so that the test
// stays on the scalar unit: there is no 64-bit scalar compare for order.
template <int DT>
__device__ __forceinline__ bool chunk_full(const DrawRows& R, int c) {
  constexpr int CH = kWave * (16 / Elt<DT>::bytes);
  return R.aligned && (c + 1) * CH <= R.V;
}

// Issue the loads of a full chunk (both rows together).
template <int DT, int MODE>
__device__ __forceinline__ void chunk_issue(const DrawRows& R, int c, RawChunk& raw) {
  constexpr int E = 16 / Elt<DT>::bytes;
  const int64_t x0 = static_cast<int64_t>(c) * (kWave * E) + static_cast<int64_t>(lane_id()) * E;
  const int64_t off = x0 * Elt<DT>::bytes;
  raw.q = *reinterpret_cast<const uint4*>(static_cast<const char*>(R.qrow) + off);
  if (MODE == kModeResidual)
    raw.p = *reinterpret_cast<const uint4*>(static_cast<const char*>(R.prow) + off);
}

// The lane's E values of both rows: from the issued loads for a full chunk,
// element by element (-inf past V) otherwise.
template <int DT, int MODE>
__device__ __forceinline__ void chunk_values(const DrawRows& R, int c, bool full,
                                             const RawChunk& raw,
                                             float (&zq)[16 / Elt<DT>::bytes],
                                             float (&zp)[16 / Elt<DT>::bytes]) {
  constexpr int E = 16 / Elt<DT>::bytes;
  if (full) {
    unpack16<DT>(raw.q, zq);
    if (MODE == kModeResidual) unpack16<DT>(raw.p, zp);
  } else {
    const int64_t x0 =
        static_cast<int64_t>(c) * (kWave * E) + static_cast<int64_t>(lane_id()) * E;
    load_group<DT>(R.qrow, x0, R.V, false, zq);
    if (MODE == kModeResidual) load_group<DT>(R.prow, x0, R.V, false, zp);
  }
}

// Exact weights of this lane's E tokens (used to re-derive the chosen chunk).
// pre: the chunk's loads, already issued (for a full chunk), or null.
template <int DT, int MODE, bool ET = false>
__device__ __forceinline__ void lane_weights(const DrawRows& R, int c, double iq, double ip,
                                             const double* tab,
                                             double (&w)[16 / Elt<DT>::bytes],
                                             const RawChunk* pre = nullptr) {
  constexpr int E = 16 / Elt<DT>::bytes;
  RawChunk raw;
  const bool full = chunk_full<DT>(R, c);
  if (full) {
    if (pre != nullptr)
      raw = *pre;
    else
      chunk_issue<DT, MODE>(R, c, raw);
  }
  float zq[E], zp[E];
  chunk_values<DT, MODE>(R, c, full, raw, zq, zp);
  if constexpr (DT == kBF16 && ET) {  // all table reads at once, from the words
    const uint4 wq = pack_bf16_words(zq);
    const unsigned q[4] = {wq.x, wq.y, wq.z, wq.w};
    double eq[E], ep[E];
    row_exp_words<false, 4>(R, q, tab, eq);
    if (MODE == kModeResidual) {
      const uint4 wp = pack_bf16_words(zp);
      const unsigned p[4] = {wp.x, wp.y, wp.z, wp.w};
      row_exp_words<true, 4>(R, p, tab, ep);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (MODE == kModeResidual) {
        const double d = eq[e] * iq - ep[e] * ip;
        w[e] = d > 0.0 ? d : 0.0;
      } else {
        w[e] = eq[e];
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const double eq = row_exp<DT, ET, false>(R, zq[e], tab);
    if (MODE == kModeResidual) {
      const double ep = row_exp<DT, ET, true>(R, zp[e], tab);
      const double d = eq * iq - ep * ip;
      w[e] = d > 0.0 ? d : 0.0;
    } else {
      w[e] = eq;
    }
  }
}

// Per-chunk results of a fast-path sweep: A and Bv valid in every lane, or
// with RS their in-row scans (the row totals in lanes 15, 31, 47, 63); the
// uncertain list valid in every lane.
struct ChunkSums {
  double A, Bv;
  int n_unc;
  // the uncertain tokens' two logits as fp32 bit patterns (bf16 rows: the
  // code in the high half), so that resolving them reads no row again
  unsigned uq[kUncMax], up[kUncMax];
};

// An empty uncertain list.
__device__ __forceinline__ void chunk_sums_init(ChunkSums& out) {
  out.n_unc = 0;
#pragma unroll
  for (int j = 0; j < kUncMax; ++j) {
    out.uq[j] = 0u;
    out.up[j] = 0u;
  }
}

// Fast-path arithmetic of one chunk.  lookup(e, eq, ep) gives the exponentials
// of the lane's tokens e .. e+H-1 of the q row (and the p row for a residual).
// Adds every token's e_q, e_p to the lane's lsq, lsp, the clearly positive
// ones to a, bb, and the chunk's uncertain tokens to out's list with their two
// logits, taken from words (the lane's 4+4 raw words of a bf16 chunk) when it
// is set, else from the lane's values zqv, zpv.
// A bonus draw needs no normaliser (its weights are e_q, the draw is
// scale-free): there every e_q goes to a alone and lsq, lsp stay as they are.
template <int DT, int MODE, int H, typename Lookup>
__device__ __forceinline__ void chunk_accumulate(const DrawRows& R, int c, Lookup lookup,
                                                 double& lsq, double& lsp, double& a, double& bb,
                                                 ChunkSums& out,
                                                 const unsigned* words = nullptr,
                                                 const float* zqv = nullptr,
                                                 const float* zpv = nullptr) {
  constexpr int E = 16 / Elt<DT>::bytes;
  unsigned long long unc_m[E];  // per token slot: the lanes whose token is uncertain
  double eqh[H], eph[H];
  const double k_hi = R.k_hi, k_lo = R.k_lo;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e % H == 0) lookup(e, eqh, eph);
    const double eq = eqh[e % H];
    if (MODE == kModeResidual) {
      lsq = lsq + eq;
      const double ep = eph[e % H];
      lsp = lsp + ep;
      // pos means e_q >= (1+kDelta) rho e_p (a token with e_q = e_p = 0
      // counts as positive and adds nothing), and lo <= 0 means
      // e_q <= (1-kDelta) rho e_p; a token with neither is uncertain.  Each
      // fma rounds once, so its sign is exact for its rounded constant.
      const double hi = fma(ep, k_hi, eq), lo = fma(ep, k_lo, eq);
      // the masks straight from the comparisons (every lane is active here)
      const unsigned long long pos_m = __ballot(hi >= 0.0), lo_m = __ballot(lo > 0.0);
      // 1.0 or 0.0 (high word only): clearly positive tokens add e_q and e_p
      const double take = __hiloint2double(hi >= 0.0 ? 0x3ff00000 : 0, 0);
      a = fma(take, eq, a);
      bb = fma(take, ep, bb);
      unc_m[e] = lo_m & ~pos_m;
    } else {
      a = a + eq;
    }
  }
  unsigned long long any_unc = 0ull;
  if (MODE == kModeResidual) {
#pragma unroll
    for (int e = 0; e < E; ++e) any_unc |= unc_m[e];
  }
  if (MODE == kModeResidual && any_unc != 0ull) {  // one scalar test for the chunk; rare
#pragma unroll
    for (int e = 0; e < E; ++e) {
      unsigned long long m = unc_m[e];
      while (m) {  // wave-uniform; rare
        const int src = __ffsll(static_cast<long long>(m)) - 1;
        unsigned bq, bp;
        if (words != nullptr) {  // token e sits in word e/2, lower id in the low half
          const unsigned wq = static_cast<unsigned>(__shfl(static_cast<int>(words[e / 2]), src, kWave));
          const unsigned wp = static_cast<unsigned>(__shfl(static_cast<int>(words[4 + e / 2]), src, kWave));
          bq = (e & 1) ? (wq & 0xFFFF0000u) : (wq << 16);
          bp = (e & 1) ? (wp & 0xFFFF0000u) : (wp << 16);
        } else {
          bq = static_cast<unsigned>(__shfl(static_cast<int>(__float_as_uint(zqv[e])), src, kWave));
          bp = static_cast<unsigned>(__shfl(static_cast<int>(__float_as_uint(zpv[e])), src, kWave));
        }
#pragma unroll
        for (int j = 0; j < kUncMax; ++j)
          if (j == out.n_unc) {
            out.uq[j] = bq;
            out.up[j] = bp;
          }
        out.n_unc += 1;
        m &= m - 1;
      }
    }
  }
}

// The sums a, bb of a sweep item into out.A, out.Bv (RS: in-row scans).
template <int MODE, bool RS>
__device__ __forceinline__ void chunk_reduce(double a, double bb, ChunkSums& out) {
  if constexpr (RS) {
    out.A = wave_scan_rows(a);
    out.Bv = MODE == kModeResidual ? wave_scan_rows(bb) : 0.0;
  } else {
    out.A = wave_sum_rows(a);
    out.Bv = MODE == kModeResidual ? wave_sum_rows(bb) : 0.0;
  }
}

// chunk_accumulate from the lane's values.
template <int DT, int MODE, bool ET = false>
__device__ __forceinline__ void chunk_acc(const DrawRows& R, int c,
                                          const float (&zq)[16 / Elt<DT>::bytes],
                                          const float (&zp)[16 / Elt<DT>::bytes],
                                          const double* tab, double& lsq, double& lsp, double& a,
                                          double& bb, ChunkSums& out) {
  constexpr int E = 16 / Elt<DT>::bytes;
  constexpr int H = E < 4 ? E : 4;  // tokens whose exponentials are formed together
  auto lookup = [&](int e, double (&eq)[H], double (&ep)[H]) {
    row_exp_n<DT, ET, false, H>(R, zq + e, tab, eq);
    if (MODE == kModeResidual) row_exp_n<DT, ET, true, H>(R, zp + e, tab, ep);
  };
  chunk_accumulate<DT, MODE, H>(R, c, lookup, lsq, lsp, a, bb, out, nullptr, zq, zp);
}

// What a one-pass sweep of a row also gathers for its statistics, on the
// bf16 codes themselves (two per word, one packed 16-bit operation each): the
// largest code read as a signed 16-bit integer -- the largest non-negative
// value when there is one --, the smallest code read as unsigned -- then the
// negative value of least magnitude, the largest --, and the largest |code|
// (above 0x7F80: a NaN).  Integer extrema need none of the canonicalising
// moves the compiler puts before a float max.
struct RowTrack {
  unsigned smax = 0x80008000u;  // i16x2 max of the codes
  unsigned umin = 0xFF80FF80u;  // u16x2 min of the codes, from -inf's code
  unsigned mag = 0u;            // u16x2 max of |code|
  // The lane's largest value (-inf when it read nothing).
  __device__ __forceinline__ float value() const {
    const i16x2 sm = __builtin_bit_cast(i16x2, smax);
    const u16x2 um = __builtin_bit_cast(u16x2, umin);
    const int p = max(static_cast<int>(sm.x), static_cast<int>(sm.y));
    const unsigned n = min(static_cast<unsigned>(um.x), static_cast<unsigned>(um.y));
    const unsigned code = p >= 0 ? static_cast<unsigned>(p) : n;
    return __uint_as_float(code << 16);
  }
};

// chunk_accumulate from the raw words of bf16 rows with the exponential tables.
// TRACK: also fold the q row's codes into *trk.
template <int MODE, bool TRACK = false>
__device__ __forceinline__ void chunk_acc_words(const DrawRows& R, int c, const uint4& wq,
                                                const uint4& wp, const double* tab, double& lsq,
                                                double& lsp, double& a, double& bb,
                                                ChunkSums& out, RowTrack* trk = nullptr) {
  if constexpr (TRACK) {
    const unsigned q4[4] = {wq.x, wq.y, wq.z, wq.w};
    u16x2 mg = __builtin_bit_cast(u16x2, trk->mag);
    i16x2 sm = __builtin_bit_cast(i16x2, trk->smax);
    u16x2 um = __builtin_bit_cast(u16x2, trk->umin);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      sm = __builtin_elementwise_max(sm, __builtin_bit_cast(i16x2, q4[k]));
      um = __builtin_elementwise_min(um, __builtin_bit_cast(u16x2, q4[k]));
      mg = __builtin_elementwise_max(mg, __builtin_bit_cast(u16x2, q4[k] & 0x7FFF7FFFu));
    }
    trk->smax = __builtin_bit_cast(unsigned, sm);
    trk->umin = __builtin_bit_cast(unsigned, um);
    trk->mag = __builtin_bit_cast(unsigned, mg);
  }
  const unsigned w8[8] = {wq.x, wq.y, wq.z, wq.w, wp.x, wp.y, wp.z, wp.w};
  auto lookup = [&](int e, double (&eq)[8], double (&ep)[8]) {
    const unsigned qw[4] = {w8[0], w8[1], w8[2], w8[3]};
    row_exp_words<false, 4>(R, qw, tab, eq);
    if (MODE == kModeResidual) {
      const unsigned pw[4] = {w8[4], w8[5], w8[6], w8[7]};
      row_exp_words<true, 4>(R, pw, tab, ep);
    }
  };
  chunk_accumulate<kBF16, MODE, 8>(R, c, lookup, lsq, lsp, a, bb, out, w8);
}


// One wave sweeps items s0, s0+stride, ... < s1; item s is the chunks G*s ..
// G*s+G-1 that are below nsub, added into one ChunkSums (one cross-lane
// reduction per item).  The next chunk's loads are issued as soon as the
// current one has been unpacked.  emit(s, sums) stores an item's results
// (RS: see ChunkSums).
template <int DT, int MODE, int G, bool ET = false, bool RS = false, typename Emit>
__device__ __forceinline__ void wave_sweep(const DrawRows& R, int s0, int s1, int stride, int nsub,
                                           const double* tab, double& lsq, double& lsp,
                                           Emit emit) {
  constexpr int E = 16 / Elt<DT>::bytes;
  RawChunk buf;
  bool full = s0 < s1 && chunk_full<DT>(R, G * s0);
  if (full) chunk_issue<DT, MODE>(R, G * s0, buf);
  for (int s = s0; s < s1; s += stride) {
    ChunkSums cs;
    chunk_sums_init(cs);
    double a = 0.0, bb = 0.0;
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
      const int c = G * s + g;
      if (c < nsub) {
        // the chunk after c in this wave's order
        const bool in_item = g + 1 < G && c + 1 < nsub;
        const int cn = in_item ? c + 1 : G * (s + stride);
        const bool has_next = in_item || s + stride < s1;
        if constexpr (DT == kBF16 && ET) {  // table lookups straight from the words
          uint4 wq = buf.q, wp = buf.p;
          if (!full) {
            float zq[E], zp[E];
            chunk_values<DT, MODE>(R, c, false, buf, zq, zp);
            wq = pack_bf16_words(zq);
            if (MODE == kModeResidual) wp = pack_bf16_words(zp);
          }
          full = has_next && chunk_full<DT>(R, cn);
          if (full) chunk_issue<DT, MODE>(R, cn, buf);
          chunk_acc_words<MODE>(R, c, wq, wp, tab, lsq, lsp, a, bb, cs);
        } else {
          float zq[E], zp[E];
          chunk_values<DT, MODE>(R, c, full, buf, zq, zp);
          full = has_next && chunk_full<DT>(R, cn);
          if (full) chunk_issue<DT, MODE>(R, cn, buf);
          chunk_acc<DT, MODE, ET>(R, c, zq, zp, tab, lsq, lsp, a, bb, cs);
        }
      }
    }
    chunk_reduce<MODE, RS>(a, bb, cs);
    emit(s, cs);
  }
}

// Running prefix over W[0..nch) by wave 0; result in sel[] / seld[] (LDS):
//   sel[0] = chosen chunk (-3: no positive weight), sel[1] = 1 if a crossing
//   was found, seld[0] = prefix before the chosen chunk, seld[1] = target,
//   seld[2] = S_w.
__device__ __forceinline__ void locate_chunk(const double* W, int nch, double u, int* sel,
                                             double* seld) {
  const int lane = lane_id();
  const int per = (nch + kWave - 1) / kWave;
  const int c0 = lane * per;
  const int c1 = min(nch, c0 + per);
  double lt = 0.0;
  for (int c = c0; c < c1; ++c) lt = lt + W[c];
  const double li = wave_incl_scan(lt);
  const double run = wave_shr1(li);
  double r = run;
  for (int c = c0; c < c1; ++c) r = r + W[c];
  const int last_lane = (nch - 1) / per;
  const double S_w = readlane_d(r, last_lane);
  const double target = u * S_w;
  int hit = -1, lastpos = -1;
  double hit_excl = 0.0, lastpos_excl = 0.0;
  r = run;
  for (int c = c0; c < c1; ++c) {
    const double tc = W[c];
    const double nr = r + tc;
    if (tc > 0.0) {
      if (hit < 0 && nr > target) {
        hit = c;
        hit_excl = r;
      }
      lastpos = c;
      lastpos_excl = r;
    }
    r = nr;
  }
  const unsigned long long hm = __ballot(hit >= 0);
  const unsigned long long pm = __ballot(lastpos >= 0);
  int s = -3;
  double ex = 0.0;
  if (hm) {
    const int src = __ffsll(static_cast<long long>(hm)) - 1;
    s = __builtin_amdgcn_readlane(hit, src);
    ex = readlane_d(hit_excl, src);
  } else if (pm) {
    const int src = 63 - __clzll(static_cast<long long>(pm));
    s = __builtin_amdgcn_readlane(lastpos, src);
    ex = readlane_d(lastpos_excl, src);
  }
  if (lane == 0) {
    sel[0] = s;
    sel[1] = hm ? 1 : 0;
    seld[0] = ex;
    seld[1] = target;
    seld[2] = S_w;
  }
}

// Draw inside chunk c (wave 0), whose tokens follow a prefix excl: returns
// the first token whose cumulative weight exceeds target (in every lane) when
// crossing is set and one does, else -1 after adding the chunk's total to
// excl and setting lastpos to its last token of positive weight, if any.
template <int DT, int MODE, bool ET = false>
__device__ __forceinline__ int draw_in_one_chunk(const DrawRows& R, int c, bool crossing,
                                                 double& excl, double target, double iq,
                                                 double ip, const double* tab, int& lastpos,
                                                 const RawChunk* pre = nullptr) {
  constexpr int E = 16 / Elt<DT>::bytes;
  const int lane = lane_id();
  double w[E];
  lane_weights<DT, MODE, ET>(R, c, iq, ip, tab, w, pre);
  double ls = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e) ls = ls + w[e];
  const double incl = wave_incl_scan(ls);
  const double lexcl = wave_shr1(incl);
  const bool lane_hit = crossing && ls > 0.0 && (excl + incl) > target;
  const unsigned long long hm = __ballot(lane_hit);
  const unsigned long long pm = __ballot(ls > 0.0);
  if (pm == 0ull) return -1;  // nothing of positive weight here (excl unchanged: all 0)
  const int src = hm ? (__ffsll(static_cast<long long>(hm)) - 1)
                     : 63 - __clzll(static_cast<long long>(pm));
  int pick = -1;
  if (lane == src) {
    const double base = excl + lexcl;
    int last = -1;
    double a = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      a = a + w[e];
      if (w[e] > 0.0) {
        if (pick < 0 && hm && (base + a) > target) pick = e;
        last = e;
      }
    }
    if (pick < 0) pick = last;
  }
  pick = c * (kWave * E) + src * E + __builtin_amdgcn_readlane(pick, src);
  if (hm) return pick;
  lastpos = pick;
  excl = excl + readlane_d(incl, kWave - 1);
  return -1;
}

// Token inside sweep item s (its chunks G*s .. G*s+G-1 below the row's end),
// in token order (wave 0): the crossing if `crossing` and one is found, else
// the item's last token of positive weight; the token id in every lane, or -1.
template <int DT, int MODE, bool ET = false, int G = 1>
__device__ __forceinline__ int draw_in_chunk(const DrawRows& R, int s, bool crossing, double excl,
                                             double target, double iq, double ip,
                                             const double* tab) {
  constexpr int CH = kWave * (16 / Elt<DT>::bytes);
  const int nsub = (R.V + CH - 1) / CH;
  // every chunk's loads at once: a later chunk's latency hides behind the earlier scans
  RawChunk pre[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int c = G * s + g;
    if (c < nsub && chunk_full<DT>(R, c)) chunk_issue<DT, MODE>(R, c, pre[g]);
  }
  int last = -1;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int c = G * s + g;
    if (c < nsub) {
      const int tok = draw_in_one_chunk<DT, MODE, ET>(R, c, crossing, excl, target, iq, ip, tab,
                                                      last, &pre[g]);
      if (tok >= 0) return tok;
    }
  }
  return last;
}

// LDS the draw routines need, per workgroup.
template <int BLOCK>
struct DrawShared {
  double tab[Exp64::kTab];
  double red[BLOCK / kWave];
  float redf[BLOCK / kWave];
  int sel[4];
  double seld[4];
  double norm[2];  // the exact normalisers S_q, S_p of a finished fast sweep
  unsigned next;   // the fast sweep's item counter
  unsigned last;   // split draw: this workgroup finishes the sequence
};

// Exact two-sweep draw (whole block).  W: nch doubles of scratch.  With
// have_s the exact normalisers Sq, Sp of a finished fast sweep are taken
// as given and the first sweep is skipped.  Returns the token (every
// thread), or -1 when no token carries positive weight.
template <int BLOCK, int DT, bool ET = false>
__device__ __forceinline__ int slow_draw(DrawRows R, int nch, double* W, double u, DrawShared<BLOCK>& sh,
                         bool have_s = false, double Sq_in = 0.0, double Sp_in = 0.0) {
  constexpr int NW = BLOCK / kWave;
  constexpr int E = 16 / Elt<DT>::bytes;
  const int tid = threadIdx.x, wv = uniform(tid / kWave), lane = lane_id();
  double iq = 1.0, ip = 1.0;
  if (R.mode == kModeResidual && have_s) {
    iq = 1.0 / Sq_in;
    ip = 1.0 / Sp_in;
  } else if (R.mode == kModeResidual) {
    double aq = 0.0, ap = 0.0;
    for (int c = wv; c < nch; c += NW) {
      RawChunk raw;
      const bool full = chunk_full<DT>(R, c);
      if (full) chunk_issue<DT, kModeResidual>(R, c, raw);
      float zq[E], zp[E];
      chunk_values<DT, kModeResidual>(R, c, full, raw, zq, zp);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        aq = aq + row_exp<DT, ET, false>(R, zq[e], sh.tab);
        ap = ap + row_exp<DT, ET, true>(R, zp[e], sh.tab);
      }
    }
    const double Sq = block_sum<BLOCK>(aq, sh.red);
    const double Sp = block_sum<BLOCK>(ap, sh.red);
    iq = 1.0 / Sq;
    ip = 1.0 / Sp;
  }
  for (int attempt = 0; attempt < 2; ++attempt) {
    for (int c = wv; c < nch; c += NW) {
      double w[E];
      if (R.mode == kModeResidual)
        lane_weights<DT, kModeResidual, ET>(R, c, iq, ip, sh.tab, w);
      else
        lane_weights<DT, kModeBonus, ET>(R, c, iq, ip, sh.tab, w);
      double ls = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) ls = ls + w[e];
      const double incl = wave_incl_scan(ls);
      if (lane == kWave - 1) W[c] = incl;
    }
    __syncthreads();
    if (wv == 0) locate_chunk(W, nch, u, sh.sel, sh.seld);
    __syncthreads();
    const bool empty_residual = R.mode == kModeResidual && !(sh.seld[2] > 0.0);
    __syncthreads();
    if (empty_residual && attempt == 0) {
      R.mode = kModeBonus;  // residual has no mass: draw from q_n
      continue;
    }
    break;
  }
  int tok = -1;
  if (sh.sel[0] >= 0 && wv == 0)
    tok = R.mode == kModeResidual
              ? draw_in_chunk<DT, kModeResidual, ET>(R, sh.sel[0], sh.sel[1] != 0, sh.seld[0],
                                                     sh.seld[1], iq, ip, sh.tab)
              : draw_in_chunk<DT, kModeBonus, ET>(R, sh.sel[0], sh.sel[1] != 0, sh.seld[0],
                                                  sh.seld[1], iq, ip, sh.tab);
  if (tid == 0) sh.sel[2] = tok;
  __syncthreads();
  tok = sh.sel[2];
  __syncthreads();
  return tok;
}

// ------------------------------------------------------ sweep item results
//
// What the fast sweep leaves per item: the sums A, Bv of the clearly positive
// tokens' e_q and e_p, the normaliser parts Lq, Lp, and the uncertain tokens
// (count and their two logits' fp32 bit patterns).  Each sum is
// kept as the four in-row scan totals of the wave that swept the item (lanes
// 15, 31, 47, 63) and added in sum_row_totals' order where it is read, so no
// result depends on which wave, or which workgroup, swept which item.

// In the LDS of the one workgroup that sweeps and draws: A, Bv, Lq, Lp as
// arrays of 4*ni doubles, then unc_n[ni], unc_q[ni*kUncMax],
// unc_p[ni*kUncMax].
struct LdsItems {
  double* A;
  double* Bv;
  double* Lq;
  double* Lp;
  int* unc_n;
  unsigned* unc_q;
  unsigned* unc_p;
  __device__ __forceinline__ LdsItems(double* base, int ni)
      : A(base), Bv(base + 4 * ni), Lq(base + 8 * ni), Lp(base + 12 * ni),
        unc_n(reinterpret_cast<int*>(base + 16 * ni)),
        unc_q(reinterpret_cast<unsigned*>(unc_n + ni)), unc_p(unc_q + ni * kUncMax) {}
  // cs.A, cs.Bv, lq, lp: in-row scans (chunk_reduce with RS); the uncertain
  // list is the same in every lane.
  __device__ __forceinline__ void emit(int s, const ChunkSums& cs, double lq, double lp) const {
    const int lane = lane_id();
    if ((lane & 15) == 15) {
      const int i = 4 * s + (lane >> 4);
      A[i] = cs.A;
      Bv[i] = cs.Bv;
      Lq[i] = lq;
      Lp[i] = lp;
    }
    if (lane == 0) {
      unc_n[s] = cs.n_unc;
#pragma unroll
      for (int j = 0; j < kUncMax; ++j) {
        unc_q[s * kUncMax + j] = cs.uq[j];
        unc_p[s * kUncMax + j] = cs.up[j];
      }
    }
  }
  __device__ __forceinline__ double a(int c) const {
    return sum_row_totals(A[4 * c], A[4 * c + 1], A[4 * c + 2], A[4 * c + 3]);
  }
  __device__ __forceinline__ double bv(int c) const {
    return sum_row_totals(Bv[4 * c], Bv[4 * c + 1], Bv[4 * c + 2], Bv[4 * c + 3]);
  }
  __device__ __forceinline__ double lq(int c) const {
    return sum_row_totals(Lq[4 * c], Lq[4 * c + 1], Lq[4 * c + 2], Lq[4 * c + 3]);
  }
  __device__ __forceinline__ double lp(int c) const {
    return sum_row_totals(Lp[4 * c], Lp[4 * c + 1], Lp[4 * c + 2], Lp[4 * c + 3]);
  }
  __device__ __forceinline__ int n_unc(int c) const { return unc_n[c]; }
  __device__ __forceinline__ unsigned uq(int c, int j) const { return unc_q[c * kUncMax + j]; }
  __device__ __forceinline__ unsigned up(int c, int j) const { return unc_p[c * kUncMax + j]; }
};

// Bytes of the LDS item arrays for ni items.
constexpr size_t lds_items_bytes(int ni) {
  return static_cast<size_t>(ni) * (16 * sizeof(double) + (1 + 2 * kUncMax) * sizeof(int));
}

// In device memory, for a sequence whose sweep is split over several
// workgroups: one record of kItemRec doubles per item -- doubles 4r..4r+3 hold
// row r's totals of A, Bv, Lq, Lp, then the 32-bit words unc_n, unc_q[kUncMax],
// unc_p[kUncMax] -- written with sc1 stores by the workgroup that swept the
// item and read with sc1 loads by the workgroup that draws, possibly on
// another XCD (device_common.hpp).  `rec` must be uniform.
constexpr int kItemRec = 20;  // doubles per record (160 bytes)
static_assert(16 + (1 + 2 * kUncMax + 1) / 2 <= kItemRec, "record layout");

struct GlobalItems {
  double* rec;
  Src<true, double> D;
  Src<true, int> I;
  __device__ __forceinline__ GlobalItems(double* base, int ni)
      : rec(base), D(base, static_cast<int64_t>(ni) * kItemRec),
        I(reinterpret_cast<const int*>(base), static_cast<int64_t>(ni) * kItemRec * 2) {}
  // Writes the records of items s0 .. s0+n-1 from their LDS copy `L`
  // (LdsItems holding them as items 0 .. n-1), the whole block one double
  // each.  The stores are issued here, after the sweep, and not item by item
  // during it: on this architecture stores count in the same vmcnt as loads,
  // so a long write-through store would hold up the sweep's next loads.
  __device__ __forceinline__ void write_from(const LdsItems& L, int s0, int n) const {
    double* base = rec + static_cast<int64_t>(s0) * kItemRec;
    for (int k = threadIdx.x; k < n * kItemRec; k += blockDim.x) {
      const int i = k / kItemRec, w = k - i * kItemRec;
      double v;
      if (w < 16) {
        const int r = w >> 2, f = w & 3;
        const double* src = f == 0 ? L.A : f == 1 ? L.Bv : f == 2 ? L.Lq : L.Lp;
        v = src[4 * i + r];
      } else {
        // int words 32 + 2(w-16), +1: unc_n, unc_q[..], unc_p[..], 0 padding
        int lo_hi[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q = 2 * (w - 16) + h;
          lo_hi[h] = q == 0 ? L.unc_n[i]
                   : q <= kUncMax ? static_cast<int>(L.unc_q[i * kUncMax + q - 1])
                   : q <= 2 * kUncMax ? static_cast<int>(L.unc_p[i * kUncMax + q - 1 - kUncMax])
                   : 0;
        }
        v = __hiloint2double(lo_hi[1], lo_hi[0]);
      }
      st<true>(&base[k], v);
    }
  }
  __device__ __forceinline__ double field(int c, int f) const {
    const int64_t o = static_cast<int64_t>(c) * kItemRec + f;
    return sum_row_totals(D[o], D[o + 4], D[o + 8], D[o + 12]);
  }
  __device__ __forceinline__ double a(int c) const { return field(c, 0); }
  __device__ __forceinline__ double bv(int c) const { return field(c, 1); }
  __device__ __forceinline__ double lq(int c) const { return field(c, 2); }
  __device__ __forceinline__ double lp(int c) const { return field(c, 3); }
  __device__ __forceinline__ int word(int c, int k) const {
    return I[static_cast<int64_t>(c) * (2 * kItemRec) + 32 + k];
  }
  __device__ __forceinline__ int n_unc(int c) const { return word(c, 0); }
  __device__ __forceinline__ unsigned uq(int c, int j) const {
    return static_cast<unsigned>(word(c, 1 + j));
  }
  __device__ __forceinline__ unsigned up(int c, int j) const {
    return static_cast<unsigned>(word(c, 1 + kUncMax + j));
  }
};

// GlobalItems whose item threadIdx.x (when below ni) has its fields for the
// finish (A, Bv and the uncertain tokens) loaded on construction.  The part
// that finishes a split draw builds it before item_normalisers, so that these
// loads travel with the normaliser parts' instead of a round trip later; the
// row totals are kept as loaded and added where they are read, in
// sum_row_totals' order, so every value is the one GlobalItems gives.
struct GlobalItemsAhead : GlobalItems {
  double ra[4], rb[4];
  int nu;
  unsigned wq[kUncMax], wp[kUncMax];
  __device__ __forceinline__ GlobalItemsAhead(const GlobalItems& g, int ni) : GlobalItems(g) {
    const int c = threadIdx.x;
    if (c < ni) {
      const int64_t o = static_cast<int64_t>(c) * kItemRec;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ra[r] = D[o + 4 * r];
        rb[r] = D[o + 4 * r + 1];
      }
      nu = GlobalItems::n_unc(c);
#pragma unroll
      for (int j = 0; j < kUncMax; ++j) {
        wq[j] = GlobalItems::uq(c, j);
        wp[j] = GlobalItems::up(c, j);
      }
    }
  }
  __device__ __forceinline__ bool mine(int c) const { return c == static_cast<int>(threadIdx.x); }
  __device__ __forceinline__ double a(int c) const {
    return mine(c) ? sum_row_totals(ra[0], ra[1], ra[2], ra[3]) : GlobalItems::a(c);
  }
  __device__ __forceinline__ double bv(int c) const {
    return mine(c) ? sum_row_totals(rb[0], rb[1], rb[2], rb[3]) : GlobalItems::bv(c);
  }
  __device__ __forceinline__ int n_unc(int c) const {
    return mine(c) ? nu : GlobalItems::n_unc(c);
  }
  __device__ __forceinline__ unsigned uq(int c, int j) const {
    return mine(c) ? wq[j] : GlobalItems::uq(c, j);
  }
  __device__ __forceinline__ unsigned up(int c, int j) const {
    return mine(c) ? wp[j] : GlobalItems::up(c, j);
  }
};

// The exact normalisers S_q, S_p of a finished fast sweep, to every thread:
// wave 0 adds the items' parts, item c in lane c % 64 in item order, then
// the lanes in wave_sum_rows' fixed order -- the same order whatever the
// block size and however many workgroups swept.  Contains a barrier.
template <int BLOCK, typename Items>
__device__ __forceinline__ void item_normalisers(const Items& it, int ni, DrawShared<BLOCK>& sh,
                                                 double& Sq, double& Sp) {
  if (threadIdx.x < kWave) {
    double lq = 0.0, lp = 0.0;
    for (int c = lane_id(); c < ni; c += kWave) {
      lq = lq + it.lq(c);
      lp = lp + it.lp(c);
    }
    lq = wave_sum_rows(lq);  // DPP row scans and four lane reads, no LDS round trips
    lp = wave_sum_rows(lp);
    if (threadIdx.x == 0) {
      sh.norm[0] = lq;
      sh.norm[1] = lp;
    }
  }
  __syncthreads();
  Sq = sh.norm[0];
  Sp = sh.norm[1];
}

// Fast-path finish (whole block) from a sweep's results: the exact
// normalisers Sq, Sp and, per item of G chunks, the view `it` (LdsItems or
// GlobalItems).  W (ni doubles of this workgroup's LDS) receives the item
// totals W_c.  sh.sel[3] must be 0, with a barrier between the clearing and
// the call.  ET: the sweep took the bf16 table path, which records the
// uncertain tokens' codes.  Returns the token, -1 (nothing to draw), -2 (take
// the slow path) or -3 (the residual has no mass: draw from q_n instead).
template <int BLOCK, int DT, bool ET, int G, typename Items>
__device__ __forceinline__ int fast_finish(const DrawRows& R, int ni, double Sq, double Sp, const Items& it,
                           double* W, double u, DrawShared<BLOCK>& sh) {
  const int tid = threadIdx.x, wv = tid / kWave;
  double iq = 1.0, ip = 1.0;
  if (R.mode == kModeResidual) {
    iq = 1.0 / Sq;
    ip = 1.0 / Sp;
    const double ratio = (Sq / Sp) / R.rho;  // exact over fp32-normaliser ratio
    bool ok = fabs(ratio - 1.0) <= kDelta / 4;
    for (int c = tid; c < ni; c += BLOCK) {
      const double a = it.a(c), bv = it.bv(c);
      const int nu = it.n_unc(c);
      double w = a * iq - bv * ip;
      w = w > 0.0 ? w : 0.0;
      if (nu > kUncMax) ok = false;
#pragma unroll
      for (int j = 0; j < kUncMax; ++j) {
        if (j < nu) {
          // the token's two logits as the sweep kept them (exact)
          const float zq = __uint_as_float(it.uq(c, j)), zp = __uint_as_float(it.up(c, j));
          const double eq = row_exp<DT, ET, false>(R, zq, sh.tab);
          const double ep = row_exp<DT, ET, true>(R, zp, sh.tab);
          const double d = eq * iq - ep * ip;
          w = w + (d > 0.0 ? d : 0.0);
        }
      }
      W[c] = w;
    }
    if (!ok) sh.sel[3] = 1;  // cleared by the caller before a barrier
    __syncthreads();
    if (sh.sel[3] != 0) return -2;
  } else {
    for (int c = tid; c < ni; c += BLOCK) W[c] = it.a(c);
    __syncthreads();
  }
  if (wv == 0) locate_chunk(W, ni, u, sh.sel, sh.seld);
  __syncthreads();
  if (R.mode == kModeResidual && !(sh.seld[2] > 0.0)) {
    __syncthreads();
    return -3;
  }
  int tok = -1;
  if (sh.sel[0] >= 0 && wv == 0)
    tok = R.mode == kModeResidual
              ? draw_in_chunk<DT, kModeResidual, ET, G>(R, sh.sel[0], sh.sel[1] != 0,
                                                        sh.seld[0], sh.seld[1], iq, ip, sh.tab)
              : draw_in_chunk<DT, kModeBonus, ET, G>(R, sh.sel[0], sh.sel[1] != 0, sh.seld[0],
                                                     sh.seld[1], iq, ip, sh.tab);
  if (tid == 0) sh.sel[2] = tok;
  __syncthreads();
  tok = sh.sel[2];
  __syncthreads();
  return tok;
}

// The fast sweep of one workgroup in items of G chunks, handed out in the
// order the waves ask for them: wave wv starts with item s0 = wv, and each
// further item comes from the LDS counter *next (which starts at the number
// of waves), claimed one item ahead so that its first chunk's loads are
// issued while the current item is computed.  Waves that the hardware
// schedules first take more items, and all finish within about one item of
// each other.  Every sum is formed per item -- a, bb and the normaliser parts
// lq, lp, each reduced to four row totals -- and emit(s, cs, lq, lp) stores
// them by item, so no result depends on which wave took which item.
template <int DT, int MODE, int G, bool ET, typename Emit, bool TRACK = false>
__device__ __forceinline__ void wave_sweep_claimed(const DrawRows& R, int s0, int ni, int nsub,
                                                   unsigned* next, const double* tab,
                                                   Emit emit, RowTrack* trk = nullptr) {
  static_assert(!TRACK || (DT == kBF16 && ET), "row tracking rides on the bf16 table path");
  constexpr int E = 16 / Elt<DT>::bytes;
  const int lane = lane_id();
  if constexpr (DT == kBF16 && ET && G == 2) {
    // Two buffers, one per chunk of an item: the second chunk's loads go to
    // b1 while the first is computed from b0, and the next item's first
    // chunk to b0 once its words are used, so no chunk's words are copied
    // out of a buffer that is about to be reloaded.
    RawChunk b0, b1;
    int s = s0;
    bool full0 = s < ni && chunk_full<DT>(R, 2 * s);
    if (full0) chunk_issue<DT, MODE>(R, 2 * s, b0);
    while (s < ni) {
      unsigned claimed = 0;
      if (lane == 0) claimed = atomicAdd(next, 1u);
      const int sn = static_cast<int>(uniform(claimed));  // the item after this one
      ChunkSums cs;
      chunk_sums_init(cs);
      double a = 0.0, bb = 0.0, lq = 0.0, lp = 0.0;
      const int c0 = 2 * s, c1 = c0 + 1;  // c0 < nsub: every item has a chunk
      const bool has1 = c1 < nsub;
      uint4 wq = b0.q, wp = b0.p;
      if (!full0) {
        float zq[E], zp[E];
        chunk_values<DT, MODE>(R, c0, false, b0, zq, zp);
        wq = pack_bf16_words(zq);
        if (MODE == kModeResidual) wp = pack_bf16_words(zp);
      }
      const bool full1 = has1 && chunk_full<DT>(R, c1);
      if (full1) chunk_issue<DT, MODE>(R, c1, b1);
      chunk_acc_words<MODE, TRACK>(R, c0, wq, wp, tab, lq, lp, a, bb, cs, trk);
      full0 = sn < ni && chunk_full<DT>(R, 2 * sn);
      if (has1) {
        uint4 vq = b1.q, vp = b1.p;
        if (!full1) {
          float zq[E], zp[E];
          chunk_values<DT, MODE>(R, c1, false, b1, zq, zp);
          vq = pack_bf16_words(zq);
          if (MODE == kModeResidual) vp = pack_bf16_words(zp);
        }
        if (full0) chunk_issue<DT, MODE>(R, 2 * sn, b0);
        chunk_acc_words<MODE, TRACK>(R, c1, vq, vp, tab, lq, lp, a, bb, cs, trk);
      } else if (full0) {
        chunk_issue<DT, MODE>(R, 2 * sn, b0);
      }
      chunk_reduce<MODE, true>(a, bb, cs);
      const double lqr = MODE == kModeResidual ? wave_scan_rows(lq) : 0.0;
      const double lpr = MODE == kModeResidual ? wave_scan_rows(lp) : 0.0;
      emit(s, cs, lqr, lpr);
      s = sn;
    }
    return;
  }
  RawChunk buf;
  int s = s0;
  bool full = s < ni && chunk_full<DT>(R, G * s);
  if (full) chunk_issue<DT, MODE>(R, G * s, buf);
  while (s < ni) {
    unsigned claimed = 0;
    if (lane == 0) claimed = atomicAdd(next, 1u);
    const int sn = static_cast<int>(uniform(claimed));  // the item after this one
    ChunkSums cs;
    chunk_sums_init(cs);
    double a = 0.0, bb = 0.0, lq = 0.0, lp = 0.0;
#pragma unroll 1
    for (int g = 0; g < G; ++g) {
      const int c = G * s + g;
      if (c < nsub) {
        // the chunk after c in this wave's order
        const bool in_item = g + 1 < G && c + 1 < nsub;
        const int cn = in_item ? c + 1 : G * sn;
        const bool has_next = in_item || sn < ni;
        if constexpr (DT == kBF16 && ET) {  // table lookups straight from the words
          uint4 wq = buf.q, wp = buf.p;
          if (!full) {
            float zq[E], zp[E];
            chunk_values<DT, MODE>(R, c, false, buf, zq, zp);
            wq = pack_bf16_words(zq);
            if (MODE == kModeResidual) wp = pack_bf16_words(zp);
          }
          full = has_next && chunk_full<DT>(R, cn);
          if (full) chunk_issue<DT, MODE>(R, cn, buf);
          chunk_acc_words<MODE, TRACK>(R, c, wq, wp, tab, lq, lp, a, bb, cs, trk);
        } else {
          float zq[E], zp[E];
          chunk_values<DT, MODE>(R, c, full, buf, zq, zp);
          full = has_next && chunk_full<DT>(R, cn);
          if (full) chunk_issue<DT, MODE>(R, cn, buf);
          chunk_acc<DT, MODE, ET>(R, c, zq, zp, tab, lq, lp, a, bb, cs);
        }
      }
    }
    chunk_reduce<MODE, true>(a, bb, cs);
    const double lqr = MODE == kModeResidual ? wave_scan_rows(lq) : 0.0;
    const double lpr = MODE == kModeResidual ? wave_scan_rows(lp) : 0.0;
    emit(s, cs, lqr, lpr);
    s = sn;
  }
}

// The whole draw for one row (pair) by one workgroup: the one-sweep fast path
// when `fast`, else or on its failure the exact two-sweep path (dyn: nch
// doubles).  The fast sweep's items are kDrawG chunks each, and dynamic LDS
// `dyn` holds, for its ni items (draw_fast_lds bytes), W: ni doubles, then
// the LdsItems arrays.  sh.tab must hold the exp table.
// Returns the token (every thread), or -1 when no token has positive weight.
template <int BLOCK, int DT, bool ET = false>
__device__ __forceinline__ int draw_block(const DrawRows& R, double u, int fast, double* dyn,
                                          DrawShared<BLOCK>& sh) {
  constexpr int E = 16 / Elt<DT>::bytes;
  constexpr int NW = BLOCK / kWave;
  const int wv = uniform(static_cast<int>(threadIdx.x) / kWave);
  const int nch = (R.V + kWave * E - 1) / (kWave * E);
  const int ni = (nch + kDrawG - 1) / kDrawG;  // sweep items
  int tok = -2;
  double Sq = 0.0, Sp = 0.0;
  if (fast) {
    double* W = dyn;  // the finish's item totals, then the sweep's item arrays
    const LdsItems it(dyn + ni, ni);
    auto emit = [&](int c, const ChunkSums& cs, double lq, double lp) { it.emit(c, cs, lq, lp); };
    if (threadIdx.x == 0) {
      sh.next = NW;
      sh.sel[3] = 0;
    }
    __syncthreads();
    if (R.mode == kModeResidual)
      wave_sweep_claimed<DT, kModeResidual, kDrawG, ET>(R, wv, ni, nch, &sh.next, sh.tab, emit);
    else
      wave_sweep_claimed<DT, kModeBonus, kDrawG, ET>(R, wv, ni, nch, &sh.next, sh.tab, emit);
    SPEC_STAMP(stamps_draw, 2);  // wave 0's last item done
    __syncthreads();
    SPEC_STAMP(stamps_draw, 3);  // every wave's
    item_normalisers<BLOCK>(it, ni, sh, Sq, Sp);
    SPEC_STAMP(stamps_draw, 4);
    tok = fast_finish<BLOCK, DT, ET, kDrawG>(R, ni, Sq, Sp, it, W, u, sh);
    SPEC_STAMP(stamps_draw, 5);
  }
  if (tok == -3) {  // residual without mass: the bonus draw from q_n
    DrawRows Rb = R;
    Rb.mode = kModeBonus;
    tok = slow_draw<BLOCK, DT, ET>(Rb, nch, dyn, u, sh);
  } else if (tok == -2) {
    tok = slow_draw<BLOCK, DT, ET>(R, nch, dyn, u, sh, fast != 0, Sq, Sp);
  }
  return tok;
}

// The final draw of sequence b with accepted count n, by the whole
// workgroup: writes out_tokens[b][n] and num_emitted[b].  Dynamic LDS `dyn`:
// the fast layout (draw_fast_lds: per item its total W, then the LdsItems
// arrays) when `fast` is set, otherwise nch doubles for the slow path; with
// `etab` (bf16) the two rows' exponential tables come first.
// n must be uniform across the workgroup.  tab_ready: sh.tab is already
// filled (and a barrier has passed since); shared_ready: so is the shared
// exponential table at dyn (fill_shared_exp_table).
template <int BLOCK, int DT>
__device__ __forceinline__ void draw_sequence(int64_t b, int n, const void* tgt, const void* dft,
                                              const float* uni, const float* tstats,
                                              const float* dstats, int K, int V, double yscale,
                                              int fast, int etab, int32_t* out_tokens,
                                              int32_t* num_emitted, double* dyn,
                                              DrawShared<BLOCK>& sh, bool tab_ready = false,
                                              bool shared_ready = false) {
  const int64_t K1 = K + 1;
  const int tid = threadIdx.x;
  if (n < 0 || n > K) {
    if (tid == 0 && num_emitted) num_emitted[b] = 0;
    return;
  }
  DrawRows R;
  const int64_t rq = b * K1 + n, rp = b * K + (n < K ? n : 0);
  if (!make_draw_rows<DT>(b, n, K, V, tgt, dft, tstats[2 * rq], tstats[2 * rq + 1],
                          dstats[2 * rp], dstats[2 * rp + 1], yscale, R)) {
    if (tid == 0) {
      out_tokens[b * K1 + n] = -1;
      if (num_emitted) num_emitted[b] = 0;
    }
    return;
  }
  if (!tab_ready) {
    fill_exp2_table(sh.tab);
    __syncthreads();
  }
  double* work = dyn;
  if (DT == kBF16 && etab) {  // dynamic LDS starts with the two rows' tables
    if (draw_rows_share_table(R)) {  // one table of exp(z/T) for both rows
      if (!shared_ready) {
        fill_shared_exp_table<BLOCK>(dyn, R.yscale, 0);
        __syncthreads();
      }
      use_shared_table(R, dyn);
    } else {  // per-row tables (rows with extreme maxima)
      fill_row_exp_tables<BLOCK>(dyn, R.mode == kModeResidual ? 2 : 1, R, sh.tab);
      __syncthreads();
      R.et = dyn;
      R.etp = dyn + kETab;
    }
    work = dyn + 2 * kETab;
  }
  const int tok = R.et != nullptr ? draw_block<BLOCK, DT, true>(R, uni[b * K1 + K], fast, work, sh)
                                  : draw_block<BLOCK, DT, false>(R, uni[b * K1 + K], fast, work, sh);
  if (tid == 0) {
    out_tokens[b * K1 + n] = tok;
    if (num_emitted) num_emitted[b] = tok >= 0 ? n + 1 : 0;
  }
  SPEC_STAMP(stamps_draw, 6);
}

// One workgroup per sequence (the spec_residual_sample path): the final draw
// with the caller's accepted counts.
template <int BLOCK, int DT>
__global__ __launch_bounds__(BLOCK) void residual_kernel(
    const void* __restrict__ tgt, const void* __restrict__ dft,
    const float* __restrict__ uni, const float* __restrict__ tstats,
    const float* __restrict__ dstats, const int32_t* __restrict__ nacc, int K, int V,
    double yscale, int fast, int etab, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ num_emitted) {
  extern __shared__ double dyn[];
  __shared__ DrawShared<BLOCK> sh;
  const int64_t b = blockIdx.x;
  draw_sequence<BLOCK, DT>(b, nacc[b], tgt, dft, uni, tstats, dstats, K, V, yscale, fast, etab,
                           out_tokens, num_emitted, dyn, sh);
}

// One workgroup per sequence (the spec_verify_sample path): wave 0 runs the
// accept tests and the first-rejection scan (verify_seq) while the other
// waves fill the exp2 table and (bf16) the shared exponential table, then the
// whole workgroup draws the final token.  The same results as spec_verify followed
// by spec_residual_sample, in one launch.
template <int BLOCK, int DT>
__global__ __launch_bounds__(BLOCK) void verify_draw_kernel(
    const void* __restrict__ tgt, const void* __restrict__ dft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uni,
    const float* __restrict__ tstats, const float* __restrict__ dstats, int K, int V,
    double invT, double yscale, int fast, int etab, int32_t* __restrict__ num_accepted,
    int32_t* __restrict__ out_tokens, float* __restrict__ probs,
    int32_t* __restrict__ num_emitted) {
  static_assert(BLOCK > kWave, "waves other than the first fill the exp2 table");
  extern __shared__ double dyn[];
  __shared__ DrawShared<BLOCK> sh;
  const int64_t b = blockIdx.x;
  // stamps: 0 start, 1 scan and tables done, then draw_block's 2-5 and 6 at the end
  SPEC_STAMP(stamps_draw, 0);
  if (threadIdx.x < kWave) {
    const int n = verify_seq<DT, false>(b, tgt, dft, tokens, uni, tstats + 2 * b * (K + 1),
                                        dstats + 2 * b * K, K, V, invT, num_accepted,
                                        out_tokens, probs, true);
    if (threadIdx.x == 0) sh.sel[0] = n;
  } else {
    fill_exp2_table(sh.tab, kWave);
    if (DT == kBF16 && etab) fill_shared_exp_table<BLOCK>(dyn, yscale, kWave);
  }
  __syncthreads();
  SPEC_STAMP(stamps_draw, 1);
  const int n = uniform(sh.sel[0]);
  __syncthreads();  // sel[] is reused by the draw
  draw_sequence<BLOCK, DT>(b, n, tgt, dft, uni, tstats, dstats, K, V, yscale, fast, etab,
                           out_tokens, num_emitted, dyn, sh, true, DT == kBF16 && etab);
}

// ======================================================= split final draw
//
// The final draw with one sequence's sweep spread over P workgroups
// ("parts"), for batches with too few sequences to fill the device one
// workgroup per sequence, and to even out the residual and bonus draws'
// different costs.  Every part runs the accept scan (wave 0, while the other
// waves fill the exponential tables), sweeps its own contiguous range of
// items and stores their results as GlobalItems records; the part that
// finishes last -- counted on parts_done[b] -- reads every record back and
// draws exactly as one workgroup does after its own sweep (the same sums in
// the same order), so the token does not depend on P or on the block size.
// Part 0 writes the scan's outputs; the last part writes out_tokens[b][n] and
// num_emitted[b] and puts parts_done[b] back to 0 (it must be zero before the
// first launch and is zero after every completed one).
//
// Dynamic LDS: with etab (bf16 rows), the table exp(z/T) both rows share
// (kETab doubles), then max(ni, nch) doubles for the finish, then the LdsItems
// arrays of the part's own items (at most ceil(ni/P)).  Rows that cannot
// share the table (|m|/T > kSharedTableMax) compute their exponentials; the
// per-row tables of the one-workgroup draw hold the same values
// (row_tok_exp), so the bits agree.
struct SplitDraw {
  const void* tgt;
  const void* dft;
  const int32_t* tokens;
  const float* uni;
  const float* tstats;
  const float* dstats;
  int32_t* num_accepted;
  int32_t* out_tokens;
  float* probs;
  int32_t* num_emitted;
  unsigned* parts_done;  // [B]
  double* items;         // [B][ni][kItemRec]
  int K, V, P, ni, nch, etab;
  double invT, yscale;
};

template <int BLOCK, int DT>
__global__ __launch_bounds__(BLOCK, 4) void verify_draw_split_kernel(SplitDraw a) {
  static_assert(BLOCK > kWave, "waves other than the first fill the tables");
  constexpr int NW = BLOCK / kWave;
  extern __shared__ double dyn[];
  __shared__ DrawShared<BLOCK> sh;
  const int64_t b = blockIdx.x / static_cast<unsigned>(a.P);
  const int part = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.P));
  const int K = a.K, V = a.V, tid = threadIdx.x;
  const int64_t K1 = K + 1;
  const bool etab = DT == kBF16 && a.etab != 0;
  // stamps: 0 start, 1 scan and tables done, 2 sweep done, 3 records stored;
  // the finishing part: 4 counted last, 5 normalisers, 6 end
  SPEC_STAMP(stamps_draw, 0);
  if (tid < kWave) {
    const int n = verify_seq<DT, false>(b, a.tgt, a.dft, a.tokens, a.uni, a.tstats + 2 * b * K1,
                                        a.dstats + 2 * b * K, K, V, a.invT, a.num_accepted,
                                        a.out_tokens, a.probs, true, part == 0);
    if (tid == 0) sh.sel[0] = n;
  } else {
    fill_exp2_table(sh.tab, kWave);
    if (etab) fill_shared_exp_table<BLOCK>(dyn, a.yscale, kWave);
  }
  __syncthreads();
  SPEC_STAMP(stamps_draw, 1);
  const int n = uniform(sh.sel[0]);
  DrawRows R;
  bool rows_ok = false;
  if (n >= 0 && n <= K) {
    const int64_t rq = b * K1 + n, rp = b * K + (n < K ? n : 0);
    rows_ok = make_draw_rows<DT>(b, n, K, V, a.tgt, a.dft, a.tstats[2 * rq],
                                 a.tstats[2 * rq + 1], a.dstats[2 * rp], a.dstats[2 * rp + 1],
                                 a.yscale, R);
  }
  if (rows_ok && etab && draw_rows_share_table(R)) use_shared_table(R, dyn);
  double* work = dyn + (etab ? kETab : 0);
  const GlobalItems it(a.items + b * static_cast<int64_t>(a.ni) * kItemRec, a.ni);
  if (rows_ok) {
    const int s0 = static_cast<int>(static_cast<int64_t>(part) * a.ni / a.P);
    const int s1 = static_cast<int>(static_cast<int64_t>(part + 1) * a.ni / a.P);
    // this part's items in LDS (after the finish's W area), written out below
    const LdsItems own(work + max(a.ni, a.nch), s1 - s0);
    if (tid == 0) sh.next = s0 + NW;
    __syncthreads();  // also orders the scan's sel[0] read before later uses of sel[]
    const int wv = uniform(tid / kWave);
    auto emit = [&](int c, const ChunkSums& cs, double lq, double lp) {
      own.emit(c - s0, cs, lq, lp);
    };
    if (R.et != nullptr) {
      if (R.mode == kModeResidual)
        wave_sweep_claimed<DT, kModeResidual, kDrawG, true>(R, s0 + wv, s1, a.nch, &sh.next,
                                                            sh.tab, emit);
      else
        wave_sweep_claimed<DT, kModeBonus, kDrawG, true>(R, s0 + wv, s1, a.nch, &sh.next, sh.tab,
                                                         emit);
    } else {
      if (R.mode == kModeResidual)
        wave_sweep_claimed<DT, kModeResidual, kDrawG, false>(R, s0 + wv, s1, a.nch, &sh.next,
                                                             sh.tab, emit);
      else
        wave_sweep_claimed<DT, kModeBonus, kDrawG, false>(R, s0 + wv, s1, a.nch, &sh.next,
                                                          sh.tab, emit);
    }
    __syncthreads();
    SPEC_STAMP(stamps_draw, 2);
    it.write_from(own, s0, s1 - s0);
  }
  // this part's records are complete (device-coherent) before it is counted
  store_complete();
  __syncthreads();
  SPEC_STAMP(stamps_draw, 3);
  if (tid == 0) {
    sh.sel[3] = 0;
    sh.last = atomic_add_dev(&a.parts_done[b], 1u) == static_cast<unsigned>(a.P - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (sh.last == 0u) return;

  // ------------------------------------- the last part: the sequence's draw
  if (n < 0 || n > K || !rows_ok) {
    if (tid == 0) {
      if (n >= 0 && n <= K) a.out_tokens[b * K1 + n] = -1;
      if (a.num_emitted) a.num_emitted[b] = 0;
      atomic_store_dev(&a.parts_done[b], 0u);
    }
    return;
  }
  SPEC_STAMP(stamps_draw, 4);
  const double u = a.uni[b * K1 + K];
  const GlobalItemsAhead ita(it, a.ni);
  double Sq, Sp;
  item_normalisers<BLOCK>(ita, a.ni, sh, Sq, Sp);  // its barrier orders the sel[3] clear
  SPEC_STAMP(stamps_draw, 5);
  int tok;
  if (R.et != nullptr) {
    tok = fast_finish<BLOCK, DT, true, kDrawG>(R, a.ni, Sq, Sp, ita, work, u, sh);
    if (tok == -3) {  // residual without mass: the bonus draw from q_n
      DrawRows Rb = R;
      Rb.mode = kModeBonus;
      tok = slow_draw<BLOCK, DT, true>(Rb, a.nch, work, u, sh);
    } else if (tok == -2) {
      tok = slow_draw<BLOCK, DT, true>(R, a.nch, work, u, sh, true, Sq, Sp);
    }
  } else {
    tok = fast_finish<BLOCK, DT, false, kDrawG>(R, a.ni, Sq, Sp, ita, work, u, sh);
    if (tok == -3) {
      DrawRows Rb = R;
      Rb.mode = kModeBonus;
      tok = slow_draw<BLOCK, DT, false>(Rb, a.nch, work, u, sh);
    } else if (tok == -2) {
      tok = slow_draw<BLOCK, DT, false>(R, a.nch, work, u, sh, true, Sq, Sp);
    }
  }
  if (tid == 0) {
    a.out_tokens[b * K1 + n] = tok;
    if (a.num_emitted) a.num_emitted[b] = tok >= 0 ? n + 1 : 0;
    atomic_store_dev(&a.parts_done[b], 0u);
  }
  SPEC_STAMP(stamps_draw, 6);
}

// ============================================================ draft sampling
//
// Draft-side sampling ("Algorithm: Speculative Sampling (SpS)", alg. 2 step
// 1; "Decoding transforms"): one token per row from softmax(z/T), by the
// same exact inverse CDF as the bonus draw (weights exp((z-m)/T) in fp64,
// ascending token id, strict >).  One workgroup per row; stats {m, s} of the
// row come from stats_kernel.

template <int BLOCK, int DT>
__global__ __launch_bounds__(BLOCK) void sample_kernel(const void* __restrict__ logits,
                                                       const float* __restrict__ stats,
                                                       const float* __restrict__ uni, int V,
                                                       double yscale, int fast, int etab,
                                                       int32_t* __restrict__ tokens) {
  extern __shared__ double dyn[];
  __shared__ DrawShared<BLOCK> sh;
  const int64_t r = blockIdx.x;
  const float m = stats[2 * r], s = stats[2 * r + 1];
  if (!row_ok(m, s)) {
    if (threadIdx.x == 0) tokens[r] = -1;
    return;
  }
  DrawRows R;
  R.qrow = static_cast<const char*>(logits) + r * static_cast<int64_t>(V) * Elt<DT>::bytes;
  R.prow = R.qrow;
  R.V = V;
  R.mode = kModeBonus;
  R.aligned = (reinterpret_cast<uintptr_t>(R.qrow) & 15) == 0;
  R.yscale = yscale;
  R.mq = m;
  R.mp = 0.0;
  R.cq = 1.0;
  R.cp = 1.0;
  R.et = nullptr;
  R.etp = nullptr;
  R.k_hi = uniform_margin(true);
  R.k_lo = uniform_margin(false);
  R.rho = 1.0;
  fill_exp2_table(sh.tab);
  __syncthreads();
  double* work = dyn;
  if (DT == kBF16 && etab) {  // dynamic LDS starts with the row's table
    fill_row_exp_tables<BLOCK>(dyn, 1, R, sh.tab);
    __syncthreads();
    R.et = dyn;
    R.etp = dyn;
    work = dyn + kETab;
  }
  const int tok = R.et != nullptr ? draw_block<BLOCK, DT, true>(R, uni[r], fast, work, sh)
                                  : draw_block<BLOCK, DT, false>(R, uni[r], fast, work, sh);
  if (threadIdx.x == 0) tokens[r] = tok;
}

// One read per row (bf16 rows whose table and fast-sweep arrays fit in LDS):
// the bonus sweep over a table of exp(z/T) also tracks the row's
// maximum and any NaN, so the row's statistics come from the sweep's own
// sums -- s = S * exp(-m/T) with S = sum_x exp(z_x/T) formed in fp64 (the
// quantity stats_kernel forms from fp32 terms, here more precise) -- and
// the draw uses the same item sums.  A row whose maximum is too large for
// that table (|m|/T > kSharedTableMax) is drawn again from a table of its
// own, with the maximum subtracted.  Rows that define no distribution get token -1 and s = NaN, as
// with stats_kernel and sample_kernel.
template <int BLOCK>
__global__ __launch_bounds__(BLOCK) void sample_onepass_kernel(const void* __restrict__ logits,
                                                               const float* __restrict__ uni,
                                                               int V, double yscale,
                                                               float* __restrict__ stats_out,
                                                               int32_t* __restrict__ tokens) {
  constexpr int DT = kBF16;
  constexpr int NW = BLOCK / kWave;
  extern __shared__ double dyn[];
  __shared__ DrawShared<BLOCK> sh;
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  DrawRows R;
  R.qrow = static_cast<const char*>(logits) + r * static_cast<int64_t>(V) * Elt<DT>::bytes;
  R.prow = R.qrow;
  R.V = V;
  R.mode = kModeBonus;
  R.aligned = (reinterpret_cast<uintptr_t>(R.qrow) & 15) == 0;
  R.yscale = yscale;
  R.mq = 0.0;
  R.mp = 0.0;
  R.cq = 1.0;
  R.cp = 1.0;
  R.et = nullptr;
  R.etp = nullptr;
  R.k_hi = uniform_margin(true);
  R.k_lo = uniform_margin(false);
  R.rho = 1.0;
  fill_exp2_table(sh.tab);
  if (tid == 0) {
    sh.next = NW;
    sh.sel[3] = 0;
  }
  __syncthreads();
  // the table of exp(z/T) (maximum 0, factor 1), from the fp64 exponential
  // the other codes and the per-row tables use
  fill_row_exp_tables<BLOCK>(dyn, 1, R, sh.tab);
  __syncthreads();
  R.et = dyn;
  R.etp = dyn;
  double* work = dyn + kETab;
  const int nch = (V + kWave * 8 - 1) / (kWave * 8);
  const int ni = (nch + kDrawG - 1) / kDrawG;
  const LdsItems it(work + ni, ni);
  auto emit = [&](int c, const ChunkSums& cs, double lq, double lp) { it.emit(c, cs, lq, lp); };
  RowTrack trk;
  wave_sweep_claimed<DT, kModeBonus, kDrawG, true, decltype(emit), true>(
      R, uniform(tid / kWave), ni, nch, &sh.next, sh.tab, emit, &trk);
  // the row's maximum and NaN flag (block_max's barriers also end the sweep)
  const float m = block_max<BLOCK>(trk.value(), sh.redf);
  const bool nan = (trk.mag & 0xFFFFu) > 0x7F80u || (trk.mag >> 16) > 0x7F80u;
  const bool bad = block_max<BLOCK>(nan ? 1.0f : 0.0f, sh.redf) > 0.0f || !__builtin_isfinite(m);
  const double invT = yscale / Exp64::kScale;
  const double u = uni[r];
  int tok = -1;
  double srow = __builtin_nan("");
  if (!bad && fabs(static_cast<double>(m)) * invT <= kSharedTableMax) {
    tok = fast_finish<BLOCK, DT, true, kDrawG>(R, ni, 1.0, 1.0, it, work, u, sh);
    srow = sh.seld[2] * exp(-static_cast<double>(m) * invT);  // S_w = sum_x exp(z_x/T)
  } else if (!bad) {
    // a table of the row's own: exp((z - m)/T); its sweep's total is s itself
    R.mq = m;
    R.et = nullptr;
    R.etp = nullptr;
    R.k_hi = uniform_margin(true);
    R.k_lo = uniform_margin(false);
    fill_row_exp_tables<BLOCK>(dyn, 1, R, sh.tab);
    __syncthreads();
    R.et = dyn;
    R.etp = dyn;
    tok = draw_block<BLOCK, DT, true>(R, u, 1, work, sh);
    srow = sh.seld[2];
  }
  if (tid == 0) {
    tokens[r] = tok;
    stats_out[2 * r] = m;
    stats_out[2 * r + 1] = static_cast<float>(srow);
  }
}

// ================================================================== greedy
//
// Greedy verify (Pitfalls, greedy mode: the general rule applied to one-hot
// distributions): a_t = argmax of target row t; accept drafted tokens while
// they equal a_t; emit a_n at the first mismatch (or a_K after K matches).
// argmax_kernel: one workgroup per target row, streaming like stats_kernel:
// per group the max (v_max3), and the group's first maximal element only when
// the group beats the thread's best so far; NaN anywhere invalidates the row.

template <int BLOCK, int DT, int VPG>
__global__ __launch_bounds__(BLOCK) void argmax_kernel(const void* __restrict__ rows, int V,
                                                       int32_t* __restrict__ argmax) {
  constexpr int EB = Elt<DT>::bytes;
  constexpr int EPV = 16 / EB;
  constexpr int STEP = BLOCK * VPG;
  constexpr int NW = BLOCK / kWave;
  __shared__ float red_v[NW];
  __shared__ int red_i[NW];
  __shared__ unsigned red_nan[NW];
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  const char* row = static_cast<const char*>(rows) + static_cast<int64_t>(blockIdx.x) * V * EB;
  const RowGeom<DT> G(row, V);
  float best = -__builtin_huge_valf();
  int best_i = 0x7fffffff;
  // NaN check in vector registers: the largest |bits| seen; a NaN is exactly
  // a value above 0x7F800000 (one ballot at the end, none in the loop)
  unsigned mag = 0u;
  auto note = [&](float v) { mag = max(mag, __float_as_uint(v) & 0x7FFFFFFFu); };
  // a candidate (value, index) that beats the best so far: larger, or equal
  // with a smaller index
  auto offer = [&](float v, int i) {
    if (v > best || (v == best && i < best_i)) {
      best = v;
      best_i = i;
    }
  };
  {  // head elements (indices below the body's)
    const float v = tid < G.head ? logit_f32<DT>(row, tid) : -__builtin_huge_valf();
    note(v);
    if (tid < G.head) offer(v, tid);
  }
  const char* body = row + static_cast<int64_t>(G.head) * EB;
  stream_body<BLOCK, DT, VPG, kLoadStream>(body, G.nvec, [&](const float(&x)[VPG * EPV], int i0) {
#pragma unroll
    for (int k = 0; k < VPG * EPV; ++k) note(x[k]);
    const float g = group_max(x);
    if (g > best) {  // rare after the first groups: find the group's first maximal element
      int gi = 0x7fffffff;
#pragma unroll
      for (int u = VPG - 1; u >= 0; --u)
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e)
          if (x[u * EPV + e] == g) gi = G.head + (i0 + u * BLOCK) * EPV + e;
      best = g;
      best_i = gi;
    }
  });
  {  // tail elements (indices above the body's), after it so that ties keep the body's
    const bool has = tid < V - G.tail0;
    const float v = has ? logit_f32<DT>(row, G.tail0 + tid) : -__builtin_huge_valf();
    note(v);
    if (has) offer(v, G.tail0 + tid);
  }
  const unsigned long long nanm = __ballot(mag > 0x7F800000u);
  // wave, then block: the largest value, and among equal values the smallest index
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, kWave);
    const int oi = __shfl_xor(best_i, o, kWave);
    if (ov > best || (ov == best && oi < best_i)) {
      best = ov;
      best_i = oi;
    }
  }
  if (lane == 0) {
    red_v[wv] = best;
    red_i[wv] = best_i;
    red_nan[wv] = nanm != 0ull ? 1u : 0u;
  }
  __syncthreads();
  if (tid == 0) {
    float bv = red_v[0];
    int bi = red_i[0];
    unsigned nan = red_nan[0];
    for (int w = 1; w < NW; ++w) {
      if (red_v[w] > bv || (red_v[w] == bv && red_i[w] < bi)) {
        bv = red_v[w];
        bi = red_i[w];
      }
      nan |= red_nan[w];
    }
    argmax[blockIdx.x] = (nan || !__builtin_isfinite(bv)) ? -1 : bi;
  }
}

// One wave per sequence: the greedy accept scan over the target argmaxes.
__global__ __launch_bounds__(kWave) void greedy_scan_kernel(const int32_t* __restrict__ argmax,
                                                            const int32_t* __restrict__ tokens,
                                                            int K, int V,
                                                            int32_t* __restrict__ num_accepted,
                                                            int32_t* __restrict__ out_tokens,
                                                            int32_t* __restrict__ num_emitted) {
  const int64_t b = blockIdx.x;
  const int64_t K1 = K + 1;
  const int t = lane_id();
  bool valid = true, mismatch = false;
  int x = -1;
  if (t <= K) valid = argmax[b * K1 + t] >= 0;
  if (t == 0) valid = valid && argmax[b * K1 + K] >= 0;  // the bonus row (lane K may not exist)
  if (t < K) {
    x = tokens[b * K + t];
    valid = valid && x >= 0 && x < V;
    mismatch = x != argmax[b * K1 + t];
  }
  const bool all_valid = __all(valid);
  const unsigned long long mm = __ballot(mismatch);
  const int n = !all_valid ? -1 : (mm ? __ffsll(static_cast<long long>(mm)) - 1 : K);
  if (t == 0) {
    num_accepted[b] = n;
    if (num_emitted) num_emitted[b] = n + 1;
  }
  for (int pos = t; pos <= K; pos += kWave) {
    int v = -1;
    if (n >= 0) v = pos < n ? tokens[b * K + pos] : (pos == n ? argmax[b * K1 + n] : -1);
    out_tokens[b * K1 + pos] = v;
  }
}

// ==================================================================== filter
//
// Decoding transforms (the card's Method, "Decoding transforms", and
// Pitfalls: temperature, top-k and nucleus applied alike to p and q before
// anything else): per row a logit threshold thr; tokens below it are removed
// (written as -inf into the output rows, and the other calls then run
// unchanged on them).
//   top-k (0 < k < V): thr_k = the k-th largest stored logit, ties kept.
//   nucleus (top_p < 1), over the top-k survivors: with masses
//     e = exp((z - m)/T), thr_p = the largest stored value v whose mass
//     sum_{z >= v} e reaches top_p * sum e.
// Both are radix selects over an order-preserving integer key of the stored
// value (16 bits for bf16, 32 for fp32), 8 bits per pass: a 256-bin
// histogram in LDS (counts, or masses) of the values whose key matches the
// digits chosen so far, and a walk from the top bin to the one where the
// running total reaches what is still needed.
//
// The thresholds of real rows lie close to the row maximum, so after a first
// pass for the maximum a second pass collects into LDS the values of a window
// at the top of the row, and the selects run over those few values.  The
// nucleus without top-k on bf16 rows usually does both in one read: it
// stages every body vector whose largest value lies near the block's running
// maximum (a superset of a window, since that maximum only grows toward the
// row's) and sums the mass of the other vectors.  The
// window is [L, m] with L the k-th largest of the per-thread maxima for top-k
// (k <= block size: at least k values lie at or above it), and otherwise the
// values within kFilterWindow powers of two of probability below the
// maximum.  A row whose nucleus threshold lies below that window (or whose
// window holds more than kFilterCap values) runs the selects over the whole
// row instead, one row read per digit.
//
// Masses are fixed-point integers (units of 2^-42 of the maximum's mass), so
// every sum is exact in any order and the kernel gives the same thresholds
// on every run.  Masses inside the window are fp64 exponentials; the mass
// below the window (needed only for the nucleus total without top-k) is a sum
// of fp32 exp2 terms each below 2^-16, rounded once to the same units.

constexpr int kFilterCap = 12288;
constexpr int kFilterMapVecs = 16384;  // 256 KB rows: bf16 up to 131072 tokens
// The 16-bit vector keys of the top-k first pass share the candidate array:
// they fill its last kFilterMapVecs / 2 floats, clear of the per-thread
// maxima the top-k window select keeps at its start.
constexpr int kFilterKeyOff = kFilterCap - kFilterMapVecs / 2;
static_assert(kFilterKeyOff >= 1024, "room for the per-thread maxima of a 1024-thread block");
constexpr float kFilterWindow = 16.0f;
// The one-read nucleus pass stages whole body vectors (16 bytes each, their
// indices as 16-bit words behind them) in the candidate array, against a
// shallower window: rows whose cut lies deeper fall back to the window pass.
constexpr float kFilterWindowOne = 12.0f;
constexpr int kStageCap = 2720;
// The staged values in the one-read window, compacted once for the selects.
constexpr int kWinCap = 3072;
// Above this top_p the cut of a typical row lies deeper than that window, and
// the two-read path (maximum, then the deeper window) is taken at once.
constexpr float kFilterOneReadMaxP = 0.97f;
static_assert(kStageCap * 18 <= kFilterCap * 4, "staged vectors and their indices fit");
constexpr double kMassScale = 4398046511104.0;  // 2^42: V * 2^42 < 2^63 for V <= 2^20

// Order-preserving key of a stored value; -0 is taken as +0 so that equal
// values share a key.
template <int DT>
__device__ __forceinline__ unsigned order_key(float x) {
  constexpr unsigned kSign = DT == kBF16 ? 0x8000u : 0x80000000u;
  constexpr unsigned kAll = DT == kBF16 ? 0xFFFFu : 0xFFFFFFFFu;
  unsigned b = __float_as_uint(x + 0.0f);
  if constexpr (DT == kBF16) b >>= 16;
  return (b & kSign) ? (~b & kAll) : (b | kSign);
}

template <int DT>
__device__ __forceinline__ float key_value(unsigned k) {
  constexpr unsigned kSign = DT == kBF16 ? 0x8000u : 0x80000000u;
  constexpr unsigned kAll = DT == kBF16 ? 0xFFFFu : 0xFFFFFFFFu;
  unsigned b = (k & kSign) ? (k & ~kSign) : (~k & kAll);
  if constexpr (DT == kBF16) b <<= 16;
  return __uint_as_float(b);
}

// Mass of one token in fixed point: round(exp((z - m)/T) * 2^42).
__device__ __forceinline__ unsigned long long mass_fixed(float z, float m, double yscale,
                                                         const double* tab) {
  const double e = exp64_scaled((static_cast<double>(z) - m) * yscale, tab);
  return static_cast<unsigned long long>(e * kMassScale + 0.5);
}

// f(x) for every stored value of a row (no padding), streaming the body with
// stream_body.
template <int BLOCK, int DT, int VPG, typename F>
__device__ __forceinline__ void for_each_value(const char* row, int V, F f) {
  constexpr int EPV = 16 / Elt<DT>::bytes;
  const int tid = threadIdx.x;
  const RowGeom<DT> G(row, V);
  if (tid < G.head) f(logit_f32<DT>(row, tid));
  const int nvec = G.nvec;
  stream_body<BLOCK, DT, VPG>(row + static_cast<int64_t>(G.head) * Elt<DT>::bytes, nvec,
                              [&](const float(&x)[VPG * EPV], int i0) {
#pragma unroll
                                for (int u = 0; u < VPG; ++u)
                                  if (i0 + u * BLOCK < nvec)
#pragma unroll
                                    for (int e = 0; e < EPV; ++e) f(x[u * EPV + e]);
                              });
  if (tid < V - G.tail0) f(logit_f32<DT>(row, G.tail0 + tid));
}

// g(x, i0) over a row in groups: x is a float array (one value for the head
// and tail elements, with i0 = -1; VPG vectors for the body, the thread's
// vectors i0 + u*BLOCK); every thread makes the same calls and entries past
// the row are -inf.  AUX: the body loads' cache policy (stream_body).
template <int BLOCK, int DT, int VPG, int AUX = kLoadDefault, typename G>
__device__ __forceinline__ void for_each_group(const char* row, int V, G g) {
  constexpr int EPV = 16 / Elt<DT>::bytes;
  const int tid = threadIdx.x;
  const RowGeom<DT> Gm(row, V);
  {
    const float x[1] = {tid < Gm.head ? logit_f32<DT>(row, tid) : -__builtin_huge_valf()};
    g(x, -1);
  }
  stream_body<BLOCK, DT, VPG, AUX>(row + static_cast<int64_t>(Gm.head) * Elt<DT>::bytes, Gm.nvec,
                                   [&](const float(&x)[VPG * EPV], int i0) { g(x, i0); });
  {
    const float x[1] = {tid < V - Gm.tail0 ? logit_f32<DT>(row, Gm.tail0 + tid)
                                           : -__builtin_huge_valf()};
    g(x, -1);
  }
}

__device__ __forceinline__ unsigned wave_incl_scan_u32(unsigned v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const unsigned o = static_cast<unsigned>(__shfl_up(static_cast<int>(v), d, kWave));
    if (lane >= d) v += o;
  }
  return v;
}

// Wave 0 walks hist[255..0] from the top: the first bin where the running
// total reaches `need`.  Writes the bin to *bin_out and what is still needed
// inside it (need minus the total above it) to *need_out.
__device__ __forceinline__ void walk_bins(const unsigned long long* hist, double need,
                                          int* bin_out, double* need_out) {
  const int lane = lane_id();
  double v[4];
  double ls = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // lane l holds bins 255-4l .. 252-4l, top first
    v[j] = static_cast<double>(hist[255 - 4 * lane - j]);
    ls = ls + v[j];
  }
  const double incl = wave_incl_scan_shfl(ls);
  const double excl = incl - ls;
  const unsigned long long hit = __ballot(incl >= need);
  // rounding of the running total can leave it a hair under `need`: then the
  // lowest bin holding anything is taken
  const int src = hit ? static_cast<int>(__builtin_ctzll(hit)) : -1;
  if (src < 0) {
    if (lane == 0) {
      int b = 0;
      for (int i = 0; i < 256; ++i)
        if (hist[i] != 0ull) {
          b = i;
          break;
        }
      *bin_out = b;
      *need_out = 0.0;
    }
    return;
  }
  if (lane == src) {
    double cum = excl;
    int b = 255 - 4 * lane - 3;
    double left = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (cum + v[j] >= need) {
        b = 255 - 4 * lane - j;
        left = need - cum;
        break;
      }
      cum = cum + v[j];
    }
    *bin_out = b;
    *need_out = left;
  }
}

template <int BLOCK>
struct FilterShared {
  double tab[Exp64::kTab];
  unsigned long long hist[256];
  float redf[BLOCK / kWave];
  double redd[BLOCK / kWave];
  unsigned long long redq[BLOCK / kWave];
  unsigned redu[BLOCK / kWave];
  int sel_bin;
  double sel_need;
  unsigned ncand;
  unsigned mkey;  // the one-read nucleus pass: order key of the running maximum
  unsigned nwin;  // ... and the count of its window values in win
  float win[kWinCap];
  // 16-byte aligned: the top-k first pass's vector keys, kept in its upper
  // part, are read back 16 bytes at a time
  alignas(16) float cand[kFilterCap];
  // one bit per 16-byte vector of the row body that holds a window value
  // (rows of at most kFilterMapVecs vectors)
  unsigned vmap[kFilterMapVecs / 32];
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <int BLOCK>
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v,
                                                            unsigned long long* red) {
  v = wave_sum_u64(v);
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  unsigned long long r = 0ull;
#pragma unroll
  for (int i = 0; i < BLOCK / kWave; ++i) r += red[i];
  return r;
}

template <int BLOCK>
__device__ __forceinline__ unsigned block_min_u32(unsigned v, unsigned* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned t = static_cast<unsigned>(__shfl_xor(static_cast<int>(v), o, kWave));
    v = t < v ? t : v;
  }
  __syncthreads();
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  unsigned r = red[0];
#pragma unroll
  for (int i = 1; i < BLOCK / kWave; ++i) r = red[i] < r ? red[i] : r;
  return r;
}

// Key (order_key) of the value at which the running total, from the top of
// the values `fe` visits (fe(f) calls f(x) once per value), first reaches the
// target: the count `target` (MASS false) or target * S in mass units (MASS
// true; S < 0: S is the mass of the visited values with key >= lower).  Only
// values with key >= lower take part.  Every visited key lies in
// [base, base + 2^span_bits); the digits are those of key - base, 8 bits a
// pass from the top, so values packed into a narrow key range still spread
// over the bins of the first pass.
template <int BLOCK, int DT, bool MASS, typename FE>
__device__ __forceinline__ unsigned radix_select(FE fe, unsigned lower, double target, double S,
                                                 float m, double yscale, unsigned base,
                                                 int span_bits, FilterShared<BLOCK>& sh) {
  const int tid = threadIdx.x, lane = lane_id();
  double need = MASS ? target * S : target;
  unsigned long long prefix = 0ull;
  bool first = true;
#pragma unroll 1
  for (int hi = span_bits; hi > 0; hi -= 8) {
    const int s = hi > 8 ? hi - 8 : 0;
    for (int i = tid; i < 256; i += BLOCK) sh.hist[i] = 0ull;
    __syncthreads();
    fe([&](float x) {
      const unsigned k = order_key<DT>(x);
      const unsigned long long d = static_cast<unsigned long long>(k - base);
      if (k >= lower && (d >> hi) == prefix)
        atomicAdd(&sh.hist[static_cast<unsigned>(d >> s) & 255u],
                  MASS ? mass_fixed(x, m, yscale, sh.tab) : 1ull);
    });
    __syncthreads();
    if (tid < kWave) {
      if (MASS && first && S < 0.0) {
        double ls = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) ls = ls + static_cast<double>(sh.hist[4 * lane + j]);
        need = target * wave_sum(ls);
      }
      walk_bins(sh.hist, need, &sh.sel_bin, &sh.sel_need);
    }
    __syncthreads();
    prefix = (prefix << (hi - s)) | static_cast<unsigned long long>(sh.sel_bin);
    need = sh.sel_need;
    first = false;
  }
  return base + static_cast<unsigned>(prefix);
}

// The last pass over a row: with WRITE, the output row (the input with every
// token below thr set to -inf; cut false: a plain copy); with STATS, this
// thread's part of the filtered row's normaliser sum exp2((z - m) c2) over
// the kept tokens (fp32 terms, fp64 sums; the same quantity as the stats
// kernel's s).  16-byte accesses where input and output rows share their
// offset within 16 bytes (or when only reading).
template <int BLOCK, int DT, bool WRITE, bool STATS>
__device__ __forceinline__ double finish_row(const char* row, char* orow, int V, bool cut,
                                             float thr, float m, float c2) {
  using Bits = typename std::conditional<DT == kBF16, uint16_t, uint32_t>::type;
  constexpr Bits kNegInf = DT == kBF16 ? Bits(0xFF80u) : Bits(0xFF800000u);
  constexpr int EB = Elt<DT>::bytes;
  const int tid = threadIdx.x;
  const Bits* src = reinterpret_cast<const Bits*>(row);
  Bits* dst = reinterpret_cast<Bits*>(orow);
  double acc = 0.0;
  // one stored value: its output bits, and its term added to t
  auto one = [&](Bits b, float& t) -> Bits {
    const float z = DT == kBF16 ? __uint_as_float(static_cast<uint32_t>(b) << 16)
                                : __uint_as_float(static_cast<uint32_t>(b));
    const bool drop = cut && z < thr;
    if (STATS) t += drop ? 0.0f : __builtin_amdgcn_exp2f((z - m) * c2);
    return drop ? kNegInf : b;
  };
  auto word = [&](uint32_t w, float& t) -> uint32_t {
    if constexpr (DT == kBF16) {
      const uint32_t lo = one(static_cast<Bits>(w & 0xFFFFu), t);
      const uint32_t hi = one(static_cast<Bits>(w >> 16), t);
      return lo | (hi << 16);
    } else {
      return one(w, t);
    }
  };
  auto scalar = [&](int i) {
    float t = 0.0f;
    const Bits o = one(src[i], t);
    if (WRITE) dst[i] = o;
    acc += static_cast<double>(t);
  };
  if (WRITE && ((reinterpret_cast<uintptr_t>(row) ^ reinterpret_cast<uintptr_t>(orow)) & 15) != 0) {
    for (int i = tid; i < V; i += BLOCK) scalar(i);
    return acc;
  }
  const RowGeom<DT> G(row, V);
  if (tid < G.head) scalar(tid);
  if (tid < V - G.tail0) scalar(G.tail0 + tid);
  // the row's last read and the output's only write: non-temporal both
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u* vs = reinterpret_cast<const v4u*>(row + static_cast<int64_t>(G.head) * EB);
  v4u* vd = reinterpret_cast<v4u*>(orow + static_cast<int64_t>(G.head) * EB);
  auto vec = [&](v4u v, int i) {
    float t = 0.0f;
    v4u o;
    o.x = word(v.x, t);
    o.y = word(v.y, t);
    o.z = word(v.z, t);
    o.w = word(v.w, t);
    if (WRITE) __builtin_nontemporal_store(o, &vd[i]);
    acc += static_cast<double>(t);
  };
  constexpr int U = 4;
  int i = tid;
  for (; i + (U - 1) * BLOCK < G.nvec; i += U * BLOCK) {
    v4u v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&vs[i + u * BLOCK]);
#pragma unroll
    for (int u = 0; u < U; ++u) vec(v[u], i + u * BLOCK);
  }
  for (; i < G.nvec; i += BLOCK) vec(__builtin_nontemporal_load(&vs[i]), i);
  return acc;
}

// The output row of a cut settled in LDS (input and output rows sharing their
// offset within 16 bytes): each body vector marked in vmap is read and cut
// (tokens below thr become -inf), every other body vector is written as
// -inf without being read; the head and tail elements are read and cut.
template <int BLOCK, int DT>
__device__ __forceinline__ void write_marked_row(const char* row, char* orow, int V, float thr,
                                                 const unsigned* vmap) {
  using Bits = typename std::conditional<DT == kBF16, uint16_t, uint32_t>::type;
  constexpr Bits kNegInf = DT == kBF16 ? Bits(0xFF80u) : Bits(0xFF800000u);
  constexpr uint32_t kNegInfWord = DT == kBF16 ? 0xFF80FF80u : 0xFF800000u;
  constexpr int EB = Elt<DT>::bytes;
  const int tid = threadIdx.x;
  const Bits* src = reinterpret_cast<const Bits*>(row);
  Bits* dst = reinterpret_cast<Bits*>(orow);
  auto one = [&](Bits b) -> Bits {
    const float z = DT == kBF16 ? __uint_as_float(static_cast<uint32_t>(b) << 16)
                                : __uint_as_float(static_cast<uint32_t>(b));
    return z < thr ? kNegInf : b;
  };
  auto word = [&](uint32_t w) -> uint32_t {
    if constexpr (DT == kBF16) {
      return static_cast<uint32_t>(one(static_cast<Bits>(w & 0xFFFFu))) |
             (static_cast<uint32_t>(one(static_cast<Bits>(w >> 16))) << 16);
    } else {
      return one(w);
    }
  };
  const RowGeom<DT> G(row, V);
  if (tid < G.head) dst[tid] = one(src[tid]);
  if (tid < V - G.tail0) dst[G.tail0 + tid] = one(src[G.tail0 + tid]);
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u* vs = reinterpret_cast<const v4u*>(row + static_cast<int64_t>(G.head) * EB);
  v4u* vd = reinterpret_cast<v4u*>(orow + static_cast<int64_t>(G.head) * EB);
  v4u ninf;
  ninf.x = ninf.y = ninf.z = ninf.w = kNegInfWord;
  for (int i = tid; i < G.nvec; i += BLOCK) {
    v4u o = ninf;
    if ((vmap[i >> 5] >> (i & 31)) & 1u) {
      const v4u v = vs[i];
      o.x = word(v.x);
      o.y = word(v.y);
      o.z = word(v.z);
      o.w = word(v.w);
    }
    __builtin_nontemporal_store(o, &vd[i]);
  }
}

// The output row of a bf16 cut settled over the one-read pass's staged
// vectors (input and output rows sharing their offset within 16 bytes): no
// body vector is read again.  Every vector not marked in vmap is written as
// -inf, and each marked one (a staged vector holding a kept token) is written
// cut from its staged copy; the head and tail elements are read and cut.
template <int BLOCK>
__device__ __forceinline__ void write_staged_row(const char* row, char* orow, int V, float thr,
                                                 const unsigned* vmap, const uint4* stage,
                                                 const unsigned short* sidx, int n_stage) {
  const int tid = threadIdx.x;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(row);
  uint16_t* dst = reinterpret_cast<uint16_t*>(orow);
  auto one = [&](uint32_t b) -> uint32_t {
    return __uint_as_float(b << 16) < thr ? 0xFF80u : b;
  };
  auto word = [&](uint32_t w) -> uint32_t { return one(w & 0xFFFFu) | (one(w >> 16) << 16); };
  const RowGeom<kBF16> G(row, V);
  if (tid < G.head) dst[tid] = static_cast<uint16_t>(one(src[tid]));
  if (tid < V - G.tail0) dst[G.tail0 + tid] = static_cast<uint16_t>(one(src[G.tail0 + tid]));
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u* vd = reinterpret_cast<v4u*>(orow + static_cast<int64_t>(G.head) * 2);
  v4u ninf;
  ninf.x = ninf.y = ninf.z = ninf.w = 0xFF80FF80u;
  for (int i = tid; i < G.nvec; i += BLOCK)
    if (((vmap[i >> 5] >> (i & 31)) & 1u) == 0u) __builtin_nontemporal_store(ninf, &vd[i]);
  for (int j = tid; j < n_stage; j += BLOCK) {
    const unsigned vi = sidx[j];
    if (vi < static_cast<unsigned>(G.nvec) && ((vmap[vi >> 5] >> (vi & 31)) & 1u) != 0u) {
      const uint4 w = stage[j];
      v4u o;
      o.x = word(w.x);
      o.y = word(w.y);
      o.z = word(w.z);
      o.w = word(w.w);
      __builtin_nontemporal_store(o, &vd[vi]);
    }
  }
}

template <int BLOCK, int DT, int VPG>
__global__ __launch_bounds__(BLOCK) void filter_kernel(const void* in, void* out, int V,
                                                       float c2, double yscale, int top_k,
                                                       float top_p, float* thr_out,
                                                       float* stats_out) {
  constexpr int NW = BLOCK / kWave;
  __shared__ FilterShared<BLOCK> sh;
  const int tid = threadIdx.x, lane = lane_id(), wv = tid / kWave;
  constexpr int EPV = 16 / Elt<DT>::bytes;
  const int64_t r = blockIdx.x;
  const char* row = static_cast<const char*>(in) + r * static_cast<int64_t>(V) * Elt<DT>::bytes;
  // whether the window pass can mark the body vectors that hold its values
  const bool map_ok = RowGeom<DT>(row, V).nvec <= kFilterMapVecs;
  fill_exp2_table(sh.tab);
  if (tid == 0) sh.ncand = 0u;

  const bool use_k = top_k > 0, use_p = top_p < 1.0f;
  // Top-k with k <= BLOCK: the window needs only the row's largest values, so
  // the first pass also keeps each body vector's largest key (its top 16
  // bits) in LDS, and the window pass reads just the vectors whose key
  // reaches the window.  Otherwise the window pass reads the whole row again.
  const bool skip = use_k && top_k <= BLOCK && map_ok;
  constexpr int KS = DT == kF32 ? 16 : 0;  // key bits dropped
  unsigned short* vkey = reinterpret_cast<unsigned short*>(sh.cand + kFilterKeyOff);
  const RowGeom<DT> Gm(row, V);

  // No transform: the threshold is -inf (NaN for a row that defines no
  // distribution), the row is copied when the output is another buffer, and
  // the stats are the row's own.  One streamed pass does all three: each
  // body vector is stored to the output as it arrives, the maximum and NaN
  // are tracked, and with stats every value folds into the stats kernel's
  // accumulator.  (An output at another offset within 16 bytes takes the
  // general path below.)
  if (!use_k && !use_p) {
    char* orow = (out != nullptr && out != in)
                     ? static_cast<char*>(out) + r * static_cast<int64_t>(V) * Elt<DT>::bytes
                     : nullptr;
    if (orow == nullptr ||
        ((reinterpret_cast<uintptr_t>(row) ^ reinterpret_cast<uintptr_t>(orow)) & 15) == 0) {
      using Bits = typename std::conditional<DT == kBF16, uint16_t, uint32_t>::type;
      const bool want = stats_out != nullptr;
      RowAcc acc;
      float mx0 = -__builtin_huge_valf();
      bool nan = false;
      auto scalar = [&](int i) {
        const float x[1] = {logit_f32<DT>(row, i)};
        if (orow != nullptr)
          reinterpret_cast<Bits*>(orow)[i] = reinterpret_cast<const Bits*>(row)[i];
        mx0 = fmaxf(mx0, x[0]);
        nan = nan || x[0] != x[0];
        if (want) fold(acc, x, c2);
      };
      if (tid < Gm.head) scalar(tid);
      if (tid < V - Gm.tail0) scalar(Gm.tail0 + tid);
      typedef unsigned int v4u __attribute__((ext_vector_type(4)));
      v4u* vd = orow != nullptr
                    ? reinterpret_cast<v4u*>(orow + static_cast<int64_t>(Gm.head) * Elt<DT>::bytes)
                    : nullptr;
      stream_body<BLOCK, DT, VPG, kLoadStream>(
          row + static_cast<int64_t>(Gm.head) * Elt<DT>::bytes, Gm.nvec,
          [&](const float(&x)[VPG * EPV], int i0) {
            if (vd != nullptr) {
#pragma unroll
              for (int u = 0; u < VPG; ++u)
                if (i0 + u * BLOCK < Gm.nvec) {  // the stored bits, repacked
                  v4u o;
                  if constexpr (DT == kBF16) {
                    float z8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) z8[e] = x[u * EPV + e];
                    const uint4 w = pack_bf16_words(z8);
                    o.x = w.x;
                    o.y = w.y;
                    o.z = w.z;
                    o.w = w.w;
                  } else {
                    o.x = __float_as_uint(x[u * EPV]);
                    o.y = __float_as_uint(x[u * EPV + 1]);
                    o.z = __float_as_uint(x[u * EPV + 2]);
                    o.w = __float_as_uint(x[u * EPV + 3]);
                  }
                  __builtin_nontemporal_store(o, &vd[i0 + u * BLOCK]);
                }
            }
            mx0 = fmaxf(mx0, group_max(x));
#pragma unroll
            for (int e = 0; e < VPG * EPV; ++e) nan = nan || x[e] != x[e];
            if (want) fold(acc, x, c2);
          });
      const float m0 = block_max<BLOCK>(mx0, sh.redf);
      const bool wave_nan = __ballot(nan) != 0ull;  // every lane votes
      if (lane == 0) sh.redu[wv] = wave_nan ? 1u : 0u;
      __syncthreads();
      bool bad0 = !__builtin_isfinite(m0);
      for (int w = 0; w < NW; ++w) bad0 = bad0 || sh.redu[w] != 0u;
      if (tid == 0) thr_out[r] = bad0 ? __builtin_nanf("") : -__builtin_huge_valf();
      if (want) {
        float sf = __builtin_nanf("");
        if (!bad0) {
          if (fabsf(m0 * c2) < kShiftMax) {
            const float kr = rintf(m0 * c2);
            const double sum =
                block_sum<BLOCK>(ldexp(acc.s, static_cast<int>(acc.k - kr)), sh.redd);
            const double t =
                static_cast<double>(kr) - static_cast<double>(m0) * static_cast<double>(c2);
            sf = static_cast<float>(sum * exp2(t));
          } else {
            sf = static_cast<float>(row_stats_wide<BLOCK, DT>(row, V, c2, m0, sh.redf, sh.redd));
          }
        }
        if (tid == 0) {
          stats_out[2 * r] = m0;
          stats_out[2 * r + 1] = sf;
        }
      }
      return;
    }
  }

  // Nucleus without top-k on bf16 rows: one streamed read stages the body
  // vectors that can hold the window (see the one_read branch below); when
  // the cut lies in that window, the output is written from the staged copies
  // of the vectors holding kept tokens, and no body vector is read again.
  const bool one_read =
      DT == kBF16 && use_p && !use_k && map_ok && top_p <= kFilterOneReadMaxP;
  uint4* stage = reinterpret_cast<uint4*>(sh.cand);
  unsigned short* sidx = reinterpret_cast<unsigned short*>(stage + kStageCap);
  // rest1's terms are exp2(x c2 - mc): mc is mref c2 rounded to fp32, and the
  // terms are exact relative to it (one rounding of the argument, in the fma)
  float mref = -__FLT_MAX__, mc = -__FLT_MAX__;
  double rest1 = 0.0;

  // max, min and NaN
  float mx = -__builtin_huge_valf(), mn = __builtin_huge_valf();
  unsigned long long nanm = 0;
  if (one_read) {
    // Streamed once (non-temporal).  A body vector whose largest value is at
    // or above zhi, kFilterWindowOne powers of two of probability below the
    // largest value the block has published so far, is staged in LDS with its
    // index (a head or tail element as a vector of its own, index 0xFFFF);
    // since that maximum never exceeds the row's, every value of the window
    // [m - kFilterWindowOne/c2, m] lies in a staged vector.  The values of
    // the other vectors lie below that window, and their fp32 masses join
    // rest1.  The first body group takes the maximum over all waves (one
    // barrier); later groups read the LDS word without waiting.
    if (tid == 0) sh.mkey = 0u;
    __syncthreads();
    const float wdepth = kFilterWindowOne / c2;
    unsigned kseen = 0u;
    bool first = true;
    float tot1 = 0.0f;  // every term: NaN iff the row holds a NaN
    for_each_group<BLOCK, DT, VPG, kLoadStream>(row, V, [&](const auto& x, int i0) {
      constexpr int N = sizeof(x) / sizeof(float);
      constexpr int NV = N > 1 ? N / EPV : 1;  // vectors
      constexpr int L = N > 1 ? EPV : 1;       // values per vector
      float vmx[NV];
      float gm = -__builtin_huge_valf();
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        vmx[v] = x[v * L];
#pragma unroll
        for (int e = 1; e < L; ++e) vmx[v] = fmaxf(vmx[v], x[v * L + e]);
        gm = fmaxf(gm, vmx[v]);
      }
      mx = fmaxf(mx, gm);
      // (no minimum: whether the cut removes anything is counted afterwards)
      const unsigned kg = order_key<DT>(gm);
      if (N > 1 && first) {
        const float wm = wave_max(gm);
        if (lane == 0) atomicMax(&sh.mkey, order_key<DT>(wm));
        __syncthreads();
        first = false;
      } else if (kg > kseen) {
        atomicMax(&sh.mkey, kg);
      }
      const unsigned kb = __hip_atomic_load(&sh.mkey, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
      kseen = kb > kseen ? kb : kseen;
      kseen = kg > kseen ? kg : kseen;
      const float ms = key_value<DT>(kseen);
      // -inf values stay below zhi (their mass is 0)
      const float zhi = fmaxf(ms - wdepth, -__FLT_MAX__);
      // a new reference once the running maximum has risen by a power of two:
      // every term then stays under 2 (tot1 cannot overflow), and those of the
      // vectors below zhi under 2^-11
      if ((ms - mref) * c2 >= 1.0f) {
        const float mc2 = ms * c2;
        rest1 *= static_cast<double>(__builtin_amdgcn_exp2f(mc - mc2));
        mref = ms;
        mc = mc2;
      }
      bool fl[NV];
      // slots in lane-major order from the ballots: the staged vectors of the
      // lanes below this one, and the wave's total
      unsigned below = 0u, total = 0u;
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float sv = __builtin_amdgcn_exp2f(__builtin_fmaf(x[v * L], c2, -mc));
#pragma unroll
        for (int e = 1; e < L; ++e) sv += __builtin_amdgcn_exp2f(__builtin_fmaf(x[v * L + e], c2, -mc));
        tot1 += sv;
        fl[v] = vmx[v] >= zhi;
        rest1 += static_cast<double>(fl[v] ? 0.0f : sv);
        const unsigned long long bm = __ballot(fl[v]);
        below += __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(bm >> 32),
                                           __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(bm), 0u));
        total += static_cast<unsigned>(__popcll(bm));
      }
      if (total != 0u) {  // wave-uniform
        unsigned base = 0u;
        if (lane == 0) base = atomicAdd(&sh.ncand, total);
        unsigned pos = uniform(base) + below;
#pragma unroll
        for (int v = 0; v < NV; ++v)
          if (fl[v]) {
            if (pos < static_cast<unsigned>(kStageCap)) {
              if constexpr (N > 1) {
                float z8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) z8[e] = x[v * L + e];
                stage[pos] = pack_bf16_words(z8);
                sidx[pos] = static_cast<unsigned short>(i0 + v * BLOCK);
              } else {
                stage[pos] = make_uint4(0xFF800000u | (__float_as_uint(x[0]) >> 16), 0xFF80FF80u,
                                        0xFF80FF80u, 0xFF80FF80u);
                sidx[pos] = 0xFFFFu;
              }
            }
            ++pos;
          }
      }
    });
    nanm |= __ballot(tot1 != tot1);
  } else if (skip) {
    // streamed once (non-temporal); padding entries are -inf and enter
    // neither the minimum nor the keys
    for_each_group<BLOCK, DT, VPG, kLoadStream>(row, V, [&](const auto& x, int i0) {
      constexpr int N = sizeof(x) / sizeof(float);
      if (N == 1) {  // a head or tail element (its minimum is taken below)
        mx = fmaxf(mx, x[0]);
        nanm |= __ballot(x[0] != x[0]);
      } else {
#pragma unroll
        for (int u = 0; u < N / EPV; ++u) {
          float vm = x[u * EPV], vn = x[u * EPV];
          bool nan = x[u * EPV] != x[u * EPV];
#pragma unroll
          for (int e = 1; e < EPV; ++e) {
            vm = fmaxf(vm, x[u * EPV + e]);
            vn = fminf(vn, x[u * EPV + e]);
            nan = nan || x[u * EPV + e] != x[u * EPV + e];
          }
          nanm |= __ballot(nan);
          mx = fmaxf(mx, vm);
          const int vi = i0 + u * BLOCK;
          if (vi < Gm.nvec) {
            mn = fminf(mn, vn);
            vkey[vi] = static_cast<unsigned short>(order_key<DT>(vm) >> KS);
          }
        }
      }
    });
    if (tid < Gm.head) mn = fminf(mn, logit_f32<DT>(row, tid));
    if (tid < V - Gm.tail0) mn = fminf(mn, logit_f32<DT>(row, Gm.tail0 + tid));
  } else {
    for_each_value<BLOCK, DT, VPG>(row, V, [&](float x) {
      mx = fmaxf(mx, x);
      mn = fminf(mn, x);
      nanm |= __ballot(x != x);
    });
  }
  const float m = block_max<BLOCK>(mx, sh.redf);
  float lo = -block_max<BLOCK>(-mn, sh.redf);  // the one-read pass leaves it for later
  if (lane == 0) sh.redu[wv] = nanm != 0ull ? 1u : 0u;
  __syncthreads();
  bool bad = !__builtin_isfinite(m);
  for (int w = 0; w < NW; ++w) bad = bad || sh.redu[w] != 0u;

  float zlo = m - kFilterWindow / c2;
  unsigned thr_key = 0;
  bool in_lds = false;  // the selects ran over the window's values in LDS
  int n_lds = 0;
  if (!bad && use_k && top_k <= BLOCK) {
    // top-k window: the k-th largest of the per-thread maxima.  Those k
    // maxima are k distinct values at or above it, so the window holds the
    // top-k set whatever its depth.
    sh.cand[tid] = mx;
    __syncthreads();
    auto fm = [&](auto f) { f(sh.cand[tid]); };
    constexpr int KB = DT == kBF16 ? 16 : 32;
    zlo = key_value<DT>(radix_select<BLOCK, DT, false>(fm, 0u, top_k, -1.0, m, yscale, 0u, KB, sh));
  }
  // The one-read nucleus pass: the cut settled over the staged vectors when
  // the window [zlo1, m] holds at least top_p of the row's mass.  Its values
  // are compacted into win once, and the selects run over that list alone.
  bool staged = false, staged_all = false;  // staged_all: the cut keeps every value
  int n_stage = 0, n_win = 0;
  float zlo1 = 0.0f;
  // f(x) for the window's values
  auto fw = [&](auto f) {
    for (int i = tid; i < n_win; i += BLOCK) f(sh.win[i]);
  };
  unsigned n_one = 0u;  // vectors the one-read pass staged (or tried to)
  if (one_read) {
    n_one = sh.ncand;
    if (tid == 0) sh.nwin = 0u;
    __syncthreads();  // read by every thread before a fallback clears it
  }
  if constexpr (DT == kBF16) {
    if (!bad && one_read && n_one <= static_cast<unsigned>(kStageCap)) {
      n_stage = static_cast<int>(n_one);
      zlo1 = m - kFilterWindowOne / c2;
      // the mass below the window: rest1, relative to mc (mref c2 rounded,
      // mref <= m), and the staged values below zlo1 as fp32 terms like the
      // window pass's; the values at or above zlo1 go to win
      double rest =
          rest1 * exp2(static_cast<double>(mc) - static_cast<double>(m) * static_cast<double>(c2));
      for (int i = tid; i < n_stage; i += BLOCK) {
        float z8[8];
        unpack16<kBF16>(stage[i], z8);
        float sv = 0.0f;
        unsigned c = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool in = z8[e] >= zlo1;
          c += in ? 1u : 0u;
          sv += in ? 0.0f : __builtin_amdgcn_exp2f((z8[e] - m) * c2);
        }
        rest += static_cast<double>(sv);
        if (c != 0u) {
          unsigned pos = atomicAdd(&sh.nwin, c);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (z8[e] >= zlo1) {
              if (pos < static_cast<unsigned>(kWinCap)) sh.win[pos] = z8[e];
              ++pos;
            }
        }
      }
      const double rest_all = block_sum<BLOCK>(rest, sh.redd);  // its barriers publish nwin
      const unsigned nw = sh.nwin;
      if (nw <= static_cast<unsigned>(kWinCap)) {
        n_win = static_cast<int>(nw);
        unsigned long long win = 0ull;
        fw([&](float x) { win += mass_fixed(x, m, yscale, sh.tab); });
        const unsigned long long win_all = block_sum_u64<BLOCK>(win, sh.redq);
        const double S = static_cast<double>(win_all) + rint(rest_all * kMassScale);
        if (static_cast<double>(win_all) >= static_cast<double>(top_p) * S) {
          staged = true;
          in_lds = true;
          unsigned kmin = 0xFFFFFFFFu;
          fw([&](float x) {
            const unsigned k = order_key<DT>(x);
            kmin = k < kmin ? k : kmin;
          });
          kmin = block_min_u32<BLOCK>(kmin, sh.redu);
          const unsigned span = order_key<DT>(m) - kmin;
          const int bits = span == 0u ? 0 : 32 - __builtin_clz(span);
          thr_key = radix_select<BLOCK, DT, true>(fw, 0u, top_p, S, m, yscale, kmin, bits, sh);
          // the cut removes something unless every value is kept: all kept
          // values lie in the window, so counting them there settles it
          const float tv = key_value<DT>(thr_key);
          unsigned long long nk = 0ull;
          fw([&](float x) { nk += x >= tv ? 1ull : 0ull; });
          staged_all = block_sum_u64<BLOCK>(nk, sh.redq) == static_cast<unsigned long long>(V);
        }
      }
    }
  }
  if (!bad && (use_k || use_p) && !staged) {
    // the window: values >= zlo go to LDS (one slot range per wave and
    // group, taken with one LDS atomic), and the body vectors that hold them
    // are marked; for the nucleus without top-k the fp32 mass below the
    // window is summed on the way
    const bool masses = use_p && !use_k;
    float rest = 0.0f;
    if (one_read) {  // the staged window missed the cut: a fresh window pass
      if (tid == 0) sh.ncand = 0u;
      __syncthreads();
      // which also takes the row's minimum (here from the head and tail)
      if (tid < Gm.head) mn = fminf(mn, logit_f32<DT>(row, tid));
      if (tid < V - Gm.tail0) mn = fminf(mn, logit_f32<DT>(row, Gm.tail0 + tid));
    }
    if (skip) {
      // the map from the keys: bit t of word w marks body vector 32w + t when
      // its key reaches zlo's (the dropped low key bits only widen the set,
      // so every value >= zlo lies in a marked vector)
      const unsigned zk = order_key<DT>(zlo) >> KS;
      const int nw = (Gm.nvec + 31) >> 5;
      constexpr int WPT = (kFilterMapVecs / 32 + BLOCK - 1) / BLOCK;  // map words per thread
      unsigned bits[WPT];
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        const int w = tid + j * BLOCK;
        unsigned b = 0u;
        if (w < nw) {
          const uint4* kv = reinterpret_cast<const uint4*>(vkey + 32 * w);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 k4 = kv[q];
            const unsigned kw[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int h = 0; h < 8; ++h) {
              const int t = 8 * q + h;
              const unsigned key = (kw[h >> 1] >> (16 * (h & 1))) & 0xFFFFu;
              b |= (32 * w + t < Gm.nvec && key >= zk) ? 1u << t : 0u;
            }
          }
          sh.vmap[w] = b;
        }
        bits[j] = b;
      }
      __syncthreads();  // every key is read before candidates overwrite them
      // values >= zlo of the head and tail elements and of the marked
      // vectors, appended with one LDS atomic per element or vector
      auto put = [&](const float* x, int nx) {
        unsigned c = 0u;
        for (int e = 0; e < nx; ++e) c += x[e] >= zlo ? 1u : 0u;
        if (c != 0u) {
          unsigned pos = atomicAdd(&sh.ncand, c);
          for (int e = 0; e < nx; ++e)
            if (x[e] >= zlo) {
              if (pos < static_cast<unsigned>(kFilterCap)) sh.cand[pos] = x[e];
              ++pos;
            }
        }
      };
      if (tid < Gm.head) {
        const float x = logit_f32<DT>(row, tid);
        put(&x, 1);
      }
      if (tid < V - Gm.tail0) {
        const float x = logit_f32<DT>(row, Gm.tail0 + tid);
        put(&x, 1);
      }
      const char* body = row + static_cast<int64_t>(Gm.head) * Elt<DT>::bytes;
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        unsigned b = bits[j];
        while (b != 0u) {
          const int vi = 32 * (tid + j * BLOCK) + __builtin_ctz(b);
          b &= b - 1u;
          float xv[EPV];
          unpack16<DT>(*reinterpret_cast<const uint4*>(body + static_cast<int64_t>(vi) * 16), xv);
          put(xv, EPV);
        }
      }
    } else {
      for (int i = tid; i < kFilterMapVecs / 32; i += BLOCK) sh.vmap[i] = 0u;
      __syncthreads();
      for_each_group<BLOCK, DT, VPG>(row, V, [&](const auto& x, int i0) {
        constexpr int N = sizeof(x) / sizeof(float);
        if (N > 1 && one_read) {  // padding past the row stays out of the minimum
#pragma unroll
          for (int u = 0; u < N / EPV; ++u) {
            float vn = x[u * EPV];
#pragma unroll
            for (int e = 1; e < EPV; ++e) vn = fminf(vn, x[u * EPV + e]);
            if (i0 + u * BLOCK < Gm.nvec) mn = fminf(mn, vn);
          }
        }
        unsigned c = 0u;
#pragma unroll
        for (int e = 0; e < N; ++e) c += x[e] >= zlo ? 1u : 0u;
        if (masses) {
#pragma unroll
          for (int e = 0; e < N; ++e) {
            const float t = __builtin_amdgcn_exp2f((x[e] - m) * c2);
            rest += x[e] >= zlo ? 0.0f : t;
          }
        }
        if (N > 1 && map_ok && c != 0u) {
#pragma unroll
          for (int u = 0; u < N / EPV; ++u) {
            bool any = false;
#pragma unroll
            for (int e = 0; e < EPV; ++e) any = any || x[u * EPV + e] >= zlo;
            const int vi = i0 + u * BLOCK;
            if (any) atomicOr(&sh.vmap[vi >> 5], 1u << (vi & 31));
          }
        }
        if (__ballot(c != 0u) != 0ull) {
          const unsigned incl = wave_incl_scan_u32(c);
          const unsigned total =
              static_cast<unsigned>(__shfl(static_cast<int>(incl), kWave - 1, kWave));
          unsigned base = 0u;
          if (lane == 0) base = atomicAdd(&sh.ncand, total);
          unsigned pos = uniform(base) + incl - c;
#pragma unroll
          for (int e = 0; e < N; ++e)
            if (x[e] >= zlo) {
              if (pos < static_cast<unsigned>(kFilterCap)) sh.cand[pos] = x[e];
              ++pos;
            }
        }
      });
    }
    if (one_read) lo = -block_max<BLOCK>(-mn, sh.redf);
    const double rest_all = masses ? block_sum<BLOCK>(static_cast<double>(rest), sh.redd) : 0.0;
    __syncthreads();
    const unsigned n = sh.ncand;
    const int nc = static_cast<int>(n);
    auto fe = [&](auto f) {
      for (int i = tid; i < nc; i += BLOCK) f(sh.cand[i]);
    };
    // the window's own mass, from the values in LDS (nucleus without top-k)
    unsigned long long win = 0ull;
    if (masses && n <= static_cast<unsigned>(kFilterCap))
      fe([&](float x) { win += mass_fixed(x, m, yscale, sh.tab); });
    const unsigned long long win_all = masses ? block_sum_u64<BLOCK>(win, sh.redq) : 0ull;
    const double S = static_cast<double>(win_all) + rint(rest_all * kMassScale);
    const bool fast = n <= static_cast<unsigned>(kFilterCap) &&
                      (use_k ? static_cast<unsigned>(top_k) <= n
                             : static_cast<double>(win_all) >= static_cast<double>(top_p) * S);
    if (fast) {
      in_lds = true;
      n_lds = nc;
      // key range of the values in LDS: [kmin, key(m)]
      unsigned kmin = 0xFFFFFFFFu;
      fe([&](float x) {
        const unsigned k = order_key<DT>(x);
        kmin = k < kmin ? k : kmin;
      });
      kmin = block_min_u32<BLOCK>(kmin, sh.redu);
      const unsigned span = order_key<DT>(m) - kmin;
      const int bits = span == 0u ? 0 : 32 - __builtin_clz(span);
      if (use_k)
        thr_key = radix_select<BLOCK, DT, false>(fe, 0u, top_k, -1.0, m, yscale, kmin, bits, sh);
      if (use_p) {
        const unsigned kp = radix_select<BLOCK, DT, true>(fe, thr_key, top_p, use_k ? -1.0 : S, m,
                                                          yscale, kmin, bits, sh);
        thr_key = thr_key > kp ? thr_key : kp;
      }
    } else {
      constexpr int KB = DT == kBF16 ? 16 : 32;
      auto fr = [&](auto f) { for_each_value<BLOCK, DT, VPG>(row, V, f); };
      if (use_k)
        thr_key = radix_select<BLOCK, DT, false>(fr, 0u, top_k, -1.0, m, yscale, 0u, KB, sh);
      if (use_p) {
        const unsigned kp =
            radix_select<BLOCK, DT, true>(fr, thr_key, top_p, -1.0, m, yscale, 0u, KB, sh);
        thr_key = thr_key > kp ? thr_key : kp;
      }
    }
  }
  float thr = -__builtin_huge_valf();
  if (bad) {
    thr = __builtin_nanf("");
  } else if (staged) {
    if (!staged_all) thr = key_value<DT>(thr_key);
  } else if ((use_k || use_p) && thr_key > order_key<DT>(lo)) {
    thr = key_value<DT>(thr_key);
  }
  if (tid == 0) thr_out[r] = thr;

  // the output row (none when out is null): removed tokens as -inf, the rest
  // copied when out != in; and the filtered row's stats {m, s} (s NaN for a
  // row that defines no distribution)
  const bool cut = thr > -__builtin_huge_valf();  // false for NaN too
  const bool write = out != nullptr && (cut || out != in);
  const bool want = stats_out != nullptr && !bad;
  // When the selects ran in LDS and something is cut, every kept token is in
  // LDS (the window lies at or below the threshold): s is summed there, in
  // fixed point (exact in any order).  Otherwise the last pass sums it.
  const bool s_lds = want && in_lds && cut;
  char* orow = write ? static_cast<char*>(out) + r * static_cast<int64_t>(V) * Elt<DT>::bytes
                     : nullptr;
  // When the cut was settled in LDS, every kept token lies in the window, so
  // a body vector that held no window value is all -inf in the output and
  // need not be read again: only the marked vectors (and the head and tail
  // elements) are, and after the one-read pass not even those.
  const bool marked = write && in_lds && cut && map_ok &&
                      ((reinterpret_cast<uintptr_t>(row) ^ reinterpret_cast<uintptr_t>(orow)) & 15) == 0;
  double part = 0.0;
  if (marked && staged) {
    // the vectors that hold a kept token: written from their staged copies
    for (int i = tid; i < kFilterMapVecs / 32; i += BLOCK) sh.vmap[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n_stage; i += BLOCK) {
      float z8[8];
      unpack16<kBF16>(stage[i], z8);
      bool keep = false;
#pragma unroll
      for (int e = 0; e < 8; ++e) keep = keep || z8[e] >= thr;
      const unsigned vi = sidx[i];
      if (keep && vi < static_cast<unsigned>(Gm.nvec)) atomicOr(&sh.vmap[vi >> 5], 1u << (vi & 31));
    }
    __syncthreads();
  }
  if (marked && staged) {
    if constexpr (DT == kBF16)
      write_staged_row<BLOCK>(row, orow, V, thr, sh.vmap, stage, sidx, n_stage);
  } else if (marked) {
    write_marked_row<BLOCK, DT>(row, orow, V, thr, sh.vmap);
  } else if (write && want && !s_lds) {
    part = finish_row<BLOCK, DT, true, true>(row, orow, V, cut, thr, m, c2);
  } else if (write) {
    (void)finish_row<BLOCK, DT, true, false>(row, orow, V, cut, thr, m, c2);
  } else if (want && !s_lds) {
    part = finish_row<BLOCK, DT, false, true>(row, nullptr, V, cut, thr, m, c2);
  }
  if (stats_out != nullptr) {
    double sum = 0.0;
    if (s_lds) {
      unsigned long long f = 0ull;
      if (staged) {
        fw([&](float z) {
          if (z >= thr) f += mass_fixed(z, m, yscale, sh.tab);
        });
      } else {
        for (int i = tid; i < n_lds; i += BLOCK) {
          const float z = sh.cand[i];
          if (z >= thr) f += mass_fixed(z, m, yscale, sh.tab);
        }
      }
      sum = static_cast<double>(block_sum_u64<BLOCK>(f, sh.redq)) * (1.0 / kMassScale);
    } else if (want) {
      sum = block_sum<BLOCK>(part, sh.redd);
    }
    if (tid == 0) {
      stats_out[2 * r] = m;
      stats_out[2 * r + 1] = want ? static_cast<float>(sum) : __builtin_nanf("");
    }
  }
}

}  // namespace spec
