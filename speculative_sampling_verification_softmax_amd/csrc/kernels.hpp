// kernels.hpp -- the three verify kernels for gfx950.
//
//   stats_kernel     one workgroup per logit row: max m and s = sum exp((z-m)/T)
//   verify_kernel    one wave per sequence: q, p at the drafted tokens, accept
//                    tests, first rejection
//   residual_kernel  one workgroup per sequence: fp64 residual (or bonus)
//                    weights on the row(s) at the first rejection, chunk sums,
//                    prefix scan and inverse-CDF draw
//
// What is computed: wikillm.com card for arXiv 2302.01318, Method
// ("Modified rejection sampling", paper sec. 4.2; "Algorithm: Speculative
// Sampling (SpS)", alg. 2 steps 2-4; "Decoding transforms") and Pitfalls.
#pragma once

#include "device_common.hpp"

namespace spec {

// ============================================================== stats_kernel
//
// HBM-bound streaming reduction.  Rows are split into an unaligned head, a
// body of 16-byte vectors (8 bf16 or 4 fp32 per load, fully coalesced across
// the wave) and a tail.  Each thread keeps a running (m, s): a group of
// VPG vectors is loaded, its max taken, s rescaled once per group, then
// s += exp2((x - m) * log2(e)/T) per element (x - m is exact for bf16
// inputs; only the product by the constant rounds).  Thread partials are
// brought to the row max and summed in fp64.

struct RowAcc {
  float m = -__builtin_huge_valf();
  float s = 0.f;
};

// Fold n values (already in fp32) into the running (m, s).
template <int N>
__device__ __forceinline__ void fold(RowAcc& a, const float (&x)[N], float c2) {
  float g = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) g = fmaxf(g, x[i]);
  const float mn = fmaxf(a.m, g);
  // While every value seen is -inf the shift is 0 and all terms are exp2(-inf)=0.
  const float ms = (mn == -__builtin_huge_valf()) ? 0.f : mn;
  float s = a.s * __builtin_amdgcn_exp2f((a.m - ms) * c2);
#pragma unroll
  for (int i = 0; i < N; ++i) s = s + __builtin_amdgcn_exp2f((x[i] - ms) * c2);
  a.m = mn;
  a.s = s;
}

template <int DT>
__device__ __forceinline__ void unpack(const uint4& v, float (&x)[16 / Elt<DT>::bytes]) {
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

template <int BLOCK, int DT, int VPG>
__global__ __launch_bounds__(BLOCK) void stats_kernel(const void* __restrict__ tgt,
                                                      const void* __restrict__ dft,
                                                      int64_t n_tgt_rows, int V, float c2,
                                                      float* __restrict__ tstats,
                                                      float* __restrict__ dstats) {
  constexpr int EB = Elt<DT>::bytes;
  constexpr int EPV = 16 / EB;  // elements per 16-byte vector
  __shared__ float red_f[BLOCK / kWave];
  __shared__ double red_d[BLOCK / kWave];

  int64_t r = blockIdx.x;
  const char* row;
  float* out;
  if (r < n_tgt_rows) {
    row = static_cast<const char*>(tgt) + r * static_cast<int64_t>(V) * EB;
    out = tstats + 2 * r;
  } else {
    r -= n_tgt_rows;
    row = static_cast<const char*>(dft) + r * static_cast<int64_t>(V) * EB;
    out = dstats + 2 * r;
  }
  const int tid = threadIdx.x;

  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int head = static_cast<int>(((16 - (addr & 15)) & 15) / EB);
  if (head > V) head = V;
  const int nvec = (V - head) / EPV;
  const int tail0 = head + nvec * EPV;

  RowAcc acc;
  // unaligned head and ragged tail: one element per thread
  if (tid < head) {
    float x[1] = {logit_f32<DT>(row, tid)};
    fold(acc, x, c2);
  }
  if (tid < V - tail0) {
    float x[1] = {logit_f32<DT>(row, tail0 + tid)};
    fold(acc, x, c2);
  }

  const uint4* vp = reinterpret_cast<const uint4*>(row + static_cast<int64_t>(head) * EB);
  constexpr int STEP = BLOCK * VPG;
  const int nfull = nvec / STEP;
  for (int it = 0; it < nfull; ++it) {
    const int i0 = it * STEP + tid;
    uint4 v[VPG];
#pragma unroll
    for (int u = 0; u < VPG; ++u) v[u] = vp[i0 + u * BLOCK];
    float x[VPG * EPV];
#pragma unroll
    for (int u = 0; u < VPG; ++u) {
      float xu[EPV];
      unpack<DT>(v[u], xu);
#pragma unroll
      for (int e = 0; e < EPV; ++e) x[u * EPV + e] = xu[e];
    }
    fold(acc, x, c2);
  }
  for (int i = nfull * STEP + tid; i < nvec; i += BLOCK) {
    uint4 v = vp[i];
    float x[EPV];
    unpack<DT>(v, x);
    fold(acc, x, c2);
  }

  // combine: row max, then every partial rescaled to it and summed in fp64
  const float m = block_max<BLOCK>(acc.m, red_f);
  const float ms = (m == -__builtin_huge_valf()) ? 0.f : m;
  const double part = static_cast<double>(acc.s * __builtin_amdgcn_exp2f((acc.m - ms) * c2));
  const double s = block_sum<BLOCK>(part, red_d);
  if (tid == 0) {
    float sf = static_cast<float>(s);
    if (!__builtin_isfinite(m)) sf = __builtin_nanf("");
    out[0] = m;
    out[1] = sf;
  }
}

// ============================================================= verify_kernel
//
// One wave per sequence; lane t runs accept test t.  q_t(x_t) and p_t(x_t)
// are formed in fp64 from the stored logit and the row stats, and the test
// is u < min(1, q/p) written as (u < 1) && (u*p < q), which also covers
// p = 0 (accept iff q > 0).  The first rejection is the lowest set bit of
// the wave's reject ballot.

template <int DT>
__global__ __launch_bounds__(kWave) void verify_kernel(
    const void* __restrict__ tgt, const void* __restrict__ dft,
    const int32_t* __restrict__ tokens, const float* __restrict__ uni,
    const float* __restrict__ tstats, const float* __restrict__ dstats,
    int K, int V, double invT, int32_t* __restrict__ num_accepted,
    int32_t* __restrict__ out_tokens, float* __restrict__ probs) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t K1 = K + 1;
  bool valid = true;
  bool reject = false;
  double q = 0.0, p = 0.0;
  int x = -1;
  if (t < K) {
    x = tokens[b * K + t];
    const int64_t rq = b * K1 + t, rp = b * K + t;
    const float mq = tstats[2 * rq], sq = tstats[2 * rq + 1];
    const float mp = dstats[2 * rp], sp = dstats[2 * rp + 1];
    valid = row_ok(mq, sq) && row_ok(mp, sp) && x >= 0 && x < V;
    if (valid) {
      const double zq = logit_f32<DT>(tgt, rq * V + x);
      const double zp = logit_f32<DT>(dft, rp * V + x);
      q = exp((zq - static_cast<double>(mq)) * invT) / static_cast<double>(sq);
      p = exp((zp - static_cast<double>(mp)) * invT) / static_cast<double>(sp);
      const double u = uni[b * K1 + t];
      const bool acc = (u < 1.0) && (u * p < q);
      reject = !acc;
    }
  }
  if (t == 0) {  // the bonus row is part of the sequence too
    const int64_t rk = b * K1 + K;
    valid = valid && row_ok(tstats[2 * rk], tstats[2 * rk + 1]);
  }
  const bool all_valid = __all(valid);
  const unsigned long long rej = __ballot(reject);
  const int n = !all_valid ? -1 : (rej ? __ffsll(static_cast<long long>(rej)) - 1 : K);
  if (t == 0) num_accepted[b] = n;
  for (int pos = t; pos <= K; pos += kWave) {
    out_tokens[b * K1 + pos] = (pos < n) ? tokens[b * K + pos] : -1;
  }
  if (probs != nullptr && t < K) {
    const float nan = __builtin_nanf("");
    probs[2 * (b * K + t)] = all_valid ? static_cast<float>(q) : nan;
    probs[2 * (b * K + t) + 1] = all_valid ? static_cast<float>(p) : nan;
  }
}

// =========================================================== residual_kernel
//
// One workgroup per sequence, on the row(s) at position n = num_accepted[b].
// Weights (all fp64):
//   residual  w(x) = max(0, e_q(x)/S_q - e_p(x)/S_p),  e(x) = exp((z(x)-m)/T)
//   fallback  w(x) = e_q(x) when the residual has no mass
//   bonus     w(x) = e_q(x) on row K
// (the draw is invariant to a common scale, so bonus/fallback weights stay
// unnormalised).  S_q, S_p are recomputed in fp64 here.
//
// Draw: the row is cut into chunks of 64*E tokens (E per lane, contiguous per
// lane, lanes contiguous).  Pass B: every wave computes, per chunk, lane sums
// in token order and their inclusive wave scan; the chunk total goes to LDS.
// Pass C (wave 0): running prefix over chunk totals in chunk order, target =
// u * S_w with S_w the final running value, first chunk whose inclusive prefix
// exceeds the target.  Pass D (wave 0): the chosen chunk's lane sums and scan
// are re-derived with the same code (identical bits under fp-contract=off),
// then the first lane and the first token whose cumulative weight exceeds the
// target.  A token of weight 0 is never chosen; if rounding leaves no
// crossing (u*S_w >= S_w is impossible for u < 1, but u >= 1 or a NaN u is
// tolerated) the last token of positive weight is chosen, as the oracle does.

enum : int { kModeResidual = 0, kModeBonus = 1 };

// Weights of the E tokens of lane `lane` in chunk `c`; tokens >= V get 0.
template <int DT, int E>
__device__ __forceinline__ void lane_weights(const void* qrow, const void* prow, int V, int c,
                                             int lane, int mode, double mq, double mp,
                                             double yscale, double iq, double ip,
                                             const double* tab, double (&w)[E]) {
  const int64_t x0 = static_cast<int64_t>(c) * (kWave * E) + static_cast<int64_t>(lane) * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t x = x0 + e;
    double v = 0.0;
    if (x < V) {
      const double zq = logit_f32<DT>(qrow, x);
      const double eq = exp64_scaled((zq - mq) * yscale, tab);
      if (mode == kModeResidual) {
        const double zp = logit_f32<DT>(prow, x);
        const double ep = exp64_scaled((zp - mp) * yscale, tab);
        const double d = eq * iq - ep * ip;
        v = d > 0.0 ? d : 0.0;
      } else {
        v = eq;
      }
    }
    w[e] = v;
  }
}

template <int BLOCK, int DT>
__global__ __launch_bounds__(BLOCK) void residual_kernel(
    const void* __restrict__ tgt, const void* __restrict__ dft,
    const float* __restrict__ uni, const float* __restrict__ tstats,
    const float* __restrict__ dstats, const int32_t* __restrict__ nacc, int K, int V,
    double invT, int32_t* __restrict__ out_tokens, int32_t* __restrict__ num_emitted) {
  constexpr int EB = Elt<DT>::bytes;
  constexpr int E = 16 / EB;
  constexpr int CH = kWave * E;
  constexpr int NW = BLOCK / kWave;
  extern __shared__ double chunk_tot[];  // [nch]
  __shared__ double tab[64];
  __shared__ double red[NW];
  __shared__ int s_sel[2];
  __shared__ double s_sel_d[2];

  const int64_t b = blockIdx.x;
  const int64_t K1 = K + 1;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int n = nacc[b];
  if (n < 0 || n > K) {
    if (tid == 0 && num_emitted) num_emitted[b] = 0;
    return;
  }
  const bool resid = n < K;
  const int64_t rq = b * K1 + n, rp = b * K + n;
  const float mqf = tstats[2 * rq], sqf = tstats[2 * rq + 1];
  float mpf = 0.f, spf = 1.f;
  if (resid) {
    mpf = dstats[2 * rp];
    spf = dstats[2 * rp + 1];
  }
  if (!row_ok(mqf, sqf) || !row_ok(mpf, spf)) {
    if (tid == 0) {
      out_tokens[b * K1 + n] = -1;
      if (num_emitted) num_emitted[b] = 0;
    }
    return;
  }
  const void* qrow = static_cast<const char*>(tgt) + rq * static_cast<int64_t>(V) * EB;
  const void* prow = static_cast<const char*>(dft) + rp * static_cast<int64_t>(V) * EB;
  const double mq = mqf, mp = mpf;
  const double yscale = invT * Exp64::kScale;
  fill_exp2_table(tab);
  __syncthreads();

  // Pass A: fp64 normalisers of both rows (residual only).
  double iq = 1.0, ip = 1.0;
  int mode = kModeBonus;
  if (resid) {
    double aq = 0.0, ap = 0.0;
    for (int64_t x = tid; x < V; x += BLOCK) {
      aq = aq + exp64_scaled((static_cast<double>(logit_f32<DT>(qrow, x)) - mq) * yscale, tab);
      ap = ap + exp64_scaled((static_cast<double>(logit_f32<DT>(prow, x)) - mp) * yscale, tab);
    }
    const double Sq = block_sum<BLOCK>(aq, red);
    const double Sp = block_sum<BLOCK>(ap, red);
    iq = 1.0 / Sq;
    ip = 1.0 / Sp;
    mode = kModeResidual;
  }
  const int nch = (V + CH - 1) / CH;
  const double u = uni[b * K1 + K];

  for (int attempt = 0; attempt < 2; ++attempt) {
    // Pass B: chunk totals.
    for (int c = wv; c < nch; c += NW) {
      double w[E];
      lane_weights<DT, E>(qrow, prow, V, c, lane, mode, mq, mp, yscale, iq, ip, tab, w);
      double ls = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) ls = ls + w[e];
      const double incl = wave_incl_scan(ls);
      if (lane == kWave - 1) chunk_tot[c] = incl;
    }
    __syncthreads();

    // Pass C (wave 0): running prefix over chunks, pick the crossing chunk.
    if (wv == 0) {
      const int per = (nch + kWave - 1) / kWave;
      const int c0 = lane * per;
      const int c1 = min(nch, c0 + per);
      double lt = 0.0;
      for (int c = c0; c < c1; ++c) lt = lt + chunk_tot[c];
      const double li = wave_incl_scan(lt);
      double run = __shfl_up(li, 1, kWave);
      if (lane == 0) run = 0.0;
      // total = running value after the last chunk (held by the lane owning it)
      const int last_lane = (nch - 1) / per;
      double run_end = run;
      for (int c = c0; c < c1; ++c) run_end = run_end + chunk_tot[c];
      const double S_w = __shfl(run_end, last_lane, kWave);
      if (attempt == 0 && mode == kModeResidual && !(S_w > 0.0)) {
        if (lane == 0) s_sel[0] = -2;  // residual has no mass: fall back to q
      } else {
        const double target = u * S_w;
        int hit = -1, lastpos = -1;
        double hit_excl = 0.0, lastpos_excl = 0.0;
        double r = run;
        for (int c = c0; c < c1; ++c) {
          const double tc = chunk_tot[c];
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
        int sel = -3;  // -3: no token carries positive weight (only with bad stats)
        double sel_excl = 0.0;
        if (hm) {
          const int src = __ffsll(static_cast<long long>(hm)) - 1;
          sel = __shfl(hit, src, kWave);
          sel_excl = __shfl(hit_excl, src, kWave);
        } else if (pm) {
          const int src = 63 - __clzll(static_cast<long long>(pm));
          sel = __shfl(lastpos, src, kWave);
          sel_excl = __shfl(lastpos_excl, src, kWave);
        }
        if (lane == 0) {
          s_sel[0] = sel;
          s_sel[1] = hm ? 1 : 0;
          s_sel_d[0] = sel_excl;
          s_sel_d[1] = target;
        }
      }
    }
    __syncthreads();
    if (s_sel[0] == -2) {
      mode = kModeBonus;  // weights e_q on the same row
      __syncthreads();
      continue;
    }
    break;
  }

  // Nothing to draw from (every weight 0 or NaN; only reachable with stats
  // that do not belong to these rows): report no token.
  if (s_sel[0] < 0) {
    if (tid == 0) {
      out_tokens[b * K1 + n] = -1;
      if (num_emitted) num_emitted[b] = 0;
    }
    return;
  }

  // Pass D (wave 0): re-derive the chosen chunk and find the token.
  if (wv == 0) {
    const int c = s_sel[0];
    const bool crossing = s_sel[1] != 0;
    const double excl = s_sel_d[0];
    const double target = s_sel_d[1];
    double w[E];
    lane_weights<DT, E>(qrow, prow, V, c, lane, mode, mq, mp, yscale, iq, ip, tab, w);
    double ls = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) ls = ls + w[e];
    const double incl = wave_incl_scan(ls);
    double lexcl = __shfl_up(incl, 1, kWave);
    if (lane == 0) lexcl = 0.0;
    const bool lane_hit = crossing && ls > 0.0 && (excl + incl) > target;
    const unsigned long long hm = __ballot(lane_hit);
    const unsigned long long pm = __ballot(ls > 0.0);
    const int src = hm ? (__ffsll(static_cast<long long>(hm)) - 1)
                       : (pm ? 63 - __clzll(static_cast<long long>(pm)) : -1);
    if (src < 0 && lane == 0) {
      out_tokens[b * K1 + n] = -1;
      if (num_emitted) num_emitted[b] = 0;
    }
    if (lane == src) {
      const double base = excl + lexcl;
      int pick = -1, lastpos = -1;
      double a = 0.0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        a = a + w[e];
        if (w[e] > 0.0) {
          if (pick < 0 && hm && (base + a) > target) pick = e;
          lastpos = e;
        }
      }
      if (pick < 0) pick = lastpos;
      const int64_t x = static_cast<int64_t>(c) * CH + static_cast<int64_t>(lane) * E + pick;
      out_tokens[b * K1 + n] = static_cast<int32_t>(x);
      if (num_emitted) num_emitted[b] = n + 1;
    }
  }
}

}  // namespace spec
