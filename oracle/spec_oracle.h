/*
 * spec_oracle.h -- plain fp64 CPU oracle for the speculative-sampling verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the GPU library and neither includes the other.
 *
 * Source of what is computed: the wikillm.com card for arXiv 2302.01318,
 * "Accelerating Large Language Model Decoding with Speculative Sampling"
 * (Chen et al., DeepMind):
 *   [MRS]   Method, "Modified rejection sampling" (paper sec. 4.2): accept the
 *           drafted token with probability min(1, q/p); on rejection draw from
 *           (q-p)_+ = max(0, q-p) / sum max(0, q-p) and stop.
 *   [ALG2]  Method, "Algorithm: Speculative Sampling (SpS)" (alg. 2), steps 2-4:
 *           K+1 target distributions, the left-to-right accept scan with r ~ U[0,1],
 *           and a bonus token from the last target distribution when all K pass.
 *   [TRANS] Method, "Decoding transforms": temperature applied to both p and q.
 *   [PIT]   Pitfalls: bonus row is the (K+1)-th target output; the ratio is taken
 *           at the drafted token; a separate accepted count; residual denominator
 *           0 falls back to q.
 *   [THM1]  Method: Theorem 1, P(X=x) = min(p(x),q(x)) + max(0, q(x)-p(x)) = q(x).
 *   [GREEDY] Pitfalls: greedy mode.  The card derives the rule by applying the
 *           general test to one-hot distributions: a drafted token survives
 *           only when it is the target row's largest entry, and the first
 *           one that is not is replaced by that entry.
 *   [DRAFT] "Algorithm: Speculative Sampling (SpS)" (alg. 2) step 1 and
 *           Pitfalls: draft tokens are sampled from the (transformed) draft
 *           distributions p.
 *
 * Every floating-point step is IEEE binary64, evaluated in the order written.
 * Logits are read exactly: fp32 widens to fp64, bf16 is the upper half of a
 * binary32 word.
 *
 * Error convention: functions return 0 on success and a negative value when
 * the input does not define the quantity (documented per function).  Nothing
 * here allocates memory that outlives a call.
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_DTYPE_F32 0
#define ORACLE_DTYPE_BF16 1

/* Distribution of one logit row under temperature T [TRANS]:
 *   a_x = z_x / T,  M = max_x a_x,  e_x = exp(a_x - M),  S = sum_x e_x,
 *   prob_x = e_x / S.
 * The shift by M only keeps exp in range; the result is softmax(z/T).
 * prob (length V) may be NULL.  Writes M and S.
 * Returns -1 (outputs untouched) when the row holds a NaN or M is not finite
 * (all -inf, or a +inf logit): such a row defines no distribution. */
int oracle_softmax_row(const void* row, int dtype, int V, double T,
                       double* prob, double* a_max, double* norm);

/* One accept test [MRS], [ALG2] step 3: accept iff u < min(1, q/p), strict.
 * p == 0: the ratio is +inf when q > 0 (accept) and undefined when q == 0;
 * the latter is read as reject (the token has no mass under either law).
 * dist (nullable) gets |u - q/p| for a finite ratio, +inf otherwise: how far
 * the uniform lies from the value that would flip the decision.
 * Returns 1 = accept, 0 = reject. */
int oracle_accept(double q, double p, double u, double* dist);

/* Residual weights [MRS], [PIT]: w_x = max(0, q_x - p_x).  If their sum is
 * not > 0 (q == p numerically) the weights become q.  The normalisation by the
 * sum is left to oracle_inverse_cdf.  Returns 1 when the q fallback was taken,
 * 0 otherwise. */
int oracle_residual_weights(const double* q, const double* p, int V, double* w);

/* Categorical draw by inverse CDF in ascending token id:
 *   S = sum_x w_x (sequential),  C(x) = sum_{y<=x} w_y (the same sequence of
 *   additions),  x* = min { x : C(x) > u*S }.
 * Zero-weight tokens can never be chosen.  dist (nullable) gets
 * min(u*S - C(x*-1), C(x*) - u*S) / S.
 * Returns x*, or -1 when S is not > 0 or not finite. */
int oracle_inverse_cdf(const double* w, int V, double u, double* dist);

/* Verify of sequences whose distributions are already known [ALG2] steps 3-4.
 *   q        [K+1][V] target distributions (row t conditioned on t draft tokens)
 *   p        [K][V]   draft distributions (row t produced draft token t)
 *   N        number of independent runs over the same distributions
 *   tokens   [N][K]   draft tokens; uniforms [N][K+1] (slot K is the final draw)
 * Outputs per run n (all nullable except num_accepted and out_tokens):
 *   num_accepted[n] in [0,K] (-1 if a token lies outside [0,V)),
 *   out_tokens[n][K+1]: accepted prefix, then the residual/bonus token, then -1,
 *   accept_dist[n][K] (+inf where no test ran), draw_dist[n],
 *   draw_kind[n]: 0 residual, 1 bonus, 2 residual fell back to q, -1 invalid.
 * Returns 0, or -1 on a bad argument. */
int oracle_verify_dists(const double* q, const double* p, int K, int V, int64_t N,
                        const int32_t* tokens, const float* uniforms,
                        int32_t* num_accepted, int32_t* out_tokens,
                        double* accept_dist, double* draw_dist, int32_t* draw_kind);

/* Full batched verify from logits [ALG2] steps 2-4, [TRANS].
 *   target [B][K+1][V], draft [B][K][V] (dtype as above, contiguous), T > 0,
 *   tokens [B][K] int32, uniforms [B][K+1] fp32 in [0,1).
 * A sequence is invalid (num_accepted = -1, out_tokens all -1, num_emitted 0,
 * draw_kind -1) when any of its 2K+1 rows defines no distribution or a draft
 * token lies outside [0,V).
 * Outputs (nullable unless stated):
 *   target_stats [B][K+1][2], draft_stats [B][K][2]: {M, S} of each row as in
 *     oracle_softmax_row (NaN, NaN for a row that defines no distribution),
 *   num_accepted [B] (required), out_tokens [B][K+1] (required), num_emitted [B],
 *   probs [B][K][2] = {q_t(x_t), p_t(x_t)}, accept_dist [B][K], draw_dist [B],
 *   draw_kind [B].
 * nthreads <= 0 uses the OpenMP default.  Sequences are independent; the
 * result does not depend on nthreads.  Returns 0, or -1 on a bad argument,
 * -2 if working memory could not be obtained. */
int oracle_verify(const void* target, const void* draft, int dtype,
                  int B, int K, int V, double T,
                  const int32_t* tokens, const float* uniforms,
                  double* target_stats, double* draft_stats,
                  int32_t* num_accepted, int32_t* out_tokens, int32_t* num_emitted,
                  double* probs, double* accept_dist, double* draw_dist,
                  int32_t* draw_kind, int nthreads);

/* Final draw alone, with the accepted count supplied by the caller:
 * n = num_accepted[b] in [0,K]: residual on rows (q_n, p_n) when n < K, bonus
 * from q_K when n == K; u = uniforms[b][K].  n < 0 or n > K, or a row that
 * defines no distribution, gives token -1 and kind -1.
 * Outputs: token [B], draw_dist [B] (nullable), draw_kind [B] (nullable). */
int oracle_final_draw(const void* target, const void* draft, int dtype,
                      int B, int K, int V, double T,
                      const float* uniforms, const int32_t* num_accepted,
                      int32_t* token, double* draw_dist, int32_t* draw_kind,
                      int nthreads);

/* Argmax of one logit row [GREEDY]: the first index holding the maximum
 * stored value (ties go to the smaller index, as numpy's argmax).
 * Returns 0 and writes *idx, or -1 when the row holds a NaN or its maximum is
 * not finite (the row defines no distribution). */
int oracle_argmax_row(const void* row, int dtype, int V, int32_t* idx);

/* Greedy verify [GREEDY]: for each sequence b,
 *   a_t = argmax of target row t (t = 0..K),
 *   n = the first t < K with tokens[b][t] != a_t, else K,
 *   out_tokens[b] = tokens[b][0..n-1], then a_n, then -1; num_emitted = n+1.
 * This is the general accept rule on one-hot p and q: q/p is 1 at the target
 * argmax and 0 elsewhere, and the residual (q-p)_+ is one-hot at a_n.
 * A sequence with a row that defines no distribution, or a draft token
 * outside [0,V), is invalid: num_accepted -1, out_tokens all -1,
 * num_emitted 0.  argmax [B][K+1] (nullable) receives a_t (-1 for an invalid
 * row); num_emitted is nullable.  Returns 0, or -1 on a bad argument. */
int oracle_greedy_verify(const void* target, int dtype, int B, int K, int V,
                         const int32_t* tokens, int32_t* argmax,
                         int32_t* num_accepted, int32_t* out_tokens,
                         int32_t* num_emitted, int nthreads);

/* Draft-side sampling [DRAFT], [TRANS]: for each of R independent rows r,
 * the token drawn from softmax(z_r / T) by oracle_inverse_cdf with uniform
 * u_r in [0,1): x = min { x : sum_{y<=x} prob_y > u_r * sum_y prob_y }.
 * tokens [R] gets x, or -1 for a row that defines no distribution; dist [R]
 * (nullable) the draw's boundary distance.  Returns 0, or -1 on a bad
 * argument. */
int oracle_sample_rows(const void* logits, int dtype, int64_t R, int V, double T,
                       const float* uniforms, int32_t* tokens, double* dist, int nthreads);

/* Decoding transforms [TRANS], [PIT]: temperature, then top-k, then nucleus
 * (top-p), applied alike to every target and draft row before anything else.
 * The result is a logit threshold thr: tokens with z < thr get probability 0,
 * the others keep their relative weights exp(z/T - M).
 *   top-k (0 < top_k < V): thr_k = the top_k-th largest stored logit; every
 *     token at or above it is kept (ties at thr_k included).
 *   nucleus (top_p < 1), over the tokens top-k kept: with e_x = exp(z_x/T - M)
 *     and the kept values taken in descending order, S = their sum and
 *     C(v) = the sum over tokens with z >= v (the same additions, a prefix of
 *     S), thr_p = the largest stored value v with C(v) >= top_p * S.
 * thr = -inf when nothing is removed.  Returns 0, or -1 when the row defines
 * no distribution (then thr is left alone) or the parameters are invalid
 * (top_p <= 0 or NaN). */
int oracle_filter_threshold(const void* row, int dtype, int V, double T, int top_k,
                            double top_p, double* thr);

/* oracle_verify on the transformed rows: every target and draft row is
 * thresholded by oracle_filter_threshold (tokens below become -inf in a copy
 * of the logits) and the copies are verified.  target_thr [B][K+1] and
 * draft_thr [B][K] (nullable) receive the thresholds (NaN for a row that
 * defines no distribution).  Other arguments and outputs as oracle_verify.
 * Returns 0, -1 on a bad argument, -2 if memory could not be obtained. */
int oracle_verify_filtered(const void* target, const void* draft, int dtype,
                           int B, int K, int V, double T, int top_k, double top_p,
                           const int32_t* tokens, const float* uniforms,
                           double* target_thr, double* draft_thr,
                           double* target_stats, double* draft_stats,
                           int32_t* num_accepted, int32_t* out_tokens, int32_t* num_emitted,
                           double* probs, double* accept_dist, double* draw_dist,
                           int32_t* draw_kind, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
