/*
 * spec_softmax.h -- C ABI of the MI355X (gfx950) speculative-sampling verify
 * library libspec_softmax.so.
 *
 * The operation is the verify step of speculative sampling (SpS) as stated on
 * the wikillm.com card for arXiv 2302.01318, "Accelerating Large Language
 * Model Decoding with Speculative Sampling" (Chen et al., DeepMind):
 *   - Method, "Algorithm: Speculative Sampling (SpS)" (alg. 2), step 2: the
 *     target model gives K+1 distributions q_0..q_K for one sequence, q_t
 *     conditioned on the first t drafted tokens; the draft model gave p_0..p_{K-1}
 *     and drew token x_t from p_t (step 1).
 *   - Method, "Decoding transforms": temperature T is applied to both p and q
 *     before anything else; here q_t = softmax(z^q_t / T), p_t = softmax(z^p_t / T).
 *   - Method, "Modified rejection sampling" (paper sec. 4.2) and alg. 2 step 3:
 *     left to right, accept x_t when u_t < min(1, q_t(x_t) / p_t(x_t)); stop at
 *     the first rejection.
 *   - Same passage and alg. 2 step 4, with the Pitfalls notes: at the first
 *     rejection, at position n, draw one token from (q_n - p_n)_+ =
 *     max(0, q_n - p_n) / sum max(0, q_n - p_n); if the residual has no mass
 *     fall back to q_n; if all K were accepted draw a bonus token from q_K.
 *   Each sequence therefore emits between 1 and K+1 tokens.
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers owned by the caller, contiguous,
 *     row-major, aligned to their element size.  The library keeps no pointer
 *     after a call returns, allocates no device memory and holds no state.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting.  Results are valid once the stream
 *     reaches that point.
 *   - Logit layouts: target [B][K+1][V] and draft [B][K][V], V contiguous.
 *     dtype SPEC_DTYPE_F32 = IEEE binary32, SPEC_DTYPE_BF16 = bfloat16 (the
 *     upper 16 bits of a binary32).  -inf logits are allowed (probability 0).
 *   - Row statistics ("stats"): float[rows][2] = {m, s} with
 *       m = max_x z[x]   (exactly the largest stored logit),
 *       s = sum_x exp((z[x] - m) / T)   (in [1, V] for a valid row).
 *     Then q(x) = exp((z[x] - m) / T) / s.  A row that holds a NaN or whose
 *     maximum is +-inf (all -inf included) defines no distribution: its s is
 *     NaN.
 *   - Uniforms: float[B][K+1] in [0, 1): slot [b][t] (t < K) drives accept
 *     test t, slot [b][K] the final residual/bonus draw.  They are inputs so
 *     that a run is reproducible; the caller draws them.
 *   - Argument errors are reported synchronously (status code, nothing
 *     enqueued).  Bad device data is reported per sequence: a draft token
 *     outside [0, V) or a row that defines no distribution makes that
 *     sequence's num_accepted -1 and its out_tokens all -1; no out-of-bounds
 *     access happens.
 *   - Limits: 1 <= B, 1 <= K <= SPEC_MAX_K, 1 <= V <= SPEC_MAX_V,
 *     T finite and > 0, B*(2K+1) <= SPEC_MAX_ROWS (the row count of one
 *     launch of 1024-thread workgroups); R <= SPEC_MAX_ROWS for the per-row
 *     calls.  Larger shapes return SPEC_ERR_INVALID_ARG.
 */
#ifndef SPEC_SOFTMAX_H
#define SPEC_SOFTMAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_DTYPE_F32 0
#define SPEC_DTYPE_BF16 1

#define SPEC_OK 0
#define SPEC_ERR_INVALID_ARG 1
#define SPEC_ERR_UNSUPPORTED 2
#define SPEC_ERR_LAUNCH 3

#define SPEC_MAX_K 64
#define SPEC_MAX_V (1 << 20)
#define SPEC_MAX_ROWS 4194303 /* (2^32 - 1) / 1024 */
#define SPEC_NOALLOC_SCRATCH_BYTES (8u << 20) /* spec_verify_step_noalloc's scratch */

/*
 * spec_softmax_stats -- temperature softmax statistics of every row.
 * Defines: "Decoding transforms" (temperature on both p and q) and alg. 2
 * step 2 ("K+1 target distributions"); q and p themselves are never stored.
 *   target_logits  [B][K+1][V]  dtype
 *   draft_logits   [B][K][V]    dtype
 *   target_stats   out float[B][K+1][2] = {m, s} per target row
 *   draft_stats    out float[B][K][2]   = {m, s} per draft row
 * Every logit is read once.  s is accumulated in fp32 from exp2 with a
 * row-wise running maximum and combined across threads in fp64; its relative
 * error is about 1e-7.
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG (null pointer, bad size, dtype or T,
 * misaligned pointer) or SPEC_ERR_LAUNCH.
 */
int spec_softmax_stats(const void* target_logits, const void* draft_logits, int dtype,
                       int B, int K, int V, float temperature,
                       float* target_stats, float* draft_stats, void* stream);

/*
 * spec_verify -- accept scan of every sequence.
 * Defines: "Modified rejection sampling" (sec. 4.2) and alg. 2 step 3:
 * accept x_t iff u_t < min(1, q_t(x_t)/p_t(x_t)); with p_t(x_t) = 0 accept iff
 * q_t(x_t) > 0.  q and p at the drafted token are formed in fp64 from the
 * stored logit and the row stats.
 *   draft_tokens   [B][K] int32 (x_t was drawn from p_t)
 *   uniforms       [B][K+1] float (slots 0..K-1 used here)
 *   target_stats, draft_stats   as written by spec_softmax_stats
 *   num_accepted   out int32[B]: n_b in [0, K], or -1 for an invalid sequence
 *   out_tokens     out int32[B][K+1]: [b][t] = x_t for t < n_b, -1 elsewhere
 *                  (position n_b is filled by spec_residual_sample)
 *   probs          optional out float[B][K][2] = {q_t(x_t), p_t(x_t)} for every t
 *                  (NaN for an invalid sequence); pass NULL to skip
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG or SPEC_ERR_LAUNCH.
 */
int spec_verify(const void* target_logits, const void* draft_logits, int dtype,
                const int32_t* draft_tokens, const float* uniforms,
                const float* target_stats, const float* draft_stats,
                int B, int K, int V, float temperature,
                int32_t* num_accepted, int32_t* out_tokens, float* probs, void* stream);

/*
 * spec_residual_sample -- the one final token of every sequence.
 * Defines: "Modified rejection sampling" (sec. 4.2), alg. 2 step 4 and the
 * Pitfalls notes.  With n = num_accepted[b]:
 *   n < K : weights w = max(0, q_n - p_n); if they have no mass, w = q_n;
 *   n == K: weights w = q_K (bonus token);
 * and the token is the inverse-CDF draw in ascending token id,
 *   x* = min { x : sum_{y<=x} w(y) > u_{b,K} * sum_y w(y) },
 * which never picks a token of weight 0.  The weights, their sums and the
 * prefix scan are formed in fp64; the row normalisers are recomputed in fp64
 * from the logits (the fp32 s in the stats is not precise enough to place
 * the draw).  Only the one or two rows at position n are read.
 *   num_accepted   int32[B] as written by spec_verify (or chosen by the caller);
 *                  a value outside [0, K] leaves out_tokens[b] untouched and
 *                  writes num_emitted[b] = 0
 *   out_tokens     in/out int32[B][K+1]: writes [b][n] only
 *   num_emitted    optional out int32[B] = n + 1 (0 when nothing was drawn)
 * A row at position n that defines no distribution writes out_tokens[b][n] = -1
 * and num_emitted[b] = 0.
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG or SPEC_ERR_LAUNCH.
 */
int spec_residual_sample(const void* target_logits, const void* draft_logits, int dtype,
                         const float* uniforms, const float* target_stats,
                         const float* draft_stats, const int32_t* num_accepted,
                         int B, int K, int V, float temperature,
                         int32_t* out_tokens, int32_t* num_emitted, void* stream);

/*
 * spec_verify_sample -- spec_verify and spec_residual_sample in one launch
 * (alg. 2 steps 2-4, sec. 4.2 and the Pitfalls readings cited above): one
 * workgroup per sequence runs the accept tests and the first-rejection scan,
 * then draws the final token.  Same inputs and outputs, and the same results,
 * as spec_verify followed by spec_residual_sample on the stats of
 * spec_softmax_stats; it saves one launch and the dependency between them.
 *   probs, num_emitted   optional outputs (NULL to skip)
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG or SPEC_ERR_LAUNCH.
 */
int spec_verify_sample(const void* target_logits, const void* draft_logits, int dtype,
                       const int32_t* draft_tokens, const float* uniforms,
                       const float* target_stats, const float* draft_stats, int B, int K, int V,
                       float temperature, int32_t* num_accepted, int32_t* out_tokens,
                       float* probs, int32_t* num_emitted, void* stream);

/*
 * spec_greedy_verify -- greedy mode.  The card's Pitfalls (greedy mode) infer
 * the rule from the general one applied to one-hot distributions: q_t is
 * one-hot at a_t = argmax_x z^q_t[x], so x_t is accepted iff x_t == a_t, and
 * the residual at the first mismatch (or the bonus row) is one-hot at a_n.
 * The draft logits are not needed and T plays no part.
 *   target_logits  [B][K+1][V], dtype as above
 *   draft_tokens   [B][K] int32
 *   target_argmax  out [B][K+1] int32: a_t, the first index of the row's
 *                  maximum (ties go to the smaller index); -1 for a row that
 *                  holds a NaN or whose maximum is not finite
 *   num_accepted   out [B]: n in [0,K], or -1 (such a row, or a draft token
 *                  outside [0,V), in the sequence)
 *   out_tokens     out [B][K+1]: x_0..x_{n-1}, then a_n, then -1 (all -1 for
 *                  an invalid sequence)
 *   num_emitted    optional out [B]: n+1, or 0 for an invalid sequence
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG or SPEC_ERR_LAUNCH.
 */
int spec_greedy_verify(const void* target_logits, int dtype, const int32_t* draft_tokens,
                       int B, int K, int V, int32_t* target_argmax, int32_t* num_accepted,
                       int32_t* out_tokens, int32_t* num_emitted, void* stream);

/*
 * spec_sample -- draft-side sampling ("Algorithm: Speculative Sampling (SpS)",
 * alg. 2 step 1, and "Decoding transforms": draft tokens are drawn from the
 * temperature-transformed p).  For each of R independent rows r:
 *   x_r = min { x : sum_{y<=x} e(y) > u_r * sum_y e(y) },  e(y) = exp((z_r[y] - m_r)/T),
 * the same exact inverse CDF in ascending token id as the bonus draw.
 *   logits      [R][V], dtype as above
 *   uniforms    [R] in [0, 1)
 *   row_stats   out [R][2] {m, s}: the same quantities as spec_softmax_stats
 *               writes (m exact; s within its rounding: bf16 rows whose
 *               draw fits in LDS are read once, and their s comes from the
 *               draw's own fp64 sum, more precise than the fp32 terms of
 *               spec_softmax_stats, so the two can differ in the last bits)
 *   tokens      out [R]: x_r, or -1 for a row that defines no distribution
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG or SPEC_ERR_LAUNCH.
 */
int spec_sample(const void* logits, int dtype, int R, int V, float temperature,
                const float* uniforms, float* row_stats, int32_t* tokens, void* stream);

/*
 * spec_filter -- the decoding transforms top-k and nucleus (the card's Method,
 * "Decoding transforms", and Pitfalls: temperature, top-k and nucleus are
 * applied alike to p and q, before the ratio, the residual and the draft
 * draws).  Run it on the target rows and on the draft rows, then give the
 * filtered rows to the calls above (and to spec_sample on the draft side).
 * For each of R independent rows, with z the stored logits:
 *   top-k (0 < top_k < V): t_k = the top_k-th largest stored value; tokens
 *     with z >= t_k are kept (ties with it all kept).
 *   nucleus (top_p < 1), over the top-k survivors: with e = exp((z - m)/T),
 *     t_p = the largest stored value v with sum_{z >= v} e >= top_p * sum e.
 *   thr = max(t_k, t_p); the kept set is {x : z[x] >= thr}.
 *   logits       [R][V], dtype as above
 *   temperature  T > 0 (used by the nucleus masses only)
 *   top_k        0 or >= V: no top-k; negative: invalid
 *   top_p        >= 1: no nucleus; <= 0 or NaN: invalid
 *   thresholds   out [R] float: thr, -inf when nothing is removed, NaN for a
 *                row that defines no distribution (a NaN, or no finite
 *                maximum; its row is copied unchanged)
 *   row_stats    optional out [R][2] float: {m, s} of the filtered row, as
 *                spec_softmax_stats defines them (the maximum is never
 *                removed, so m is the input row's; s sums the kept tokens;
 *                s is NaN for a row that defines no distribution).  With it
 *                the verify calls take the filtered rows and these stats
 *                directly, without a spec_softmax_stats pass over them.
 *   filtered     optional out [R][V], dtype as logits: z with removed tokens
 *                set to -inf.  May equal logits (in place; then rows with
 *                nothing removed are not written); may not overlap it
 *                otherwise.  NULL: thresholds only.
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG or SPEC_ERR_LAUNCH.
 */
int spec_filter(const void* logits, int dtype, int R, int V, float temperature, int top_k,
                float top_p, float* thresholds, float* row_stats, void* filtered, void* stream);

/*
 * spec_verify_step_workspace_size -- bytes of device workspace spec_verify_step
 * needs for this shape (0 for an invalid shape).  Independent of T and of the
 * device.
 */
size_t spec_verify_step_workspace_size(int B, int K, int V, int dtype);

/*
 * spec_verify_step -- the whole verify step (what spec_softmax_stats followed
 * by spec_verify_sample computes: alg. 2 steps 2-4, sec. 4.2, "Decoding
 * transforms" and the Pitfalls readings cited above) in two launches.  With
 * 64 sequences or fewer, too few to occupy the device one workgroup per
 * sequence, each sequence's final draw is split over several workgroups
 * that sweep parts of its row(s) and hand their sums to the one that
 * finishes last; from 65 sequences on it is spec_softmax_stats followed by
 * spec_verify_sample.  The outputs are the same bits as those two calls give
 * (the split draw forms the same sums in the same order).
 *   inputs         as for the calls above (target, draft, tokens, uniforms)
 *   target_stats, draft_stats, num_accepted, out_tokens   outputs as above
 *   probs, num_emitted   optional outputs as above (NULL to skip)
 *   workspace      device memory of at least spec_verify_step_workspace_size
 *                  bytes, 256-byte aligned, owned by the caller.  It must be
 *                  all zero before its first use; every completed call leaves
 *                  its counters zero again, so it can be reused by any later
 *                  call whose workspace size is not larger.  Two calls in
 *                  flight at the same time need two workspaces.
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG (also for a workspace that is too
 * small or misaligned) or SPEC_ERR_LAUNCH.
 */
int spec_verify_step(const void* target_logits, const void* draft_logits, int dtype,
                     const int32_t* draft_tokens, const float* uniforms,
                     int B, int K, int V, float temperature,
                     float* target_stats, float* draft_stats,
                     int32_t* num_accepted, int32_t* out_tokens, float* probs,
                     int32_t* num_emitted, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * spec_verify_step_noalloc -- spec_verify_step for callers that cannot
 * allocate or pass device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments minus the
 * workspace, same launches and the same bits; the workspace is instead a
 * file-scope device array of SPEC_NOALLOC_SCRATCH_BYTES (8 MiB) inside the
 * library, of which each GPU the library runs on holds its own copy until the
 * process ends.  No hipMalloc, hipFree or allocating routine is called.
 *   - The first call on a device looks the array up and clears it with one
 *     fill kernel on `stream`, ahead of its own launches.
 *   - Every call on a GPU shares that GPU's array (each completed call leaves
 *     its counters zero for the next): calls that overlap on one GPU, on
 *     different streams or from different threads, race and must not be
 *     issued.
 *   - A shape whose spec_verify_step_workspace_size exceeds the array returns
 *     SPEC_ERR_UNSUPPORTED with nothing enqueued (only batches of 64
 *     sequences or fewer use it: 64 sequences of up to about 800K bf16 or
 *     400K fp32 tokens fit, 32 of any bf16 vocabulary up to SPEC_MAX_V).
 * Returns SPEC_OK, SPEC_ERR_INVALID_ARG, SPEC_ERR_UNSUPPORTED or
 * SPEC_ERR_LAUNCH (also if the array cannot be looked up).
 */
int spec_verify_step_noalloc(const void* target_logits, const void* draft_logits, int dtype,
                             const int32_t* draft_tokens, const float* uniforms,
                             int B, int K, int V, float temperature,
                             float* target_stats, float* draft_stats,
                             int32_t* num_accepted, int32_t* out_tokens, float* probs,
                             int32_t* num_emitted, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* spec_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_SOFTMAX_H */
