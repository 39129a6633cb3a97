/*
 * spec_oracle.c -- plain fp64 CPU oracle for the speculative-sampling verify
 * step.  TEST INFRASTRUCTURE ONLY (tests/, __graft_entry__.smoke(), the
 * cpu_baseline leg of bench.py).  Deliberately slow and literal: every row is
 * turned into a full probability vector, then the algorithm runs on those
 * vectors exactly as the method states it.  Citations are listed in
 * spec_oracle.h ([MRS], [ALG2], [TRANS], [PIT], [THM1]).
 */
#include "spec_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of one stored logit to binary64. */
static double logit_at(const void* base, int dtype, int64_t i)
{
    if (dtype == ORACLE_DTYPE_F32)
        return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_softmax_row(const void* row, int dtype, int V, double T,
                       double* prob, double* a_max, double* norm)
{
    if (!row || V < 1 || !(T > 0.0))
        return -1;
    /* a_x = z_x / T and its maximum [TRANS]. */
    double M = -INFINITY;
    int saw_nan = 0;
    for (int x = 0; x < V; ++x) {
        double a = logit_at(row, dtype, x) / T;
        if (isnan(a))
            saw_nan = 1;
        else if (a > M)
            M = a;
    }
    if (saw_nan || !isfinite(M))
        return -1;
    /* e_x = exp(a_x - M), S = sum e_x, prob_x = e_x / S. */
    double S = 0.0;
    for (int x = 0; x < V; ++x) {
        double e = exp(logit_at(row, dtype, x) / T - M);
        if (prob)
            prob[x] = e;
        S += e;
    }
    if (prob)
        for (int x = 0; x < V; ++x)
            prob[x] = prob[x] / S;
    if (a_max)
        *a_max = M;
    if (norm)
        *norm = S;
    return 0;
}

int oracle_accept(double q, double p, double u, double* dist)
{
    /* ratio q/p at the drafted token [MRS], [PIT]. */
    double rho;
    if (p > 0.0)
        rho = q / p;
    else
        rho = (q > 0.0) ? INFINITY : 0.0;
    double threshold = rho < 1.0 ? rho : 1.0;
    if (dist)
        *dist = isfinite(rho) ? fabs(u - rho) : INFINITY;
    return u < threshold ? 1 : 0;
}

int oracle_residual_weights(const double* q, const double* p, int V, double* w)
{
    double S = 0.0;
    for (int x = 0; x < V; ++x) {
        double d = q[x] - p[x];
        w[x] = d > 0.0 ? d : 0.0;
        S += w[x];
    }
    if (S > 0.0 && isfinite(S))
        return 0;
    /* q == p numerically: rejection had probability 0 but happened; fall back
     * to q as the pitfalls note suggests [PIT]. */
    for (int x = 0; x < V; ++x)
        w[x] = q[x];
    return 1;
}

int oracle_inverse_cdf(const double* w, int V, double u, double* dist)
{
    double S = 0.0;
    for (int x = 0; x < V; ++x)
        S += w[x];
    if (!(S > 0.0) || !isfinite(S))
        return -1;
    double target = u * S;
    double C = 0.0;
    int last_positive = -1;
    for (int x = 0; x < V; ++x) {
        double next = C + w[x];
        if (w[x] > 0.0)
            last_positive = x;
        if (next > target) {
            if (dist) {
                double lo = target - C, hi = next - target;
                *dist = (lo < hi ? lo : hi) / S;
            }
            return x;
        }
        C = next;
    }
    /* Unreachable for u < 1 (C after the last token equals S and u*S < S);
     * kept so that a rounding surprise still yields a token of positive mass. */
    if (dist)
        *dist = 0.0;
    return last_positive;
}

/* One run of steps 3-4 of alg. 2 on known distributions.  w is V doubles of
 * scratch.  Returns the accepted count, -1 for an out-of-range token. */
static int verify_one(const double* q, const double* p, int K, int V,
                      const int32_t* tok, const float* uni, double* w,
                      int32_t* out, double* adist, double* ddist, int32_t* kind)
{
    for (int t = 0; t <= K; ++t)
        out[t] = -1;
    if (adist)
        for (int t = 0; t < K; ++t)
            adist[t] = INFINITY;
    for (int t = 0; t < K; ++t)
        if (tok[t] < 0 || tok[t] >= V) {
            if (ddist)
                *ddist = INFINITY;
            if (kind)
                *kind = -1;
            return -1;
        }

    /* Step 3: left to right, stop at the first rejection; n counts accepted
     * tokens separately from any position index [PIT]. */
    int n = 0;
    for (int t = 0; t < K; ++t) {
        const double* qt = q + (int64_t)t * V;
        const double* pt = p + (int64_t)t * V;
        double u = (double)uni[t];
        int acc = oracle_accept(qt[tok[t]], pt[tok[t]], u, adist ? &adist[t] : NULL);
        if (!acc)
            break;
        out[n] = tok[t];
        n += 1;
    }

    /* Residual draw at the rejected position, or the bonus token from the
     * (K+1)-th target distribution [MRS], [ALG2] step 4, [PIT]. */
    const double* qn = q + (int64_t)n * V;
    int k;
    if (n < K) {
        k = oracle_residual_weights(qn, p + (int64_t)n * V, V, w) ? 2 : 0;
    } else {
        memcpy(w, qn, sizeof(double) * (size_t)V);
        k = 1;
    }
    out[n] = oracle_inverse_cdf(w, V, (double)uni[K], ddist);
    if (kind)
        *kind = k;
    return n;
}

int oracle_verify_dists(const double* q, const double* p, int K, int V, int64_t N,
                        const int32_t* tokens, const float* uniforms,
                        int32_t* num_accepted, int32_t* out_tokens,
                        double* accept_dist, double* draw_dist, int32_t* draw_kind)
{
    if (!q || !p || K < 1 || V < 1 || N < 0 || !tokens || !uniforms || !num_accepted || !out_tokens)
        return -1;
    double* w = (double*)malloc(sizeof(double) * (size_t)V);
    if (!w)
        return -2;
    for (int64_t i = 0; i < N; ++i) {
        num_accepted[i] = verify_one(q, p, K, V, tokens + i * K, uniforms + i * (K + 1), w,
                                     out_tokens + i * (K + 1),
                                     accept_dist ? accept_dist + i * K : NULL,
                                     draw_dist ? draw_dist + i : NULL,
                                     draw_kind ? draw_kind + i : NULL);
    }
    free(w);
    return 0;
}

/* Distributions of all rows of one sequence [ALG2] step 2.  Returns 0 when
 * every row defines a distribution. */
static int sequence_dists(const void* target, const void* draft, int dtype, int b, int K, int V,
                          double T, double* q, double* p, double* tstats, double* dstats)
{
    int bad = 0;
    for (int t = 0; t <= K; ++t) {
        int64_t r = (int64_t)b * (K + 1) + t;
        const char* row = (const char*)target + r * V * (dtype == ORACLE_DTYPE_F32 ? 4 : 2);
        double M = NAN, S = NAN;
        if (oracle_softmax_row(row, dtype, V, T, q + (int64_t)t * V, &M, &S) != 0)
            bad = 1;
        if (tstats) {
            tstats[2 * r] = M;
            tstats[2 * r + 1] = S;
        }
    }
    for (int t = 0; t < K; ++t) {
        int64_t r = (int64_t)b * K + t;
        const char* row = (const char*)draft + r * V * (dtype == ORACLE_DTYPE_F32 ? 4 : 2);
        double M = NAN, S = NAN;
        if (oracle_softmax_row(row, dtype, V, T, p + (int64_t)t * V, &M, &S) != 0)
            bad = 1;
        if (dstats) {
            dstats[2 * r] = M;
            dstats[2 * r + 1] = S;
        }
    }
    return bad ? -1 : 0;
}

int oracle_verify(const void* target, const void* draft, int dtype,
                  int B, int K, int V, double T,
                  const int32_t* tokens, const float* uniforms,
                  double* target_stats, double* draft_stats,
                  int32_t* num_accepted, int32_t* out_tokens, int32_t* num_emitted,
                  double* probs, double* accept_dist, double* draw_dist,
                  int32_t* draw_kind, int nthreads)
{
    if (!target || !draft || !tokens || !uniforms || !num_accepted || !out_tokens)
        return -1;
    if (B < 1 || K < 1 || V < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    int nt = 1;
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        size_t per_seq = (size_t)(2 * K + 2) * (size_t)V;
        double* buf = (double*)malloc(sizeof(double) * per_seq);
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b) {
            if (!buf)
                continue;
            double* q = buf;                       /* [K+1][V] */
            double* p = q + (size_t)(K + 1) * V;   /* [K][V]   */
            double* w = p + (size_t)K * V;         /* [V]      */
            int32_t* out = out_tokens + (int64_t)b * (K + 1);
            const int32_t* tok = tokens + (int64_t)b * K;
            int ok = sequence_dists(target, draft, dtype, b, K, V, T, q, p,
                                    target_stats, draft_stats) == 0;
            for (int t = 0; t < K && ok; ++t)
                if (tok[t] < 0 || tok[t] >= V)
                    ok = 0;
            if (probs)
                for (int t = 0; t < K; ++t) {
                    double* pr = probs + ((int64_t)b * K + t) * 2;
                    int in_range = tok[t] >= 0 && tok[t] < V;
                    pr[0] = ok && in_range ? q[(int64_t)t * V + tok[t]] : NAN;
                    pr[1] = ok && in_range ? p[(int64_t)t * V + tok[t]] : NAN;
                }
            if (!ok) {
                num_accepted[b] = -1;
                for (int t = 0; t <= K; ++t)
                    out[t] = -1;
                if (num_emitted)
                    num_emitted[b] = 0;
                if (accept_dist)
                    for (int t = 0; t < K; ++t)
                        accept_dist[(int64_t)b * K + t] = INFINITY;
                if (draw_dist)
                    draw_dist[b] = INFINITY;
                if (draw_kind)
                    draw_kind[b] = -1;
                continue;
            }
            int n = verify_one(q, p, K, V, tok, uniforms + (int64_t)b * (K + 1), w, out,
                               accept_dist ? accept_dist + (int64_t)b * K : NULL,
                               draw_dist ? draw_dist + b : NULL,
                               draw_kind ? draw_kind + b : NULL);
            num_accepted[b] = n;
            if (num_emitted)
                num_emitted[b] = n + 1;
        }
        free(buf);
    }
    return failed ? -2 : 0;
}

int oracle_final_draw(const void* target, const void* draft, int dtype,
                      int B, int K, int V, double T,
                      const float* uniforms, const int32_t* num_accepted,
                      int32_t* token, double* draw_dist, int32_t* draw_kind,
                      int nthreads)
{
    if (!target || !draft || !uniforms || !num_accepted || !token)
        return -1;
    if (B < 1 || K < 1 || V < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    int nt = 1;
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double* buf = (double*)malloc(sizeof(double) * (size_t)V * 3);
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int b = 0; b < B; ++b) {
            if (!buf)
                continue;
            double* q = buf;
            double* p = buf + V;
            double* w = buf + 2 * (size_t)V;
            int n = num_accepted[b];
            token[b] = -1;
            if (draw_dist)
                draw_dist[b] = INFINITY;
            if (draw_kind)
                draw_kind[b] = -1;
            if (n < 0 || n > K)
                continue;
            size_t esz = dtype == ORACLE_DTYPE_F32 ? 4 : 2;
            const char* qrow = (const char*)target + ((int64_t)b * (K + 1) + n) * V * esz;
            if (oracle_softmax_row(qrow, dtype, V, T, q, NULL, NULL) != 0)
                continue;
            int kind;
            if (n < K) {
                const char* prow = (const char*)draft + ((int64_t)b * K + n) * V * esz;
                if (oracle_softmax_row(prow, dtype, V, T, p, NULL, NULL) != 0)
                    continue;
                kind = oracle_residual_weights(q, p, V, w) ? 2 : 0;
            } else {
                memcpy(w, q, sizeof(double) * (size_t)V);
                kind = 1;
            }
            double u = (double)uniforms[(int64_t)b * (K + 1) + K];
            token[b] = oracle_inverse_cdf(w, V, u, draw_dist ? draw_dist + b : NULL);
            if (draw_kind)
                draw_kind[b] = kind;
        }
        free(buf);
    }
    return failed ? -2 : 0;
}

/* ---------------------------------------------------------------- greedy */

int oracle_argmax_row(const void* row, int dtype, int V, int32_t* idx)
{
    double best = 0.0;
    int32_t at = -1;
    for (int x = 0; x < V; ++x) {
        const double z = logit_at(row, dtype, x);
        if (isnan(z))
            return -1;
        if (at < 0 || z > best) {
            best = z;
            at = x;
        }
    }
    if (at < 0 || !isfinite(best))
        return -1;
    *idx = at;
    return 0;
}

int oracle_greedy_verify(const void* target, int dtype, int B, int K, int V,
                         const int32_t* tokens, int32_t* argmax,
                         int32_t* num_accepted, int32_t* out_tokens,
                         int32_t* num_emitted, int nthreads)
{
    if (!target || !tokens || !num_accepted || !out_tokens || B < 0 || K < 1 || V < 1)
        return -1;
    if ((dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16) || K > 64)
        return -1;
    const int eb = dtype == ORACLE_DTYPE_F32 ? 4 : 2;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    int nt = 1;
    (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int b = 0; b < B; ++b) {
        int valid = 1;
        int32_t a[65];
        for (int t = 0; t <= K; ++t) {
            const char* row = (const char*)target + ((int64_t)b * (K + 1) + t) * (int64_t)V * eb;
            if (oracle_argmax_row(row, dtype, V, &a[t]) != 0) {
                a[t] = -1;
                valid = 0;
            }
            if (argmax)
                argmax[(int64_t)b * (K + 1) + t] = a[t];
        }
        for (int t = 0; t < K; ++t) {
            const int32_t x = tokens[(int64_t)b * K + t];
            if (x < 0 || x >= V)
                valid = 0;
        }
        int32_t* out = out_tokens + (int64_t)b * (K + 1);
        for (int t = 0; t <= K; ++t)
            out[t] = -1;
        if (!valid) {
            num_accepted[b] = -1;
            if (num_emitted)
                num_emitted[b] = 0;
            continue;
        }
        int n = 0;
        while (n < K && tokens[(int64_t)b * K + n] == a[n]) {
            out[n] = tokens[(int64_t)b * K + n];
            ++n;
        }
        out[n] = a[n];
        num_accepted[b] = n;
        if (num_emitted)
            num_emitted[b] = n + 1;
    }
    return 0;
}

/* ------------------------------------------------------- draft sampling */

int oracle_sample_rows(const void* logits, int dtype, int64_t R, int V, double T,
                       const float* uniforms, int32_t* tokens, double* dist, int nthreads)
{
    if (!logits || !uniforms || !tokens || R < 0 || V < 1 || !(T > 0.0) || !isfinite(T))
        return -1;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
    const int eb = dtype == ORACLE_DTYPE_F32 ? 4 : 2;
#ifdef _OPENMP
    int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    int nt = 1;
    (void)nthreads;
#endif
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double* prob = (double*)malloc(sizeof(double) * (size_t)V);
        if (!prob) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < R; ++r) {
            if (!prob)
                continue;
            const char* row = (const char*)logits + r * (int64_t)V * eb;
            double M, S, d = 0.0;
            int32_t x = -1;
            if (oracle_softmax_row(row, dtype, V, T, prob, &M, &S) == 0)
                x = oracle_inverse_cdf(prob, V, (double)uniforms[r], &d);
            tokens[r] = x;
            if (dist)
                dist[r] = x >= 0 ? d : INFINITY;
        }
        free(prob);
    }
    return failed ? -2 : 0;
}

/* -------------------------------------------------- decoding transforms */

static int cmp_desc(const void* a, const void* b)
{
    const double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

int oracle_filter_threshold(const void* row, int dtype, int V, double T, int top_k,
                            double top_p, double* thr)
{
    if (!row || !thr || V < 1 || !(T > 0.0) || !isfinite(T) || !(top_p > 0.0))
        return -1;
    double* v = (double*)malloc(sizeof(double) * (size_t)V);
    if (!v)
        return -1;
    double mx = -INFINITY;
    for (int x = 0; x < V; ++x) {
        v[x] = logit_at(row, dtype, x);
        if (isnan(v[x])) {
            free(v);
            return -1;
        }
        if (v[x] > mx)
            mx = v[x];
    }
    if (!isfinite(mx)) {
        free(v);
        return -1;
    }
    qsort(v, (size_t)V, sizeof(double), cmp_desc);
    double t = -INFINITY;
    int n = V;  /* kept values are v[0..n) */
    if (top_k > 0 && top_k < V) {
        t = v[top_k - 1];
        while (n > 0 && v[n - 1] < t)
            --n;
    }
    if (top_p < 1.0) {
        const double M = v[0] / T;
        double S = 0.0;
        for (int i = 0; i < n; ++i)
            S += exp(v[i] / T - M);
        double c = 0.0;
        int i = 0;
        while (i < n) {
            const double val = v[i];
            while (i < n && v[i] == val)
                c += exp(v[i++] / T - M);
            if (c >= top_p * S) {
                if (val > t)
                    t = val;
                break;
            }
        }
    }
    /* a threshold at or below the smallest logit removes nothing */
    if (t <= v[V - 1])
        t = -INFINITY;
    *thr = t;
    free(v);
    return 0;
}

int oracle_verify_filtered(const void* target, const void* draft, int dtype,
                           int B, int K, int V, double T, int top_k, double top_p,
                           const int32_t* tokens, const float* uniforms,
                           double* target_thr, double* draft_thr,
                           double* target_stats, double* draft_stats,
                           int32_t* num_accepted, int32_t* out_tokens, int32_t* num_emitted,
                           double* probs, double* accept_dist, double* draw_dist,
                           int32_t* draw_kind, int nthreads)
{
    if (!target || !draft || B < 1 || K < 1 || V < 1 || !(top_p > 0.0))
        return -1;
    if (dtype != ORACLE_DTYPE_F32 && dtype != ORACLE_DTYPE_BF16)
        return -1;
    const size_t eb = dtype == ORACLE_DTYPE_F32 ? 4 : 2;
    const int64_t nt = (int64_t)B * (K + 1), nd = (int64_t)B * K;
    char* tc = (char*)malloc((size_t)nt * (size_t)V * eb);
    char* dc = (char*)malloc((size_t)nd * (size_t)V * eb);
    if (!tc || !dc) {
        free(tc);
        free(dc);
        return -2;
    }
    memcpy(tc, target, (size_t)nt * (size_t)V * eb);
    memcpy(dc, draft, (size_t)nd * (size_t)V * eb);
    for (int64_t r = 0; r < nt + nd; ++r) {
        char* row = r < nt ? tc + r * (int64_t)V * (int64_t)eb : dc + (r - nt) * (int64_t)V * (int64_t)eb;
        double t;
        if (oracle_filter_threshold(row, dtype, V, T, top_k, top_p, &t) != 0)
            t = NAN;
        if (r < nt) {
            if (target_thr)
                target_thr[r] = t;
        } else if (draft_thr) {
            draft_thr[r - nt] = t;
        }
        if (!(t > -INFINITY))
            continue;  /* nothing removed, or an invalid row (left as it is) */
        for (int x = 0; x < V; ++x) {
            if (logit_at(row, dtype, x) < t) {
                if (dtype == ORACLE_DTYPE_F32) {
                    ((float*)row)[x] = -INFINITY;
                } else {
                    ((uint16_t*)row)[x] = 0xFF80u;  /* bf16 -inf */
                }
            }
        }
    }
    const int rc = oracle_verify(tc, dc, dtype, B, K, V, T, tokens, uniforms, target_stats,
                                 draft_stats, num_accepted, out_tokens, num_emitted, probs,
                                 accept_dist, draw_dist, draw_kind, nthreads);
    free(tc);
    free(dc);
    return rc;
}
