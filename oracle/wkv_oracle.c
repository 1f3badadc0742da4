/*
 * CPU fp64 oracle for the RWKV-4 WKV operator.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only
 * tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may
 * load it.  It shares no code, header, table or helper with the HIP library
 * and includes nothing from it.
 *
 * Every routine is plain, slow and written to be checked by eye against the
 * pages it cites:
 *   [aiwiki]     aiwiki.thehackersbrain.dev/entries/rwkv  ("RWKV")
 *   [tm-math]    aicassindra.com blogs/transformer_math/tm_rwkv_math.html
 *   [vanos]      vanos001.github.io placement_prep/llm/architectures/rwkv.html
 *   [multigrid]  multigrid.ai/learn/rwkv
 *
 * Conventions (the readings are listed with their reasons in the design notes):
 *   - decay rate w > 0 per channel; the per-step factor is e^{-w}
 *     ([tm-math] "The WKV operator: attention with a fixed decay").
 *   - k, v, y are [B,T,C] row-major: element (b,t,c) at (b*T+t)*C+c.
 *   - a state is three [B,C] arrays (a, b, p); the true accumulators are
 *     e^p*a and e^p*b ([tm-math] "Numerical stability: carry the exponent").
 *     A NULL state means the empty history a=b=0, p=-inf.
 *   - all arithmetic is IEEE double; build with -ffp-contract=off and without
 *     fast-math so no step is fused or reordered.
 *   - OpenMP parallelises over independent (b,c) columns only, so results do
 *     not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int wkv_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Two terms with log-weights x1 and x2, brought to a common scale: returns
 * the larger exponent m and sets *e1 = e^{x1-m}, *e2 = e^{x2-m} (both <= 1,
 * one of them exactly 1).  This is the shift that keeps every exp argument
 * <= 0 ([tm-math] "Numerical stability: carry the exponent").
 */
static double scaled_weights(double x1, double x2, double *e1, double *e2)
{
    double m = fmax(x1, x2);
    *e1 = exp(x1 - m);
    *e2 = exp(x2 - m);
    return m;
}

/*
 * One token of one channel on the state (a, b, p), whose true sums are
 * e^p*a (weighted values) and e^p*b (weights) ([tm-math] "Numerical
 * stability: carry the exponent"; the sums themselves are those of "The WKV
 * operator: attention with a fixed decay").
 *
 * Output: the history, at log-weight p, mixed with the current value, at
 * log-weight u + k (the bonus applies to the current token only and is not
 * stored).  State: the history decays by one token (log-weight p - w) and
 * the current value joins it at log-weight k; the larger of the two becomes
 * the new exponent.
 */
static double stabilised_token(double *a, double *b, double *p,
                               double k, double v, double w, double u)
{
    double hist, cur;   /* scaled weights of the history and of the current token */

    scaled_weights(*p, u + k, &hist, &cur);
    double y = (hist * *a + cur * v) / (hist * *b + cur);

    double p_next = scaled_weights(*p - w, k, &hist, &cur);
    *a = hist * *a + cur * v;
    *b = hist * *b + cur;
    *p = p_next;
    return y;
}

/*
 * Training/prefill form over all positions: the stabilised recurrence run
 * along t for every (b,c) column ([tm-math] "Why it collapses into a
 * recurrence": the scan over time parallelises across batch and channels),
 * returning y and the state after the last token ([multigrid] "Prefill,
 * decode, and where each form is used").
 * a_in/b_in/p_in: all NULL (empty history) or all non-NULL [B,C].
 * a_out/b_out/p_out: all NULL or all non-NULL [B,C].
 */
int wkv_oracle_forward(int64_t B, int64_t T, int64_t C,
                       const double *w, const double *u,
                       const double *k, const double *v,
                       const double *a_in, const double *b_in, const double *p_in,
                       double *y,
                       double *a_out, double *b_out, double *p_out)
{
    if (B < 0 || T < 0 || C < 0) return -2;
    int64_t ncol = B * C;
#pragma omp parallel for schedule(static)
    for (int64_t col = 0; col < ncol; col++) {
        int64_t bb = col / C, c = col % C;
        double a = 0.0, b = 0.0, p = -INFINITY;
        if (a_in) {
            a = a_in[col];
            b = b_in[col];
            p = p_in[col];
        }
        for (int64_t t = 0; t < T; t++) {
            int64_t i = (bb * T + t) * C + c;
            y[i] = stabilised_token(&a, &b, &p, k[i], v[i], w[c], u[c]);
        }
        if (a_out) {
            a_out[col] = a;
            b_out[col] = b;
            p_out[col] = p;
        }
    }
    return 0;
}

/*
 * Decode step: one token for every (l,s,c) of [L,S,C], with per-layer
 * parameters w,u [L,C] ([aiwiki] "wkv_step"; [vanos] "The WKV Operator",
 * inference mode; [multigrid] "Prefill, decode, ...", decode).
 * The state arrays are [L,S,C]; *_out may equal *_in.
 */
int wkv_oracle_step(int64_t L, int64_t S, int64_t C,
                    const double *w, const double *u,
                    const double *k, const double *v,
                    const double *a_in, const double *b_in, const double *p_in,
                    double *y,
                    double *a_out, double *b_out, double *p_out)
{
    if (L < 0 || S < 0 || C < 0) return -2;
    int64_t n = L * S * C;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++) {
        int64_t l = i / (S * C), c = i % C;
        double a = a_in[i], b = b_in[i], p = p_in[i];
        y[i] = stabilised_token(&a, &b, &p, k[i], v[i], w[l * C + c], u[l * C + c]);
        a_out[i] = a;
        b_out[i] = b;
        p_out[i] = p;
    }
    return 0;
}

/*
 * The summed (definition) form, O(T^2):
 *   wkv_t = [ sum_{i<t} e^{-(t-1-i)w + k_i} v_i + e^{u+k_t} v_t ]
 *         / [ sum_{i<t} e^{-(t-1-i)w + k_i}     + e^{u+k_t}     ]
 * ([tm-math] "The WKV operator: attention with a fixed decay"; [aiwiki]
 * introduction), with t and i counted from 0 here.  A prior state (a0,b0,p0)
 * stands for the sums accumulated before token 0; at output t it carries the
 * weight e^{p0 - t w} on a0 (numerator) and b0 (denominator).
 * Every weight is evaluated as e^{x - m} with m the largest exponent x of the
 * sum: numerator and denominator share the factor e^{-m}, so the ratio is
 * the definition's exactly ([tm-math] "Numerical stability": the
 * log-sum-exp shift).
 * The state after the last token comes from the same sums (the closed form of
 * the recurrence): p = the largest exponent among the terms of a_{T-1},
 * a = sum e^{x-p} v, b = sum e^{x-p}.
 */
int wkv_oracle_direct(int64_t B, int64_t T, int64_t C,
                      const double *w, const double *u,
                      const double *k, const double *v,
                      const double *a_in, const double *b_in, const double *p_in,
                      double *y,
                      double *a_out, double *b_out, double *p_out)
{
    if (B < 0 || T < 0 || C < 0) return -2;
    int64_t ncol = B * C;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t col = 0; col < ncol; col++) {
        int64_t bb = col / C, c = col % C;
        double wc = w[c], uc = u[c];
        int has_prior = a_in != NULL && p_in[col] > -INFINITY;
        for (int64_t t = 0; t < T; t++) {
            /* largest exponent among the terms of output t */
            double m = uc + k[(bb * T + t) * C + c];
            for (int64_t i = 0; i < t; i++) {
                double x = -(double)(t - 1 - i) * wc + k[(bb * T + i) * C + c];
                if (x > m) m = x;
            }
            double x0 = 0.0;
            if (has_prior) {
                x0 = p_in[col] - (double)t * wc;
                if (x0 > m) m = x0;
            }
            double num = 0.0, den = 0.0;
            if (has_prior) {
                num += exp(x0 - m) * a_in[col];
                den += exp(x0 - m) * b_in[col];
            }
            for (int64_t i = 0; i < t; i++) {
                int64_t ii = (bb * T + i) * C + c;
                double e = exp(-(double)(t - 1 - i) * wc + k[ii] - m);
                num += e * v[ii];
                den += e;
            }
            int64_t it = (bb * T + t) * C + c;
            double e_now = exp(uc + k[it] - m);
            num += e_now * v[it];
            den += e_now;
            y[it] = num / den;
        }
        if (a_out) {
            /* a_{T-1} = e^{-T w} A0 + sum_{i<T} e^{-(T-1-i)w + k_i} v_i */
            double m = -INFINITY;
            double x0 = 0.0;
            if (has_prior) {
                x0 = p_in[col] - (double)T * wc;
                m = x0;
            }
            for (int64_t i = 0; i < T; i++) {
                double x = -(double)(T - 1 - i) * wc + k[(bb * T + i) * C + c];
                if (x > m) m = x;
            }
            double sa = 0.0, sb = 0.0;
            if (has_prior) {
                sa += exp(x0 - m) * a_in[col];
                sb += exp(x0 - m) * b_in[col];
            }
            for (int64_t i = 0; i < T; i++) {
                int64_t ii = (bb * T + i) * C + c;
                double e = exp(-(double)(T - 1 - i) * wc + k[ii] - m);
                sa += e * v[ii];
                sb += e;
            }
            if (T == 0 && !has_prior) {
                sa = 0.0;
                sb = 0.0;
                m = -INFINITY;
                if (a_in) {           /* an explicit empty history passes through */
                    sa = a_in[col];
                    sb = b_in[col];
                    m = p_in[col];
                }
            }
            a_out[col] = sa;
            b_out[col] = sb;
            p_out[col] = m;
        }
    }
    return 0;
}

/*
 * Token shift, the two-tap causal lerp applied before the projections
 * ([tm-math] "Token shift: a two-tap causal convolution"; [multigrid]
 * "Token shift and channel mixing"), for the three blends mu_r, mu_k, mu_v:
 *   xbar_t = mu * x_t + (1 - mu) * x_{t-1}
 * x_{-1} is x_prev[b,:] when given, else 0 (causal zero padding).
 * x_last (optional) receives x_{T-1}, the shift state for the next call.
 */
int wkv_oracle_token_shift(int64_t B, int64_t T, int64_t C,
                           const double *x, const double *x_prev,
                           const double *mu_r, const double *mu_k, const double *mu_v,
                           double *xr, double *xk, double *xv, double *x_last)
{
    if (B < 0 || T < 0 || C < 0) return -2;
    int64_t ncol = B * C;
#pragma omp parallel for schedule(static)
    for (int64_t col = 0; col < ncol; col++) {
        int64_t bb = col / C, c = col % C;
        double prev = x_prev ? x_prev[col] : 0.0;
        for (int64_t t = 0; t < T; t++) {
            int64_t i = (bb * T + t) * C + c;
            double cur = x[i];
            xr[i] = mu_r[c] * cur + (1.0 - mu_r[c]) * prev;
            xk[i] = mu_k[c] * cur + (1.0 - mu_k[c]) * prev;
            xv[i] = mu_v[c] * cur + (1.0 - mu_v[c]) * prev;
            prev = cur;
        }
        if (x_last) x_last[col] = prev;
    }
    return 0;
}
