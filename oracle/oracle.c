/*
 * CPU oracle of the DFlash 2 lightweight path selector -- TEST INFRASTRUCTURE.
 * See oracle.h for the sources and the contract of every function.  Only the
 * tests, the package smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Plain loops, fp64 throughout, OpenMP over independent rows / positions.
 * No blocking, fusion or reordering beyond the definitions on the pages.
 */
#define _POSIX_C_SOURCE 199309L /* clock_gettime */
#include "oracle.h"

#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

static double bf16_to_f64(uint16_t u) {
    uint32_t bits = (uint32_t)u << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double logit_at(const void *logits, int dtype, int64_t idx) {
    if (dtype == 0) return (double)((const float *)logits)[idx];
    return bf16_to_f64(((const uint16_t *)logits)[idx]);
}

/* Total order of candidates: is (a, ia) ranked above (b, ib)?
 * Non-NaN above NaN; larger value first (-0.0 == +0.0 under IEEE compare);
 * equal values (or two NaNs) -> lower id first. */
static int ranks_above(double a, int64_t ia, double b, int64_t ib) {
    int an = isnan(a), bn = isnan(b);
    if (an != bn) return bn;
    if (!an && a != b) return a > b;
    return ia < ib;
}

/* ---------------------------------------------------------------- top-16 --- */
/* [P1 Method > Lightweight Path Selector; P3 "Selection beats correction"]:
 * the selector keeps the 16 best candidates of each draft position.  The first
 * 16 of the total order above, found by one pass of sorted insertion. */
int ora_select_topk(const void *logits, int dtype, int64_t rows, int64_t V, int64_t ld,
                    int32_t *cand_id, float *cand_u) {
    if (!logits || !cand_id || !cand_u || rows < 0 || V < ORA_K || ld < V) return -1;
    if (dtype != 0 && dtype != 1) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < rows; ++row) {
        double val[ORA_K];
        int64_t id[ORA_K];
        int n = 0;
        for (int64_t v = 0; v < V; ++v) {
            double x = logit_at(logits, dtype, row * ld + v);
            if (n == ORA_K && !ranks_above(x, v, val[ORA_K - 1], id[ORA_K - 1])) continue;
            int pos = (n < ORA_K) ? n : ORA_K - 1;     /* slot that gets overwritten */
            while (pos > 0 && ranks_above(x, v, val[pos - 1], id[pos - 1])) {
                val[pos] = val[pos - 1];
                id[pos] = id[pos - 1];
                --pos;
            }
            val[pos] = x;
            id[pos] = v;
            if (n < ORA_K) ++n;
        }
        for (int k = 0; k < ORA_K; ++k) {
            cand_id[row * ORA_K + k] = (int32_t)id[k];
            cand_u[row * ORA_K + k] = (float)val[k];   /* exact: the value came from fp32/bf16 */
        }
    }
    return 0;
}

/* ------------------------------------------------------------ projections --- */
/* y[c] = sum_k W[c,k] x[k] in fp64 (linear-layer layout W[r,d]). */
static void matvec(const uint16_t *W, const uint16_t *x, int64_t r, int64_t d, double *y) {
    for (int64_t c = 0; c < r; ++c) {
        double acc = 0.0;
        for (int64_t k = 0; k < d; ++k) acc += bf16_to_f64(W[c * d + k]) * bf16_to_f64(x[k]);
        y[c] = acc;
    }
}

/* [P1 Method, eq. S_t and the paragraph after it; P3]: A and B map a token to a
 * 256-d vector (here A(x) = W_A E[x], B(x) = W_B E[x]); H(h_t) is a gate from the
 * drafter's hidden state at position t (here sigmoid(W_H h_t)).  Predecessors:
 * the walk starts from the last verified token, so position 0 has one
 * predecessor; position t >= 1 has the 16 candidates of position t-1. */
int ora_project(const uint16_t *E, int64_t V, int64_t d,
                const uint16_t *W_A, const uint16_t *W_B, const uint16_t *W_H, int64_t r,
                const uint16_t *h, const int32_t *cand_id, const int32_t *verified,
                int64_t B, int64_t L, double *A_prev, double *B_cur, double *G) {
    if (!E || !W_A || !W_B || !W_H || !h || !cand_id || !verified || !A_prev || !B_cur || !G)
        return -1;
    if (V < 1 || d < 1 || r < 1 || B < 0 || L < 1) return -1;
    for (int64_t b = 0; b < B; ++b)
        if (verified[b] < 0 || verified[b] >= V) return -2;
    for (int64_t i = 0; i < B * L * ORA_K; ++i)
        if (cand_id[i] < 0 || cand_id[i] >= V) return -2;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bt = 0; bt < B * L; ++bt) {
        int64_t b = bt / L, t = bt % L;
        double *Ap = A_prev + bt * ORA_K * r;
        double *Bc = B_cur + bt * ORA_K * r;
        for (int i = 0; i < ORA_K; ++i) {
            if (t == 0) {
                if (i == 0) matvec(W_A, E + (int64_t)verified[b] * d, r, d, Ap);
                else for (int64_t c = 0; c < r; ++c) Ap[i * r + c] = 0.0;
            } else {
                int32_t tok = cand_id[(bt - 1) * ORA_K + i];
                matvec(W_A, E + (int64_t)tok * d, r, d, Ap + i * r);
            }
            matvec(W_B, E + (int64_t)cand_id[bt * ORA_K + i] * d, r, d, Bc + i * r);
        }
        double *g = G + bt * r;
        matvec(W_H, h + bt * d, r, d, g);
        for (int64_t c = 0; c < r; ++c) g[c] = 1.0 / (1.0 + exp(-g[c]));
    }
    return 0;
}

/* ----------------------------------------------------------------- scores --- */
/* [P1 eq. S_t]: S_t(a,b) = U_t(b) + < A(a) (.) H(h_t), B(b) >, U_t(b) the
 * drafter's raw logit of candidate b at position t. */
int ora_score_pairs(const float *cand_u, const double *A_prev, const double *B_cur,
                    const double *G, int64_t B, int64_t L, int64_t r, double *S) {
    if (!cand_u || !A_prev || !B_cur || !G || !S || B < 0 || L < 1 || r < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < B * L; ++bt) {
        int64_t t = bt % L;
        int n_t = (t == 0) ? 1 : ORA_K;
        for (int i = 0; i < ORA_K; ++i)
            for (int j = 0; j < ORA_K; ++j) {
                double *s = S + (bt * ORA_K + i) * ORA_K + j;
                if (i >= n_t) { *s = -INFINITY; continue; }
                double acc = 0.0;
                for (int64_t c = 0; c < r; ++c)
                    acc += A_prev[(bt * ORA_K + i) * r + c] * G[bt * r + c] *
                           B_cur[(bt * ORA_K + j) * r + c];
                *s = (double)cand_u[bt * ORA_K + j] + acc;
            }
    }
    return 0;
}

/* ------------------------------------------------------------------- walk --- */
/* [P1 Method, last paragraph; P3 "Selection beats correction"]: the only
 * sequential step walks the precomputed scores from the last verified token;
 * greedy follows the best successor, sampling draws from the same scores. */
int ora_step(const double *S_bt, int row, int mode, double u, double T,
             int *choice, double *aux, double *q) {
    if (!S_bt || !choice || !aux || row < 0 || row >= ORA_K) return -1;
    const double *s = S_bt + row * ORA_K;
    int best = 0;
    for (int j = 1; j < ORA_K; ++j)
        if (ranks_above(s[j], j, s[best], best)) best = j;

    if (mode == 0) {
        int second = (best == 0) ? 1 : 0;
        for (int j = 0; j < ORA_K; ++j)
            if (j != best && ranks_above(s[j], j, s[second], second)) second = j;
        *choice = best;
        *aux = s[best] - s[second];
        if (q) for (int j = 0; j < ORA_K; ++j) q[j] = (j == best) ? 1.0 : 0.0;
        return 0;
    }
    if (mode != 1 || !(T > 0.0)) return -1;

    /* softmax(S_row / T) with NaN entries given zero weight. */
    double m = -INFINITY;
    for (int j = 0; j < ORA_K; ++j)
        if (!isnan(s[j]) && s[j] > m) m = s[j];
    double e[ORA_K];
    if (m == -INFINITY) {            /* no entry has weight: fall back to the greedy pick */
        *choice = best;
        *aux = INFINITY;
        if (q) for (int j = 0; j < ORA_K; ++j) q[j] = (j == best) ? 1.0 : 0.0;
        return 0;
    }
    for (int j = 0; j < ORA_K; ++j) {
        if (isnan(s[j])) e[j] = 0.0;
        else if (m == INFINITY) e[j] = (s[j] == INFINITY) ? 1.0 : 0.0;
        else e[j] = exp((s[j] - m) / T);
    }
    double Z = 0.0, C[ORA_K];
    for (int j = 0; j < ORA_K; ++j) { Z += e[j]; C[j] = Z; }
    double uz = u * Z;
    int pick = -1;
    for (int j = 0; j < ORA_K; ++j)
        if (uz < C[j]) { pick = j; break; }
    if (pick < 0)
        for (int j = ORA_K - 1; j >= 0; --j)
            if (e[j] > 0.0) { pick = j; break; }
    double lo = (pick == 0) ? 0.0 : C[pick - 1];
    double d0 = fabs(uz - C[pick]), d1 = fabs(uz - lo);
    *choice = pick;
    *aux = ((d0 < d1) ? d0 : d1) / Z;
    if (q) for (int j = 0; j < ORA_K; ++j) q[j] = e[j] / Z;
    return 0;
}

int ora_walk(const double *S, const int32_t *cand_id, const float *uniforms, double T,
             int mode, int64_t B, int64_t L, int32_t *path_tok, int32_t *path_slot,
             double *path_s, double *aux, double *q) {
    if (!S || !cand_id || !path_tok || !path_slot || !path_s || !aux || B < 0 || L < 1) return -1;
    if (mode == 1 && (!uniforms || !(T > 0.0))) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t b = 0; b < B; ++b) {
        int row = 0;                                   /* the last verified token */
        for (int64_t t = 0; t < L; ++t) {
            int64_t bt = b * L + t;
            const double *S_bt = S + bt * ORA_K * ORA_K;
            int j = 0;
            double a = 0.0;
            double u = (mode == 1) ? (double)uniforms[bt] : 0.0;
            if (ora_step(S_bt, row, mode, u, T, &j, &a, q ? q + bt * ORA_K : NULL) != 0) {
                bad = 1;
                break;
            }
            path_slot[bt] = j;
            path_tok[bt] = cand_id[bt * ORA_K + j];
            path_s[bt] = S_bt[row * ORA_K + j];
            aux[bt] = a;
            row = j;
        }
    }
    return bad ? -1 : 0;
}

int ora_step_table(const double *S, const float *uniforms, double T, int mode,
                   int64_t B, int64_t L, int32_t *choice, double *aux) {
    if (!S || !choice || !aux || B < 0 || L < 1) return -1;
    if (mode == 1 && (!uniforms || !(T > 0.0))) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t bt = 0; bt < B * L; ++bt) {
        int n_t = (bt % L == 0) ? 1 : ORA_K;
        for (int row = 0; row < ORA_K; ++row) {
            if (row >= n_t) {
                choice[bt * ORA_K + row] = -1;
                aux[bt * ORA_K + row] = NAN;
                continue;
            }
            int j = 0;
            double a = 0.0;
            double u = (mode == 1) ? (double)uniforms[bt] : 0.0;
            if (ora_step(S + bt * ORA_K * ORA_K, row, mode, u, T, &j, &a, NULL) != 0) bad = 1;
            choice[bt * ORA_K + row] = j;
            aux[bt * ORA_K + row] = a;
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------ verification ---- */
/* [P1] Method (lossless rejection sampling restores the target's sampling
 * distribution) and Setup; [P3] "One pass to draft, one pass to verify".
 * Plain definitions, fp64: softmax over the whole vocabulary, the min(1, p/q)
 * acceptance as a multiply-compare, and the inverse-CDF draw in token order. */

/* arg max of a row, ties to the lower id, NaN lowest */
static int64_t row_argmax(const void *tl, int dtype, int64_t base, int64_t V) {
    int64_t best = 0;
    double bv = logit_at(tl, dtype, base);
    for (int64_t v = 1; v < V; ++v) {
        double x = logit_at(tl, dtype, base + v);
        if (ranks_above(x, v, bv, best)) {
            bv = x;
            best = v;
        }
    }
    return best;
}

/* max and sum of exp((z - max) / T) of a row */
static void row_softmax_stats(const void *tl, int dtype, int64_t base, int64_t V, double T, double *m,
                              double *Z) {
    double mx = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(tl, dtype, base + v);
        if (x > mx) mx = x;
    }
    double z = 0.0;
    for (int64_t v = 0; v < V; ++v) z += exp((logit_at(tl, dtype, base + v) - mx) / T);
    *m = mx;
    *Z = z;
}

/* q_t(v) of token v at (b, t): the candidate's weight, 0 off the candidates */
static double draft_q(const int32_t *cand_id, const double *q, int64_t bt, int64_t v) {
    for (int j = 0; j < ORA_K; ++j)
        if (cand_id[bt * ORA_K + j] == v) return q[bt * ORA_K + j];
    return 0.0;
}

/* inverse-CDF draw over the vocabulary from w(v) = p(v) (residual = 0) or
 * max(0, p(v) - q(v)) (residual = 1); p(v) = exp((z_v - m) / T) / Z */
static void draw_token(const void *tl, int dtype, int64_t base, int64_t V, double T, double m, double Z,
                       const int32_t *cand_id, const double *q, int64_t bt, int residual, double u,
                       int32_t *tok, double *margin) {
    double *w = (double *)malloc((size_t)V * sizeof(double));
    double tot = 0.0;
    for (int64_t v = 0; v < V; ++v) {
        double p = exp((logit_at(tl, dtype, base + v) - m) / T) / Z;
        if (residual) {
            double d = p - draft_q(cand_id, q, bt, v);
            p = d > 0.0 ? d : 0.0;
        }
        w[v] = p;
        tot += p;
    }
    const double target = u * tot;
    double c = 0.0, prev = 0.0;
    int64_t pick = -1, last_pos = -1;
    for (int64_t v = 0; v < V; ++v) {
        prev = c;
        c += w[v];
        if (w[v] > 0.0) last_pos = v;
        if (target < c) {
            pick = v;
            break;
        }
    }
    if (pick < 0) {  /* u Z at or past the total (rounding): the last token with weight */
        pick = last_pos;
        prev = c - (pick >= 0 ? w[pick] : 0.0);
    }
    *tok = (int32_t)pick;
    if (margin) {
        double lo = target - prev, hi = c - target;
        *margin = (tot > 0.0 ? (lo < hi ? lo : hi) / tot : NAN);
    }
    free(w);
}

int ora_verify_draw(const void *tlogits, int dtype, int64_t B, int64_t L, int64_t V, int64_t ld,
                    const int32_t *cand_id, const double *q, int mode, double T, const float *u_res,
                    int64_t b, int64_t t, int residual, int32_t *tok, double *margin) {
    if (!tlogits || !tok || b < 0 || b >= B || t < 0 || t > L || V < 1 || ld < V) return -1;
    const int64_t base = (b * (L + 1) + t) * ld;
    if (mode == 0) {
        *tok = (int32_t)row_argmax(tlogits, dtype, base, V);
        if (margin) *margin = NAN;
        return 0;
    }
    if (mode != 1 || !(T > 0.0) || !u_res || (residual && (!cand_id || !q || t >= L))) return -1;
    double m, Z;
    row_softmax_stats(tlogits, dtype, base, V, T, &m, &Z);
    draw_token(tlogits, dtype, base, V, T, m, Z, cand_id, q, b * L + t, residual, (double)u_res[b], tok,
               margin);
    return 0;
}

int ora_verify(const void *tlogits, int dtype, int64_t B, int64_t L, int64_t V, int64_t ld,
               const int32_t *cand_id, const int32_t *path_slot, const double *q, int mode,
               double T, const float *u_acc, const float *u_res, int32_t *n_acc,
               int32_t *out_tok, double *m_acc, double *m_draw) {
    /* L = 0 is a block that drafted nothing: no test, the extra token from row 0 */
    if (!tlogits || !n_acc || !out_tok || B < 0 || L < 0 || V < 1 || ld < V) return -1;
    if (L > 0 && (!cand_id || !path_slot)) return -1;
    if (dtype != 0 && dtype != 1) return -1;
    if (mode == 1 && (!u_res || !(T > 0.0) || (L > 0 && (!q || !u_acc)))) return -1;
    if (mode != 0 && mode != 1) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        int64_t t = 0;
        for (; t < L; ++t) {
            const int64_t bt = b * L + t;
            const int32_t x = cand_id[bt * ORA_K + path_slot[bt]];
            const int64_t base = (b * (L + 1) + t) * ld;
            int ok;
            if (mode == 0) {
                ok = row_argmax(tlogits, dtype, base, V) == x;
                if (m_acc) m_acc[bt] = NAN;
            } else {
                double m, Z;
                row_softmax_stats(tlogits, dtype, base, V, T, &m, &Z);
                const double px = exp((logit_at(tlogits, dtype, base + x) - m) / T) / Z;
                const double lhs = (double)u_acc[bt] * q[bt * ORA_K + path_slot[bt]];
                ok = lhs < px;
                if (m_acc) m_acc[bt] = fabs(lhs - px);
            }
            if (!ok) break;
            out_tok[b * (L + 1) + t] = x;
        }
        for (int64_t s = t + 1; s < L; ++s)
            if (m_acc) m_acc[b * L + s] = NAN;
        n_acc[b] = (int32_t)t;
        int32_t tok;
        double mg = NAN;
        ora_verify_draw(tlogits, dtype, B, L, V, ld, cand_id, q, mode, T, u_res, b, t, t < L, &tok, &mg);
        out_tok[b * (L + 1) + t] = tok;
        for (int64_t s = t + 1; s <= L; ++s) out_tok[b * (L + 1) + s] = -1;
        if (m_draw) m_draw[b] = mg;
    }
    return 0;
}

/* ------------------------------------------------- dynamic short conv --- */
/* [P1 Method > Lightweight Local Convolution, eq. Conv_k; P3 section "The decay
 * at the end of the block"]: y_t = k_{t,0} x_t + k_{t,1} x_{t-1}, each coefficient the base
 * kernel plus the correction of its 16-channel group, computed from x_t; the
 * block's first position reads the last verified token. */
int ora_dyn_conv(const uint16_t *x, const uint16_t *x_prev, const uint16_t *base, const uint16_t *W_c,
                 int64_t B, int64_t L, int64_t d, double *y, double *corr) {
    if (!x || !x_prev || !base || !W_c || !y || B < 0 || L < 1 || d < 16 || d % 16 != 0) return -1;
    const int64_t G = d / 16;  /* correction groups per tap */
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < B * L; ++bt) {
        const int64_t b = bt / L, t = bt % L;
        const uint16_t *xt = x + bt * d;
        const uint16_t *xp = t == 0 ? x_prev + b * d : x + (bt - 1) * d;
        double *c = (double *)malloc((size_t)(2 * G) * sizeof(double));
        for (int64_t n = 0; n < 2 * G; ++n) {  /* corr_t = W_c x_t */
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k) acc += bf16_to_f64(W_c[n * d + k]) * bf16_to_f64(xt[k]);
            c[n] = acc;
        }
        for (int64_t ch = 0; ch < d; ++ch) {
            const double k0 = bf16_to_f64(base[ch]) + c[ch / 16];
            const double k1 = bf16_to_f64(base[d + ch]) + c[G + ch / 16];
            y[bt * d + ch] = k0 * bf16_to_f64(xt[ch]) + k1 * bf16_to_f64(xp[ch]);
        }
        if (corr)
            for (int64_t n = 0; n < 2 * G; ++n) corr[bt * 2 * G + n] = c[n];
        free(c);
    }
    return 0;
}

/* ------------------------------------------------- LM head + top-16 --- */
/* [P1 Method: candidates are the drafter's own top-16 logits, with no extra
 * LM-head forward]: z = h W^T in fp64, then sorted insertion under the same
 * total order as ora_select_topk, keeping 17 so the caller can see the margin
 * of the 16th. */
int ora_lmhead_topk(const uint16_t *h, const uint16_t *W, int64_t rows, int64_t V, int64_t d,
                    int32_t *cand_id, double *cand_z) {
    if (!h || !W || !cand_id || !cand_z || rows < 0 || V < ORA_K || d < 1) return -1;
    enum { KK = ORA_K + 1 };
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t row = 0; row < rows; ++row) {
        double val[KK];
        int64_t id[KK];
        int n = 0;
        double *hr = (double *)malloc((size_t)d * sizeof(double));
        for (int64_t k = 0; k < d; ++k) hr[k] = bf16_to_f64(h[row * d + k]);
        for (int64_t v = 0; v < V; ++v) {
            double z = 0.0;
            for (int64_t k = 0; k < d; ++k) z += hr[k] * bf16_to_f64(W[v * d + k]);
            if (n == KK && !ranks_above(z, v, val[KK - 1], id[KK - 1])) continue;
            int pos = (n < KK) ? n : KK - 1;
            while (pos > 0 && ranks_above(z, v, val[pos - 1], id[pos - 1])) {
                val[pos] = val[pos - 1];
                id[pos] = id[pos - 1];
                --pos;
            }
            val[pos] = z;
            id[pos] = v;
            if (n < KK) ++n;
        }
        for (int j = 0; j < ORA_K; ++j) cand_id[row * ORA_K + j] = (int32_t)id[j];
        for (int j = 0; j < KK; ++j) cand_z[row * KK + j] = j < n ? val[j] : -INFINITY;
        free(hr);
    }
    return 0;
}

/* ---------------------------------------------------- timed selector ---- */
static double mono_s(void) {
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

int ora_time_selector(const void *logits, int dtype, int64_t V, const uint16_t *E, int64_t d,
                      const uint16_t *W_A, const uint16_t *W_B, const uint16_t *W_H, int64_t r,
                      const uint16_t *h, const int32_t *verified, const float *uniforms, double T,
                      int mode, int64_t B, int64_t L, int32_t *path_slot, double *sec, int *threads) {
    if (!logits || !path_slot || !sec || B < 1 || L < 1 || r < 1) return -1;
    const int64_t pos = B * L;
    int32_t *cand_id = malloc(sizeof(int32_t) * pos * ORA_K);
    float *cand_u = malloc(sizeof(float) * pos * ORA_K);
    double *A = malloc(sizeof(double) * pos * ORA_K * r), *Bm = malloc(sizeof(double) * pos * ORA_K * r);
    double *G = malloc(sizeof(double) * pos * r), *S = malloc(sizeof(double) * pos * ORA_K * ORA_K);
    int32_t *tok = malloc(sizeof(int32_t) * pos);
    double *ps = malloc(sizeof(double) * pos), *aux = malloc(sizeof(double) * pos);
    int rc = -1;
    if (cand_id && cand_u && A && Bm && G && S && tok && ps && aux) {
        const double t0 = mono_s();
        rc = ora_select_topk(logits, dtype, pos, V, V, cand_id, cand_u);
        const double t1 = mono_s();
        if (rc == 0) rc = ora_project(E, V, d, W_A, W_B, W_H, r, h, cand_id, verified, B, L, A, Bm, G);
        const double t2 = mono_s();
        if (rc == 0) rc = ora_score_pairs(cand_u, A, Bm, G, B, L, r, S);
        const double t3 = mono_s();
        if (rc == 0) rc = ora_walk(S, cand_id, uniforms, T, mode, B, L, tok, path_slot, ps, aux, NULL);
        const double t4 = mono_s();
        sec[0] = t1 - t0;
        sec[1] = t2 - t1;
        sec[2] = t3 - t2;
        sec[3] = t4 - t3;
    }
    if (threads) *threads = omp_get_max_threads();
    free(cand_id);
    free(cand_u);
    free(A);
    free(Bm);
    free(G);
    free(S);
    free(tok);
    free(ps);
    free(aux);
    return rc;
}
