/*
 * CPU oracle of the DFlash 2 lightweight path selector -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The product path (the HIP library and its
 * binding) never links, imports or calls it, and the two share no code.
 *
 * Sources (web pages):
 *   [P1] "DFlash 2: Keep Drafting Parallel" (papercache.org summary):
 *        Quick read; Method > Lightweight Path Selector (eq. S_t, Table 2).
 *   [P3] "DFlash 2: The Drafter Stopped Guessing Alone" (rohitghumare.com):
 *        section "Selection beats correction".
 *
 * All arithmetic is fp64; bf16 inputs are widened exactly (bf16 -> f32 -> f64).
 * Arrays are host memory, row-major, owned by the caller.
 * Every function returns 0 on success, -1 on a bad size/pointer, -2 on a token
 * id outside [0, vocab).
 */
#ifndef DSEL_ORACLE_H
#define DSEL_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORA_K 16

/* [P1 Method, P3]: keep the 16 highest-scoring candidates of every draft
 * position.  Order: value descending, ties to the lower token id; -0.0 equals
 * +0.0; NaN ranks below -inf.  logits: rows x ld elements (fp32 when dtype==0,
 * bf16 bit patterns when dtype==1), first V of each row used. */
int ora_select_topk(const void *logits, int dtype, int64_t rows, int64_t V, int64_t ld,
                    int32_t *cand_id, float *cand_u);

/* [P1 Method, eq. S_t; P3]: A(x)=W_A.E[x], B(x)=W_B.E[x], H(h)=sigmoid(W_H.h).
 * A_prev[b,t,i,:] = A(pred_i(b,t)) with pred(b,0) = {verified[b]} (rows i>=1 of
 * t=0 are zero) and pred(b,t>=1) = cand_id[b,t-1,:];  B_cur[b,t,j,:] =
 * B(cand_id[b,t,j]);  G[b,t,:] = H(h[b,t,:]).
 * E [V,d], W_* [r,d], h [B,L,d] bf16 bits; outputs fp64
 * A_prev/B_cur [B,L,16,r], G [B,L,r]. */
int ora_project(const uint16_t *E, int64_t V, int64_t d,
                const uint16_t *W_A, const uint16_t *W_B, const uint16_t *W_H, int64_t r,
                const uint16_t *h, const int32_t *cand_id, const int32_t *verified,
                int64_t B, int64_t L, double *A_prev, double *B_cur, double *G);

/* [P1 eq. S_t]: S[b,t,i,j] = U[b,t,j] + sum_c A_prev[b,t,i,c] G[b,t,c] B_cur[b,t,j,c]
 * for i < n_t (n_0 = 1, n_t = 16); S[b,0,i>=1,:] = -inf.  U = cand_u. */
int ora_score_pairs(const float *cand_u, const double *A_prev, const double *B_cur,
                    const double *G, int64_t B, int64_t L, int64_t r, double *S);

/* One step of the walk from predecessor row `row` of S[b,t] (16x16).
 * mode 0 (greedy, [P1 Method; P3]): the highest score, ties to the lowest slot,
 *   NaN below -inf; aux = best minus runner-up.
 * mode 1 (sampled): inverse-CDF draw from softmax(S_row / T) in slot order with
 *   the caller's uniform u: the first j with u*Z < C_j; aux = distance of u*Z to
 *   the nearest CDF edge of the chosen slot, divided by Z.
 * q (16 entries, nullable) receives the step's distribution (one-hot for greedy). */
int ora_step(const double *S_bt, int row, int mode, double u, double T,
             int *choice, double *aux, double *q);

/* Walk every block from row 0: path_tok/path_slot [B,L] int32, path_s/aux [B,L],
 * q [B,L,16] nullable.  uniforms [B,L] used only in mode 1. */
int ora_walk(const double *S, const int32_t *cand_id, const float *uniforms, double T,
             int mode, int64_t B, int64_t L, int32_t *path_tok, int32_t *path_slot,
             double *path_s, double *aux, double *q);

/* Decision table: the step's choice and aux for every predecessor row:
 * choice/aux [B,L,16] (rows >= n_t are filled with -1 / NaN). */
int ora_step_table(const double *S, const float *uniforms, double T, int mode,
                   int64_t B, int64_t L, int32_t *choice, double *aux);

/* The whole selector (ora_select_topk, ora_project, ora_score_pairs, ora_walk
 * in that order) with each stage timed on the monotonic clock
 * (clock_gettime(CLOCK_MONOTONIC)), for the benchmark's CPU baseline: no
 * arithmetic of its own.  logits [B*L, V] (dtype as ora_select_topk),
 * uniforms [B,L] (mode 1).  Outputs path_slot [B,L]; sec[4] receives the
 * seconds of the four stages; threads receives omp_get_max_threads(). */
int ora_time_selector(const void *logits, int dtype, int64_t V, const uint16_t *E, int64_t d,
                      const uint16_t *W_A, const uint16_t *W_B, const uint16_t *W_H, int64_t r,
                      const uint16_t *h, const int32_t *verified, const float *uniforms, double T,
                      int mode, int64_t B, int64_t L, int32_t *path_slot, double *sec, int *threads);

/* ------------------------------------------------------ verification ---- */
/* Lossless verification of a drafted block against the target model ([P1]
 * Method, last paragraph, and Setup: sampling stays lossless through rejection
 * sampling; [P3] "One pass to draft, one pass to verify": the accepted prefix
 * is kept and the first miss is replaced by the target's own choice).
 *
 * target logits: rows (b, t), t = 0..L (row L follows the block), ld elements
 * apart, fp32 (dtype 0) or bf16 bits (dtype 1).  The drafted token of position
 * t is cand_id[b,t,path_slot[b,t]], drawn from q[b,t,:] (the walk's 16-way
 * distribution over the candidates).  L = 0 is allowed: a block that drafted
 * nothing tests nothing and takes its extra token from row 0 (plain decoding);
 * cand_id, path_slot, q and u_acc may then be NULL.
 *
 * mode 0 (greedy): accept while the drafted token is the target's arg max
 *   (ties to the lower id, NaN lowest); the first miss, or row L if all
 *   are accepted, contributes the target's arg max.
 * mode 1 (sampled, T > 0): p_t = softmax(z_t / T) over the vocabulary.
 *   Position t accepts its token x iff u_acc[b,t] * q_t(x) < p_t(x) (so with
 *   probability min(1, p/q)).  At the first rejection the extra token is drawn
 *   from r(v) = max(0, p_t(v) - q_t(v)) / Z_r, q_t being zero off the
 *   candidates; if all L are accepted it is drawn from p_L.  The draw is the
 *   inverse CDF in token-id order: the first v with u_res[b] * Z < C_v.
 *
 * Outputs: n_acc[b]; out_tok[b, 0..L]: the n_acc accepted tokens, then the
 * extra token at index n_acc, -1 after it.  Diagnostics (nullable):
 *   m_acc[b,t]  sampled: |u q - p| of each tested position (NaN when untested);
 *               greedy: NaN.
 *   m_draw[b]   sampled: distance of u Z to the nearest CDF edge of the drawn
 *               token, divided by Z; greedy: NaN. */
int ora_verify(const void *tlogits, int dtype, int64_t B, int64_t L, int64_t V, int64_t ld,
               const int32_t *cand_id, const int32_t *path_slot, const double *q, int mode,
               double T, const float *u_acc, const float *u_res, int32_t *n_acc,
               int32_t *out_tok, double *m_acc, double *m_draw);

/* The extra token alone, for a given position t of block b: with residual = 1
 * the draw from max(0, p_t - q_t), else from p_t (mode 1), or the arg max of
 * row t (mode 0).  *tok and *margin as above. */
int ora_verify_draw(const void *tlogits, int dtype, int64_t B, int64_t L, int64_t V, int64_t ld,
                    const int32_t *cand_id, const double *q, int mode, double T, const float *u_res,
                    int64_t b, int64_t t, int residual, int32_t *tok, double *margin);

/* Dynamic two-tap short convolution ([P1] Method > Lightweight Local
 * Convolution, eq. Conv_k; [P3] section "The decay at the end of the block"): a depthwise
 * convolution over the positions of each drafted block that reaches one
 * position back,
 *     y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1},
 * with every coefficient a learned base kernel plus a correction computed from
 * the current hidden state, one correction per 16 channels and tap:
 *     corr_t = W_c x_t                       (2 d/16 values, no bias),
 *     k_{t,j}[c] = base[j][c] + corr_t[j d/16 + c/16].
 * The first position of a block reads the last verified token's
 * representation: x_{-1} = x_prev[b].
 *   x       [B, L, d] bf16 bits      x_prev  [B, d] bf16 bits
 *   base    [2, d] bf16 bits (tap 0 = current position, tap 1 = previous)
 *   W_c     [2 d / 16, d] bf16 bits  (row j d/16 + g: tap j, channel group g)
 *   y       out [B, L, d] fp64;  corr  out [B, L, 2 d / 16] fp64 (nullable)
 * d must be a multiple of 16.  fp64 throughout. */
int ora_dyn_conv(const uint16_t *x, const uint16_t *x_prev, const uint16_t *base, const uint16_t *W_c,
                 int64_t B, int64_t L, int64_t d, double *y, double *corr);

/* LM head with the top-16 taken from its output ([P1] Method: the selector
 * reuses the drafter's logits, no extra LM-head forward; the head's top-16
 * are the selector's candidates): logits z[r, v] = sum_k h[r, k] W[v, k] in
 * fp64, then the first 16 of every row under the top-16 order (value
 * descending, ties to the lower id, NaN lowest).
 *   h      [rows, d] bf16 bits (the drafter's final hidden states)
 *   W      [V, d] bf16 bits (the LM-head weight, linear-layer layout)
 *   cand_id out [rows, 16] int32;  cand_z  out [rows, 17] fp64: the values of
 *          the 17 best (the 17th bounds what was left out; -inf if V = 16). */
int ora_lmhead_topk(const uint16_t *h, const uint16_t *W, int64_t rows, int64_t V, int64_t d,
                    int32_t *cand_id, double *cand_z);

#ifdef __cplusplus
}
#endif
#endif
