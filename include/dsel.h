/*
 * dsel -- the DFlash 2 lightweight path selector on AMD MI355X (gfx950).
 *
 * C ABI of libdsel.so.  Sources (web pages):
 *   [P1] "DFlash 2: Keep Drafting Parallel" (papercache.org summary),
 *        Quick read; Method > Lightweight Path Selector (eq. S_t, Table 2).
 *   [P3] "DFlash 2: The Drafter Stopped Guessing Alone" (rohitghumare.com),
 *        section "Selection beats correction".
 *
 * The selector keeps the top-16 candidates of every draft position, scores
 * every adjacent candidate pair with
 *     S_t(a, b) = U_t(b) + < A(a) (.) H(h_t), B(b) >
 * in one parallel pass, and walks the precomputed scores from the last verified
 * token, greedily or by sampling.  Here A(x) = W_A E[x], B(x) = W_B E[x] and
 * H(h) = sigmoid(W_H h) (three r x d matrices: the shape whose parameter count
 * matches the 2.0M of [P1] Table 2 at d = 2560, r = 256).
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers owned by the caller; layouts are
 *     contiguous row-major unless a leading dimension is given.  bf16 tensors
 *     are passed as their 16-bit patterns (uint16_t).
 *   - The library allocates nothing and keeps no pointer after a call returns.
 *     Inputs are never written; outputs must not alias inputs.
 *   - Every argument is validated on the host before anything is launched.  On
 *     a validation failure the call returns a negative status and writes
 *     nothing.  A failed launch returns DSEL_E_HIP.  A call with no work
 *     (batch * block == 0) returns DSEL_OK after checking its sizes; its
 *     pointers may then be NULL.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream); results are valid once the stream has been synchronised.  No
 *     C++ exception crosses the boundary.  Calls on different streams may run
 *     concurrently, except that the device error word (dsel_device_error) is
 *     shared by all calls on one device.
 *
 * Ragged batches.  The block size is a per-request knob ([P1] supplementary
 * deployment notes: oMLX runs blocks of 5, the release tables use 8 and 16;
 * [P3] "What to check on your own serving").  Every call that takes `batch`
 * and `block` also takes `block_len`: NULL for a uniform batch, else a DEVICE
 * array [batch] of int32 (4-byte aligned) giving block b's valid positions,
 * 0 <= block_len[b] <= block, in the same padded [batch, block] layout.  Block
 * b is then computed exactly as it would be alone at length block_len[b]
 * (same bits).  Outputs at padding positions (t >= block_len[b]) are not
 * written, except where a call says so, and inputs there never affect a result
 * (they may hold anything, NaN included); a length outside [0, block] makes the
 * block empty and sets DSEL_DEVERR_BLOCK_LEN.  The launch geometry is that of
 * the padded batch: workgroups with only padding to do exit at once.
 */
#ifndef DSEL_H
#define DSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSEL_K 16          /* candidates kept per draft position ([P1] Method) */
#define DSEL_MAX_BLOCK 32  /* longest draft block accepted by score_pairs / walk */
#define DSEL_MAX_RANK 256  /* largest selector rank r ([P1]: 256-d token vectors) */

typedef void *dsel_stream_t; /* a hipStream_t */

typedef enum {
    DSEL_OK = 0,
    DSEL_E_ARG = -1,       /* null pointer, bad size or out-of-range scalar */
    DSEL_E_DTYPE = -2,     /* unknown dtype or walk mode */
    DSEL_E_ALIGN = -3,     /* pointer or leading dimension misaligned */
    DSEL_E_WORKSPACE = -4, /* workspace missing or too small */
    DSEL_E_HIP = -5        /* a HIP runtime call or kernel launch failed */
} dsel_status;

typedef enum { DSEL_F32 = 0, DSEL_BF16 = 1 } dsel_dtype;
typedef enum { DSEL_GREEDY = 0, DSEL_SAMPLED = 1 } dsel_walk_mode;

/* Device error word bits (see dsel_device_error). */
#define DSEL_DEVERR_TOKEN_RANGE 1 /* dsel_project met a token id outside [0, vocab) */
#define DSEL_DEVERR_BLOCK_LEN 2   /* a block_len entry outside [0, block] */

/* Bytes of device workspace dsel_select_topk needs for `rows` = batch*block rows
 * of `vocab` logits of type `dt` (0 when it needs none).  Returns 0 for
 * invalid arguments too; dsel_select_topk validates. */
size_t dsel_topk_workspace_bytes(int64_t rows, int64_t vocab, dsel_dtype dt);

/* select_topk -- [P1] Method > Lightweight Path Selector, [P3]: keep the 16
 * best candidates of every draft position.
 *   logits   [batch*block rows][ld] of dtype `dt` (fp32, or bf16 bits); the
 *            first `vocab` entries of each row are the position's raw logits.
 *            Pointer aligned to the element size; any ld >= vocab.  Only the
 *            first vocab elements of each row are read.
 *   cand_id  out [batch, block, 16] int32: token ids, ordered by logit
 *            descending, ties to the lower id; -0.0 equals +0.0 and NaN ranks
 *            below -inf.  The ordered list is unique, so results are bit-exact.
 *   cand_u   out [batch, block, 16] fp32: the logit of each candidate, widened
 *            exactly (these are U_t(b) of eq. S_t).
 *   workspace  device scratch of at least dsel_topk_workspace_bytes() bytes
 *            (may be NULL when that is 0); contents need no initialisation.
 * Requirements: 16 <= vocab < 2^31, ld >= vocab, batch*block >= 0. */
dsel_status dsel_select_topk(const void *logits, dsel_dtype dt, int64_t batch, int64_t block,
                             const int32_t *block_len, int64_t vocab, int64_t ld, int32_t *cand_id,
                             float *cand_u, void *workspace, size_t workspace_bytes,
                             dsel_stream_t stream);

/* project -- [P1] Method (the paragraph after eq. S_t), [P3]: the compact token
 * vectors and the context gate, for every candidate and predecessor.
 *   E        [vocab, d] bf16: the drafter's token embedding table.
 *   W_A, W_B, W_H  [r, d] bf16 (linear-layer layout: y = W x).
 *   h        [batch, block, d] bf16: drafter hidden state of every position.
 *   cand_id  [batch, block, 16] int32 (from dsel_select_topk).
 *   verified [batch] int32: last verified token of every block (the walk's
 *            start, [P1] Method last paragraph).
 *   A_prev   out [batch, block, 16, r] fp32: A of each predecessor.  Position 0
 *            has one predecessor (row 0 = A(verified)); rows 1..15 of position
 *            0 are written as zeros.  Position t >= 1: row i = A(cand_id[t-1][i]).
 *            (Ragged batches: an empty block reads no verified token and has
 *            no position 0.)
 *   B_cur    out [batch, block, 16, r] fp32: row j = B(cand_id[t][j]).
 *   G        out [batch, block, r] fp32: sigmoid(W_H h[t]).
 * Products are bf16 x bf16 with fp32 accumulation (MFMA).  A token id outside
 * [0, vocab) reads a zero embedding row and sets DSEL_DEVERR_TOKEN_RANGE in the
 * device error word.
 *   workspace  device scratch of at least dsel_project_workspace_bytes() bytes
 *            (may be NULL when that is 0); contents need no initialisation.
 * Requirements: d % 64 == 0, r % 32 == 0, 32 <= r <= 256, 1 <= block,
 * batch >= 0, 1 <= vocab < 2^31; all pointers 16-byte aligned. */
dsel_status dsel_project(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                         const uint16_t *W_B, const uint16_t *W_H, int64_t r, const uint16_t *h,
                         const int32_t *cand_id, const int32_t *verified, int64_t batch,
                         int64_t block, const int32_t *block_len, float *A_prev, float *B_cur,
                         float *G, void *workspace, size_t workspace_bytes, dsel_stream_t stream);

/* Bytes of device workspace dsel_project needs (0 when none; also 0 for
 * invalid arguments, which the calls themselves reject).  Small GEMMs are split
 * along d across workgroups and their partial sums kept here. */
size_t dsel_project_workspace_bytes(int64_t batch, int64_t block, int64_t d, int64_t r);

/* The two halves of dsel_project, for callers that schedule them apart:
 * project_gate needs no candidates (G and position 0's predecessor rows of
 * A_prev), so it may run while dsel_select_topk is still running, e.g. on a
 * second stream; project_cand computes B_cur and A_prev of positions >= 1 from
 * the candidates.  Arguments, layouts and requirements as for dsel_project;
 * each writes only the outputs named here.  Both take a workspace sized by
 * dsel_project_workspace_bytes and use disjoint parts of it, so one workspace
 * can serve both calls, even while they run concurrently on two streams (two
 * calls of the same half must not share one workspace concurrently). */
dsel_status dsel_project_gate(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                              const uint16_t *W_H, int64_t r, const uint16_t *h,
                              const int32_t *verified, int64_t batch, int64_t block,
                              const int32_t *block_len, float *A_prev, float *G, void *workspace,
                              size_t workspace_bytes, dsel_stream_t stream);
/* project_gate for running beside another kernel, e.g. dsel_select_topk on a
 * second stream: the same outputs as dsel_project_gate, bit for bit except
 * for the order of the fp32 sums over d, computed with one workgroup per
 * 128-row output tile, no split along d and no workspace, so it occupies few
 * CUs (9 at 64 x 16 positions) for longer instead of the whole chip briefly.
 * Arguments, layouts and requirements as for dsel_project_gate. */
dsel_status dsel_project_gate_overlap(const uint16_t *E, int64_t vocab, int64_t d,
                                      const uint16_t *W_A, const uint16_t *W_H, int64_t r,
                                      const uint16_t *h, const int32_t *verified, int64_t batch,
                                      int64_t block, const int32_t *block_len, float *A_prev,
                                      float *G, dsel_stream_t stream);
dsel_status dsel_project_cand(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                              const uint16_t *W_B, int64_t r, const int32_t *cand_id, int64_t batch,
                              int64_t block, const int32_t *block_len, float *A_prev, float *B_cur,
                              void *workspace, size_t workspace_bytes, dsel_stream_t stream);

/* Walk arguments ([P1] Method last paragraph, [P3]: the only sequential step;
 * greedy follows the best successor, sampling draws from the same scores).
 *   mode        DSEL_GREEDY: at each position take the highest score in the row
 *               of the previous pick (row 0 at position 0), ties to the lowest
 *               slot, NaN below -inf.
 *               DSEL_SAMPLED: draw from softmax(S_row / temperature) by inverse
 *               CDF in slot order: the first slot j with u*Z < C_j (Z the sum
 *               of the exponentials, C_j their running sum, u the caller's
 *               uniform); NaN scores get zero weight; a row with no weight
 *               falls back to the greedy pick.
 *   temperature > 0 (SAMPLED only).
 *   uniforms    [batch, block] fp32 in [0, 1) (SAMPLED only, else may be NULL).
 *   cand_id     [batch, block, 16] int32.
 *   path_tok    out [batch, block] int32: the chosen token at every position.
 *   path_slot   out [batch, block] int32: its slot in cand_id.
 *   path_s      out [batch, block] fp32: its score (nullable).
 *   q           out [batch, block, 16] fp32: the step's distribution over the
 *               16 successors (one-hot for greedy) (nullable). */
typedef struct {
    int32_t mode;
    float temperature;
    const float *uniforms;
    const int32_t *cand_id;
    int32_t *path_tok;
    int32_t *path_slot;
    float *path_s;
    float *q;
} dsel_walk_args;

/* score_pairs -- [P1] eq. S_t, [P3]: every adjacent candidate pair scored in one
 * parallel pass:
 *   S[b,t,i,j] = cand_u[b,t,j] + sum_c A_prev[b,t,i,c] G[b,t,c] B_cur[b,t,j,c]
 * for i < n_t (n_0 = 1, n_t = 16 for t >= 1); S[b,0,i>=1,:] = -inf.
 * fp32 arithmetic.  Inputs as produced by dsel_project / dsel_select_topk.
 *   S     out [batch, block, 16, 16] fp32 (required: the walk reads it).
 *   walk  nullable: when given, the walk over S follows on the same stream.
 * Requirements: 1 <= block <= DSEL_MAX_BLOCK, r % 32 == 0, 32 <= r <= 256;
 * pointers 16-byte aligned. */
dsel_status dsel_score_pairs(const float *cand_u, const float *A_prev, const float *B_cur,
                             const float *G, int64_t batch, int64_t block, const int32_t *block_len,
                             int64_t r, float *S, const dsel_walk_args *walk, dsel_stream_t stream);

/* walk -- the walk alone over given scores S [batch, block, 16, 16] fp32 (same
 * rules as the fused walk of dsel_score_pairs; row 0 is the predecessor at
 * position 0).  Ragged batches: block b walks its first block_len[b]
 * positions.  Requirements: 1 <= block <= DSEL_MAX_BLOCK. */
dsel_status dsel_walk(const float *S, int64_t batch, int64_t block, const int32_t *block_len,
                      const dsel_walk_args *walk, dsel_stream_t stream);

/* project_pairs -- dsel_project_cand and the pair term of dsel_score_pairs in
 * one kernel, for blocks of at most 16 positions ([P1] Method > Lightweight
 * Path Selector: A and B map tokens to 256-d vectors, eq. S_t scores every
 * adjacent pair in one parallel pass).  One workgroup per tile of whole blocks
 * (floor(16 / block) blocks, 256 candidate rows) and column group q of the
 * rank (CW = 64 columns when r % 64 == 0 and r >= 128, else 32; nq = r / CW
 * groups, dsel_pair_groups(r)) computes A and B of the group for every
 * candidate of the tile on bf16 MFMA (fp32 accumulation) and then
 *     partials[b,t,q,i,j] = sum_{c in group q} A_prev[b,t,i,c] G[b,t,c] B_cur[b,t,j,c]
 * in fp32 (for position 0 only row i = 0 is meaningful: its one predecessor is
 * the verified token).  A and B stay on chip unless asked for.
 *   cand_id    [batch, block, 16] int32 (from dsel_select_topk).
 *   G          [batch, block, r] fp32 (from dsel_project_gate).
 *   A_ver, ver_stride  A(verified token of block b) is read at A_ver + b *
 *              ver_stride (r floats; ver_stride >= r, a multiple of 4): e.g.
 *              the A_prev written by dsel_project_gate with ver_stride =
 *              block * 16 * r.
 *   partials   out [batch, block, nq, 16, 16] fp32.
 *   A_prev, B_cur  optional outputs (both NULL or both given), written as
 *              dsel_project_cand writes them (A_prev of position 0 is not).
 * dsel_walk_pairs then adds the groups in order to cand_u; the result has the
 * same bits as dsel_project_cand + dsel_score_pairs.  Token ids outside [0,
 * vocab) read a zero row and set DSEL_DEVERR_TOKEN_RANGE.
 * Requirements: 1 <= block <= 16; otherwise as dsel_project_cand. */
int64_t dsel_pair_groups(int64_t r); /* nq for rank r (0 for an invalid r) */
dsel_status dsel_project_pairs(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                               const uint16_t *W_B, int64_t r, const int32_t *cand_id, const float *G,
                               const float *A_ver, int64_t ver_stride, int64_t batch, int64_t block,
                               const int32_t *block_len, float *partials, float *A_prev, float *B_cur,
                               dsel_stream_t stream);

/* walk_pairs -- the scores from dsel_project_pairs' partial tables and the walk
 * over them: S[b,t,i,j] = cand_u[b,t,j] + (((partials[b,t,0,i,j] +
 * partials[b,t,1,i,j]) + ...) with S[b,0,i>=1,:] = -inf, then the walk of
 * dsel_score_pairs (same bits).
 *   partials  [batch, block, nq, 16, 16] fp32, nq = dsel_pair_groups(r).
 *   S      out [batch, block, 16, 16] fp32, nullable (the walk does not need it).
 *   walk   required.
 * Requirements: 1 <= block <= DSEL_MAX_BLOCK, 1 <= nq <= 8; partials 16-byte
 * aligned. */
dsel_status dsel_walk_pairs(const float *cand_u, const float *partials, int64_t batch, int64_t block,
                            const int32_t *block_len, int64_t nq, float *S, const dsel_walk_args *walk,
                            dsel_stream_t stream);

/* select_path -- the whole selector in one call ([P1] Method > Lightweight Path
 * Selector, [P3] "Selection beats correction"): dsel_select_topk, dsel_project
 * (gate and candidates), dsel_score_pairs and the walk, on one stream, with the
 * same outputs bit for bit as those calls made one after the other.  The gate
 * GEMM's split-K reduction runs inside the top-16 launch, beside it, instead of
 * as a launch of its own.
 *   Inputs and outputs are those of the separate calls; `vocab` is the
 *   logits' width in use, and E needs at least `vocab` rows (every candidate
 *   id is below it; the projections' id check uses it).  cand_id and cand_u
 *   are required.  A_prev and B_cur are optional together (both NULL or both
 *   given), G and S are optional each: a NULL output is not written.
 *   Route.  For blocks of at most 16 positions and batches large enough to
 *   fill the chip (ceil(batch / floor(16 / block)) * dsel_pair_groups(r) >=
 *   128 workgroups), the candidate projections and the pair term run as the
 *   kernels of dsel_project_pairs and dsel_walk_pairs: A and B stay on chip
 *   and only each group's 16 x 16 partial table per position leaves it.
 *   Otherwise, for small batches (at most 32 positions) whose gate GEMM is
 *   split along K with column tiles at most 64 wide, and when
 *   A_prev, B_cur and G are not asked for, three launches do the work: the
 *   top-16 in partial lists beside the gate GEMM; the candidate GEMM, each of
 *   its workgroups merging the lists of its own positions first; and, per
 *   position and group of the rank, the split sums, the pair table and (by
 *   the last workgroup of each block to finish, counted with an atomic
 *   counter) the walk.  Otherwise the separate kernels run and A_prev, B_cur
 *   and S pass through the workspace when not asked for.  Every route gives
 *   the same bits; dsel_select_path_route tells which one a call takes.
 *   walk       the walk arguments (required), as for dsel_score_pairs.
 *   workspace  at least dsel_select_path_workspace_bytes() bytes (256-byte
 *              aligned); contents need no initialisation.
 * Requirements: those of every step (d % 64 == 0; r % 32 == 0, 32 <= r <= 256;
 * 1 <= block <= DSEL_MAX_BLOCK; 16 <= vocab < 2^31; ld >= vocab). */
typedef struct {
    const void *logits;   /* [batch*block][ld] of dtype dt */
    dsel_dtype dt;
    int64_t vocab, ld;
    const uint16_t *E;    /* [>= vocab, d] bf16 */
    int64_t d;
    const uint16_t *W_A, *W_B, *W_H; /* [r, d] bf16 */
    int64_t r;
    const uint16_t *h;    /* [batch, block, d] bf16 */
    const int32_t *verified; /* [batch] */
    int64_t batch, block;
    const int32_t *block_len; /* [batch] or NULL (see "Ragged batches") */
    int32_t *cand_id;     /* out [batch, block, 16] */
    float *cand_u;        /* out [batch, block, 16] */
    float *A_prev, *B_cur; /* out [batch, block, 16, r], both or neither (nullable) */
    float *G;             /* out [batch, block, r] (nullable) */
    float *S;             /* out [batch, block, 16, 16] (nullable) */
} dsel_path_args;
size_t dsel_select_path_workspace_bytes(int64_t batch, int64_t block, int64_t vocab, dsel_dtype dt, int64_t d,
                                        int64_t r);
dsel_status dsel_select_path(const dsel_path_args *args, const dsel_walk_args *walk, void *workspace,
                             size_t workspace_bytes, dsel_stream_t stream);
/* The route dsel_select_path takes for these arguments (only the shape and
 * which outputs are given are read): DSEL_ROUTE_FUSED, DSEL_ROUTE_SMALL or
 * DSEL_ROUTE_SEPARATE; -1 for an empty batch or an invalid shape. */
#define DSEL_ROUTE_SEPARATE 0
#define DSEL_ROUTE_FUSED 1
#define DSEL_ROUTE_SMALL 2
int dsel_select_path_route(const dsel_path_args *args);

/* select_path_noalloc -- dsel_select_path for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and outputs bit for bit, without a caller
 * workspace.  Its workspace is a fixed device array of the library, one per
 * device (DSEL_NOALLOC_MAX_WORKSPACE bytes, 48 MiB: enough for 256 blocks of
 * 16 positions at vocab 202,048, d 6,144, r 256, which need 33 MiB), looked
 * up on the device that is current at the call.  The call allocates nothing.
 * A shape whose dsel_select_path_workspace_bytes() exceeds the array returns
 * DSEL_E_WORKSPACE before anything is launched.  Every call on one device
 * shares that device's array: calls that overlap on one device (two streams,
 * two threads) race and must not be issued; calls in one stream are ordered.
 * Nothing in the array needs to start at zero.  Returns DSEL_E_HIP when the
 * array's address cannot be looked up. */
#define DSEL_NOALLOC_MAX_WORKSPACE (48u << 20)
dsel_status dsel_select_path_noalloc(const dsel_path_args *args, const dsel_walk_args *walk,
                                     dsel_stream_t stream);

/* gather_probe -- a measurement aid, not a step of the path: the gather of
 * dsel_project_cand alone.  Rows E[cand_id[m]] (m over batch*block*16) are
 * moved into LDS with the same LDS-DMA addressing as the candidate GEMM, with
 * no arithmetic, so the gather's HBM rate can be measured apart from the MFMAs
 * it feeds.  Each thread folds what it sees into one word of `out` (so no load
 * can be dropped); the words mean nothing else.
 *   out        device array of at least dsel_gather_probe_words() uint32.
 * Requirements: as dsel_project_cand (d % 64 == 0). */
size_t dsel_gather_probe_words(int64_t batch, int64_t block, int64_t d);
dsel_status dsel_gather_probe(const uint16_t *E, int64_t vocab, int64_t d, const int32_t *cand_id,
                              int64_t batch, int64_t block, uint32_t *out, size_t out_words,
                              dsel_stream_t stream);

/* verify -- lossless verification of the drafted blocks against the target
 * model, the step after the walk ([P1] Method, last paragraph, and Setup:
 * sampling stays lossless through rejection sampling; [P3] "One pass to draft,
 * one pass to verify": the accepted prefix is kept and the first miss is
 * replaced by the target's own choice).
 *   target_logits  [batch * (block + 1)][ld] of dtype `dt`: row (b, t) holds
 *                  the target's logits for position t of block b (row t = block
 *                  is the position after the block).  Row starts must be 16-byte
 *                  aligned (pointer and ld * element size); 16 <= vocab <=
 *                  4,194,304; ld >= vocab.
 *   cand_id, path_slot, q   the walk's candidates [batch, block, 16], chosen
 *                  slots [batch, block] and (sampled mode) its 16-way step
 *                  distributions q [batch, block, 16] (nullable when greedy).
 *   mode           DSEL_GREEDY: position t is accepted while its drafted token
 *                  is the arg max of target row t (ties to the lower id, NaN
 *                  lowest); the extra token is the arg max of the first rejected
 *                  row, or of row `block` when all are accepted.
 *                  DSEL_SAMPLED (temperature T > 0): p_t = softmax(z_t / T); t
 *                  accepts its token x iff u_acc[b,t] * q_t(x) < p_t(x); the
 *                  extra token is the inverse-CDF draw (token order, uniform
 *                  u_res[b]) from max(0, p_t - q_t) at the first rejection (q_t
 *                  is zero off the candidates), or from p_block if none.  Target
 *                  logits must then be finite or -inf, with a finite row max.
 *   n_accepted     out [batch] int32: accepted positions n (0..block).
 *   out_tok        out [batch, block + 1] int32: the n accepted tokens, the
 *                  extra token at index n, -1 after it.
 *   Ragged batches: block b has block_len[b] = n_b drafted positions and reads
 *   target rows 0 .. n_b (row n_b follows its last drafted token: the row
 *   `block` of the rules above); its whole out_tok row is written.  An empty
 *   block (n_b = 0) tests nothing and takes its extra token from row 0.
 *   workspace      device scratch of dsel_verify_workspace_bytes() bytes;
 *                  contents need no initialisation.
 * Requirements: 1 <= block <= DSEL_MAX_BLOCK. */
size_t dsel_verify_workspace_bytes(int64_t batch, int64_t block, int64_t vocab);
dsel_status dsel_verify(const void *target_logits, dsel_dtype dt, int64_t batch, int64_t block,
                        const int32_t *block_len, int64_t vocab, int64_t ld, const int32_t *cand_id,
                        const int32_t *path_slot, const float *q, dsel_walk_mode mode,
                        float temperature, const float *u_acc, const float *u_res,
                        int32_t *n_accepted, int32_t *out_tok, void *workspace,
                        size_t workspace_bytes, dsel_stream_t stream);

/* Synchronise `stream`, then read and clear the device error word of the
 * current device (bits DSEL_DEVERR_*; 0 = no error). */
dsel_status dsel_device_error(int32_t *out_code, dsel_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char *dsel_status_string(dsel_status s);

/* lmhead_topk -- [P1] Method > Lightweight Path Selector: the candidates are
 * the drafter's own 16 best logits, with no extra LM-head forward.  The LM
 * head z = h W^T and the top-16 of every row in one pass: the logits stay on
 * chip and never reach HBM.
 *   h        [rows, d] bf16: the drafter's final hidden states (rows =
 *            batch * block positions).
 *   W        [vocab, d] bf16: the LM-head weight (linear-layer layout; with
 *            tied embeddings, the embedding table E).
 *   cand_id  out [rows, 16] int32, cand_u out [rows, 16] fp32: the 16 best
 *            logits of each row, value descending, ties to the lower id (as
 *            dsel_select_topk on the logits); a zero logit comes out as +0.0.
 *   workspace  at least dsel_lmhead_topk_workspace_bytes() bytes (per-split
 *            partial lists); contents need no initialisation.
 * Arithmetic: bf16 MFMA with fp32 accumulation; the order is taken on those
 * fp32 logits.  Requirements: 16 <= vocab < 2^31, d % 64 == 0, rows >= 0, h
 * and W 16-byte aligned. */
size_t dsel_lmhead_topk_workspace_bytes(int64_t rows, int64_t vocab);
dsel_status dsel_lmhead_topk(const uint16_t *h, const uint16_t *W, int64_t rows, int64_t vocab, int64_t d,
                             int32_t *cand_id, float *cand_u, void *workspace, size_t workspace_bytes,
                             dsel_stream_t stream);

/* dyn_conv -- [P1] Method > Lightweight Local Convolution (eq. Conv_k), [P3]
 * section "The decay at the end of the block": the drafter's dynamic two-tap short convolution
 * over the positions of each drafted block,
 *     y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1},
 *     k_{t,j}[c] = base[j][c] + corr_t[j d/16 + c/16],  corr_t = W_c x_t,
 * one correction per 16 channels and tap, computed from the current position's
 * input; position 0 reads the last verified token (x_{-1} = x_prev[b]).
 *   x        [batch, block, d] bf16: the unit's input at every drafted position.
 *   x_prev   [batch, d] bf16: the last verified token's representation.
 *   base     [2, d] bf16: the learned base kernel, tap 0 (current position)
 *            then tap 1 (previous position).
 *   W_c      [2 d / 16, d] bf16, linear-layer layout: row j d/16 + g is the
 *            correction of tap j, channel group g (no bias).
 *   y        out [batch, block, d] bf16 (round to nearest even); must not
 *            overlap x.
 *   workspace  device scratch of at least dsel_dyn_conv_workspace_bytes()
 *            bytes; contents need no initialisation.
 * Arithmetic: corr by bf16 MFMA with fp32 accumulation, the taps in fp32.
 * Requirements: d % 512 == 0, 512 <= d <= 65536, block >= 1, batch >= 0, all
 * pointers 16-byte aligned. */
size_t dsel_dyn_conv_workspace_bytes(int64_t batch, int64_t block, int64_t d);
dsel_status dsel_dyn_conv(const uint16_t *x, const uint16_t *x_prev, const uint16_t *base,
                          const uint16_t *W_c, int64_t batch, int64_t block,
                          const int32_t *block_len, int64_t d, uint16_t *y, void *workspace,
                          size_t workspace_bytes, dsel_stream_t stream);

/* ABI version of this header (major * 100 + minor). */
int32_t dsel_version(void);
#define DSEL_VERSION 200

#ifdef __cplusplus
}
#endif
#endif /* DSEL_H */
