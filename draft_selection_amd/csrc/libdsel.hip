// libdsel.so: the C ABI declared in include/dsel.h.  Host-side validation,
// launch geometry and status codes; the kernels live in the headers below.
// The whole library is one translation unit (so the device error word needs no
// relocatable device code).
#include <hip/hip_runtime.h>

#include <limits.h>

#include <mutex>

#include "dsel.h"
#include "common.h"
#include "conv.h"
#include "fused.h"
#include "latency.h"
#include "lmhead.h"
#include "pairwalk.h"
#include "path.h"
#include "project.h"
#include "topk16.h"
#include "verify.h"

#define DSEL_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace dsel;

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline dsel_status launch(const void *kernel, dim3 grid, dim3 block, void *arg, size_t shmem,
                          dsel_stream_t stream) {
    void *args[] = {arg};
    hipError_t e = hipLaunchKernel(kernel, grid, block, args, shmem, (hipStream_t)stream);
    return e == hipSuccess ? DSEL_OK : DSEL_E_HIP;
}

#ifndef DSEL_VERIFY_WGS
#define DSEL_VERIFY_WGS 2048
#endif


dsel_status check_walk(const dsel_walk_args *w, WalkParams *out) {
    if (!w) return DSEL_E_ARG;
    if (w->mode != DSEL_GREEDY && w->mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    if (!w->cand_id || !w->path_tok || !w->path_slot) return DSEL_E_ARG;
    if (w->mode == DSEL_SAMPLED && (!w->uniforms || !(w->temperature > 0.0f))) return DSEL_E_ARG;
    if (!aligned(w->cand_id, 4) || !aligned(w->path_tok, 4) || !aligned(w->path_slot, 4) ||
        !aligned(w->path_s, 4) || !aligned(w->q, 4) || !aligned(w->uniforms, 4))
        return DSEL_E_ALIGN;
    out->mode = w->mode;
    out->temperature = w->mode == DSEL_SAMPLED ? w->temperature : 1.0f;
    out->uniforms = w->uniforms;
    out->cand_id = w->cand_id;
    out->path_tok = w->path_tok;
    out->path_slot = w->path_slot;
    out->path_s = w->path_s;
    out->q = w->q;
    return DSEL_OK;
}

}  // namespace

DSEL_API size_t dsel_topk_workspace_bytes(int64_t rows, int64_t vocab, dsel_dtype dt) {
    if (rows <= 0 || vocab < kK || vocab >= (int64_t)INT_MAX || (dt != DSEL_F32 && dt != DSEL_BF16))
        return 0;
    int ns = topk_nsplit(rows, vocab);
    return ns > 1 ? (size_t)rows * (size_t)ns * kK * sizeof(uint64_t) : 0;
}

namespace {

// Validation and launch geometry of each step, shared by its own entry point
// and by dsel_select_path.  A plan with `empty` set has nothing to launch.
struct TopkPlan {
    TopkParams p;
    bool bf16 = false, empty = false;
};

dsel_status plan_topk(const void *logits, dsel_dtype dt, int64_t batch, int64_t block, const int32_t *block_len,
                      int64_t vocab, int64_t ld, int32_t *cand_id, float *cand_u, void *workspace,
                      size_t workspace_bytes, TopkPlan *t) {
    if (dt != DSEL_F32 && dt != DSEL_BF16) return DSEL_E_DTYPE;
    if (batch < 0 || block < 0 || vocab < kK || vocab >= (int64_t)INT_MAX || ld < vocab) return DSEL_E_ARG;
    const int64_t rows = batch * block;
    if (block != 0 && rows / block != batch) return DSEL_E_ARG;
    t->empty = rows == 0;
    if (t->empty) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!logits || !cand_id || !cand_u) return DSEL_E_ARG;
    const size_t es = dt == DSEL_BF16 ? 2 : 4;
    if (!aligned(logits, es) || !aligned(cand_id, 4) || !aligned(cand_u, 4) || !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    if (ld > INT64_MAX / (int64_t)es / rows) return DSEL_E_ARG;
    const int ns = topk_nsplit(rows, vocab);
    if ((int64_t)ns * rows >= (int64_t)INT_MAX) return DSEL_E_ARG;
    const size_t need = dsel_topk_workspace_bytes(rows, vocab, dt);
    if (need && (!workspace || workspace_bytes < need)) return DSEL_E_WORKSPACE;
    if (need && !aligned(workspace, 8)) return DSEL_E_ALIGN;
    TopkParams &p = t->p;
    p.logits = (const char *)logits;
    p.rows = rows;
    p.V = vocab;
    p.ld = ld;
    p.nsplit = ns;
    p.L = (int)block;
    p.len = block_len;
    p.cand_id = cand_id;
    p.cand_u = cand_u;
    p.partial = (uint64_t *)workspace;
    t->bf16 = dt == DSEL_BF16;
    return DSEL_OK;
}

// The top-16 launch; with `gate` (a split gate job) its reduction rides along
// as extra workgroups (path.h).
dsel_status launch_topk(const TopkPlan &t, const GateParams *gate, int64_t gate_units, dsel_stream_t stream) {
    TopkParams p = t.p;
    const int64_t wgs = p.rows * p.nsplit;
    dsel_status s;
    if (gate) {
        GateParams gp = *gate;
        int64_t tw = wgs;
        constexpr int TT = 64 * kTopkWaves;
        const int64_t grid = wgs + (gate_units + TT - 1) / TT;
        if (grid >= (int64_t)INT_MAX) return DSEL_E_ARG;
        const void *k = t.bf16 ? (const void *)topk16_gate_kernel<true, kTopkUnroll<true>>
                               : (const void *)topk16_gate_kernel<false, kTopkUnroll<false>>;
        void *args[] = {&p, &gp, &tw};
        s = hipLaunchKernel(k, dim3((unsigned)grid), dim3(64 * kTopkWaves), args, 0, (hipStream_t)stream) == hipSuccess
                ? DSEL_OK : DSEL_E_HIP;
    } else {
        const void *k = t.bf16 ? (const void *)topk16_kernel<true, kTopkUnroll<true>>
                               : (const void *)topk16_kernel<false, kTopkUnroll<false>>;
        s = launch(k, dim3((unsigned)wgs), dim3(64 * kTopkWaves), &p, 0, stream);
    }
    if (s != DSEL_OK || p.nsplit == 1) return s;
    const void *k2 = t.bf16 ? (const void *)topk16_merge_kernel<true> : (const void *)topk16_merge_kernel<false>;
    return launch(k2, dim3((unsigned)p.rows), dim3(256), &p, 0, stream);
}

}  // namespace

DSEL_API dsel_status dsel_select_topk(const void *logits, dsel_dtype dt, int64_t batch,
                                      int64_t block, const int32_t *block_len, int64_t vocab, int64_t ld,
                                      int32_t *cand_id, float *cand_u, void *workspace, size_t workspace_bytes,
                                      dsel_stream_t stream) {
    TopkPlan t;
    dsel_status st = plan_topk(logits, dt, batch, block, block_len, vocab, ld, cand_id, cand_u, workspace,
                               workspace_bytes, &t);
    if (st != DSEL_OK || t.empty) return st;
    return launch_topk(t, nullptr, 0, stream);
}

namespace {

dsel_status check_project_common(const uint16_t *E, int64_t vocab, int64_t d, int64_t r,
                                 int64_t batch, int64_t block) {
    if (vocab < 1 || vocab >= (int64_t)INT_MAX || d < 64 || d % 64 != 0 || d > (1 << 20)) return DSEL_E_ARG;
    if (r < 32 || r > DSEL_MAX_RANK || r % 32 != 0) return DSEL_E_ARG;
    if (batch < 0 || block < 1 || batch > (1 << 24) || block > (1 << 16)) return DSEL_E_ARG;
    if (batch > 0 && !E) return DSEL_E_ARG;
    if (!aligned(E, 16)) return DSEL_E_ALIGN;
    return DSEL_OK;
}

// Workspace layout shared by dsel_project, dsel_project_gate and
// dsel_project_cand: the gate's partial tiles first, then (256-byte aligned)
// the candidate job's, so the two halves never touch each other's part.
size_t cand_workspace_offset(int64_t batch, int64_t block, int64_t d, int64_t r) {
    return (gate_workspace_bytes(batch, block, d, r) + 255) / 256 * 256;
}

}  // namespace

DSEL_API size_t dsel_project_workspace_bytes(int64_t batch, int64_t block, int64_t d, int64_t r) {
    if (batch <= 0 || block < 1 || d < 64 || d % 64 != 0 || r < 32 || r > DSEL_MAX_RANK || r % 32 != 0)
        return 0;
    const size_t c = cand_workspace_bytes(batch, block, d, r);
    return c ? cand_workspace_offset(batch, block, d, r) + c : gate_workspace_bytes(batch, block, d, r);
}

namespace {

struct GatePlan {
    GateParams p;
    int BN = 0;
    bool empty = false;
};

// The gate job; `split` = false runs one workgroup per output tile with no
// K split and no workspace.
dsel_status plan_gate(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A, const uint16_t *W_H,
                      int64_t r, const uint16_t *h, const int32_t *verified, int64_t batch, int64_t block,
                      const int32_t *block_len, float *A_prev, float *G, void *workspace, size_t workspace_bytes,
                      bool split, GatePlan *g) {
    dsel_status st = check_project_common(E, vocab, d, r, batch, block);
    g->empty = batch == 0;
    if (st != DSEL_OK || g->empty) return st;
    if (!W_A || !W_H || !h || !verified || !A_prev || !G) return DSEL_E_ARG;
    if (!aligned(W_A, 16) || !aligned(W_H, 16) || !aligned(h, 16) || !aligned(verified, 4) ||
        !aligned(A_prev, 16) || !aligned(G, 16) || !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    const size_t need = split ? gate_workspace_bytes(batch, block, d, r) : 0;
    if (need && (!workspace || workspace_bytes < need)) return DSEL_E_WORKSPACE;
    if (need && !aligned(workspace, 16)) return DSEL_E_ALIGN;
    GateParams &p = g->p;
    p.E = E;
    p.V = vocab;
    p.d = (int)d;
    p.r = (int)r;
    p.WA = W_A;
    p.WH = W_H;
    p.h = h;
    p.ver = verified;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    p.A_prev = A_prev;
    p.G = G;
    p.A_ver = A_prev;
    p.ver_stride = block * kK * r;
    p.ver_zero = true;
    p.part = (float *)workspace;
    g->BN = gate_bn(batch, block, r);
    p.nside = (int)(r / g->BN);
    p.mt_gate = (int)((batch * block + 127) / 128);
    p.mt_ver = (int)((batch + 127) / 128);
    p.nsplit = split ? gate_nsplit(batch, block, d, r) : 1;
    const int64_t grid = (int64_t)(p.mt_gate + p.mt_ver) * p.nside * p.nsplit;
    if (grid >= (int64_t)INT_MAX) return DSEL_E_ARG;
    return DSEL_OK;
}

// Output elements of the gate's reduction (0 when it is not split).
// Work units (four output elements each) of the gate reduction; 0 when unsplit.
int64_t gate_reduce_units(const GatePlan &g) {
    return g.p.nsplit > 1 ? ((int64_t)g.p.B * g.p.L + g.p.B) * g.p.r / 4 : 0;
}

dsel_status launch_gate_gemm(const GatePlan &g, dsel_stream_t stream) {
    GateParams p = g.p;
    const int64_t grid = (int64_t)(p.mt_gate + p.mt_ver) * p.nside * p.nsplit;
    const void *k = g.BN == 256 ? (const void *)project_gate_kernel<256>
                  : g.BN == 128 ? (const void *)project_gate_kernel<128>
                  : g.BN == 64  ? (const void *)project_gate_kernel<64>
                                : (const void *)project_gate_kernel<32>;
    return launch(k, dim3((unsigned)grid), dim3(tile_threads(g.BN)), &p, 0, stream);
}

dsel_status launch_gate_reduce(const GatePlan &g, dsel_stream_t stream) {
    GateParams p = g.p;
    const int64_t elems = gate_reduce_units(g);
    if (elems == 0) return DSEL_OK;
    return launch((const void *)project_gate_reduce_kernel, dim3((unsigned)((elems + 255) / 256)), dim3(256), &p,
                  0, stream);
}

// The gate's split-K reduction and the top-16 (the reduction is needed only
// after the top-16).  Where the top-16 is one round of workgroups (at most
// DSEL_FOLD_MAX_TOPK_WG: four rows per CU), the reduction rides in its
// launch as extra workgroups, beside it; beyond, those workgroups would land
// on the last round, so the reduction is a launch of its own before it
// (MI355X: 1,024 bf16 rows, folded 120.8 / 160.8 us per step against
// 124.6 / 164.1 at the two shapes of 1,024 rows; 4,096 fp32 rows, 912.1 us
// separate against 921.0 folded).
#ifndef DSEL_FOLD_MAX_TOPK_WG
#define DSEL_FOLD_MAX_TOPK_WG 1024
#endif
dsel_status launch_topk_and_gate_reduce(const TopkPlan &t, const GatePlan &g, dsel_stream_t stream) {
    const int64_t ge = gate_reduce_units(g);
    if (ge == 0 || t.p.rows * t.p.nsplit <= DSEL_FOLD_MAX_TOPK_WG)
        return launch_topk(t, ge ? &g.p : nullptr, ge, stream);
    dsel_status st = launch_gate_reduce(g, stream);
    return st == DSEL_OK ? launch_topk(t, nullptr, 0, stream) : st;
}

dsel_status project_gate_impl(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                              const uint16_t *W_H, int64_t r, const uint16_t *h, const int32_t *verified,
                              int64_t batch, int64_t block, const int32_t *block_len, float *A_prev, float *G,
                              void *workspace, size_t workspace_bytes, bool split, dsel_stream_t stream) {
    GatePlan g;
    dsel_status st = plan_gate(E, vocab, d, W_A, W_H, r, h, verified, batch, block, block_len, A_prev, G, workspace,
                               workspace_bytes, split, &g);
    if (st != DSEL_OK || g.empty) return st;
    st = launch_gate_gemm(g, stream);
    if (st != DSEL_OK) return st;
    return launch_gate_reduce(g, stream);
}

}  // namespace

DSEL_API dsel_status dsel_project_gate(const uint16_t *E, int64_t vocab, int64_t d,
                                       const uint16_t *W_A, const uint16_t *W_H, int64_t r,
                                       const uint16_t *h, const int32_t *verified, int64_t batch,
                                       int64_t block, const int32_t *block_len, float *A_prev, float *G,
                                       void *workspace, size_t workspace_bytes, dsel_stream_t stream) {
    return project_gate_impl(E, vocab, d, W_A, W_H, r, h, verified, batch, block, block_len, A_prev, G,
                             workspace, workspace_bytes, true, stream);
}

DSEL_API dsel_status dsel_project_gate_overlap(const uint16_t *E, int64_t vocab, int64_t d,
                                               const uint16_t *W_A, const uint16_t *W_H, int64_t r,
                                               const uint16_t *h, const int32_t *verified, int64_t batch,
                                               int64_t block, const int32_t *block_len, float *A_prev,
                                               float *G, dsel_stream_t stream) {
    return project_gate_impl(E, vocab, d, W_A, W_H, r, h, verified, batch, block, block_len, A_prev, G, nullptr,
                             0, false, stream);
}

namespace {

struct CandPlan {
    CandParams p;
    int BN = 0;
    bool empty = false;
};

dsel_status plan_cand(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A, const uint16_t *W_B,
                      int64_t r, const int32_t *cand_id, int64_t batch, int64_t block, const int32_t *block_len,
                      float *A_prev, float *B_cur, void *workspace, size_t workspace_bytes, CandPlan *c) {
    dsel_status st = check_project_common(E, vocab, d, r, batch, block);
    c->empty = batch == 0;
    if (st != DSEL_OK || c->empty) return st;
    if (!W_A || !W_B || !cand_id || !A_prev || !B_cur) return DSEL_E_ARG;
    if (!aligned(W_A, 16) || !aligned(W_B, 16) || !aligned(cand_id, 4) || !aligned(A_prev, 16) ||
        !aligned(B_cur, 16) || !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    const size_t cneed = cand_workspace_bytes(batch, block, d, r);
    const size_t coff = cand_workspace_offset(batch, block, d, r);
    if (cneed && (!workspace || workspace_bytes < coff + cneed)) return DSEL_E_WORKSPACE;
    if (cneed && !aligned(workspace, 16)) return DSEL_E_ALIGN;
    CandParams &p = c->p;
    p.E = E;
    p.V = vocab;
    p.d = (int)d;
    p.r = (int)r;
    p.WA = W_A;
    p.WB = W_B;
    p.cand = cand_id;
    p.L = (int)block;
    p.len = block_len;
    p.M = batch * block * kK;
    p.A_prev = A_prev;
    p.B_cur = B_cur;
    p.tk_part = nullptr;
    p.tk_nsplit = 0;
    p.cand_id = nullptr;
    p.cand_u = nullptr;
    p.logits = nullptr;
    p.ld = p.V_logits = 0;
    p.logits_bf16 = false;
    constexpr int BM = 128;
    c->BN = cand_bn(batch, block, r);
    p.nside = (int)(r / c->BN);
    p.mt = (int)((p.M + BM - 1) / BM);
    p.mt_pad = (p.mt + 7) / 8 * 8;
    p.nsplit = cand_nsplit(batch, block, d, r);
    p.part = cneed ? (float *)((char *)workspace + coff) : nullptr;
    const int64_t grid = (int64_t)p.mt_pad * 2 * p.nside * p.nsplit;
    if (grid >= (int64_t)INT_MAX || p.M * 2 * r >= (int64_t)INT_MAX * 256) return DSEL_E_ARG;
    return DSEL_OK;
}

dsel_status launch_cand_gemm(const CandPlan &c, dsel_stream_t stream) {
    CandParams p = c.p;
    const int BN = c.BN;
    const int64_t grid = (int64_t)p.mt_pad * 2 * p.nside * p.nsplit;
    const void *k = BN == 256 ? (const void *)project_cand_kernel<256>
                  : BN == 128 ? (const void *)project_cand_kernel<128>
                  : BN == 64  ? (const void *)project_cand_kernel<64>
                              : (const void *)project_cand_kernel<32>;
    return launch(k, dim3((unsigned)grid), dim3(tile_threads(BN)), &p, 0, stream);
}

dsel_status launch_cand(const CandPlan &c, dsel_stream_t stream) {
    CandParams p = c.p;
    const int BN = c.BN;
    dsel_status st = launch_cand_gemm(c, stream);
    if (st != DSEL_OK || p.nsplit == 1) return st;
    const int64_t elems = p.M * 2 * p.r;
    const void *kr = BN == 256 ? (const void *)project_cand_reduce_kernel<256>
                   : BN == 128 ? (const void *)project_cand_reduce_kernel<128>
                   : BN == 64  ? (const void *)project_cand_reduce_kernel<64>
                               : (const void *)project_cand_reduce_kernel<32>;
    return launch(kr, dim3((unsigned)((elems + 255) / 256)), dim3(256), &p, 0, stream);
}

}  // namespace

DSEL_API dsel_status dsel_project_cand(const uint16_t *E, int64_t vocab, int64_t d,
                                       const uint16_t *W_A, const uint16_t *W_B, int64_t r,
                                       const int32_t *cand_id, int64_t batch, int64_t block,
                                       const int32_t *block_len, float *A_prev, float *B_cur,
                                       void *workspace, size_t workspace_bytes, dsel_stream_t stream) {
    CandPlan c;
    dsel_status st = plan_cand(E, vocab, d, W_A, W_B, r, cand_id, batch, block, block_len, A_prev, B_cur,
                               workspace, workspace_bytes, &c);
    if (st != DSEL_OK || c.empty) return st;
    return launch_cand(c, stream);
}

DSEL_API dsel_status dsel_project(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                                  const uint16_t *W_B, const uint16_t *W_H, int64_t r,
                                  const uint16_t *h, const int32_t *cand_id,
                                  const int32_t *verified, int64_t batch, int64_t block,
                                  const int32_t *block_len, float *A_prev, float *B_cur, float *G,
                                  void *workspace, size_t workspace_bytes, dsel_stream_t stream) {
    dsel_status st = check_project_common(E, vocab, d, r, batch, block);
    if (st != DSEL_OK || batch == 0) return st;
    if (!W_A || !W_B || !W_H || !h || !cand_id || !verified || !A_prev || !B_cur || !G)
        return DSEL_E_ARG;
    const size_t need = dsel_project_workspace_bytes(batch, block, d, r);
    if (need && (!workspace || workspace_bytes < need)) return DSEL_E_WORKSPACE;
    st = dsel_project_gate(E, vocab, d, W_A, W_H, r, h, verified, batch, block, block_len, A_prev, G,
                           workspace, workspace_bytes, stream);
    if (st != DSEL_OK) return st;
    return dsel_project_cand(E, vocab, d, W_A, W_B, r, cand_id, batch, block, block_len, A_prev, B_cur,
                             workspace, workspace_bytes, stream);
}

namespace {

const void *pair_kernel_for(int64_t r) {
    switch (r) {
        case 32: return (const void *)pair_kernel<32>;
        case 64: return (const void *)pair_kernel<64>;
        case 96: return (const void *)pair_kernel<96>;
        case 128: return (const void *)pair_kernel<128>;
        case 160: return (const void *)pair_kernel<160>;
        case 192: return (const void *)pair_kernel<192>;
        case 224: return (const void *)pair_kernel<224>;
        case 256: return (const void *)pair_kernel<256>;
    }
    return nullptr;
}

dsel_status launch_walk(PairParams &p, dsel_stream_t stream) {
    const int waves = p.L < 16 ? p.L : 16;
    const size_t shmem = pair_walk_shmem(p.L, p.w.q != nullptr);
    return launch((const void *)walk_kernel, dim3((unsigned)p.B), dim3(waves * kWave), &p, shmem, stream);
}

}  // namespace

namespace {

struct PairPlan {
    PairParams p = {};
    bool walk = false, empty = false;
};

dsel_status plan_pairs(const float *cand_u, const float *A_prev, const float *B_cur, const float *G, int64_t batch,
                       int64_t block, const int32_t *block_len, int64_t r, float *S, const dsel_walk_args *walk,
                       PairPlan *q) {
    if (batch < 0 || batch >= (int64_t)INT_MAX / DSEL_MAX_BLOCK || block < 1 || block > DSEL_MAX_BLOCK)
        return DSEL_E_ARG;
    if (r < 32 || r > DSEL_MAX_RANK || r % 32 != 0) return DSEL_E_ARG;
    if (walk && walk->mode != DSEL_GREEDY && walk->mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    q->empty = batch == 0;
    if (q->empty) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!cand_u || !A_prev || !B_cur || !G || !S) return DSEL_E_ARG;
    if (!aligned(A_prev, 16) || !aligned(B_cur, 16) || !aligned(G, 16) || !aligned(cand_u, 4) ||
        !aligned(S, 4) || !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    PairParams &p = q->p;
    if (walk) {
        dsel_status s = check_walk(walk, &p.w);
        if (s != DSEL_OK) return s;
    }
    q->walk = walk != nullptr;
    p.cand_u = cand_u;
    p.A_prev = A_prev;
    p.B_cur = B_cur;
    p.G = G;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    p.r = (int)r;
    p.S = S;
    p.S_in = S;
    return DSEL_OK;
}

dsel_status launch_pairs(const PairPlan &q, dsel_stream_t stream) {
    PairParams p = q.p;
    const int64_t positions = (int64_t)p.B * p.L;
    dsel_status st = launch(pair_kernel_for(p.r), dim3((unsigned)positions), dim3(256), &p, 0, stream);
    if (st != DSEL_OK || !q.walk) return st;
    return launch_walk(p, stream);
}

}  // namespace

DSEL_API dsel_status dsel_score_pairs(const float *cand_u, const float *A_prev, const float *B_cur,
                                      const float *G, int64_t batch, int64_t block,
                                      const int32_t *block_len, int64_t r, float *S,
                                      const dsel_walk_args *walk, dsel_stream_t stream) {
    PairPlan q;
    dsel_status st = plan_pairs(cand_u, A_prev, B_cur, G, batch, block, block_len, r, S, walk, &q);
    if (st != DSEL_OK || q.empty) return st;
    return launch_pairs(q, stream);
}

DSEL_API dsel_status dsel_walk(const float *S, int64_t batch, int64_t block, const int32_t *block_len,
                               const dsel_walk_args *walk, dsel_stream_t stream) {
    if (!walk) return DSEL_E_ARG;
    if (batch < 0 || batch >= (int64_t)INT_MAX || block < 1 || block > DSEL_MAX_BLOCK) return DSEL_E_ARG;
    if (walk->mode != DSEL_GREEDY && walk->mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    if (batch == 0) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!S) return DSEL_E_ARG;
    if (!aligned(S, 4) || !aligned(block_len, 4)) return DSEL_E_ALIGN;
    PairParams p = {};
    dsel_status s = check_walk(walk, &p.w);
    if (s != DSEL_OK) return s;
    p.S_in = S;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    return launch_walk(p, stream);
}

// ---- measurement aid: the candidate gather alone -----------------------------

DSEL_API dsel_status dsel_gather_probe(const uint16_t *E, int64_t vocab, int64_t d, const int32_t *cand_id,
                                       int64_t batch, int64_t block, uint32_t *out, size_t out_words,
                                       dsel_stream_t stream) {
    dsel_status st = check_project_common(E, vocab, d, 32, batch, block);
    if (st != DSEL_OK || batch == 0) return st;
    if (!cand_id || !out) return DSEL_E_ARG;
    if (!aligned(cand_id, 4) || !aligned(out, 4)) return DSEL_E_ALIGN;
    GatherProbeParams p;
    p.E = E;
    p.V = vocab;
    p.d = (int)d;
    p.cand = cand_id;
    p.M = batch * block * kK;
    const int64_t mt = (p.M + 127) / 128;
    p.nsplit = gather_probe_nsplit(p.M, d);
    const int64_t grid = mt * p.nsplit;
    if (grid >= (int64_t)INT_MAX / 256 || out_words < (size_t)grid * 256) return DSEL_E_ARG;
    p.mt = (int)mt;
    p.out = out;
    return launch((const void *)gather_probe_kernel, dim3((unsigned)grid), dim3(256), &p, 0, stream);
}

DSEL_API size_t dsel_gather_probe_words(int64_t batch, int64_t block, int64_t d) {
    if (batch <= 0 || block < 1 || d < 64 || d % 64 != 0) return 0;
    const int64_t M = batch * block * kK;
    return (size_t)((M + 127) / 128) * (size_t)gather_probe_nsplit(M, d) * 256;
}

// ---- the whole selector ----------------------------------------------------

namespace {

inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of dsel_select_path, in this order (each part 256-byte aligned):
// the top-16's partial lists; the projections' split-K partials; G; then, on
// the fused route, A(verified) [B][r] and the pair partials, else A_prev,
// B_cur [B, L, 16, r] and S [B, L, 16, 16].  The parts for outputs the caller
// supplies are reserved but unused.
struct PathLayout {
    size_t topk = 0, proj = 0, g = 0, aver = 0, part = 0, a = 0, b = 0, s = 0, lat = 0, cnt = 0, total = 0;
    bool fused = false;
};

bool path_layout(int64_t batch, int64_t block, int64_t vocab, dsel_dtype dt, int64_t d, int64_t r,
                 PathLayout *l) {
    if (batch <= 0 || block < 1 || block > DSEL_MAX_BLOCK || batch > (int64_t)INT_MAX / block) return false;
    if (d < 64 || d % 64 != 0 || r < 32 || r > DSEL_MAX_RANK || r % 32 != 0) return false;
    const int64_t pos = batch * block;
    size_t off = align256(dsel_topk_workspace_bytes(pos, vocab, dt));
    l->topk = 0;
    l->proj = off;
    off += align256(dsel_project_workspace_bytes(batch, block, d, r));
    l->g = off;
    off += align256((size_t)pos * r * sizeof(float));
    l->fused = use_fused(batch, block, r);
    if (l->fused) {
        l->aver = off;
        off += align256((size_t)batch * r * sizeof(float));
        l->part = off;
        off += align256(fused_partial_bytes(batch, block, r));
    } else {
        const size_t ab = align256((size_t)pos * kK * r * sizeof(float));
        l->a = off;
        off += ab;
        l->b = off;
        off += ab;
        l->s = off;
        off += align256((size_t)pos * kK * kK * sizeof(float));
        // the small-batch route's decision tables (slot, score, distribution
        // per predecessor row), group tables and arrival counters (per
        // position, then per block)
        l->lat = off;
        off += align256((size_t)pos * kK) + align256((size_t)pos * kK * sizeof(float)) +
               align256((size_t)pos * kK * kK * sizeof(float)) +
               align256((size_t)pos * (r / pair_cw((int)r)) * kK * kK * sizeof(float));
        l->cnt = off;
        off += align256((size_t)(pos + batch) * sizeof(int));
    }
    l->total = off;
    return true;
}

struct FusedPlan {
    FusedParams p;
    int CW = 64;
    int NG = 1;  // rank groups per workgroup
};

dsel_status plan_fused(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A, const uint16_t *W_B,
                       int64_t r, const int32_t *cand_id, const float *G, const float *A_ver, int64_t ver_stride,
                       int64_t batch, int64_t block, const int32_t *block_len, float *P, float *A_prev,
                       float *B_cur, FusedPlan *f) {
    dsel_status st = check_project_common(E, vocab, d, r, batch, block);
    if (st != DSEL_OK) return st;
    if (fused_blocks_per_tile(block) == 0 || batch > (int64_t)INT_MAX / 16) return DSEL_E_ARG;
    if (!W_A || !W_B || !cand_id || !G || !A_ver || !P || ver_stride < r) return DSEL_E_ARG;
    if ((A_prev == nullptr) != (B_cur == nullptr)) return DSEL_E_ARG;
    if (!aligned(W_A, 16) || !aligned(W_B, 16) || !aligned(cand_id, 4) || !aligned(G, 16) || !aligned(A_ver, 16) ||
        ver_stride % 4 != 0 || !aligned(P, 16) || !aligned(A_prev, 16) || !aligned(B_cur, 16) ||
        !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    FusedParams &p = f->p;
    p.E = E;
    p.V = vocab;
    p.d = (int)d;
    p.r = (int)r;
    p.WA = W_A;
    p.WB = W_B;
    p.cand = cand_id;
    p.G = G;
    p.A_ver = A_ver;
    p.ver_stride = ver_stride;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    p.nb = fused_blocks_per_tile(block);
    p.ntile = (int)fused_grid_tiles(batch, block, block_len != nullptr);
    f->CW = pair_group_width((int)r);
    f->NG = fused_groups(batch, block, r, block_len != nullptr);
    p.nq = (int)(r / f->CW);
    p.P = P;
    p.A_prev = A_prev;
    p.B_cur = B_cur;
    if (fused_grid(batch, block, r, block_len != nullptr) >= (int64_t)INT_MAX) return DSEL_E_ARG;
    return DSEL_OK;
}

dsel_status launch_fused(const FusedPlan &f, dsel_stream_t stream) {
    FusedParams p = f.p;
    const int64_t grid = fused_grid(p.B, p.L, p.r, p.len != nullptr);
    const void *k = f.CW == 32 ? (const void *)project_pair_kernel<32, 1>
                    : f.NG == 2 ? (const void *)project_pair_kernel<64, 2>
                                : (const void *)project_pair_kernel<64, 1>;
    const int nt = f.CW == 32 ? FusedTile<32, 1>::NT : f.NG == 2 ? FusedTile<64, 2>::NT : FusedTile<64, 1>::NT;
    return launch(k, dim3((unsigned)grid), dim3(nt), &p, 0, stream);
}

}  // namespace

DSEL_API size_t dsel_select_path_workspace_bytes(int64_t batch, int64_t block, int64_t vocab, dsel_dtype dt,
                                                 int64_t d, int64_t r) {
    PathLayout l;
    return path_layout(batch, block, vocab, dt, d, r, &l) ? l.total : 0;
}

DSEL_API int64_t dsel_pair_groups(int64_t r) {
    if (r < 32 || r > DSEL_MAX_RANK || r % 32 != 0) return 0;
    return r / pair_group_width((int)r);
}

DSEL_API dsel_status dsel_project_pairs(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                                        const uint16_t *W_B, int64_t r, const int32_t *cand_id, const float *G,
                                        const float *A_ver, int64_t ver_stride, int64_t batch, int64_t block,
                                        const int32_t *block_len, float *partials, float *A_prev, float *B_cur,
                                        dsel_stream_t stream) {
    if (batch == 0 && block >= 1 && block <= 16) {
        dsel_status st = check_project_common(E, vocab, d, r, batch, block);
        return st;  // nothing to do; pointers may be NULL
    }
    FusedPlan f;
    dsel_status st = plan_fused(E, vocab, d, W_A, W_B, r, cand_id, G, A_ver, ver_stride, batch, block, block_len,
                                partials, A_prev, B_cur, &f);
    if (st != DSEL_OK) return st;
    return launch_fused(f, stream);
}

DSEL_API dsel_status dsel_walk_pairs(const float *cand_u, const float *partials, int64_t batch, int64_t block,
                                     const int32_t *block_len, int64_t nq, float *S, const dsel_walk_args *walk,
                                     dsel_stream_t stream) {
    if (!walk) return DSEL_E_ARG;
    if (batch < 0 || batch >= (int64_t)INT_MAX / DSEL_MAX_BLOCK || block < 1 || block > DSEL_MAX_BLOCK) return DSEL_E_ARG;
    if (nq < 1 || nq > DSEL_MAX_RANK / 32) return DSEL_E_ARG;
    if (walk->mode != DSEL_GREEDY && walk->mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    if (batch == 0) return DSEL_OK;
    if (!cand_u || !partials) return DSEL_E_ARG;
    if (!aligned(cand_u, 4) || !aligned(partials, 16) || !aligned(S, 4) || !aligned(block_len, 4)) return DSEL_E_ALIGN;
    PairParams p = {};
    dsel_status st = check_walk(walk, &p.w);
    if (st != DSEL_OK) return st;
    p.cand_u = cand_u;
    p.P = partials;
    p.nq = (int)nq;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    p.S = S;
    return launch_walk(p, stream);
}

// ---- the small-batch route (latency.h) ----------------------------------------

// Top-16 workgroups beside the gate GEMM's in the first launch: the gate's LDS
// ring leaves room for two workgroups per CU, 512 in all.
#ifndef DSEL_LAT_TOPK_WG
#define DSEL_LAT_TOPK_WG 448
#endif
// Partial lists per top-16 row at most (measured at one block of 16, bf16 rows
// of 151,936: 8, 16 and 24 lists within 1 us of each other, 24 ahead; 4
// lists 8 us slower).
#ifndef DSEL_LAT_TOPK_LISTS
#define DSEL_LAT_TOPK_LISTS 24
#endif
// Partial lists per row that the candidate GEMM's merge can stage in its LDS
// ring (8 positions per tile, 16 keys of 8 bytes per list).
constexpr int kLatMaxLists = (int)(3 * 128 * kBK * sizeof(uint16_t) / (8 * kK * sizeof(uint64_t)));

struct LatPlan {
    TopkPlan t;
    GatePlan g;
    CandPlan c;
    LatParams k;
    int64_t topk_wgs = 0, gate_wgs = 0;
    bool use = false;
};

// The small-batch route serves a call of at most DSEL_LAT_MAX_ROWS positions
// that is not on the fused route and asks for no intermediates (A_prev,
// B_cur, G), when the gate GEMM is split with column tiles of at most 64 (its
// LDS ring then leaves room for the top-16 beside it); otherwise lp->use stays
// false.
// Workspace: the top-16 lists, the gate and candidate partials (or, from an
// unsplit candidate GEMM, A_prev and B_cur) where the separate route keeps
// them; the decision tables and the arrival counters in regions of their own.
// Positions up to which the small-batch route runs.  Beyond, the separate
// kernels are faster: the top-16 rows split fewer ways in the shared launch,
// and the last-arrival hand-offs grow with the positions (MI355X, blocks of 16
// at d 2560: 1 and 2 blocks 48.5 / 53.2 us against 52.6 / 54.1 separate; 4 and
// 8 blocks 65.4 / 87.7 us against 59.8 / 64.7).
#ifndef DSEL_LAT_MAX_ROWS
#define DSEL_LAT_MAX_ROWS 32
#endif

bool latency_route(int64_t batch, int64_t block, int64_t d, int64_t r, bool fused, bool intermediates) {
    return !fused && !intermediates && batch * block <= DSEL_LAT_MAX_ROWS && gate_bn(batch, block, r) <= 64 &&
           gate_nsplit(batch, block, d, r) > 1;
}

dsel_status plan_latency(const dsel_path_args *a, const dsel_walk_args *walk, char *ws, const PathLayout &l,
                         LatPlan *lp) {
    lp->use = false;
    if (!latency_route(a->batch, a->block, a->d, a->r, l.fused, a->A_prev || a->G)) return DSEL_OK;
    const int64_t rows = a->batch * a->block;
    float *A_buf = (float *)(ws + l.a), *B_buf = (float *)(ws + l.b);  // written by an unsplit candidate GEMM
    dsel_status st = plan_topk(a->logits, a->dt, a->batch, a->block, a->block_len, a->vocab, a->ld, a->cand_id,
                               a->cand_u, ws, l.proj, &lp->t);
    if (st != DSEL_OK) return st;
    st = plan_gate(a->E, a->vocab, a->d, a->W_A, a->W_H, a->r, a->h, a->verified, a->batch, a->block,
                   a->block_len, A_buf, A_buf, ws + l.proj, l.g - l.proj, true, &lp->g);
    if (st != DSEL_OK) return st;
    st = plan_cand(a->E, a->vocab, a->d, a->W_A, a->W_B, a->r, a->cand_id, a->batch, a->block, a->block_len,
                   A_buf, B_buf, ws + l.proj, l.g - l.proj, &lp->c);
    if (st != DSEL_OK) return st;
    if (lp->g.BN > 64 || lp->g.p.nsplit < 2) return DSEL_OK;
    if (!a->cand_u || !aligned(a->S, 4)) return !a->cand_u ? DSEL_E_ARG : DSEL_E_ALIGN;
    const GateParams &gp = lp->g.p;
    lp->gate_wgs = (int64_t)(gp.mt_gate + gp.mt_ver) * gp.nside * gp.nsplit;
    TopkParams &tp = lp->t.p;
    if (tp.nsplit > 1) {
        int64_t ns = (DSEL_LAT_TOPK_WG - lp->gate_wgs) / rows;
        if (ns > tp.nsplit) ns = tp.nsplit;
        if (ns > DSEL_LAT_TOPK_LISTS) ns = DSEL_LAT_TOPK_LISTS;
        if (ns > kLatMaxLists) ns = kLatMaxLists;
        tp.nsplit = (int)(ns < 1 ? 1 : ns);
    }
    lp->topk_wgs = rows * tp.nsplit;
    CandParams &cp = lp->c.p;
    if (tp.nsplit > 1) {  // the candidate GEMM merges the lists itself
        cp.tk_part = tp.partial;
        cp.tk_nsplit = tp.nsplit;
        cp.cand_id = a->cand_id;
        cp.cand_u = a->cand_u;
        cp.logits = (const char *)a->logits;
        cp.ld = a->ld;
        cp.V_logits = a->vocab;
        cp.logits_bf16 = a->dt == DSEL_BF16;
    }
    LatParams &k = lp->k;
    k = LatParams{};
    st = check_walk(walk, &k.pw.w);
    if (st != DSEL_OK) return st;
    k.pw.cand_u = a->cand_u;
    k.pw.B = (int)a->batch;
    k.pw.L = (int)a->block;
    k.pw.r = (int)a->r;
    k.pw.len = a->block_len;
    k.pw.S = a->S;
    k.pw.A_prev = A_buf;
    k.pw.B_cur = B_buf;
    k.ch = (uint8_t *)(ws + l.lat);
    k.sc = (float *)(ws + l.lat + align256((size_t)rows * kK));
    const size_t qoff = l.lat + align256((size_t)rows * kK) + align256((size_t)rows * kK * sizeof(float));
    k.Q = walk->q ? (float *)(ws + qoff) : nullptr;
    k.P = (float *)(ws + qoff + align256((size_t)rows * kK * kK * sizeof(float)));
    k.pw.nq = (int)(a->r / pair_cw((int)a->r));
    k.cpart = cp.part;
    k.c_nsplit = cp.nsplit;
    k.c_mt = cp.mt;
    k.c_nside = cp.nside;
    k.c_BN = lp->c.BN;
    k.gpart = gp.part;
    k.g_nsplit = gp.nsplit;
    k.cand = a->cand_id;
    k.V = a->vocab;
    k.pos_count = (int *)(ws + l.cnt);
    k.count = k.pos_count + rows;
    if (lp->topk_wgs + lp->gate_wgs >= (int64_t)INT_MAX) return DSEL_OK;
    lp->use = true;
    return DSEL_OK;
}

dsel_status launch_latency(LatPlan &lp, dsel_stream_t stream) {
    TopkParams tp = lp.t.p;
    GateParams gp = lp.g.p;
    int64_t tw = lp.topk_wgs;
    int *count = lp.k.pos_count;  // then the block counters
    int ncount = lp.k.pw.B * lp.k.pw.L + lp.k.pw.B;
    const int BN = lp.g.BN;
    const void *k1 = lp.t.bf16 ? (BN == 64 ? (const void *)topk16_gate_gemm_kernel<true, kTopkUnroll<true>, 64>
                                           : (const void *)topk16_gate_gemm_kernel<true, kTopkUnroll<true>, 32>)
                               : (BN == 64 ? (const void *)topk16_gate_gemm_kernel<false, kTopkUnroll<false>, 64>
                                           : (const void *)topk16_gate_gemm_kernel<false, kTopkUnroll<false>, 32>);
    void *args[] = {&tp, &gp, &tw, &count, &ncount};
    if (hipLaunchKernel(k1, dim3((unsigned)(lp.topk_wgs + lp.gate_wgs)), dim3(64 * kTopkWaves), args, 0,
                        (hipStream_t)stream) != hipSuccess)
        return DSEL_E_HIP;
    dsel_status st = launch_cand_gemm(lp.c, stream);
    if (st != DSEL_OK) return st;
    LatParams k = lp.k;
    const int CW = pair_cw(k.pw.r);
    const void *k3 = CW == 64 ? (const void *)pair_walk_lat_kernel<64> : (const void *)pair_walk_lat_kernel<32>;
    return launch(k3, dim3((unsigned)((int64_t)k.pw.B * k.pw.L * k.pw.nq)), dim3(CW / 16 * kWave), &k, 0, stream);
}

DSEL_API int dsel_select_path_route(const dsel_path_args *a) {
    if (!a) return -1;
    PathLayout l;
    if (a->batch <= 0 || !path_layout(a->batch, a->block, a->vocab, a->dt, a->d, a->r, &l)) return -1;
    if (l.fused) return DSEL_ROUTE_FUSED;
    return latency_route(a->batch, a->block, a->d, a->r, false, a->A_prev || a->G) ? DSEL_ROUTE_SMALL
                                                                                      : DSEL_ROUTE_SEPARATE;
}

DSEL_API dsel_status dsel_select_path(const dsel_path_args *a, const dsel_walk_args *walk, void *workspace,
                                      size_t workspace_bytes, dsel_stream_t stream) {
    if (!a || !walk) return DSEL_E_ARG;
    if (a->batch < 0 || a->block < 1 || a->block > DSEL_MAX_BLOCK || a->batch > (int64_t)INT_MAX / a->block)
        return DSEL_E_ARG;
    if ((a->A_prev == nullptr) != (a->B_cur == nullptr)) return DSEL_E_ARG;  // both or neither
    PathLayout l;
    if (a->batch > 0) {
        if (!path_layout(a->batch, a->block, a->vocab, a->dt, a->d, a->r, &l)) return DSEL_E_ARG;
        if (!workspace || workspace_bytes < l.total) return DSEL_E_WORKSPACE;
        if (!aligned(workspace, 256)) return DSEL_E_ALIGN;
    }
    char *ws = (char *)workspace;
    float *G = a->G ? a->G : (float *)(ws + l.g);
    // every step is validated before anything is launched
    TopkPlan t;
    GatePlan g;
    dsel_status st = plan_topk(a->logits, a->dt, a->batch, a->block, a->block_len, a->vocab, a->ld, a->cand_id,
                               a->cand_u, ws, l.proj, &t);
    if (st != DSEL_OK || a->batch == 0) return st;
    if (l.fused) {
        // gate GEMM; top-16 with the gate's reduction beside it; the fused
        // candidate projection + pair partials; the walk, which also forms S
        const bool ab = a->A_prev != nullptr;
        float *A_ver = ab ? a->A_prev : (float *)(ws + l.aver);
        st = plan_gate(a->E, a->vocab, a->d, a->W_A, a->W_H, a->r, a->h, a->verified, a->batch, a->block,
                       a->block_len, ab ? a->A_prev : A_ver, G, ws + l.proj, l.g - l.proj, true, &g);
        if (st != DSEL_OK) return st;
        if (!ab) {  // A(verified) to the compact buffer
            g.p.A_ver = A_ver;
            g.p.ver_stride = a->r;
            g.p.ver_zero = false;
        }
        FusedPlan f;
        st = plan_fused(a->E, a->vocab, a->d, a->W_A, a->W_B, a->r, a->cand_id, G, A_ver,
                        ab ? a->block * kK * a->r : a->r, a->batch, a->block, a->block_len, (float *)(ws + l.part),
                        a->A_prev, a->B_cur, &f);
        if (st != DSEL_OK) return st;
        PairPlan q;
        if (!a->cand_u || !aligned(a->S, 4)) return !a->cand_u ? DSEL_E_ARG : DSEL_E_ALIGN;
        st = check_walk(walk, &q.p.w);
        if (st != DSEL_OK) return st;
        q.p.cand_u = a->cand_u;
        q.p.P = f.p.P;
        q.p.nq = f.p.nq;
        q.p.B = (int)a->batch;
        q.p.L = (int)a->block;
        q.p.len = a->block_len;
        q.p.r = (int)a->r;
        q.p.S = a->S;
        st = launch_gate_gemm(g, stream);
        if (st == DSEL_OK) st = launch_topk_and_gate_reduce(t, g, stream);
        if (st == DSEL_OK) st = launch_fused(f, stream);
        if (st == DSEL_OK) st = launch_walk(q.p, stream);
        return st;
    }
    {
        LatPlan lp;
        st = plan_latency(a, walk, ws, l, &lp);
        if (st != DSEL_OK) return st;
        if (lp.use) return launch_latency(lp, stream);
    }
    // the separate kernels: gate GEMM; top-16 with the gate's reduction beside
    // it; candidate GEMM; pair scores and the walk (intermediates the caller
    // does not want live in the workspace)
    float *A_prev = a->A_prev ? a->A_prev : (float *)(ws + l.a);
    float *B_cur = a->B_cur ? a->B_cur : (float *)(ws + l.b);
    float *S = a->S ? a->S : (float *)(ws + l.s);
    CandPlan c;
    PairPlan q;
    st = plan_gate(a->E, a->vocab, a->d, a->W_A, a->W_H, a->r, a->h, a->verified, a->batch, a->block,
                   a->block_len, A_prev, G, ws + l.proj, l.g - l.proj, true, &g);
    if (st == DSEL_OK)
        st = plan_cand(a->E, a->vocab, a->d, a->W_A, a->W_B, a->r, a->cand_id, a->batch, a->block, a->block_len,
                       A_prev, B_cur, ws + l.proj, l.g - l.proj, &c);
    if (st == DSEL_OK)
        st = plan_pairs(a->cand_u, A_prev, B_cur, G, a->batch, a->block, a->block_len, a->r, S, walk, &q);
    if (st != DSEL_OK) return st;
    st = launch_gate_gemm(g, stream);
    if (st == DSEL_OK) st = launch_topk_and_gate_reduce(t, g, stream);
    if (st == DSEL_OK) st = launch_cand(c, stream);
    if (st == DSEL_OK) st = launch_pairs(q, stream);
    return st;
}

// ---- the whole selector without a caller workspace ---------------------------

namespace {

// The workspace of dsel_select_path_noalloc: one array per device, which the
// HIP runtime places when the library's code is loaded on that device and
// keeps until the process ends.  Host code never passes `scratch` itself to a
// kernel (its name is a host-side stand-in, not the device address); it uses
// the address hipGetSymbolAddress returns, looked up once per device.
constexpr size_t kScratchBytes = (size_t)DSEL_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

dsel_status scratch_for_current_device(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSEL_E_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return DSEL_E_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DSEL_OK;
}

}  // namespace

DSEL_API dsel_status dsel_select_path_noalloc(const dsel_path_args *a, const dsel_walk_args *walk,
                                              dsel_stream_t stream) {
    if (!a || !walk) return DSEL_E_ARG;
    if (a->batch < 0 || a->block < 1 || a->block > DSEL_MAX_BLOCK || a->batch > (int64_t)INT_MAX / a->block)
        return DSEL_E_ARG;
    size_t need = 0;
    if (a->batch > 0) {
        PathLayout l;
        if (!path_layout(a->batch, a->block, a->vocab, a->dt, a->d, a->r, &l)) return DSEL_E_ARG;
        need = l.total;
        if (need > kScratchBytes) return DSEL_E_WORKSPACE;  // beyond the fixed scratch array
    }
    void *ws = nullptr;
    if (need) {
        dsel_status st = scratch_for_current_device(&ws);
        if (st != DSEL_OK) return st;
    }
    return dsel_select_path(a, walk, ws, need ? kScratchBytes : 0, stream);
}

DSEL_API dsel_status dsel_device_error(int32_t *out_code, dsel_stream_t stream) {
    if (!out_code) return DSEL_E_ARG;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return DSEL_E_HIP;
    int v = 0, zero = 0;
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(dsel::g_device_error), sizeof(int), 0,
                            hipMemcpyDeviceToHost) != hipSuccess)
        return DSEL_E_HIP;
    if (hipMemcpyToSymbol(HIP_SYMBOL(dsel::g_device_error), &zero, sizeof(int), 0,
                          hipMemcpyHostToDevice) != hipSuccess)
        return DSEL_E_HIP;
    *out_code = v;
    return DSEL_OK;
}

DSEL_API const char *dsel_status_string(dsel_status s) {
    switch (s) {
        case DSEL_OK: return "DSEL_OK";
        case DSEL_E_ARG: return "DSEL_E_ARG: invalid argument";
        case DSEL_E_DTYPE: return "DSEL_E_DTYPE: unknown dtype or walk mode";
        case DSEL_E_ALIGN: return "DSEL_E_ALIGN: misaligned pointer or leading dimension";
        case DSEL_E_WORKSPACE: return "DSEL_E_WORKSPACE: workspace missing or too small";
        case DSEL_E_HIP: return "DSEL_E_HIP: HIP runtime or launch failure";
    }
    return "unknown dsel status";
}

DSEL_API int32_t dsel_version(void) { return DSEL_VERSION; }

// ---- LM head with the top-16 ------------------------------------------------

DSEL_API size_t dsel_lmhead_topk_workspace_bytes(int64_t rows, int64_t vocab) {
    if (rows <= 0 || vocab < kK || vocab >= (int64_t)INT_MAX) return 0;
    return lmhead_workspace_bytes(rows, vocab);
}

DSEL_API dsel_status dsel_lmhead_topk(const uint16_t *h, const uint16_t *W, int64_t rows, int64_t vocab,
                                      int64_t d, int32_t *cand_id, float *cand_u, void *workspace,
                                      size_t workspace_bytes, dsel_stream_t stream) {
    if (rows < 0 || rows > (1 << 24) || vocab < kK || vocab >= (int64_t)INT_MAX || d < 64 || d % 64 != 0 ||
        d > (1 << 20))
        return DSEL_E_ARG;
    if (rows == 0) return DSEL_OK;
    if (!h || !W || !cand_id || !cand_u) return DSEL_E_ARG;
    if (!aligned(h, 16) || !aligned(W, 16) || !aligned(cand_id, 4) || !aligned(cand_u, 4)) return DSEL_E_ALIGN;
    const size_t need = lmhead_workspace_bytes(rows, vocab);
    if (!workspace || workspace_bytes < need) return DSEL_E_WORKSPACE;
    if (!aligned(workspace, 16)) return DSEL_E_ALIGN;
    LmheadParams p;
    p.h = h;
    p.W = W;
    p.R = rows;
    p.V = vocab;
    p.d = (int)d;
    p.mt = (int)((rows + 127) / 128);
    p.nct = (int)((vocab + kLmBN - 1) / kLmBN);
    p.nvs = lmhead_nvs(rows, vocab);
    p.cpw = (p.nct + p.nvs - 1) / p.nvs;
    p.partial = (uint64_t *)workspace;
    const int64_t grid = (int64_t)p.mt * p.nvs;
    if (grid >= (int64_t)INT_MAX) return DSEL_E_ARG;
    dsel_status st = launch((const void *)lmhead_topk_kernel, dim3((unsigned)grid), dim3(LmTile::NT), &p, 0, stream);
    if (st != DSEL_OK) return st;
    TopkParams tp;
    tp.logits = nullptr;
    tp.rows = rows;
    tp.V = vocab;
    tp.ld = vocab;
    tp.nsplit = p.nvs;
    tp.L = 1;
    tp.len = nullptr;
    tp.cand_id = cand_id;
    tp.cand_u = cand_u;
    tp.partial = p.partial;
    return launch((const void *)topk16_merge_kernel<true>, dim3((unsigned)rows), dim3(256), &tp, 0, stream);
}

// ---- dynamic short convolution ---------------------------------------------

DSEL_API size_t dsel_dyn_conv_workspace_bytes(int64_t batch, int64_t block, int64_t d) {
    if (batch <= 0 || block < 1 || d < 512 || d % 512 != 0 || d > (1 << 16)) return 0;
    return conv_workspace_bytes(batch, block, d);
}

DSEL_API dsel_status dsel_dyn_conv(const uint16_t *x, const uint16_t *x_prev, const uint16_t *base,
                                   const uint16_t *W_c, int64_t batch, int64_t block,
                                   const int32_t *block_len, int64_t d, uint16_t *y, void *workspace,
                                   size_t workspace_bytes, dsel_stream_t stream) {
    if (batch < 0 || block < 1 || d < 512 || d % 512 != 0 || d > (1 << 16)) return DSEL_E_ARG;
    if (batch > (int64_t)INT_MAX / block) return DSEL_E_ARG;
    if (batch == 0) return DSEL_OK;
    if (!x || !x_prev || !base || !W_c || !y) return DSEL_E_ARG;
    if (!aligned(x, 16) || !aligned(x_prev, 16) || !aligned(base, 16) || !aligned(W_c, 16) || !aligned(y, 16) ||
        !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    const size_t need = conv_workspace_bytes(batch, block, d);
    if (!workspace || workspace_bytes < need) return DSEL_E_WORKSPACE;
    if (!aligned(workspace, 16)) return DSEL_E_ALIGN;
    ConvParams p;
    p.x = x;
    p.x_prev = x_prev;
    p.base = base;
    p.W_c = W_c;
    p.y = y;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    p.d = (int)d;
    p.M = batch * block;
    p.N = (int)(d / 8);
    p.mt = (int)((p.M + 127) / 128);
    const int BN = conv_bn(p.M, p.N);
    p.nt = p.N / BN;
    p.nsplit = conv_nsplit(batch, block, d);
    p.part = (float *)workspace;
    const int64_t grid = (int64_t)p.mt * p.nt * p.nsplit;
    if (grid >= (int64_t)INT_MAX) return DSEL_E_ARG;
    const void *kc = BN == 256 ? (const void *)conv_corr_kernel<256> : (const void *)conv_corr_kernel<64>;
    dsel_status st = launch(kc, dim3((unsigned)grid), dim3(tile_threads(BN)), &p, 0, stream);
    if (st != DSEL_OK) return st;
    return launch((const void *)conv_apply_kernel, dim3((unsigned)p.M), dim3(256), &p,
                  (size_t)p.N * sizeof(float), stream);
}

// ---- verify ----------------------------------------------------------------

DSEL_API size_t dsel_verify_workspace_bytes(int64_t batch, int64_t block, int64_t vocab) {
    if (batch <= 0 || block < 1 || block > DSEL_MAX_BLOCK || vocab < kK ||
        vocab > kVMaxVocab)
        return 0;
    return verify_workspace_bytes(batch, block, vocab);
}

DSEL_API dsel_status dsel_verify(const void *target_logits, dsel_dtype dt, int64_t batch,
                                 int64_t block, const int32_t *block_len, int64_t vocab, int64_t ld,
                                 const int32_t *cand_id,
                                 const int32_t *path_slot, const float *q, dsel_walk_mode mode,
                                 float temperature, const float *u_acc, const float *u_res,
                                 int32_t *n_accepted, int32_t *out_tok, void *workspace,
                                 size_t workspace_bytes, dsel_stream_t stream) {
    if (dt != DSEL_F32 && dt != DSEL_BF16) return DSEL_E_DTYPE;
    if (mode != DSEL_GREEDY && mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    if (batch < 0 || batch >= (int64_t)INT_MAX / (DSEL_MAX_BLOCK + 1) || block < 1 || block > DSEL_MAX_BLOCK)
        return DSEL_E_ARG;
    if (vocab < kK || vocab > kVMaxVocab || ld < vocab) return DSEL_E_ARG;
    if (mode == DSEL_SAMPLED && !(temperature > 0.0f && temperature < __builtin_inff())) return DSEL_E_ARG;
    if (batch == 0) return DSEL_OK;
    if (!target_logits || !cand_id || !path_slot || !n_accepted || !out_tok) return DSEL_E_ARG;
    if (mode == DSEL_SAMPLED && (!q || !u_acc || !u_res)) return DSEL_E_ARG;
    const int64_t es = dt == DSEL_BF16 ? 2 : 4;
    const int64_t rows = batch * (block + 1);
    if (ld > INT64_MAX / es / rows) return DSEL_E_ARG;
    if (!aligned(target_logits, 16) || (ld * es) % 16 != 0) return DSEL_E_ALIGN;
    if (!aligned(cand_id, 4) || !aligned(path_slot, 4) || !aligned(n_accepted, 4) || !aligned(out_tok, 4) ||
        (q && !aligned(q, 4)) || (u_acc && !aligned(u_acc, 4)) || (u_res && !aligned(u_res, 4)) ||
        !aligned(block_len, 4))
        return DSEL_E_ALIGN;
    const size_t need = verify_workspace_bytes(batch, block, vocab);
    if (!workspace || workspace_bytes < need) return DSEL_E_WORKSPACE;
    if (!aligned(workspace, 16)) return DSEL_E_ALIGN;

    VerifyParams p;
    p.logits = (const char *)target_logits;
    p.V = vocab;
    p.ld = ld;
    p.B = (int)batch;
    p.L = (int)block;
    p.len = block_len;
    p.scale = mode == DSEL_SAMPLED ? (float)(1.4426950408889634 / (double)temperature) : 0.0f;
    p.cand_id = cand_id;
    p.path_slot = path_slot;
    p.q = q;
    p.u_acc = u_acc;
    p.u_res = u_res;
    p.n_acc = n_accepted;
    p.out_tok = out_tok;
    const bool bf = dt == DSEL_BF16, sm = mode == DSEL_SAMPLED;
    // chunks of 256 16-byte vectors; enough workgroups per row for about 2048
    // in all (8 per CU), at most kVMaxSplit, none of them empty
    const int64_t chunk_tokens = (int64_t)kVChunkVecs * (bf ? 8 : 4);
    p.nchunk = (int)((vocab + chunk_tokens - 1) / chunk_tokens);
    int64_t ns = (DSEL_VERIFY_WGS + rows - 1) / rows;
    ns = ns < 1 ? 1 : ns > kVMaxSplit ? kVMaxSplit : ns;
    ns = ns < p.nchunk ? ns : p.nchunk;
    p.cps = (int)((p.nchunk + ns - 1) / ns);
    p.nsplit = (p.nchunk + p.cps - 1) / p.cps;
    if (rows * p.nsplit > (int64_t)INT_MAX) return DSEL_E_ARG;
    p.part = (VerifyPart *)workspace;
    p.chunk = (float2 *)((char *)workspace + verify_part_bytes(batch, block));
    const void *k1 = bf ? (sm ? (const void *)verify_stats_kernel<true, true> : (const void *)verify_stats_kernel<true, false>)
                        : (sm ? (const void *)verify_stats_kernel<false, true> : (const void *)verify_stats_kernel<false, false>);
    const void *k2 = bf ? (sm ? (const void *)verify_draw_kernel<true, true> : (const void *)verify_draw_kernel<true, false>)
                        : (sm ? (const void *)verify_draw_kernel<false, true> : (const void *)verify_draw_kernel<false, false>);
    dsel_status st = launch(k1, dim3((unsigned)(rows * p.nsplit)), dim3(256), &p, 0, stream);
    if (st != DSEL_OK) return st;
    return launch(k2, dim3((unsigned)batch), dim3(256), &p, 0, stream);
}
