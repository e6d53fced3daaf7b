// libdsel.so: the C ABI declared in include/dsel.h.  Host-side validation,
// launch geometry and status codes; the kernels live in the headers below.
// The whole library is one translation unit (so the device error word needs no
// relocatable device code).
#include <hip/hip_runtime.h>

#include <limits.h>

#include "dsel.h"
#include "common.h"
#include "pairwalk.h"
#include "project.h"
#include "topk16.h"

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

constexpr int kTopkUnroll = 4;

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

DSEL_API dsel_status dsel_select_topk(const void *logits, dsel_dtype dt, int64_t batch,
                                      int64_t block, int64_t vocab, int64_t ld, int32_t *cand_id,
                                      float *cand_u, void *workspace, size_t workspace_bytes,
                                      dsel_stream_t stream) {
    if (dt != DSEL_F32 && dt != DSEL_BF16) return DSEL_E_DTYPE;
    if (batch < 0 || block < 0 || vocab < kK || vocab >= (int64_t)INT_MAX || ld < vocab) return DSEL_E_ARG;
    const int64_t rows = batch * block;
    if (block != 0 && rows / block != batch) return DSEL_E_ARG;
    if (rows == 0) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!logits || !cand_id || !cand_u) return DSEL_E_ARG;
    const size_t es = dt == DSEL_BF16 ? 2 : 4;
    if (!aligned(logits, es) || !aligned(cand_id, 4) || !aligned(cand_u, 4)) return DSEL_E_ALIGN;
    if (ld > INT64_MAX / (int64_t)es / rows) return DSEL_E_ARG;
    const int ns = topk_nsplit(rows, vocab);
    if ((int64_t)ns * rows >= (int64_t)INT_MAX) return DSEL_E_ARG;
    const size_t need = dsel_topk_workspace_bytes(rows, vocab, dt);
    if (need && (!workspace || workspace_bytes < need)) return DSEL_E_WORKSPACE;
    if (need && !aligned(workspace, 8)) return DSEL_E_ALIGN;

    TopkParams p;
    p.logits = (const char *)logits;
    p.rows = rows;
    p.V = vocab;
    p.ld = ld;
    p.nsplit = ns;
    p.cand_id = cand_id;
    p.cand_u = cand_u;
    p.partial = (uint64_t *)workspace;
    const void *k1 = dt == DSEL_BF16 ? (const void *)topk16_kernel<true, kTopkUnroll>
                                     : (const void *)topk16_kernel<false, kTopkUnroll>;
    dsel_status s = launch(k1, dim3((unsigned)(rows * ns)), dim3(256), &p, 0, stream);
    if (s != DSEL_OK || ns == 1) return s;
    const void *k2 = dt == DSEL_BF16 ? (const void *)topk16_merge_kernel<true>
                                     : (const void *)topk16_merge_kernel<false>;
    return launch(k2, dim3((unsigned)rows), dim3(64), &p, 0, stream);
}

DSEL_API dsel_status dsel_project(const uint16_t *E, int64_t vocab, int64_t d, const uint16_t *W_A,
                                  const uint16_t *W_B, const uint16_t *W_H, int64_t r,
                                  const uint16_t *h, const int32_t *cand_id,
                                  const int32_t *verified, int64_t batch, int64_t block,
                                  float *A_prev, float *B_cur, float *G, dsel_stream_t stream) {
    if (vocab < 1 || vocab >= (int64_t)INT_MAX || d < 64 || d % 64 != 0 || d > (1 << 20)) return DSEL_E_ARG;
    if (r < 32 || r > DSEL_MAX_RANK || r % 32 != 0) return DSEL_E_ARG;
    if (batch < 0 || block < 1 || batch > (1 << 24) || block > (1 << 16)) return DSEL_E_ARG;
    if (batch == 0) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!E || !W_A || !W_B || !W_H || !h || !cand_id || !verified || !A_prev || !B_cur || !G)
        return DSEL_E_ARG;
    if (!aligned(E, 16) || !aligned(W_A, 16) || !aligned(W_B, 16) || !aligned(W_H, 16) ||
        !aligned(h, 16) || !aligned(cand_id, 4) || !aligned(verified, 4) || !aligned(A_prev, 4) ||
        !aligned(B_cur, 4) || !aligned(G, 4))
        return DSEL_E_ALIGN;

    const bool big = (r % 128) == 0;
    const int BM = big ? 128 : 64, BN = big ? 128 : 32;
    ProjParams p;
    p.E = E;
    p.V = vocab;
    p.d = (int)d;
    p.r = (int)r;
    p.WA = W_A;
    p.WB = W_B;
    p.WH = W_H;
    p.h = h;
    p.cand = cand_id;
    p.ver = verified;
    p.B = (int)batch;
    p.L = (int)block;
    p.A_prev = A_prev;
    p.B_cur = B_cur;
    p.G = G;
    p.m_cand = batch * block * kK;
    p.m_ver = batch;
    p.m_gate = batch * block;
    p.nt_cand = (int)(2 * r / BN);
    p.nt_ver = p.nt_gate = (int)(r / BN);
    p.mt_cand = (int)((p.m_cand + BM - 1) / BM);
    p.mt_cand_pad = (p.mt_cand + 7) / 8 * 8;
    p.mt_ver = (int)((p.m_ver + BM - 1) / BM);
    p.mt_gate = (int)((p.m_gate + BM - 1) / BM);
    p.wg_cand = (int64_t)p.mt_cand_pad * p.nt_cand;
    p.wg_ver = (int64_t)p.mt_ver * p.nt_ver;
    const int64_t grid = p.wg_cand + p.wg_ver + (int64_t)p.mt_gate * p.nt_gate;
    if (grid >= (int64_t)INT_MAX) return DSEL_E_ARG;
    const void *k = big ? (const void *)project_kernel<128, 128> : (const void *)project_kernel<64, 32>;
    return launch(k, dim3((unsigned)grid), dim3(256), &p, 0, stream);
}

DSEL_API dsel_status dsel_score_pairs(const float *cand_u, const float *A_prev, const float *B_cur,
                                      const float *G, int64_t batch, int64_t block, int64_t r,
                                      float *S, const dsel_walk_args *walk, dsel_stream_t stream) {
    if (batch < 0 || batch >= (int64_t)INT_MAX || block < 1 || block > DSEL_MAX_BLOCK) return DSEL_E_ARG;
    if (r < 32 || r > DSEL_MAX_RANK || r % 32 != 0) return DSEL_E_ARG;
    if (walk && walk->mode != DSEL_GREEDY && walk->mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    if (batch == 0) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!cand_u || !A_prev || !B_cur || !G) return DSEL_E_ARG;
    if (!S && !walk) return DSEL_E_ARG;
    if (!aligned(A_prev, 16) || !aligned(B_cur, 16) || !aligned(G, 16) || !aligned(cand_u, 4) ||
        !aligned(S, 4))
        return DSEL_E_ALIGN;
    PairParams p;
    p.do_walk = walk != nullptr;
    if (walk) {
        dsel_status s = check_walk(walk, &p.w);
        if (s != DSEL_OK) return s;
    } else {
        p.w = WalkParams{};
    }
    p.cand_u = cand_u;
    p.A_prev = A_prev;
    p.B_cur = B_cur;
    p.G = G;
    p.B = (int)batch;
    p.L = (int)block;
    p.r = (int)r;
    p.S = S;
    const int waves = block < 16 ? (int)block : 16;
    const size_t shmem = (size_t)block * kK * kK * sizeof(float);
    return launch((const void *)pair_walk_kernel, dim3((unsigned)batch), dim3(waves * kWave), &p,
                  shmem, stream);
}

DSEL_API dsel_status dsel_walk(const float *S, int64_t batch, int64_t block,
                               const dsel_walk_args *walk, dsel_stream_t stream) {
    if (!walk) return DSEL_E_ARG;
    if (batch < 0 || batch >= (int64_t)INT_MAX / 4 || block < 1 || block > DSEL_MAX_BLOCK) return DSEL_E_ARG;
    if (walk->mode != DSEL_GREEDY && walk->mode != DSEL_SAMPLED) return DSEL_E_DTYPE;
    if (batch == 0) return DSEL_OK;  // nothing to read or write; pointers may be NULL
    if (!S) return DSEL_E_ARG;
    if (!aligned(S, 4)) return DSEL_E_ALIGN;
    WalkParams w;
    dsel_status s = check_walk(walk, &w);
    if (s != DSEL_OK) return s;
    struct {
        const float *S;
        int B, L;
        WalkParams w;
    } a = {S, (int)batch, (int)block, w};
    void *args[] = {&a.S, &a.B, &a.L, &a.w};
    hipError_t e = hipLaunchKernel((const void *)walk_kernel, dim3((unsigned)((batch + 3) / 4)),
                                   dim3(256), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? DSEL_OK : DSEL_E_HIP;
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
