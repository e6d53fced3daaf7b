// The selector for small batches in three launches.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector:
// top-16 per position, the projections and the gate, every adjacent pair
// scored in one parallel pass, then the walk.)
//
// With a few blocks each step has far too little work to fill the chip, and
// a step's cost is mostly the latency of its launch and of its first loads.
// So the separate kernels' work is regrouped into three launches, with the
// same arithmetic in the same order (every output has the bits of the
// separate calls):
//   topk16_gate_gemm_kernel  the top-16 split into partial lists and, in the
//       same grid, the split-K gate GEMM (h W_H^T and E[verified] W_A^T
//       partials); the two do not depend on each other.
//   project_cand_kernel      (project.h, merge mode) each workgroup first merges
//       the partial top-16 lists of its tile's positions itself, then the
//       split-K candidate GEMM.
//   pair_walk_lat_kernel     one workgroup per position and group of the rank:
//       sums the candidate and gate partials in split order (what the reduce
//       kernels would write) and the group's pair table; the last group of a
//       position to finish takes the position's step decisions, and the last
//       position of each block to finish walks it.
// The last-to-finish hand-offs count arrivals per position and per block with
// atomic counters, which the first launch clears; no workgroup ever waits.
#pragma once

#include "pairwalk.h"
#include "project.h"
#include "topk16.h"

namespace dsel {

// Workgroups [0, topk_wgs) run the top-16 splits, the rest the gate GEMM's
// tiles; workgroup 0 also clears the arrival counters of the last launch.
template <bool BF16, int U, int BN>
__global__ __launch_bounds__(64 * kTopkWaves) void topk16_gate_gemm_kernel(TopkParams tp, GateParams gp,
                                                                           int64_t topk_wgs, int *count, int ncount) {
    static_assert(CandTile<BN>::NT == 64 * kTopkWaves, "one workgroup size for both jobs");
    const int64_t bid = blockIdx.x;
    if (bid == 0)
        for (int i = threadIdx.x; i < ncount; i += blockDim.x) count[i] = 0;
    if (bid < topk_wgs) topk16_block<BF16, U>(tp, bid);
    else gate_gemm_block<BN>(gp, (int)(bid - topk_wgs));
}

struct LatParams {
    PairParams pw;        // cand_u, nq, B, L, r, len, S (nullable), the walk
    // candidate GEMM: with c_nsplit > 1 its partials [c_nsplit][c_mt * 2 *
    // c_nside][128][c_BN]; else A_prev / B_cur as it writes them (pw)
    const float *cpart;
    int c_nsplit, c_mt, c_nside, c_BN;
    const float *gpart;   // gate GEMM partials [g_nsplit][B L + B][r]
    int g_nsplit;
    const int32_t *cand;  // merged candidates (an id outside [0, V) gives a zero row)
    int64_t V;
    // decisions of every position (walk_block's tables, per block of L
    // positions): chosen slot and its score per predecessor row, and the step
    // distributions when q is asked for
    uint8_t *ch;          // [B L][16]
    float *sc;            // [B L][16]
    float *Q;             // [B L][16][16] (nullable)
    float *P;             // [B L][nq][16][16] group tables
    int *pos_count;       // [B L] arrivals per position (groups)
    int *count;           // [B] arrivals per block (positions)
};

// Split sums of up to three float4 streams at once (src_i + k stride_i for
// k < n_i, each summed in split order): the loads of all three go out six
// splits at a time, so that one batch costs one memory latency.  A null
// stream sums to zero.
__device__ __forceinline__ void split_sum3(const float *s0, int64_t t0, int n0, const float *s1, int64_t t1, int n1,
                                           const float *s2, int64_t t2, int n2, floatx4 &o0, floatx4 &o1,
                                           floatx4 &o2) {
    constexpr int NB = 6;
    o0 = o1 = o2 = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if (!s0) n0 = 0;
    if (!s1) n1 = 0;
    if (!s2) n2 = 0;
    const int n = n0 > n1 ? (n0 > n2 ? n0 : n2) : (n1 > n2 ? n1 : n2);
    for (int k0 = 0; k0 < n; k0 += NB) {
        floatx4 v0[NB], v1[NB], v2[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (k0 + u < n0) v0[u] = *(const floatx4 *)(s0 + (k0 + u) * t0);
            if (k0 + u < n1) v1[u] = *(const floatx4 *)(s1 + (k0 + u) * t1);
            if (k0 + u < n2) v2[u] = *(const floatx4 *)(s2 + (k0 + u) * t2);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (k0 + u < n0) o0 += v0[u];
            if (k0 + u < n1) o1 += v1[u];
            if (k0 + u < n2) o2 += v2[u];
        }
    }
}

// First partial of candidate row m, side 0 (W_A) or 1 (W_B), 4 columns c..
__device__ __forceinline__ const float *lat_cand_src(const LatParams &p, int64_t m, int side, int c) {
    const int BN = p.c_BN, ncol = 2 * p.c_nside;
    const int64_t mt = m / 128, rl = m % 128;
    const int ct = side * p.c_nside + c / BN;
    return p.cpart + (mt * ncol + ct) * (128 * BN) + rl * BN + (c % BN);
}

// Workgroup (b t) nq + q: group q of the rank (columns q CW .. q CW + CW - 1)
// of position (b, t), CW / 16 waves.  Wave s sums slice s (columns q CW + 16 s
// ..) of the operands as pair_kernel loads them (lane (fr, fg): row fr, columns
// 16 s + 4 fg ..): A row fr of the position's predecessors (the candidates of
// t - 1; at t = 0 the verified token's row, then zeros), B row fr of its own
// candidates, and the gate (sigmoid of the summed logit).  Wave 0 runs
// pair_kernel's MFMA chain of the group and stores the table.  The last group
// of a position to arrive adds the tables in group order and U (S, as
// pair_kernel writes it) and takes the position's step decisions
// (walk_kernel's) into the block's decision tables in global memory; the
// last position of a block to arrive then walks it: the chain of look-ups
// from row 0 and the outputs.
template <int CW>
__global__ __launch_bounds__(CW / 16 * kWave) void pair_walk_lat_kernel(LatParams p) {
    constexpr int SPG = CW / 16;
    __shared__ floatx4 sa[SPG][kWave], sb[SPG][kWave], sg[SPG][kWave];
    __shared__ uint8_t lch[DSEL_MAX_BLOCK * kK];
    __shared__ int lrow[DSEL_MAX_BLOCK];
    __shared__ int last;
    const int L = p.pw.L, R = p.pw.r, nq = p.pw.nq;
    const int64_t bt = blockIdx.x / nq;
    const int q = (int)(blockIdx.x % nq);
    const int b = (int)(bt / L), t = (int)(bt % L);
    const int n = block_len_of(p.pw.len, b, L);
    if (t >= n) return;  // padding position: the walk waits for n positions
    const int wave = (int)(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const int fr = (int)(lane & 15), fg = (int)(lane >> 4);
    {
        const int c = q * CW + 16 * wave + 4 * fg;
        const int64_t grows = ((int64_t)p.pw.B * L + p.pw.B) * R;  // gate partial stride
        const int64_t cstride = (int64_t)p.c_mt * 2 * p.c_nside * 128 * p.c_BN;
        // A: the candidates of t - 1, or at t = 0 the verified token (row 0 only)
        const float *as = nullptr;
        int64_t at = 0;
        int an = 0;
        if (t > 0) {
            as = p.c_nsplit > 1 ? lat_cand_src(p, (bt - 1) * kK + fr, 0, c) : p.pw.A_prev + (bt * kK + fr) * R + c;
            at = cstride;
            an = p.c_nsplit;
        } else if (fr == 0) {
            as = p.gpart + ((int64_t)p.pw.B * L + b) * R + c;
            at = grows;
            an = p.g_nsplit;
        }
        const float *bs = p.c_nsplit > 1 ? lat_cand_src(p, bt * kK + fr, 1, c) : p.pw.B_cur + (bt * kK + fr) * R + c;
        // ids outside [0, V) give zero rows, as the reduce writes them (the
        // check goes out with the partial loads, not before them)
        const int32_t ta = t > 0 ? p.cand[(bt - 1) * kK + fr] : 0, tb = p.cand[bt * kK + fr];
        floatx4 a, bb, gs;
        split_sum3(as, at, an, bs, cstride, p.c_nsplit, p.gpart + bt * R + c, grows, p.g_nsplit, a, bb, gs);
        const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        if (p.c_nsplit > 1 && t > 0 && (ta < 0 || (int64_t)ta >= p.V)) a = zero;
        if (p.c_nsplit > 1 && (tb < 0 || (int64_t)tb >= p.V)) bb = zero;
        floatx4 g;
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = 1.0f / (1.0f + expf(-gs[e]));
        sa[wave][lane] = a;
        sb[wave][lane] = bb;
        sg[wave][lane] = g;
    }
    __syncthreads();
    const int64_t blk0 = (int64_t)b * L;  // the block's first position
    if (wave == 0) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SPG; ++s) {
            const floatx4 a = sa[s][lane], g = sg[s][lane], bb = sb[s][lane];
            const floatx4 ag = {a[0] * g[0], a[1] * g[1], a[2] * g[2], a[3] * g[3]};
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[0], bb[0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[1], bb[1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[2], bb[2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[3], bb[3], acc, 0, 0, 0);
        }
        float *Pq = p.P + (bt * nq + q) * (kK * kK) + fr;
#pragma unroll
        for (int v = 0; v < 4; ++v) Pq[(4 * fg + v) * kK] = acc[v];
        __threadfence();  // the table is visible device-wide before the arrival counts
        bool mine = false;
        if (lane == 0) mine = atomicAdd(&p.pos_count[bt], 1) == nq - 1;
        if (__builtin_amdgcn_readfirstlane((int)mine)) {
            __threadfence();  // the other groups' tables are visible to this wave's loads
            const float *P0 = p.P + bt * nq * (kK * kK) + 4 * fg * kK + fr;
            floatx4 sum;
#pragma unroll
            for (int v = 0; v < 4; ++v) sum[v] = P0[v * kK];
            for (int k = 1; k < nq; ++k) {
                floatx4 x;
#pragma unroll
                for (int v = 0; v < 4; ++v) x[v] = P0[k * (kK * kK) + v * kK];
                sum += x;
            }
            const float u = p.pw.cand_u[bt * kK + fr];
            float sc[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 4 * fg + v;
                sc[v] = (t == 0 && i >= 1) ? -__builtin_inff() : u + sum[v];
                if (p.pw.S) p.pw.S[(bt * kK + i) * kK + fr] = sc[v];
            }
            BlockShared dec;  // this block's decision tables (global memory)
            dec.Q = p.Q ? p.Q + blk0 * kK * kK : nullptr;
            dec.sc = p.sc + blk0 * kK;
            dec.ch = p.ch + blk0 * kK;
            dec.row = nullptr;
            const float uu = p.pw.w.mode == 1 ? p.pw.w.uniforms[bt] : 0.0f;
            decide_position(sc, t, p.pw.w, uu, p.Q != nullptr, dec);
            __threadfence();  // the decisions are visible device-wide before the arrival counts
            if (lane == 0) mine = atomicAdd(&p.count[b], 1) == n - 1;
            mine = __builtin_amdgcn_readfirstlane((int)mine);
        } else {
            mine = false;
        }
        if (lane == 0) last = mine;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();  // every decision of the block is visible to this workgroup's loads
    for (int e = threadIdx.x; e < n * kK; e += blockDim.x) lch[e] = p.ch[blk0 * kK + e];
    __syncthreads();
    if (threadIdx.x == 0) {
        int row = 0;  // the last verified token
        for (int tt = 0; tt < n; ++tt) {
            lrow[tt] = row;
            row = lch[tt * kK + row];
        }
    }
    __syncthreads();
    const WalkParams &w = p.pw.w;
    for (int e = threadIdx.x; e < n * kK; e += blockDim.x) {
        const int tt = e / kK, j = e % kK;
        const int64_t pos = blk0 + tt;
        const int row = lrow[tt];
        if (j == 0) {
            const int c = lch[tt * kK + row];
            w.path_slot[pos] = c;
            w.path_tok[pos] = w.cand_id[pos * kK + c];
            if (w.path_s) w.path_s[pos] = p.sc[pos * kK + row];
        }
        if (w.q) w.q[pos * kK + j] = p.Q[(pos * kK + row) * kK + j];
    }
}

}  // namespace dsel
