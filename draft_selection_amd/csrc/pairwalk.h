// score_pairs + walk.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector:
// eq. S_t scores every adjacent candidate pair in one parallel pass; the only
// sequential step walks the precomputed scores from the last verified token,
// greedily or by sampling.  "DFlash 2: The Drafter Stopped Guessing Alone",
// "Selection beats correction", says the same.)
//
// Two kernels:
//  pair_kernel: one workgroup per position (b, t), its 4 waves sharing the
//     rank so that enough loads are in flight over the whole chip.  The 16 x 16
//     table P[i][j] = sum_c A_prev[i][c] G[c] B_cur[j][c] is an fp32 MFMA
//     accumulation (v_mfma_f32_16x16x4_f32, r/4 steps over the 4 waves, summed
//     through LDS).  S = U + P (row i >= 1 of position 0 is -inf) is written.
//  walk_kernel: one workgroup per draft block, wave w loading the score tables
//     of positions t = w, w + nw, ... (16 KB per block), then:
//  1. Decisions, in parallel for every predecessor row of every position: the
//     greedy successor (highest score, ties to the lowest slot, NaN lowest), or
//     the sampled one (inverse CDF of softmax(S_row / T) with the position's
//     uniform).  In the MFMA output layout a row's 16 scores sit in one 16-lane
//     DPP row, so every reduction and scan is four DPP steps.
//  2. The walk itself is then a chain of L table look-ups from row 0 (the
//     verified token), after which all lanes write the outputs.
#pragma once

#include "common.h"

namespace dsel {

struct WalkParams {
    int mode;  // 0 greedy, 1 sampled
    float temperature;
    const float *uniforms;
    const int32_t *cand_id;
    int32_t *path_tok, *path_slot;
    float *path_s, *q;
};

struct PairParams {
    const float *cand_u, *A_prev, *B_cur, *G;
    const float *S_in;  // stand-alone walk: scores to walk
    const float *P;     // or the group partials of the pair term [B * L][nq][16][16] (S_in unused)
    int nq;
    int B, L, r;
    const int32_t *len;  // ragged batch: valid positions per block (nullptr: all L)
    float *S;  // scores out
    WalkParams w;
};

// DPP controls (gfx9): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror; row_shr:n is 0x110 + n.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Max over each 16-lane row, result in every lane of the row.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
    x = max(x, dpp_u32<kDppXor1>(x));
    x = max(x, dpp_u32<kDppXor2>(x));
    x = max(x, dpp_u32<kDppHalfMirror>(x));
    x = max(x, dpp_u32<kDppMirror>(x));
    return x;
}

__device__ __forceinline__ float row16_max_f(float x) {
    x = fmaxf(x, __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<kDppXor2>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(x))));
    x = fmaxf(x, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(x))));
    return x;
}

// Inclusive prefix sum over each 16-lane row (slot order): DPP row_shr with
// zeros shifted in at the row start.
template <int SH>
__device__ __forceinline__ float shr_row(float x) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(x), 0x110 + SH, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_scan(float x) {
    x += shr_row<1>(x);
    x += shr_row<2>(x);
    x += shr_row<4>(x);
    x += shr_row<8>(x);
    return x;
}

// Per-block LDS: for each position the chosen slot of every predecessor row,
// its score, and (when q is requested) every row's step distribution.
struct BlockShared {
    float *Q;     // [L][16][16] (only when q is requested)
    float *sc;    // [L][16] score of the chosen slot of each row
    uint8_t *ch;  // [L][16] chosen slot of each row
    int *row;     // [L] predecessor row of the walk at each position
};

// Decisions of one position from its score table held in the MFMA layout:
// s[v] = S[i = 4 g + v][j = lane & 15] with g = lane >> 4.
__device__ __forceinline__ void decide_position(const float (&s)[4], int t, const WalkParams &w,
                                                float u, bool want_q, BlockShared &sh) {
    const uint32_t lane = lane_id();
    const int g = (int)(lane >> 4), j = (int)(lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int i = 4 * g + v;
        // greedy successor of row i: highest order key, lowest slot among ties
        const uint32_t ob = order_bits(s[v]);
        const uint32_t mx = row16_max_u32(ob);
        const uint32_t seg_eq = (uint32_t)(ballot(ob == mx) >> (16 * g)) & 0xFFFFu;
        int pick = __builtin_ctz(seg_eq);
        if (w.mode == 1) {
            const bool isnum = s[v] == s[v];
            const float m = row16_max_f(isnum ? s[v] : -__builtin_inff());
            float e;
            if (m == -__builtin_inff()) e = (j == pick) ? 1.0f : 0.0f;  // no weight: greedy pick
            else if (!isnum) e = 0.0f;
            else if (m == __builtin_inff()) e = (s[v] == __builtin_inff()) ? 1.0f : 0.0f;
            else e = expf((s[v] - m) / w.temperature);
            const float c = row16_scan(e);
            const float Z = shfl_idxf(c, (lane & ~15u) | 15u);
            const uint32_t seg_hit = (uint32_t)(ballot(u * Z < c) >> (16 * g)) & 0xFFFFu;
            const uint32_t seg_pos = (uint32_t)(ballot(e > 0.0f) >> (16 * g)) & 0xFFFFu;
            if (seg_hit) pick = __builtin_ctz(seg_hit);
            else if (seg_pos) pick = 31 - __builtin_clz(seg_pos);
            if (want_q) sh.Q[(t * kK + i) * kK + j] = e / Z;
        } else if (want_q) {
            sh.Q[(t * kK + i) * kK + j] = (j == pick) ? 1.0f : 0.0f;
        }
        const float sp = shfl_idxf(s[v], (lane & ~15u) | (uint32_t)pick);
        if (j == 0) {
            sh.ch[t * kK + i] = (uint8_t)pick;
            sh.sc[t * kK + i] = sp;
        }
    }
}

// Columns of the rank per group of the pair sum: 64 when r is a multiple of 64
// and at least 128, else 32.  The pair term of a position is summed group by
// group (each group one chain of MFMAs over its columns in order), then the
// groups in order; project_pair_kernel produces the same group partials.
__host__ __device__ constexpr int pair_cw(int r) { return (r % 64 == 0 && r >= 128) ? 64 : 32; }

// One position (b, t) per workgroup of 4 waves.  Group g of the rank (columns
// g CW .. g CW + CW - 1) goes to wave g % 4; each wave issues every load of
// its groups up front (so the whole grid keeps enough bytes in flight for HBM)
// and accumulates each group's 16 x 16 table with v_mfma_f32_16x16x4_f32: lane
// (fr, fg) supplies row fr and column 16 s + 4 fg + c of slice s's c-th MFMA
// (the order of the sum over a group is a permutation of its columns).  The
// group tables are summed through LDS in group order.
template <int R>
__global__ __launch_bounds__(256) void pair_kernel(PairParams p) {
    constexpr int CW = pair_cw(R), NQ = R / CW;  // groups of the rank
    constexpr int GPW = (NQ + 3) / 4;            // groups per wave (the last waves may get fewer)
    constexpr int SPG = CW / 16;                 // 16-wide slices per group
    const int64_t bt = blockIdx.x;
    if (!position_live(p.len, blockIdx.x, p.L)) return;  // padding position (ragged batches)
    const int t = (int)(blockIdx.x % (uint32_t)p.L);
    const int wave = (int)(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const int fr = lane & 15, fg = lane >> 4;
    const float *Ap = p.A_prev + (bt * kK + fr) * R + 4 * fg;
    const float *Bp = p.B_cur + (bt * kK + fr) * R + 4 * fg;
    const float *Gp = p.G + bt * R + 4 * fg;
    float4 a[GPW][SPG], g[GPW][SPG], b[GPW][SPG];
#pragma unroll
    for (int k = 0; k < GPW; ++k) {
        const int grp = wave + 4 * k;
        const int c0 = (grp < NQ ? grp : 0) * CW;  // a wave past the last group loads group 0, unused
#pragma unroll
        for (int s = 0; s < SPG; ++s) {
            a[k][s] = *(const float4 *)(Ap + c0 + 16 * s);
            g[k][s] = *(const float4 *)(Gp + c0 + 16 * s);
            b[k][s] = *(const float4 *)(Bp + c0 + 16 * s);
        }
    }
    __shared__ floatx4 part[NQ][kWave];
#pragma unroll
    for (int k = 0; k < GPW; ++k) {
        const int grp = wave + 4 * k;
        if (grp >= NQ) break;  // wave-uniform
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SPG; ++s) {
            const float4 ag = float4{a[k][s].x * g[k][s].x, a[k][s].y * g[k][s].y, a[k][s].z * g[k][s].z,
                                     a[k][s].w * g[k][s].w};
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag.x, b[k][s].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag.y, b[k][s].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag.z, b[k][s].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag.w, b[k][s].w, acc, 0, 0, 0);
        }
        part[grp][lane] = acc;
    }
    __syncthreads();
    if (wave != 0) return;
    floatx4 sum = part[0][lane];
#pragma unroll
    for (int k = 1; k < NQ; ++k) sum += part[k][lane];
    // acc layout (16x16x4 f32): lane (fr, fg) holds rows i = 4 fg + v, column fr
    const float u = p.cand_u[bt * kK + fr];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int i = 4 * fg + v;
        p.S[(bt * kK + i) * kK + fr] = (t == 0 && i >= 1) ? -__builtin_inff() : u + sum[v];
    }
}

// The walk of block b over scores in global memory (S_in, or the group
// partials P) by the whole workgroup, its tables in `smem`
// (pair_walk_shmem bytes).
__device__ __forceinline__ void walk_block(const PairParams &p, int b, unsigned char *smem) {
    const int L = p.L;
    const bool want_q = p.w.q != nullptr;
    BlockShared sh;
    sh.Q = (float *)smem;
    sh.sc = sh.Q + (want_q ? L * kK * kK : 0);
    sh.row = (int *)(sh.sc + L * kK);
    sh.ch = (uint8_t *)(sh.row + L);

    const int n = block_len_of(p.len, b, L);  // positions to walk (ragged batches: the block's own)
    if (n == 0) return;
    const int nwave = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const uint32_t lane = lane_id();
    for (int t = wave; t < n; t += nwave) {
        const int64_t bt = (int64_t)b * L + t;
        float s[4];
        if (p.P != nullptr) {
            // S = U + (((P_0 + P_1) + P_2) + ...), the groups in order, as
            // pair_kernel sums them; rows i >= 1 of position 0 are -inf
            const int j = (int)(lane & 15);
            const float u = p.cand_u[bt * kK + j];
            const float *pp = p.P + bt * p.nq * (kK * kK) + 4 * (lane >> 4) * kK + j;
            floatx4 sum;
#pragma unroll
            for (int v = 0; v < 4; ++v) sum[v] = pp[v * kK];
            for (int k = 1; k < p.nq; ++k) {
                floatx4 x;
#pragma unroll
                for (int v = 0; v < 4; ++v) x[v] = pp[k * (kK * kK) + v * kK];
                sum += x;
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 4 * (int)(lane >> 4) + v;
                s[v] = (t == 0 && i >= 1) ? -__builtin_inff() : u + sum[v];
                if (p.S != nullptr) p.S[(bt * kK + i) * kK + j] = s[v];
            }
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) s[v] = p.S_in[(bt * kK + 4 * (lane >> 4) + v) * kK + (lane & 15)];
        }
        const float u = p.w.mode == 1 ? p.w.uniforms[bt] : 0.0f;
        decide_position(s, t, p.w, u, want_q, sh);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int row = 0;  // the last verified token
        for (int t = 0; t < n; ++t) {
            sh.row[t] = row;
            row = sh.ch[t * kK + row];
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n * kK; e += blockDim.x) {
        const int t = e / kK, j = e % kK;
        const int64_t bt = (int64_t)b * L + t;
        const int row = sh.row[t];
        if (j == 0) {
            const int c = sh.ch[t * kK + row];
            p.w.path_slot[bt] = c;
            p.w.path_tok[bt] = p.w.cand_id[bt * kK + c];
            if (p.w.path_s) p.w.path_s[bt] = sh.sc[t * kK + row];
        }
        if (want_q) p.w.q[bt * kK + j] = sh.Q[(t * kK + row) * kK + j];
    }
}

// The walk over scores in global memory: one workgroup per block.
__global__ __launch_bounds__(1024) void walk_kernel(PairParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    walk_block(p, blockIdx.x, smem);
}

inline size_t pair_walk_shmem(int L, bool want_q) {
    return (size_t)L * ((want_q ? kK * kK * sizeof(float) : 0) + kK * sizeof(float) + sizeof(int) + kK);
}

}  // namespace dsel
