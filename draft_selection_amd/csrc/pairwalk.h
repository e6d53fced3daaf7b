// score_pairs + walk.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector:
// eq. S_t scores every adjacent candidate pair in one parallel pass; the only
// sequential step walks the precomputed scores from the last verified token,
// greedily or by sampling.  "DFlash 2: The Drafter Stopped Guessing Alone",
// "Selection beats correction", says the same.)
//
// One workgroup per draft block.  Wave w scores positions t = w, w + nw, ...:
// the 16 x 16 table P[i][j] = sum_c A_prev[i][c] G[c] B_cur[j][c] is one fp32
// MFMA accumulation (v_mfma_f32_16x16x4_f32, r/4 steps); every lane streams
// 16-byte slices of its own A and B row straight from global memory, so the
// operands need no LDS staging.  S = U + P goes to LDS (and to global memory
// when asked); then wave 0 walks the block.
#pragma once

#include "common.h"

namespace dsel {

struct WalkParams {
    int mode;          // 0 greedy, 1 sampled
    float temperature;
    const float *uniforms;
    const int32_t *cand_id;
    int32_t *path_tok, *path_slot;
    float *path_s, *q;
};

struct PairParams {
    const float *cand_u, *A_prev, *B_cur, *G;
    int B, L, r;
    float *S;        // nullable
    int do_walk;
    WalkParams w;
};

// One walk step over the 16 scores s (lanes 0..15 hold slot j = lane).
// Returns the chosen slot (wave-uniform) and writes q (lanes 0..15) if asked.
__device__ __forceinline__ int walk_step(float s, int mode, float T, float u, float *q_out) {
    const uint32_t lane = lane_id();
    const bool act = lane < (uint32_t)kK;
    // greedy pick: highest score, ties to the lowest slot, NaN lowest
    uint64_t key = act ? (((uint64_t)order_bits(s) << 32) | (uint32_t)(31 - lane)) : 0ull;
#pragma unroll
    for (int o = 1; o < kK; o <<= 1) {
        uint64_t other = shfl_idx64(key, lane ^ (uint32_t)o);
        key = other > key ? other : key;
    }
    const int greedy = 31 - (int)(readlane64(key, 0) & 0xFFu);
    if (mode == 0) {
        if (q_out && act) *q_out = (lane == (uint32_t)greedy) ? 1.0f : 0.0f;
        return greedy;
    }
    // sampled: softmax(s / T) over the 16 slots, NaN given zero weight
    float sv = (act && s == s) ? s : -__builtin_inff();
    float m = sv;
#pragma unroll
    for (int o = 1; o < kK; o <<= 1) m = fmaxf(m, shfl_idxf(m, lane ^ (uint32_t)o));
    m = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(m), 0));  // lane 0 holds the 16-slot max
    if (m == -__builtin_inff()) {
        if (q_out && act) *q_out = (lane == (uint32_t)greedy) ? 1.0f : 0.0f;
        return greedy;
    }
    float e;
    if (!act || !(s == s)) e = 0.0f;
    else if (m == __builtin_inff()) e = (s == __builtin_inff()) ? 1.0f : 0.0f;
    else e = expf((s - m) / T);
    // inclusive prefix sum over lanes 0..15 in slot order
    float c = e;
#pragma unroll
    for (int o = 1; o < kK; o <<= 1) {
        float y = shfl_idxf(c, lane >= (uint32_t)o ? lane - o : lane);
        if ((lane & 15u) >= (uint32_t)o) c += y;
    }
    const float Z = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(c), kK - 1));
    const float uz = u * Z;
    uint64_t hit = ballot(act && uz < c);
    int pick;
    const uint64_t pos = ballot(act && e > 0.0f);  // never empty: the max has weight 1
    if (hit) pick = (int)__builtin_ctzll(hit);
    else if (pos) pick = 63 - (int)__builtin_clzll(pos);
    else pick = greedy;
    if (q_out && act) *q_out = e / Z;
    return pick;
}

// Walk one block; S_row(t, row) returns lane j's score S[b,t,row,j].
template <typename RowFn>
__device__ __forceinline__ void walk_block(const WalkParams &w, int b, int L, RowFn S_row) {
    const uint32_t lane = lane_id();
    int row = 0;  // the last verified token
    for (int t = 0; t < L; ++t) {
        const int64_t bt = (int64_t)b * L + t;
        float s = lane < (uint32_t)kK ? S_row(t, row, (int)lane) : 0.0f;
        float u = w.mode == 1 ? w.uniforms[bt] : 0.0f;
        float *qp = w.q ? w.q + bt * kK + lane : nullptr;
        int j = walk_step(s, w.mode, w.temperature, u, qp);
        float sj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(s), j));
        if (lane == 0) {
            w.path_slot[bt] = j;
            w.path_tok[bt] = w.cand_id[bt * kK + j];
            if (w.path_s) w.path_s[bt] = sj;
        }
        row = j;
    }
}

__global__ __launch_bounds__(1024) void pair_walk_kernel(PairParams p) {
    extern __shared__ float Ssh[];  // [L][16][16]
    const int b = blockIdx.x;
    const int nwave = blockDim.x / kWave;
    const int wave = threadIdx.x / kWave;
    const uint32_t lane = lane_id();
    const int r = p.r;
    const int fr = lane & 15, fg = lane >> 4;

    for (int t = wave; t < p.L; t += nwave) {
        const int64_t bt = (int64_t)b * p.L + t;
        const float *Ap = p.A_prev + (bt * kK + fr) * r + 4 * fg;
        const float *Bp = p.B_cur + (bt * kK + fr) * r + 4 * fg;
        const float *Gp = p.G + bt * r + 4 * fg;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < r; c0 += 16) {
            const float4 a = *(const float4 *)(Ap + c0);
            const float4 g = *(const float4 *)(Gp + c0);
            const float4 bb = *(const float4 *)(Bp + c0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x * g.x, bb.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y * g.y, bb.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z * g.z, bb.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w * g.w, bb.w, acc, 0, 0, 0);
        }
        // acc[v] = P[i = 4 fg + v][j = fr]
        const float u = p.cand_u[bt * kK + fr];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 4 * fg + v;
            const float sv = (t == 0 && i >= 1) ? -__builtin_inff() : u + acc[v];
            Ssh[(t * kK + i) * kK + fr] = sv;
            if (p.S) p.S[(bt * kK + i) * kK + fr] = sv;
        }
    }
    if (!p.do_walk) return;
    __syncthreads();
    if (wave == 0)
        walk_block(p.w, b, p.L, [&](int t, int row, int j) { return Ssh[(t * kK + row) * kK + j]; });
}

// The walk alone over scores in global memory: one wave per block.
__global__ __launch_bounds__(256) void walk_kernel(const float *S, int B, int L, WalkParams w) {
    const int b = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
    if (b >= B) return;
    walk_block(w, b, L, [&](int t, int row, int j) {
        return S[((((int64_t)b * L + t) * kK) + row) * kK + j];
    });
}

}  // namespace dsel
