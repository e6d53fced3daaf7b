// project_pair: the candidate projections and the pair term in one kernel.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector:
// A and B map tokens to 256-d vectors, H(h_t) gates them, and eq. S_t scores
// every adjacent candidate pair in one parallel pass.)
//
// A workgroup owns whole draft blocks (a tile of up to 16 positions, 256
// gathered candidate rows E[cand]) and one group of CW columns of the rank.
// It computes, on bf16 MFMA with fp32 accumulation, both sides of that group:
//     A(x)[c] = W_A[c] . E[x]   and   B(x)[c] = W_B[c] . E[x],  c in the group,
// for every candidate x of the tile (a 256 x 2 CW tile; the main loop is the
// LDS-DMA pipeline of project.h).  Because the tile holds whole blocks, every
// position's predecessors are in the tile too, except position 0's: the last
// verified token, whose A row the gate job has already written.  The epilogue
// stages A and B in LDS (fp32) and forms the group's share of the pair term
//     P_q[t][i][j] = sum_{c in group q} A(pred_i(t))[c] G[t][c] B(cand_j(t))[c]
// with fp32 MFMA (v_mfma_f32_16x16x4_f32), for every position of the tile.
// Only these partial tables (1 KB per position and group) leave the chip;
// the walk kernel adds the groups in order and the logit U.
//
// The per-group arithmetic is exactly pair_kernel's (same operand order, the
// gate multiplied into the A operand, same slice and component order), and
// A and B accumulate over K in the same order as project_cand_kernel, so the
// scores and (when asked for) A_prev / B_cur have the same bits as the
// separate calls.
//
// Workgroup order is XCD-aware: the nq groups of one tile run on one XCD, so
// its gathered rows come from HBM once and from that XCD's L2 afterwards.
#pragma once

#include "pairwalk.h"
#include "project.h"

namespace dsel {

// Columns per group of the rank (per side): 64 when r is a multiple of 64 and
// at least 128, else 32.  nq = r / CW groups.
__host__ __device__ constexpr int pair_group_width(int r) { return (r % 64 == 0 && r >= 128) ? 64 : 32; }

// Wave grid: DSEL_FUSED_GM row slabs x 2 (A side, B side); 4 slabs = 8 waves
// (two per SIMD, wave tile 64 x CW).
#ifndef DSEL_FUSED_GM
#define DSEL_FUSED_GM 4
#endif
template <int CW>
using FusedTile = TileShape<256, 2 * CW, DSEL_FUSED_GM, 2>;

struct FusedParams {
    const uint16_t *E;
    int64_t V;
    int d, r;
    const uint16_t *WA, *WB;
    const int32_t *cand;    // [B * L * 16]
    const float *G;         // [B * L][r] gate
    const float *A_ver;     // A(verified_b) at A_ver + b * ver_stride, r floats
    int64_t ver_stride;
    int B, L;
    const int32_t *len;     // ragged batch: valid positions per block (nullptr: all L)
    int nb;                 // blocks per tile (16 / L)
    int ntile;              // row tiles (ceil(B / nb))
    int nq;                 // column groups (r / CW)
    float *P;               // [B * L][nq][16][16] partial pair tables
    float *A_prev, *B_cur;  // optional [B * L * 16][r] (nullptr: not written)
};

template <int CW>
__global__ __launch_bounds__(FusedTile<CW>::NT) void project_pair_kernel(FusedParams p) {
    using T = FusedTile<CW>;
    constexpr int BM = 256, BN = 2 * CW, NW = T::NW, XI = T::DXI, WI = T::DWI;
    static_assert(T::WN == CW, "one wave column per side");
    constexpr int RING = 3 * (BM + BN) * kBK;  // bf16 elements of the DMA ring
    constexpr int SROW = CW + 4;               // staged row stride in floats (bank skew)
    constexpr int STAGE = 2 * BM * SROW * 2;   // bf16-element size of the staged A and B
    __shared__ __attribute__((aligned(16))) uint16_t smem[RING > STAGE ? RING : STAGE];
    __shared__ uint32_t okw[BM / 32];
    // the gate of the tile's positions and A(verified) of its blocks, for this
    // column group, staged before the main loop so their latency hides there
    __shared__ __attribute__((aligned(16))) float Gs[16][CW];
    __shared__ __attribute__((aligned(16))) float Vs[16][CW];
    uint16_t *const Xs = smem;
    uint16_t *const Ws = smem + 3 * BM * kBK;

    // XCD-aware order: workgroups w and w + 8 share an XCD; consecutive slots of
    // one XCD take the column groups of one tile.
    const int w = (int)blockIdx.x;
    const int xcd = w & 7, slot = w >> 3;
    const int q = slot % p.nq;
    const int tile = (slot / p.nq) * 8 + xcd;
    if (tile >= p.ntile) return;
    asm volatile("" ::: "a0");  // keep the accumulators in AGPRs (see project_cand_kernel)
    const uint32_t lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const int L = p.L, d = p.d, r = p.r;
    const int b0 = tile * p.nb;
    const int npos = p.nb * L;  // positions the tile can hold (<= 16)

    // bit pp of validq: local position pp (flat position b0 L + pp) is a real
    // one; of succq: it also has a successor in its block.  Same in every wave.
    uint32_t validq, succq;
    {
        bool v = false, sc = false;
        if ((int)lane < npos) {
            const int b = b0 + (int)lane / L, t = (int)lane % L;
            if (b < p.B) {
                const int n = block_len_of(p.len, b, L);
                v = t < n;
                sc = t + 1 < n;
            }
        }
        validq = (uint32_t)ballot(v);
        succq = (uint32_t)ballot(sc);
    }
    if (validq == 0) return;  // padding only (workgroup-uniform, before any barrier)

    const int64_t row0 = (int64_t)b0 * L * kK;  // the tile's first candidate row
    // Gathered rows: padding positions and out-of-range ids load E row 0; the
    // latter become zero rows.
    const uint16_t *xsrc[XI];
    uint32_t xok = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = dma_row<T>(u);
        int64_t tok = 0;
        if ((validq >> (row >> 4)) & 1u) {
            const int32_t t = p.cand[row0 + row];
            if (t >= 0 && (int64_t)t < p.V) {
                tok = t;
                xok |= 1u << u;
            } else if ((lane & 7) == 0 && q == 0) {
                atomicOr(&g_device_error, 1);
            }
        }
        xsrc[u] = p.E + tok * d + dma_chunk_elems(row);
    }
    // W tile rows: W_A[q CW + n] for n < CW, then W_B[q CW + n - CW]
    const uint16_t *wsrc[WI];
#pragma unroll
    for (int u = 0; u < WI; ++u) {
        const int n = dma_row<T>(u);
        const uint16_t *base = n < CW ? p.WA + (int64_t)(q * CW + n) * d : p.WB + (int64_t)(q * CW + n - CW) * d;
        wsrc[u] = base + dma_chunk_elems(n);
    }

    // This thread's share of the epilogue's small operands, loaded now (their
    // latency overlaps the main loop's first DMA steps) and put in LDS after
    // it: float4 e of G[b0 L + pp][q CW ..] (pp = e / (CW / 4)) for real
    // positions, and of A(verified of block b0 + pp) for the tile's real blocks.
    constexpr int NV4 = 16 * CW / 4;  // float4s of a 16 x CW table
    static_assert(NV4 <= T::NT, "one float4 per thread");
    const int e4 = (int)threadIdx.x, epp = e4 / (CW / 4), ec = (e4 % (CW / 4)) * 4;
    const bool gload = e4 < NV4 && ((validq >> epp) & 1u);
    const bool vload = e4 < NV4 && epp < p.nb && ((validq >> (epp * L)) & 1u);
    float4 gv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
    if (gload) gv = *(const float4 *)(p.G + ((int64_t)b0 * L + epp) * r + q * CW + ec);
    if (vload) vv = *(const float4 *)(p.A_ver + (int64_t)(b0 + epp) * p.ver_stride + q * CW + ec);

    // Id-validity bits of the 256 rows (word k: rows 32 k .. 32 k + 31); the
    // main loop's barriers publish them
    {
        uint8_t *bytes = (uint8_t *)okw;
#pragma unroll
        for (int u = 0; u < XI; ++u) {
            const uint64_t bl = ballot(((xok >> u) & 1u) != 0);
            uint32_t byte = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) byte |= (uint32_t)((bl >> (8 * k)) & 1u) << k;
            if (lane == 0) bytes[wave + NW * u] = (uint8_t)byte;
        }
    }

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    mma_tile_dma_src<T>(xsrc, wsrc, 0, d / kBK, Xs, Ws, acc);

    __syncthreads();  // every wave is done with the ring (its LDS is reused below)
    auto row_ok = [&](int rl) { return ((okw[rl >> 5] >> (rl & 31)) & 1u) != 0; };
    const int wn = wave % T::GNv;  // 0: A side, 1: B side
    const int cq = q * CW;

    // Optional outputs, as project_cand_kernel writes them: candidate row m of
    // side A becomes predecessor row of position t + 1 (output row m + 16),
    // written only where that position exists; side B for every real position.
    if (p.A_prev != nullptr) {
        float *const out = wn == 0 ? p.A_prev + (row0 + kK) * r : p.B_cur + row0 * r;
        const uint32_t wq = wn == 0 ? succq : validq;
        for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) {
            if (!((wq >> (rl >> 4)) & 1u)) return;
            *(floatx4 *)(out + (int64_t)rl * r + cq + (cl - wn * CW)) =
                row_ok(rl) ? v : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        });
    }

    if (gload) *(float4 *)&Gs[epp][ec] = gv;
    if (vload) *(float4 *)&Vs[epp][ec] = vv;
    // Stage both sides in LDS as fp32 rows (zero rows for out-of-range ids).
    float *const As = (float *)smem;
    float *const Bs = As + BM * SROW;
    {
        // straight from the MFMA layout: lane l holds column l % 32 of each
        // 32 x 32 block, rows 8 g + 4 (l / 32) + e (element 4 g + e); a store
        // instruction then covers 32 consecutive columns of two rows
        float *const Ss = wn == 0 ? As : Bs;
        const int wm = wave / T::GNv;
        const int c0 = (int)(lane & 31), h4 = 4 * (int)(lane >> 5);
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rl = wm * T::WM + 32 * i + 8 * g + h4 + e;
                    const bool ok = row_ok(rl);
#pragma unroll
                    for (int j = 0; j < T::TN; ++j) Ss[rl * SROW + 32 * j + c0] = ok ? acc[i][j][4 * g + e] : 0.0f;
                }
    }
    __syncthreads();

    // Pair partials: wave w takes local positions w, w + NW, ..., two at a time
    // with their MFMA chains interleaved.  Lane (fr, fg) supplies row fr and
    // columns 16 s + 4 fg + {0..3} of slice s, one v_mfma_f32_16x16x4_f32 per
    // column; the result holds rows i = 4 fg + v, column j = fr.  A position
    // that is padding is computed on whatever LDS holds and not stored.
    const int fr = (int)(lane & 15), fg = (int)(lane >> 4);
    static_assert(16 % (2 * NW) == 0, "positions in pairs");
#pragma unroll
    for (int pr = 0; pr < 16 / (2 * NW); ++pr) {
        int pps[2];
        const float *ap[2], *bp[2], *gp[2];
        bool arow[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int pp = wave + NW * (2 * pr + k);
            const int t = pp % L;
            pps[k] = pp;
            gp[k] = &Gs[pp][4 * fg];
            bp[k] = Bs + (kK * pp + fr) * SROW + 4 * fg;
            ap[k] = t > 0 ? As + (kK * (pp - 1) + fr) * SROW + 4 * fg : &Vs[pp < p.nb * L ? pp / L : 0][4 * fg];
            arow[k] = t > 0 || fr == 0;  // position 0 has one predecessor row
        }
        if (!((validq >> pps[0]) & 1u) && !((validq >> pps[1]) & 1u)) continue;  // wave-uniform
        floatx4 pacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < CW / 16; ++s) {
            float4 ag[2], b[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const float4 a = arow[k] ? *(const float4 *)(ap[k] + 16 * s) : float4{0.f, 0.f, 0.f, 0.f};
                const float4 g = *(const float4 *)(gp[k] + 16 * s);
                b[k] = *(const float4 *)(bp[k] + 16 * s);
                ag[k] = float4{a.x * g.x, a.y * g.y, a.z * g.z, a.w * g.w};
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) pacc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[k].x, b[k].x, pacc[k], 0, 0, 0);
#pragma unroll
            for (int k = 0; k < 2; ++k) pacc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[k].y, b[k].y, pacc[k], 0, 0, 0);
#pragma unroll
            for (int k = 0; k < 2; ++k) pacc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[k].z, b[k].z, pacc[k], 0, 0, 0);
#pragma unroll
            for (int k = 0; k < 2; ++k) pacc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[k].w, b[k].w, pacc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            if (!((validq >> pps[k]) & 1u)) continue;
            float *Pp = p.P + (((int64_t)b0 * L + pps[k]) * p.nq + q) * (kK * kK) + fr;
#pragma unroll
            for (int v = 0; v < 4; ++v) Pp[(4 * fg + v) * kK] = pacc[k][v];
        }
    }
}

// Blocks per tile and tiles of a batch for the fused kernel (block <= 16).
inline int fused_blocks_per_tile(int64_t block) { return block >= 1 && block <= 16 ? (int)(16 / block) : 0; }
inline int64_t fused_tiles(int64_t batch, int64_t block) {
    const int nb = fused_blocks_per_tile(block);
    return nb ? (batch + nb - 1) / nb : 0;
}
inline int64_t fused_grid(int64_t batch, int64_t block, int64_t r) {
    const int64_t nt = fused_tiles(batch, block);
    return (nt + 7) / 8 * 8 * (r / pair_group_width((int)r));
}

// Does dsel_select_path run the fused kernel for this shape?  It needs whole
// blocks in a 256-row tile (block <= 16) and enough workgroups to spread over
// the chip; small batches take the split-K candidate GEMM instead.
#ifndef DSEL_FUSED_MIN_WG
#define DSEL_FUSED_MIN_WG 128
#endif
inline bool use_fused(int64_t batch, int64_t block, int64_t r) {
    return fused_blocks_per_tile(block) > 0 && fused_tiles(batch, block) * (r / pair_group_width((int)r)) >= DSEL_FUSED_MIN_WG;
}

inline size_t fused_partial_bytes(int64_t batch, int64_t block, int64_t r) {
    return (size_t)batch * (size_t)block * (size_t)(r / pair_group_width((int)r)) * kK * kK * sizeof(float);
}

}  // namespace dsel
