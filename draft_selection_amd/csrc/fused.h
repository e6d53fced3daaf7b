// project_pair: the candidate projections and the pair term in one kernel.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector:
// A and B map tokens to 256-d vectors, H(h_t) gates them, and eq. S_t scores
// every adjacent candidate pair in one parallel pass.)
//
// A workgroup owns whole draft blocks (a tile of up to 16 positions, 256
// gathered candidate rows E[cand]) and one group of CW columns of the rank
// (two on the wide tile, below).
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
//
// Large uniform batches take a wide tile: one workgroup computes two groups (a
// 256 x 4 CW tile, wave tile 128 x CW instead of 64 x CW), so per MFMA it
// reads three quarters of the fragments from LDS and moves two thirds of the
// DMA bytes, and the grid has half as many workgroups, each with its setup and
// epilogue.  Its K steps are 32 deep, so that a step still has 16 MFMAs per
// wave between barriers and a four-stage ring (128 KB) fits; the MFMAs of
// every accumulator run in the same K order, so the bits are those of the
// narrow tile.
//
// A uniform batch puts floor(16 / L) consecutive blocks in a tile.  A ragged
// batch packs its blocks by their real lengths (packed_tile), so that the
// grid's first tiles hold all the work and the padding costs no MFMA time.
#pragma once

#include "pairwalk.h"
#include "project.h"

namespace dsel {

// Columns per group of the rank (per side): 64 when r is a multiple of 64 and
// at least 128, else 32.  nq = r / CW groups.
__host__ __device__ constexpr int pair_group_width(int r) { return (r % 64 == 0 && r >= 128) ? 64 : 32; }

// Wave grid of the narrow tile (NG = 1 group per workgroup): DSEL_FUSED_GM
// row slabs x 2 (A side, B side); 4 slabs = 8 waves (two per SIMD, wave tile
// 64 x CW), 64-deep K steps, a three-stage ring.  The wide tile (NG = 2): 2
// row slabs x 4 (A and B of each group), wave tile 128 x CW, 32-deep K steps,
// a four-stage ring.  Per step and wave both run 16 MFMAs; the LDS traffic of
// a step (DMA writes plus fragment reads) is 176 KB against 128 KB.
#ifndef DSEL_FUSED_GM
#define DSEL_FUSED_GM 4
#endif
template <int CW, int NG>
struct FusedShape;
template <int CW>
struct FusedShape<CW, 1> {
    using T = TileShape<256, 2 * CW, DSEL_FUSED_GM, 2>;
    static constexpr int NS = 3;
};
template <int CW>
struct FusedShape<CW, 2> {
    using T = TileShape<256, 4 * CW, 2, 4, 32>;
    static constexpr int NS = 4;
};
template <int CW, int NG = 1>
using FusedTile = typename FusedShape<CW, NG>::T;

// Tiles of a ragged batch, by harmonic bin packing (C. C. Lee and D. T. Lee,
// "A simple on-line bin-packing algorithm", J. ACM 32(3), 1985): a block with
// n >= 1 real positions has class c = floor(16 / n) and shares its tile with
// up to c - 1 other blocks of that class; slot k of the tile takes the local
// positions [k S, k S + n) with S = floor(16 / c) >= n.  Tiles are numbered
// class by class (c = 1, 2, 3, 4, 5, 8, 16), a class's blocks in index order;
// empty blocks take no slot.  There are at most floor(B / nb) + 7 tiles when
// every block has at most L positions (nb = floor(16 / L) <= c).  Called by a
// whole wave (wave-uniform result): one pass over the lengths for the class
// sizes, one to collect the tile's blocks.
struct TileBlocks {
    int S;      // local positions per slot
    int nslot;  // blocks in the tile (0: no such tile)
    int blk;    // lane k < nslot: the block of slot k (other lanes: -1)
};

__device__ __forceinline__ TileBlocks packed_tile(const int32_t *len, int B, int L, int tile) {
    constexpr int NC = 7;
    constexpr int C[NC] = {1, 2, 3, 4, 5, 8, 16};
    const uint32_t lane = lane_id();
    const uint64_t below = (1ull << lane) - 1ull;  // lanes under this one
    int cnt[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) cnt[i] = 0;
    for (int b0 = 0; b0 < B; b0 += kWave) {
        const int b = b0 + (int)lane;
        const int n = b < B ? block_len_of(len, b, L) : 0;
        const int c = n > 0 ? 16 / n : 0;
#pragma unroll
        for (int i = 0; i < NC; ++i) cnt[i] += __popcll(ballot(c == C[i]));
    }
    TileBlocks t{1, 0, -1};
    int cc = 0, first = 0, base = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int nt = (cnt[i] + C[i] - 1) / C[i];
        if (cc == 0 && tile < base + nt) {
            cc = C[i];
            first = (tile - base) * C[i];
            t.nslot = cnt[i] - first < C[i] ? cnt[i] - first : C[i];
        }
        base += nt;
    }
    if (cc == 0) return t;
    t.S = 16 / cc;
    int r0 = 0;
    for (int b0 = 0; b0 < B && r0 < first + t.nslot; b0 += kWave) {
        const int b = b0 + (int)lane;
        const int n = b < B ? block_len_of(len, b, L) : 0;
        const bool mine = n > 0 && 16 / n == cc;
        const uint64_t m = ballot(mine);
        const int rank = r0 + __popcll(m & below);
        uint64_t hit = ballot(mine && rank >= first && rank < first + t.nslot);
        while (hit) {
            const int src = __builtin_ctzll(hit);
            hit &= hit - 1;
            if ((int)lane == __builtin_amdgcn_readlane(rank, src) - first) t.blk = b0 + src;
        }
        r0 += __popcll(m);
    }
    return t;
}

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
    int nb;                 // blocks per tile of a uniform batch (16 / L)
    int ntile;              // row tiles of the grid (ceil(B / nb), + 7 for a ragged batch)
    int nq;                 // column groups (r / CW); a workgroup takes NG of them
    float *P;               // [B * L][nq][16][16] partial pair tables
    float *A_prev, *B_cur;  // optional [B * L * 16][r] (nullptr: not written)
};

template <int CW, int NG>
__global__ __launch_bounds__((FusedTile<CW, NG>::NT)) void project_pair_kernel(FusedParams p) {
    using T = FusedTile<CW, NG>;
    constexpr int NS = FusedShape<CW, NG>::NS;
    constexpr int BM = 256, BN = 2 * NG * CW, NW = T::NW, XI = T::DXI, WI = T::DWI, BK = T::BK;
    static_assert(T::BNv == BN && T::WN % CW == 0, "wave columns hold whole (side, group) column ranges");
    constexpr int RING = NS * (BM + BN) * BK;  // bf16 elements of the DMA ring
    constexpr int SROW = CW + 4;               // staged row stride in floats (bank skew)
    constexpr int STAGE = 2 * BM * SROW * 2;   // bf16-element size of one group's staged A and B
    __shared__ __attribute__((aligned(16))) uint16_t smem[RING > STAGE ? RING : STAGE];
    __shared__ uint32_t okw[BM / 32];
    // the gate of the tile's positions and A(verified) of its blocks, for the
    // workgroup's groups (row 16 g + position), staged before the main loop so
    // their latency hides there
    __shared__ __attribute__((aligned(16))) float Gs[16 * NG][CW];
    __shared__ __attribute__((aligned(16))) float Vs[16 * NG][CW];
    __shared__ int gposs[16];  // flat position of each local position (-1: none)
    uint16_t *const Xs = smem;
    uint16_t *const Ws = smem + NS * BM * BK;

    // XCD-aware order: workgroups w and w + 8 share an XCD; consecutive slots of
    // one XCD take the column groups of one tile (NG at a time: q0 .. q0 + NG - 1).
    const int w = (int)blockIdx.x;
    const int xcd = w & 7, slot = w >> 3;
    const int nqg = p.nq / NG;
    const int q0 = (slot % nqg) * NG;
    const int tile = (slot / nqg) * 8 + xcd;
    if (tile >= p.ntile) return;
    asm volatile("" ::: "a0");  // keep the accumulators in AGPRs (see project_cand_kernel)
    const uint32_t lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const int L = p.L, d = p.d, r = p.r;

    // The tile's blocks: slot k holds block `blk` of lane k and local positions
    // [k S, k S + S).  Same in every wave.
    TileBlocks tb;
    if (p.len == nullptr) {
        tb.S = L;
        tb.nslot = p.B - tile * p.nb < p.nb ? p.B - tile * p.nb : p.nb;
        tb.blk = (int)lane < tb.nslot ? tile * p.nb + (int)lane : -1;
    } else {
        tb = packed_tile(p.len, p.B, L, tile);
    }
    if (tb.nslot <= 0) return;  // no such tile (workgroup-uniform, before any barrier)
    const int S = tb.S;

    // Lane pp < 16: flat position gp of local position pp (slot k, step t).
    // Bit pp of validq: it is a real position; of succq: it also has a
    // successor in its block.
    uint32_t validq, succq;
    int gp = -1;
    {
        const int k = (int)(lane & 15) / S, t = (int)(lane & 15) - k * S;
        const int bk = (int)shfl_idx32((uint32_t)tb.blk, (uint32_t)k);
        bool v = false, sc = false;
        if (lane < 16u && k < tb.nslot) {
            const int n = block_len_of(p.len, bk, L);
            v = t < n;
            sc = t + 1 < n;
            gp = bk * L + t;
        }
        validq = (uint32_t)ballot(v);
        succq = (uint32_t)ballot(sc);
    }
    if (validq == 0) return;  // padding only (workgroup-uniform, before any barrier)
    if (wave == 0 && lane < 16u) gposs[lane] = (validq >> lane) & 1u ? gp : -1;  // the main loop's barriers publish it

    // Gathered rows: padding positions and out-of-range ids load E row 0; the
    // latter become zero rows.
    const uint16_t *xsrc[XI];
    uint32_t xok = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = dma_row<T>(u);
        const int gpr = (int)shfl_idx32((uint32_t)gp, (uint32_t)(row >> 4));
        int64_t tok = 0;
        if ((validq >> (row >> 4)) & 1u) {
            const int32_t t = p.cand[(int64_t)gpr * kK + (row & 15)];
            if (t >= 0 && (int64_t)t < p.V) {
                tok = t;
                xok |= 1u << u;
            } else if (lane % T::CPR == 0 && q0 == 0) {
                atomicOr(&g_device_error, 1);
            }
        }
        xsrc[u] = p.E + tok * d + dma_chunk_elems<T>(row);
    }
    // W tile rows, CW per side and group: W_A[(q0 + g) CW + c] at n = 2 CW g + c,
    // W_B[(q0 + g) CW + c] at n = 2 CW g + CW + c
    const uint16_t *wsrc[WI];
#pragma unroll
    for (int u = 0; u < WI; ++u) {
        const int n = dma_row<T>(u);
        const int wr = (q0 + n / (2 * CW)) * CW + n % CW;
        wsrc[u] = ((n / CW) % 2 == 0 ? p.WA : p.WB) + (int64_t)wr * d + dma_chunk_elems<T>(n);
    }

    // This thread's share of the epilogue's small operands, moved into LDS now
    // by LDS-DMA (no registers held across the main loop; the loop's first
    // wait covers them, being issued before its loads): float4 e of Gs and Vs
    // is G[gp(pp)][(q0 + g) CW ..] (g = e / (4 CW), pp = e / (CW / 4) % 16)
    // for real positions, and A(verified of the block of slot pp) for its
    // real slots; the other entries are not used.
    constexpr int NV4 = NG * 16 * CW / 4;  // float4s of NG 16 x CW tables
#pragma unroll
    for (int it = 0; it < (NV4 + T::NT - 1) / T::NT; ++it) {
        const int ew = wave + NW * it;  // the 1 KB piece of each table this wave fills
        if (ew * kWave < NV4) {         // wave-uniform
            const int e4 = ew * kWave + (int)lane, egi = e4 / (4 * CW), epp = (e4 / (CW / 4)) % 16;
            const int ecol = (q0 + egi) * CW + (e4 % (CW / 4)) * 4;
            const int gpe = (int)shfl_idx32((uint32_t)gp, (uint32_t)epp);
            const int vbk = (int)shfl_idx32((uint32_t)tb.blk, (uint32_t)epp);
            // lane l fills float4 64 ew + l
            if ((validq >> epp) & 1u) lds_dma16(p.G + (int64_t)gpe * r + ecol, (uint16_t *)&Gs[0][0] + 512 * ew);
            if (epp < tb.nslot && ((validq >> (epp * S)) & 1u))
                lds_dma16(p.A_ver + (int64_t)vbk * p.ver_stride + ecol, (uint16_t *)&Vs[0][0] + 512 * ew);
        }
    }

    // Id-validity bits of the 256 rows (word k: rows 32 k .. 32 k + 31), RPI
    // bits per (wave, DMA load); the main loop's barriers publish them
    {
#pragma unroll
        for (int u = 0; u < XI; ++u) {
            const uint64_t bl = ballot(((xok >> u) & 1u) != 0);
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < T::RPI; ++k) bits |= (uint32_t)((bl >> (T::CPR * k)) & 1u) << k;
            if (lane == 0) {
                if constexpr (T::RPI == 8) ((uint8_t *)okw)[wave + NW * u] = (uint8_t)bits;
                else ((uint16_t *)okw)[wave + NW * u] = (uint16_t)bits;
            }
        }
    }

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    mma_tile_dma_src<T, NS>(xsrc, wsrc, 0, d / BK, Xs, Ws, acc);

    __syncthreads();  // every wave is done with the ring (its LDS is reused below)
    auto row_ok = [&](int rl) { return ((okw[rl >> 5] >> (rl & 31)) & 1u) != 0; };
    const int wn = wave % T::GNv;
    // tile column n holds side (n / CW) % 2 (A, B) of group q0 + n / (2 CW),
    // column n % CW of it; a 32-column MFMA block lies in one such range

    // Optional outputs, as project_cand_kernel writes them: candidate row m of
    // side A becomes predecessor row of position t + 1 (output row m + 16),
    // written only where that position exists; side B for every real position.
    if (p.A_prev != nullptr) {
        for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) {
            const int side = (cl / CW) & 1;
            if (!(((side == 0 ? succq : validq) >> (rl >> 4)) & 1u)) return;
            float *const out = side == 0 ? p.A_prev + kK * r : p.B_cur;
            const int64_t grow = (int64_t)gposs[rl >> 4] * kK + (rl & 15);
            *(floatx4 *)(out + grow * r + (q0 + cl / (2 * CW)) * CW + cl % CW) =
                row_ok(rl) ? v : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        });
    }

    float *const As = (float *)smem;
    float *const Bs = As + BM * SROW;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        if (gi > 0) __syncthreads();  // the previous group's tables are done with LDS
        // Stage both sides of group q0 + gi in LDS as fp32 rows (zero rows for
        // out-of-range ids).
        {
            // straight from the MFMA layout: lane l holds column l % 32 of each
            // 32 x 32 block, rows 8 g + 4 (l / 32) + e (element 4 g + e); a store
            // instruction then covers 32 consecutive columns of two rows
            const int wm = wave / T::GNv;
            const int c0 = (int)(lane & 31), h4 = 4 * (int)(lane >> 5);
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int n0 = wn * T::WN + 32 * j;  // first tile column of block column j
                if (n0 / (2 * CW) != gi) continue;    // wave-uniform
                float *const Ss = ((n0 / CW) & 1 ? Bs : As) + n0 % CW + c0;
#pragma unroll
                for (int i = 0; i < T::TM; ++i)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int rl = wm * T::WM + 32 * i + 8 * g + h4 + e;
                            Ss[rl * SROW] = row_ok(rl) ? acc[i][j][4 * g + e] : 0.0f;
                        }
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
            const float *ap[2], *bp[2], *gsp[2];
            bool arow[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int pp = wave + NW * (2 * pr + k);
                const int t = pp % S;
                pps[k] = pp;
                gsp[k] = &Gs[16 * gi + pp][4 * fg];
                bp[k] = Bs + (kK * pp + fr) * SROW + 4 * fg;
                ap[k] = t > 0 ? As + (kK * (pp - 1) + fr) * SROW + 4 * fg
                              : &Vs[16 * gi + (pp < tb.nslot * S ? pp / S : 0)][4 * fg];
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
                    const float4 g = *(const float4 *)(gsp[k] + 16 * s);
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
                float *Pp = p.P + ((int64_t)gposs[pps[k]] * p.nq + q0 + gi) * (kK * kK) + fr;
#pragma unroll
                for (int v = 0; v < 4; ++v) Pp[(4 * fg + v) * kK] = pacc[k][v];
            }
        }
    }
}

// Blocks per tile and tiles of a batch for the fused kernel (block <= 16).
inline int fused_blocks_per_tile(int64_t block) { return block >= 1 && block <= 16 ? (int)(16 / block) : 0; }
inline int64_t fused_tiles(int64_t batch, int64_t block) {
    const int nb = fused_blocks_per_tile(block);
    return nb ? (batch + nb - 1) / nb : 0;
}
// Tiles of the grid: a ragged batch can need up to 7 more (packed_tile).
inline int64_t fused_grid_tiles(int64_t batch, int64_t block, bool ragged) {
    const int64_t nt = fused_tiles(batch, block);
    return nt && ragged ? nt + 7 : nt;
}
// Groups per workgroup: the wide tile (2) for a uniform batch whose grid
// still has DSEL_FUSED_WIDE_MIN workgroups (two rounds over the chip's 256
// CUs), else the narrow one; at fewer rounds the narrow tile's twice as many
// workgroups keep more CUs busy.  A ragged batch keeps the narrow tile: its
// live tiles (not known on the host) can be far fewer than the grid's, and
// then the finer unit balances better (c4's 5/8/16 mix: 155 live tiles of
// 263, 620 narrow workgroups against 310 wide).
#ifndef DSEL_FUSED_WIDE_MIN
#define DSEL_FUSED_WIDE_MIN 512
#endif
inline int fused_groups(int64_t batch, int64_t block, int64_t r, bool ragged) {
    const int cw = pair_group_width((int)r);
    const int64_t nq = r / cw;
    return !ragged && cw == 64 && nq % 2 == 0 && fused_tiles(batch, block) * (nq / 2) >= DSEL_FUSED_WIDE_MIN ? 2 : 1;
}
inline int64_t fused_grid(int64_t batch, int64_t block, int64_t r, bool ragged) {
    const int64_t nt = fused_grid_tiles(batch, block, ragged);
    return (nt + 7) / 8 * 8 * (r / pair_group_width((int)r) / fused_groups(batch, block, r, ragged));
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
