// lmhead_topk: the drafter's LM head with the top-16 taken in its epilogue, so
// the logits never reach HBM.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: the
// candidates are the drafter's own 16 best logits of every position, and the
// selector needs no extra LM-head forward.)
//
//   lmhead_topk_kernel  workgroup (row tile, vocab split): 128 hidden-state
//       rows against a run of 256-column tiles of W.  Per column tile the
//       logits come from the LDS-DMA MFMA pipeline of project.h (bf16 in, fp32
//       accumulation), go through LDS (the pipeline's ring, free once the tile
//       is done), and each wave updates the running top-16 of its 16 rows:
//       lane l takes columns 4l .. 4l+3.  While a row's list is not full
//       (its first tile) the 16 best of the 64 lane maxima are sorted in
//       (64-lane bitonic sort on DPP and row swaps, one ds_bpermute to
//       reverse it, then a 32-lane bitonic merge with the list);
//       every other value is screened against the row's 16th key and the rare
//       survivors are inserted one at a time.  The lists live in LDS
//       between tiles; at the end they go out as 64-bit keys, one list per
//       (row, vocab split).
//   topk16_merge_kernel (topk16.h) merges the splits of every row.
#pragma once

#include "project.h"
#include "topk16.h"

namespace dsel {

struct LmheadParams {
    const uint16_t *h, *W;
    int64_t R, V;      // rows (positions), vocabulary
    int d;
    int mt;            // 128-row tiles
    int nvs, cpw;      // vocab splits, column tiles per split
    int nct;           // column tiles in all
    uint64_t *partial; // [R][nvs][16] keys
};

// 128 x 256 on 8 waves (2 x 4, wave tile 64 x 64), two waves per SIMD, with
// the lean pipeline (fragments one slice ahead): 256 registers per wave hold
// it, the accumulators and the top-16 state without spilling.
using LmTile = CandTile<256>;
constexpr int kLmBN = 256;

// LDS: the pipeline ring (3 stages of 128 + 256 rows x 128 bytes = 144 KB),
// which also holds a finished tile's 128 x 256 fp32 logits (128 KB), and the
// running lists (128 rows x 16 keys = 16 KB): 160 KB, all of it.
constexpr int kLmRingBytes = 3 * (128 + kLmBN) * kBK * 2;
constexpr int kLmListBytes = 128 * kK * 8;

// Merge a wave-uniform batch of candidate keys (one per lane, 0 = none) into the
// sorted list held in lanes 0..15 (descending): sort the 64 candidates, put the
// best 16 reversed beside the list (a bitonic 32-sequence) and merge.
__device__ __forceinline__ uint64_t list_merge64(uint64_t list, uint64_t cand) {
    const uint32_t lane = lane_id();
    const uint64_t srt = wave_sort64_desc(cand);
    const uint64_t rev = shfl_idx64(srt, lane >= 16 && lane < 32 ? 31 - lane : lane);
    uint64_t k = lane < 16 ? list : (lane < 32 ? rev : 0ull);
    k = bitonic_stage<16>(k, true);
    k = bitonic_stage<8>(k, true);
    k = bitonic_stage<4>(k, true);
    k = bitonic_stage<2>(k, true);
    k = bitonic_stage<1>(k, true);
    return lane < 16 ? k : 0ull;
}

__global__ __launch_bounds__(LmTile::NT) void lmhead_topk_kernel(LmheadParams p) {
    constexpr int BM = 128, BN = kLmBN;
    using T = LmTile;
    constexpr int NW = T::NW, XI = T::DXI;
    __shared__ __attribute__((aligned(16))) char lds[kLmRingBytes + kLmListBytes];
    uint16_t *Xs = (uint16_t *)lds;
    uint16_t *Ws = Xs + 3 * BM * kBK;
    float *tile = (float *)lds;                              // [128][BN], after a tile's GEMM
    uint64_t *lists = (uint64_t *)(lds + kLmRingBytes);      // [128][16]

    // XCD-aware order: the row tiles of one vocab split run on one XCD, so every
    // W tile comes from HBM once and from that XCD's L2 for the other row tiles.
    const int w = blockIdx.x;
    const int xcd = w & 7, slot = w >> 3;
    const int mt = slot % p.mt;
    const int vs = (slot / p.mt) * 8 + xcd;
    if (vs >= p.nvs) return;  // workgroup-uniform, before any barrier
    const int64_t m0 = (int64_t)mt * BM;
    const int d = p.d, nk = d / kBK;
    const uint32_t lane = lane_id();
    const int wave = threadIdx.x >> 6;

    const uint16_t *xsrc[XI];
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        xsrc[u] = p.h + (m < p.R ? m : 0) * d + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
    }
    for (int i = threadIdx.x; i < BM * kK; i += T::NT) lists[i] = 0ull;

    const int ct0 = vs * p.cpw;
    const int ct1 = ct0 + p.cpw < p.nct ? ct0 + p.cpw : p.nct;
    for (int ct = ct0; ct < ct1; ++ct) {
        const int64_t n0 = (int64_t)ct * BN;
        const int64_t left = p.V - n0;
        floatx16 acc[T::TM][T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
        __syncthreads();  // the previous tile's logits have been read
        mma_tile_dma_lean<T>(xsrc, p.W + n0 * d, d, 0, nk, Xs, Ws, acc, left < BN ? (int)left : BN);
        __syncthreads();  // every wave is done with the ring
        for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) { *(floatx4 *)(tile + rl * BN + cl) = v; });
        __syncthreads();
        // wave w updates rows 16 w .. 16 w + 15; lane l takes columns 4l .. 4l+3
        for (int rr = 0; rr < BM / T::NW; ++rr) {
            const int r = wave * (BM / T::NW) + rr;
            if (m0 + r >= p.R) break;  // wave-uniform
            WaveTop st;
            st.key = lane < 16 ? lists[r * kK + lane] : 0ull;
            st.refresh();
            const floatx4 v = *(const floatx4 *)(tile + r * BN + 4 * lane);
            bool ok[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ok[e] = (int64_t)(4 * lane + e) < left;
            const uint32_t cbase = (uint32_t)n0 + 4 * lane;
            int skip = -1;
            if (st.thr == 0ull) {
                // list not full (the row's first tile): seed it with the 16
                // best of the 64 lane maxima, real values that bound the rest,
                // beside the entries it already has
                uint64_t best = 0ull;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint64_t k = ok[e] ? cand_key(v[e], cbase + e) : 0ull;
                    if (k > best) {
                        best = k;
                        skip = e;
                    }
                }
                st.key = list_merge64(st.key, best);
                st.refresh();
            }
            // the rest, screened by value against the 16th key, one insertion
            // per survivor (rare once the list is full)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool pass = ok[e] && e != skip && !(v[e] < st.thr_f);
                st.offer(v[e], pass, [&](uint32_t src) { return (uint32_t)n0 + 4 * src + e; });
            }
            if (lane < 16) lists[r * kK + lane] = st.key;
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < BM * kK; i += T::NT) {
        const int r = i / kK;
        if (m0 + r < p.R) p.partial[((m0 + r) * p.nvs + vs) * kK + (i % kK)] = lists[i];
    }
}

// Vocab splits: about 256 workgroups (one per CU: the kernel holds 160 KB of
// LDS), rounded up to a multiple of 8 for the XCD order.
inline int lmhead_nvs(int64_t rows, int64_t V) {
    const int64_t mt = (rows + 127) / 128, nct = (V + kLmBN - 1) / kLmBN;
    int64_t nvs = (256 + mt - 1) / mt;
    if (nvs > nct) nvs = nct;
    nvs = (nvs + 7) / 8 * 8;
    return (int)nvs;
}

inline size_t lmhead_workspace_bytes(int64_t rows, int64_t V) {
    return (size_t)rows * (size_t)lmhead_nvs(rows, V) * kK * sizeof(uint64_t);
}

}  // namespace dsel
