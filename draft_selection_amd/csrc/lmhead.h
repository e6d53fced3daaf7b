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
//       is done), and each wave updates the running top-16 of its 16 rows,
//       four rows at a time: a 16-lane row of the wave holds one row's sorted
//       list and screens that row's 256 logits (16 per lane) against the
//       list's 16th key; each round, every lane offers its best survivor, the
//       row's 16 offers are sorted and merged into the list (bitonic networks
//       on DPP lane swaps within the 16-lane row), and survivors below the new
//       16th drop out.  The lists live in LDS between tiles; at the end they
//       go out as 64-bit keys, one list per (row, vocab split).
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

// Bitonic sort, descending, of the 16 keys of every 16-lane row of the wave.
__device__ __forceinline__ uint64_t sort16_rows(uint64_t k) {
    const uint32_t lane = lane_id();
    k = bitonic_stage<1>(k, (lane & 2u) == 0);
    k = bitonic_stage<2>(k, (lane & 4u) == 0);
    k = bitonic_stage<1>(k, (lane & 4u) == 0);
    k = bitonic_stage<4>(k, (lane & 8u) == 0);
    k = bitonic_stage<2>(k, (lane & 8u) == 0);
    k = bitonic_stage<1>(k, (lane & 8u) == 0);
    k = bitonic_stage<8>(k, true);
    k = bitonic_stage<4>(k, true);
    k = bitonic_stage<2>(k, true);
    return bitonic_stage<1>(k, true);
}

// Top 16, sorted descending, of two sorted 16-lists in the same 16-lane rows:
// the elementwise max of one and the other reversed is bitonic (Batcher's
// merge), then four half-cleaner stages.
__device__ __forceinline__ uint64_t merge16_rows(uint64_t a, uint64_t b) {
    constexpr int kMirror = 0x140;  // DPP row_mirror: lane j of a row reads lane 15 - j
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, kMirror, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), kMirror, 0xF, 0xF, false);
    const uint64_t br = ((uint64_t)hi << 32) | lo;
    uint64_t k = a > br ? a : br;
    k = bitonic_stage<8>(k, true);
    k = bitonic_stage<4>(k, true);
    k = bitonic_stage<2>(k, true);
    return bitonic_stage<1>(k, true);
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
        // wave w updates rows 16 w .. 16 w + 15, four at a time: 16-lane row g
        // of the wave holds row r's list (lane j: entry j) and screens the
        // row's columns 64 i + 4 j .. 64 i + 4 j + 3 (i < 4) against its 16th
        // key.  Each round every lane offers its best remaining survivor; the
        // row's 16 offers are sorted and merged with its list (bitonic), the
        // threshold rises, and survivors below it drop out.
        const int g = (int)(lane >> 4), j = (int)(lane & 15);
        for (int pass = 0; pass < BM / T::NW / 4; ++pass) {
            const int r = wave * (BM / T::NW) + 4 * pass + g;
            const bool rok = m0 + r < p.R;
            uint64_t key = lists[r * kK + j];
            float thr_f = key_threshold(shfl_idx64(key, (lane & ~15u) | 15u));
            float v[16];
            uint32_t ob[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const floatx4 x = *(const floatx4 *)(tile + r * BN + 64 * i + 4 * j);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * i + e] = x[e];
            }
            uint32_t bits = 0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int col = 64 * (k >> 2) + 4 * j + (k & 3);  // increases with k
                ob[k] = order_bits(v[k]);
                if (rok && (int64_t)col < left && !(v[k] < thr_f)) bits |= 1u << k;
            }
            while (ballot(bits != 0) != 0ull) {
                // the lane's best survivor: highest order, then the lowest column
                int bk = -1;
                uint32_t bo = 0;
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (((bits >> k) & 1u) && (bk < 0 || ob[k] > bo)) {
                        bk = k;
                        bo = ob[k];
                    }
                uint64_t c = 0ull;
                if (bk >= 0) {
                    const uint32_t id = (uint32_t)n0 + 64 * (bk >> 2) + 4 * j + (bk & 3);
                    c = ((uint64_t)bo << 32) | (uint32_t)(~id);
                    bits &= ~(1u << bk);
                }
                key = merge16_rows(key, sort16_rows(c));
                thr_f = key_threshold(shfl_idx64(key, (lane & ~15u) | 15u));
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    if (v[k] < thr_f) bits &= ~(1u << k);
            }
            lists[r * kK + j] = key;
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
