// project: the compact token vectors A(x) = W_A E[x], B(x) = W_B E[x] of every
// candidate and predecessor, and the context gate G = sigmoid(W_H h_t).
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector, the
// paragraph after eq. S_t: A and B map tokens to 256-d vectors, H(h_t) gates
// them.)
//
// Both kernels compute tiles of C[m, n] = sum_k X[m, k] W[n, k] with bf16
// MFMA (v_mfma_f32_32x32x16_bf16) and fp32 accumulation; X rows may be gathered.
//
//   project_cand_kernel  X row m = E[cand_id[m]] (m over batch*block*16).  Tile
//       128 rows x BN columns of one side: side 0 is W_A (the row becomes
//       predecessor row j of position t+1), side 1 is W_B (candidate row j of
//       position t).  The two sides of a row tile run on the same XCD, back to
//       back, so the gathered rows come from HBM once and from L2 the second
//       time.
//   project_gate_kernel  the context gate (X = h, W = W_H, sigmoid epilogue) and
//       the verified tokens (X = E[verified], W = W_A: predecessor row 0 of
//       position 0; rows 1..15 of position 0 are written as zeros), split along
//       K over workgroups and summed by project_gate_reduce_kernel.  It does
//       not depend on select_topk.
//
// Main loop (mma_tile_dma): a K step is 64 deep (128 bytes of every row), or
// 32 deep for tiles that set BK = 32.  Tiles move from global memory straight
// into an LDS ring of three or more stages (global_load_lds_dwordx4, no
// staging registers), two or more steps ahead of the MFMAs.  In LDS the
// 16-byte chunk c of tile row `row` sits at chunk c ^ key(row): a fragment
// read serves 16 lanes (16 consecutive rows, one chunk each, 256 bytes) per
// LDS pass, and the key spreads them over all 64 banks.  128-byte rows:
// key(row) = (row / 2) % 8, the 8 even and the 8 odd rows (lower and upper 32
// banks) hit 8 distinct chunks each; 64-byte rows: key(row) = (row / 4) % 4,
// the four rows of each 16-bank quarter hit 4 distinct chunks.  The waves of
// a workgroup form a GM x GN grid, each owning (BM/GM) x (BN/GN) of the tile
// as 32 x 32 MFMA blocks.
#pragma once

#include <type_traits>

#include "common.h"
#include "topk16.h"

namespace dsel {

constexpr int kBK = 64;  // K elements per step (128 bytes per row)

// Fragment reads of the next step issued after each MFMA of the current one:
// 2 front-loads them into the first half of the step, so they have landed
// well before the wait at the next barrier.
#ifndef DSEL_MMA_RPM
#define DSEL_MMA_RPM 2
#endif
constexpr int RPM = DSEL_MMA_RPM;
// The step's DMA loads go out one per MFMA from MFMA number DSEL_MMA_DMA_AT
// (default: half way through the step's MFMAs, after the fragment reads of
// the next step have been issued).  Measured on the 256 x 128 fused tile: 4-5%
// faster main loop than issuing them from the first MFMA, at every workload.
#ifndef DSEL_MMA_DMA_AT
#define DSEL_MMA_DMA_AT (NMF / 2)
#endif


// BM x BN tile computed by GM x GN waves, each owning WM x WN as 32 x 32 MFMA
// blocks (v_mfma_f32_32x32x16_bf16: one wave keeps the matrix core near its
// peak, which the 16 x 16 shape does not).
template <int BM, int BN, int GM, int GN, int BK_ = kBK>
struct TileShape {
    static constexpr int BMv = BM, BNv = BN, GMv = GM, GNv = GN;
    static constexpr int BK = BK_;                         // K elements per step
    static constexpr int CPR = BK / 8;                     // 16-byte chunks per tile row
    static constexpr int RPI = 64 / CPR;                   // tile rows one LDS-DMA instruction fills
    static constexpr int NT = 64 * GM * GN;                // threads
    static constexpr int NW = GM * GN;                     // waves
    static constexpr int WM = BM / GM, WN = BN / GN;       // wave tile
    static constexpr int TM = WM / 32, TN = WN / 32;       // MFMA blocks per wave
    static constexpr int DXI = BM / RPI / NW, DWI = BN / RPI / NW;  // LDS-DMA loads per wave per step
    static_assert(BK == 64 || BK == 32, "K step");
    static_assert(TM >= 1 && TN >= 1 && DXI >= 1 && DWI >= 1, "tile shape");
    // chunk swizzle of a tile row (depends on row % 16 only)
    __device__ static __forceinline__ int key(int row) { return BK == 64 ? (row >> 1) & 7 : (row >> 2) & 3; }
};

// ---- direct-to-LDS pipeline --------------------------------------------------
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight
// into LDS (64 lanes fill 1 KB = 8 tile rows of 128 bytes, or 16 of 64), so
// no registers stage the tiles.  A ring of three LDS stages holds steps k,
// k+1, k+2 while step k computes.  Waits are explicit: `s_waitcnt vmcnt(n)` with n = the
// loads issued after the awaited step, then `s_barrier` (LDS-DMA completion is
// tracked by vmcnt; the barrier also tells every wave that nobody still reads
// the stage about to be refilled).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane into LDS at lds_base + 16 * lane (lds_base wave-uniform).
// Written as inline asm so that the compiler, which cannot tell which LDS bytes
// an LDS-DMA writes, does not wait for every outstanding DMA before each LDS
// read; the main loop has no other vector-memory loads and does its own waits.
__device__ __forceinline__ void lds_dma16(const void *src, uint16_t *lds_base) {
    const uint32_t m0v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_base;
    // m0 (the LDS destination base) is an input operand, so the compiler
    // loads it and knows its value
    asm volatile("global_load_lds_dwordx4 %1, off"
                 :
                 : "{m0}"(__builtin_amdgcn_readfirstlane(m0v)), "v"(src)
                 : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0): own LDS reads done and all but the last N
// vector-memory loads landed.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | ((N >> 4) << 14));
}

// acc += X * W^T over K steps [k0, k1) (T::BK-deep steps), k1 > k0.  W rows at
// or past `wrows` (a ragged last tile) load row wrows - 1; their results are
// the caller's to ignore.
//
// Schedule of one step kt: the wave waits for its own LDS reads of step kt
// (issued one step earlier) and its own DMA of step kt+1, then meets the
// others at the barrier: after it nobody reads step kt's stage any more and
// step kt+1 is complete in LDS.  It refills kt's stage with step kt+NS, issues
// all fragment reads of step kt+1 (KS x (TM + TN) ds_read_b128, into the other
// register set) and runs the MFMAs of step kt from registers while they fly.
// Keeping a whole step of reads in flight is what lets LDS reach its streaming
// rate; one slice at a time leaves it latency-bound.
// The tile row a lane's u-th DMA load fills (rows RPI (wave + NW u) +
// lane / CPR) and the source offset of its 16-byte chunk within that row:
// physical chunk lane % CPR of tile row `row` holds logical chunk
// (lane % CPR) ^ key(row).
template <class T>
__device__ __forceinline__ int dma_row(int u) {
    return T::RPI * ((int)(threadIdx.x >> 6) + T::NW * u) + (int)(lane_id() / T::CPR);
}
template <class T>
__device__ __forceinline__ int dma_chunk_elems(int row) {
    return (((int)(lane_id() % T::CPR)) ^ T::key(row)) << 3;
}

template <class T, int NS = 3>
__device__ __forceinline__ void mma_tile_dma_src(const uint16_t *const (&xsrc)[T::DXI],
                                                 const uint16_t *const (&wsrc)[T::DWI], int k0, int k1,
                                                 uint16_t *Xs, uint16_t *Ws, floatx16 (&acc)[T::TM][T::TN]);

// W rows from one row-major matrix (row stride wstride); tile rows at or past
// `wrows` re-read row wrows - 1.  NS: stages of the LDS ring (Xs and Ws hold
// NS steps each).
template <class T, int NS = 3>
__device__ __forceinline__ void mma_tile_dma(const uint16_t *const (&xsrc)[T::DXI], const uint16_t *wbase,
                                             int64_t wstride, int k0, int k1, uint16_t *Xs,
                                             uint16_t *Ws, floatx16 (&acc)[T::TM][T::TN],
                                             int wrows = T::BNv) {
    const uint16_t *wsrc[T::DWI];
#pragma unroll
    for (int u = 0; u < T::DWI; ++u) {
        const int row = dma_row<T>(u);
        const int srow = row < wrows ? row : wrows - 1;
        wsrc[u] = wbase + (int64_t)srow * wstride + dma_chunk_elems<T>(row);
    }
    mma_tile_dma_src<T, NS>(xsrc, wsrc, k0, k1, Xs, Ws, acc);
}

// The main loop proper: xsrc / wsrc are the lane's DMA sources at K = 0 (row
// pointer plus its swizzled chunk offset).  The ring has NS stages, so the DMA
// of a step goes out NS - 1 steps ahead of its MFMAs: more stages hide more
// latency where a step has little MFMA work (small column tiles).
template <class T, int NS>
__device__ __forceinline__ void mma_tile_dma_src(const uint16_t *const (&xsrc)[T::DXI],
                                                 const uint16_t *const (&wsrc)[T::DWI], int k0, int k1,
                                                 uint16_t *Xs, uint16_t *Ws, floatx16 (&acc)[T::TM][T::TN]) {
    constexpr int BM = T::BMv, BN = T::BNv, NW = T::NW;
    constexpr int XI = T::DXI, WI = T::DWI, BK = T::BK;
    static_assert(XI >= 1 && WI >= 1 && XI * NW * T::RPI == BM && WI * NW * T::RPI == BN, "DMA tile shape");
    constexpr int PER = XI + WI;  // loads per wave per step
    static_assert(NS >= 3 && (NS - 1) * PER < 64, "ring depth");
    constexpr int KS = BK / 16;  // 16-deep slices per step
    const uint32_t lane = lane_id();
    // wave-uniform, so the LDS-DMA destinations below are scalar arithmetic
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / T::GNv, wn = wave % T::GNv;
    const int fr = lane & 31, fk = lane >> 5;  // fragment row / column, 8-element K half
    // LDS element offsets of the rows of this lane's fragments, relative to a
    // stage; every such row is = fr (mod 32), so chunk (2 s + fk) of it sits
    // at physical chunk (2 s + fk) ^ key(fr)
    int aoff[T::TM], boff[T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i) aoff[i] = (wm * T::WM + i * 32 + fr) * BK;
#pragma unroll
    for (int j = 0; j < T::TN; ++j) boff[j] = (wn * T::WN + j * 32 + fr) * BK;
    const int rsw = T::key(fr);
#define DSEL_ISSUE(k, stage)                                                                   \
    do {                                                                                       \
        const int kk_ = ((k) < k1 ? (k) : k1 - 1) * BK;                                       \
        _Pragma("unroll") for (int u = 0; u < XI; ++u)                                         \
            lds_dma16(xsrc[u] + kk_, Xs + (stage) * BM * BK + (T::RPI * (wave + NW * u)) * BK);   \
        _Pragma("unroll") for (int u = 0; u < WI; ++u)                                         \
            lds_dma16(wsrc[u] + kk_, Ws + (stage) * BN * BK + (T::RPI * (wave + NW * u)) * BK);   \
    } while (0)
#define DSEL_READ_STEP(set, stage)                                                             \
    do {                                                                                       \
        const uint16_t *xb_ = Xs + (stage) * BM * BK, *wb_ = Ws + (stage) * BN * BK;         \
        _Pragma("unroll") for (int s_ = 0; s_ < KS; ++s_) {                                    \
            const int ch_ = ((s_ * 2 + fk) ^ rsw) << 3;                                        \
            _Pragma("unroll") for (int i = 0; i < T::TM; ++i)                                  \
                fa[set][s_][i] = *(const bf16x8 *)(xb_ + aoff[i] + ch_);                       \
            _Pragma("unroll") for (int j = 0; j < T::TN; ++j)                                  \
                fb[set][s_][j] = *(const bf16x8 *)(wb_ + boff[j] + ch_);                       \
        }                                                                                      \
    } while (0)
    bf16x8 fa[2][KS][T::TM], fb[2][KS][T::TN];
    // DMA load q of a step (q < XI: X rows, then W rows) into stage `stage`
    auto dma = [&](int q, int kk, int stage) {
        if (q < XI) lds_dma16(xsrc[q] + kk, Xs + stage * BM * BK + (T::RPI * (wave + NW * q)) * BK);
        else lds_dma16(wsrc[q - XI] + kk, Ws + stage * BN * BK + (T::RPI * (wave + NW * (q - XI))) * BK);
    };
    // One step kt whose fragments are in register set SET: the MFMAs of kt
    // with the fragment reads of kt+1 (from the next stage) interleaved one or
    // two per MFMA, so the matrix pipe starts at once and LDS serves a steady
    // stream rather than a burst from every wave right after the barrier; the
    // DMA of kt+NS into kt's stage goes out one load per MFMA from MFMA
    // DSEL_MMA_DMA_AT on.
    // (Past the last step the reads fetch a stale stage into the unused set:
    // in bounds and harmless.)
    // fragment read rr of a step: slice rr / (TM + TN), then its A fragments
    // and its B fragments
    constexpr int NR = KS * (T::TM + T::TN);
    auto frag_read = [&](int rr, const uint16_t *xb, const uint16_t *wb, auto setc) {
        constexpr int S2 = decltype(setc)::value;
        const int s_ = rr / (T::TM + T::TN), f = rr % (T::TM + T::TN);
        const int ch = ((s_ * 2 + fk) ^ rsw) << 3;
        if (f < T::TM) fa[S2][s_][f] = *(const bf16x8 *)(xb + aoff[f] + ch);
        else fb[S2][s_][f - T::TM] = *(const bf16x8 *)(wb + boff[f - T::TM] + ch);
    };
    int cur = 0;
    auto step = [&](int kt, auto setc) {
        constexpr int SET = decltype(setc)::value;
        wait_vmcnt_lgkm0<(NS - 2) * PER>();  // own reads of kt done, own DMA of kt+1 landed
        wg_barrier();             // everyone's: kt's stage is free, kt+1 is complete
        __builtin_amdgcn_sched_barrier(0);
        const int nxt = cur == NS - 1 ? 0 : cur + 1;
        const uint16_t *xb = Xs + nxt * BM * BK, *wb = Ws + nxt * BN * BK;
        const int kk = (kt + NS < k1 ? kt + NS : k1 - 1) * BK;
        constexpr int NMF = KS * T::TM * T::TN;
#pragma unroll
        for (int s_ = 0; s_ < KS; ++s_) {
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
                    const int q = (s_ * T::TM + i) * T::TN + j;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[SET][s_][i], fb[SET][s_][j],
                                                                        acc[i][j], 0, 0, 0);
#pragma unroll
                    for (int rr = q * RPM; rr < (q + 1) * RPM; ++rr)
                        if (rr < NR) frag_read(rr, xb, wb, std::integral_constant<int, SET ^ 1>());
                    if (q >= DSEL_MMA_DMA_AT && q < DSEL_MMA_DMA_AT + PER) dma(q - DSEL_MMA_DMA_AT, kk, cur);
                    __builtin_amdgcn_sched_barrier(0);  // keep this order
                }
        }
#pragma unroll
        for (int rr = NMF * RPM; rr < NR; ++rr) frag_read(rr, xb, wb, std::integral_constant<int, SET ^ 1>());
#pragma unroll
        for (int q = NMF; q < DSEL_MMA_DMA_AT + PER; ++q)
            if (q >= DSEL_MMA_DMA_AT) dma(q - DSEL_MMA_DMA_AT, kk, cur);
        cur = nxt;
    };
#pragma unroll
    for (int st = 0; st < NS; ++st) DSEL_ISSUE(k0 + st, st);
    wait_vmcnt<(NS - 1) * PER>();
    wg_barrier();
    DSEL_READ_STEP(0, 0);
    // Steps in pairs (register sets 0 then 1), then an odd last step in set 0.
    // One loop exit: a break between the two steps made the compiler copy
    // every accumulator on each trip.
    int kt = k0;
    for (; kt + 1 < k1; kt += 2) {
        step(kt, std::integral_constant<int, 0>());
        step(kt + 1, std::integral_constant<int, 1>());
    }
    if (kt < k1) step(kt, std::integral_constant<int, 0>());
    wait_vmcnt<0>();  // drain the redundant tail loads before LDS is released
#undef DSEL_ISSUE
#undef DSEL_READ_STEP
#undef DSEL_STEP
}

// The same product with a leaner register footprint: fragments are read one
// 16-deep slice ahead (two sets of TM + TN fragments instead of two whole K
// steps), for kernels that keep other state live beside the GEMM.  While
// slice s multiplies, slice s+1 is read; at a step's last slice the wave
// waits for its own reads and its DMA of the next step, meets the others at
// the barrier, refills the stage NS steps ahead and reads the next step's
// first fragments ahead of the last slice's MFMAs.
template <class T, int NS = 3>
__device__ __forceinline__ void mma_tile_dma_lean_src(const uint16_t *const (&xsrc)[T::DXI],
                                                      const uint16_t *const (&wsrc)[T::DWI], int k0, int k1,
                                                      uint16_t *Xs, uint16_t *Ws, floatx16 (&acc)[T::TM][T::TN]) {
    constexpr int BM = T::BMv, BN = T::BNv, NW = T::NW;
    constexpr int XI = T::DXI, WI = T::DWI;
    static_assert(XI >= 1 && WI >= 1 && XI * NW * 8 == BM && WI * NW * 8 == BN, "DMA tile shape");
    constexpr int PER = XI + WI;
    static_assert(NS >= 2 && (NS - 1) * PER < 64, "ring depth");
    constexpr int KS = kBK / 16;
    static_assert(T::BK == kBK, "64-deep steps");
    const uint32_t lane = lane_id();
    // wave-uniform, so the LDS-DMA destinations below are scalar arithmetic
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / T::GNv, wn = wave % T::GNv;
    const int fr = lane & 31, fk = lane >> 5;
    int aoff[T::TM], boff[T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i) aoff[i] = (wm * T::WM + i * 32 + fr) * kBK;
#pragma unroll
    for (int j = 0; j < T::TN; ++j) boff[j] = (wn * T::WN + j * 32 + fr) * kBK;
    const int rsw = T::key(fr);
    auto issue = [&](int k, int stage) {
        const int kk = (k < k1 ? k : k1 - 1) * kBK;
#pragma unroll
        for (int u = 0; u < XI; ++u) lds_dma16(xsrc[u] + kk, Xs + stage * BM * kBK + (8 * (wave + NW * u)) * kBK);
#pragma unroll
        for (int u = 0; u < WI; ++u) lds_dma16(wsrc[u] + kk, Ws + stage * BN * kBK + (8 * (wave + NW * u)) * kBK);
    };
    bf16x8 a[2][T::TM], b[2][T::TN];
    auto frag = [&](int buf, const uint16_t *xb, const uint16_t *wb, int sl) {
        const int ch = ((sl * 2 + fk) ^ rsw) << 3;
#pragma unroll
        for (int i = 0; i < T::TM; ++i) a[buf][i] = *(const bf16x8 *)(xb + aoff[i] + ch);
#pragma unroll
        for (int j = 0; j < T::TN; ++j) b[buf][j] = *(const bf16x8 *)(wb + boff[j] + ch);
    };
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(k0 + st, st);
    wait_vmcnt<(NS - 1) * PER>();
    wg_barrier();
    frag(0, Xs, Ws, 0);
    int cur = 0;
    for (int kt = k0; kt < k1; ++kt) {
        const int nxt = cur == NS - 1 ? 0 : cur + 1;
        const uint16_t *xb = Xs + cur * BM * kBK;
        const uint16_t *wb = Ws + cur * BN * kBK;
#pragma unroll
        for (int sl = 0; sl < KS; ++sl) {
            const int c = sl & 1, n = c ^ 1;
            if (sl + 1 < KS) {
                frag(n, xb, wb, sl + 1);
            } else {
                wait_vmcnt_lgkm0<(NS - 2) * PER>();
                wg_barrier();
                issue(kt + NS, cur);
                frag(n, Xs + nxt * BM * kBK, Ws + nxt * BN * kBK, 0);
            }
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
        }
        cur = nxt;
    }
    wait_vmcnt<0>();
}

// W rows from one row-major matrix (row stride wstride); tile rows at or past
// `wrows` re-read row wrows - 1.
template <class T>
__device__ __forceinline__ void mma_tile_dma_lean(const uint16_t *const (&xsrc)[T::DXI], const uint16_t *wbase,
                                                  int64_t wstride, int k0, int k1, uint16_t *Xs, uint16_t *Ws,
                                                  floatx16 (&acc)[T::TM][T::TN], int wrows = T::BNv) {
    const uint16_t *wsrc[T::DWI];
#pragma unroll
    for (int u = 0; u < T::DWI; ++u) {
        const int row = dma_row<T>(u);
        const int srow = row < wrows ? row : wrows - 1;
        wsrc[u] = wbase + (int64_t)srow * wstride + dma_chunk_elems<T>(row);
    }
    mma_tile_dma_lean_src<T, 3>(xsrc, wsrc, k0, k1, Xs, Ws, acc);
}

// Valid-row mask of a BM-row tile, shared through LDS.  Rows are loaded by
// lanes with lane % 8 == 0 of wave w as rows 8 (w + NW u) + lane / 8, u < XI;
// bit u of `xok` says the row's source was valid.  Each (wave, u) pair owns one
// byte of the mask, so word q of `lds` (read as uint32) afterwards holds rows
// 32 q .. 32 q + 31.  A second mask, `xlive` (the row is a real position of
// the batch, whatever its token), goes to words 4 .. 7 the same way.  Call after
// the main loop: LDS is reused, and the leading barrier also retires every
// wave's last LDS-DMA.
template <int NW, int XI>
__device__ __forceinline__ void tile_row_mask(uint32_t xok, uint16_t *lds, uint32_t xlive = 0u) {
    uint8_t *bytes = (uint8_t *)lds;
    const int wave = threadIdx.x >> 6;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const uint64_t b = ballot(((xok >> u) & 1u) != 0);
        const uint64_t bl = ballot(((xlive >> u) & 1u) != 0);
        uint32_t byte = 0, bytel = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            byte |= (uint32_t)((b >> (8 * k)) & 1u) << k;
            bytel |= (uint32_t)((bl >> (8 * k)) & 1u) << k;
        }
        if (lane_id() == 0) {
            bytes[wave + NW * u] = (uint8_t)byte;
            bytes[16 + wave + NW * u] = (uint8_t)bytel;
        }
    }
    __syncthreads();
}

// Bit rl of the masks tile_row_mask left in LDS.
__device__ __forceinline__ bool tile_row_ok(const uint16_t *lds, int rl) {
    return (((const uint32_t *)lds)[rl >> 5] >> (rl & 31)) & 1u;
}
__device__ __forceinline__ bool tile_row_live(const uint16_t *lds, int rl) {
    return (((const uint32_t *)lds)[4 + (rl >> 5)] >> (rl & 31)) & 1u;
}

// The accumulator layout of v_mfma_f32_32x32x16 gives lane l the column l % 32
// of a 32 x 32 block, rows 8 g + 4 (l / 32) + e (element 4 g + e, e < 4): four
// rows of one column per group g.  A 4 x 4 transpose inside each quad of lanes
// (DPP quad permutes, two exchange stages) turns that into one row of four
// consecutive columns per lane, so the epilogue stores 16 bytes per lane and
// a quarter of the store instructions.  Lane 4 q + k then holds row
// 8 g + 4 (l / 32) + k, columns 4 q .. 4 q + 3 of the block.
__device__ __forceinline__ float dpp_quad_xor1(float x) {  // quad_perm [1, 0, 3, 2]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {  // quad_perm [2, 3, 0, 1]
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ floatx4 quad_transpose4(float x0, float x1, float x2, float x3) {
    const uint32_t k = lane_id() & 3u;
    float x[4] = {x0, x1, x2, x3};
#pragma unroll
    for (int pr = 0; pr < 4; pr += 2) {  // exchange with lane k ^ 1: rows r and r ^ 1
        const float recv = dpp_quad_xor1((k & 1u) ? x[pr] : x[pr + 1]);
        if (k & 1u) x[pr] = recv;
        else x[pr + 1] = recv;
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {  // exchange with lane k ^ 2: rows r and r ^ 2
        const float recv = dpp_quad_xor2((k & 2u) ? x[pr] : x[pr + 2]);
        if (k & 2u) x[pr] = recv;
        else x[pr + 2] = recv;
    }
    return floatx4{x[0], x[1], x[2], x[3]};
}

// Hand every accumulator of the wave to `put(rl, cl, v)` as rows of four:
// tile row rl, tile columns cl .. cl + 3 (cl a multiple of 4), values v.
template <class T, class Put>
__device__ __forceinline__ void for_tile_rows4(const floatx16 (&acc)[T::TM][T::TN], Put put) {
    const uint32_t lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int wm = wave / T::GNv, wn = wave % T::GNv;
    const int rq = 4 * (int)(lane >> 5) + (int)(lane & 3);  // row within a group of 8
    const int cq = (int)(lane & 31) & ~3;                   // first column of the quad
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const floatx4 v = quad_transpose4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                                  acc[i][j][4 * g + 3]);
                put(wm * T::WM + i * 32 + 8 * g + rq, wn * T::WN + j * 32 + cq, v);
            }
}

struct CandParams {
    const uint16_t *E;
    int64_t V;
    int d, r;
    const uint16_t *WA, *WB;
    const int32_t *cand;
    int L;
    const int32_t *len;  // ragged batch: valid positions per block (nullptr: all L)
    int64_t M;        // batch * block * 16 gathered rows
    int mt, mt_pad;   // row tiles (mt_pad: rounded up to a multiple of 8)
    int nside;        // column tiles per side (r / BN)
    int nsplit;       // K splits (small batches); > 1: partial tiles go to `part`
    float *part;      // [nsplit][mt * 2 * nside][128][BN] partial tiles
    float *A_prev, *B_cur;
    // With tk_part set, the candidates are not in `cand` yet: each workgroup
    // merges the top-16's partial lists [rows][tk_nsplit][16] of its tile's
    // positions itself, and the workgroups of split 0, column tile 0 write
    // cand_id / cand_u (cand_u's two merged codes read back from the logits,
    // bf16 or fp32 rows ld elements apart).
    const uint64_t *tk_part;
    int tk_nsplit;
    int32_t *cand_id;
    float *cand_u;
    const char *logits;
    int64_t ld, V_logits;
    bool logits_bf16;
};

// Column tile BN of one side: BN = 256 on 8 waves (2 x 4, wave tile 64 x 64:
// two waves per SIMD hide each other's LDS latency), BN = 128 and 64 on 4 waves
// (2 x 2), BN = 32 on 4 waves (4 x 1).
#ifndef DSEL_CAND_XCD_SIDE
#define DSEL_CAND_XCD_SIDE 0
#endif
#ifndef DSEL_CAND_GM256
#define DSEL_CAND_GM256 2
#endif
#ifndef DSEL_CAND_GN256
#define DSEL_CAND_GN256 4
#endif
template <int BN>
using CandTile = TileShape<128, BN, (BN == 32 ? 4 : BN == 256 ? DSEL_CAND_GM256 : 2),
                           (BN == 32 ? 1 : BN == 256 ? DSEL_CAND_GN256 : 2)>;
inline int tile_threads(int BN) {
    return BN == 256 ? CandTile<256>::NT : BN == 128 ? CandTile<128>::NT : BN == 64 ? CandTile<64>::NT
                                                                                 : CandTile<32>::NT;
}

template <int BN>
__global__ __launch_bounds__(CandTile<BN>::NT) void project_cand_kernel(CandParams p) {
    constexpr int BM = 128;
    using T = CandTile<BN>;
    constexpr int NW = T::NW;
    constexpr int XI = T::DXI;
    __shared__ __attribute__((aligned(16))) uint16_t Xs[3 * BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[3 * BN * kBK];

    // XCD-aware tile order: workgroups w and w + 8 share an XCD; consecutive
    // slots of one XCD take the column tiles of one row tile.  With K splits
    // the grid repeats that order once per split.
    const int ncol = 2 * p.nside;
    const int per_split = p.mt_pad * ncol;
    const int ks = (int)(blockIdx.x / per_split);
    const int w = (int)(blockIdx.x % per_split);
    const int xcd = w & 7, slot = w >> 3;
#if DSEL_CAND_XCD_SIDE
    // XCDs 0-3 take side 0, 4-7 side 1: each L2 holds one W
    const int side = xcd >> 2;
    const int mt = (slot / p.nside) * 4 + (xcd & 3);
    const int n0 = (slot % p.nside) * BN;
    const int ct = side * p.nside + slot % p.nside;
#else
    const int ct = slot % ncol;
    const int mt = (slot / ncol) * 8 + xcd;
    const int side = ct / p.nside;  // 0: W_A, 1: W_B
    const int n0 = (ct % p.nside) * BN;
#endif
    if (mt >= p.mt) return;
    // Declaring an AGPR clobber tells the compiler the kernel uses AGPRs, so it
    // keeps the MFMA accumulators there (the AGPR form of the instruction)
    // instead of in VGPRs: the LDS fragment reads then land in a register file
    // the MFMAs do not read and write every cycle (measured 1-3% faster on the
    // 80- and 96-step K loops, same bits).
    asm volatile("" ::: "a0");
    const int64_t m0 = (int64_t)mt * BM;
    const int tid = threadIdx.x;
    const int d = p.d, r = p.r;
    const uint32_t lane = lane_id();
    const int wave = tid >> 6;

    // The tile's 8 positions (16 candidate rows each): bit q of `validq` says
    // position q is a real one (t < its block's length), of `succq` that it
    // has a successor in its block (t + 1 < length).  The same in every wave.
    uint32_t validq, succq;
    {
        const int64_t bt = m0 / kK + (lane & 7);
        bool v = false, sc = false;
        if (lane < 8 && bt * kK < p.M) {
            const uint32_t b = (uint32_t)bt / (uint32_t)p.L;
            const int n = block_len_of(p.len, b, p.L);
            const int t = (int)((uint32_t)bt - b * (uint32_t)p.L);
            v = t < n;
            sc = t + 1 < n;
        }
        validq = (uint32_t)ballot(v);
        succq = (uint32_t)ballot(sc);
    }
    if (validq == 0) return;  // padding only (workgroup-uniform, before any barrier)

    // The merge of the top-16's partial lists: every list of the tile's real
    // positions goes into LDS at once (the DMA ring is free until the main
    // loop), then one position per wave at a time is folded from there.
    __shared__ int32_t mid[BM];
    if (p.tk_part != nullptr) {
        const bool owner = ks == 0 && ct == 0;
        uint64_t *lists = (uint64_t *)Xs;  // [8][tk_nsplit][16]; the planner keeps it within Xs
        const int per = p.tk_nsplit * kK, all = (BM / kK) * per;
        // every load in flight before the first LDS write
        constexpr int EPT = (3 * BM * kBK * 2 / 8 + NW * kWave - 1) / (NW * kWave);  // keys per thread, at most
        uint64_t v[EPT];
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + u * NW * kWave, pq = e / per;
            if (e < all && ((validq >> pq) & 1u)) v[u] = p.tk_part[(m0 / kK + pq) * per + (e - pq * per)];
        }
#pragma unroll
        for (int u = 0; u < EPT; ++u) {
            const int e = tid + u * NW * kWave, pq = e / per;
            if (e < all && ((validq >> pq) & 1u)) lists[e] = v[u];
        }
        __syncthreads();
        for (int pq = wave; pq < BM / kK; pq += NW) {
            if (!((validq >> pq) & 1u)) continue;  // wave-uniform
            const int64_t bt = m0 / kK + pq;
            const uint64_t best = wave_merge_lists(lists + pq * per, p.tk_nsplit);
            if (lane < (uint32_t)kK) {
                mid[pq * kK + lane] = (int32_t)key_id(best);
                if (owner) {
                    p.cand_id[bt * kK + lane] = (int32_t)key_id(best);
                    p.cand_u[bt * kK + lane] =
                        p.logits_bf16 ? merged_value<true>(best, p.logits + bt * p.ld * 2, p.V_logits)
                                      : merged_value<false>(best, p.logits + bt * p.ld * 4, p.V_logits);
                }
            }
        }
        __syncthreads();
    }

    // Gathered source rows of this lane's DMA loads.  Rows past M, of padding
    // positions or with an out-of-range id load E row 0; the last are written
    // as zeros, the others not at all.
    const uint16_t *xsrc[XI];
    uint32_t xok = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        int64_t tok = 0;
        if (m < p.M && ((validq >> (row >> 4)) & 1u)) {
            const int32_t t = p.tk_part ? mid[row] : p.cand[m];
            if (t >= 0 && (int64_t)t < p.V) {
                tok = t;
                xok |= 1u << u;
            } else if ((lane & 7) == 0 && side == 0) {
                atomicOr(&g_device_error, 1);
            }
        }
        xsrc[u] = p.E + tok * d + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
    }
    const uint16_t *W = (side == 0 ? p.WA : p.WB) + (int64_t)n0 * d;

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const int nk = d / kBK;
    const int k0 = (int)((int64_t)nk * ks / p.nsplit), k1 = (int)((int64_t)nk * (ks + 1) / p.nsplit);
    if (k1 > k0) mma_tile_dma<T>(xsrc, W, d, k0, k1, Xs, Ws, acc);

    if (p.nsplit > 1) {
        // partial tile, row-major; validity and placement are the reduce's
        float *tp = p.part + ((int64_t)ks * p.mt * ncol + (int64_t)mt * ncol + ct) * (BM * BN);
        for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) { *(floatx4 *)(tp + rl * BN + cl) = v; });
        return;
    }

    // Epilogue.  Token validity comes from the tile's mask; which positions
    // are written from the position masks: B for every real position, A for
    // those with a successor.
    tile_row_mask<NW, XI>(xok, Xs);
    const uint32_t wq = side == 0 ? succq : validq;
    // Candidate row m = (b t) * 16 + j of side 0 becomes predecessor row j of
    // position t + 1: output row m + 16.
    float *const out = side == 0 ? p.A_prev + (int64_t)kK * r : p.B_cur;
    for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) {
        if (!((wq >> (rl >> 4)) & 1u)) return;  // padding, or no successor position
        const int64_t m = m0 + rl;
        *(floatx4 *)(out + m * r + n0 + cl) = tile_row_ok(Xs, rl) ? v : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    });
}

// Sum the K splits of the candidate job in split order, then the epilogue of
// project_cand_kernel: one thread per output element (row m, side, column n).
template <int BN>
__global__ __launch_bounds__(256) void project_cand_reduce_kernel(CandParams p) {
    constexpr int BM = 128;
    const int r = p.r;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= p.M * 2 * r) return;
    const int n = (int)(e % r);
    const int side = (int)((e / r) & 1);
    const int64_t m = e / (2 * r);
    const int ncol = 2 * p.nside;
    const int mt = (int)(m / BM), rl = (int)(m % BM);
    const int ct = side * p.nside + n / BN;
    // padding positions, and on side 0 the last position of a block, are not written
    const uint32_t bt = (uint32_t)(m / kK), b = bt / (uint32_t)p.L;
    const int pos = (int)(bt - b * (uint32_t)p.L), len = block_len_of(p.len, b, p.L);
    if (side == 0 ? pos + 1 >= len : pos >= len) return;
    const int64_t stride = (int64_t)p.mt * ncol * BM * BN;
    const float *src = p.part + ((int64_t)mt * ncol + ct) * (BM * BN) + rl * BN + (n % BN);
    float sum = 0.0f;
    for (int ks = 0; ks < p.nsplit; ++ks) sum += src[ks * stride];
    const int32_t t = p.cand[m];
    const bool ok = t >= 0 && (int64_t)t < p.V;
    if (side == 0) p.A_prev[(m + kK) * r + n] = ok ? sum : 0.0f;
    else p.B_cur[m * r + n] = ok ? sum : 0.0f;
}

// Measurement aid: the candidate job's gather alone.  Gathered rows E[cand[m]]
// go into a three-stage LDS ring through the same LDS-DMA addressing as
// project_cand_kernel (128-row tiles, chunk swizzle, waits and barriers per
// 64-deep step), with no MFMA; each thread folds its four 16-byte LDS chunks per
// step into an XOR word and stores it, so no load can be dropped.  The K range of a
// tile is split over workgroups so that about 512 of them run.  Algorithmic
// bytes: every gathered row once, M d 2.
struct GatherProbeParams {
    const uint16_t *E;
    int64_t V;
    int d;
    const int32_t *cand;
    int64_t M;       // gathered rows
    int mt, nsplit;  // 128-row tiles, K splits
    uint32_t *out;   // [grid * 256]
};

__global__ __launch_bounds__(256) void gather_probe_kernel(GatherProbeParams p) {
    constexpr int BM = 128, NW = 4, XI = BM / 8 / NW;
    __shared__ __attribute__((aligned(16))) uint16_t Xs[3 * BM * kBK];
    const int ks = (int)(blockIdx.x / p.mt), mt = (int)(blockIdx.x % p.mt);
    const int64_t m0 = (int64_t)mt * BM;
    const int d = p.d, nk = d / kBK;
    const int k0 = (int)((int64_t)nk * ks / p.nsplit), k1 = (int)((int64_t)nk * (ks + 1) / p.nsplit);
    const uint32_t lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const uint16_t *xsrc[XI];
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        int64_t tok = 0;
        if (m < p.M) {
            const int32_t t = p.cand[m];
            if (t >= 0 && (int64_t)t < p.V) tok = t;
        }
        xsrc[u] = p.E + tok * d + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
    }
    auto issue = [&](int k, int stage) {
#pragma unroll
        for (int u = 0; u < XI; ++u)
            lds_dma16(xsrc[u] + (int64_t)k * kBK, Xs + stage * BM * kBK + (8 * (wave + NW * u)) * kBK);
    };
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (k1 > k0) issue(k0, 0);
    if (k1 > k0 + 1) issue(k0 + 1, 1);
    for (int k = k0; k < k1; ++k) {
        const int st = (k - k0) % 3;
        if (k + 2 < k1) {
            issue(k + 2, (k - k0 + 2) % 3);
            wait_vmcnt<2 * XI>();  // step k landed; k+1 and k+2 may still fly
        } else {
            wait_vmcnt<0>();
        }
        wg_barrier();
#pragma unroll
        for (int j = 0; j < BM * kBK / (256 * 8); ++j)
            acc ^= *(const u32x4 *)(Xs + st * BM * kBK + (threadIdx.x + 256 * j) * 8);
        wg_barrier();  // the stage is refilled two steps later
    }
    wait_vmcnt<0>();
    p.out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

inline int gather_probe_nsplit(int64_t M, int64_t d) {
    const int64_t mt = (M + 127) / 128, nk = d / kBK;
    int64_t s = (512 + mt - 1) / mt;
    if (s > nk / 4) s = nk / 4;
    return (int)(s < 1 ? 1 : s);
}

// K splits of the candidate job: only when its tiles cannot fill the chip,
// keeping at least DSEL_CAND_MIN_STEPS K steps per split (one block of 16 at
// d 2560: 5 splits 47.8 us per step, 10 splits 48.4-49.0, 20 splits 64, 40
// splits 81; 2 to 16 blocks level between 5 and 10 splits).
#ifndef DSEL_CAND_MIN_STEPS
#define DSEL_CAND_MIN_STEPS 8
#endif
// Column tile of the candidate job: the widest that divides r and still
// gives at least 256 tiles (one per CU), else 32.  Narrow tiles re-read the
// gathered rows from L2 once per column tile but let small batches spread
// over the chip without a K split (measured at 2-32 blocks of 16 positions:
// 25-35% faster than 256-wide tiles).  With one or two row tiles the K split
// carries the parallelism and 256-wide tiles stay fastest.
inline int cand_bn(int64_t batch, int64_t block, int64_t r) {
    const int64_t rt = (batch * block * kK + 127) / 128;
    int widest = 256;
    while (widest > 32 && r % widest != 0) widest >>= 1;
    if (rt <= 2) return widest;
    for (int bn = widest; bn > 32; bn >>= 1)
        if (r % bn == 0 && rt * 2 * (r / bn) >= 256) return bn;
    return 32;
}
inline int cand_nsplit(int64_t batch, int64_t block, int64_t d, int64_t r) {
    const int64_t BN = cand_bn(batch, block, r);
    const int64_t tiles = (batch * block * kK + 127) / 128 * 2 * (r / BN);
    if (tiles >= 128) return 1;
    const int64_t nk = d / kBK;
    int64_t s = 256 / (tiles > 0 ? tiles : 1);
    if (s > nk / DSEL_CAND_MIN_STEPS) s = nk / DSEL_CAND_MIN_STEPS;
    return (int)(s < 1 ? 1 : s);
}

inline size_t cand_workspace_bytes(int64_t batch, int64_t block, int64_t d, int64_t r) {
    const int s = cand_nsplit(batch, block, d, r);
    const int64_t mt = (batch * block * kK + 127) / 128;
    return s > 1 ? (size_t)s * (size_t)mt * 128 * 2 * (size_t)r * sizeof(float) : 0;
}

#ifndef DSEL_GATE_STAGES
#define DSEL_GATE_STAGES 3
#endif

struct GateParams {
    const uint16_t *E;
    int64_t V;
    int d, r;
    const uint16_t *WA, *WH, *h;
    const int32_t *ver;
    int B, L;
    const int32_t *len;  // ragged batch: valid positions per block (nullptr: all L)
    float *A_prev, *G;
    // A(verified_b) goes to A_ver + b * ver_stride; with ver_zero the 15 rows
    // after it (position 0's unused predecessor rows of A_prev) are zeroed.
    // The separate calls point A_ver at A_prev (stride L * 16 * r, zeroing);
    // the fused selector at a compact [B][r] buffer.
    float *A_ver;
    int64_t ver_stride;
    bool ver_zero;
    float *part;        // [nsplit][rows_gate + rows_ver][r] partial sums (nsplit > 1)
    int mt_gate, mt_ver, nside, nsplit;  // 128-row tiles of each job, column tiles, K splits
};

// Rows of the gate job: 0 .. B*L-1 are h rows (W = W_H); then B verified
// tokens (X = E[verified], W = W_A).  Tile 128 x BN on the direct-to-LDS
// pipeline; the K range is split nsplit ways across workgroups so that this
// small GEMM (M = batch*block) still fills the chip.  With nsplit == 1 the
// epilogue is applied here; otherwise the partial tile is stored and
// project_gate_reduce_kernel sums the splits in a fixed order.
// Stages of the gate GEMM's LDS ring.  Deeper rings (4 and 6 stages for the
// narrow tiles, 4 for the 128-wide ones) measured the same at 64-256 blocks
// and within noise at one block, so the default stays at three.
template <int BN>
constexpr int gate_stages() { return BN >= 256 ? 3 : DSEL_GATE_STAGES; }

// The work of workgroup `bid` of the gate job.
template <int BN>
__device__ __forceinline__ void gate_gemm_block(const GateParams &p, int bid) {
    constexpr int BM = 128;
    using T = CandTile<BN>;
    constexpr int NW = T::NW;
    constexpr int XI = T::DXI;
    constexpr int NSG = gate_stages<BN>();
    __shared__ __attribute__((aligned(16))) uint16_t Xs[NSG * BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[NSG * BN * kBK];

    const int tiles = (p.mt_gate + p.mt_ver) * p.nside;
    const int ks = bid / tiles;
    const int tw = bid % tiles;
    const bool gate = tw < p.mt_gate * p.nside;
    const int tt = gate ? tw : tw - p.mt_gate * p.nside;
    const int64_t m0 = (int64_t)(tt / p.nside) * BM;
    const int n0 = (tt % p.nside) * BN;
    const int64_t M = gate ? (int64_t)p.B * p.L : (int64_t)p.B;
    const int d = p.d, r = p.r;
    const int nk = d / kBK;
    const int k0 = (int)((int64_t)nk * ks / p.nsplit), k1 = (int)((int64_t)nk * (ks + 1) / p.nsplit);
    const uint32_t lane = lane_id();
    const int wave = threadIdx.x >> 6;

    // Rows past M and rows of padding positions (gate: t >= length; verified
    // token: an empty block) load h row 0 and are never written.
    const uint16_t *xsrc[XI];
    uint32_t xok = 0, xlive = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        const uint16_t *base = p.h;
        bool live = m < M;
        if (live && p.len) live = gate ? position_live(p.len, (uint32_t)m, p.L) : block_len_of(p.len, m, p.L) > 0;
        if (live) {
            xlive |= 1u << u;
            if (gate) {
                base = p.h + m * d;
                xok |= 1u << u;
            } else {
                const int32_t t = p.ver[m];
                const bool ok = t >= 0 && (int64_t)t < p.V;
                base = p.E + (int64_t)(ok ? t : 0) * d;
                if (ok) xok |= 1u << u;
                else if ((lane & 7) == 0 && ks == 0 && n0 == 0) atomicOr(&g_device_error, 1);
            }
        }
        xsrc[u] = base + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
    }
    const uint16_t *W = (gate ? p.WH : p.WA) + (int64_t)n0 * d;
    // a tile of padding only has nothing to write (ragged batches)
    if (p.len && !__syncthreads_or(xlive != 0)) return;

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if (k1 > k0) mma_tile_dma<T, NSG>(xsrc, W, d, k0, k1, Xs, Ws, acc);

    tile_row_mask<NW, XI>(xok, Xs, xlive);
    const int64_t rows_all = (int64_t)p.B * p.L + p.B;
    for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) {
        if (!tile_row_live(Xs, rl)) return;
        const int64_t m = m0 + rl;
        if (!tile_row_ok(Xs, rl)) v = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        const int n = n0 + cl;
        if (p.nsplit > 1) {
            const int64_t row = gate ? m : (int64_t)p.B * p.L + m;
            *(floatx4 *)(p.part + ((int64_t)ks * rows_all + row) * r + n) = v;
        } else if (gate) {
            floatx4 gv;
#pragma unroll
            for (int e = 0; e < 4; ++e) gv[e] = 1.0f / (1.0f + expf(-v[e]));
            *(floatx4 *)(p.G + m * r + n) = gv;
        } else {
            float *base = p.A_ver + m * p.ver_stride + n;
            *(floatx4 *)base = v;
            if (p.ver_zero)
                for (int z = 1; z < kK; ++z) *(floatx4 *)(base + (int64_t)z * r) = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    });
}

template <int BN>
__global__ __launch_bounds__(CandTile<BN>::NT) void project_gate_kernel(GateParams p) {
    gate_gemm_block<BN>(p, blockIdx.x);
}

// Sum the K splits of the gate job in split order, then the epilogue, for
// output elements 4u .. 4u + 3 (row 4u / r, columns 4u % r ..; r % 4 == 0):
// 16-byte loads, with every split's load in flight before the sums.
__device__ __forceinline__ void gate_reduce_unit(const GateParams &p, int64_t u) {
    const int64_t rows_all = (int64_t)p.B * p.L + p.B;
    const int64_t e = 4 * u;
    if (e >= rows_all * p.r) return;
    const int64_t row = e / p.r;
    const int n = (int)(e % p.r);
    if (p.len) {  // padding positions and empty blocks: nothing to write
        const bool gate = row < (int64_t)p.B * p.L;
        if (gate ? !position_live(p.len, (uint32_t)row, p.L) : block_len_of(p.len, row - (int64_t)p.B * p.L, p.L) == 0)
            return;
    }
    const float *src = p.part + row * p.r + n;
    const int64_t stride = rows_all * p.r;
    floatx4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < p.nsplit; k0 += 8) {
        floatx4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k0 + k < p.nsplit) v[k] = *(const floatx4 *)(src + (k0 + k) * stride);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k0 + k < p.nsplit) sum += v[k];
    }
    if (row < (int64_t)p.B * p.L) {
        floatx4 g;
#pragma unroll
        for (int i = 0; i < 4; ++i) g[i] = 1.0f / (1.0f + expf(-sum[i]));
        *(floatx4 *)(p.G + row * p.r + n) = g;
    } else {
        const int64_t b = row - (int64_t)p.B * p.L;
        float *base = p.A_ver + b * p.ver_stride + n;
        *(floatx4 *)base = sum;
        if (p.ver_zero)
            for (int z = 1; z < kK; ++z) *(floatx4 *)(base + (int64_t)z * p.r) = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
}

__global__ __launch_bounds__(256) void project_gate_reduce_kernel(GateParams p) {
    gate_reduce_unit(p, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Column tile and K splits of the gate job (M = batch*block + batch rows, a
// short GEMM).  Few row tiles (up to 16, e.g. 64 x 16 positions): 64-wide
// column tiles and splits of at least 10 K steps; more: 128-wide tiles and
// splits of at least 8 steps; in both cases about 256 workgroups.  Measured
// on MI355X: 64 x 16 positions, d 2560: 14 us (against 20 us for 256-wide
// tiles split 10 ways); 256 x 16, d 6144: 35 us.  The column tile is the
// largest of 256, 128, 64, 32 that divides r and is at most that width.
inline int gate_row_tiles(int64_t batch, int64_t block) {
    return (int)((batch * block + 127) / 128 + (batch + 127) / 128);
}
// Column tile of the gate job, narrower for fewer row tiles (measured: 32 up
// to 4 row tiles, 64 up to 16, 128 beyond).
inline int gate_bn(int64_t batch, int64_t block, int64_t r) {
    const int rt = gate_row_tiles(batch, block);
    const int cap = rt <= 4 ? 32 : rt <= 16 ? 64 : 128;
    for (int bn = 256; bn > 32; bn >>= 1)
        if (bn <= cap && r % bn == 0) return bn;
    return 32;
}
#ifndef DSEL_GATE_MIN_STEPS_NARROW
#define DSEL_GATE_MIN_STEPS_NARROW 10
#endif
#ifndef DSEL_GATE_MIN_STEPS_WIDE
#define DSEL_GATE_MIN_STEPS_WIDE 8
#endif
#ifndef DSEL_GATE_TARGET_WG
#define DSEL_GATE_TARGET_WG 256
#endif
inline int gate_nsplit(int64_t batch, int64_t block, int64_t d, int64_t r) {
    const int64_t BN = gate_bn(batch, block, r);
    const int64_t tiles = (int64_t)gate_row_tiles(batch, block) * (r / BN);
    const int64_t nk = d / kBK;
    const int64_t min_steps = BN <= 64 ? DSEL_GATE_MIN_STEPS_NARROW : DSEL_GATE_MIN_STEPS_WIDE;
    int64_t s = DSEL_GATE_TARGET_WG / (tiles > 0 ? tiles : 1);
    if (s > nk / min_steps) s = nk / min_steps;
    if (s < 1) s = 1;
    return (int)s;
}

inline size_t gate_workspace_bytes(int64_t batch, int64_t block, int64_t d, int64_t r) {
    const int s = gate_nsplit(batch, block, d, r);
    return s > 1 ? (size_t)s * (size_t)(batch * block + batch) * (size_t)r * sizeof(float) : 0;
}

}  // namespace dsel
