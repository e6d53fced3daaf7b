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
// Main loop (mma_tile_dma): a K step is 64 deep (128 bytes of every row).
// Tiles move from global memory straight into a three-stage LDS ring
// (global_load_lds_dwordx4, no staging registers), two steps ahead of the
// MFMAs.  In LDS the 16-byte chunks of each row are XOR-swizzled by (row & 7)
// so the fragment reads are bank-conflict free.  The waves of a workgroup form
// a GM x GN grid, each owning (BM/GM) x (BN/GN) of the tile as 32 x 32 MFMA
// blocks.
#pragma once

#include "common.h"

namespace dsel {

constexpr int kBK = 64;  // K elements per step (128 bytes per row)

// Element offset of 16-byte chunk `ch` (0..7) of tile row `row` in one buffer.
__device__ __forceinline__ int lds_off(int row, int ch) { return row * kBK + ((ch ^ (row & 7)) << 3); }

// BM x BN tile computed by GM x GN waves, each owning WM x WN as 32 x 32 MFMA
// blocks (v_mfma_f32_32x32x16_bf16: one wave keeps the matrix core near its
// peak, which the 16 x 16 shape does not).
template <int BM, int BN, int GM, int GN>
struct TileShape {
    static constexpr int BMv = BM, BNv = BN, GMv = GM, GNv = GN;
    static constexpr int NT = 64 * GM * GN;                // threads
    static constexpr int NW = GM * GN;                     // waves
    static constexpr int WM = BM / GM, WN = BN / GN;       // wave tile
    static constexpr int TM = WM / 32, TN = WN / 32;       // MFMA blocks per wave
    static constexpr int DXI = BM / 8 / NW, DWI = BN / 8 / NW;  // LDS-DMA loads per wave per step
    static_assert(TM >= 1 && TN >= 1 && DXI >= 1 && DWI >= 1, "tile shape");
};

// ---- direct-to-LDS pipeline --------------------------------------------------
// global_load_lds_dwordx4 moves 16 bytes per lane from global memory straight
// into LDS (64 lanes fill 1 KB = 8 tile rows of 128 bytes), so no registers
// stage the tiles.  A ring of three LDS stages holds steps k, k+1, k+2 while
// step k computes.  Waits are explicit: `s_waitcnt vmcnt(n)` with n = the
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
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(m0v)), "v"(src)
                 : "memory", "m0");
}

// acc += X * W^T over K steps [k0, k1) (64-deep steps).
template <class T>
__device__ __forceinline__ void mma_tile_dma(const uint16_t *const (&xsrc)[T::DXI], const uint16_t *wbase,
                                             int64_t wstride, int k0, int k1, uint16_t *Xs,
                                             uint16_t *Ws, floatx16 (&acc)[T::TM][T::TN]) {
    constexpr int BM = T::BMv, BN = T::BNv, NW = T::NW;
    constexpr int XI = T::DXI, WI = T::DWI;
    static_assert(XI >= 1 && WI >= 1 && XI * NW * 8 == BM && WI * NW * 8 == BN, "DMA tile shape");
    constexpr int PER = XI + WI;  // loads per wave per step
    constexpr int NS = 3;
    const int tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const int wave = tid >> 6;
    const int wm = wave / T::GNv, wn = wave % T::GNv;
    const int fr = lane & 31, fk = lane >> 5;  // fragment row / column, 8-element K half
    // this lane's W source rows 8 (wave + NW u) + lane / 8; physical chunk
    // lane % 8 of row `row` holds logical chunk (lane % 8) ^ (row & 7).
    const int lrow = (int)(lane >> 3), pch = (int)(lane & 7);
    const uint16_t *wsrc[WI];
#pragma unroll
    for (int u = 0; u < WI; ++u) {
        const int row = 8 * (wave + NW * u) + lrow;
        wsrc[u] = wbase + (int64_t)row * wstride + ((pch ^ (row & 7)) << 3);
    }
#define DSEL_ISSUE(k, stage)                                                                   \
    do {                                                                                       \
        const int kk_ = ((k) < k1 ? (k) : k1 - 1) * kBK;                                       \
        _Pragma("unroll") for (int u = 0; u < XI; ++u)                                         \
            lds_dma16(xsrc[u] + kk_, Xs + (stage) * BM * kBK + (8 * (wave + NW * u)) * kBK);   \
        _Pragma("unroll") for (int u = 0; u < WI; ++u)                                         \
            lds_dma16(wsrc[u] + kk_, Ws + (stage) * BN * kBK + (8 * (wave + NW * u)) * kBK);   \
    } while (0)

    DSEL_ISSUE(k0, 0);
    DSEL_ISSUE(k0 + 1, 1);
    int cur = 0;
    for (int kt = k0; kt < k1; ++kt) {
        wait_vmcnt<PER>();  // this wave's loads of step kt have landed
        wg_barrier();       // ... everyone's have, and step kt-1 is no longer read
        DSEL_ISSUE(kt + 2, cur == 0 ? 2 : cur - 1);
        const uint16_t *xb = Xs + cur * BM * kBK;
        const uint16_t *wb = Ws + cur * BN * kBK;
        // fragments of K slice kk+1 are read while slice kk multiplies
        bf16x8 a[2][T::TM], b[2][T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) a[0][i] = *(const bf16x8 *)(xb + lds_off(wm * T::WM + i * 32 + fr, fk));
#pragma unroll
        for (int j = 0; j < T::TN; ++j) b[0][j] = *(const bf16x8 *)(wb + lds_off(wn * T::WN + j * 32 + fr, fk));
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int c = kk & 1, n = c ^ 1;
            if (kk + 1 < kBK / 16) {
#pragma unroll
                for (int i = 0; i < T::TM; ++i)
                    a[n][i] = *(const bf16x8 *)(xb + lds_off(wm * T::WM + i * 32 + fr, (kk + 1) * 2 + fk));
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    b[n][j] = *(const bf16x8 *)(wb + lds_off(wn * T::WN + j * 32 + fr, (kk + 1) * 2 + fk));
            }
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
        }
        cur = cur == NS - 1 ? 0 : cur + 1;
    }
    wait_vmcnt<0>();  // drain the redundant tail loads before LDS is released
#undef DSEL_ISSUE
}

struct CandParams {
    const uint16_t *E;
    int64_t V;
    int d, r;
    const uint16_t *WA, *WB;
    const int32_t *cand;
    int L;
    int64_t M;        // batch * block * 16 gathered rows
    int mt, mt_pad;   // row tiles (mt_pad: rounded up to a multiple of 8)
    int nside;        // column tiles per side (r / BN)
    float *A_prev, *B_cur;
};

// Column tile BN of one side on 4 waves: 2 x 2 (wave tile 64 x BN/2), or 4 x 1
// when BN = 32.
#ifndef DSEL_CAND_GN256
#define DSEL_CAND_GN256 4
#endif
template <int BN>
using CandTile = TileShape<128, BN, (BN == 32 ? 4 : 2), (BN == 32 ? 1 : BN == 256 ? DSEL_CAND_GN256 : 2)>;

template <int BN>
__global__ __launch_bounds__(CandTile<BN>::NT) void project_cand_kernel(CandParams p) {
    constexpr int BM = 128;
    using T = CandTile<BN>;
    constexpr int NW = T::NW;
    constexpr int XI = T::DXI;
    __shared__ __attribute__((aligned(16))) uint16_t Xs[3 * BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[3 * BN * kBK];

    // XCD-aware tile order: workgroups w and w + 8 share an XCD; consecutive
    // slots of one XCD take the column tiles of one row tile.
    const int w = blockIdx.x;
    const int xcd = w & 7, slot = w >> 3;
    const int ncol = 2 * p.nside;
    const int ct = slot % ncol;
    const int mt = (slot / ncol) * 8 + xcd;
    if (mt >= p.mt) return;
    const int side = ct / p.nside;  // 0: W_A, 1: W_B
    const int n0 = (ct % p.nside) * BN;
    const int64_t m0 = (int64_t)mt * BM;
    const int tid = threadIdx.x;
    const int d = p.d, r = p.r;
    const uint32_t lane = lane_id();
    const int wave = tid >> 6;

    // Gathered source rows of this lane's DMA loads.  Rows past M or with an
    // out-of-range id load E row 0 and are written as zeros.
    const uint16_t *xsrc[XI];
    uint32_t xok = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        int64_t tok = 0;
        if (m < p.M) {
            const int32_t t = p.cand[m];
            if (t >= 0 && (int64_t)t < p.V) {
                tok = t;
                xok |= 1u << u;
            } else if ((lane & 7) == 0 && side == 0) {
                atomicOr(&g_device_error, 1);
            }
        }
        xsrc[u] = p.E + tok * d + (((lane & 7) ^ (row & 7)) << 3);
    }
    const uint16_t *W = (side == 0 ? p.WA : p.WB) + (int64_t)n0 * d;

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    mma_tile_dma<T>(xsrc, W, d, 0, d / kBK, Xs, Ws, acc);

    // Row validity for the epilogue, through LDS (a global re-load per row
    // would put one memory round trip per output row on the critical path).
    __syncthreads();
    uint8_t *rowok = (uint8_t *)Xs;
    if ((lane & 7) == 0) {
#pragma unroll
        for (int u = 0; u < XI; ++u) rowok[8 * (wave + NW * u) + (lane >> 3)] = (xok >> u) & 1u;
    }
    __syncthreads();

    // acc[i][j][e] = C[row, col]: row = wm*WM + 32 i + 8 (e / 4) + 4 (lane / 32)
    // + e % 4, col = wn*WN + 32 j + lane % 32.
    const int wm = wave / T::GNv, wn = wave % T::GNv;
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rl = wm * T::WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int64_t m = m0 + rl;
            if (m >= p.M) continue;
            const bool ok = rowok[rl] != 0;
            const int64_t bt = m / kK;
            const int slotj = (int)(m % kK);
            float *dst;
            if (side == 0) {
                if ((bt % p.L) + 1 >= p.L) continue;  // the last position has no successor
                dst = p.A_prev + ((bt + 1) * kK + slotj) * r;
            } else {
                dst = p.B_cur + (bt * kK + slotj) * r;
            }
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                dst[n0 + wn * T::WN + j * 32 + (lane & 31)] = ok ? acc[i][j][v] : 0.0f;
        }
}

struct GateParams {
    const uint16_t *E;
    int64_t V;
    int d, r;
    const uint16_t *WA, *WH, *h;
    const int32_t *ver;
    int B, L;
    float *A_prev, *G;
    float *part;        // [nsplit][rows_gate + rows_ver][r] partial sums (nsplit > 1)
    int mt_gate, mt_ver, nside, nsplit;  // 128-row tiles of each job, column tiles, K splits
};

// Rows of the gate job: 0 .. B*L-1 are h rows (W = W_H); then B verified
// tokens (X = E[verified], W = W_A).  Tile 128 x BN on the direct-to-LDS
// pipeline; the K range is split nsplit ways across workgroups so that this
// small GEMM (M = batch*block) still fills the chip.  With nsplit == 1 the
// epilogue is applied here; otherwise the partial tile is stored and
// project_gate_reduce_kernel sums the splits in a fixed order.
template <int BN>
__global__ __launch_bounds__(CandTile<BN>::NT) void project_gate_kernel(GateParams p) {
    constexpr int BM = 128;
    using T = CandTile<BN>;
    constexpr int NW = T::NW;
    constexpr int XI = T::DXI;
    __shared__ __attribute__((aligned(16))) uint16_t Xs[3 * BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[3 * BN * kBK];

    const int tiles = (p.mt_gate + p.mt_ver) * p.nside;
    const int ks = blockIdx.x / tiles;
    const int tw = blockIdx.x % tiles;
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

    const uint16_t *xsrc[XI];
    uint32_t xok = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        const uint16_t *base = p.h;  // rows past M load h row 0 and are never written
        if (m < M) {
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
        xsrc[u] = base + (((lane & 7) ^ (row & 7)) << 3);
    }
    const uint16_t *W = (gate ? p.WH : p.WA) + (int64_t)n0 * d;

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if (k1 > k0) mma_tile_dma<T>(xsrc, W, d, k0, k1, Xs, Ws, acc);

    __syncthreads();
    uint8_t *rowok = (uint8_t *)Xs;
    if ((lane & 7) == 0) {
#pragma unroll
        for (int u = 0; u < XI; ++u) rowok[8 * (wave + NW * u) + (lane >> 3)] = (xok >> u) & 1u;
    }
    __syncthreads();

    const int wm = wave / T::GNv, wn = wave % T::GNv;
    const int64_t rows_all = (int64_t)p.B * p.L + p.B;
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rl = wm * T::WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            const int64_t m = m0 + rl;
            if (m >= M) continue;
            const bool ok = rowok[rl] != 0;
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                const int n = n0 + wn * T::WN + j * 32 + (int)(lane & 31);
                const float val = ok ? acc[i][j][v] : 0.0f;
                if (p.nsplit > 1) {
                    const int64_t row = gate ? m : (int64_t)p.B * p.L + m;
                    p.part[((int64_t)ks * rows_all + row) * r + n] = val;
                } else if (gate) {
                    p.G[m * r + n] = 1.0f / (1.0f + expf(-val));
                } else {
                    float *base = p.A_prev + (m * p.L * kK) * r + n;
                    base[0] = val;
#pragma unroll
                    for (int z = 1; z < kK; ++z) base[(int64_t)z * r] = 0.0f;
                }
            }
        }
}

// Sum the K splits of the gate job in split order, then the epilogue.
__global__ __launch_bounds__(256) void project_gate_reduce_kernel(GateParams p) {
    const int64_t rows_all = (int64_t)p.B * p.L + p.B;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= rows_all * p.r) return;
    const int64_t row = e / p.r;
    const int n = (int)(e % p.r);
    float sum = 0.0f;
    for (int ks = 0; ks < p.nsplit; ++ks) sum += p.part[((int64_t)ks * rows_all + row) * p.r + n];
    if (row < (int64_t)p.B * p.L) {
        p.G[row * p.r + n] = 1.0f / (1.0f + expf(-sum));
    } else {
        const int64_t b = row - (int64_t)p.B * p.L;
        float *base = p.A_prev + (b * p.L * kK) * p.r + n;
        base[0] = sum;
        for (int z = 1; z < kK; ++z) base[(int64_t)z * p.r] = 0.0f;
    }
}

// K splits of the gate job and the workspace they need.
#ifndef DSEL_GATE_MIN_STEPS
#define DSEL_GATE_MIN_STEPS 4
#endif
inline int gate_nsplit(int64_t batch, int64_t block, int64_t d, int64_t r) {
    const int64_t BN = r % 256 == 0 ? 256 : r % 128 == 0 ? 128 : r % 64 == 0 ? 64 : 32;
    const int64_t tiles = ((batch * block + 127) / 128 + (batch + 127) / 128) * (r / BN);
    const int64_t nk = d / kBK;
    int64_t s = 256 / (tiles > 0 ? tiles : 1);
    if (s > nk / DSEL_GATE_MIN_STEPS) s = nk / DSEL_GATE_MIN_STEPS;
    if (s < 1) s = 1;
    return (int)s;
}

inline size_t gate_workspace_bytes(int64_t batch, int64_t block, int64_t d, int64_t r) {
    const int s = gate_nsplit(batch, block, d, r);
    return s > 1 ? (size_t)s * (size_t)(batch * block + batch) * (size_t)r * sizeof(float) : 0;
}

}  // namespace dsel
