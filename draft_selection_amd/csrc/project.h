// project: the compact token vectors A(x) = W_A E[x], B(x) = W_B E[x] of every
// candidate and predecessor, and the context gate G = sigmoid(W_H h_t).
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector, the
// paragraph after eq. S_t: A and B map tokens to 256-d vectors, H(h_t) gates
// them.)
//
// One launch, three jobs of C[m, n] = sum_k X[m, k] W[n, k] on bf16 MFMA with
// fp32 accumulation:
//   CAND  X row m = E[cand_id[m]] (m over batch*block*16), W = [W_A; W_B]
//         (N = 2r): one gathered row feeds both projections.  The A half of
//         candidate (b, t, j) is the predecessor row j of position t + 1.
//   VER   X row b = E[verified[b]], W = W_A: predecessor row 0 of position 0
//         (rows 1..15 of position 0 are written as zeros).
//   GATE  X row m = h[m] (m over batch*block), W = W_H, sigmoid epilogue.
// Tiles are BM x BN with a 64-deep K step, double-buffered through LDS with the
// 16-byte chunks of every row XOR-swizzled by (row & 7) so that the MFMA
// fragment reads are bank-conflict free.  Four waves per workgroup in a 2 x 2
// arrangement; each wave owns (BM/2) x (BN/2) of the tile as 16 x 16 MFMA
// blocks (v_mfma_f32_16x16x32_bf16).  The N tiles of one row tile are placed
// on the same XCD (workgroup ids congruent mod 8) so the gathered rows are
// fetched from HBM once and re-read from that XCD's L2.
#pragma once

#include "common.h"

namespace dsel {

enum { JOB_CAND = 0, JOB_VER = 1, JOB_GATE = 2 };

struct ProjParams {
    const uint16_t *E;
    int64_t V;
    int d, r;
    const uint16_t *WA, *WB, *WH, *h;
    const int32_t *cand, *ver;
    int B, L;
    float *A_prev, *B_cur, *G;
    // tile grid of every job; rows are M, columns N
    int64_t m_cand, m_ver, m_gate;
    int mt_cand, nt_cand, mt_ver, nt_ver, mt_gate, nt_gate;
    int mt_cand_pad;     // mt_cand rounded up to a multiple of 8
    int64_t wg_cand, wg_ver;  // workgroup id ranges: [0, wg_cand) cand, then ver, then gate
};

constexpr int kBK = 64;  // K elements per LDS stage (128 bytes per row)

// Element offset of 16-byte chunk `ch` (0..7) of tile row `row` in LDS.
__device__ __forceinline__ int lds_off(int row, int ch) { return row * kBK + ((ch ^ (row & 7)) << 3); }

template <int BM, int BN>
__global__ __launch_bounds__(256) void project_kernel(ProjParams p) {
    constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
    constexpr int TM = WM / 16, TN = WN / 16; // MFMA blocks per wave
    constexpr int XL = BM * 8 / 256;          // X chunks loaded per thread per stage
    constexpr int WL = BN * 8 / 256;          // W chunks loaded per thread per stage
    static_assert(XL >= 1 && WL >= 1 && TM >= 1 && TN >= 1, "tile too small");

    __shared__ __attribute__((aligned(16))) uint16_t Xs[2][BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * kBK];

    // ---- which job and tile ------------------------------------------------
    int64_t wg = blockIdx.x;
    int job, mt, nt;
    if (wg < p.wg_cand) {
        // XCD-aware: ids i and i + 8k share an XCD; give them the N tiles of one
        // row tile.
        int64_t xcd = wg & 7, slot = wg >> 3;
        nt = (int)(slot % p.nt_cand);
        mt = (int)((slot / p.nt_cand) * 8 + xcd);
        job = JOB_CAND;
        if (mt >= p.mt_cand) return;
    } else if (wg < p.wg_cand + p.wg_ver) {
        wg -= p.wg_cand;
        job = JOB_VER;
        mt = (int)(wg / p.nt_ver);
        nt = (int)(wg % p.nt_ver);
    } else {
        wg -= p.wg_cand + p.wg_ver;
        job = JOB_GATE;
        mt = (int)(wg / p.nt_gate);
        nt = (int)(wg % p.nt_gate);
        if (mt >= p.mt_gate) return;
    }
    const int64_t M = job == JOB_CAND ? p.m_cand : job == JOB_VER ? p.m_ver : p.m_gate;
    const int64_t m0 = (int64_t)mt * BM;
    const int n0 = nt * BN;
    const int d = p.d, r = p.r;
    const int tid = threadIdx.x;

    // ---- per-thread source rows --------------------------------------------
    // Thread tid loads chunk (tid & 7) of tile rows (tid >> 3) + 32 i.
    const int ch = tid & 7;
    const uint16_t *xrow[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
        int64_t m = m0 + (tid >> 3) + 32 * i;
        const uint16_t *src = nullptr;
        if (m < M) {
            if (job == JOB_GATE) {
                src = p.h + m * d;
            } else {
                int32_t tok = job == JOB_CAND ? p.cand[m] : p.ver[m];
                if (tok >= 0 && (int64_t)tok < p.V) src = p.E + (int64_t)tok * d;
                else if (ch == 0) atomicOr(&g_device_error, 1);
            }
        }
        xrow[i] = src;
    }
    const uint16_t *wrow[WL];
#pragma unroll
    for (int i = 0; i < WL; ++i) {
        int n = n0 + (tid >> 3) + 32 * i;
        const uint16_t *w;
        if (job == JOB_CAND) w = n < r ? p.WA + (int64_t)n * d : p.WB + (int64_t)(n - r) * d;
        else if (job == JOB_VER) w = p.WA + (int64_t)n * d;
        else w = p.WH + (int64_t)n * d;
        wrow[i] = w;
    }

    u32x4 xr[XL], wr[WL];
#define DSEL_GLOAD(k0)                                                                           \
    do {                                                                                         \
        _Pragma("unroll") for (int i = 0; i < XL; ++i) xr[i] =                                   \
            xrow[i] ? *(const u32x4 *)(xrow[i] + (k0) + ch * 8) : u32x4{0u, 0u, 0u, 0u};    \
        _Pragma("unroll") for (int i = 0; i < WL; ++i) wr[i] = *(const u32x4 *)(wrow[i] + (k0) + ch * 8); \
    } while (0)
#define DSEL_LSTORE(buf)                                                                         \
    do {                                                                                         \
        _Pragma("unroll") for (int i = 0; i < XL; ++i)                                           \
            *(u32x4 *)(&Xs[buf][lds_off((tid >> 3) + 32 * i, ch)]) = xr[i];                      \
        _Pragma("unroll") for (int i = 0; i < WL; ++i)                                           \
            *(u32x4 *)(&Ws[buf][lds_off((tid >> 3) + 32 * i, ch)]) = wr[i];                      \
    } while (0)

    const uint32_t lane = lane_id();
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int fr = lane & 15;        // fragment row (A) / column (B)
    const int fk = lane >> 4;        // which 8-element K group of the 32

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nk = d / kBK;
    DSEL_GLOAD(0);
    DSEL_LSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) DSEL_GLOAD((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                a[i] = *(const bf16x8 *)(&Xs[buf][lds_off(wm * WM + i * 16 + fr, kk * 4 + fk)]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                b[j] = *(const bf16x8 *)(&Ws[buf][lds_off(wn * WN + j * 16 + fr, kk * 4 + fk)]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) DSEL_LSTORE(buf ^ 1);
        __syncthreads();
    }

#undef DSEL_GLOAD
#undef DSEL_LSTORE

    // ---- epilogue ------------------------------------------------------------
    // acc[i][j][v] is C[row, col] with row = wm*WM + 16 i + 4 (lane >> 4) + v,
    // col = wn*WN + 16 j + (lane & 15).
    const int K16 = kK;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t m = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + v;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn * WN + j * 16 + (int)(lane & 15);
                const float val = acc[i][j][v];
                if (job == JOB_CAND) {
                    const int64_t bt = m / K16;
                    const int slot = (int)(m % K16);
                    if (n < r) {
                        if ((bt % p.L) + 1 < p.L) p.A_prev[((bt + 1) * K16 + slot) * r + n] = val;
                    } else {
                        p.B_cur[(bt * K16 + slot) * r + (n - r)] = val;
                    }
                } else if (job == JOB_VER) {
                    float *base = p.A_prev + (m * p.L * K16) * r + n;
                    base[0] = val;
#pragma unroll
                    for (int z = 1; z < K16; ++z) base[(int64_t)z * r] = 0.0f;
                } else {
                    p.G[m * r + n] = 1.0f / (1.0f + expf(-val));
                }
            }
        }
}

}  // namespace dsel
