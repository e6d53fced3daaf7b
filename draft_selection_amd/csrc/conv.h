// dyn_conv: the dynamic two-tap short convolution of the drafter.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Local Convolution,
// eq. Conv_k; "DFlash 2: The Drafter Stopped Guessing Alone", section "The decay
// at the end of the block".)  Over the positions of each drafted block,
//     y_t = k_{t,0} (.) x_t + k_{t,1} (.) x_{t-1},
//     k_{t,j}[c] = base[j][c] + corr_t[j G + c / 16],  corr_t = W_c x_t,
// G = d / 16 correction groups per tap; position 0 reads the last verified
// token's representation x_prev[b].
//
// Two kernels:
//   conv_corr_kernel   corr = X W_c^T for all B L positions (N = 2 G columns),
//       on the MFMA tile machinery of project.h (128 rows x 64 or 256
//       columns, bf16 MFMA, fp32 accumulation).  The GEMM is short (B L rows), so K = d is
//       split over workgroups and each split writes its own fp32 partial
//       [split][B L][2 G] (a few MB).
//   conv_apply_kernel  one workgroup per position: sums the position's
//       partial corrections in split order (deterministic) into LDS, then
//       both taps in fp32 for 8 channels per thread, rounded to bf16 (nearest
//       even); 16-byte loads of x_t, x_{t-1} and the two base rows, one
//       16-byte store.
#pragma once

#include "project.h"

namespace dsel {

struct ConvParams {
    const uint16_t *x, *x_prev, *base, *W_c;
    uint16_t *y;
    int B, L, d;
    const int32_t *len;  // ragged batch: valid positions per block (nullptr: all L)
    int64_t M;     // B L positions
    int N;         // 2 G correction columns
    int mt, nt;    // 128-row tiles, column tiles
    int nsplit;    // K splits
    float *part;   // [nsplit][M][N]
};

// Column tile of the correction GEMM: 256 (8 waves, wave tile 64 x 64) when
// N allows it and there are at least 64 such tiles, else 64 (4 waves, wave
// tile 64 x 32) for more workgroups on short GEMMs.
inline int conv_bn(int64_t M, int64_t N) {
    return (N % 256 == 0 && (M + 127) / 128 * (N / 256) >= 64) ? 256 : 64;
}

template <int BN>
__global__ __launch_bounds__(CandTile<BN>::NT) void conv_corr_kernel(ConvParams p) {
    constexpr int BM = 128;
    using T = CandTile<BN>;
    constexpr int NW = T::NW, XI = T::DXI;
    __shared__ __attribute__((aligned(16))) uint16_t Xs[3 * BM * kBK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[3 * BN * kBK];

    const int tiles = p.mt * p.nt;
    const int ks = blockIdx.x / tiles;
    const int tw = blockIdx.x % tiles;
    const int64_t m0 = (int64_t)(tw / p.nt) * BM;
    const int n0 = (tw % p.nt) * BN;
    const int d = p.d;
    const int nk = d / kBK;
    const int k0 = (int)((int64_t)nk * ks / p.nsplit), k1 = (int)((int64_t)nk * (ks + 1) / p.nsplit);
    const uint32_t lane = lane_id();
    const int wave = threadIdx.x >> 6;

    // rows past M and padding positions load row 0 and are never stored
    const uint16_t *xsrc[XI];
    uint32_t xlive = 0;
#pragma unroll
    for (int u = 0; u < XI; ++u) {
        const int row = 8 * (wave + NW * u) + (int)(lane >> 3);
        const int64_t m = m0 + row;
        const bool live = m < p.M && position_live(p.len, (uint32_t)m, p.L);
        if (live) xlive |= 1u << u;
        xsrc[u] = p.x + (live ? m : 0) * d + (((lane & 7) ^ ((row >> 1) & 7)) << 3);
    }
    // a tile of padding only has nothing to store (ragged batches)
    if (p.len && !__syncthreads_or(xlive != 0)) return;
    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if (k1 > k0) mma_tile_dma<T>(xsrc, p.W_c + (int64_t)n0 * d, d, k0, k1, Xs, Ws, acc);

    float *out = p.part + (int64_t)ks * p.M * p.N;
    if (p.len) tile_row_mask<NW, XI>(xlive, Xs, xlive);  // workgroup-uniform branch
    for_tile_rows4<T>(acc, [&](int rl, int cl, floatx4 v) {
        const int64_t m = m0 + rl;
        if (p.len ? tile_row_live(Xs, rl) : m < p.M) *(floatx4 *)(out + m * p.N + n0 + cl) = v;
    });
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (b >> 16) | 0x40u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// One workgroup per position m: first the row's 2 G corrections, summed over
// the splits in order into LDS (coalesced loads of the partial rows), then
// 8 channels per thread and step.
__global__ __launch_bounds__(256) void conv_apply_kernel(ConvParams p) {
    extern __shared__ float corr[];  // [N]
    const int64_t m = blockIdx.x;
    if (!position_live(p.len, (uint32_t)m, p.L)) return;  // padding position (ragged batches)
    const int tid = (int)threadIdx.x;
    const int N = p.N, G = p.d / 16;
    for (int n = tid; n < N; n += 256) {
        float c = 0.0f;
        for (int s = 0; s < p.nsplit; ++s) c += p.part[((int64_t)s * p.M + m) * N + n];
        corr[n] = c;
    }
    __syncthreads();
    const int t = (int)(m % p.L);
    const uint16_t *xr = p.x + m * p.d;
    const uint16_t *pr = t == 0 ? p.x_prev + (m / p.L) * p.d : xr - p.d;
    uint16_t *yr = p.y + m * p.d;
    for (int c0 = tid * 8; c0 < p.d; c0 += 256 * 8) {
        const float k0c = corr[c0 / 16], k1c = corr[G + c0 / 16];
        float a[8], q[8], e0[8], e1[8];
        widen_vec<true>(*(const u32x4 *)(xr + c0), a);
        widen_vec<true>(*(const u32x4 *)(pr + c0), q);
        widen_vec<true>(*(const u32x4 *)(p.base + c0), e0);
        widen_vec<true>(*(const u32x4 *)(p.base + p.d + c0), e1);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float ylo = (e0[e] + k0c) * a[e] + (e1[e] + k1c) * q[e];
            const float yhi = (e0[e + 1] + k0c) * a[e + 1] + (e1[e + 1] + k1c) * q[e + 1];
            w[e >> 1] = f32_to_bf16_rne(ylo) | (f32_to_bf16_rne(yhi) << 16);
        }
        *(u32x4 *)(yr + c0) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// K splits of the correction GEMM: about 256 workgroups, at least 6 K steps
// per split.
inline int conv_nsplit(int64_t batch, int64_t block, int64_t d) {
    const int64_t M = batch * block, N = d / 8;
    const int64_t tiles = (M + 127) / 128 * (N / conv_bn(M, N));
    const int64_t nk = d / kBK;
    int64_t s = 256 / (tiles > 0 ? tiles : 1);
    if (s > nk / 6) s = nk / 6;
    return (int)(s < 1 ? 1 : s);
}

inline size_t conv_workspace_bytes(int64_t batch, int64_t block, int64_t d) {
    return (size_t)conv_nsplit(batch, block, d) * (size_t)(batch * block) * (size_t)(d / 8) * sizeof(float);
}

}  // namespace dsel
