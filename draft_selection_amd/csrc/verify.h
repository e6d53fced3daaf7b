// verify: lossless verification of the drafted blocks against the target model.
// ("DFlash 2: Keep Drafting Parallel", Method, last paragraph, and Setup: the
// sampled walk stays lossless through rejection sampling; "DFlash 2: The
// Drafter Stopped Guessing Alone", "One pass to draft, one pass to verify": the
// accepted prefix is kept and the first miss is replaced by the target's own
// choice.)
//
// Rules (greedy / sampled with temperature T):
//   greedy   position t is accepted while its drafted token is the arg max of
//            target row t (ties to the lower id, NaN lowest); the extra token
//            is the arg max of the first rejected row, or of row L.
//   sampled  p_t = softmax(z_t / T); position t accepts its token x iff
//            u_acc[b,t] * q_t(x) < p_t(x) (probability min(1, p/q)); the extra
//            token is drawn by inverse CDF in token order, with u_res[b], from
//            max(0, p_t - q_t) at the first rejection (q_t is zero off the 16
//            candidates), or from p_L when every position is accepted.
//
// Two kernels:
//   verify_stats_kernel  one workgroup (4 waves) per target row, HBM-bound: one
//       pass over the row gives its arg max and, for the sampled rule, its max
//       m and Z = sum exp2((z - m) s) (s = log2(e) / T), plus the same two
//       numbers for every chunk of 2048 tokens (the draw needs them).
//   verify_draw_kernel   one workgroup per block: the L acceptance tests run in
//       parallel (one lane each) and the first miss is a ballot; the extra
//       token's inverse CDF walks the chunk masses (prefix scan over chunks),
//       then scans the one chunk where u_res * Z falls.
#pragma once

#include "common.h"

namespace dsel {

constexpr int kVChunk = 2048;        // tokens per chunk of the row statistics
constexpr int kVMaxChunks = 2048;    // vocab <= 2048 chunks = 4,194,304 tokens

struct VerifyParams {
    const char *logits;  // target row (b, t), t = 0..L, starts at logits + (b (L+1) + t) ld es
    int64_t V, ld;
    int B, L;
    int nchunk;          // ceil(V / kVChunk)
    float scale;         // log2(e) / T (sampled)
    const int32_t *cand_id, *path_slot;
    const float *q, *u_acc, *u_res;
    int32_t *n_acc, *out_tok;
    float *row_stat;     // [rows][4]: max, Z, arg max (int bits), unused
    float *chunk_stat;   // [rows][nchunk][2]: chunk max, chunk sum of exp2((z - chunk max) s)
};

__device__ __forceinline__ float wave_max_f(float x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = __builtin_fmaxf(x, shfl_idxf(x, lane ^ (uint32_t)o));
    return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += shfl_idxf(x, lane ^ (uint32_t)o);
    return x;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint64_t y = shfl_idx64(x, lane ^ (uint32_t)o);
        x = y > x ? y : x;
    }
    return x;
}
// inclusive prefix sum across the wave
__device__ __forceinline__ float wave_scan_f(float x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float y = shfl_idxf(x, lane >= (uint32_t)o ? lane - (uint32_t)o : lane);
        if (lane >= (uint32_t)o) x += y;
    }
    return x;
}

// exp2((x - m) s), 0 for x = -inf (also when m = -inf)
__device__ __forceinline__ float exp2_rel(float x, float m, float s) {
    return x == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f((x - m) * s);
}

template <bool BF16>
__device__ __forceinline__ float logit_elem(const char *rowp, int64_t i) {
    if constexpr (BF16) return __uint_as_float((uint32_t)(*(const uint16_t *)(rowp + i * 2)) << 16);
    else return *(const float *)(rowp + i * 4);
}

// One pass over a target row: arg max (64-bit candidate keys), and for the
// sampled rule the row's and every chunk's max / sum of exp2.  Wave w takes
// chunks w, w + 4, ...; lane l holds elements of vectors c * (2048 / EPV) +
// u * 64 + l of its chunk (16-byte loads; row starts are 16-byte aligned).
template <bool BF16, bool SAMPLED>
__global__ __launch_bounds__(256) void verify_stats_kernel(VerifyParams p) {
    constexpr int EPV = BF16 ? 8 : 4;
    constexpr int U = kVChunk / (kWave * EPV);  // vectors per lane per chunk
    const int64_t row = blockIdx.x;
    const int wave = (int)(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const char *rowp = p.logits + row * p.ld * (BF16 ? 2 : 4);
    const u32x4 *vb = (const u32x4 *)rowp;
    const float s = p.scale;

    float wm = -__builtin_inff(), ws = 0.0f;  // this wave's running max and sum
    uint64_t wkey = 0;
    for (int c = wave; c < p.nchunk; c += 4) {
        float x[U][EPV];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e0 = ((int64_t)c * (kVChunk / EPV) + u * kWave + lane) * EPV;
            if (e0 + EPV <= p.V) {
                const u32x4 w = __builtin_nontemporal_load(vb + e0 / EPV);
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const uint32_t word = w[BF16 ? e >> 1 : e];
                    x[u][e] = BF16 ? __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16))
                                   : __uint_as_float(word);
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    x[u][e] = e0 + e < p.V ? logit_elem<BF16>(rowp, e0 + e) : __builtin_nanf("");
            }
        }
        uint64_t key = 0;
        float lm = -__builtin_inff();
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int64_t id = ((int64_t)c * (kVChunk / EPV) + u * kWave + lane) * EPV + e;
                if (id < p.V) {
                    const uint64_t k = cand_key(x[u][e], (uint32_t)id);
                    key = k > key ? k : key;
                    lm = __builtin_fmaxf(lm, x[u][e]);
                }
            }
        key = wave_max_u64(key);
        wkey = key > wkey ? key : wkey;
        if constexpr (SAMPLED) {
            const float mc = wave_max_f(lm);
            float ls = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const int64_t id = ((int64_t)c * (kVChunk / EPV) + u * kWave + lane) * EPV + e;
                    if (id < p.V) ls += exp2_rel(x[u][e], mc, s);
                }
            const float sc = wave_sum_f(ls);
            if (lane == 0) {
                float *cs = p.chunk_stat + (row * p.nchunk + c) * 2;
                cs[0] = mc;
                cs[1] = sc;
            }
            const float nm = __builtin_fmaxf(wm, mc);
            ws = ws * exp2_rel(wm, nm, s) + sc * exp2_rel(mc, nm, s);
            wm = nm;
        }
    }
    __shared__ float sm[4], ss[4];
    __shared__ uint64_t sk[4];
    if (lane == 0) {
        sm[wave] = wm;
        ss[wave] = ws;
        sk[wave] = wkey;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t k = sk[0];
        float m = sm[0];
        for (int w = 1; w < 4; ++w) {
            k = sk[w] > k ? sk[w] : k;
            m = __builtin_fmaxf(m, sm[w]);
        }
        float z = 0.0f;
        for (int w = 0; w < 4; ++w) z += ss[w] * exp2_rel(sm[w], m, s);
        float *rs = p.row_stat + row * 4;
        rs[0] = m;
        rs[1] = z;
        rs[2] = __uint_as_float(key_id(k));
        rs[3] = 0.0f;
    }
}

// Block-wide exclusive prefix of one float per thread (256 threads), and the
// total.  Fixed order, so the result is deterministic.
__device__ __forceinline__ float block_exclusive_scan(float x, float *total, float *lds4) {
    const int wave = (int)(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const float inc = wave_scan_f(x);
    if (lane == kWave - 1) lds4[wave] = inc;
    __syncthreads();
    float off = 0.0f, tot = 0.0f;
    for (int w = 0; w < 4; ++w) {
        if (w < wave) off += lds4[w];
        tot += lds4[w];
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

template <bool BF16, bool SAMPLED>
__global__ __launch_bounds__(256) void verify_draw_kernel(VerifyParams p) {
    const int b = blockIdx.x;
    const int L = p.L;
    const int tid = (int)threadIdx.x;
    const uint32_t lane = lane_id();
    const int64_t es = BF16 ? 2 : 4;
    __shared__ float w[kVMaxChunks];
    __shared__ float lds4[4];
    __shared__ int s_n, s_k, s_tok, s_last;
    __shared__ float s_cbefore;

    // 1. acceptance tests, one lane per position
    if (tid < kWave) {
        bool acc = false;
        int32_t x = -1;
        if ((int)lane < L) {
            const int64_t bt = (int64_t)b * L + lane;
            const int slot = p.path_slot[bt] & (kK - 1);
            x = p.cand_id[bt * kK + slot];
            const int64_t row = (int64_t)b * (L + 1) + lane;
            if (x >= 0 && (int64_t)x < p.V) {
                if constexpr (SAMPLED) {
                    const float *rs = p.row_stat + row * 4;
                    const float zx = logit_elem<BF16>(p.logits + row * p.ld * es, x);
                    const float px = exp2_rel(zx, rs[0], p.scale) / rs[1];
                    acc = p.u_acc[bt] * p.q[bt * kK + slot] < px;
                } else {
                    acc = (uint32_t)x == __float_as_uint(p.row_stat[row * 4 + 2]);
                }
            }
        }
        const uint64_t miss = ballot((int)lane < L && !acc);
        const int n = miss ? (int)__builtin_ctzll(miss) : L;
        if ((int)lane < n) p.out_tok[(int64_t)b * (L + 1) + lane] = x;
        if (lane == 0) s_n = n;
    }
    __syncthreads();
    const int n = s_n;
    const int64_t row = (int64_t)b * (L + 1) + n;
    int32_t tok;
    if constexpr (!SAMPLED) {
        tok = (int32_t)__float_as_uint(p.row_stat[row * 4 + 2]);
    } else {
        // 2. mass of every chunk of the draw's distribution
        const bool residual = n < L;
        const float m = p.row_stat[row * 4], Z = p.row_stat[row * 4 + 1], s = p.scale;
        const char *rowp = p.logits + row * p.ld * es;
        for (int c = tid; c < p.nchunk; c += 256) {
            const float *cs = p.chunk_stat + (row * p.nchunk + c) * 2;
            w[c] = cs[1] * exp2_rel(cs[0], m, s) / Z;
        }
        __syncthreads();
        // residual: subtract min(p, q) of each candidate from its chunk, in
        // candidate order (one thread, values gathered by 16 lanes)
        int32_t cj = -1;
        float qj = 0.0f, pj = 0.0f;
        if (residual && tid < kK) {
            const int64_t bt = (int64_t)b * L + n;
            cj = p.cand_id[bt * kK + tid];
            qj = p.q[bt * kK + tid];
            if (cj >= 0 && (int64_t)cj < p.V) pj = exp2_rel(logit_elem<BF16>(rowp, cj), m, s) / Z;
        }
        if (residual && tid < kWave) {
            for (int j = 0; j < kK; ++j) {
                const int32_t c = __builtin_amdgcn_readlane(cj, j);
                const float pq = __builtin_fminf(__uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(pj), j)),
                                                 __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(qj), j)));
                if (tid == 0 && c >= 0 && (int64_t)c < p.V) w[c / kVChunk] -= pq;
            }
        }
        __syncthreads();
        // 3. the chunk where u Z_r falls: thread i owns chunks [i per, (i+1) per)
        const int per = (p.nchunk + 255) / 256;
        const int c0 = tid * per, c1 = c0 + per < p.nchunk ? c0 + per : p.nchunk;
        float mine = 0.0f;
        int lastpos = -1;
        for (int c = c0; c < c1; ++c) {
            const float v = w[c] > 0.0f ? w[c] : 0.0f;
            mine += v;
            if (v > 0.0f) lastpos = c;
        }
        float Zr;
        const float before = block_exclusive_scan(mine, &Zr, lds4);
        const float tau = p.u_res[b] * Zr;
        if (tid == 0) {
            s_k = 0x7FFFFFFF;
            s_last = -1;
        }
        __syncthreads();
        float cum = before;
        for (int c = c0; c < c1; ++c) {
            const float v = w[c] > 0.0f ? w[c] : 0.0f;
            if (tau < cum + v) {
                atomicMin(&s_k, c);
                break;
            }
            cum += v;
        }
        atomicMax(&s_last, lastpos);
        __syncthreads();
        int k = s_k != 0x7FFFFFFF ? s_k : s_last;  // past the total (rounding): the last chunk with mass
        if (k < 0) k = 0;
        __syncthreads();  // everyone has read s_k / s_last before they are reused
        // cumulative mass before chunk k (the owner of k recomputes it)
        if (k >= c0 && k < c1) {
            float cb = before;
            for (int c = c0; c < k; ++c) cb += w[c] > 0.0f ? w[c] : 0.0f;
            s_cbefore = cb;
        }
        if (tid == 0) {
            s_tok = 0x7FFFFFFF;
            s_last = -1;
        }
        __syncthreads();
        // 4. scan chunk k: thread i takes tokens k 2048 + 8 i .. + 7
        float wv[8];
        float tsum = 0.0f;
        int tlast = -1;
        const int64_t v0 = (int64_t)k * kVChunk + 8 * tid;
        int32_t cand[kK];
        float candq[kK];
        if (residual) {
            const int64_t bt = (int64_t)b * L + n;
#pragma unroll
            for (int j = 0; j < kK; ++j) {
                cand[j] = p.cand_id[bt * kK + j];
                candq[j] = p.q[bt * kK + j];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t v = v0 + e;
            float x = 0.0f;
            if (v < p.V) {
                x = exp2_rel(logit_elem<BF16>(rowp, v), m, s) / Z;
                if (residual) {
#pragma unroll
                    for (int j = 0; j < kK; ++j)
                        if (cand[j] == v) x -= candq[j];
                    x = x > 0.0f ? x : 0.0f;
                }
            }
            wv[e] = x;
            tsum += x;
            if (x > 0.0f) tlast = (int)e;
        }
        float dummy;
        float cum2 = s_cbefore + block_exclusive_scan(tsum, &dummy, lds4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (tau < cum2 + wv[e]) {
                atomicMin(&s_tok, (int)(v0 + e));
                break;
            }
            cum2 += wv[e];
        }
        if (tlast >= 0) atomicMax(&s_last, (int)(v0 + tlast));
        __syncthreads();
        tok = s_tok != 0x7FFFFFFF ? s_tok : s_last;  // past the chunk's mass (rounding): its last token with mass
    }
    if (tid == 0) {
        p.out_tok[(int64_t)b * (L + 1) + n] = tok;
        p.n_acc[b] = n;
    }
    for (int t = n + 1 + tid; t <= L; t += 256) p.out_tok[(int64_t)b * (L + 1) + t] = -1;
}

inline size_t verify_workspace_bytes(int64_t batch, int64_t block, int64_t vocab) {
    const int64_t rows = batch * (block + 1);
    const int64_t nchunk = (vocab + kVChunk - 1) / kVChunk;
    return (size_t)rows * 4 * sizeof(float) + (size_t)rows * nchunk * 2 * sizeof(float);
}

}  // namespace dsel
