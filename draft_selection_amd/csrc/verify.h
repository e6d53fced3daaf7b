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
//   verify_stats_kernel  HBM-bound, nsplit workgroups (4 waves) per target row.
//       A row is cut into chunks of 256 16-byte vectors (2048 bf16 or 1024
//       fp32 tokens); each wave streams whole chunks with non-temporal loads,
//       the next chunk in flight while the current one is reduced.  Greedy: a
//       per-vector max screens the exact (value, id) key compare of the arg
//       max.  Sampled: per chunk its max mc and sum of exp2((z - mc) s),
//       s = log2(e) / T, kept for the draw; the wave folds the chunks into
//       one (max, sum) by rescaling.  Each workgroup writes one partial.
//   verify_draw_kernel   one workgroup per block: the L acceptance tests run in
//       parallel (one lane each, partials combined in a fixed order) and the
//       first miss is a ballot.  The sampled extra token's inverse CDF prefix-
//       scans the chunk masses (candidate corrections added per chunk), then
//       loads the one chunk that holds u_res * Z, one vector per thread, and
//       prefix-scans its tokens.
#pragma once

#include "common.h"

namespace dsel {

constexpr int64_t kVMaxVocab = 1 << 22;  // 4,194,304 tokens
#ifndef DSEL_VERIFY_U
#define DSEL_VERIFY_U 4
#endif
constexpr int kVU = DSEL_VERIFY_U;       // 16-byte vectors per lane per chunk
constexpr int kVChunkVecs = kWave * kVU; // vectors per chunk
constexpr int kVMaxSplit = 16;           // workgroups per row, at most

// One workgroup's partial result for its slice of a row.
struct alignas(16) VerifyPart {
    float m, z;         // sampled: max and sum of exp2((z - m) s) over the slice
    uint32_t klo, khi;  // greedy: the slice's best (value, id) key
};

struct VerifyParams {
    const char *logits;  // target row (b, t), t = 0..L, starts at logits + (b (L+1) + t) ld es
    int64_t V, ld;
    int B, L;
    const int32_t *len;  // ragged batch: drafted positions per block (nullptr: all L)
    int nsplit;          // workgroups per row
    int nchunk;          // chunks per row: ceil(V / (256 EPV))
    int cps;             // chunks per workgroup (the last one may have fewer)
    float scale;         // log2(e) / T (sampled)
    const int32_t *cand_id, *path_slot;
    const float *q, *u_acc, *u_res;
    int32_t *n_acc, *out_tok;
    VerifyPart *part;    // [rows][nsplit]
    float2 *chunk;       // [rows][nchunk]: chunk max, sum of exp2((z - max) s) (sampled)
};

// Butterfly reductions over the wave (partners lane ^ 32, ^ 16, ..., ^ 1; the
// same order on every lane, so every lane ends with the same bits).
__device__ __forceinline__ float fxor_max(float x, uint32_t y) { return __builtin_fmaxf(x, __uint_as_float(y)); }
__device__ __forceinline__ float wave_max_f(float x) {
    x = fxor_max(x, xor_lane32<32>(__float_as_uint(x)));
    x = fxor_max(x, xor_lane32<16>(__float_as_uint(x)));
    x = fxor_max(x, xor_lane32<8>(__float_as_uint(x)));
    x = fxor_max(x, xor_lane32<4>(__float_as_uint(x)));
    x = fxor_max(x, xor_lane32<2>(__float_as_uint(x)));
    x = fxor_max(x, xor_lane32<1>(__float_as_uint(x)));
    return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
    x += __uint_as_float(xor_lane32<32>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane32<16>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane32<8>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane32<4>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane32<2>(__float_as_uint(x)));
    x += __uint_as_float(xor_lane32<1>(__float_as_uint(x)));
    return x;
}
__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = u64_max(x, xor_lane64<32>(x));
    x = u64_max(x, xor_lane64<16>(x));
    x = u64_max(x, xor_lane64<8>(x));
    x = u64_max(x, xor_lane64<4>(x));
    x = u64_max(x, xor_lane64<2>(x));
    x = u64_max(x, xor_lane64<1>(x));
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

// Load chunk c of a row: lane l takes vectors c 256 + u 64 + l (u < kVU); an
// index past the row's whole vectors is clamped to the last one (its values
// are not used).  The loads are issued unconditionally, so the next chunk can
// be in flight while the current one is reduced.
__device__ __forceinline__ void verify_load_chunk(u32x4 (&w)[kVU], const u32x4 *vb, int64_t c, int64_t nfull) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int u = 0; u < kVU; ++u) {
        int64_t vi = c * kVChunkVecs + u * kWave + lane;
        vi = vi < nfull ? vi : nfull - 1;
        w[u] = __builtin_nontemporal_load(vb + vi);
    }
}

// Workgroup (row, sp) takes chunks [sp cps, min(nchunk, (sp + 1) cps)); wave w
// takes every fourth of them starting at the w-th.
template <bool BF16, bool SAMPLED>
__global__ __launch_bounds__(256) void verify_stats_kernel(VerifyParams p) {
    constexpr int EPV = BF16 ? 8 : 4;
    const int64_t row = blockIdx.x / p.nsplit;
    const int sp = (int)(blockIdx.x - row * p.nsplit);
    // ragged batches: block b reads its rows 0 .. len only (row len follows its last token)
    if (p.len) {
        const uint32_t b = (uint32_t)row / (uint32_t)(p.L + 1);
        if ((int)((uint32_t)row - b * (uint32_t)(p.L + 1)) > block_len_of(p.len, b, p.L)) return;
    }
    const int tid = (int)threadIdx.x, wave = tid >> 6;
    const uint32_t lane = lane_id();
    const char *rowp = p.logits + row * p.ld * (BF16 ? 2 : 4);
    const u32x4 *vb = (const u32x4 *)rowp;
    const int64_t nfull = p.V / EPV;              // whole vectors
    const int tail = (int)(p.V - nfull * EPV);    // tokens of the partial last vector
    const int c0 = sp * p.cps;
    const int c1 = c0 + p.cps < p.nchunk ? c0 + p.cps : p.nchunk;
    const float s = p.scale;

    float bv = -__builtin_inff();  // greedy: the lane's best value and key
    uint64_t bkey = 0;
    float wbv = -__builtin_inff();  // greedy: the wave's best value (max of bv)
    float wm = -__builtin_inff(), wz = 0.0f;  // sampled: the wave's running max and sum

    u32x4 cur[kVU], nxt[kVU];
    // reduce the chunk c held in cur
    auto process = [&](int c) {
        if constexpr (!SAMPLED) {
            // screen: can any element of the lane's chunk reach the wave's best
            // so far (wbv, wave-uniform)?  Nothing below it can be the row's
            // arg max, so lanes skip it even when it beats their own best.
            bool pass;
            if (BF16 && wbv > 0.0f) {  // on the packed bits (wbv is a bf16 value)
                const uint32_t floor = bf16_pk_floor(wbv);
                uint32_t m = floor;
#pragma unroll
                for (int u = 0; u < kVU; ++u) m = pk_max_i16(m, bf16x8_pk_max(cur[u]));
                pass = m != floor;
            } else {
                float cm = -__builtin_inff();
#pragma unroll
                for (int u = 0; u < kVU; ++u) {
                    float x[EPV];
                    widen_vec<BF16>(cur[u], x);
#pragma unroll
                    for (int e = 0; e < EPV; ++e) cm = __builtin_fmaxf(cm, x[e]);
                }
                // ties, the first chunk (wbv = -inf) and NaN-only chunks pass;
                // v_max drops a NaN beside a number, and a NaN never beats a
                // real key
                pass = !(cm < wbv) || cm != cm;
            }
            // the row's partial last vector always takes the exact compare
            const int64_t vt = nfull - (int64_t)c * kVChunkVecs;  // its place in this chunk
            if (tail && vt >= 0 && vt < kVChunkVecs && (int64_t)(vt % kWave) == (int64_t)lane) pass = true;
            if (ballot(pass)) {
                if (pass) {
#pragma unroll
                    for (int u = 0; u < kVU; ++u) {
                        const int64_t vi = (int64_t)c * kVChunkVecs + u * kWave + lane;
                        const int cnt = vi < nfull ? EPV : (vi == nfull ? tail : 0);
                        float x[EPV];
                        if (vi < nfull) {
                            widen_vec<BF16>(cur[u], x);
                        } else {
#pragma unroll
                            for (int e = 0; e < EPV; ++e)
                                x[e] = e < cnt ? logit_elem<BF16>(rowp, nfull * EPV + e) : -__builtin_inff();
                        }
#pragma unroll
                        for (int e = 0; e < EPV; ++e) {
                            const uint64_t k = cand_key(x[e], (uint32_t)(vi * EPV + e));
                            const bool better = e < cnt && k > bkey;
                            bkey = better ? k : bkey;
                            bv = better && x[e] == x[e] ? x[e] : bv;
                        }
                    }
                }
                wbv = wave_max_f(bv);
            }
        } else {
            // x = -inf stands for "no element": it leaves the max alone and
            // adds exp2(-inf) = 0 to the sum, so only the row's last chunk
            // (clamped vectors, the partial vector) needs per-vector care.
            float x[kVU][EPV];
#pragma unroll
            for (int u = 0; u < kVU; ++u) widen_vec<BF16>(cur[u], x[u]);
            if (c == p.nchunk - 1) {  // wave-uniform
#pragma unroll
                for (int u = 0; u < kVU; ++u) {
                    const int64_t vi = (int64_t)c * kVChunkVecs + u * kWave + lane;
                    const int cnt = vi < nfull ? EPV : (vi == nfull ? tail : 0);
                    if (cnt < EPV) {
#pragma unroll
                        for (int e = 0; e < EPV; ++e)
                            x[u][e] = e < cnt ? logit_elem<BF16>(rowp, nfull * EPV + e) : -__builtin_inff();
                    }
                }
            }
            float lm = -__builtin_inff();
#pragma unroll
            for (int u = 0; u < kVU; ++u)
#pragma unroll
                for (int e = 0; e < EPV; ++e) lm = __builtin_fmaxf(lm, x[u][e]);
            const float mc = wave_max_f(lm);
            float ls = 0.0f;
            if (mc != -__builtin_inff()) {  // wave-uniform; then x = -inf gives exp2(-inf) = 0
#pragma unroll
                for (int u = 0; u < kVU; ++u)
#pragma unroll
                    for (int e = 0; e < EPV; ++e) ls += __builtin_amdgcn_exp2f((x[u][e] - mc) * s);
            }
            const float zc = wave_sum_f(ls);
            if (lane == 0) p.chunk[row * p.nchunk + c] = make_float2(mc, zc);
            const float nm = __builtin_fmaxf(wm, mc);
            wz = wz * exp2_rel(wm, nm, s) + zc * exp2_rel(mc, nm, s);
            wm = nm;
        }
    };
    // the next chunk's loads go out before the current one is reduced; the
    // last chunk is peeled off so that no load is issued past the range
    int c = c0 + wave;
    if (c < c1) {
        verify_load_chunk(cur, vb, c, nfull);
        for (; c + 4 < c1; c += 4) {
            verify_load_chunk(nxt, vb, c + 4, nfull);
            process(c);
#pragma unroll
            for (int u = 0; u < kVU; ++u) cur[u] = nxt[u];
        }
        process(c);
    }
    // the workgroup's partial: waves combined in a fixed order
    __shared__ float sm[4], sz[4];
    __shared__ uint64_t sk[4];
    if constexpr (!SAMPLED) {
        bkey = wave_max_u64(bkey);
        if (lane == 0) sk[wave] = bkey;
    } else if (lane == 0) {
        sm[wave] = wm;
        sz[wave] = wz;
    }
    __syncthreads();
    if (tid == 0) {
        VerifyPart out;
        if constexpr (!SAMPLED) {
            uint64_t k = sk[0];
            for (int w = 1; w < 4; ++w) k = sk[w] > k ? sk[w] : k;
            out.m = 0.0f;
            out.z = 0.0f;
            out.klo = (uint32_t)k;
            out.khi = (uint32_t)(k >> 32);
        } else {
            float m = sm[0];
            for (int w = 1; w < 4; ++w) m = __builtin_fmaxf(m, sm[w]);
            float z = 0.0f;
            for (int w = 0; w < 4; ++w) z += sz[w] * exp2_rel(sm[w], m, s);
            out.m = m;
            out.z = z;
            out.klo = out.khi = 0u;
        }
        p.part[row * p.nsplit + sp] = out;
    }
}

// A row's arg max (greedy) from its partials.
__device__ __forceinline__ uint32_t verify_row_argmax(const VerifyParams &p, int64_t row) {
    uint64_t k = 0;
    for (int i = 0; i < p.nsplit; ++i) {
        const VerifyPart &q = p.part[row * p.nsplit + i];
        const uint64_t ki = ((uint64_t)q.khi << 32) | q.klo;
        k = ki > k ? ki : k;
    }
    return key_id(k);
}

// A row's max m and Z = sum exp2((z - m) s) (sampled) from its partials, in a
// fixed order, so every reader of a row gets the same two numbers.
__device__ __forceinline__ void verify_row_mz(const VerifyParams &p, int64_t row, float *m, float *Z) {
    float mm = -__builtin_inff();
    for (int i = 0; i < p.nsplit; ++i) mm = __builtin_fmaxf(mm, p.part[row * p.nsplit + i].m);
    float z = 0.0f;
    for (int i = 0; i < p.nsplit; ++i) {
        const VerifyPart &q = p.part[row * p.nsplit + i];
        z += q.z * exp2_rel(q.m, mm, p.scale);
    }
    *m = mm;
    *Z = z;
}

// Block-wide prefix of one non-negative float per thread (256 threads): the
// thread's interval [lo, hi) of the running sum, and the total.  Each thread's
// lo is bit-identical to the previous thread's hi (both come from the same
// additions in the same order), so the intervals tile [0, total) with no gap or
// overlap and exactly one thread holds any tau in that range.
__device__ __forceinline__ void block_scan_edges(float x, float *lo, float *hi, float *total, float *lds4) {
    const int wave = (int)(threadIdx.x >> 6);
    const uint32_t lane = lane_id();
    const float inc = wave_scan_f(x);
    const float prev = shfl_idxf(inc, lane ? lane - 1 : 0);
    if (lane == kWave - 1) lds4[wave] = inc;
    __syncthreads();
    float off = 0.0f, tot = 0.0f;
    for (int w = 0; w < 4; ++w) {
        if (w < wave) off += lds4[w];
        tot += lds4[w];
    }
    __syncthreads();
    *total = tot;
    *hi = off + inc;
    *lo = lane ? off + prev : off;
}

template <bool BF16, bool SAMPLED>
__global__ __launch_bounds__(256) void verify_draw_kernel(VerifyParams p) {
    constexpr int EPV = BF16 ? 8 : 4;
    constexpr int CT = kVChunkVecs * EPV;  // tokens per chunk
    const int b = blockIdx.x;
    const int L = p.L;
    const int nb = block_len_of(p.len, b, L);  // drafted positions (ragged batches: the block's own)
    const int tid = (int)threadIdx.x;
    const uint32_t lane = lane_id();
    const int64_t es = BF16 ? 2 : 4;
    __shared__ float lds4[4];
    __shared__ int s_n, s_tok, s_last, s_chunk, s_clast;
    __shared__ float s_off;
    __shared__ int32_t s_cid[kK];
    __shared__ float s_cq[kK], s_cadj[kK];

    // 1. acceptance tests, one lane per position
    if (tid < kWave) {
        bool acc = false;
        int32_t x = -1;
        if ((int)lane < nb) {
            const int64_t bt = (int64_t)b * L + lane;
            const int slot = p.path_slot[bt] & (kK - 1);
            x = p.cand_id[bt * kK + slot];
            const int64_t row = (int64_t)b * (L + 1) + lane;
            if (x >= 0 && (int64_t)x < p.V) {
                if constexpr (SAMPLED) {
                    float m, Z;
                    verify_row_mz(p, row, &m, &Z);
                    const float zx = logit_elem<BF16>(p.logits + row * p.ld * es, x);
                    const float px = exp2_rel(zx, m, p.scale) / Z;
                    acc = p.u_acc[bt] * p.q[bt * kK + slot] < px;
                } else {
                    acc = (uint32_t)x == verify_row_argmax(p, row);
                }
            }
        }
        const uint64_t miss = ballot((int)lane < nb && !acc);
        const int n = miss ? (int)__builtin_ctzll(miss) : nb;
        if ((int)lane < n) p.out_tok[(int64_t)b * (L + 1) + lane] = x;
        if (lane == 0) {
            s_n = n;
            s_tok = 0x7FFFFFFF;
            s_last = -1;
            s_chunk = -1;
            s_clast = -1;
        }
    }
    __syncthreads();
    const int n = s_n;
    const int64_t row = (int64_t)b * (L + 1) + n;
    int32_t tok;
    if constexpr (!SAMPLED) {
        tok = (int32_t)verify_row_argmax(p, row);
    } else {
        // 2. the draw's weights: w(v) = p(v), less q(v) (clamped at 0) at the
        // candidates when position n was rejected.
        const bool residual = n < nb;
        const float s = p.scale;
        float m, Z;
        verify_row_mz(p, row, &m, &Z);
        const char *rowp = p.logits + row * p.ld * es;
        if (tid < kK) {
            int32_t c = -1;
            float qc = 0.0f, adj = 0.0f;
            if (residual) {
                const int64_t bt = (int64_t)b * L + n;
                c = p.cand_id[bt * kK + tid];
                qc = p.q[bt * kK + tid];
                for (int j = 0; j < tid; ++j)  // a repeated id takes the first slot's q
                    if (p.cand_id[bt * kK + j] == c) c = -1;
                if (c >= 0 && (int64_t)c < p.V) {
                    const float pc = exp2_rel(logit_elem<BF16>(rowp, c), m, s) / Z;
                    adj = __builtin_fmaxf(pc - qc, 0.0f) - pc;
                } else {
                    c = -1;
                }
            }
            s_cid[tid] = c;
            s_cq[tid] = qc;
            s_cadj[tid] = adj;
        }
        __syncthreads();
        // chunk masses from the chunk statistics; thread i owns the contiguous
        // chunks [i cpt, (i + 1) cpt)
        const int cpt = (p.nchunk + 255) >> 8;
        const int ca = tid * cpt, cb = ca + cpt < p.nchunk ? ca + cpt : p.nchunk;
        uint32_t cmask = 0;
#pragma unroll
        for (int j = 0; j < kK; ++j)
            if (s_cid[j] >= 0 && s_cid[j] / CT >= ca && s_cid[j] / CT < cb) cmask |= 1u << j;
        const float2 *cs = p.chunk + row * p.nchunk;
        auto cmass = [&](int c) {
            const float2 st = cs[c];
            float w = st.y * exp2_rel(st.x, m, s) / Z;
            for (uint32_t mk = cmask; mk; mk &= mk - 1) {
                const int j = __builtin_ctz(mk);
                if (s_cid[j] / CT == c) w += s_cadj[j];
            }
            return w > 0.0f ? w : 0.0f;
        };
        float mine = 0.0f;
        int lastc = -1;
        for (int c = ca; c < cb; ++c) {
            const float w = cmass(c);
            mine += w;
            if (w > 0.0f) lastc = c;
        }
        float lo, hi, Zr;
        block_scan_edges(mine, &lo, &hi, &Zr, lds4);
        const float tau = p.u_res[b] * Zr;
        if (lastc >= 0) atomicMax(&s_clast, lastc);
        if (tau >= lo && tau < hi) {  // exactly one thread
            float cum = lo;
            int pick = -1;
            float off = __builtin_inff();
            for (int c = ca; c < cb; ++c) {
                const float w = cmass(c);
                if (w > 0.0f && tau < cum + w) {
                    pick = c;
                    off = tau - cum;
                    break;
                }
                cum += w;
            }
            s_chunk = pick >= 0 ? pick : lastc;  // the rescan rounds differently: last chunk with mass
            s_off = off;
        }
        __syncthreads();
        int ch = s_chunk;
        float target = s_off;
        if (ch < 0) {  // u Z rounded up to the total: the last chunk with mass
            ch = s_clast;
            target = __builtin_inff();
        }
        if (ch < 0) {
            tok = -1;  // no token has mass
        } else {
            // 3. the chunk's tokens, one vector per thread
            const int64_t nfull = p.V / EPV;
            const int tail = (int)(p.V - nfull * EPV);
            const int64_t vi = (int64_t)ch * kVChunkVecs + tid;
            const int64_t t0 = vi * EPV;
            float x[EPV];
            int cnt = 0;
            if (vi < nfull) {
                widen_vec<BF16>(*((const u32x4 *)rowp + vi), x);
                cnt = EPV;
            } else if (vi == nfull && tail) {
#pragma unroll
                for (int e = 0; e < EPV; ++e) x[e] = e < tail ? logit_elem<BF16>(rowp, t0 + e) : -__builtin_inff();
                cnt = tail;
            }
            uint32_t tmask = 0;
#pragma unroll
            for (int j = 0; j < kK; ++j)
                if (cnt && s_cid[j] >= t0 && s_cid[j] < t0 + cnt) tmask |= 1u << j;
            float w[EPV];
            float ms = 0.0f;
            int lastpos = -1;
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                float we = 0.0f;
                if (e < cnt) {
                    we = exp2_rel(x[e], m, s) / Z;
                    for (uint32_t mk = tmask; mk; mk &= mk - 1) {
                        const int j = __builtin_ctz(mk);
                        if (s_cid[j] == t0 + e) {
                            const float d = we - s_cq[j];
                            we = d > 0.0f ? d : 0.0f;
                        }
                    }
                }
                w[e] = we;
                ms += we;
                if (we > 0.0f) lastpos = (int)(t0 + e);
            }
            float lo2, hi2, tot2;
            block_scan_edges(ms, &lo2, &hi2, &tot2, lds4);
            if (lastpos >= 0) atomicMax(&s_last, lastpos);
            if (target >= lo2 && target < hi2) {  // exactly one thread
                float cum = lo2;
                int pick = -1;
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    if (pick < 0 && w[e] > 0.0f && target < cum + w[e]) pick = (int)(t0 + e);
                    cum += w[e];
                }
                s_tok = pick >= 0 ? pick : lastpos;  // the rescan rounds differently
            }
            __syncthreads();
            // target past the chunk's total (rounding): its last token with mass
            tok = s_tok != 0x7FFFFFFF ? s_tok : s_last;
            if (tok < 0) tok = (int32_t)(ch * (int64_t)CT);  // the chunk's tokens all round to 0
        }
    }
    if (tid == 0) {
        p.out_tok[(int64_t)b * (L + 1) + n] = tok;
        p.n_acc[b] = n;
    }
    for (int t = n + 1 + tid; t <= L; t += 256) p.out_tok[(int64_t)b * (L + 1) + t] = -1;
}

// Partials [rows][kVMaxSplit] and chunk statistics [rows][ceil(V / 1024)]
// (the fp32 chunk, the smaller of the two chunk sizes).
inline size_t verify_part_bytes(int64_t batch, int64_t block) {
    return (size_t)(batch * (block + 1)) * kVMaxSplit * sizeof(VerifyPart);
}
inline size_t verify_workspace_bytes(int64_t batch, int64_t block, int64_t vocab) {
    const int64_t nchunk = (vocab + kVChunkVecs * 4 - 1) / (kVChunkVecs * 4);
    return verify_part_bytes(batch, block) + (size_t)(batch * (block + 1) * nchunk) * sizeof(float2);
}

}  // namespace dsel
