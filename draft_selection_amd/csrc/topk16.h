// select_topk: the 16 best candidates of every draft position.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: the
// selector keeps the top-16 candidates of each position.)
//
// HBM-bound streaming selection.  One workgroup (4 waves) scans one row, or a
// 1/nsplit slice of it when there are too few rows to fill the chip; each wave
// streams a contiguous range of 16-byte vectors with non-temporal loads.
// Every wave keeps its running top-16 as one 64-bit key per lane in lanes
// 0..15 (sorted, lane 0 best) and filters incoming elements against the float
// value of its 16th key: almost every element fails that single compare, and
// the rare survivors are inserted one at a time with a cross-lane shift.  The
// first 64 x U elements of a wave seed the list with the sorted lane maxima
// (the 16 best of them bound the rest).  Waves merge through LDS with a 64-key
// bitonic sort; split rows merge in a second, one-wave-per-row kernel.
#pragma once

#include "common.h"

namespace dsel {

struct TopkParams {
    const char *logits;   // row r starts at logits + r * ld * elem_size
    int64_t rows, V, ld;  // ld in elements
    int nsplit;           // workgroups per row
    int32_t *cand_id;
    float *cand_u;
    uint64_t *partial;    // [rows][nsplit][16] keys, used when nsplit > 1
};

template <bool BF16>
__device__ __forceinline__ float vec_elem(const u32x4 &w, int e) {
    if constexpr (BF16) {
        uint32_t x = (e >> 1) == 0 ? w.x : (e >> 1) == 1 ? w.y : (e >> 1) == 2 ? w.z : w.w;
        return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
    } else {
        uint32_t x = e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
        return __uint_as_float(x);
    }
}

template <bool BF16>
__device__ __forceinline__ float load_elem(const char *rowp, int64_t i) {
    if constexpr (BF16) {
        uint32_t u = *(const uint16_t *)(rowp + i * 2);
        return __uint_as_float(u << 16);
    } else {
        return *(const float *)(rowp + i * 4);
    }
}

// Running top-16 of one wave: lanes 0..15 of `key` hold the list, best first.
struct WaveTop {
    uint64_t key;
    uint64_t thr;  // key of the 16th entry (wave-uniform)
    float thr_f;   // its value as a filter threshold (wave-uniform)

    __device__ __forceinline__ void refresh() {
        thr = readlane64(key, 15);
        thr_f = key_threshold(thr);
    }
    // Insert a wave-uniform key known to rank above thr.
    __device__ __forceinline__ void insert(uint64_t c) {
        const uint32_t lane = lane_id();
        bool gt = lane < (uint32_t)kK && c > key;
        uint64_t m = ballot(gt);
        uint64_t prev = shfl_idx64(key, lane == 0 ? 0 : lane - 1);
        bool prev_gt = lane >= 1 && ((m >> (lane - 1)) & 1ull);
        key = gt ? (prev_gt ? prev : c) : key;
        refresh();
    }
    // Offer every lane's x (with element id computed from the lane) where
    // `pass` holds; survivors of the exact compare are inserted in lane order.
    template <typename IdOf>
    __device__ __forceinline__ void offer(float x, bool pass, IdOf id_of) {
        uint64_t m = ballot(pass);
        while (m) {
            uint32_t src = (uint32_t)__builtin_ctzll(m);
            m &= m - 1;
            float xv = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(x), (int)src));
            uint64_t c = cand_key(xv, id_of(src));
            if (c > thr) insert(c);
        }
    }
};

template <bool BF16, int U, bool CHECK, bool FIRST>
__device__ __forceinline__ void topk_chunk(WaveTop &st, const u32x4 *vbase, int64_t v0, int64_t ve,
                                           int64_t h0) {
    constexpr int EPV = BF16 ? 8 : 4;
    const uint32_t lane = lane_id();
    u32x4 w[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t vi = v0 + u * kWave + lane;
        ok[u] = !CHECK || vi < ve;
        if (ok[u]) w[u] = __builtin_nontemporal_load(vbase + vi);
        else w[u] = u32x4{0u, 0u, 0u, 0u};
    }
    int skip = -1;
    if constexpr (FIRST) {
        // Seed: the 16 best lane maxima are real elements, so they bound the
        // rest; each lane's maximum is then not offered again.
        uint64_t best = 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                uint64_t k = cand_key(vec_elem<BF16>(w[u], e),
                                      (uint32_t)(h0 + (v0 + u * kWave + lane) * EPV + e));
                if (ok[u] && k > best) {
                    best = k;
                    skip = u * EPV + e;
                }
            }
        uint64_t srt = wave_sort64_desc(best);
        st.key = lane < (uint32_t)kK ? srt : 0ull;
        st.refresh();
    }
    bool any = false;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            bool p = !(vec_elem<BF16>(w[u], e) < st.thr_f);
            if (CHECK) p = p && ok[u];
            if (FIRST) p = p && (u * EPV + e != skip);
            any |= p;
        }
    if (ballot(any) == 0) return;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            float x = vec_elem<BF16>(w[u], e);
            bool p = !(x < st.thr_f);
            if (CHECK) p = p && ok[u];
            if (FIRST) p = p && (u * EPV + e != skip);
            const int64_t vrow = v0 + u * kWave;
            st.offer(x, p, [&](uint32_t src) { return (uint32_t)(h0 + (vrow + src) * EPV + e); });
        }
}

template <bool BF16, int U>
__global__ __launch_bounds__(256) void topk16_kernel(TopkParams p) {
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int EPV = 16 / ES;
    const int64_t row = blockIdx.x / p.nsplit;
    const int split = (int)(blockIdx.x % p.nsplit);
    const int wave = (int)(threadIdx.x / kWave);
    const uint32_t lane = lane_id();
    const char *rowp = p.logits + row * p.ld * ES;

    // Row geometry: `h0` head elements before the first 16-byte boundary, then
    // `nvec` whole vectors, then the tail elements [tail0, V).
    const uint32_t mis = (uint32_t)(((uintptr_t)rowp & 15u) / ES);
    const int64_t h0 = mis ? (EPV - mis) : 0;
    const int64_t nvec = (p.V - h0) / EPV;
    const int64_t tail0 = h0 + nvec * EPV;
    const u32x4 *vbase = (const u32x4 *)(rowp + h0 * ES);

    const int64_t nw = (int64_t)p.nsplit * 4;
    const int64_t gw = (int64_t)split * 4 + wave;
    const int64_t vb = nvec * gw / nw, ve = nvec * (gw + 1) / nw;

    WaveTop st;
    st.key = 0ull;
    st.thr = 0ull;
    st.thr_f = -__builtin_inff();

    constexpr int STEP = U * kWave;
    int64_t v0 = vb;
    if (v0 < ve) {
        if (v0 + STEP <= ve) topk_chunk<BF16, U, false, true>(st, vbase, v0, ve, h0);
        else topk_chunk<BF16, U, true, true>(st, vbase, v0, ve, h0);
        v0 += STEP;
        for (; v0 + STEP <= ve; v0 += STEP) topk_chunk<BF16, U, false, false>(st, vbase, v0, ve, h0);
        if (v0 < ve) topk_chunk<BF16, U, true, false>(st, vbase, v0, ve, h0);
    }
    if (gw == 0) {  // head and tail elements outside the whole vectors
        int64_t idx = -1;
        if ((int64_t)lane < h0) idx = lane;
        else if (lane >= 8 && (int64_t)(lane - 8) < p.V - tail0) idx = tail0 + (lane - 8);
        float x = idx >= 0 ? load_elem<BF16>(rowp, idx) : 0.0f;
        bool pass = idx >= 0 && !(x < st.thr_f);
        st.offer(x, pass, [&](uint32_t src) {
            return (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)idx, (int)src);
        });
    }

    __shared__ uint64_t sk[4 * kK];
    if (lane < (uint32_t)kK) sk[wave * kK + lane] = st.key;
    __syncthreads();
    if (wave == 0) {
        uint64_t srt = wave_sort64_desc(sk[lane]);
        if (lane < (uint32_t)kK) {
            if (p.nsplit == 1) {
                uint32_t id = key_id(srt);  // always < V: every row has >= 16 real keys
                p.cand_id[row * kK + lane] = (int32_t)id;
                p.cand_u[row * kK + lane] = (int64_t)id < p.V ? load_elem<BF16>(rowp, id) : __builtin_nanf("");
            } else {
                p.partial[(row * p.nsplit + split) * kK + lane] = srt;
            }
        }
    }
}

// Merge the nsplit partial lists of a row: one wave per row, 3 lists per step
// sorted together with the running best 16.
template <bool BF16>
__global__ __launch_bounds__(64) void topk16_merge_kernel(TopkParams p) {
    constexpr int ES = BF16 ? 2 : 4;
    const int64_t row = blockIdx.x;
    const uint32_t lane = lane_id();
    const uint64_t *src = p.partial + row * p.nsplit * kK;
    uint64_t best = 0ull;
    for (int s0 = 0; s0 < p.nsplit; s0 += 3) {
        uint64_t k = best;
        if (lane >= (uint32_t)kK) {
            int s = s0 + (int)(lane - kK) / kK;
            k = s < p.nsplit ? src[s * kK + (lane % kK)] : 0ull;
        }
        best = wave_sort64_desc(k);
    }
    if (lane < (uint32_t)kK) {
        const char *rowp = p.logits + row * p.ld * ES;
        uint32_t id = key_id(best);
        p.cand_id[row * kK + lane] = (int32_t)id;
        p.cand_u[row * kK + lane] = (int64_t)id < p.V ? load_elem<BF16>(rowp, id) : __builtin_nanf("");
    }
}

// Workgroups per row: enough rows x splits to fill 256 CUs several times over,
// but never slices shorter than 4096 elements.
#ifndef DSEL_TOPK_TARGET_WG
#define DSEL_TOPK_TARGET_WG 1024
#endif
inline int topk_nsplit(int64_t rows, int64_t V) {
    if (rows <= 0) return 1;
    int64_t want = (DSEL_TOPK_TARGET_WG + rows - 1) / rows;
    int64_t cap = V / 4096;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want > 256) want = 256;
    return (int)(want < 1 ? 1 : want);
}

}  // namespace dsel
