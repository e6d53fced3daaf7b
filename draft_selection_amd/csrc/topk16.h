// select_topk: the 16 best candidates of every draft position.
// ("DFlash 2: Keep Drafting Parallel", Method > Lightweight Path Selector: the
// selector keeps the top-16 candidates of each position.)
//
// HBM-bound streaming selection.  One workgroup (4 waves) scans one row, or a
// 1/nsplit slice of it when there are too few rows to fill the chip; its waves
// take turns chunk by chunk over one contiguous stretch, with 16-byte
// non-temporal loads.  Every wave keeps its running top-16 as one 64-bit key
// per lane in lanes 0..15 (sorted, lane 0 best) and filters incoming elements
// against the value of its 16th key: almost every chunk fails that single
// compare, and the rare survivors are inserted one at a time (a DPP shift of
// the list).  The first chunk of a wave seeds the list with its sorted lane
// maxima (the 16 best of them bound the rest).  Loads are buffered three or
// four deep in registers, so a chunk's HBM latency hides behind the previous
// chunks' filters.  Waves merge through LDS with a 64-key bitonic sort (DPP and
// permlane swaps); split rows merge in a second kernel, one workgroup per row.
// On a ragged batch the real rows are compacted onto the first workgroups of
// the padded grid (live_position), so that they spread evenly over the chip.
#pragma once

#include "common.h"

#ifndef DSEL_TOPK_INTERLEAVE
#define DSEL_TOPK_INTERLEAVE 1
#endif
// Register buffers per wave: DEPTH - 1 chunks in flight while one is filtered
// (MI355X, 1,024 bf16 rows of 151,936: 3 is 1-2 us faster than 2, and 4-5 us
// faster on ragged batches of the 5 / 8 / 16 mix; 4 is 1.2 us faster again,
// 2.2 us at 1,024 rows of 152,064; fp32 rows of 202,048 level between 3 and 4).
#ifndef DSEL_TOPK_DEPTH_BF16
#define DSEL_TOPK_DEPTH_BF16 4
#endif
#ifndef DSEL_TOPK_DEPTH_F32
#define DSEL_TOPK_DEPTH_F32 3
#endif
// Waves per row workgroup, 4 or 8 (MI355X, 1,024 bf16 rows of 151,936: 54.5 us
// at 4 waves against 60.3 at 8, which doubles each row's loads in flight).
#ifndef DSEL_TOPK_WAVES
#define DSEL_TOPK_WAVES 4
#endif

namespace dsel {

constexpr int kTopkWaves = DSEL_TOPK_WAVES;
static_assert(kTopkWaves == 4 || kTopkWaves == 8, "top-16 waves per workgroup");

// 16-byte vectors per lane and chunk (a wave's chunk is 64 U vectors).  Measured
// on MI355X (one row per workgroup, 1,024 rows): bf16 rows of 151,936 take
// 54.8 us at U = 2 against 57.8 at 4, 58.3 at 1 and 74.9 at 8; fp32 rows of
// 202,048 (4,096 rows) are level between 2 and 4 and 2% faster at 4 when a
// ragged batch leaves fewer rows.
#ifndef DSEL_TOPK_UNROLL_BF16
#define DSEL_TOPK_UNROLL_BF16 2
#endif
#ifndef DSEL_TOPK_UNROLL_F32
#define DSEL_TOPK_UNROLL_F32 4
#endif
template <bool BF16>
constexpr int kTopkUnroll = BF16 ? DSEL_TOPK_UNROLL_BF16 : DSEL_TOPK_UNROLL_F32;

struct TopkParams {
    const char *logits;   // row r starts at logits + r * ld * elem_size
    int64_t rows, V, ld;  // ld in elements
    int nsplit;           // workgroups per row
    int L;                // positions per block (row r is position r % L of block r / L)
    const int32_t *len;   // ragged batch: valid positions per block (nullptr: all L)
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
//
// The waves of a workgroup share a bound through LDS: each publishes the
// value half (order bits) of its 4th and 16th keys.  Every list holds
// distinct elements of the row, so with b = max(max over waves of the 16th,
// min over waves of the 4th) at least 16 elements of the row have order bits
// >= b; an element whose order bits are below b is not among the row's 16
// best, and an element that is passes every wave's filter until the end.  So
// a wave filters against max(its own 16th key, b << 32), which (the 4th-key
// term above all) rises far faster than its own 16th key alone.
struct WaveTop {
    uint64_t key;
    uint64_t own;       // key of the wave's own 16th entry (wave-uniform)
    uint64_t thr;       // filter key: max(own, bound << 32) (wave-uniform)
    float thr_f;        // its value as a filter threshold (wave-uniform)
    uint32_t bound;     // the workgroup bound last read
    uint32_t *pub;      // LDS: this wave's two published order halves
    const uint32_t *all;  // LDS: every wave's, kTopkWaves x {4th, 16th}

    __device__ __forceinline__ void set_thr() {
        const uint64_t b = (uint64_t)bound << 32;
        thr = own > b ? own : b;
        thr_f = key_threshold(thr);
    }
    __device__ __forceinline__ void refresh() {
        own = readlane64(key, 15);
        const uint32_t h3 = (uint32_t)(readlane64(key, 3) >> 32);
        if (lane_id() == 0u) {
            pub[0] = h3;
            pub[1] = (uint32_t)(own >> 32);
        }
        set_thr();
    }
    // Read the other waves' halves (at most a few chunks old: both only rise).
    __device__ __forceinline__ void sync() {
        uint32_t mx16 = 0u, mn4 = 0xFFFFFFFFu;
#pragma unroll
        for (int v = 0; v < kTopkWaves; ++v) {
            const uint32_t a = all[2 * v], b = all[2 * v + 1];
            mn4 = a < mn4 ? a : mn4;
            mx16 = b > mx16 ? b : mx16;
        }
        const uint32_t nb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(mx16 > mn4 ? mx16 : mn4));
        if (nb > bound) {
            bound = nb;
            set_thr();
        }
    }
    // Insert a wave-uniform key known to rank above thr.  The list is DPP row
    // 0 (lanes 0..15), so the shift by one slot is a row_shr:1 of both halves
    // (VALU, no trip through the LDS crossbar).
    __device__ __forceinline__ void insert(uint64_t c) {
        const uint32_t lane = lane_id();
        bool gt = lane < (uint32_t)kK && c > key;
        uint64_t m = ballot(gt);
        const uint32_t plo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)key, 0x111, 0xF, 0xF, false);
        const uint32_t phi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(key >> 32), 0x111, 0xF, 0xF, false);
        uint64_t prev = ((uint64_t)phi << 32) | plo;  // key of lane - 1 (lanes 1..15)
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

// One chunk = U vectors of 16 bytes per lane (U x 64 vectors per wave), at
// vector index v0 + u * 64 + lane.  Loads are always issued (indices past the
// wave's range `ve` are clamped to its last vector and flagged in `ok`) so the
// compiler's wait counts never depend on a branch, and the next chunk's loads
// can be in flight while this one is filtered.
template <int U>
__device__ __forceinline__ void load_chunk(u32x4 (&w)[U], const u32x4 *vbase, int64_t v0, int64_t ve) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t vi = v0 + u * kWave + lane;
        vi = vi < ve ? vi : ve - 1;
        w[u] = __builtin_nontemporal_load(vbase + vi);
    }
}

// Largest element of the lane's chunk (invalid vectors excluded), as a float.
// v_max ignores NaN, so a NaN-only chunk gives NaN, which passes the
// `!(max < thr)` screen like NaN itself would.
template <bool BF16, int U>
__device__ __forceinline__ float chunk_max(const u32x4 (&w)[U], int64_t v0, int64_t ve) {
    const uint32_t lane = lane_id();
    float m = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = v0 + u * kWave + lane < ve;
        float mu;
        if constexpr (BF16) {
            const float a0 = __uint_as_float(w[u].x << 16), a1 = __uint_as_float(w[u].x & 0xFFFF0000u);
            const float b0 = __uint_as_float(w[u].y << 16), b1 = __uint_as_float(w[u].y & 0xFFFF0000u);
            const float c0 = __uint_as_float(w[u].z << 16), c1 = __uint_as_float(w[u].z & 0xFFFF0000u);
            const float d0 = __uint_as_float(w[u].w << 16), d1 = __uint_as_float(w[u].w & 0xFFFF0000u);
            mu = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(a0, a1), __builtin_fmaxf(b0, b1)),
                                 __builtin_fmaxf(__builtin_fmaxf(c0, c1), __builtin_fmaxf(d0, d1)));
        } else {
            mu = __builtin_fmaxf(__builtin_fmaxf(__uint_as_float(w[u].x), __uint_as_float(w[u].y)),
                                 __builtin_fmaxf(__uint_as_float(w[u].z), __uint_as_float(w[u].w)));
        }
        m = ok ? __builtin_fmaxf(m, mu) : m;
    }
    return m;
}

// Offer every element of the chunk that passes the threshold (exact path).
// `skip` (first chunk only) is the element the seed already holds.
template <bool BF16, int U>
__device__ __forceinline__ void chunk_offer(WaveTop &st, const u32x4 (&w)[U], int64_t v0, int64_t ve,
                                            int64_t h0, int skip) {
    constexpr int EPV = BF16 ? 8 : 4;
    const uint32_t lane = lane_id();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = v0 + u * kWave + lane < ve;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const float x = vec_elem<BF16>(w[u], e);
            const bool p = ok && !(x < st.thr_f) && (u * EPV + e != skip);
            const int64_t vrow = v0 + u * kWave;
            st.offer(x, p, [&](uint32_t src) { return (uint32_t)(h0 + (vrow + src) * EPV + e); });
        }
    }
}

// Filter one chunk: a single compare of the lane's chunk maximum screens out
// (almost) every chunk once the list has filled.
// For bf16 rows with a positive threshold the screen works on the packed bits
// (pk_max_i16); a clamped duplicate vector past the range can only cause an
// extra exact pass, which checks each element's range itself.
template <bool BF16, int U>
__device__ __forceinline__ void chunk_filter(WaveTop &st, const u32x4 (&w)[U], int64_t v0, int64_t ve,
                                             int64_t h0) {
    st.sync();
    if constexpr (BF16) {
        if (st.thr_f > 0.0f) {  // wave-uniform; thr_f is itself a bf16 value
            const uint32_t floor = bf16_pk_floor(st.thr_f);
            uint32_t m = floor;
#pragma unroll
            for (int u = 0; u < U; ++u) m = pk_max_i16(m, bf16x8_pk_max(w[u]));
            if (ballot(m != floor) == 0) return;
            chunk_offer<BF16, U>(st, w, v0, ve, h0, -1);
            return;
        }
    }
    const float m = chunk_max<BF16, U>(w, v0, ve);
    if (ballot(!(m < st.thr_f)) == 0) return;
    chunk_offer<BF16, U>(st, w, v0, ve, h0, -1);
}

// First chunk of a wave: seed the list with the 16 best lane maxima (real
// elements, so they bound the rest), then offer the remaining elements.
template <bool BF16, int U>
__device__ __forceinline__ void chunk_seed(WaveTop &st, const u32x4 (&w)[U], int64_t v0, int64_t ve,
                                           int64_t h0) {
    constexpr int EPV = BF16 ? 8 : 4;
    const uint32_t lane = lane_id();
    uint64_t best = 0;
    int skip = -1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = v0 + u * kWave + lane < ve;
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const uint64_t k = cand_key(vec_elem<BF16>(w[u], e),
                                        (uint32_t)(h0 + (v0 + u * kWave + lane) * EPV + e));
            if (ok && k > best) {
                best = k;
                skip = u * EPV + e;
            }
        }
    }
    const uint64_t srt = wave_sort64_desc(best);
    st.key = lane < (uint32_t)kK ? srt : 0ull;
    st.refresh();
    chunk_offer<BF16, U>(st, w, v0, ve, h0, skip);
}

// The work of workgroup `bid`: split `bid % nsplit` of row `bid / nsplit`.
template <bool BF16, int U>
__device__ __forceinline__ void topk16_block(const TopkParams &p, int64_t bid) {
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int EPV = 16 / ES;
    // a ragged batch's real rows go to the first workgroups (compaction), so
    // they spread evenly over the XCDs and the rest exit at once
    const int64_t row = p.len ? live_position(p.len, p.rows / p.L, p.L, bid / p.nsplit) : bid / p.nsplit;
    const int split = (int)(bid % p.nsplit);
    if (row < 0) return;  // past the last real row (ragged batches)
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

#if DSEL_TOPK_INTERLEAVE
    // The workgroup owns vectors [wb, we) of the row; its waves take turns
    // chunk by chunk, so the four waves sweep one contiguous stretch together.
    const int64_t wb = nvec * split / p.nsplit, we = nvec * (split + 1) / p.nsplit;
    const int64_t gw = (int64_t)split * kTopkWaves + wave;
#else
    const int64_t nw = (int64_t)p.nsplit * kTopkWaves;
    const int64_t gw = (int64_t)split * kTopkWaves + wave;
    const int64_t vb = nvec * gw / nw, ve = nvec * (gw + 1) / nw;
#endif

    // published order halves of every wave (0: nothing yet, below every key)
    __shared__ uint32_t s_bound[2 * kTopkWaves];
    if (lane < 2u) s_bound[2 * wave + lane] = 0u;
    __syncthreads();
    WaveTop st;
    st.key = 0ull;
    st.own = 0ull;
    st.bound = 0u;
    st.pub = &s_bound[2 * wave];
    st.all = s_bound;
    st.set_thr();

    // Stream the wave's range chunk by chunk, the next chunks' loads always in
    // flight while the current one is filtered (DSEL_TOPK_DEPTH register buffers).
    constexpr int STEP = U * kWave;
#if DSEL_TOPK_INTERLEAVE
    constexpr int64_t CS = kTopkWaves * STEP;  // distance between a wave's chunks
    const int64_t vb = wb + wave * STEP, ve = we;
    if (vb < ve) {
        const int64_t nch = (ve - vb + CS - 1) / CS;
#else
    constexpr int64_t CS = STEP;
    if (vb < ve) {
        const int64_t nch = (ve - vb + CS - 1) / CS;
#endif
        constexpr int DEPTH = BF16 ? DSEL_TOPK_DEPTH_BF16 : DSEL_TOPK_DEPTH_F32;
        static_assert(DEPTH >= 2 && DEPTH <= 4, "top-16 stream depth");
        if constexpr (DEPTH == 4) {
            u32x4 wa[U], wb2[U], wc[U], wd[U];
            load_chunk<U>(wa, vbase, vb, ve);
            load_chunk<U>(wb2, vbase, vb + CS, ve);
            load_chunk<U>(wc, vbase, vb + 2 * CS, ve);
            load_chunk<U>(wd, vbase, vb + 3 * CS, ve);
            chunk_seed<BF16, U>(st, wa, vb, ve, h0);
            for (int64_t c = 1; c < nch; c += 4) {
                const int64_t v0 = vb + c * CS;
                load_chunk<U>(wa, vbase, v0 + 3 * CS, ve);
                chunk_filter<BF16, U>(st, wb2, v0, ve, h0);
                if (c + 1 >= nch) break;
                load_chunk<U>(wb2, vbase, v0 + 4 * CS, ve);
                chunk_filter<BF16, U>(st, wc, v0 + CS, ve, h0);
                if (c + 2 >= nch) break;
                load_chunk<U>(wc, vbase, v0 + 5 * CS, ve);
                chunk_filter<BF16, U>(st, wd, v0 + 2 * CS, ve, h0);
                if (c + 3 >= nch) break;
                load_chunk<U>(wd, vbase, v0 + 6 * CS, ve);
                chunk_filter<BF16, U>(st, wa, v0 + 3 * CS, ve, h0);
            }
        } else if constexpr (DEPTH == 3) {
            // three register buffers: two chunks in flight while one is filtered
            u32x4 wa[U], wb2[U], wc[U];
            load_chunk<U>(wa, vbase, vb, ve);
            load_chunk<U>(wb2, vbase, vb + CS, ve);
            load_chunk<U>(wc, vbase, vb + 2 * CS, ve);
            chunk_seed<BF16, U>(st, wa, vb, ve, h0);
            for (int64_t c = 1; c < nch; c += 3) {
                const int64_t v0 = vb + c * CS;
                load_chunk<U>(wa, vbase, v0 + 2 * CS, ve);
                chunk_filter<BF16, U>(st, wb2, v0, ve, h0);
                if (c + 1 >= nch) break;
                load_chunk<U>(wb2, vbase, v0 + 3 * CS, ve);
                chunk_filter<BF16, U>(st, wc, v0 + CS, ve, h0);
                if (c + 2 >= nch) break;
                load_chunk<U>(wc, vbase, v0 + 4 * CS, ve);
                chunk_filter<BF16, U>(st, wa, v0 + 2 * CS, ve, h0);
            }
        } else {
            u32x4 wa[U], wb2[U];
            load_chunk<U>(wa, vbase, vb, ve);
            load_chunk<U>(wb2, vbase, vb + CS, ve);
            chunk_seed<BF16, U>(st, wa, vb, ve, h0);
            for (int64_t c = 1; c < nch; c += 2) {
                const int64_t v0 = vb + c * CS;
                load_chunk<U>(wa, vbase, v0 + CS, ve);
                chunk_filter<BF16, U>(st, wb2, v0, ve, h0);
                if (c + 1 >= nch) break;
                load_chunk<U>(wb2, vbase, v0 + 2 * CS, ve);
                chunk_filter<BF16, U>(st, wa, v0 + CS, ve, h0);
            }
        }
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

    __shared__ uint64_t sk[kTopkWaves * kK];
    if (lane < (uint32_t)kK) sk[wave * kK + lane] = st.key;
    __syncthreads();
    if constexpr (kTopkWaves == 8) {
        // waves 0 and 4 each sort four lists; wave 0 then sorts the two bests
        uint64_t best = 0ull;
        if (wave == 0 || wave == 4) best = wave_sort64_desc(sk[wave * kK + lane]);
        __syncthreads();
        if ((wave == 0 || wave == 4) && lane < (uint32_t)kK) sk[(wave / 4) * kK + lane] = best;
        __syncthreads();
    }
    if (wave == 0) {
        uint64_t srt = wave_sort64_desc(kTopkWaves == 8 ? (lane < 2u * kK ? sk[lane] : 0ull) : sk[lane]);
        if (lane < (uint32_t)kK) {
            if (p.nsplit == 1) {
                uint32_t id = key_id(srt);  // always < V: every row has >= 16 real keys
                p.cand_id[row * kK + lane] = (int32_t)id;
                float u;  // the logit, from the key (no memory round trip) unless it is 0 or NaN
                if (!key_value(srt, &u)) u = (int64_t)id < p.V ? load_elem<BF16>(rowp, id) : __builtin_nanf("");
                p.cand_u[row * kK + lane] = u;
            } else {
                p.partial[(row * p.nsplit + split) * kK + lane] = srt;
            }
        }
    }
}

template <bool BF16, int U>
__global__ __launch_bounds__(64 * kTopkWaves) void topk16_kernel(TopkParams p) {
    topk16_block<BF16, U>(p, blockIdx.x);
}

// Fold lists s0, s0 + 1, s0 + 2, then s0 + step, ... of the nsplit sorted
// partial lists of a row (16 keys each, at src) into a wave's running best 16
// (lanes 0..15, sorted): one 64-key sort per 3 lists.
__device__ __forceinline__ uint64_t wave_fold_lists(const uint64_t *src, int nsplit, int s0, int step,
                                                    uint64_t best) {
    const uint32_t lane = lane_id();
    for (; s0 < nsplit; s0 += step) {
        uint64_t k = best;
        if (lane >= (uint32_t)kK) {
            const int s = s0 + (int)(lane - kK) / kK;
            k = s < nsplit ? src[s * kK + (lane % kK)] : 0ull;
        }
        best = wave_sort64_desc(k);
    }
    return best;
}

// Top 16 of the sorted lists held by 16-lane rows r and r ^ (D / 16) (D = 16
// or 32), sorted, in both rows.  The elementwise maximum of one list and the
// other reversed is a bitonic sequence that holds the 16 best of the two; four
// half-cleaner stages sort it (Batcher's bitonic merge).
template <int D>
__device__ __forceinline__ uint64_t merge_row_lists(uint64_t k) {
    constexpr int kMirror = 0x140;  // DPP row_mirror: lane j of a row reads lane 15 - j
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, kMirror, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), kMirror, 0xF, 0xF, false);
    const uint64_t other = xor_lane64<D>(((uint64_t)hi << 32) | lo);
    k = k > other ? k : other;
    k = bitonic_stage<8>(k, true);
    k = bitonic_stage<4>(k, true);
    k = bitonic_stage<2>(k, true);
    return bitonic_stage<1>(k, true);
}

// Top 16, sorted, in lanes 0..15, of the nsplit sorted lists of a row (16 keys
// each, at src, in LDS or global memory): the running best and three new lists
// sit in the wave's four 16-lane rows and are merged pairwise, then the pairs'
// results (two bitonic merges per three lists).
__device__ __forceinline__ uint64_t wave_merge_lists(const uint64_t *src, int nsplit) {
    const uint32_t lane = lane_id();
    const int row = (int)(lane >> 4), j = (int)(lane & 15);
    uint64_t best = 0ull;
    for (int s0 = 0; s0 < nsplit; s0 += 3) {
        const int s = s0 + row - 1;
        uint64_t k = row == 0 ? best : (s < nsplit ? src[s * kK + j] : 0ull);
        k = merge_row_lists<16>(k);
        best = merge_row_lists<32>(k);
    }
    return best;
}

// The value of a merged key: from the key itself, or for the two codes that
// merge several inputs (NaN, and +0.0 with -0.0) the exact bits read back from
// the row (rowp == nullptr: NaN, or +0.0).
template <bool BF16>
__device__ __forceinline__ float merged_value(uint64_t key, const char *rowp, int64_t V) {
    float u;
    if (key_value(key, &u)) return u;
    const uint32_t id = key_id(key);
    if (rowp) return (int64_t)id < V ? load_elem<BF16>(rowp, id) : __builtin_nanf("");
    return (uint32_t)(key >> 32) == 0u ? __builtin_nanf("") : 0.0f;
}

// Merge the nsplit partial lists of a row: one workgroup (4 waves) per row.
// With logits == nullptr (lists from the LM-head kernel) a zero value comes out
// as +0.0.
// Wave w folds lists 3w, 3w+1, 3w+2, then 3w+12, ... into its running best 16
// (one 64-key sort per 3 lists), and wave 0 sorts the four waves' lists.
template <bool BF16>
__global__ __launch_bounds__(256) void topk16_merge_kernel(TopkParams p) {
    constexpr int ES = BF16 ? 2 : 4;
    const int64_t row = p.len ? live_position(p.len, p.rows / p.L, p.L, blockIdx.x) : (int64_t)blockIdx.x;
    if (row < 0) return;  // past the last real row (ragged batches)
    const uint32_t lane = lane_id();
    const int wave = (int)(threadIdx.x / kWave);
    const uint64_t *src = p.partial + row * p.nsplit * kK;
    uint64_t best = wave_fold_lists(src, p.nsplit, 3 * wave, 12, 0ull);
    __shared__ uint64_t sk[4 * kK];
    if (lane < (uint32_t)kK) sk[wave * kK + lane] = best;
    __syncthreads();
    if (wave != 0) return;
    best = wave_sort64_desc(sk[lane]);
    if (lane < (uint32_t)kK) {
        p.cand_id[row * kK + lane] = (int32_t)key_id(best);
        p.cand_u[row * kK + lane] = merged_value<BF16>(best, p.logits ? p.logits + row * p.ld * ES : nullptr, p.V);
    }
}

// Workgroups per row: below 512 rows, enough rows x splits to fill 256 CUs
// four times over, but never slices shorter than 4096 elements; from 512 rows
// on, one workgroup per row (the merge launch costs more than the balance it
// buys).  Measured with bf16 rows of 151,936 against a target of 512
// workgroups: 16 rows 14.5 against 15.1 us, 256 rows 30.9 against 33.6 us,
// 64 rows 20.5 against 20.0 us; splitting 512 or 768 rows in two was 10-15%
// slower than not splitting them.
#ifndef DSEL_TOPK_TARGET_WG
#define DSEL_TOPK_TARGET_WG 1024
#endif
inline int topk_nsplit(int64_t rows, int64_t V) {
    if (rows <= 0 || rows >= 512) return 1;
    int64_t want = (DSEL_TOPK_TARGET_WG + rows - 1) / rows;
    int64_t cap = V / 4096;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want > 256) want = 256;
    return (int)(want < 1 ? 1 : want);
}

}  // namespace dsel
