// Device helpers shared by the selector kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsel {

constexpr int kK = 16;       // candidates per draft position
constexpr int kWave = 64;    // CDNA wavefront width

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lane_id() {
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint32_t shfl_idx32(uint32_t x, uint32_t src_lane) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src_lane << 2), (int)x);
}

__device__ __forceinline__ uint64_t shfl_idx64(uint64_t x, uint32_t src_lane) {
    uint32_t lo = shfl_idx32((uint32_t)x, src_lane);
    uint32_t hi = shfl_idx32((uint32_t)(x >> 32), src_lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t x, uint32_t l) {
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, (int)l);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), (int)l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float shfl_idxf(float x, uint32_t src_lane) {
    return __uint_as_float(shfl_idx32(__float_as_uint(x), src_lane));
}

// Monotone 32-bit image of a float for the candidate order: larger = ranks
// higher.  -0.0 maps like +0.0 and every NaN maps to 0, below -inf (0x007FFFFF).
__device__ __forceinline__ uint32_t order_bits(float v) {
    uint32_t b = __float_as_uint(v);
    if (v != v) return 0u;
    if (b == 0x80000000u) b = 0u;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Candidate key: (order_bits(value), ~id).  A larger key ranks higher; equal
// values rank the lower id higher.  Key 0 is an empty slot (every real key has a
// low word >= 2^31 because ids are < 2^31).
__device__ __forceinline__ uint64_t cand_key(float v, uint32_t id) {
    return ((uint64_t)order_bits(v) << 32) | (uint32_t)(~id);
}

__device__ __forceinline__ uint32_t key_id(uint64_t k) { return ~(uint32_t)k; }

// The value a key was made from, when its order bits identify it exactly:
// false for the two codes that merge several inputs (every NaN, and +0.0 with
// -0.0), whose bits must be read back from the input.
__device__ __forceinline__ bool key_value(uint64_t k, float *v) {
    const uint32_t hi = (uint32_t)(k >> 32);
    if (hi == 0u || hi == 0x80000000u) return false;
    *v = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi);
    return true;
}

// The float a key's value part stands for, used as the fast filter threshold:
// empty or NaN-level keys give -inf so that every element (NaN included, since
// !(NaN < -inf) holds) goes on to the exact key compare.
__device__ __forceinline__ float key_threshold(uint64_t k) {
    uint32_t hi = (uint32_t)(k >> 32);
    if (hi <= 0x007FFFFFu) return -__builtin_inff();
    uint32_t b = (hi & 0x80000000u) ? (hi & 0x7FFFFFFFu) : ~hi;
    return __uint_as_float(b);
}

// Lane-wise signed 16-bit max of two words (v_pk_max_i16).  Read as int16, the
// bits of non-negative bf16 values order like the values, and every negative
// value (sign bit set) lies below them; so for a threshold t > 0, "some bf16 of
// these words is >= t" becomes "some int16 half of their pk_max is >= bits(t)",
// with no unpacking.  (Positive NaNs also pass; callers re-check exactly.)
typedef short short2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(short2v, a),
                                                                  __builtin_bit_cast(short2v, b)));
}
__device__ __forceinline__ uint32_t bf16x8_pk_max(const u32x4 &w) {
    return pk_max_i16(pk_max_i16(w.x, w.y), pk_max_i16(w.z, w.w));
}
// Both halves hold bits(t) - 1 for a bf16 value t > 0: pk_max_i16(m, floor) !=
// floor exactly when a half of m is >= bits(t).
__device__ __forceinline__ uint32_t bf16_pk_floor(float t) {
    return ((__float_as_uint(t) >> 16) - 1u) * 0x10001u;
}

// x of lane (lane ^ J), for J a power of two below 64, without the LDS
// crossbar: DPP quad_perm for 1 and 2; row_ror:4 / row_ror:12 (lane l reads
// (l - 4) or (l + 4) mod 16 of its row) for 4; row_ror:8 for 8; and the gfx950
// row swaps for 16 and 32: with both operands x, v_permlane16_swap returns
// (rows 0, 2: own, rows 1, 3: x[l - 16]) and (rows 0, 2: x[l + 16], rows 1, 3:
// own), v_permlane32_swap likewise across the two 32-lane halves.  Every lane
// must be active.
template <int J>
__device__ __forceinline__ uint32_t xor_lane32(uint32_t x) {
    static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "lane distance");
    if constexpr (J == 1) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);
    } else if constexpr (J == 2) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);
    } else if constexpr (J == 4) {
        const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false);
        const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x12C, 0xF, 0xF, false);
        return (lane_id() & 4u) ? dn : up;
    } else if constexpr (J == 8) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
    } else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane_id() & 16u) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane_id() & 32u) ? r[0] : r[1];
    }
}
template <int J>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t x) {
    return ((uint64_t)xor_lane32<J>((uint32_t)(x >> 32)) << 32) | xor_lane32<J>((uint32_t)x);
}

// One compare-exchange stage of a bitonic network: lanes with bit J clear keep
// the larger key when `desc` holds for them.
template <int J>
__device__ __forceinline__ uint64_t bitonic_stage(uint64_t key, bool desc) {
    const uint64_t other = xor_lane64<J>(key);
    const bool lower = (lane_id() & (uint32_t)J) == 0;
    const uint64_t mx = key > other ? key : other;
    const uint64_t mn = key > other ? other : key;
    return (lower == desc) ? mx : mn;
}

// Bitonic sort of one 64-bit key per lane across the wave, descending
// (lane 0 receives the largest key); every lane must be active.
__device__ __forceinline__ uint64_t wave_sort64_desc(uint64_t key) {
    const uint32_t lane = lane_id();
    key = bitonic_stage<1>(key, (lane & 2u) == 0);
    key = bitonic_stage<2>(key, (lane & 4u) == 0);
    key = bitonic_stage<1>(key, (lane & 4u) == 0);
    key = bitonic_stage<4>(key, (lane & 8u) == 0);
    key = bitonic_stage<2>(key, (lane & 8u) == 0);
    key = bitonic_stage<1>(key, (lane & 8u) == 0);
    key = bitonic_stage<8>(key, (lane & 16u) == 0);
    key = bitonic_stage<4>(key, (lane & 16u) == 0);
    key = bitonic_stage<2>(key, (lane & 16u) == 0);
    key = bitonic_stage<1>(key, (lane & 16u) == 0);
    key = bitonic_stage<16>(key, (lane & 32u) == 0);
    key = bitonic_stage<8>(key, (lane & 32u) == 0);
    key = bitonic_stage<4>(key, (lane & 32u) == 0);
    key = bitonic_stage<2>(key, (lane & 32u) == 0);
    key = bitonic_stage<1>(key, (lane & 32u) == 0);
    key = bitonic_stage<32>(key, true);
    key = bitonic_stage<16>(key, true);
    key = bitonic_stage<8>(key, true);
    key = bitonic_stage<4>(key, true);
    key = bitonic_stage<2>(key, true);
    key = bitonic_stage<1>(key, true);
    return key;
}

// The 8 bf16 or 4 fp32 values of a 16-byte vector, widened to float
template <bool BF16>
__device__ __forceinline__ void widen_vec(const u32x4 &w, float (&x)[BF16 ? 8 : 4]) {
#pragma unroll
    for (int e = 0; e < (BF16 ? 8 : 4); ++e) {
        const uint32_t word = w[BF16 ? e >> 1 : e];
        x[e] = BF16 ? __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16)) : __uint_as_float(word);
    }
}

// Sticky device error word (bits DSEL_DEVERR_*), one per device.  The library
// is a single translation unit, so this is its only definition.
__device__ int g_device_error = 0;

// Ragged batches keep the padded [batch, L] layout with a valid length per
// block.  The valid positions of block b: len[b], or L for a uniform batch
// (len == nullptr).  A length outside [0, L] counts as 0 (the block is empty)
// and sets bit 2 (DSEL_DEVERR_BLOCK_LEN) of the device error word.
__device__ __forceinline__ int block_len_of(const int32_t *len, int64_t b, int L) {
    if (len == nullptr) return L;
    const int n = len[b];
    if (n >= 0 && n <= L) return n;
    atomicOr(&g_device_error, 2);
    return 0;
}

// Is flat position i = b L + t (i < 2^31) of a padded batch a real one
// (t < the length of block b)?  Always, for a uniform batch.
__device__ __forceinline__ bool position_live(const int32_t *len, uint32_t i, int L) {
    if (len == nullptr) return true;
    const uint32_t b = i / (uint32_t)L;
    return (int)(i - b * (uint32_t)L) < block_len_of(len, b, L);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const uint32_t lane = lane_id();
#pragma unroll
    for (uint32_t o = 1; o < 64; o <<= 1) {
        const int y = (int)shfl_idx32((uint32_t)x, lane >= o ? lane - o : lane);
        if (lane >= o) x += y;
    }
    return x;
}

// Compaction of a ragged batch: the flat index b L + t of its w-th real
// position (flat order), or -1 when it has no more than w.  For a uniform
// batch (len == nullptr) that is w itself while w < B L.  Called by a whole
// wave with a wave-uniform w; two rounds of loads and a wave scan (lane k
// first sums the lengths of blocks [k c, k c + c), c = ceil(B / 64), then the
// blocks of the one lane range that holds position w are scanned).  Lets a
// kernel launched for the padded batch put the real positions on its first
// workgroups, so they spread evenly over the chip and the rest exit at once.
__device__ __forceinline__ int64_t live_position(const int32_t *len, int64_t B, int L, int64_t w) {
    if (len == nullptr) return w < B * L ? w : -1;
    const uint32_t lane = lane_id();
    const int64_t c = (B + 63) / 64;
    int s = 0;
    for (int64_t k = 0; k < c; ++k) {
        const int64_t b = (int64_t)lane * c + k;
        if (b < B) s += block_len_of(len, b, L);
    }
    const int incl = wave_incl_scan(s);
    const uint64_t m = ballot((int64_t)incl > w);
    if (m == 0) return -1;
    const uint32_t j = (uint32_t)__builtin_ctzll(m);
    int64_t base = (int64_t)__builtin_amdgcn_readlane(incl - s, (int)j);  // positions before lane j's blocks
    const int64_t b0 = (int64_t)j * c;
    if (c == 1) return b0 * L + (w - base);
    for (int64_t k0 = 0; k0 < c; k0 += 64) {
        const int64_t k = k0 + lane, b = b0 + k;
        const int n = (k < c && b < B) ? block_len_of(len, b, L) : 0;
        const int inc2 = wave_incl_scan(n);
        const uint64_t m2 = ballot(base + inc2 > w);
        if (m2) {
            const uint32_t i = (uint32_t)__builtin_ctzll(m2);
            const int64_t before = base + __builtin_amdgcn_readlane(inc2 - n, (int)i);
            return (b0 + k0 + i) * L + (w - before);
        }
        base += __builtin_amdgcn_readlane(inc2, 63);
    }
    return -1;  // not reached: lane j's blocks hold position w
}

}  // namespace dsel
