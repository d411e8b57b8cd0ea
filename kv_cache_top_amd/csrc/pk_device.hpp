// Device helpers shared by the ParisKV kernels (gfx950, wave64).
//
// Vector layout used by every kernel that touches a 128-dim key or query:
// 16 consecutive lanes hold one vector, lane l16 = lane & 15 holding the 8
// coordinates [8*l16, 8*l16+8).  With m = 8 a lane therefore owns exactly one
// subspace of the rotated vector, so ids, codes and scales are lane-local and
// a wave processes four vectors at once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pk {

constexpr int kD = 128;          // head dim
constexpr int kSub = 16;         // bucket-id bytes per key = rows of the scan's vote table
// Subspaces: B = 16 of m = 8 coordinates (one id byte each), or B = 32 of m = 4
// (two 4-bit ids per byte: subspace 2i in the low half of byte i).  Either way
// a key has 16 id bytes, and the vote table the scan reads has one 256-entry
// row per id byte (for m = 4 an entry is the sum of the two subspaces' votes).
// Record of a key: 64 B of nibbles (coordinate 2i in the low half of byte i),
// then B fp32 scales w.
template <int M>
constexpr int rec_bytes() { return 64 + 4 * (kD / M); }   // 128 (m = 8), 192 (m = 4), 96 (m = 16)
// B = 8 subspaces of m = 16 also keep the 16 sign bytes (the id of subspace b
// is the little-endian 16-bit word at byte 2b), but 65536 centroids per
// subspace leave no room for a dense vote row: each subspace gets a 256-slot
// hash table of its (at most G * rho) voted centroids instead, 1 KB of u32
// entries (vote << 16 | centroid; 0 = empty), linear probing from hash16(id).
template <int M>
constexpr int lut_bytes() { return M == 16 ? 8192 : 4096; }   // vote table per unit

__device__ __forceinline__ uint32_t hash16(uint32_t id) {      // Fibonacci hash to 8 bits
    return ((id * 40503u) & 0xffffu) >> 8;
}

// votes of centroid `id` in one subspace's hash table, given the entry `e`
// at its home slot (a bounded probe: the table never holds more than 64 of
// its 256 slots, so an empty slot ends it; an empty home slot reads as vote 0)
__device__ __forceinline__ uint32_t hashed_vote(const uint32_t* tab, uint32_t id, uint32_t e) {
    if ((e & 0xffffu) == id || e == 0u) return e >> 16;
    uint32_t slot = hash16(id);
    for (int k = 0; k < 255; ++k) {
        slot = (slot + 1u) & 255u;
        e = tab[slot];
        if (e == 0u) return 0u;
        if ((e & 0xffffu) == id) return e >> 16;
    }
    return 0u;
}

// coarse score of one key over the 8 hash tables: the 8 home slots are read
// before any is resolved
__device__ __forceinline__ uint32_t hashed_score(const uint32_t* tabs, const uint32_t w[4]) {
    uint32_t id[8], e[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        id[b] = (w[b >> 1] >> (16 * (b & 1))) & 0xffffu;
        e[b] = tabs[256 * b + hash16(id[b])];
    }
    uint32_t sc = 0;
#pragma unroll
    for (int b = 0; b < 8; ++b) sc += hashed_vote(tabs + 256 * b, id[b], e[b]);
    return sc;
}
constexpr int kRhoMax = 8;
constexpr int kMaxBins = 4096;   // coarse-score histogram bins (B * G * max weight + 1)
constexpr int kMaxChunks = 2048; // scan chunks per unit
constexpr int kBlock = 256;      // threads per block of the streaming kernels
// Fourth word of a raw (untyped, stride 0) buffer resource descriptor on the
// gfx9 family: 32-bit data format, offsets checked against the record count
// (loads past it return zero).
constexpr int kBufferRsrcWord3 = 0x00020000;

// Histogram bins per lane of the scan's suffix-count wave: the nbins bins
// spread over 64 lanes in runs of a multiple of 4 (16-byte LDS reads, 8-byte
// stores).  The scan's LDS histogram holds 64 * this many entries.
__host__ __device__ constexpr int scan_bins_per_lane(int nbins) { return 4 * ((nbins + 255) / 256); }

struct CodeTables {
    float sq_thr[7];   // fp32(t_l^2), ascending
    float levels[8];   // fp32 Lloyd-Max levels
    int32_t sub_dim;   // m: 8, 4 or 16
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 8 consecutive elements -> fp32
__device__ __forceinline__ void load8(const float* p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
}

// 8 consecutive elements kept in their storage type until used (bf16 rows
// take 4 VGPRs instead of 8).
// 16-byte load marked nontemporal (streamed once: keeps the cache for data
// that is read again)
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}

template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
    uint4 a;
    __device__ __forceinline__ void load(const uint16_t* p) { a = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void load_stream(const uint16_t* p) {
        a = load_nt(reinterpret_cast<const uint4*>(p));
    }
    __device__ __forceinline__ float operator[](int i) const {
        const uint32_t w = (i >> 1) == 0 ? a.x : (i >> 1) == 1 ? a.y : (i >> 1) == 2 ? a.z : a.w;
        return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
    }
};
template <> struct Raw8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void load_stream(const float* p) {
        const uint4 x = load_nt(reinterpret_cast<const uint4*>(p));
        const uint4 y = load_nt(reinterpret_cast<const uint4*>(p + 4));
        a = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
        b = make_float4(__uint_as_float(y.x), __uint_as_float(y.y), __uint_as_float(y.z), __uint_as_float(y.w));
    }
    __device__ __forceinline__ float operator[](int i) const {
        return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : i == 3 ? a.w
             : i == 4 ? b.x : i == 5 ? b.y : i == 6 ? b.z : b.w;
    }
};

// The 8 sign bits of the SRHT diagonal that fall on lane l16's coordinates.
__device__ __forceinline__ uint32_t lane_sign_byte(uint64_t lo, uint64_t hi, int l16) {
    const uint64_t w = (l16 < 8) ? lo : hi;
    return (uint32_t)(w >> (8 * (l16 & 7))) & 0xffu;
}

__device__ __forceinline__ void apply_signs(float v[8], uint32_t bits) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
        if ((bits >> r) & 1u) v[r] = -v[r];
}

// Lane exchanges inside each row of 16 lanes by DPP (data-parallel
// primitives: the permutation is a modifier of one VALU move, no LDS
// traffic).  xor16<M>(x) returns x of lane (l16 ^ M).  Every lane of the row
// must be active.
//   M = 1, 2: quad permutations [1,0,3,2], [2,3,0,1]
//   M = 4:    half-row mirror (l ^ 7), then quad permutation [3,2,1,0] (l ^ 3)
//   M = 8:    row rotation by 8
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
template <int M>
__device__ __forceinline__ int xor16(int x) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8, "lane mask");
    if constexpr (M == 1) return dpp_mov<0xB1>(x);
    if constexpr (M == 2) return dpp_mov<0x4E>(x);
    if constexpr (M == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(x));
    return dpp_mov<0x128>(x);
}
template <int M>
__device__ __forceinline__ float xor16(float x) {
    return __int_as_float(xor16<M>(__float_as_int(x)));
}

// Unnormalised 128-point Walsh-Hadamard transform across a 16-lane group.
// Stages h = 1, 2, 4 are inside the lane; h = 8, 16, 32, 64 pair lane l16
// with lane l16 ^ (h / 8).  Every butterfly is (a + b, a - b) with a the lower
// index, one IEEE fp32 add/sub, and the stages run in ascending order, so the
// result is bit-identical to any other implementation of that order.
template <int LM>
__device__ __forceinline__ void fwht_lane_stage(float v[8], int l16) {
    const bool upper = (l16 & LM) != 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float o = xor16<LM>(v[r]);
        v[r] = upper ? (o - v[r]) : (v[r] + o);
    }
}
__device__ __forceinline__ void fwht128_g16(float v[8], int l16) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if ((r & h) == 0) {
                const float a = v[r], b = v[r + h];
                v[r] = a + b;
                v[r + h] = a - b;
            }
        }
    }
    fwht_lane_stage<1>(v, l16);
    fwht_lane_stage<2>(v, l16);
    fwht_lane_stage<4>(v, l16);
    fwht_lane_stage<8>(v, l16);
}

// Workgroup barrier that orders LDS accesses only.  Every barrier in these
// kernels exchanges data through LDS; none hands global memory between the
// threads of a block.  Unlike __syncthreads(), it does not wait for the
// wave's outstanding global loads, so loads issued before it stay in flight.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ((t0+t1)+(t2+t3)) + ((t4+t5)+(t6+t7)), fp32
__device__ __forceinline__ float tree8(const float t[8]) {
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// Sum over a row of 16 lanes: pairs, quads, half rows (mirror), rows
// (mirror).  Each step adds the same two operands in every lane of the
// group it joins, so all 16 lanes end with the same value.
__device__ __forceinline__ float sum16(float x) {
    x += xor16<1>(x);
    x += xor16<2>(x);
    x += __int_as_float(dpp_mov<0x141>(__float_as_int(x)));
    x += __int_as_float(dpp_mov<0x140>(__float_as_int(x)));
    return x;
}

// Maximum over a row of 16 lanes (every lane gets it).
__device__ __forceinline__ uint32_t max16(uint32_t x) {
    x = max(x, (uint32_t)xor16<1>((int)x));
    x = max(x, (uint32_t)xor16<2>((int)x));
    x = max(x, (uint32_t)dpp_mov<0x141>((int)x));
    x = max(x, (uint32_t)dpp_mov<0x140>((int)x));
    return x;
}

// Maximum over the wave, returned in every lane (wave-uniform).
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
    x = max16(x);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
    return max(max(a, b), max(c, d));
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele inside each
// row of 16 lanes with zero-filling row shifts (DPP), then the totals of the
// rows below are added.  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_zfill(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_zfill<0x111>(x);   // row_shr:1
    x += dpp_zfill<0x112>(x);   // row_shr:2
    x += dpp_zfill<0x114>(x);   // row_shr:4
    x += dpp_zfill<0x118>(x);   // row_shr:8
    const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
    const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
    const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return x + (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
}

// Sum of x over lanes {l, l^16, l^32, l^48}: the four rows of the wave
// (v_permlane16_swap / v_permlane32_swap exchange rows without LDS).  Both
// lanes of each exchange add the same two operands in the same order.
__device__ __forceinline__ float sum_rows4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Wave-uniform maximum / sum of a float over the 64 lanes.
__device__ __forceinline__ float wave_max_f(float x) {
    x = fmaxf(x, xor16<1>(x));
    x = fmaxf(x, xor16<2>(x));
    x = fmaxf(x, __int_as_float(dpp_mov<0x141>(__float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_mov<0x140>(__float_as_int(x))));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
__device__ __forceinline__ float wave_sum_f(float x) {
    x = sum16(x);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (a + b) + (c + d);
}

// order-preserving map of fp32 to uint32 (larger float -> larger key)
// (-0 and +0 map to the same key, as they compare equal)
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    const uint32_t b = __float_as_uint(f + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// its inverse (a zero comes back as +0)
__device__ __forceinline__ float order_key_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Block-wide exclusive scan of one uint32 per thread for a block of NT
// threads.  `tmp` must hold NT / 64 entries.  Returns the exclusive prefix;
// the block total goes to *total.  Contains two LDS barriers.
// kReuse: a closing barrier, so that tmp can be written again right after
template <int NT, bool kReuse = true>
__device__ __forceinline__ uint32_t block_excl_scan_t(uint32_t v, uint32_t* tmp, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) tmp[wave] = x;
    lds_sync();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t t = tmp[w];
        if (w < wave) before += t;
        all += t;
    }
    if constexpr (kReuse) lds_sync();
    *total = all;
    return before + x - v;
}

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
    return block_excl_scan_t<kBlock>(v, tmp, total);
}

}  // namespace pk
