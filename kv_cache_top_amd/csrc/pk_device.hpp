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
constexpr int kSub = 16;         // B
constexpr int kSubDim = 8;       // m
constexpr int kRec = 128;        // record bytes per key: 64 B nibbles + 16 x f32 w
constexpr int kRhoMax = 8;
constexpr int kMaxBins = 4096;   // coarse-score histogram bins (B * G * max weight + 1)
constexpr int kMaxChunks = 2048; // scan chunks per unit
constexpr int kBlock = 256;      // threads per block of the streaming kernels

struct CodeTables {
    float sq_thr[7];   // fp32(t_l^2), ascending
    float levels[8];   // fp32 Lloyd-Max levels
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

// Unnormalised 128-point Walsh-Hadamard transform across a 16-lane group.
// Stages h = 1, 2, 4 are inside the lane; h = 8, 16, 32, 64 pair lane l16
// with lane l16 ^ (h / 8).  Every butterfly is (a + b, a - b) with a the lower
// index, one IEEE fp32 add/sub, and the stages run in ascending order, so the
// result is bit-identical to any other implementation of that order.
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
#pragma unroll
    for (int lm = 1; lm < 16; lm <<= 1) {
        const bool upper = (l16 & lm) != 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float o = __shfl_xor(v[r], lm, 16);
            v[r] = upper ? (o - v[r]) : (v[r] + o);
        }
    }
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

__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 8, 16);
    x += __shfl_xor(x, 4, 16);
    x += __shfl_xor(x, 2, 16);
    x += __shfl_xor(x, 1, 16);
    return x;
}

// order-preserving map of fp32 to uint32 (larger float -> larger key)
// (-0 and +0 map to the same key, as they compare equal)
__device__ __forceinline__ uint32_t f32_order_key(float f) {
    const uint32_t b = __float_as_uint(f + 0.0f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block-wide exclusive scan of one uint32 per thread for a block of NT
// threads.  `tmp` must hold NT / 64 entries.  Returns the exclusive prefix;
// the block total goes to *total.  Contains two LDS barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_t(uint32_t v, uint32_t* tmp, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    lds_sync();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const uint32_t t = tmp[w];
        if (w < wave) before += t;
        all += t;
    }
    lds_sync();
    *total = all;
    return before + x - v;
}

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
    return block_excl_scan_t<kBlock>(v, tmp, total);
}

}  // namespace pk
