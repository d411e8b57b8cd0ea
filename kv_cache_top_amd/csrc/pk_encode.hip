// Per-key encode, per-query preparation and the decode append (gfx950).
//
// ParisKV page, "Drift-robust analytic centroids" (normalisation and shared
// SRHT rotation; sign-pattern centroids), "Coarse candidate generation"
// (nearest centroid per subspace; top-rho centroids per query subspace with
// rank weights), "Candidate reranking (RSQ-IP)" (sign + 3-bit magnitude code,
// calibration scale w computed when the key is stored).
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

// ---------------------------------------------------------------------------
// encode: one 16-lane group per key.  Reads the key row once (256 B bf16 /
// 512 B fp32) and writes 16 B of ids and a 128 B record.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kBlock) void encode_kernel(const T* __restrict__ K, int64_t cap,
                                                         int64_t p0, int64_t count, int64_t total,
                                                         uint8_t* __restrict__ ids,
                                                         uint8_t* __restrict__ rec, uint64_t sign_lo,
                                                         uint64_t sign_hi, CodeTables tab) {
    __shared__ float s_lev[8];
    if (threadIdx.x < 8) s_lev[threadIdx.x] = tab.levels[threadIdx.x];
    lds_sync();

    const int l16 = threadIdx.x & 15;
    const uint32_t sbits = lane_sign_byte(sign_lo, sign_hi, l16);
    const int64_t ngroups = (int64_t)gridDim.x * (kBlock / 16);
    for (int64_t key = (int64_t)blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4); key < total;
         key += ngroups) {
        const int64_t u = key / count;
        const int64_t pos = p0 + (key - u * count);
        const int64_t row = u * cap + pos;
        float v[8];
        load8(K + row * kD + 8 * l16, v);
        apply_signs(v, sbits);
        fwht128_g16(v, l16);

        uint32_t id = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) id |= (v[r] < 0.0f ? 1u : 0u) << r;

        float sq[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) sq[r] = __fmul_rn(v[r], v[r]);
        const float ss = tree8(sq);
        float bound[7];
#pragma unroll
        for (int l = 0; l < 7; ++l) bound[l] = __fmul_rn(tab.sq_thr[l], ss);

        uint32_t packed = 0;
        double s2 = 0.0, s1 = 0.0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            uint32_t mag = 0;
#pragma unroll
            for (int l = 0; l < 7; ++l) mag += (sq[r] >= bound[l]) ? 1u : 0u;
            packed |= ((((id >> r) & 1u) << 3) | mag) << (4 * r);
            const double ax = fabs((double)v[r]);
            s2 += ax * ax;
            s1 += (double)s_lev[mag] * ax;
        }
        float w = 0.0f;
        if (ss == 0.0f) {
            packed = 0;
        } else {
            // w = ||x_b|| / sqrt(d) / <v_b, x_b / ||x_b||> = ||x_b||^2 / (sqrt(d) <v_b, x_b>)
            w = (float)(s2 / (11.313708498984761 * s1));
        }
        ids[row * kSub + l16] = (uint8_t)id;
        uint8_t* r = rec + row * kRec;
        reinterpret_cast<uint32_t*>(r)[l16] = packed;
        reinterpret_cast<float*>(r + 64)[l16] = w;
    }
}

// ---------------------------------------------------------------------------
// query preparation: one 1024-thread block per unit.
//   y_g = H D q_g (spec arithmetic), Ysum = sum_g y_g (for the rerank);
//   per (g, b): top-rho of the 256 centroid scores by (score desc, c asc);
//   vote table L[b][c] = sum_g weight(rank of c).
// A 16-lane group serves one (g, b): lane chi scores the 16 centroids
// c = 16 chi + clo.  Scores come from shared partial sums -- pair sums over
// coordinates (0,1), (2,3), (4,5), (6,7) in their 4 sign variants, then
// quad_lo[c & 15] + quad_hi[c >> 4] -- the same fp32 operations in the same
// order as the direct pairwise tree.  Top-rho = rho rounds of a 16-lane
// argmax, each removing the winner.
// The block may also copy the step's new K/V token into the store.
// ---------------------------------------------------------------------------
struct VoteWeights {
    uint32_t w[kRhoMax];
};

constexpr int kQBlock = 1024;

__device__ __forceinline__ bool better(float s, int c, float ts, int tc) {
    return s > ts || (s == ts && c < tc);
}

template <typename T>
__global__ __launch_bounds__(kQBlock) void qprep_kernel(
    const T* __restrict__ q, int G, uint64_t sign_lo, uint64_t sign_hi, int rho, VoteWeights wts,
    uint8_t* __restrict__ lut, float* __restrict__ ysum,
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, uint8_t* __restrict__ K,
    uint8_t* __restrict__ V, int64_t row_bytes, int64_t cap, int64_t new_pos) {
    const int u = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ float s_y[8][kD];
    __shared__ uint32_t s_lut[kSub * 256];
    for (int i = tid; i < kSub * 256; i += kQBlock) s_lut[i] = 0;
    if (k_new != nullptr) {
        const int per_row = (int)(row_bytes / 16);
        if (tid < per_row) {
            const int64_t dst = ((u * cap + new_pos) * row_bytes) / 16 + tid;
            reinterpret_cast<uint4*>(K)[dst] = k_new[(int64_t)u * per_row + tid];
            reinterpret_cast<uint4*>(V)[dst] = v_new[(int64_t)u * per_row + tid];
        }
    }
    if (tid < 16 * G) {
        const int g = tid >> 4, l16 = tid & 15;
        float v[8];
        load8(q + ((int64_t)u * G + g) * kD + 8 * l16, v);
        apply_signs(v, lane_sign_byte(sign_lo, sign_hi, l16));
        fwht128_g16(v, l16);
#pragma unroll
        for (int r = 0; r < 8; ++r) s_y[g][8 * l16 + r] = v[r];
    }
    lds_sync();
    if (tid < kD) {
        float a = s_y[0][tid];
        for (int g = 1; g < G; ++g) a += s_y[g][tid];
        ysum[(int64_t)u * kD + tid] = a;
    }

    const int combos = G * kSub;
    const int chi = tid & 15;
    for (int base = 0; base < combos; base += kQBlock / 16) {
        const int combo = base + (tid >> 4);
        const bool active = combo < combos;
        const int g = active ? combo / kSub : 0, b = combo % kSub;
        const float* y = &s_y[g][8 * b];
        float p01[4], p23[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p01[i] = ((i & 1) ? -y[0] : y[0]) + ((i & 2) ? -y[1] : y[1]);
            p23[i] = ((i & 1) ? -y[2] : y[2]) + ((i & 2) ? -y[3] : y[3]);
        }
        const float y4 = (chi & 1) ? -y[4] : y[4], y5 = (chi & 2) ? -y[5] : y[5];
        const float y6 = (chi & 4) ? -y[6] : y[6], y7 = (chi & 8) ? -y[7] : y[7];
        const float qhi = (y4 + y5) + (y6 + y7);
        float sc[16];
#pragma unroll
        for (int clo = 0; clo < 16; ++clo) sc[clo] = (p01[clo & 3] + p23[clo >> 2]) + qhi;
        uint32_t removed = 0;
        for (int r = 0; r < rho; ++r) {
            float bs = -INFINITY;
            int bc = 0x7fffffff;
#pragma unroll
            for (int clo = 0; clo < 16; ++clo) {
                const int c = chi * 16 + clo;
                if (!((removed >> clo) & 1u) && better(sc[clo], c, bs, bc)) {
                    bs = sc[clo];
                    bc = c;
                }
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
                const float os = __shfl_xor(bs, m, 16);
                const int oc = __shfl_xor(bc, m, 16);
                if (better(os, oc, bs, bc)) {
                    bs = os;
                    bc = oc;
                }
            }
            if ((bc >> 4) == chi) removed |= 1u << (bc & 15);
            if (active && chi == 0) atomicAdd(&s_lut[b * 256 + bc], wts.w[r]);
        }
    }
    lds_sync();
    uint32_t* out = reinterpret_cast<uint32_t*>(lut + (int64_t)u * kSub * 256);
    for (int i = tid; i < kSub * 256 / 4; i += kQBlock) {
        out[i] = (s_lut[4 * i] & 0xffu) | ((s_lut[4 * i + 1] & 0xffu) << 8) |
                 ((s_lut[4 * i + 2] & 0xffu) << 16) | ((s_lut[4 * i + 3] & 0xffu) << 24);
    }
}

// ---------------------------------------------------------------------------
// decode append: copy one token per unit into the store at position pos
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void append_kernel(const uint4* __restrict__ k_new,
                                                         const uint4* __restrict__ v_new,
                                                         uint8_t* __restrict__ K,
                                                         uint8_t* __restrict__ V, int64_t row_bytes,
                                                         int64_t cap, int64_t pos, int units) {
    const int per_row = (int)(row_bytes / 16);
    const int64_t n = (int64_t)units * per_row;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t u = i / per_row, j = i - u * per_row;
        const int64_t dst = ((u * cap + pos) * row_bytes) / 16 + j;
        reinterpret_cast<uint4*>(K)[dst] = k_new[i];
        reinterpret_cast<uint4*>(V)[dst] = v_new[i];
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_encode(bool bf16, const void* K, int64_t cap, int units, int64_t p0,
                         int64_t count, uint8_t* ids, uint8_t* rec, const uint64_t sign[2],
                         const CodeTables& tab, hipStream_t st) {
    const int64_t total = (int64_t)units * count;
    if (total <= 0) return hipSuccess;
    const int64_t groups_needed = total;
    int64_t blocks = (groups_needed + (kBlock / 16) - 1) / (kBlock / 16);
    if (blocks > 65536) blocks = 65536;
    if (bf16)
        encode_kernel<uint16_t><<<dim3((unsigned)blocks), dim3(kBlock), 0, st>>>(
            (const uint16_t*)K, cap, p0, count, total, ids, rec, sign[0], sign[1], tab);
    else
        encode_kernel<float><<<dim3((unsigned)blocks), dim3(kBlock), 0, st>>>(
            (const float*)K, cap, p0, count, total, ids, rec, sign[0], sign[1], tab);
    return hipGetLastError();
}

hipError_t launch_qprep(bool bf16, const void* q, int units, int G, const uint64_t sign[2],
                        int rho, const uint8_t* weights, uint8_t* lut, float* ysum,
                        const void* k_new, const void* v_new, void* K, void* V, int64_t row_bytes,
                        int64_t cap, int64_t new_pos, hipStream_t st) {
    VoteWeights w;
    for (int i = 0; i < kRhoMax; ++i) w.w[i] = (i < rho) ? weights[i] : 0u;
    if (bf16)
        qprep_kernel<uint16_t><<<dim3(units), dim3(kQBlock), 0, st>>>(
            (const uint16_t*)q, G, sign[0], sign[1], rho, w, lut, ysum,
            (const uint4*)k_new, (const uint4*)v_new, (uint8_t*)K, (uint8_t*)V, row_bytes, cap,
            new_pos);
    else
        qprep_kernel<float><<<dim3(units), dim3(kQBlock), 0, st>>>(
            (const float*)q, G, sign[0], sign[1], rho, w, lut, ysum,
            (const uint4*)k_new, (const uint4*)v_new, (uint8_t*)K, (uint8_t*)V, row_bytes, cap,
            new_pos);
    return hipGetLastError();
}

hipError_t launch_append(const void* k_new, const void* v_new, void* K, void* V,
                         int64_t row_bytes, int64_t cap, int64_t pos, int units, hipStream_t st) {
    const int64_t n = (int64_t)units * (row_bytes / 16);
    const int blocks = (int)((n + kBlock - 1) / kBlock);
    append_kernel<<<dim3(blocks), dim3(kBlock), 0, st>>>((const uint4*)k_new, (const uint4*)v_new,
                                                          (uint8_t*)K, (uint8_t*)V, row_bytes, cap,
                                                          pos, units);
    return hipGetLastError();
}

}  // namespace pk
