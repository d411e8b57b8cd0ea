// Fine top-k selection over the reranked candidates (gfx950), device code
// shared by the selection kernel and the fused selection + hot-zone
// attention kernel.
#pragma once

#include "pk_device.hpp"

namespace pk {

// ---------------------------------------------------------------------------
// fine top-k: one 1024-thread block per unit.  The k-th largest estimate is
// found by value bucketing: 2048 equal-width buckets over [min, max] (the
// bucket index (v - min) * 2048 / (max - min), truncated, is non-decreasing
// in v, so higher buckets hold only larger values), a digit search for the
// bucket holding the k-th, and an exact rank count among that bucket's
// members.  If the bucket is too full (or the range degenerate), an
// MSB-first radix select over the order keys in three passes (11, 11, 10
// bits) decides instead.  Then compaction in candidate (= position) order,
// each thread owning a contiguous segment; ties at the k-th go to the lower
// positions.
// Up to kFineReg candidates, thread t keeps its segment [t*SEG, t*SEG+SEG)
// in registers for every pass; beyond that the passes stream the estimates
// from memory.
// ---------------------------------------------------------------------------
constexpr int kFBlock = 1024;
constexpr int kFineReg = 16 * kFBlock;  // candidates held in registers
constexpr int kRadixBins = 2048;
constexpr int kRankMax = 1024;   // bucket members ranked directly

__device__ __forceinline__ float order_key_to_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// one wave finds the digit d of the histogram h[0..nb) (nb = 64 * per, per <=
// 32) holding the `remaining`-th largest element: above(d) < remaining <=
// above(d) + h[d], above(d) = sum of h over digits > d, for 1 <= remaining <=
// sum of h.  Writes d and above(d).  Two levels: lane l first sums the digits
// [l*per, l*per+per) (higher digits belong to higher lanes) to find the lane
// holding d, then lanes 0..per-1 take that lane's digits in descending order.
__device__ __forceinline__ void digit_search(const uint32_t* s_h, int nb, uint32_t remaining,
                                             int lane, uint32_t* s_digit, uint32_t* s_above) {
    const int per = nb / 64;
    uint32_t segsum = 0;
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
        if (4 * q4 < per) {
            const uint4 x = reinterpret_cast<const uint4*>(s_h + lane * per)[q4];
            segsum += (x.x + x.y) + (x.z + x.w);
        }
    }
    const uint32_t incl = wave_incl_scan(segsum);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t above = total - incl;       // digits of the higher lanes
    const uint64_t hit = __ballot(above < remaining && above + segsum >= remaining);
    const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
    const uint32_t aL = (uint32_t)__builtin_amdgcn_readlane((int)above, L);
    const int top = L * per + per - 1;
    const uint32_t h = lane < per ? s_h[top - lane] : 0u;
    const uint32_t ab = aL + wave_incl_scan(h) - h;
    const uint64_t hit2 = __ballot(lane < per && ab < remaining && ab + h >= remaining);
    if (hit2 != 0 && lane == __ffsll((unsigned long long)hit2) - 1) {
        *s_digit = (uint32_t)(top - lane);
        *s_above = ab;
    }
}

// Shared steps of both variants.  Keys are f32 order keys (larger key =
// larger estimate).  ForAll(f) calls f(key) for every candidate of this
// thread; the result is kth and `remaining` = ties at kth to take.
struct FineShared {
    uint32_t h[kRadixBins];
    uint32_t mem[kRankMax];
    uint32_t tmp[kFBlock / 64];
    uint32_t wmax[kFBlock / 64], wmin[kFBlock / 64];
    uint32_t digit, above, cnt, kth, gt;
};

template <typename ForAll>
__device__ __forceinline__ void fine_threshold(FineShared& sh, uint32_t kmax, uint32_t kmin_inv,
                                               int k_eff, ForAll&& for_all, uint32_t& kth,
                                               uint32_t& remaining) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    kmax = wave_max(kmax);
    kmin_inv = wave_max(kmin_inv);
    if (lane == 0) {
        sh.wmax[wave] = kmax;
        sh.wmin[wave] = kmin_inv;
    }
    if (tid == 0) {
        sh.cnt = 0;
        sh.digit = 0;
        sh.above = 0;
    }
    lds_sync();
    kth = 0;
    remaining = (uint32_t)k_eff;
    kmax = 0;
    kmin_inv = 0;
#pragma unroll
    for (int w = 0; w < kFBlock / 64; ++w) {
        kmax = max(kmax, sh.wmax[w]);
        kmin_inv = max(kmin_inv, sh.wmin[w]);
    }
    const float vmax = order_key_to_f32(kmax), vmin = order_key_to_f32(~kmin_inv);
    const float span = vmax - vmin;
    const float scale = (float)kRadixBins / span;
    // finite, positive span and scale: (v - vmin) * scale is then finite and in [0, ~2048]
    if (span > 0.0f && span <= 3.0e38f && scale <= 3.0e38f) {
        const float topb = (float)(kRadixBins - 1);
        auto bucket = [&](uint32_t key) -> uint32_t {
            return (uint32_t)fminf((order_key_to_f32(key) - vmin) * scale, topb);
        };
        for (int b = tid; b < kRadixBins; b += kFBlock) sh.h[b] = 0;
        lds_sync();
        for_all([&](uint32_t key) { atomicAdd(&sh.h[bucket(key)], 1u); });
        lds_sync();
        if (wave == 0) digit_search(sh.h, kRadixBins, remaining, lane, &sh.digit, &sh.above);
        lds_sync();
        const uint32_t bstar = sh.digit;
        const uint32_t rem = remaining - sh.above;   // 1 <= rem <= members of bstar
        const uint32_t n_b = sh.h[bstar];
        if (n_b <= (uint32_t)kRankMax) {
            for_all([&](uint32_t key) {
                if (bucket(key) == bstar) sh.mem[atomicAdd(&sh.cnt, 1u)] = key;
            });
            lds_sync();
            // exact rank of every member: the k-th value has gt < rem <= ge
            for (int m = tid; m < (int)n_b; m += kFBlock) {
                const uint32_t km = sh.mem[m];
                uint32_t gt = 0, ge = 0;
                for (int j = 0; j < (int)n_b; ++j) {
                    const uint32_t kj = sh.mem[j];
                    gt += kj > km ? 1u : 0u;
                    ge += kj >= km ? 1u : 0u;
                }
                if (gt < rem && rem <= ge) {  // every writer writes the same values
                    sh.kth = km;
                    sh.gt = gt;
                }
            }
            lds_sync();
            kth = sh.kth;
            remaining = rem - sh.gt;
            return;
        }
    }
    // radix select over the order keys
    uint32_t prefix = 0, pmask = 0;
    for (int p = 0; p < 3; ++p) {
        const int width = p == 2 ? 10 : 11;               // digits of 11, 11, 10 bits
        const int shift = p == 0 ? 21 : (p == 1 ? 10 : 0);
        const uint32_t dmask = (1u << width) - 1u;
        const int nb = 1 << width;
        for (int b = tid; b < nb; b += kFBlock) sh.h[b] = 0;
        lds_sync();
        for_all([&](uint32_t key) {
            if ((key & pmask) == prefix) atomicAdd(&sh.h[(key >> shift) & dmask], 1u);
        });
        lds_sync();
        if (wave == 0) digit_search(sh.h, nb, remaining, lane, &sh.digit, &sh.above);
        lds_sync();
        prefix |= sh.digit << shift;
        pmask |= dmask << shift;
        remaining -= sh.above;
        lds_sync();
    }
    kth = prefix;
}

// The unit's coarse-score histogram row (tstride words) is read by every
// rerank block of a step; the fine selection, which runs after all of them,
// zeroes it for the next step's scan (no host-chosen table, so a captured
// retrieval replays correctly).  Called after the block's last load.
__device__ __forceinline__ void clear_unit_hist(uint32_t* tot, int tstride, int u) {
    if (tot == nullptr) return;
    for (int i = threadIdx.x; i < tstride; i += blockDim.x) tot[(int64_t)u * tstride + i] = 0u;
}

// candidates held in registers: C <= SEG * kFBlock, SEG in {4, 8, 16, 32, 64}
// (C < 65536); the candidate rows hold a multiple of SEG entries, so the
// 16-byte vector loads of a segment that starts below C stay inside the row
template <int SEG>
__device__ __forceinline__ void fine_reg_body(const int32_t* __restrict__ cand_pos,
                                              const float* __restrict__ cand_est, int64_t cmax,
                                              int C, int top_k, int32_t* __restrict__ sel,
                                              int32_t* __restrict__ sel_n, int u, FineShared& sh,
                                              uint32_t* unit_hist, int tstride) {
    const int tid = threadIdx.x;
    const int k_eff = C < top_k ? C : top_k;
    const int b0 = tid * SEG;
    const int bl = b0 < C ? b0 : 0;          // a segment past C loads the row's start
    // up to 16 candidates per thread the positions stay in registers too; with
    // more, they are read (all at once) after the threshold is known
    constexpr bool kPosReg = SEG <= 16;
    const int32_t* upos = cand_pos + (int64_t)u * cmax;
    uint32_t key[SEG];
    int32_t pos[kPosReg ? SEG : 1];
    int32_t pos2[kPosReg ? 1 : SEG];   // read back after the threshold (SEG > 16)
    {
        const float4* e4 = reinterpret_cast<const float4*>(cand_est + (int64_t)u * cmax + bl);
        const int4* p4 = reinterpret_cast<const int4*>(upos + bl);
        float4 e[SEG / 4];
        int4 pv[kPosReg ? SEG / 4 : 1];
#pragma unroll
        for (int q = 0; q < SEG / 4; ++q) {
            e[q] = e4[q];
            if constexpr (kPosReg) pv[q] = p4[q];
        }
#pragma unroll
        for (int q = 0; q < SEG / 4; ++q) {
            key[4 * q] = f32_order_key(e[q].x);
            key[4 * q + 1] = f32_order_key(e[q].y);
            key[4 * q + 2] = f32_order_key(e[q].z);
            key[4 * q + 3] = f32_order_key(e[q].w);
            if constexpr (kPosReg) {
                pos[4 * q] = pv[q].x;
                pos[4 * q + 1] = pv[q].y;
                pos[4 * q + 2] = pv[q].z;
                pos[4 * q + 3] = pv[q].w;
            }
        }
    }
    const int nv = C - b0 < 0 ? 0 : (C - b0 < SEG ? C - b0 : SEG);   // valid entries
    const bool all = k_eff >= C;
    uint32_t kth = 0, remaining = (uint32_t)k_eff;
    if (!all) {
        uint32_t kmax = 0, kmin_inv = 0;
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            kmax = max(kmax, j < nv ? key[j] : 0u);
            kmin_inv = max(kmin_inv, j < nv ? ~key[j] : 0u);
        }
        fine_threshold(sh, kmax, kmin_inv, k_eff,
                       [&](auto&& f) {
#pragma unroll
                           for (int j = 0; j < SEG; ++j)
                               if (j < nv) f(key[j]);
                       },
                       kth, remaining);
    }
    // compaction: one block scan of (ties at kth, keys above kth) gives both
    // offsets (C < 65536: the halves never carry)
    uint32_t eqc = 0, gtc = 0;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        gtc += (j < nv && (all || key[j] > kth)) ? 1u : 0u;
        eqc += (j < nv && !all && key[j] == kth) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t packed = block_excl_scan_t<kFBlock>((eqc << 16) | gtc, sh.tmp, &tot);
    uint32_t r = packed >> 16;                 // ties at kth before this segment
    uint32_t o = (packed & 0xffffu) + (r < remaining ? r : remaining);
    int32_t* usel = sel + (int64_t)u * top_k;
    if constexpr (!kPosReg) {                  // this run's positions, all requested at once
        const int4* p4 = reinterpret_cast<const int4*>(upos + bl);
#pragma unroll
        for (int q = 0; q < SEG / 4; ++q) {
            const int4 x = p4[q];
            pos2[4 * q] = x.x;
            pos2[4 * q + 1] = x.y;
            pos2[4 * q + 2] = x.z;
            pos2[4 * q + 3] = x.w;
        }
    }
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        const bool eq = j < nv && !all && key[j] == kth;
        const bool in = j < nv && (all || key[j] > kth || (eq && r < remaining));
        r += eq ? 1u : 0u;
        if (in && o < (uint32_t)k_eff) {
            if constexpr (kPosReg) usel[o] = pos[j];
            else usel[o] = pos2[j];
        }
        o += in ? 1u : 0u;
    }
    clear_unit_hist(unit_hist, tstride, u);
    if (tid == 0) sel_n[u] = k_eff;
}

}  // namespace pk
