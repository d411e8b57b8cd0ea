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
// Below 65536 candidates thread t keeps its segment [t*SEG, t*SEG+SEG) in
// registers for every pass (SEG up to 64; up to kFineReg, 16 per thread, in
// the launch fused with the hot-zone attention); beyond that the passes
// stream the estimates from memory.
// ---------------------------------------------------------------------------
constexpr int kFBlock = 1024;
constexpr int kFineReg = 16 * kFBlock;  // candidates the fused launch holds in registers
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
// larger estimate).  ForAll(f) calls f(key, j) for every candidate of this
// thread, j its slot (0 <= j < NC) when the thread holds its candidates in
// registers, in which case each key's bucket is kept in a register between
// the histogram and the member passes (NC = 0: recomputed); the result is kth
// and `remaining` = ties at kth to take.
struct FineShared {
    uint32_t h[kRadixBins];
    uint32_t mem[kRankMax];
    uint32_t tmp[kFBlock / 64];
    uint32_t wmax[kFBlock / 64], wmin[kFBlock / 64];
    uint32_t digit, above, cnt, kth, gt;
};

template <int NC, typename ForAll>
__device__ __forceinline__ void fine_threshold(FineShared& sh, uint32_t kmax, uint32_t kmin_inv,
                                               int k_eff, ForAll&& for_all, uint32_t& kth,
                                               uint32_t& remaining) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the bucket histogram is zeroed ahead of the range's barrier (no pass of
    // the caller reads sh.h past its own last barrier)
    for (int b = tid; b < kRadixBins; b += kFBlock) sh.h[b] = 0;
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
        uint32_t bc[NC > 0 ? NC : 1];
        for_all([&](uint32_t key, int j) {
            const uint32_t bk = bucket(key);
            if constexpr (NC > 0) bc[j] = bk;
            atomicAdd(&sh.h[bk], 1u);
        });
        lds_sync();
        if (wave == 0) digit_search(sh.h, kRadixBins, remaining, lane, &sh.digit, &sh.above);
        lds_sync();
        const uint32_t bstar = sh.digit;
        const uint32_t rem = remaining - sh.above;   // 1 <= rem <= members of bstar
        const uint32_t n_b = sh.h[bstar];
        if (n_b <= (uint32_t)kRankMax) {
            for_all([&](uint32_t key, int j) {
                uint32_t bk;
                if constexpr (NC > 0) bk = bc[j];
                else bk = bucket(key);
                if (bk == bstar) sh.mem[atomicAdd(&sh.cnt, 1u)] = key;
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
        // every thread has read n_b before the radix passes rewrite sh.h
        lds_sync();
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
        for_all([&](uint32_t key, int) {
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

// Survivors of the sampled prefilter kept in LDS (keys and candidate indices).
constexpr int kSurvMax = 8 * kFBlock;

// The sampled prefilter of fine_reg_body (described there).  key[0..nv) are
// this thread's candidates b0..b0+nv-1; writes the selection's positions to
// usel[0..k_eff) and returns true, or returns false (nothing written) when
// fewer than k_eff or more than kSurvMax keys survive.
template <int SEG>
__device__ __forceinline__ bool fine_sampled(const uint32_t (&key)[SEG], int nv, int b0, int C,
                                          int k_eff, const int32_t* __restrict__ upos,
                                          int32_t* __restrict__ usel, FineShared& sh,
                                          uint32_t* surv) {
    const int tid = threadIdx.x;
    // the sample: the first key of every thread holding candidates
    const int n_samp = (C + SEG - 1) / SEG;
    int r = (int)(((int64_t)2 * k_eff * n_samp + C - 1) / C);
    r = r < 1 ? 1 : (r > n_samp ? n_samp : r);
    uint32_t t_low = 0, rem_s = 0;
    fine_threshold<1>(sh, nv > 0 ? key[0] : 0u, nv > 0 ? ~key[0] : 0u, r,
                      [&](auto&& f) { if (nv > 0) f(key[0], 0); }, t_low, rem_s);
    // survivors: keys >= t_low, counted and placed in candidate order
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < SEG; ++j) cnt += (j < nv && key[j] >= t_low) ? 1u : 0u;
    uint32_t n_sur;
    uint32_t w = block_excl_scan_t<kFBlock, false>(cnt, sh.tmp, &n_sur);
    if (n_sur < (uint32_t)k_eff || n_sur > (uint32_t)kSurvMax) return false;   // block-uniform
    uint32_t* skey = surv;
    uint32_t* sidx = surv + kSurvMax;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        if (j < nv && key[j] >= t_low) {
            skey[w] = key[j];
            sidx[w] = (uint32_t)(b0 + j);
            ++w;
        }
    }
    lds_sync();
    // exact selection over the survivors: thread t holds survivors [8t, 8t + 8)
    constexpr int SS = kSurvMax / kFBlock;
    const int s0 = tid * SS;
    const int nv2 = (int)n_sur - s0 < 0 ? 0 : ((int)n_sur - s0 < SS ? (int)n_sur - s0 : SS);
    uint32_t k2[SS];
    uint32_t kmax = 0, kmin_inv = 0;
#pragma unroll
    for (int j = 0; j < SS; ++j) {
        k2[j] = j < nv2 ? skey[s0 + j] : 0u;
        kmax = max(kmax, j < nv2 ? k2[j] : 0u);
        kmin_inv = max(kmin_inv, j < nv2 ? ~k2[j] : 0u);
    }
    uint32_t kth = 0, remaining = (uint32_t)k_eff;
    fine_threshold<SS>(sh, kmax, kmin_inv, k_eff,
                       [&](auto&& f) {
#pragma unroll
                           for (int j = 0; j < SS; ++j)
                               if (j < nv2) f(k2[j], j);
                       },
                       kth, remaining);
    uint32_t eqc = 0, gtc = 0;
#pragma unroll
    for (int j = 0; j < SS; ++j) {
        gtc += (j < nv2 && k2[j] > kth) ? 1u : 0u;
        eqc += (j < nv2 && k2[j] == kth) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t packed = block_excl_scan_t<kFBlock, false>((eqc << 16) | gtc, sh.tmp, &tot);
    uint32_t rr = packed >> 16;
    uint32_t o = (packed & 0xffffu) + (rr < remaining ? rr : remaining);
#pragma unroll
    for (int j = 0; j < SS; ++j) {
        const bool eq = j < nv2 && k2[j] == kth;
        const bool in = j < nv2 && (k2[j] > kth || (eq && rr < remaining));
        rr += eq ? 1u : 0u;
        if (in && o < (uint32_t)k_eff) usel[o] = upos[sidx[s0 + j]];
        o += in ? 1u : 0u;
    }
    return true;
}

// candidates held in registers: C <= SEG * kFBlock, SEG in {4, 8, 16, 32, 64}
// (C < 65536); the candidate rows hold a multiple of SEG entries, so the
// 16-byte vector loads of a segment that starts below C stay inside the row.
//
// With many candidates per selected key (SEG >= 32, C >= 8 k), every pass
// over all the register-held keys costs the block several microseconds of
// VALU time, so the selection first narrows them: t_low = the r-th largest
// of a systematic sample (each thread's first key, r about twice the
// sample's share of k), the keys >= t_low (an upper set of the values, kept
// in candidate order in LDS, at most kSurvMax), and the exact selection over
// those alone.  It is exact whenever at least k keys survive: then the k-th
// largest key and every key equal to it are survivors, so the threshold, the
// ties taken (lowest positions first) and the selected set are those of the
// full selection; otherwise (or with too many survivors) the full selection
// runs.  surv: 2 * kSurvMax words of LDS (SEG >= 32).
template <int SEG>
__device__ __forceinline__ void fine_reg_body(const int32_t* __restrict__ cand_pos,
                                              const float* __restrict__ cand_est, int64_t cmax,
                                              int C, int top_k, int32_t* __restrict__ sel,
                                              int32_t* __restrict__ sel_n, int u, FineShared& sh,
                                              uint32_t* unit_hist, int tstride,
                                              uint32_t* surv = nullptr) {
    const int tid = threadIdx.x;
    const int k_eff = C < top_k ? C : top_k;
    const int b0 = tid * SEG;
    const int bl = b0 < C ? b0 : 0;          // a segment past C loads the row's start
    // up to 16 candidates per thread the positions stay in registers too; with
    // more, only the selected ones are read, after the threshold is known
    constexpr bool kPosReg = SEG <= 16;
    const int32_t* upos = cand_pos + (int64_t)u * cmax;
    uint32_t key[SEG];
    int32_t pos[kPosReg ? SEG : 1];
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
    if constexpr (SEG >= 32) {
        if (!all && surv != nullptr && C >= 8 * k_eff &&
            fine_sampled(key, nv, b0, C, k_eff, upos, sel + (int64_t)u * top_k, sh, surv)) {
            clear_unit_hist(unit_hist, tstride, u);
            if (tid == 0) sel_n[u] = k_eff;
            return;
        }
    }
    if (!all) {
        uint32_t kmax = 0, kmin_inv = 0;
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            kmax = max(kmax, j < nv ? key[j] : 0u);
            kmin_inv = max(kmin_inv, j < nv ? ~key[j] : 0u);
        }
        fine_threshold<(SEG <= 16 ? SEG : 0)>(sh, kmax, kmin_inv, k_eff,
                                              [&](auto&& f) {
#pragma unroll
                                                  for (int j = 0; j < SEG; ++j)
                                                      if (j < nv) f(key[j], j);
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
    const uint32_t packed = block_excl_scan_t<kFBlock, false>((eqc << 16) | gtc, sh.tmp, &tot);
    uint32_t r = packed >> 16;                 // ties at kth before this segment
    uint32_t o = (packed & 0xffffu) + (r < remaining ? r : remaining);
    int32_t* usel = sel + (int64_t)u * top_k;
    // fresh copies of kth and nv for the emit loop: otherwise the compiler keeps
    // every comparison of the counting loop alive across the scan's barriers
    // (SEG of them), which no longer fits the registers for SEG = 64
    const uint32_t kth_e = (uint32_t)__builtin_amdgcn_readfirstlane((int)kth);
    int nv_e = nv;
    asm volatile("" : "+v"(nv_e));
    // positions not held in registers (SEG > 16): the selected candidates'
    // indices go to LDS (the histogram's words, dead by now) and their
    // positions are then gathered in one round, one output per thread and pass
    const bool stage = !kPosReg && k_eff <= kRadixBins;
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        const bool eq = j < nv_e && !all && key[j] == kth_e;
        const bool in = j < nv_e && (all || key[j] > kth_e || (eq && r < remaining));
        r += eq ? 1u : 0u;
        if (in && o < (uint32_t)k_eff) {
            if constexpr (kPosReg) usel[o] = pos[j];
            else if (stage) sh.h[o] = (uint32_t)(b0 + j);
            else usel[o] = upos[b0 + j];
        }
        o += in ? 1u : 0u;
    }
    if (stage) {
        lds_sync();
        for (int i = tid; i < k_eff; i += kFBlock) usel[i] = upos[sh.h[i]];
    }
    clear_unit_hist(unit_hist, tstride, u);
    if (tid == 0) sel_n[u] = k_eff;
}

}  // namespace pk
