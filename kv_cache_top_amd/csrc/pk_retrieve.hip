// Coarse-to-fine retrieval (gfx950).
//
// ParisKV page, "Two-stage GPU-native retrieval pipeline":
//  * coarse (collision based): every retrieval-zone key's integer score is the
//    sum over subspaces of the votes its bucket received; a small top fraction
//    of keys is kept;
//  * rerank (RSQ-IP): each candidate's raw score <k, q> is estimated from its
//    4-bit codes and scales only, and the top-k are selected.
//
// The scan kernel is in pk_scan.hip; here the rerank and the fine
// selection.  No cross-block synchronisation inside any kernel (on gfx950 an
// agent-scope release fence writes back the XCD's L2 and costs far more per
// block than a kernel boundary):
//  rerank  one 256-thread block per (chunk, unit): from the unit histogram
//          the coarse threshold T (largest score with #{score >= T} >= C) and
//          the ties at T to take, from the earlier chunks' suffix counts the
//          candidates before this chunk; then compacts the chunk's candidates
//          in position order and estimates them with RSQ-IP;
//  fine    one 1024-thread block per unit: the k-th largest estimate by
//          value bucketing (radix select as the fallback), ties to the lower
//          position, compaction in order.
#include <type_traits>

#include "pk_device.hpp"
#include "pk_fine.hpp"
#include "pk_launch.hpp"

namespace pk {

// rerank.  Coarse selection, per unit: ge[s] = #{score >= s} from the unit
// histogram; T = max s with ge[s] >= C; the ties at T taken are the first
// need = C - ge[T+1] in position order.  Chunk c holds gt_c = sfx_c[T+1]
// keys above T and eq_c = sfx_c[T] - gt_c ties; this chunk's candidates start
// after the earlier chunks' keys above T and the ties taken among theirs.
template <int KPT, int M>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(KPT <= 8 ? 8 : 1))) void rerank_kernel(
    const uint8_t* __restrict__ scores, int64_t sstride, const uint8_t* __restrict__ rec,
    const uint8_t* __restrict__ ids, const uint8_t* __restrict__ lut,
    int64_t cap, int64_t sink_end, int64_t n_r, int max_chunks, const uint16_t* __restrict__ hist,
    int hstride, const uint32_t* __restrict__ tot, int nbins,
    int64_t C, int top_k,
    const float* __restrict__ ysum, CodeTables tab, int32_t* __restrict__ cand_pos,
    float* __restrict__ cand_est, int64_t cmax, int32_t* __restrict__ meta, int units_fastest) {
    constexpr int chunk = KPT * kBlock;
    static_assert(kBlock == 256, "one pair-table entry and one prefetched piece per thread");
    const int u = units_fastest ? blockIdx.x : blockIdx.y;   // block order: see launch_rerank
    const int ch = units_fastest ? blockIdx.y : blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = tid & 15;
    constexpr int kLutWords = (M == 16 ? lut_bytes<16>() : lut_bytes<8>()) / 4;
    __shared__ __align__(16) int32_t s_list[chunk < kLutWords ? kLutWords : chunk];   // also the vote table
    __shared__ float2 s_pair[256];     // nibble byte (code of coord 2i+1 << 4 | code of 2i)
    __shared__ float s_lv[16];         // signed level of each 4-bit code
    __shared__ __align__(16) uint4 s_pre[kBlock];   // prefetched suffix counts (below)
    __shared__ uint32_t s_T, s_need, s_gt, s_eq;
    __shared__ __align__(16) uint32_t s_wtot[kBlock / 64];
    // Every block resident on a CU runs the part before the record gather at
    // the same time, so its instructions are paid by all of them: work that
    // one wave can do is done by one wave.
    // signed level of code tid < 16: sign bit 3, magnitude index bits 0..2.
    // The levels are read as wave-uniform values outside the branch: a
    // per-lane select over the argument entries otherwise compiles to a vector
    // load of the argument segment and a wait ahead of wave 0's first requests.
    {
        float lv[8];
#pragma unroll
        for (int l = 0; l < 8; ++l)
            lv[l] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tab.levels[l])));
        if (tid < 16) {
            float m = lv[0];
#pragma unroll
            for (int l = 1; l < 8; ++l) m = ((tid & 7) == l) ? lv[l] : m;
            s_lv[tid] = (tid & 8) ? -m : m;
        }
    }

    // one round of loads: the unit histogram (its first 512 bins requested
    // before anything else), the first W suffix counts of the earlier chunks
    // (up to 64 of them; thread 4c + q holds entries 8q .. 8q+7 of chunk c,
    // rows being hstride entries, a multiple of 8), this chunk's scores
    // (contiguous per thread, vector loads; rows are padded so these never
    // leave the buffer) and the summed rotated query
    const uint32_t* ut = tot + (int64_t)u * ((nbins + 1) & ~1);
    const uint32_t t0 = tid < nbins ? ut[tid] : 0u;
    const uint32_t t1 = tid + kBlock < nbins ? ut[tid + kBlock] : 0u;
    const int W = hstride < 32 ? hstride : 32;
    {
        const int pc = tid >> 2, pq = tid & 3;
        uint4 pre = make_uint4(0u, 0u, 0u, 0u);
        if (pc < ch && 8 * pq < W)
            pre = *reinterpret_cast<const uint4*>(hist + ((int64_t)u * max_chunks + pc) * hstride + 8 * pq);
        s_pre[tid] = pre;
    }
    const int64_t start = (int64_t)ch * chunk;
    const int kbase = (int)start + tid * KPT;   // retrieval zone < 2^24 keys
    uint32_t s[KPT];
    {
        const uint8_t* sp = scores + u * sstride + start + (int64_t)tid * KPT;
        uint32_t w[(KPT + 3) / 4];
        if constexpr (KPT >= 16) {
#pragma unroll
            for (int q = 0; q < KPT / 16; ++q) {
                const uint4 x = reinterpret_cast<const uint4*>(sp)[q];
                w[4 * q] = x.x; w[4 * q + 1] = x.y; w[4 * q + 2] = x.z; w[4 * q + 3] = x.w;
            }
        } else if constexpr (KPT == 8) {
            const uint2 x = *reinterpret_cast<const uint2*>(sp);
            w[0] = x.x; w[1] = x.y;
        } else if constexpr (KPT == 4) {
            w[0] = *reinterpret_cast<const uint32_t*>(sp);
        } else if constexpr (KPT == 2) {
            w[0] = *reinterpret_cast<const uint16_t*>(sp);
        } else {
            w[0] = sp[0];
        }
#pragma unroll
        for (int j = 0; j < KPT; ++j) s[j] = (w[j >> 2] >> (8 * (j & 3))) & 255u;
    }
    float y[8];
    load8(ysum + (int64_t)u * kD + 8 * l16, y);
    extern __shared__ uint32_t s_ut[];   // the unit histogram (nbins entries, sized at launch)
    if (tid < nbins) s_ut[tid] = t0;
    if (tid + kBlock < nbins) s_ut[tid + kBlock] = t1;
    for (int b = tid + 2 * kBlock; b < nbins; b += kBlock) s_ut[b] = ut[b];
    lds_sync();
    s_pair[tid] = make_float2(s_lv[tid & 15], s_lv[tid >> 4]);   // read after later barriers

    // Wave 0: T and need.  ge[s] = #{score >= s} is non-increasing in s, and T
    // is the one bin where it reaches C.  Lane l sums the bins [l*per, l*per +
    // per) (per = ceil(nbins / 64) <= 64); a wave scan of the lane sums gives
    // the keys above each lane's bins, and each lane walks its own bins from
    // the top: the one lane whose range holds T finds it there.
    if (wave == 0) {
        const uint32_t Cu = (uint32_t)C;   // 1 <= C <= n_r < 2^24
        const int per = (nbins + 63) >> 6;
        const int b0 = lane * per;
        int tb = -1;
        uint32_t nd = 0;
        if (per <= 8) {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = (j < per && b0 + j < nbins) ? s_ut[b0 + j] : 0u;
            const uint32_t seg = ((h[0] + h[1]) + (h[2] + h[3])) + ((h[4] + h[5]) + (h[6] + h[7]));
            const uint32_t incl = wave_incl_scan(seg);
            uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
#pragma unroll
            for (int j = 7; j >= 0; --j) {
                if (tb < 0 && run < Cu && run + h[j] >= Cu) {
                    tb = b0 + j;
                    nd = Cu - run;
                }
                run += h[j];
            }
        } else {
            uint32_t seg = 0;
            for (int j = 0; j < per; ++j) seg += b0 + j < nbins ? s_ut[b0 + j] : 0u;
            const uint32_t incl = wave_incl_scan(seg);
            uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
            for (int j = per - 1; j >= 0; --j) {
                const uint32_t h = b0 + j < nbins ? s_ut[b0 + j] : 0u;
                if (tb < 0 && run < Cu && run + h >= Cu) {
                    tb = b0 + j;
                    nd = Cu - run;
                }
                run += h;
            }
        }
        const uint64_t hit = __ballot(tb >= 0);
        const int L = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
        const int Tw = hit ? __builtin_amdgcn_readlane(tb, L) : 0;
        const uint32_t need_w = hit ? (uint32_t)__builtin_amdgcn_readlane((int)nd, L) : 0u;
        if (lane == 0) {
            s_T = (uint32_t)Tw;
            s_need = need_w;
        }
    }
    lds_sync();
    const int T = (int)(s_T < (uint32_t)nbins ? s_T : (uint32_t)nbins - 1u);
    const uint32_t need = s_need;

    // Wave 0 again, while the others count their keys: the earlier chunks'
    // keys above T and ties at T.  Chunk c holds sfx_c[T+1] keys above T and
    // sfx_c[T] - sfx_c[T+1] ties, read from the prefetched entries when both
    // are among them, else from memory.
    uint32_t g_w = 0, e_w = 0;
    if (wave == 0) {
        const int Wv = W < nbins ? W : nbins;
        const uint16_t* pre16 = reinterpret_cast<const uint16_t*>(s_pre);
        for (int c = lane; c < ch; c += 64) {
            uint32_t at_t, above_t;   // sfx_c[T], sfx_c[T+1]
            if (c < kBlock / 4 && T + 1 < Wv) {
                at_t = pre16[c * 32 + T];
                above_t = pre16[c * 32 + T + 1];
            } else {
                const uint16_t* row = hist + ((int64_t)u * max_chunks + c) * hstride;
                at_t = row[T];
                above_t = T + 1 < nbins ? row[T + 1] : 0u;
            }
            g_w += above_t;
            e_w += at_t - above_t;
        }
        g_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(g_w), 63);
        e_w = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(e_w), 63);
    }

    // a stored 255 stands for 255 or more: when the threshold is that high the
    // saturated keys are rescored from their bucket ids (block-uniform branch)
    if (T >= 255) {
        constexpr int kTabB = M == 16 ? lut_bytes<16>() : lut_bytes<8>();
        for (int i = tid; i < kTabB / 16; i += kBlock)
            reinterpret_cast<uint4*>(s_list)[i] = reinterpret_cast<const uint4*>(lut + (int64_t)u * kTabB)[i];
        lds_sync();
        const uint8_t* lut8 = reinterpret_cast<const uint8_t*>(s_list);
        const uint4* idrow = reinterpret_cast<const uint4*>(ids) + u * cap + sink_end;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (s[j] == 255u && kbase + j < (int)n_r) {
                const uint4 v = idrow[kbase + j];
                const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
                uint32_t sc = 0;
                if constexpr (M == 16) {
                    sc = hashed_score(reinterpret_cast<const uint32_t*>(s_list), wv);
                } else {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int k = 0; k < 4; ++k) sc += lut8[(4 * a + k) * 256 + ((wv[a] >> (8 * k)) & 255u)];
                }
                s[j] = sc;
            }
        }
        lds_sync();                            // the table is dead before s_list is written
    }

    // this chunk's candidates, in position order: keys above T, and ties at T
    // while the unit's tie budget lasts.  Keys past the zone's end (last chunk
    // only) read as -1, which is neither above nor equal to T >= 0.
    if (start + chunk > n_r) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (kbase + j >= (int)n_r) s[j] = 0xffffffffu;
    }
    uint32_t eqc = 0, gtc = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        gtc += (int)s[j] > T ? 1u : 0u;
        eqc += (int)s[j] == T ? 1u : 0u;
    }
    // packed (ties, above) exclusive scan over the block (a chunk holds at
    // most 8192 keys: the halves never carry)
    uint32_t packed, tot_c;
    {
        const uint32_t v = (eqc << 16) | gtc;
        const uint32_t x = wave_incl_scan(v);
        if (lane == 63) s_wtot[wave] = x;
        if (wave == 0 && lane == 0) {
            s_gt = g_w;
            s_eq = e_w;
        }
        lds_sync();
        const uint4 wt = *reinterpret_cast<const uint4*>(s_wtot);
        const uint32_t before = (wave > 0 ? wt.x : 0u) + (wave > 1 ? wt.y : 0u) + (wave > 2 ? wt.z : 0u);
        packed = before + x - v;
        tot_c = (wt.x + wt.y) + (wt.z + wt.w);
    }
    const uint32_t gt_chunk = s_gt, eq_chunk = s_eq;
    const uint32_t eq_t = packed >> 16, gt_t = packed & 0xffffu;
    const uint32_t taken_before_chunk = eq_chunk < need ? eq_chunk : need;
    auto taken = [&](uint32_t e) { return (e < need ? e : need) - taken_before_chunk; };
    uint32_t at = gt_t + taken(eq_chunk + eq_t);
    const uint32_t cand_before = gt_chunk + taken_before_chunk;
    // each wave lists its own candidates (a contiguous range of the chunk's
    // list) and estimates them itself, so no block barrier stands between the
    // list and the record requests
    const int w_lo = __builtin_amdgcn_readfirstlane((int)at);   // lane 0's first slot
    uint32_t rank = eq_chunk + eq_t;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool in = (int)s[j] > T || ((int)s[j] == T && rank < need);
        rank += (int)s[j] == T ? 1u : 0u;
        if (in) s_list[at] = (int32_t)(sink_end + start + (int64_t)tid * KPT + j);
        at += in ? 1u : 0u;
    }
    const int w_hi = __builtin_amdgcn_readlane((int)at, 63);   // past lane 63's last slot
    (void)tot_c;
    // the list entries other lanes of this wave wrote are complete before any is read
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();

    // RSQ-IP: est = sum_b w_b <v_b, Ysum_b> / sqrt(d), Ysum = sum_g H D q_g;
    // 16 lanes per candidate, lane l reading the nibble word of coordinates
    // 8l..8l+7 and their w (one subspace for m = 8, two for m = 4, half of
    // subspace l / 2 for m = 16).
    // A group fetches the records of up to kBatch candidates before using any
    // (8 for m = 4, whose lanes read 12 B each).  17 rather than 16 lets the
    // crowded waves of the first chunks finish in one fewer round; it is the
    // largest batch that stays under 64 VGPRs (8 waves per SIMD) without
    // scratch (measured against the same session: 16 -> 12.1 us, 17 -> 11.8,
    // 18 -> 12.2 at 128K x 4).
    // Codes are dequantised two at a time from the byte-indexed level pairs.
    // Record offsets within the unit fit 32 bits (capacity <= 2^24 keys).
    constexpr int kBatch = M == 4 ? 8 : 17;
    constexpr uint32_t kRecB = (uint32_t)rec_bytes<M>();
    using WT = typename std::conditional<M == 4, float2, float>::type;   // a lane's w
    const float inv_sqrt_d = 0.08838834764831845f;
    const int grp = lane >> 4;         // 16-lane group within the wave
    // the unit's records through a buffer descriptor: 32-bit offsets (a unit
    // holds at most 2^24 records of <= 192 B), half the address registers of
    // 64-bit pointers for the batch in flight
    const __amdgpu_buffer_rsrc_t urec = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(rec + (int64_t)u * cap * kRecB), (short)0,
        (int)(uint32_t)((uint64_t)cap * kRecB), kBufferRsrcWord3);
    int32_t* upos = cand_pos + (int64_t)u * cmax;
    float* uest = cand_est + (int64_t)u * cmax;
    const uint32_t w_off = 64u + (M == 4 ? 8u * (uint32_t)l16 : 4u * (uint32_t)(M == 16 ? (l16 >> 1) : l16));
    for (int i0 = w_lo + grp; i0 < w_hi; i0 += kBatch * 4) {
        uint32_t nib[kBatch];
        WT w[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * 4;
            const int32_t p = s_list[i < w_hi ? i : i0];
            const uint32_t ro = (uint32_t)p * kRecB;
            nib[k] = __builtin_amdgcn_raw_buffer_load_b32(urec, ro + 4u * (uint32_t)l16, 0, 0);
            if constexpr (M == 4) {
                const uint32_t a = __builtin_amdgcn_raw_buffer_load_b32(urec, ro + w_off, 0, 0);
                const uint32_t b = __builtin_amdgcn_raw_buffer_load_b32(urec, ro + w_off + 4u, 0, 0);
                w[k] = make_float2(__uint_as_float(a), __uint_as_float(b));
            } else {
                w[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(urec, ro + w_off, 0, 0));
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * 4;
            if (i >= w_hi) break;                // uniform in the 16-lane group
            float part;
            if constexpr (M != 4) {   // one w for the lane's 8 coordinates
                float dot = 0.0f;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float2 lv = s_pair[(nib[k] >> (8 * b)) & 255u];
                    dot = fmaf(lv.x, y[2 * b], dot);
                    dot = fmaf(lv.y, y[2 * b + 1], dot);
                }
                part = w[k] * dot;
            } else {
                float dot[2] = {0.0f, 0.0f};
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float2 lv = s_pair[(nib[k] >> (8 * b)) & 255u];
                    dot[b >> 1] = fmaf(lv.x, y[2 * b], dot[b >> 1]);
                    dot[b >> 1] = fmaf(lv.y, y[2 * b + 1], dot[b >> 1]);
                }
                part = fmaf(w[k].x, dot[0], w[k].y * dot[1]);
            }
            const float e = sum16(part);
            const uint32_t o = cand_before + (uint32_t)i;
            if (l16 == 0 && (int64_t)o < cmax) {
                upos[o] = s_list[i];
                uest[o] = e * inv_sqrt_d;
            }
        }
    }
    // (stored last: a store ahead of a load's wait would be waited for too)
    if (ch == 0 && tid == 0) {
        meta[u * 4 + 0] = T;
        meta[u * 4 + 1] = (int32_t)need;
        meta[u * 4 + 2] = (int32_t)C;
        meta[u * 4 + 3] = (int32_t)(C < top_k ? C : top_k);
    }
}

template <int SEG>
__global__ __launch_bounds__(kFBlock) void fine_reg_kernel(const int32_t* __restrict__ cand_pos,
                                                           const float* __restrict__ cand_est,
                                                           int64_t cmax, int C, int top_k,
                                                           int32_t* __restrict__ sel,
                                                           int32_t* __restrict__ sel_n,
                                                           uint32_t* __restrict__ tot,
                                                           int tstride) {
    __shared__ FineShared sh;
    __shared__ uint32_t s_surv[SEG >= 32 ? 2 * kSurvMax : 1];   // survivors of the sampled prefilter
    fine_reg_body<SEG>(cand_pos, cand_est, cmax, C, top_k, sel, sel_n, blockIdx.x, sh, tot,
                       tstride, SEG >= 32 ? s_surv : nullptr);
}

// more candidates than registers hold: the threshold passes stream the
// estimates from memory (coalesced, kMemBatch loads in flight per thread);
// the compaction goes through LDS in tiles of kMemTile keys and positions,
// loaded coalesced, thread t taking the contiguous run [t*8, t*8+8) of a tile,
// so the output stays in candidate order.
constexpr int kMemBatch = 32;
constexpr int kMemTile = 8 * kFBlock;
constexpr int kMemOut = 8192;   // selections staged in LDS and stored at the end (k <= 8192)
__global__ __launch_bounds__(kFBlock) void fine_mem_kernel(const int32_t* __restrict__ cand_pos,
                                                           const float* __restrict__ cand_est,
                                                           int64_t cmax, int C, int top_k,
                                                           int32_t* __restrict__ sel,
                                                           int32_t* __restrict__ sel_n,
                                                           uint32_t* __restrict__ tot,
                                                           int tstride) {
    const int u = blockIdx.x, tid = threadIdx.x;
    __shared__ FineShared sh;
    __shared__ __align__(16) uint32_t s_tile[kMemTile];
    __shared__ __align__(16) int32_t s_tpos[kMemTile];
    __shared__ int32_t s_out[kMemOut];
    __shared__ uint32_t s_red[2 * kFBlock / 64];
    const float* est = cand_est + (int64_t)u * cmax;
    const int32_t* cpos = cand_pos + (int64_t)u * cmax;
    const int k_eff = C < top_k ? C : top_k;
    // 16-byte loads, four estimates each (rows hold a multiple of 64 entries, so
    // a vector starting below C stays in the row); few CUs run this kernel, and
    // a CU's bytes in flight bound each pass
    const int C4 = (C + 3) / 4;
    const float4* est4 = reinterpret_cast<const float4*>(est);
    auto for_all = [&](auto&& f) {
        for (int q0 = tid; q0 < C4; q0 += (kMemBatch / 4) * kFBlock) {
            float4 e[kMemBatch / 4];
#pragma unroll
            for (int k = 0; k < kMemBatch / 4; ++k) {
                const int q = q0 + k * kFBlock;
                e[k] = est4[q < C4 ? q : C4 - 1];      // clamped: a real vector
            }
#pragma unroll
            for (int k = 0; k < kMemBatch / 4; ++k) {
                const int i = 4 * (q0 + k * kFBlock);
                if (i < C) f(f32_order_key(e[k].x), 0);
                if (i + 1 < C) f(f32_order_key(e[k].y), 0);
                if (i + 2 < C) f(f32_order_key(e[k].z), 0);
                if (i + 3 < C) f(f32_order_key(e[k].w), 0);
            }
        }
    };
    const bool all = k_eff >= C;
    uint32_t kth = 0, remaining = (uint32_t)k_eff;
    if (!all) {
        uint32_t kmax = 0, kmin_inv = 0;
        for_all([&](uint32_t key, int) {
            kmax = max(kmax, key);
            kmin_inv = max(kmin_inv, ~key);
        });
        fine_threshold<0>(sh, kmax, kmin_inv, k_eff, for_all, kth, remaining);
    }
    // compaction, tile by tile: ties at kth before this thread's run and keys
    // above kth before it, from one scan per tile plus the earlier tiles' totals
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t gt_carry = 0, eq_carry = 0;
    int32_t* usel = sel + (int64_t)u * top_k;
    // the next tile is requested while the current one is compacted
    constexpr int kPer4 = kMemTile / (4 * kFBlock);   // 16-byte vectors per thread per tile
    float4 e[kPer4];
    int4 pv[kPer4];
    const int4* cpos4 = reinterpret_cast<const int4*>(cpos);
    auto fetch = [&](int base) {
#pragma unroll
        for (int k = 0; k < kPer4; ++k) {
            const int q = base / 4 + k * kFBlock + tid;
            e[k] = est4[q < C4 ? q : C4 - 1];
            pv[k] = cpos4[q < C4 ? q : C4 - 1];
        }
    };
    fetch(0);
    for (int base = 0; base < C; base += kMemTile) {
#pragma unroll
        for (int k = 0; k < kPer4; ++k) {
            reinterpret_cast<uint4*>(s_tile)[k * kFBlock + tid] =
                make_uint4(f32_order_key(e[k].x), f32_order_key(e[k].y), f32_order_key(e[k].z),
                           f32_order_key(e[k].w));
            reinterpret_cast<int4*>(s_tpos)[k * kFBlock + tid] = pv[k];
        }
        lds_sync();
        if (base + kMemTile < C) fetch(base + kMemTile);
        uint32_t key[8];
        int32_t kp[8];
        {
            // 16-byte reads: eight consecutive words per thread without 8-way bank conflicts
            const uint4 k0 = reinterpret_cast<const uint4*>(s_tile)[2 * tid];
            const uint4 k1 = reinterpret_cast<const uint4*>(s_tile)[2 * tid + 1];
            const int4 p0 = reinterpret_cast<const int4*>(s_tpos)[2 * tid];
            const int4 p1 = reinterpret_cast<const int4*>(s_tpos)[2 * tid + 1];
            key[0] = k0.x; key[1] = k0.y; key[2] = k0.z; key[3] = k0.w;
            key[4] = k1.x; key[5] = k1.y; key[6] = k1.z; key[7] = k1.w;
            kp[0] = p0.x; kp[1] = p0.y; kp[2] = p0.z; kp[3] = p0.w;
            kp[4] = p1.x; kp[5] = p1.y; kp[6] = p1.z; kp[7] = p1.w;
        }
        int nv = C - base - tid * 8;
        nv = nv < 0 ? 0 : (nv > 8 ? 8 : nv);
        uint32_t gtc = 0, eqc = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            gtc += (j < nv && (all || key[j] > kth)) ? 1u : 0u;
            eqc += (j < nv && !all && key[j] == kth) ? 1u : 0u;
        }
        // block scan of (gtc, eqc): both fit 16 bits within a tile of 8192
        const uint32_t v = (eqc << 16) | gtc;
        const uint32_t x = wave_incl_scan(v);
        if (lane == 63) s_red[wave] = x;
        lds_sync();
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kFBlock / 64; ++w) {
            const uint32_t t = s_red[w];
            before += w < wave ? t : 0u;
            tot += t;
        }
        const uint32_t packed = before + x - v;
        uint32_t r = eq_carry + (packed >> 16);                 // ties before this run
        uint32_t o = gt_carry + (packed & 0xffffu) + (r < remaining ? r : remaining);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool eq = j < nv && !all && key[j] == kth;
            const bool in = j < nv && (all || key[j] > kth || (eq && r < remaining));
            r += eq ? 1u : 0u;
            if (in && o < (uint32_t)k_eff) {
                // staged: a store here would sit ahead of the next tile's load waits
                if (k_eff <= kMemOut) s_out[o] = kp[j];
                else usel[o] = kp[j];
            }
            o += in ? 1u : 0u;
        }
        gt_carry += tot & 0xffffu;
        eq_carry += tot >> 16;
        lds_sync();                            // the tile and s_red are rewritten next
    }
    if (k_eff <= kMemOut)
        for (int i = tid; i < k_eff; i += kFBlock) usel[i] = s_out[i];
    clear_unit_hist(tot, tstride, u);
    if (tid == 0) sel_n[u] = k_eff;
}

__global__ void empty_select_kernel(int units, int32_t* sel_n, int32_t* meta) {
    const int u = blockIdx.x * blockDim.x + threadIdx.x;
    if (u < units) {
        sel_n[u] = 0;
        meta[u * 4 + 0] = 0;
        meta[u * 4 + 1] = 0;
        meta[u * 4 + 2] = 0;
        meta[u * 4 + 3] = 0;
    }
}

hipError_t probe_kernel_image() {
    hipFuncAttributes attr;
    return hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(&empty_select_kernel));
}


hipError_t launch_rerank(int chunk, const uint8_t* scores, int64_t sstride, const uint8_t* rec,
                         const uint8_t* ids, const uint8_t* lut,
                         int64_t cap, int units, int64_t sink_end, int64_t n_r, int n_chunks,
                         int max_chunks, const uint16_t* hist, int hstride, const uint32_t* tot,
                         int nbins, int64_t C, int top_k, const float* ysum,
                         const CodeTables& tab, int32_t* cand_pos, float* cand_est, int64_t cmax,
                         int32_t* meta, hipStream_t st) {
    if (nbins < 1 || nbins > kMaxBins || hstride < nbins || n_chunks > max_chunks || C < 1 ||
        C > n_r)
        return hipErrorInvalidValue;
    // Units fastest up to 64 chunks per unit: blocks are dealt to the 8 XCDs
    // round-robin in launch order, so all of a unit's blocks share one XCD and
    // its L2, which then fetches the unit's histogram and suffix-count rows
    // once instead of once per XCD (11.8 -> 10.3 us at 128K x 4; also faster
    // at 256K and 384K; the selection, attention and merge launches take the
    // same order).  With more chunks (1M tokens x 4: 128 chunks of 8192 keys,
    // four rounds of resident blocks) each XCD then holds whole units and the
    // units' uneven candidate counts leave XCDs idle: 65.3 us chunk-major
    // against 77.0 us, so chunks go fastest there.  The scan and the query
    // preparation keep chunks fastest at every size: the unit order made each
    // about 0.5 us slower at 128K.
    const int uf = n_chunks <= 64 ? 1 : 0;
    const dim3 grid(uf ? units : n_chunks, uf ? n_chunks : units), blk(kBlock);
    const size_t hist_bytes = (size_t)nbins * sizeof(uint32_t);
    if (tab.sub_dim != 8 && tab.sub_dim != 4 && tab.sub_dim != 16) return hipErrorInvalidValue;
#define PK_RERANK_M(K, MM)                                                                         \
    launch(rerank_kernel<K, MM>, grid, blk, hist_bytes, st, scores, sstride, rec, ids, lut, cap,   \
           sink_end, n_r, max_chunks, hist, hstride, tot, nbins, C, top_k, ysum, tab,              \
           cand_pos, cand_est, cmax, meta, uf)
#define PK_RERANK(K)                                                                               \
    return tab.sub_dim == 8 ? PK_RERANK_M(K, 8)                                                    \
                            : (tab.sub_dim == 4 ? PK_RERANK_M(K, 4) : PK_RERANK_M(K, 16))
    switch (chunk / kBlock) {
        case 1: PK_RERANK(1);
        case 2: PK_RERANK(2);
        case 4: PK_RERANK(4);
        case 8: PK_RERANK(8);
        case 16: PK_RERANK(16);
        case 32: PK_RERANK(32);
        default: return hipErrorInvalidValue;
    }
#undef PK_RERANK
#undef PK_RERANK_M
}

hipError_t launch_fine(const int32_t* cand_pos, const float* cand_est, int64_t cmax, int units,
                       int C, int top_k, int32_t* sel, int32_t* sel_n, uint32_t* tot, int tstride,
                       hipStream_t st) {
    // registers hold up to 64 candidates per thread (SEG of them in rows padded
    // to a multiple of SEG); beyond that (C >= 65536) the passes stream from memory
    if (C < 1 || C > cmax) return hipErrorInvalidValue;
    const dim3 grid(units), blk(kFBlock);
#define PK_FREG(S)                                                                              \
    if (C <= S * kFBlock && C < 65536 && cmax % S == 0)                                         \
    return launch(fine_reg_kernel<S>, grid, blk, 0, st, cand_pos, cand_est, cmax, C, top_k, sel, \
                  sel_n, tot, tstride)
    PK_FREG(4);
    PK_FREG(8);
    PK_FREG(16);
    PK_FREG(32);
    PK_FREG(64);
#undef PK_FREG
    return launch(fine_mem_kernel, grid, blk, 0, st, cand_pos, cand_est, cmax, C, top_k, sel,
                  sel_n, tot, tstride);
}

hipError_t launch_empty_select(int units, int32_t* sel_n, int32_t* meta, hipStream_t st) {
    return launch(empty_select_kernel, dim3((units + 63) / 64), dim3(64), 0, st, units, sel_n,
                  meta);
}

}  // namespace pk
