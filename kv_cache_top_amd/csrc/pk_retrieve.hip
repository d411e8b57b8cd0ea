// Coarse-to-fine retrieval (gfx950).
//
// ParisKV page, "Two-stage GPU-native retrieval pipeline":
//  * coarse (collision based): every retrieval-zone key's integer score is the
//    sum over subspaces of the votes its bucket received; a small top fraction
//    of keys is kept;
//  * rerank (RSQ-IP): each candidate's raw score <k, q> is estimated from its
//    4-bit codes and scales only, and the top-k are selected.
//
// Four kernels, no cross-block synchronisation inside any of them (on gfx950
// an agent-scope release fence writes back the XCD's L2 and costs far more
// per block than a kernel boundary):
//  scan    one 256-thread block per (chunk, unit): coarse scores and the
//          chunk's score histogram;
//  select  one 1024-thread block per unit: the coarse threshold T (largest
//          score with #{score >= T} >= C), the ties at T to take, and for
//          every chunk the candidates and ties at T in the chunks before it;
//  rerank  one 256-thread block per (chunk, unit): compacts the chunk's
//          candidates in position order and estimates them with RSQ-IP;
//  fine    one 1024-thread block per unit: the k-th largest estimate by
//          value bucketing (radix select as the fallback), ties to the lower
//          position, compaction in order.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

template <int KPT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(KPT <= 8 ? 8 : 1))) void scan_kernel(
    const uint8_t* __restrict__ ids, int64_t cap, int64_t sink_end, int64_t n_r, int max_chunks,
    const uint8_t* __restrict__ lut, uint16_t* __restrict__ scores, int64_t sstride,
    uint16_t* __restrict__ hist, int hstride, int nbins) {
    constexpr int chunk = KPT * kBlock;
    const int u = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    __shared__ uint32_t s_lut[kSub * 256 / 4];
    extern __shared__ uint32_t s_hist[];  // nbins entries (sized at launch)
    const uint8_t* lut8 = reinterpret_cast<const uint8_t*>(s_lut);

    // The vote table is requested first and the key id rows right after, all
    // before any is used: scoring key j then waits only for its own row.
    const uint4 lut_part = reinterpret_cast<const uint4*>(lut + (int64_t)u * kSub * 256)[tid];
    const int64_t start = (int64_t)ch * chunk;
    const uint4* idrow = reinterpret_cast<const uint4*>(ids) + u * cap + sink_end;
    // loads are unconditional (index clamped to the last key, n_r >= 1) so the
    // compiler can count them and wait for each row individually
    uint4 v[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int64_t i = start + j * kBlock + tid;
        v[j] = idrow[i < n_r ? i : n_r - 1];
    }
    reinterpret_cast<uint4*>(s_lut)[tid] = lut_part;
    for (int b = tid; b < nbins; b += kBlock) s_hist[b] = 0;
    lds_sync();

    // histogram: scores 0..7, which most keys have, go to eight byte counters
    // per thread (at most KPT <= 32 keys each, no overflow), summed over the
    // wave at the end; larger scores go to LDS atomics
    uint64_t c8 = 0;
    uint16_t* srow = scores + u * sstride;
    const bool full = start + chunk <= n_r;   // no tail in this chunk
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int64_t i = start + j * kBlock + tid;
        const bool valid = full || i < n_r;
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t sc = 0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int k = 0; k < 4; ++k) sc += lut8[(4 * a + k) * 256 + ((w[a] >> (8 * k)) & 255u)];
        }
        if (valid) srow[i] = (uint16_t)sc;
        c8 += (valid && sc < 8u) ? (1ull << (sc << 3)) : 0ull;
        if (valid && sc >= 8u) atomicAdd(&s_hist[sc], 1u);
    }
    {
        // bytes 0..7 of c8 = counts of scores 0..7; widen to 16-bit fields
        // (a wave holds at most 64 * 32 per score) and sum over the wave
        const uint32_t lo = (uint32_t)c8, hi = (uint32_t)(c8 >> 32);
        uint32_t f[4] = {lo & 0x00ff00ffu, (lo >> 8) & 0x00ff00ffu,     // scores {0,2}, {1,3}
                         hi & 0x00ff00ffu, (hi >> 8) & 0x00ff00ffu};    // scores {4,6}, {5,7}
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t x = f[q];
            x += (uint32_t)xor16<1>((int)x);
            x += (uint32_t)xor16<2>((int)x);
            x += (uint32_t)dpp_mov<0x141>((int)x);
            x += (uint32_t)dpp_mov<0x140>((int)x);
            f[q] = (uint32_t)__builtin_amdgcn_readlane((int)x, 0) +
                   (uint32_t)__builtin_amdgcn_readlane((int)x, 16) +
                   (uint32_t)__builtin_amdgcn_readlane((int)x, 32) +
                   (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
        }
        const int lane = tid & 63;
        if (lane < 8 && lane < nbins) {
            const uint32_t fq = f[0] * (lane == 0 || lane == 2) + f[1] * (lane == 1 || lane == 3) +
                                f[2] * (lane == 4 || lane == 6) + f[3] * (lane == 5 || lane == 7);
            const uint32_t cnt = (lane & 2) ? (fq >> 16) : (fq & 0xffffu);
            if (cnt) atomicAdd(&s_hist[lane], cnt);
        }
    }
    lds_sync();

    // the chunk's histogram row (a chunk holds at most 8192 keys: uint16)
    uint16_t* myh = hist + ((int64_t)u * max_chunks + ch) * hstride;
    for (int b = tid; b < nbins; b += kBlock) myh[b] = (uint16_t)s_hist[b];
}

// ---------------------------------------------------------------------------
// select: per unit, from the chunks' histogram rows h_c
//   tot[s] = sum_c h_c[s];  ge[s] = sum_{s' >= s} tot[s'] = #{score >= s};
//   T = max s with ge[s] >= C;  need = C - ge[T+1] ties at T are taken
//   (lowest positions first);  per chunk: gt_c = sum_{s > T} h_c[s],
//   eq_c = h_c[T];  off[c] = {sum_{c'<c} gt_c', sum_{c'<c} eq_c'}.
// Chunk rows are staged through LDS (all at once for up to 80 KB of rows).
// ---------------------------------------------------------------------------
constexpr int kSBlock = 1024;
constexpr int kSelLds = 40960;      // uint16 entries of staged rows (80 KB)

// Exclusive scans of two uint32 per thread over a block of NT threads, sharing
// the barriers.  `tmp` must hold 2 * NT / 64 entries.
template <int NT>
__device__ __forceinline__ void block_excl_scan2(uint32_t& a, uint32_t& b, uint32_t* tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(a), y = wave_incl_scan(b);
    if (lane == 63) {
        tmp[wave] = x;
        tmp[NT / 64 + wave] = y;
    }
    lds_sync();
    uint32_t bx = 0, by = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        if (w < wave) {
            bx += tmp[w];
            by += tmp[NT / 64 + w];
        }
    }
    a = bx + x - a;
    b = by + y - b;
}

__global__ __launch_bounds__(kSBlock) void select_kernel(const uint16_t* __restrict__ hist,
                                                         int hstride, int max_chunks, int n_chunks,
                                                         int nbins, int64_t C, int top_k,
                                                         int32_t* __restrict__ off,
                                                         int32_t* __restrict__ meta) {
    const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ __align__(16) uint16_t s_rows[kSelLds];
    __shared__ uint32_t s_tot[kMaxBins];
    __shared__ uint32_t s_gt[kMaxChunks], s_eq[kMaxChunks];
    __shared__ uint32_t s_tmp[2 * kSBlock / 64];
    __shared__ uint32_t s_T, s_need;
    const uint16_t* H0 = hist + (int64_t)u * max_chunks * hstride;
    const int row_vec = hstride / 8;          // uint4 per row
    const int tile = kSelLds / hstride;       // rows staged at once
    const bool one_tile = n_chunks <= tile;

    // bin totals: the four lanes of a quad sum every fourth row of one bin
    for (int c0 = 0; c0 < n_chunks; c0 += tile) {
        const int rows = (n_chunks - c0) < tile ? (n_chunks - c0) : tile;
        if (c0 > 0) lds_sync();               // previous tile fully read
        for (int i = tid; i < rows * row_vec; i += kSBlock)
            reinterpret_cast<uint4*>(s_rows)[i] =
                reinterpret_cast<const uint4*>(H0 + (int64_t)c0 * hstride)[i];
        lds_sync();
        const int q = tid & 3;
        for (int b0 = 0; b0 < nbins; b0 += kSBlock / 4) {
            const int b = b0 + (tid >> 2);
            uint32_t a = 0;
            if (b < nbins)
                for (int r = q; r < rows; r += 4) a += s_rows[r * hstride + b];
            a += (uint32_t)xor16<1>((int)a);
            a += (uint32_t)xor16<2>((int)a);
            if (q == 0 && b < nbins) s_tot[b] = (c0 == 0 ? 0u : s_tot[b]) + a;
        }
    }
    lds_sync();

    // wave 0: suffix counts ge[s] = #{score >= s} (lane l owns the per bins
    // [l*per, l*per+per) of the descending order), T = max s with ge[s] >= C
    // (ge is non-increasing: T + 1 = number of bins with ge >= C), need = C -
    // ge[T+1] ties at T
    if (wave == 0) {
        const int per = (nbins + 63) / 64;
        uint32_t seg = 0;
        for (int j = 0; j < per; ++j) {
            const int r = lane * per + j;
            if (r < nbins) seg += s_tot[nbins - 1 - r];
        }
        uint32_t run = wave_incl_scan(seg) - seg;
        uint32_t n_ge = 0, ge_next = 0;       // ge of the bin just above the highest counted
        for (int j = 0; j < per; ++j) {
            const int r = lane * per + j;
            if (r < nbins) {
                const uint32_t before = run;  // ge[s + 1]
                run += s_tot[nbins - 1 - r];  // ge[s]
                if ((int64_t)run >= C) {
                    ++n_ge;
                    if ((int64_t)before < C) ge_next = before;   // s = T: ge[T+1]
                }
            }
        }
        const uint32_t T1 = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(n_ge), 63);
        const uint32_t above = (uint32_t)wave_max((uint32_t)ge_next);
        if (lane == 0) {
            s_T = T1 - 1;
            s_need = (uint32_t)(C - (int64_t)above);
        }
    }
    lds_sync();
    const int T = (int)s_T;

    // per-chunk counts: a 16-lane group per chunk sums h_c[s] over s > T
    for (int w0 = 0; w0 < n_chunks * 16; w0 += kSBlock) {
        const int w = w0 + tid;
        const int c = w >> 4, l16 = w & 15;
        const uint16_t* row = one_tile ? s_rows + c * hstride : H0 + (int64_t)c * hstride;
        uint32_t a = 0;
        if (c < n_chunks)
            for (int b = T + 1 + l16; b < nbins; b += 16) a += row[b];
        a += (uint32_t)xor16<1>((int)a);        // 16-lane sum (every lane active)
        a += (uint32_t)xor16<2>((int)a);
        a += (uint32_t)dpp_mov<0x141>((int)a);
        a += (uint32_t)dpp_mov<0x140>((int)a);
        if (c < n_chunks && l16 == 0) {
            s_gt[c] = a;
            s_eq[c] = row[T];
        }
    }
    lds_sync();
    // exclusive scans over chunks
    if (n_chunks <= 64) {
        if (wave == 0) {
            const uint32_t g = lane < n_chunks ? s_gt[lane] : 0u;
            const uint32_t e = lane < n_chunks ? s_eq[lane] : 0u;
            const uint32_t gb = wave_incl_scan(g) - g, eb = wave_incl_scan(e) - e;
            if (lane < n_chunks) {
                off[((int64_t)u * max_chunks + lane) * 2] = (int32_t)gb;
                off[((int64_t)u * max_chunks + lane) * 2 + 1] = (int32_t)eb;
            }
        }
    } else {
        const int per = (n_chunks + kSBlock - 1) / kSBlock;
        uint32_t gt_run = 0, eq_run = 0;
        for (int j = 0; j < per; ++j) {
            const int c = tid * per + j;
            if (c < n_chunks) {
                gt_run += s_gt[c];
                eq_run += s_eq[c];
            }
        }
        block_excl_scan2<kSBlock>(gt_run, eq_run, s_tmp);
        for (int j = 0; j < per; ++j) {
            const int c = tid * per + j;
            if (c < n_chunks) {
                off[((int64_t)u * max_chunks + c) * 2] = (int32_t)gt_run;
                off[((int64_t)u * max_chunks + c) * 2 + 1] = (int32_t)eq_run;
                gt_run += s_gt[c];
                eq_run += s_eq[c];
            }
        }
    }
    if (tid == 0) {
        meta[u * 4 + 0] = T;
        meta[u * 4 + 1] = (int32_t)s_need;
        meta[u * 4 + 2] = (int32_t)C;
        meta[u * 4 + 3] = (int32_t)(C < top_k ? C : top_k);
    }
}

// ---------------------------------------------------------------------------
// rerank
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(KPT <= 8 ? 8 : 1))) void rerank_kernel(
    const uint16_t* __restrict__ scores, int64_t sstride, const uint8_t* __restrict__ rec,
    int64_t cap, int64_t sink_end, int64_t n_r, int max_chunks, const int32_t* __restrict__ off,
    const int32_t* __restrict__ meta, const float* __restrict__ ysum, CodeTables tab,
    int32_t* __restrict__ cand_pos, float* __restrict__ cand_est, int64_t cmax) {
    constexpr int chunk = KPT * kBlock;
    const int u = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int l16 = tid & 15;
    __shared__ int32_t s_list[chunk];
    __shared__ float2 s_pair[256];     // nibble byte (code of coord 2i+1 << 4 | code of 2i)
    __shared__ uint32_t s_tmp[kBlock / 64];
    {
        // signed level of a 4-bit code: sign bit 3, magnitude index bits 0..2
        auto level = [&](uint32_t c) {
            float m = tab.levels[0];
#pragma unroll
            for (int l = 1; l < 8; ++l) m = ((c & 7u) == (uint32_t)l) ? tab.levels[l] : m;
            return (c & 8u) ? -m : m;
        };
        for (int b = tid; b < 256; b += kBlock) s_pair[b] = make_float2(level(b & 15u), level(b >> 4));
    }

    // one round of loads: this chunk's scores (contiguous per thread, vector
    // loads; rows are padded so these never leave the buffer), the threshold
    // and this chunk's offsets, the summed rotated query
    const int64_t start = (int64_t)ch * chunk;
    uint32_t s[KPT];
    {
        const uint16_t* sp = scores + u * sstride + start + (int64_t)tid * KPT;
        if constexpr (KPT >= 8) {
            uint4 raw[KPT / 8];
#pragma unroll
            for (int q = 0; q < KPT / 8; ++q) raw[q] = reinterpret_cast<const uint4*>(sp)[q];
#pragma unroll
            for (int q = 0; q < KPT / 8; ++q) {
                const uint32_t w4[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    s[8 * q + 2 * k] = w4[k] & 0xffffu;
                    s[8 * q + 2 * k + 1] = w4[k] >> 16;
                }
            }
        } else if constexpr (KPT == 4) {
            const uint2 raw = *reinterpret_cast<const uint2*>(sp);
            s[0] = raw.x & 0xffffu; s[1] = raw.x >> 16; s[2] = raw.y & 0xffffu; s[3] = raw.y >> 16;
        } else if constexpr (KPT == 2) {
            const uint32_t raw = *reinterpret_cast<const uint32_t*>(sp);
            s[0] = raw & 0xffffu; s[1] = raw >> 16;
        } else {
            s[0] = sp[0];
        }
    }
    const int T = meta[u * 4 + 0];
    const uint32_t need = (uint32_t)meta[u * 4 + 1];
    const uint32_t gt_chunk = (uint32_t)off[((int64_t)u * max_chunks + ch) * 2];
    const uint32_t eq_chunk = (uint32_t)off[((int64_t)u * max_chunks + ch) * 2 + 1];
    float y[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) y[r] = ysum[(int64_t)u * kD + 8 * l16 + r];

    // this chunk's candidates, in position order: keys above T, and ties at T
    // while the unit's tie budget lasts.  One packed scan of (ties, above).
    uint32_t eqc = 0, gtc = 0;
    const int kbase = (int)start + tid * KPT;   // retrieval zone < 2^24 keys
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (kbase + j >= (int)n_r) s[j] = 0xffffffffu;
        gtc += (s[j] != 0xffffffffu && s[j] > (uint32_t)T) ? 1u : 0u;
        eqc += (s[j] == (uint32_t)T) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t packed = block_excl_scan((eqc << 16) | gtc, s_tmp, &tot);
    const uint32_t eq_t = packed >> 16, gt_t = packed & 0xffffu;
    const uint32_t taken_before_chunk = eq_chunk < need ? eq_chunk : need;
    auto taken = [&](uint32_t e) { return (e < need ? e : need) - taken_before_chunk; };
    uint32_t at = gt_t + taken(eq_chunk + eq_t);
    const uint32_t n_mem = (tot & 0xffffu) + taken(eq_chunk + (tot >> 16));
    const uint32_t cand_before = gt_chunk + taken_before_chunk;
    uint32_t rank = eq_chunk + eq_t;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        bool in = false;
        if (s[j] != 0xffffffffu) {
            if (s[j] > (uint32_t)T) in = true;
            else if (s[j] == (uint32_t)T) in = (rank++ < need);
        }
        if (in) s_list[at++] = (int32_t)(sink_end + start + (int64_t)tid * KPT + j);
    }
    lds_sync();

    // RSQ-IP: est = sum_b w_b <v_b, Ysum_b> / sqrt(d), Ysum = sum_g H D q_g;
    // 16 lanes per candidate, lane b reading subspace b's nibble word and w.
    // A group fetches the records of up to kBatch candidates before using any.
    // Codes are dequantised two at a time from the byte-indexed level pairs.
    // Record offsets within the unit fit 32 bits (capacity <= 2^24 keys).
    constexpr int kBatch = 16;
    const float inv_sqrt_d = 0.08838834764831845f;
    const int grp = tid >> 4;
    const uint8_t* urec = rec + (int64_t)u * cap * kRec;
    int32_t* upos = cand_pos + (int64_t)u * cmax;
    float* uest = cand_est + (int64_t)u * cmax;
    for (int i0 = grp; i0 < (int)n_mem; i0 += kBatch * (kBlock / 16)) {
        uint32_t nib[kBatch];
        float w[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * (kBlock / 16);
            const int32_t p = s_list[i < (int)n_mem ? i : i0];
            const uint32_t ro = (uint32_t)p * (uint32_t)kRec + 4u * (uint32_t)l16;
            nib[k] = *reinterpret_cast<const uint32_t*>(urec + ro);
            w[k] = *reinterpret_cast<const float*>(urec + ro + 64u);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int i = i0 + k * (kBlock / 16);
            if (i >= (int)n_mem) break;          // uniform in the 16-lane group
            float dot = 0.0f;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float2 lv = s_pair[(nib[k] >> (8 * b)) & 255u];
                dot = fmaf(lv.x, y[2 * b], dot);
                dot = fmaf(lv.y, y[2 * b + 1], dot);
            }
            const float e = sum16(w[k] * dot);
            const uint32_t o = cand_before + (uint32_t)i;
            if (l16 == 0 && (int64_t)o < cmax) {
                upos[o] = s_list[i];
                uest[o] = e * inv_sqrt_d;
            }
        }
    }
}

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
// ---------------------------------------------------------------------------
constexpr int kFBlock = 1024;
constexpr int kFineLds = 16384;  // candidates held in LDS; more are read from memory
constexpr int kRadixBins = 2048;
constexpr int kRankMax = 1024;   // bucket members ranked directly

__device__ __forceinline__ float order_key_to_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// one wave finds the digit d of the histogram h[0..nb) holding the
// `remaining`-th largest element: above(d) < remaining <= above(d) + h[d],
// above(d) = sum of h over digits > d.  Writes d and above(d).
__device__ __forceinline__ void digit_search(const uint32_t* s_h, int nb, uint32_t remaining,
                                             int lane, uint32_t* s_digit, uint32_t* s_above) {
    // lane owns the per = nb/64 digits [lane*per, lane*per+per), read as
    // 16-byte vectors; larger digits belong to higher lanes
    const int per = nb / 64;
    uint32_t h[32];
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
        if (4 * q4 < per) {
            const uint4 x = reinterpret_cast<const uint4*>(s_h + lane * per)[q4];
            h[4 * q4] = x.x;
            h[4 * q4 + 1] = x.y;
            h[4 * q4 + 2] = x.z;
            h[4 * q4 + 3] = x.w;
        } else {
            h[4 * q4] = h[4 * q4 + 1] = h[4 * q4 + 2] = h[4 * q4 + 3] = 0;
        }
    }
    uint32_t segsum = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) segsum += h[j];
    // counts in the digits of the lanes above this one
    const uint32_t incl = wave_incl_scan(segsum);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    uint32_t above = total - incl;
    if (above < remaining && above + segsum >= remaining) {
#pragma unroll
        for (int j = 31; j >= 0; --j) {
            if (j < per) {
                if (above < remaining && above + h[j] >= remaining) {
                    *s_digit = (uint32_t)(lane * per + j);
                    *s_above = above;
                }
                above += h[j];
            }
        }
    }
}

template <int SEG, bool IN_LDS>
__global__ __launch_bounds__(kFBlock) void fine_kernel(const int32_t* __restrict__ cand_pos,
                                                       const float* __restrict__ cand_est,
                                                       int64_t cmax, int C, int top_k,
                                                       int32_t* __restrict__ sel,
                                                       int32_t* __restrict__ sel_n) {
    const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ uint32_t s_key[SEG * kFBlock];
    __shared__ int32_t s_pos[SEG * kFBlock];
    __shared__ __align__(16) uint32_t s_h[kRadixBins];
    __shared__ uint32_t s_mem[kRankMax];
    __shared__ uint32_t s_tmp[kFBlock / 64];
    __shared__ uint32_t s_wmax[kFBlock / 64], s_wmin[kFBlock / 64];
    __shared__ uint32_t s_digit, s_above, s_cnt, s_kth, s_gt;
    const float* est = cand_est + (int64_t)u * cmax;
    const int32_t* cpos = cand_pos + (int64_t)u * cmax;
    const int k_eff = C < top_k ? C : top_k;
    constexpr bool in_lds = IN_LDS;   // all candidates held in LDS (C <= SEG * kFBlock)
    // estimates and positions are read once, coalesced, into LDS; thread t
    // later compacts the contiguous segment [t*seg, (t+1)*seg)
    const int seg = (C + kFBlock - 1) / kFBlock;
    const int b0 = tid * seg;
    uint32_t kmax = 0, kmin_inv = 0;  // running max of keys and of ~keys
    if constexpr (in_lds) {
        float e[SEG];
        int32_t p[SEG];
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            const int i = j * kFBlock + tid;
            const int ic = i < C ? i : C - 1;   // clamped: a real element
            e[j] = est[ic];
            p[j] = cpos[ic];
        }
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            const int i = j * kFBlock + tid;
            const uint32_t key = f32_order_key(e[j]);
            if (i < C) {
                s_key[i] = key;
                s_pos[i] = p[j];
            }
            kmax = max(kmax, key);
            kmin_inv = max(kmin_inv, ~key);
        }
    } else {
        for (int i0 = tid; i0 < C; i0 += 8 * kFBlock) {
            float e[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * kFBlock;
                e[k] = est[i < C ? i : C - 1];        // clamped: a real element
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t key = f32_order_key(e[k]);
                kmax = max(kmax, key);
                kmin_inv = max(kmin_inv, ~key);
            }
        }
    }
    kmax = wave_max(kmax);
    kmin_inv = wave_max(kmin_inv);
    if (lane == 0) {
        s_wmax[wave] = kmax;
        s_wmin[wave] = kmin_inv;
    }
    if (tid == 0) s_cnt = 0;
    lds_sync();
    // f(i, key) for every candidate i = tid + j * kFBlock; from memory (too many
    // candidates for LDS) eight loads are in flight at a time
    auto for_all = [&](auto&& f) {
        if constexpr (in_lds) {
            for (int i = tid; i < C; i += kFBlock) f(i, s_key[i]);
            return;
        }
        for (int i0 = tid; i0 < C; i0 += 8 * kFBlock) {
            float e[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * kFBlock;
                e[k] = est[i < C ? i : C - 1];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * kFBlock;
                if (i < C) f(i, f32_order_key(e[k]));
            }
        }
    };
    // f(i, key) for this thread's segment [b0, b0 + seg), in order
    auto for_segment = [&](auto&& f) {
        if constexpr (in_lds) {
            for (int j = 0; j < seg; ++j)
                if (b0 + j < C) f(b0 + j, s_key[b0 + j]);
            return;
        }
        for (int j0 = 0; j0 < seg; j0 += 8) {
            float e[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = b0 + j0 + k;
                e[k] = est[(j0 + k < seg && i < C) ? i : C - 1];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = b0 + j0 + k;
                if (j0 + k < seg && i < C) f(i, f32_order_key(e[k]));
            }
        }
    };

    uint32_t kth = 0, remaining = (uint32_t)k_eff;
    const bool all = k_eff >= C;
    bool found = all;
    if (!all) {
        kmax = 0;
        kmin_inv = 0;
#pragma unroll
        for (int w = 0; w < kFBlock / 64; ++w) {
            kmax = max(kmax, s_wmax[w]);
            kmin_inv = max(kmin_inv, s_wmin[w]);
        }
        const float vmax = order_key_to_f32(kmax), vmin = order_key_to_f32(~kmin_inv);
        const float span = vmax - vmin;
        const float scale = (float)kRadixBins / span;
        // finite, positive span and scale: (v - vmin) * scale is then finite and in [0, ~2048]
        if (span > 0.0f && span <= 3.0e38f && scale <= 3.0e38f) {
            const float top = (float)(kRadixBins - 1);
            auto bucket = [&](uint32_t key) -> uint32_t {
                return (uint32_t)fminf((order_key_to_f32(key) - vmin) * scale, top);
            };
            for (int b = tid; b < kRadixBins; b += kFBlock) s_h[b] = 0;
            lds_sync();
            for_all([&](int, uint32_t key) { atomicAdd(&s_h[bucket(key)], 1u); });
            lds_sync();
            if (tid < 64) digit_search(s_h, kRadixBins, remaining, lane, &s_digit, &s_above);
            lds_sync();
            const uint32_t bstar = s_digit;
            const uint32_t rem = remaining - s_above;   // 1 <= rem <= members of bstar
            const uint32_t n_b = s_h[bstar];
            if (n_b <= (uint32_t)kRankMax) {
                for_all([&](int, uint32_t key) {
                    if (bucket(key) == bstar) s_mem[atomicAdd(&s_cnt, 1u)] = key;
                });
                lds_sync();
                // exact rank of every member: the k-th value has gt < rem <= ge
                for (int m = tid; m < (int)n_b; m += kFBlock) {
                    const uint32_t km = s_mem[m];
                    uint32_t gt = 0, ge = 0;
                    for (int j = 0; j < (int)n_b; ++j) {
                        const uint32_t kj = s_mem[j];
                        gt += kj > km ? 1u : 0u;
                        ge += kj >= km ? 1u : 0u;
                    }
                    if (gt < rem && rem <= ge) {  // every writer writes the same values
                        s_kth = km;
                        s_gt = gt;
                    }
                }
                lds_sync();
                kth = s_kth;
                remaining = rem - s_gt;
                found = true;
            }
        }
    }
    if (!found) {
        uint32_t prefix = 0, pmask = 0;
        for (int p = 0; p < 3; ++p) {
            const int width = p == 2 ? 10 : 11;               // digits of 11, 11, 10 bits
            const int shift = p == 0 ? 21 : (p == 1 ? 10 : 0);
            const uint32_t dmask = (1u << width) - 1u;
            const int nb = 1 << width;
            for (int b = tid; b < nb; b += kFBlock) s_h[b] = 0;
            lds_sync();
            for_all([&](int, uint32_t key) {
                if ((key & pmask) == prefix) atomicAdd(&s_h[(key >> shift) & dmask], 1u);
            });
            lds_sync();
            if (tid < 64) digit_search(s_h, nb, remaining, lane, &s_digit, &s_above);
            lds_sync();
            prefix |= s_digit << shift;
            pmask |= dmask << shift;
            remaining -= s_above;
            lds_sync();
        }
        kth = prefix;
    }
    // compaction: thread t owns candidates [t*seg, (t+1)*seg); one block scan of
    // (ties at kth, keys above kth) gives both offsets
    uint32_t eqc = 0, gtc = 0;
    for_segment([&](int, uint32_t key) {
        gtc += (all || key > kth) ? 1u : 0u;
        eqc += (!all && key == kth) ? 1u : 0u;
    });
    uint32_t tot, r, gt_before;
    if (C < 65536) {
        const uint32_t packed = block_excl_scan_t<kFBlock>((eqc << 16) | gtc, s_tmp, &tot);
        r = packed >> 16;                       // ties at kth before this segment
        gt_before = packed & 0xffffu;
    } else {
        r = block_excl_scan_t<kFBlock>(eqc, s_tmp, &tot);
        gt_before = block_excl_scan_t<kFBlock>(gtc, s_tmp, &tot);
    }
    uint32_t o = gt_before + (r < remaining ? r : remaining);
    for_segment([&](int i, uint32_t key) {
        const bool eq = !all && key == kth;
        const bool in = all || key > kth || (eq && r < remaining);
        r += eq ? 1u : 0u;
        if (in && o < (uint32_t)k_eff) {
            int32_t pj;
            if constexpr (in_lds) pj = s_pos[i];
            else pj = cpos[i];
            sel[(int64_t)u * top_k + o] = pj;
        }
        o += in ? 1u : 0u;
    });
    if (tid == 0) sel_n[u] = k_eff;
}

// writes an empty selection (retrieval zone empty)
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

hipError_t launch_scan(const uint8_t* ids, int64_t cap, int units, int64_t sink_end, int64_t n_r,
                       int chunk, int n_chunks, int max_chunks, const uint8_t* lut,
                       uint16_t* scores, int64_t sstride, uint16_t* hist, int hstride, int nbins,
                       hipStream_t st) {
    if (nbins < 1 || nbins > kMaxBins) return hipErrorInvalidValue;
    const dim3 grid(n_chunks, units), blk(kBlock);
    // the histogram is the only dynamic LDS: small vote tables keep the
    // block small enough for eight resident blocks per CU
    const size_t hist_bytes = (size_t)nbins * sizeof(uint32_t);
#define PK_SCAN(K)                                                                         \
    return launch(scan_kernel<K>, grid, blk, hist_bytes, st, ids, cap, sink_end, n_r,        \
                  max_chunks, lut, scores, sstride, hist, hstride, nbins)
    switch (chunk / kBlock) {
        case 1: PK_SCAN(1);
        case 2: PK_SCAN(2);
        case 4: PK_SCAN(4);
        case 8: PK_SCAN(8);
        case 16: PK_SCAN(16);
        case 32: PK_SCAN(32);
        default: return hipErrorInvalidValue;
    }
#undef PK_SCAN
}

hipError_t launch_select(const uint16_t* hist, int hstride, int max_chunks, int n_chunks,
                         int units, int nbins, int64_t C, int top_k, int32_t* off, int32_t* meta,
                         hipStream_t st) {
    if (n_chunks < 1 || n_chunks > kMaxChunks || hstride > kSelLds) return hipErrorInvalidValue;
    return launch(select_kernel, dim3(units), dim3(kSBlock), 0, st, hist, hstride, max_chunks,
                  n_chunks, nbins, C, top_k, off, meta);
}

hipError_t launch_rerank(int chunk, const uint16_t* scores, int64_t sstride, const uint8_t* rec,
                         int64_t cap, int units, int64_t sink_end, int64_t n_r, int n_chunks,
                         int max_chunks, const int32_t* off, const int32_t* meta,
                         const float* ysum, const CodeTables& tab, int32_t* cand_pos,
                         float* cand_est, int64_t cmax, hipStream_t st) {
    const dim3 grid(n_chunks, units), blk(kBlock);
#define PK_RERANK(K)                                                                        \
    return launch(rerank_kernel<K>, grid, blk, 0, st, scores, sstride, rec, cap, sink_end, n_r, \
                  max_chunks, off, meta, ysum, tab, cand_pos, cand_est, cmax)
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
}

hipError_t launch_fine(const int32_t* cand_pos, const float* cand_est, int64_t cmax, int units,
                       int C, int top_k, int32_t* sel, int32_t* sel_n, hipStream_t st) {
    // the segment length covers C in LDS up to kFineLds candidates; beyond that
    // the keys are read from memory
    const dim3 grid(units), blk(kFBlock);
    if (C <= 4 * kFBlock)
        return launch(fine_kernel<4, true>, grid, blk, 0, st, cand_pos, cand_est, cmax, C, top_k,
                      sel, sel_n);
    if (C <= 8 * kFBlock)
        return launch(fine_kernel<8, true>, grid, blk, 0, st, cand_pos, cand_est, cmax, C, top_k,
                      sel, sel_n);
    if (C <= kFineLds)
        return launch(fine_kernel<kFineLds / kFBlock, true>, grid, blk, 0, st, cand_pos, cand_est,
                      cmax, C, top_k, sel, sel_n);
    return launch(fine_kernel<1, false>, grid, blk, 0, st, cand_pos, cand_est, cmax, C, top_k, sel,
                  sel_n);
}

hipError_t launch_empty_select(int units, int32_t* sel_n, int32_t* meta, hipStream_t st) {
    return launch(empty_select_kernel, dim3((units + 63) / 64), dim3(64), 0, st, units, sel_n,
                  meta);
}

}  // namespace pk
