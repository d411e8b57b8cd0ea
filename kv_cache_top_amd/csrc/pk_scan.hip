// Collision-vote scan (gfx950): the coarse stage's per-key pass.
//
// ParisKV page, "Two-stage GPU-native retrieval pipeline", coarse candidate
// generation (collision based): every retrieval-zone key's integer score is
// the sum over subspaces of the votes its bucket received from the query
// group.  One 256-thread block per (chunk, unit) scores the chunk's keys, stores
// them as bytes, writes the chunk's suffix counts sfx_c[s] = #{score >= s} and
// adds the chunk's histogram to the unit's (device atomics into a table that
// the previous step's fine selection zeroed, or zero since creation).  The rerank (pk_retrieve.hip)
// takes the coarse threshold from these.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

// key id rows requested before the vote table's barrier (A/B on the 128K
// batch-4 workload: 8 rows 14.3 us, 4 rows 14.3, 2 rows 14.15, 1 row 13.9,
// none 14.3: with none, memory idles until the tables have arrived)
constexpr int kScanEarlyRows = 1;

// M = 8: the vote table holds one 256-entry byte row per id byte (also m = 4,
// whose rows sum two subspaces); M = 16: one hash table per 16-bit id.
template <int KPT, int M>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(KPT <= 8 ? 8 : 1))) void scan_kernel(
    const uint8_t* __restrict__ ids, int64_t cap, int64_t sink_end, int64_t n_r, int max_chunks,
    const uint8_t* __restrict__ lut, uint8_t* __restrict__ scores, int64_t sstride,
    uint16_t* __restrict__ hist, int hstride, uint32_t* __restrict__ tot, int nbins) {
    constexpr int chunk = KPT * kBlock;
    const int u = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    constexpr int kLutParts = lut_bytes<M>() / (16 * kBlock);   // 16-byte pieces per thread
    __shared__ uint32_t s_lut[lut_bytes<M>() / 4];
    extern __shared__ uint32_t s_hist[];  // scan_hist_slots(nbins) entries (sized at launch)
    const uint8_t* lut8 = reinterpret_cast<const uint8_t*>(s_lut);

    // The vote table is requested first, then the first kEarly key id rows;
    // the other rows only after the table is in LDS (the block's barrier).  A block's requests queue
    // behind those of the blocks dispatched before it on the same CU, so
    // holding back most rows until the table has arrived keeps that queue
    // short; the early rows keep memory busy meanwhile.  Scoring key j waits
    // only for its own row.
    constexpr int kEarly = KPT < kScanEarlyRows ? KPT : kScanEarlyRows;
    uint4 lut_part[kLutParts];
#pragma unroll
    for (int i = 0; i < kLutParts; ++i)
        lut_part[i] = reinterpret_cast<const uint4*>(lut + (int64_t)u * lut_bytes<M>())[tid + i * kBlock];
    const int64_t start = (int64_t)ch * chunk;
    const uint4* idrow = reinterpret_cast<const uint4*>(ids) + u * cap + sink_end;
    // loads are unconditional (index clamped to the last key, n_r >= 1) so the
    // compiler can count them and wait for each row individually
    uint4 v[KPT];
#pragma unroll
    for (int j = 0; j < kEarly; ++j) {
        const int64_t i = start + j * kBlock + tid;
        v[j] = load_nt(idrow + (i < n_r ? i : n_r - 1));
    }
#pragma unroll
    for (int i = 0; i < kLutParts; ++i) reinterpret_cast<uint4*>(s_lut)[tid + i * kBlock] = lut_part[i];
    const int per = scan_bins_per_lane(nbins);
    for (int b = tid; b < 64 * per; b += kBlock) s_hist[b] = 0;
    lds_sync();
#pragma unroll
    for (int j = kEarly; j < KPT; ++j) {
        const int64_t i = start + j * kBlock + tid;
        v[j] = load_nt(idrow + (i < n_r ? i : n_r - 1));
    }

    // histogram: scores 0..7, which most keys have, go to eight byte counters
    // per thread (at most KPT <= 32 keys each, no overflow), summed over the
    // wave at the end; larger scores go to LDS atomics
    // The scores are stored only after every key is scored: vector memory
    // counters cover loads and stores alike, so a store issued before the
    // wait for a later key's row would make that wait cover the store too.
    uint64_t c8 = 0;
    const int nval = (int)(n_r - start < chunk ? n_r - start : chunk);   // valid keys of the chunk
    uint32_t scv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const bool valid = j * kBlock + tid < nval;
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t sc = 0;
        if constexpr (M == 16) {
            sc = hashed_score(s_lut, w);
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int k = 0; k < 4; ++k) sc += lut8[(4 * a + k) * 256 + ((w[a] >> (8 * k)) & 255u)];
            }
        }
        scv[j] = sc;
        c8 += (valid && sc < 8u) ? (1ull << (sc << 3)) : 0ull;
        if (valid && sc >= 8u) atomicAdd(&s_hist[sc], 1u);
    }
    // stored as bytes, saturated at 255 (the rerank rescores saturated keys in
    // the rare case that the threshold reaches 255): staged in LDS in chunk
    // order and written after the barrier below, each thread its KPT
    // consecutive bytes in one piece, as nontemporal stores (14.1 -> 13.85 us
    // at 128K x 4; the same for the rerank's and the attention's outputs made
    // their consumers slower)
    __shared__ __align__(16) uint8_t s_sc[chunk];
#pragma unroll
    for (int j = 0; j < KPT; ++j) s_sc[j * kBlock + tid] = (uint8_t)min(scv[j], 255u);
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
    {
        uint8_t* srow = scores + u * sstride + start;
        const int b0 = tid * KPT;
        if (b0 + KPT <= nval) {
            if constexpr (KPT >= 8) {
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int q = 0; q < KPT / 8; ++q)
                    __builtin_nontemporal_store(reinterpret_cast<const u32x2*>(s_sc + b0)[q],
                                                reinterpret_cast<u32x2*>(srow + b0) + q);
            } else if constexpr (KPT == 4) {
                *reinterpret_cast<uint32_t*>(srow + b0) = *reinterpret_cast<const uint32_t*>(s_sc + b0);
            } else if constexpr (KPT == 2) {
                *reinterpret_cast<uint16_t*>(srow + b0) = *reinterpret_cast<const uint16_t*>(s_sc + b0);
            } else {
                srow[b0] = s_sc[b0];
            }
        } else {
            for (int j = 0; j < KPT && b0 + j < nval; ++j) srow[b0 + j] = s_sc[b0 + j];
        }
    }

    // waves 1..: add the chunk's counts to the unit's score histogram (zeroed
    // by the previous step's fine selection, or at creation).  wave 0: the chunk's suffix
    // counts sfx[b] = #{keys with score >= b} (a chunk holds at most 8192
    // keys: uint16).  Lane l owns the `per` consecutive bins [l*per,
    // l*per + per) (per a multiple of 4): one wave scan of the lane totals
    // gives the count above each lane's range, and each lane stores its
    // entries as 8-byte pieces, adjacent lanes at adjacent addresses.
    const int wave = tid >> 6;
    if (wave > 0) {
        // two bins per 64-bit atomic (a count stays below 2^24: no carry
        // between the halves); rows of (nbins + 1) & ~1 entries
        uint64_t* ut = reinterpret_cast<uint64_t*>(tot + (int64_t)u * ((nbins + 1) & ~1));
        for (int i = tid - 64; 2 * i < nbins; i += kBlock - 64) {
            const uint64_t h = (uint64_t)s_hist[2 * i] |
                               ((uint64_t)(2 * i + 1 < nbins ? s_hist[2 * i + 1] : 0u) << 32);
            if (h != 0u) __hip_atomic_fetch_add(ut + i, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        const int lane = tid;
        const uint4* mine = reinterpret_cast<const uint4*>(s_hist + lane * per);
        uint32_t tl = 0;
        for (int i = 0; i < per / 4; ++i) {
            const uint4 h4 = mine[i];
            tl += (h4.x + h4.y) + (h4.z + h4.w);
        }
        const uint32_t incl = wave_incl_scan(tl);
        // keys scoring above this lane's bins: the totals of the higher lanes
        uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl;
        uint2* myh = reinterpret_cast<uint2*>(hist + ((int64_t)u * max_chunks + ch) * hstride);
        for (int i = per / 4 - 1; i >= 0; --i) {
            const uint4 h4 = mine[i];
            const uint32_t s3 = run + h4.w, s2 = s3 + h4.z, s1 = s2 + h4.y, s0 = s1 + h4.x;
            run = s0;
            // rows hold hstride entries (a multiple of 8): a piece is wholly inside or outside
            if (lane * per + 4 * i < hstride)
                myh[(lane * per) / 4 + i] = make_uint2(s0 | (s1 << 16), s2 | (s3 << 16));
        }
    }
}

hipError_t launch_scan(const uint8_t* ids, int64_t cap, int units, int64_t sink_end, int64_t n_r,
                       int chunk, int n_chunks, int max_chunks, const uint8_t* lut,
                       uint8_t* scores, int64_t sstride, uint16_t* hist, int hstride,
                       uint32_t* tot, int nbins, int sub_dim, hipStream_t st) {
    if (nbins < 1 || nbins > kMaxBins || hstride < nbins || n_chunks > max_chunks)
        return hipErrorInvalidValue;
    if (sub_dim != 4 && sub_dim != 8 && sub_dim != 16) return hipErrorInvalidValue;
    const dim3 grid(n_chunks, units), blk(kBlock);
    // the histogram is the only dynamic LDS: small vote tables keep the
    // block small enough for eight resident blocks per CU
    const size_t hist_bytes = (size_t)64 * scan_bins_per_lane(nbins) * sizeof(uint32_t);
#define PK_SCAN(K)                                                                              \
    return sub_dim == 16                                                                          \
               ? launch(scan_kernel<K, 16>, grid, blk, hist_bytes, st, ids, cap, sink_end, n_r,   \
                        max_chunks, lut, scores, sstride, hist, hstride, tot, nbins)              \
               : launch(scan_kernel<K, 8>, grid, blk, hist_bytes, st, ids, cap, sink_end, n_r,    \
                        max_chunks, lut, scores, sstride, hist, hstride, tot, nbins)
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

}  // namespace pk
