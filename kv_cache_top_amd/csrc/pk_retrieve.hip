// Coarse-to-fine retrieval (gfx950).
//
// ParisKV page, "Two-stage GPU-native retrieval pipeline":
//  * coarse (collision based): every retrieval-zone key's integer score is the
//    sum over subspaces of the votes its bucket received; a small top fraction
//    of keys is kept;
//  * rerank (RSQ-IP): each candidate's raw score <k, q> is estimated from its
//    4-bit codes and scales only, and the top-k are selected.
//
// Work split.  The retrieval zone of every unit is cut into chunks; the scan
// and the rerank launch one 256-thread block per (chunk, unit).  Each unit's
// last finishing block (an atomic ticket per unit, no spinning) does that
// unit's serial tail: the coarse threshold after the scan, the fine top-k
// after the rerank.  Tickets are reset by the block that takes the last one,
// so nothing needs clearing between launches.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

// per-unit coarse-selection summary written by the scan's last block
//   meta[u] = {threshold score T, ties at T taken, C, k_eff}
//   off[u][chunk] = {candidates before this chunk, keys scoring T before this chunk}

__global__ __launch_bounds__(kBlock) void scan_kernel(
    const uint8_t* __restrict__ ids, int64_t cap, int64_t sink_end, int64_t n_r, int chunk,
    int n_chunks, int max_chunks, const uint8_t* __restrict__ lut, uint16_t* __restrict__ scores,
    uint32_t* __restrict__ bhist, int nbins, uint32_t* __restrict__ tickets,
    int32_t* __restrict__ meta, int32_t* __restrict__ off, int64_t C, int top_k) {
    const int u = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    __shared__ uint32_t s_lut[kSub * 256 / 4];
    __shared__ uint32_t s_hist[kMaxBins];
    __shared__ uint32_t s_tmp[kBlock / 64];
    __shared__ int s_last;
    const uint8_t* lut8 = reinterpret_cast<const uint8_t*>(s_lut);

    reinterpret_cast<uint4*>(s_lut)[tid] =
        reinterpret_cast<const uint4*>(lut + (int64_t)u * kSub * 256)[tid];
    for (int b = tid; b < nbins; b += kBlock) s_hist[b] = 0;
    __syncthreads();

    const int64_t start = (int64_t)ch * chunk;
    const int64_t end = (start + chunk < n_r) ? start + chunk : n_r;
    const uint4* idrow = reinterpret_cast<const uint4*>(ids) + u * cap + sink_end;
    uint16_t* srow = scores + u * cap;
    for (int64_t i = start + tid; i < end; i += kBlock) {
        const uint4 v = idrow[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int k = 0; k < 4; ++k) s += lut8[(4 * j + k) * 256 + ((w[j] >> (8 * k)) & 255u)];
        }
        srow[i] = (uint16_t)s;
        atomicAdd(&s_hist[s], 1u);
    }
    __syncthreads();
    uint32_t* myhist = bhist + ((int64_t)u * max_chunks + ch) * nbins;
    for (int b = tid; b < nbins; b += kBlock) myhist[b] = s_hist[b];

    // ---- ticket: the unit's last block derives the threshold and chunk offsets
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&tickets[u], 1u) == (uint32_t)(n_chunks - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    for (int b = tid; b < nbins; b += kBlock) {
        uint32_t a = 0;
        const uint32_t* col = bhist + (int64_t)u * max_chunks * nbins + b;
        for (int c = 0; c < n_chunks; ++c) a += col[(int64_t)c * nbins];
        s_hist[b] = a;
    }
    __syncthreads();

    // T = largest score s with #{score >= s} >= C.  Thread t owns the bins
    // with reversed index r = nbins-1-s in [t*per, t*per+per).
    __shared__ int s_T, s_need;
    if (tid == 0) {
        s_T = 0;
        s_need = 0;
    }
    const int per = (nbins + kBlock - 1) / kBlock;
    uint32_t seg = 0;
    for (int j = 0; j < per; ++j) {
        const int r = tid * per + j;
        if (r < nbins) seg += s_hist[nbins - 1 - r];
    }
    uint32_t tot;
    uint32_t run = block_excl_scan(seg, s_tmp, &tot);
    for (int j = 0; j < per; ++j) {
        const int r = tid * per + j;
        if (r < nbins) {
            const uint32_t h = s_hist[nbins - 1 - r];
            if ((int64_t)run < C && (int64_t)(run + h) >= C) {
                s_T = nbins - 1 - r;
                s_need = (int)(C - run);
            }
            run += h;
        }
    }
    __syncthreads();
    const int T = s_T, need = s_need;

    // per-chunk counts above / at the threshold, then two exclusive scans
    __shared__ uint32_t s_gt[kMaxChunks], s_eq[kMaxChunks];
    for (int c = tid; c < n_chunks; c += kBlock) {
        const uint32_t* h = bhist + ((int64_t)u * max_chunks + c) * nbins;
        uint32_t gt = 0;
        for (int b = T + 1; b < nbins; ++b) gt += h[b];
        s_gt[c] = gt;
        s_eq[c] = h[T];
    }
    __syncthreads();
    const int cper = (n_chunks + kBlock - 1) / kBlock;
    uint32_t eq_seg = 0;
    for (int j = 0; j < cper; ++j) {
        const int c = tid * cper + j;
        if (c < n_chunks) eq_seg += s_eq[c];
    }
    uint32_t eq_run = block_excl_scan(eq_seg, s_tmp, &tot);
    uint32_t take_seg = 0;
    for (int j = 0; j < cper; ++j) {
        const int c = tid * cper + j;
        if (c < n_chunks) {
            const int64_t left = (int64_t)need - eq_run;
            const uint32_t take_eq =
                left <= 0 ? 0u : (left >= (int64_t)s_eq[c] ? s_eq[c] : (uint32_t)left);
            s_gt[c] += take_eq;          // now: candidates contributed by chunk c
            off[((int64_t)u * max_chunks + c) * 2 + 1] = (int32_t)eq_run;
            eq_run += s_eq[c];
            take_seg += s_gt[c];
        }
    }
    uint32_t cand_run = block_excl_scan(take_seg, s_tmp, &tot);
    for (int j = 0; j < cper; ++j) {
        const int c = tid * cper + j;
        if (c < n_chunks) {
            off[((int64_t)u * max_chunks + c) * 2] = (int32_t)cand_run;
            cand_run += s_gt[c];
        }
    }
    if (tid == 0) {
        meta[u * 4 + 0] = T;
        meta[u * 4 + 1] = need;
        meta[u * 4 + 2] = (int32_t)C;
        meta[u * 4 + 3] = (int32_t)(C < top_k ? C : top_k);
        tickets[u] = 0;
    }
}

// ---------------------------------------------------------------------------
// rerank: compact the chunk's candidates (score > T, or = T within the first
// `need` ties in position order), estimate each with RSQ-IP, write
// (position, estimate) at the candidate's global rank.  16 lanes per
// candidate, lane b reading subspace b's 4 nibble bytes and its w.
// est = sum_b w_b <v_b, Ysum_b> / sqrt(d), Ysum = sum_g H D q_g.
// ---------------------------------------------------------------------------
template <int KPT>
__global__ __launch_bounds__(kBlock) void rerank_kernel(
    const uint16_t* __restrict__ scores, const uint8_t* __restrict__ rec, int64_t cap,
    int64_t sink_end, int64_t n_r, int n_chunks, int max_chunks, const int32_t* __restrict__ meta,
    const int32_t* __restrict__ off, const float* __restrict__ ysum, CodeTables tab,
    int32_t* __restrict__ cand_pos, float* __restrict__ cand_est, int64_t cmax,
    uint32_t* __restrict__ tickets, int top_k, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_n) {
    constexpr int chunk = KPT * kBlock;
    const int u = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
    const int l16 = tid & 15;
    __shared__ int32_t s_list[chunk];
    __shared__ float s_tbl[16];
    __shared__ uint32_t s_tmp[kBlock / 64];
    __shared__ int s_last;
    if (tid < 16) s_tbl[tid] = ((tid & 8) ? -1.0f : 1.0f) * tab.levels[tid & 7];

    const int T = meta[u * 4 + 0], need = meta[u * 4 + 1];
    const int C = meta[u * 4 + 2];
    const int32_t cand_before = off[((int64_t)u * max_chunks + ch) * 2];
    const int32_t eq_before = off[((int64_t)u * max_chunks + ch) * 2 + 1];
    const int64_t start = (int64_t)ch * chunk;

    uint32_t s[KPT];
    uint32_t eqc = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int64_t i = start + (int64_t)tid * KPT + j;
        s[j] = (i < n_r) ? (uint32_t)scores[u * cap + i] : 0xffffffffu;
        eqc += (s[j] == (uint32_t)T) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t rank = eq_before + block_excl_scan(eqc, s_tmp, &tot);
    uint32_t mask = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        bool in = false;
        if (s[j] != 0xffffffffu) {
            if (s[j] > (uint32_t)T) in = true;
            else if (s[j] == (uint32_t)T) in = (rank++ < (uint32_t)need);
        }
        mask |= (in ? 1u : 0u) << j;
    }
    uint32_t mine = __popc(mask);
    uint32_t n_mem;
    uint32_t at = block_excl_scan(mine, s_tmp, &n_mem);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if ((mask >> j) & 1u) s_list[at++] = (int32_t)(sink_end + start + (int64_t)tid * KPT + j);
    __syncthreads();

    float y[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) y[r] = ysum[(int64_t)u * kD + 8 * l16 + r];
    const float inv_sqrt_d = 0.08838834764831845f;
    for (int i = tid >> 4; i < (int)n_mem; i += kBlock / 16) {
        const int32_t pos = s_list[i];
        const uint8_t* r = rec + ((int64_t)u * cap + pos) * kRec;
        const uint32_t nib = reinterpret_cast<const uint32_t*>(r)[l16];
        const float w = reinterpret_cast<const float*>(r + 64)[l16];
        float dot = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) dot = fmaf(s_tbl[(nib >> (4 * k)) & 15u], y[k], dot);
        const float e = sum16(w * dot);
        if (l16 == 0 && cand_before + i < cmax) {
            cand_pos[(int64_t)u * cmax + cand_before + i] = pos;
            cand_est[(int64_t)u * cmax + cand_before + i] = e * inv_sqrt_d;
        }
    }

    // ---- ticket: the unit's last block selects the top-k among its C candidates
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&tickets[u], 1u) == (uint32_t)(n_chunks - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int k_eff = C < top_k ? C : top_k;
    const float* est = cand_est + (int64_t)u * cmax;
    const int32_t* cpos = cand_pos + (int64_t)u * cmax;
    __shared__ uint32_t s_h[256];
    __shared__ uint32_t s_digit, s_above;
    uint32_t prefix = 0, pmask = 0;
    uint32_t remaining = (uint32_t)k_eff;
    if (k_eff < C) {
        // MSB-first radix select of the k_eff-th largest order key, 8 bits a pass
        for (int shift = 24; shift >= 0; shift -= 8) {
            s_h[tid] = 0;
            __syncthreads();
            for (int i = tid; i < C; i += kBlock) {
                const uint32_t key = f32_order_key(est[i]);
                if ((key & pmask) == prefix) atomicAdd(&s_h[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            // thread t looks at digit 255 - t; inclusive count of digits >= it
            const uint32_t hcount = s_h[255 - tid];
            uint32_t ge_tot;
            const uint32_t above = block_excl_scan(hcount, s_tmp, &ge_tot);  // digits > 255-t
            if (above < remaining && above + hcount >= remaining) {
                s_digit = 255u - tid;
                s_above = above;
            }
            __syncthreads();
            prefix |= s_digit << shift;
            pmask |= 255u << shift;
            remaining -= s_above;
            __syncthreads();
        }
    } else {
        prefix = 0;           // everything qualifies
        pmask = 0;
        remaining = 0xffffffffu;
    }
    const uint32_t kth = prefix;
    // compaction in candidate (= position) order
    uint32_t eq_run = 0, out_run = 0;
    for (int base = 0; base < C; base += kBlock) {
        const int i = base + tid;
        uint32_t key = 0;
        bool valid = i < C;
        if (valid) key = f32_order_key(est[i]);
        const bool eq = valid && (k_eff < C) && key == kth;
        uint32_t eq_tot;
        const uint32_t eq_rank = eq_run + block_excl_scan(eq ? 1u : 0u, s_tmp, &eq_tot);
        const bool in = valid && ((k_eff >= C) || key > kth || (eq && eq_rank < remaining));
        uint32_t in_tot;
        const uint32_t o = out_run + block_excl_scan(in ? 1u : 0u, s_tmp, &in_tot);
        if (in && o < (uint32_t)k_eff) sel[(int64_t)u * top_k + o] = cpos[i];
        eq_run += eq_tot;
        out_run += in_tot;
    }
    if (tid == 0) {
        sel_n[u] = k_eff;
        tickets[u] = 0;
    }
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

hipError_t launch_scan(const uint8_t* ids, int64_t cap, int units, int64_t sink_end, int64_t n_r,
                       int chunk, int n_chunks, int max_chunks, const uint8_t* lut,
                       uint16_t* scores, uint32_t* bhist, int nbins, uint32_t* tickets,
                       int32_t* meta, int32_t* off, int64_t C, int top_k, hipStream_t st) {
    scan_kernel<<<dim3(n_chunks, units), dim3(kBlock), 0, st>>>(
        ids, cap, sink_end, n_r, chunk, n_chunks, max_chunks, lut, scores, bhist, nbins, tickets,
        meta, off, C, top_k);
    return hipGetLastError();
}

hipError_t launch_rerank(int chunk, const uint16_t* scores, const uint8_t* rec, int64_t cap,
                         int units, int64_t sink_end, int64_t n_r, int n_chunks, int max_chunks,
                         const int32_t* meta, const int32_t* off, const float* ysum,
                         const CodeTables& tab, int32_t* cand_pos, float* cand_est, int64_t cmax,
                         uint32_t* tickets, int top_k, int32_t* sel, int32_t* sel_n,
                         hipStream_t st) {
    const dim3 grid(n_chunks, units), blk(kBlock);
#define PK_RERANK(K)                                                                           \
    rerank_kernel<K><<<grid, blk, 0, st>>>(scores, rec, cap, sink_end, n_r, n_chunks,          \
                                           max_chunks, meta, off, ysum, tab, cand_pos,         \
                                           cand_est, cmax, tickets, top_k, sel, sel_n)
    switch (chunk / kBlock) {
        case 1: PK_RERANK(1); break;
        case 2: PK_RERANK(2); break;
        case 4: PK_RERANK(4); break;
        case 8: PK_RERANK(8); break;
        case 16: PK_RERANK(16); break;
        case 32: PK_RERANK(32); break;
        default: return hipErrorInvalidValue;
    }
#undef PK_RERANK
    return hipGetLastError();
}

hipError_t launch_empty_select(int units, int32_t* sel_n, int32_t* meta, hipStream_t st) {
    empty_select_kernel<<<dim3((units + 63) / 64), dim3(64), 0, st>>>(units, sel_n, meta);
    return hipGetLastError();
}

}  // namespace pk
