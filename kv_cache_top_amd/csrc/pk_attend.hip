// Sparse GQA decode attention kernels (gfx950): one split per 256-thread
// block (the split itself is in pk_attend.hpp), and the merge of the splits.
#include "pk_attend.hpp"
#include "pk_launch.hpp"

namespace pk {

// split sp0 + blockIdx.y of unit blockIdx.x (units fastest: a unit's blocks share an XCD)
template <typename T, int G, bool RING>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendArgs<T> a, int sp0) {
    __shared__ AttendLds<G> lds;
    attend_split<T, G, RING>(a, blockIdx.x, sp0 + blockIdx.y, threadIdx.x, true, lds);
}

// merge of the split partials: one 128-thread block per (query head, unit),
// thread d owning output coordinate d.  Splits are folded in groups of CG
// (24 when that covers them all, as in a decode step with a few hot-zone
// splits and the selection's 16; else 32), everything of a group requested
// before any is used: lane k of each wave reads (m, l) of split s0 + k, the
// group maximum M' rescales the running sums, lane k's weight e^(m - M') is
// broadcast to the wave, and acc += o_s e^(m_s - M'), L += l_s e^(m_s - M').
// out = acc / L.  No branch stands between a group's loads and their use (a
// branch there lets the compiler sink the row loads below it: two memory
// round trips instead of one).  A split with nothing attended has m = -inf,
// l = 0, o = 0 and weight 0; a unit's partials span less than 2^31 floats,
// so offsets are 32-bit.
template <int CG>
__global__ __launch_bounds__(kD) void combine_kernel(const float* __restrict__ part, int G,
                                                     int n_splits, float* __restrict__ out) {
    const int g = blockIdx.y, u = blockIdx.x, d = threadIdx.x, lane = d & 63;
    const int stride = G * (kD + 2);      // floats between splits
    const float* hp = part + (int64_t)u * n_splits * stride + g * (kD + 2);
    float M = -INFINITY, L = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += CG) {
        const int nk = n_splits - s0 < CG ? n_splits - s0 : CG;
        const float* gp = hp + s0 * stride;
        const int sl = lane < nk ? lane : nk - 1;
        float ml = gp[sl * stride];
        float ll = gp[sl * stride + 1];
        float ov[CG];
#pragma unroll
        for (int k = 0; k < CG; ++k) ov[k] = gp[(k < nk ? k : nk - 1) * stride + 2 + d];
        if (lane >= nk) {
            ml = -INFINITY;
            ll = 0.0f;
        }
        const float Mg = fmaxf(M, wave_max_f(ml));
        const float r = (M == -INFINITY) ? 0.0f : __expf(M - Mg);
        const float f = (ml == -INFINITY) ? 0.0f : __expf(ml - Mg);
        L = fmaf(L, r, wave_sum_f(ll * f));
        // lanes k >= nk hold weight 0, and their ov[k] (a copy of split
        // s0 + nk - 1) is finite, so every term is taken unconditionally
        float a = acc * r;
#pragma unroll
        for (int k = 0; k < CG; ++k)
            a = fmaf(ov[k], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), k)), a);
        acc = a;
        M = Mg;
    }
    out[((int64_t)u * G + g) * kD + d] = acc / L;
}

template <typename T>
static hipError_t launch_attend_t(int G, const AttendArgs<T>& a, int units, int sp0, bool ring,
                                  hipStream_t st) {
    const dim3 grid(units, a.n_splits - sp0), blk(kAttThreads);
#define PK_ATT(GG)                                                                       \
    return ring ? launch(attend_kernel<T, GG, true>, grid, blk, 0, st, a, sp0)           \
                : launch(attend_kernel<T, GG, false>, grid, blk, 0, st, a, sp0)
    switch (G) {
        case 1: PK_ATT(1);
        case 2: PK_ATT(2);
        case 4: PK_ATT(4);
        case 8: PK_ATT(8);
        default: return hipErrorInvalidValue;
    }
#undef PK_ATT
}

int attend_split_keys() { return kSplit; }
int attend_max_splits() { return kMaxSplits; }

hipError_t launch_combine(const float* part, int units, int G, int n_splits, float* out,
                          hipStream_t st) {
    if (n_splits <= 24)
        return launch(combine_kernel<24>, dim3(units, G), dim3(kD), 0, st, part, G, n_splits, out);
    return launch(combine_kernel<32>, dim3(units, G), dim3(kD), 0, st, part, G, n_splits, out);
}

hipError_t launch_attend(bool bf16, int G, const void* K, const void* V, int64_t cap, int units,
                         const void* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                         const int32_t* sel, const int32_t* sel_n, int top_k, int n_splits,
                         int n_hot_splits, int sp0, float* part, const HotRing& ring,
                         hipStream_t st) {
    if (ring.span < 1 || sp0 < 0 || sp0 >= n_splits || n_splits > kMaxSplits)
        return hipErrorInvalidValue;
    const bool rg = ring.k != nullptr;
    if (bf16)
        return launch_attend_t<uint16_t>(
            G, attend_args<uint16_t>(K, V, cap, q, sink_end, r_end, n_tok, sel, sel_n, top_k,
                                     n_splits, n_hot_splits, part, ring),
            units, sp0, rg, st);
    return launch_attend_t<float>(G, attend_args<float>(K, V, cap, q, sink_end, r_end, n_tok, sel,
                                                        sel_n, top_k, n_splits, n_hot_splits,
                                                        part, ring),
                                  units, sp0, rg, st);
}

}  // namespace pk
