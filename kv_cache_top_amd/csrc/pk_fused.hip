// Fine top-k selection fused with the hot-zone attention splits (gfx950).
//
// The selection is one 1024-thread block per unit: a chain of short,
// latency-bound steps that leaves most CUs and the memory idle.  The attention
// splits over the hot tokens (sink, local window, update buffer) need only the
// query and the stores, not the selection, so they run as extra blocks of the
// same launch, one split per 1024-thread block on its first four waves (the
// other twelve only pass the split's barriers): the splits' row requests are
// then spread over as many CUs as there are splits, which is what a gather of
// this size needs.  The attention launch that follows covers the retrieved
// splits only.
// Used for bf16 stores in device memory with G <= 4 (the split's registers fit
// the 128-register budget of a 1024-thread block).
#include "pk_attend.hpp"
#include "pk_fine.hpp"
#include "pk_launch.hpp"

namespace pk {

template <int SEG, int G>
__global__ __launch_bounds__(kFBlock) void fine_hot_kernel(const int32_t* __restrict__ cand_pos,
                                                           const float* __restrict__ cand_est,
                                                           int64_t cmax, int C, int top_k,
                                                           int32_t* __restrict__ sel,
                                                           int32_t* __restrict__ sel_n, int units,
                                                           uint32_t* __restrict__ tot, int tstride,
                                                           AttendArgs<uint16_t> a) {
    constexpr size_t kFineBytes = sizeof(FineShared);
    constexpr size_t kAttBytes = sizeof(AttendLds<G>);
    __shared__ __align__(16) unsigned char s_raw[kFineBytes > kAttBytes ? kFineBytes : kAttBytes];
    if ((int)blockIdx.x < units) {
        fine_reg_body<SEG>(cand_pos, cand_est, cmax, C, top_k, sel, sel_n, blockIdx.x,
                           *reinterpret_cast<FineShared*>(s_raw), tot, tstride);
        return;
    }
    // hot split gs = split * units + unit (units fastest: a unit's blocks share an XCD)
    if (threadIdx.x >= kAttThreads) {
        attend_split_idle();
        return;
    }
    const int gs = (int)blockIdx.x - units;
    attend_split<uint16_t, G, false>(a, gs % units, gs / units, threadIdx.x,
                                     true, *reinterpret_cast<AttendLds<G>*>(s_raw));
}

bool fine_hot_supported(bool bf16, int G, bool ring, int C, int64_t cmax) {
    return bf16 && !ring && (G == 1 || G == 2 || G == 4) && C >= 1 && C <= kFineReg &&
           C <= cmax && cmax % 16 == 0;
}

hipError_t launch_fine_hot(const int32_t* cand_pos, const float* cand_est, int64_t cmax,
                           int units, int C, int top_k, int32_t* sel, int32_t* sel_n, int G,
                           const void* K, const void* V, int64_t cap, const void* q,
                           int64_t sink_end, int64_t r_end, int64_t n_tok, int n_splits,
                           int n_hot_splits, float* part, uint32_t* tot, int tstride,
                           hipStream_t st) {
    if (!fine_hot_supported(true, G, false, C, cmax) || n_hot_splits < 1 ||
        n_hot_splits > n_splits || n_splits > kMaxSplits)
        return hipErrorInvalidValue;
    const AttendArgs<uint16_t> a =
        attend_args<uint16_t>(K, V, cap, q, sink_end, r_end, n_tok, sel, sel_n, top_k, n_splits,
                              n_hot_splits, part, HotRing{});
    const dim3 grid(units + units * n_hot_splits), blk(kFBlock);
    const int seg = C <= 4 * kFBlock ? 4 : (C <= 8 * kFBlock ? 8 : 16);
#define PK_FH(S, GG)                                                                          \
    return launch(fine_hot_kernel<S, GG>, grid, blk, 0, st, cand_pos, cand_est, cmax, C, top_k, \
                  sel, sel_n, units, tot, tstride, a)
#define PK_FH_G(S)                      \
    switch (G) {                        \
        case 1: PK_FH(S, 1);            \
        case 2: PK_FH(S, 2);            \
        default: PK_FH(S, 4);           \
    }
    if (seg == 4) PK_FH_G(4);
    if (seg == 8) PK_FH_G(8);
    PK_FH_G(16);
#undef PK_FH_G
#undef PK_FH
}

}  // namespace pk
