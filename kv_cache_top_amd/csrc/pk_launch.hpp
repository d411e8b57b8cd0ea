// Kernel launchers (host side), one per kernel family.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace pk {

// Kernel timing attached to the dispatch itself: when `start` is set, the next
// launch() records start/stop with the kernel's own begin and end
// (hipExtLaunchKernel) and clears them.  Host-thread local.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming& launch_timing();

template <typename Tuple, size_t... I>
inline void arg_addresses(Tuple& t, void** out, std::index_sequence<I...>) {
    ((out[I] = static_cast<void*>(&std::get<I>(t))), ...);
}

// kernel<<<grid, block, shm, st>>>(args...), or the timed form of it.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shm,
                         hipStream_t st, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    LaunchTiming& t = launch_timing();
    if (t.start != nullptr) {
        std::tuple<KArgs...> tup{static_cast<KArgs>(args)...};
        void* addr[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
        arg_addresses(tup, addr, std::index_sequence_for<KArgs...>{});
        const hipEvent_t a = t.start, b = t.stop;
        t.start = t.stop = nullptr;
        return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, addr, shm, st,
                                  a, b, 0);
    }
    kernel<<<grid, block, shm, st>>>(static_cast<KArgs>(args)...);
    return hipGetLastError();
}

struct CodeTables;

// Device copy of the always-attended rows (sink, local, update buffer) kept
// when the caller's K/V store is host memory: attention then reads only the
// retrieved rows over the host link.  Row of position p: p for sink tokens,
// n_sink + (p mod span) for the local/buffer zone (span = n_local + U rows).
struct HotRing {
    void* k = nullptr;        // [units][rows][d], nullptr: no ring (device store)
    void* v = nullptr;
    int64_t rows = 0;         // n_sink + span
    int64_t n_sink = 0;
    int64_t span = 1;
};
// Ring row of position p given the window's sink end: the sink rows hold
// positions [0, sink_end); every later position (local window, update buffer)
// cycles through the span rows after the n_sink reserved ones.  A prefill
// shorter than n_sink leaves sink_end < n_sink, and the tokens appended after
// it are local tokens, read by the attention from the span rows.
inline int64_t ring_slot(const HotRing& r, int64_t sink_end, int64_t p) {
    return p < sink_end ? p : r.n_sink + p % r.span;
}


hipError_t launch_encode(bool bf16, const void* K, int64_t cap, int units, int64_t p0,
                         int64_t count, uint8_t* ids, uint8_t* rec, const uint64_t sign[2],
                         const CodeTables& tab, hipStream_t st);
// query rotation, vote tables and summed query (plus the step's append)
hipError_t launch_qprep(bool bf16, const void* q, int units, int G, const uint64_t sign[2],
                        int rho, const uint8_t* weights, const float* cents, uint8_t* lut,
                        float* ysum, int sub_dim,
                        const void* k_new, const void* v_new, void* K, void* V, int64_t row_bytes,
                        int64_t cap, int64_t new_pos, int64_t ring_slot, const HotRing& ring,
                        hipStream_t st);
// learned-centroid comparison stage: fit (seed, then iters rounds of assign +
// normalise) and bucket ids of keys [p0, p0 + count) under the fitted tables
hipError_t launch_km_fit(bool bf16, const void* K, int64_t cap, int units, int64_t n_fit,
                         const int32_t* init_pos, int iters, const uint64_t sign[2], float* cents,
                         long long* S, hipStream_t st);
hipError_t launch_km_ids(bool bf16, const void* K, int64_t cap, int units, int64_t p0,
                         int64_t count, const uint64_t sign[2], const float* cents, uint8_t* ids,
                         hipStream_t st);
hipError_t launch_append(const void* k_new, const void* v_new, void* K, void* V,
                         int64_t row_bytes, int64_t cap, int64_t pos, int64_t ring_slot, int units,
                         const HotRing& ring, hipStream_t st);
hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, hipStream_t st);
hipError_t launch_gather_read(const void* src, int64_t n_rows, int rec_bytes, const int32_t* idx,
                              int64_t count, uint32_t* sink, hipStream_t st);
// copy rows [0, sink_end) and [r_end, n) of every unit from the store into the ring
hipError_t launch_ring_fill(const void* K, const void* V, int64_t row_bytes, int64_t cap,
                            int units, int64_t sink_end, int64_t r_end, int64_t n,
                            const HotRing& ring, hipStream_t st);
// coarse scores, per-chunk suffix counts, and the unit histogram added into
// tot[units][(nbins + 1) & ~1] (zero beforehand)
hipError_t launch_scan(const uint8_t* ids, int64_t cap, int units, int64_t sink_end, int64_t n_r,
                       int chunk, int n_chunks, int max_chunks, const uint8_t* lut,
                       uint8_t* scores, int64_t sstride, uint16_t* hist, int hstride,
                       uint32_t* tot, int nbins, int sub_dim, hipStream_t st);
// coarse threshold and candidates (meta = {T, ties taken, C, k_eff} per unit),
// then the RSQ-IP estimates of the candidates; ids and lut rescore the keys
// whose stored score saturated when the threshold reaches 255
hipError_t launch_rerank(int chunk, const uint8_t* scores, int64_t sstride, const uint8_t* rec,
                         const uint8_t* ids, const uint8_t* lut,
                         int64_t cap, int units, int64_t sink_end, int64_t n_r, int n_chunks,
                         int max_chunks, const uint16_t* hist, int hstride, const uint32_t* tot,
                         int nbins, int64_t C, int top_k, const float* ysum,
                         const CodeTables& tab, int32_t* cand_pos, float* cand_est, int64_t cmax,
                         int32_t* meta, hipStream_t st);
// fine top-k; also zeroes the units' coarse-score histogram rows tot[units][tstride]
// (null: none) for the next step's scan
hipError_t launch_fine(const int32_t* cand_pos, const float* cand_est, int64_t cmax, int units,
                       int C, int top_k, int32_t* sel, int32_t* sel_n, uint32_t* tot, int tstride,
                       hipStream_t st);
hipError_t launch_empty_select(int units, int32_t* sel_n, int32_t* meta, hipStream_t st);
// hipSuccess when the current device can run this library's code object
hipError_t probe_kernel_image();
int attend_split_keys();   // keys per attention split
int attend_max_splits();
// split-K attention (partials per split) over splits sp0 .. n_splits-1; the
// first n_hot_splits splits cover the hot tokens, the rest the selection
hipError_t launch_attend(bool bf16, int G, const void* K, const void* V, int64_t cap, int units,
                         const void* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                         const int32_t* sel, const int32_t* sel_n, int top_k, int n_splits,
                         int n_hot_splits, int sp0, float* part, const HotRing& ring,
                         hipStream_t st);
// fine selection plus the hot-zone attention splits in one launch (bf16
// device stores, G <= 4, C <= 16384 register-held candidates)
bool fine_hot_supported(bool bf16, int G, bool ring, int C, int64_t cmax);
hipError_t launch_fine_hot(const int32_t* cand_pos, const float* cand_est, int64_t cmax,
                           int units, int C, int top_k, int32_t* sel, int32_t* sel_n, int G,
                           const void* K, const void* V, int64_t cap, const void* q,
                           int64_t sink_end, int64_t r_end, int64_t n_tok, int n_splits,
                           int n_hot_splits, float* part, uint32_t* tot, int tstride,
                           hipStream_t st);
hipError_t launch_combine(const float* part, int units, int G, int n_splits, float* out,
                          hipStream_t st);

}  // namespace pk
