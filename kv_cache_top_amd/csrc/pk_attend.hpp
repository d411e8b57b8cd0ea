// One split of the sparse GQA decode attention (gfx950), as a device
// function: the attention kernel runs one split per 256-thread block, and the
// fused fine-selection kernel runs hot-zone splits on blocks of 1024 threads
// next to its selection blocks.
//
// ParisKV page, "Problem definition": decoding attends only a top-k subset of
// past tokens; "Sliding-window update mechanism": sink, local and buffer
// tokens are always at hand; "UVA offloading": the retrieved rows may be read
// directly from host memory by the kernel.
//
// Split-K over the attended list of a unit: the hot tokens (sink, then the
// local window with the update buffer) in ceil(n_hot / kSplit) splits, then
// the selected positions in ceil(top_k / kSplit) splits; kSplit = 128 keys.
// A 16-lane group handles one key row at a time (8 coordinates per lane); the
// G query heads of the group share every K and V row read.  Each split writes
// its partial (max, sum, unnormalised output) per query head; a second kernel
// merges the splits of each unit.
#pragma once

#include <type_traits>

#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

constexpr int kSplit = 128;
constexpr int kMaxSplits = 65535;   // splits per unit (the dense pass takes n / kSplit; a grid dimension)
constexpr int kAttThreads = 256;   // threads of one split
static_assert(kSplit % 64 == 0, "softmax statistics take 64 keys per wave pass");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct AttendArgs {
    const T* K;                 // [units][cap][d] stores
    const T* V;
    int64_t cap;
    const T* q;                 // [units][G][d]
    int64_t sink_end, r_end, n_tok;
    const int32_t* sel;         // [units][top_k]
    const int32_t* sel_n;       // [units]
    int top_k;
    int n_splits, n_hot_splits; // splits per unit; the first n_hot_splits cover the hot tokens
    float* part;                // [units][n_splits][G][2 + d]
    const T* rk;                // device ring of the hot rows (host-memory stores), else null
    const T* rv;
    int64_t ring_rows, ring_sink, ring_span, ring_base;
};

// kernel arguments of the splits of one attention pass
template <typename T>
inline AttendArgs<T> attend_args(const void* K, const void* V, int64_t cap, const void* q,
                          int64_t sink_end, int64_t r_end, int64_t n_tok, const int32_t* sel,
                          const int32_t* sel_n, int top_k, int n_splits, int n_hot_splits,
                          float* part, const HotRing& ring) {
    AttendArgs<T> a;
    a.K = (const T*)K;
    a.V = (const T*)V;
    a.cap = cap;
    a.q = (const T*)q;
    a.sink_end = sink_end;
    a.r_end = r_end;
    a.n_tok = n_tok;
    a.sel = sel;
    a.sel_n = sel_n;
    a.top_k = top_k;
    a.n_splits = n_splits;
    a.n_hot_splits = n_hot_splits;
    a.part = part;
    a.rk = (const T*)ring.k;
    a.rv = (const T*)ring.v;
    a.ring_rows = ring.rows;
    a.ring_sink = ring.n_sink;
    a.ring_span = ring.span;
    a.ring_base = r_end % ring.span;
    return a;
}
template <int G>
struct alignas(16) AttendLds {
    float p[G][kSplit];
    float red[kAttThreads / 64][G][kD];
    float m[G], l[G];
};

// Split sp of unit u, computed by the 256 threads t = 0..255 of a group of four
// waves.  It holds kSplitBarriers block-wide barriers: in a block of several
// groups every group calls it, or attend_split_idle, which passes the same
// barriers and does nothing else.  An inactive group runs the same steps on
// masked keys and writes nothing.
constexpr int kSplitBarriers = 3;
__device__ __forceinline__ void attend_split_idle() {
#pragma unroll
    for (int i = 0; i < kSplitBarriers; ++i) lds_sync();
}

template <typename T, int G, bool RING>
__device__ __forceinline__ void attend_split(const AttendArgs<T>& a, int u, int sp, int t,
                                             bool active, AttendLds<G>& L) {
    const int lane = t & 63, wave = t >> 6, grp = lane >> 4, l16 = lane & 15;
    constexpr bool kMfma = sizeof(T) == 2;   // bf16: q k^T on the matrix cores
    constexpr int kPer = kSplit / (kAttThreads / 16);   // keys per 16-lane group
    static_assert(kSplit == 32 * (kAttThreads / 64), "a wave owns 32 keys of the split");
    static_assert(!kMfma || G <= 8, "query heads fill MFMA rows 0..G-1 of 16");
    constexpr float kInvSqrtD = 0.08838834764831845f;
    const T* __restrict__ K = a.K;
    const T* __restrict__ V = a.V;
    const T* __restrict__ q = a.q;
    const T* __restrict__ rk = a.rk;
    const T* __restrict__ rv = a.rv;
    const int64_t cap = a.cap, sink_end = a.sink_end, r_end = a.r_end, n_tok = a.n_tok;
    const int64_t ring_rows = a.ring_rows, ring_sink = a.ring_sink, ring_span = a.ring_span,
                  ring_base = a.ring_base;
    const int top_k = a.top_k;

    // Wave w owns keys [32w, 32w + 32) of the split.  Values: the wave reads
    // each of its 32 rows whole, lane l taking coordinates 2l and 2l + 1.
    // Keys (bf16): MFMA tiles of 16 keys, lane l16 loading key 32w + 16h + l16;
    // (fp32): the 16-lane group grp handles keys 32w + grp + 4j (j < 8), 8
    // coordinates per lane.
    // Hot splits read neither sel nor sel_n (the fused kernel computes them
    // at the same time).
    // The count and the positions are loaded without a branch (a branch per
    // load lets the compiler wait for each before issuing the next): a hot
    // split points its loads at the query instead and discards the values.
    const int64_t n_hot = sink_end + (n_tok - r_end);
    const bool hot_split = sp < a.n_hot_splits;
    const int32_t* sel_row = hot_split ? reinterpret_cast<const int32_t*>(q)
                                       : a.sel + (int64_t)u * top_k;
    const int32_t* sel_cnt = hot_split ? reinterpret_cast<const int32_t*>(q) : a.sel_n + u;
    const int64_t i0 = hot_split ? (int64_t)sp * kSplit
                                 : n_hot + (int64_t)(sp - a.n_hot_splits) * kSplit;
    auto sel_at = [&](int kk) -> int32_t {
        const int64_t i = i0 + kk - n_hot;
        const int32_t c = sel_row[hot_split ? 0 : (i < 0 ? 0 : (i < top_k ? (int)i : top_k - 1))];
        return hot_split ? 0 : c;
    };
    constexpr int kPerK = kMfma ? 1 : kPer;
    int32_t cand_v[kPerK], cand_k[2];
    const int kl = lane & 31;
    const int32_t cand_r = sel_at(32 * wave + kl);
    if constexpr (kMfma) {
#pragma unroll
        for (int h = 0; h < 2; ++h) cand_k[h] = sel_at(32 * wave + 16 * h + l16);
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) cand_v[j] = sel_at(32 * wave + grp + 4 * j);
    }
    int nsel = *sel_cnt;
    // query operand.  bf16: A rows = heads, lane l holds head l16's dims 32s +
    // 8 grp .. +8 of step s; rows >= G load head G - 1 (no branch around the
    // loads), and their products are never stored.  fp32: this lane's 8 dims
    // of every head.
    uint4 qa[4];
    Raw8<T> qv[kMfma ? 1 : G];
    if constexpr (kMfma) {
        const int qh = l16 < G ? l16 : G - 1;
#pragma unroll
        for (int st = 0; st < 4; ++st)
            qa[st] = *reinterpret_cast<const uint4*>(q + ((int64_t)u * G + qh) * kD + 32 * st + 8 * grp);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g].load(q + ((int64_t)u * G + g) * kD + 8 * l16);
    }
    nsel = nsel < 0 ? 0 : (nsel > top_k ? top_k : nsel);
    const int64_t end = hot_split ? n_hot : n_hot + nsel;
    const int nk = active ? (int)((end - i0) < kSplit ? (end - i0 > 0 ? end - i0 : 0) : kSplit) : 0;

    // position of attended key kk (out of range, or stale, for a masked key).
    // Positions and list indices stay below 2^26 (capacity <= 2^24), so this
    // is 32-bit selects, not a branch the position load could sink into.
    const int n_hot32 = (int)n_hot, sink32 = (int)sink_end, i032 = (int)i0;
    const int hot_off = (int)r_end - sink32;   // list index -> position past the sink
    auto pos_of = [&](int kk, int32_t c) -> int64_t {
        const int i = i032 + kk;
        const int ph = i < sink32 ? i : i + hot_off;
        return (int64_t)(i < n_hot32 ? ph : c);
    };
    // key kk is attended: inside the split's count and a valid position
    auto attended = [&](int kk, int32_t c) -> bool {
        const int64_t p = pos_of(kk, c);
        return kk < nk && p >= 0 && p < n_tok;
    };
    // row of attended key kk: from the device ring for the hot zone when the
    // store is host memory, else from the store.  With a device store the row
    // depends only on the position's range (a masked key reads a valid row
    // and its score is masked later), so the row requests need not wait for
    // the split's count; with a host store a masked key reads a ring row, so
    // nothing crosses the host link for it.
    auto place = [&](int kk, int32_t c, bool& hot) -> int64_t {
        const int64_t i = i0 + kk;
        const int64_t p = pos_of(kk, c);
        if constexpr (!RING) {
            hot = false;
            return (int64_t)u * cap + ((p >= 0 && p < n_tok) ? p : 0);
        }
        if (!attended(kk, c)) {
            hot = true;
            return (int64_t)u * ring_rows;
        }
        hot = i < n_hot;
        if (hot) {
            if (i < sink_end) return (int64_t)u * ring_rows + i;
            int64_t s = ring_base + (i - sink_end);
            s = s >= ring_span ? s - ring_span : s;
            return (int64_t)u * ring_rows + ring_sink + s;
        }
        return (int64_t)u * cap + p;
    };
    bool hot_v[kPerK], hot_k[2], hot_r;
    int64_t row_v[kPerK], row_k[2];
    const int64_t row_r = place(32 * wave + kl, cand_r, hot_r);
    if constexpr (kMfma) {
#pragma unroll
        for (int h = 0; h < 2; ++h) row_k[h] = place(32 * wave + 16 * h + l16, cand_k[h], hot_k[h]);
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) row_v[j] = place(32 * wave + grp + 4 * j, cand_v[j], hot_v[j]);
    }
    // every K and V row is requested before any is used
    uint4 kb[2][4];
    Raw8<T> kv[kPerK];
    if constexpr (kMfma) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const T* kr = (RING && hot_k[h] ? rk : K) + row_k[h] * kD + 8 * grp;
#pragma unroll
            for (int st = 0; st < 4; ++st)
                kb[h][st] = load_nt(reinterpret_cast<const uint4*>(kr + 32 * st));
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            kv[j].load_stream((RING && hot_v[j] ? rk : K) + row_v[j] * kD + 8 * l16);
    }
    // value rows: key 32w + k is placed by lane k; its row address is uniform
    // across the wave
    typedef uint32_t VPairBf16;                                   // two bf16
    typedef float VPairF32 __attribute__((ext_vector_type(2)));   // two fp32
    using VPair = std::conditional_t<kMfma, VPairBf16, VPairF32>;
    VPair vw[32];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)row_r, k);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(row_r >> 32), k);
        const int64_t r = (int64_t)(((uint64_t)hi << 32) | lo);
        const bool hk = RING && __builtin_amdgcn_readlane((int)hot_r, k) != 0;
        const VPair* vr = reinterpret_cast<const VPair*>((hk ? rv : V) + r * kD);
        vw[k] = __builtin_nontemporal_load(vr + lane);
    }
    // keep the scheduler from hoisting the first q k^T products (which wait
    // for the first key rows) above the value-row requests
    __builtin_amdgcn_sched_barrier(0);

    // scores / sqrt(d) into L.p[head][key]
    if constexpr (kMfma) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x4_t c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, qa[st]),
                                                            __builtin_bit_cast(bf16x8_t, kb[h][st]),
                                                            c, 0, 0, 0);
            // lane holds rows (heads) 4 grp + i of column (key) l16
            const int kk = 32 * wave + 16 * h + l16;
            const bool ok = attended(kk, cand_k[h]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int g = 4 * grp + i;
                if (g < G) L.p[g][kk] = ok ? c[i] * kInvSqrtD : -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int kk = 32 * wave + grp + 4 * j;
            const bool ok = attended(kk, cand_v[j]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.0f;
#pragma unroll
                for (int r = 0; r < 8; ++r) d = fmaf(qv[g][r], kv[j][r], d);
                d = sum16(d) * kInvSqrtD;
                if (l16 == 0) L.p[g][kk] = ok ? d : -INFINITY;
            }
        }
    }
    lds_sync();
    // softmax statistics of the split, one wave per head (strided)
    constexpr int kSlots = kSplit / 64;   // scores per lane
    for (int g = wave; g < G; g += kAttThreads / 64) {
        float sv[kSlots];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int kk = lane + 64 * k;
            sv[k] = (kk < nk) ? L.p[g][kk] : -INFINITY;
            mx = fmaxf(mx, sv[k]);
        }
        const float m = wave_max_f(mx);
        float es = 0.0f;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int kk = lane + 64 * k;
            const float e = (kk < nk && m != -INFINITY) ? __expf(sv[k] - m) : 0.0f;
            L.p[g][kk] = e;                    // 0 for the masked keys
            es += e;
        }
        const float l = wave_sum_f(es);
        if (lane == 0) {
            L.m[g] = m;
            L.l[g] = l;
        }
    }
    lds_sync();
    // weighted values: lane l accumulates coordinates 2l, 2l + 1 over the
    // wave's 32 keys, reading the weights of four keys at a time
    float acc[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g][0] = acc[g][1] = 0.0f;
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4) {
        float4 pg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pg[g] = *reinterpret_cast<const float4*>(&L.p[g][32 * wave + 4 * k4]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float v0, v1;
            if constexpr (kMfma) {
                const uint32_t x = vw[4 * k4 + kk];
                v0 = __uint_as_float(x << 16);
                v1 = __uint_as_float(x & 0xffff0000u);
            } else {
                v0 = vw[4 * k4 + kk].x;
                v1 = vw[4 * k4 + kk].y;
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = kk == 0 ? pg[g].x : (kk == 1 ? pg[g].y : (kk == 2 ? pg[g].z : pg[g].w));
                acc[g][0] = fmaf(p, v0, acc[g][0]);
                acc[g][1] = fmaf(p, v1, acc[g][1]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
        *reinterpret_cast<float2*>(&L.red[wave][g][2 * lane]) = make_float2(acc[g][0], acc[g][1]);
    lds_sync();
    // partial record per (unit, split, head): [m, l, o[128]]
    if (!active) return;
    float* myp = a.part + ((int64_t)u * a.n_splits + sp) * G * (kD + 2);
    for (int i = t; i < G * kD; i += kAttThreads) {
        const int g = i / kD, d = i - g * kD;
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kAttThreads / 64; ++w) o += L.red[w][g][d];
        myp[g * (kD + 2) + 2 + d] = o;
    }
    if (t < G) {
        myp[t * (kD + 2)] = L.m[t];
        myp[t * (kD + 2) + 1] = L.l[t];
    }
}

}  // namespace pk
