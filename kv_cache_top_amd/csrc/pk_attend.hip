// Sparse GQA decode attention over sink + local + update buffer + retrieved
// keys (gfx950).
//
// ParisKV page, "Problem definition": decoding attends only a top-k subset of
// past tokens; "Sliding-window update mechanism": sink, local and buffer
// tokens are always at hand; "UVA offloading": the retrieved rows may be read
// directly from host memory by the kernel.
//
// Split-K: the attended list of a unit (hot tokens first, then the selected
// positions) is cut into splits of kSplit = 128 keys, one 256-thread block each.
// A 16-lane group handles one key row at a time (8 coordinates per lane);
// the G query heads of the group share every K and V row read.  Each block
// writes its partial (max, sum, unnormalised output) per query head; a second
// kernel merges the splits of each unit.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

constexpr int kSplit = 128;
constexpr int kMaxSplits = 1024;
static_assert(kSplit % 64 == 0, "softmax statistics take 64 keys per wave pass");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T, int G, bool RING>
__global__ __launch_bounds__(kBlock) void attend_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int64_t cap, const T* __restrict__ q,
    int64_t sink_end, int64_t r_end, int64_t n_tok, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_n, int top_k, int n_splits, float* __restrict__ part,
    const T* __restrict__ rk, const T* __restrict__ rv, int64_t ring_rows, int64_t ring_sink,
    int64_t ring_span, int64_t ring_base) {
    const int u = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, l16 = lane & 15;
    constexpr bool kMfma = sizeof(T) == 2;   // bf16: q k^T on the matrix cores
    constexpr int kPer = kSplit / (kBlock / 16);   // keys per 16-lane group
    static_assert(kSplit == 32 * (kBlock / 64), "a wave owns 32 keys of the split");
    static_assert(!kMfma || G <= 8, "query heads fill MFMA rows 0..G-1 of 16");
    __shared__ float s_p[G][kSplit];
    __shared__ float s_red[kBlock / 64][G][kD];
    __shared__ float s_m[G], s_l[G];
    constexpr float kInvSqrtD = 0.08838834764831845f;

    // Wave w owns keys [32w, 32w + 32) of the split.  Values: the 16-lane
    // group grp handles keys 32w + grp + 4j (j < 8), 8 coordinates per lane.
    // Keys (bf16): MFMA tiles of 16 keys, lane l16 loading key 32w + 16h + l16.
    const int64_t n_hot = sink_end + (n_tok - r_end);
    const int64_t i0 = (int64_t)sp * kSplit;
    auto sel_at = [&](int kk) -> int32_t {
        const int64_t i = i0 + kk - n_hot;
        return sel[(int64_t)u * top_k + (i < 0 ? 0 : (i < top_k ? i : top_k - 1))];
    };
    int32_t cand_v[kPer], cand_k[2];
#pragma unroll
    for (int j = 0; j < kPer; ++j) cand_v[j] = sel_at(32 * wave + grp + 4 * j);
    if constexpr (kMfma) {
#pragma unroll
        for (int h = 0; h < 2; ++h) cand_k[h] = sel_at(32 * wave + 16 * h + l16);
    }
    int nsel = sel_n[u];

    // query operand.  bf16: A rows = heads (rows >= G zero), lane l holds head
    // l16's dims 32s + 8 grp .. +8 of step s.  fp32: this lane's 8 dims of every head.
    uint4 qa[4];
    Raw8<T> qv[kMfma ? 1 : G];
    if constexpr (kMfma) {
#pragma unroll
        for (int st = 0; st < 4; ++st)
            qa[st] = (l16 < G) ? *reinterpret_cast<const uint4*>(
                                     q + ((int64_t)u * G + l16) * kD + 32 * st + 8 * grp)
                               : make_uint4(0u, 0u, 0u, 0u);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g].load(q + ((int64_t)u * G + g) * kD + 8 * l16);
    }

    nsel = nsel < 0 ? 0 : (nsel > top_k ? top_k : nsel);
    const int64_t total = n_hot + nsel;
    const int nk = (int)((total - i0) < kSplit ? (total - i0 > 0 ? total - i0 : 0) : kSplit);
    // row of attended key kk: from the device ring for the hot zone when the
    // store is host memory, else from the store
    auto place = [&](int kk, int32_t c, bool& ok, bool& hot) -> int64_t {
        const int64_t i = i0 + kk;
        const int64_t p = (i < n_hot) ? ((i < sink_end) ? i : r_end + (i - sink_end)) : (int64_t)c;
        ok = kk < nk && p >= 0 && p < n_tok;
        if constexpr (!RING) {
            hot = false;
            return (int64_t)u * cap + (ok ? p : 0);
        }
        if (!ok) {                          // masked: any valid row, on the device
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
    bool ok_v[kPer], ok_k[2], hot_v[kPer], hot_k[2];
    int64_t row_v[kPer], row_k[2];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        row_v[j] = place(32 * wave + grp + 4 * j, cand_v[j], ok_v[j], hot_v[j]);
    if constexpr (kMfma) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            row_k[h] = place(32 * wave + 16 * h + l16, cand_k[h], ok_k[h], hot_k[h]);
    }
    // every K and V row is requested before any is used
    uint4 kb[2][4];
    Raw8<T> kv[kMfma ? 1 : kPer], vv[kPer];
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
#pragma unroll
    for (int j = 0; j < kPer; ++j)
        vv[j].load_stream((RING && hot_v[j] ? rv : V) + row_v[j] * kD + 8 * l16);

    // scores / sqrt(d) into s_p[head][key]
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
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int g = 4 * grp + i;
                if (g < G) s_p[g][kk] = ok_k[h] ? c[i] * kInvSqrtD : -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int kk = 32 * wave + grp + 4 * j;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.0f;
#pragma unroll
                for (int r = 0; r < 8; ++r) d = fmaf(qv[g][r], kv[j][r], d);
                d = sum16(d) * kInvSqrtD;
                if (l16 == 0) s_p[g][kk] = ok_v[j] ? d : -INFINITY;
            }
        }
    }
    lds_sync();
    // softmax statistics of the split, one wave per head (strided)
    constexpr int kSlots = kSplit / 64;   // scores per lane
    for (int g = wave; g < G; g += kBlock / 64) {
        float a[kSlots];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int kk = lane + 64 * k;
            a[k] = (kk < nk) ? s_p[g][kk] : -INFINITY;
            mx = fmaxf(mx, a[k]);
        }
        const float m = wave_max_f(mx);
        float es = 0.0f;
#pragma unroll
        for (int k = 0; k < kSlots; ++k) {
            const int kk = lane + 64 * k;
            const float e = (kk < nk && m != -INFINITY) ? __expf(a[k] - m) : 0.0f;
            if (kk < nk) s_p[g][kk] = e;
            es += e;
        }
        const float l = wave_sum_f(es);
        if (lane == 0) {
            s_m[g] = m;
            s_l[g] = l;
        }
    }
    lds_sync();
    // weighted values
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[g][r] = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int kk = 32 * wave + grp + 4 * j;
        if (kk < nk) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pg = s_p[g][kk];
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[g][r] = fmaf(pg, vv[j][r], acc[g][r]);
            }
        }
    }
    // sum over the four 16-lane groups of the wave (lane exchanges across rows)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[g][r] = sum_rows4(acc[g][r]);
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < 8; ++r) s_red[wave][g][8 * l16 + r] = acc[g][r];
    }
    lds_sync();
    // partial record per (unit, split, head): [m, l, o[128]]
    float* myp = part + ((int64_t)u * n_splits + sp) * G * (kD + 2);
    for (int i = tid; i < G * kD; i += kBlock) {
        const int g = i / kD, d = i - g * kD;
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kBlock / 64; ++w) o += s_red[w][g][d];
        myp[g * (kD + 2) + 2 + d] = o;
    }
    if (tid < G) {
        myp[tid * (kD + 2)] = s_m[tid];
        myp[tid * (kD + 2) + 1] = s_l[tid];
    }
}

// merge of the split partials: one 128-thread block per (query head, unit),
// thread d owning output coordinate d.  Splits are folded in groups of 64,
// everything of a group requested before any is used: lane k of each wave
// reads (m, l) of split s0 + k, the group maximum M' rescales the running
// sums, lane k's weight e^(m - M') is broadcast to the wave, and
// acc += o_s e^(m_s - M'), L += l_s e^(m_s - M').  out = acc / L.
constexpr int kCGroup = 32;

__global__ __launch_bounds__(kD) void combine_kernel(const float* __restrict__ part, int G,
                                                     int n_splits, float* __restrict__ out) {
    const int g = blockIdx.x, u = blockIdx.y, d = threadIdx.x, lane = d & 63;
    const int64_t stride = (int64_t)G * (kD + 2);      // between splits
    const float* hp = part + (int64_t)u * n_splits * stride + (int64_t)g * (kD + 2);
    float M = -INFINITY, L = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < n_splits; s0 += kCGroup) {
        const int nk = n_splits - s0 < kCGroup ? n_splits - s0 : kCGroup;
        const int sl = s0 + (lane < nk ? lane : nk - 1);
        float ml = hp[sl * stride];
        float ll = hp[sl * stride + 1];
        float ov[kCGroup];
#pragma unroll
        for (int k = 0; k < kCGroup; ++k) {
            const int s = s0 + (k < nk ? k : nk - 1);
            ov[k] = hp[s * stride + 2 + d];
        }
        if (lane >= nk) {
            ml = -INFINITY;
            ll = 0.0f;
        }
        const float Mg = fmaxf(M, wave_max_f(ml));
        if (Mg == -INFINITY) continue;                  // nothing attended yet
        const float r = (M == -INFINITY) ? 0.0f : __expf(M - Mg);
        const float f = (ml == -INFINITY) ? 0.0f : __expf(ml - Mg);
        L = fmaf(L, r, wave_sum_f(ll * f));
        float a = acc * r;
#pragma unroll
        for (int k = 0; k < kCGroup; ++k) {
            if (k < nk) a = fmaf(ov[k], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), k)), a);
        }
        acc = a;
        M = Mg;
    }
    out[((int64_t)u * G + g) * kD + d] = acc / L;
}

template <typename T>
static hipError_t launch_attend_t(int G, const T* K, const T* V, int64_t cap, int units,
                                  const T* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                                  const int32_t* sel, const int32_t* sel_n, int top_k,
                                  int n_splits, float* part, const HotRing& ring,
                                  hipStream_t st) {
    const dim3 grid(n_splits, units), blk(kBlock);
    const int64_t base = r_end % ring.span;
#define PK_ATT(GG)                                                                            \
    return ring.k != nullptr                                                                  \
               ? launch(attend_kernel<T, GG, true>, grid, blk, 0, st, K, V, cap, q, sink_end,  \
                        r_end, n_tok, sel, sel_n, top_k, n_splits, part, (const T*)ring.k,     \
                        (const T*)ring.v, ring.rows, ring.n_sink, ring.span, base)             \
               : launch(attend_kernel<T, GG, false>, grid, blk, 0, st, K, V, cap, q, sink_end, \
                        r_end, n_tok, sel, sel_n, top_k, n_splits, part, (const T*)nullptr,    \
                        (const T*)nullptr, ring.rows, ring.n_sink, ring.span, base)
    switch (G) {
        case 1: PK_ATT(1);
        case 2: PK_ATT(2);
        case 4: PK_ATT(4);
        case 8: PK_ATT(8);
        default: return hipErrorInvalidValue;
    }
#undef PK_ATT
}

int attend_split() { return kSplit; }

hipError_t launch_combine(const float* part, int units, int G, int n_splits, float* out,
                          hipStream_t st) {
    return launch(combine_kernel, dim3(G, units), dim3(kD), 0, st, part, G, n_splits, out);
}
int attend_max_splits() { return kMaxSplits; }

hipError_t launch_attend(bool bf16, int G, const void* K, const void* V, int64_t cap, int units,
                         const void* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                         const int32_t* sel, const int32_t* sel_n, int top_k, int n_splits,
                         float* part, const HotRing& ring, hipStream_t st) {
    if (ring.span < 1) return hipErrorInvalidValue;
    if (bf16)
        return launch_attend_t<uint16_t>(G, (const uint16_t*)K, (const uint16_t*)V, cap, units,
                                         (const uint16_t*)q, sink_end, r_end, n_tok, sel, sel_n,
                                         top_k, n_splits, part, ring, st);
    return launch_attend_t<float>(G, (const float*)K, (const float*)V, cap, units, (const float*)q,
                                  sink_end, r_end, n_tok, sel, sel_n, top_k, n_splits, part, ring,
                                  st);
}

}  // namespace pk
