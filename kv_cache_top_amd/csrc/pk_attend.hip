// Sparse GQA decode attention over sink + local + update buffer + retrieved
// keys (gfx950).
//
// ParisKV page, "Problem definition": decoding attends only a top-k subset of
// past tokens; "Sliding-window update mechanism": sink, local and buffer
// tokens are always at hand; "UVA offloading": the retrieved rows may be read
// directly from host memory by the kernel.
//
// Split-K: the attended list of a unit (hot tokens first, then the selected
// positions) is cut into splits of kSplit keys, one 256-thread block each.
// A 16-lane group handles one key row at a time (8 coordinates per lane);
// the G query heads of the group share every K and V row read.  Each block
// writes its partial (max, sum, unnormalised output) per query head; a second
// kernel merges the splits of each unit.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

constexpr int kSplit = 64;
constexpr int kMaxSplits = 1024;

template <typename T, int G>
__global__ __launch_bounds__(kBlock) void attend_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int64_t cap, const T* __restrict__ q,
    int64_t sink_end, int64_t r_end, int64_t n_tok, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_n, int top_k, int n_splits, float* __restrict__ part) {
    const int u = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, l16 = lane & 15;
    __shared__ float s_p[G][kSplit];
    __shared__ float s_red[kBlock / 64][G][kD];
    __shared__ float s_m[G], s_l[G];

    // the key slots of this 16-lane group: kk = wave*4 + grp + 16*j, j < kPer.
    // Selected positions are read together with their count (entries past the
    // count are masked afterwards).
    constexpr int kPer = kSplit / (kBlock / 16);
    const int64_t n_hot = sink_end + (n_tok - r_end);
    const int64_t i0 = (int64_t)sp * kSplit;
    int32_t cand[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = i0 + wave * 4 + grp + j * (kBlock / 16) - n_hot;
        cand[j] = sel[(int64_t)u * top_k + (i < 0 ? 0 : (i < top_k ? i : top_k - 1))];
    }
    int nsel = sel_n[u];

    // this lane's 8 coordinates of every query head of the group, pre-scaled by 1/sqrt(d)
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        load8(q + ((int64_t)u * G + g) * kD + 8 * l16, qv[g]);
#pragma unroll
        for (int r = 0; r < 8; ++r) qv[g][r] *= 0.08838834764831845f;
    }

    nsel = nsel < 0 ? 0 : (nsel > top_k ? top_k : nsel);
    const int64_t total = n_hot + nsel;
    const int nk = (int)((total - i0) < kSplit ? (total - i0 > 0 ? total - i0 : 0) : kSplit);
    int64_t pos[kPer];
    bool ok[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int kk = wave * 4 + grp + j * (kBlock / 16);
        const int64_t i = i0 + kk;
        const int64_t p = (i < n_hot) ? ((i < sink_end) ? i : r_end + (i - sink_end)) : (int64_t)cand[j];
        ok[j] = kk < nk && p >= 0 && p < n_tok;
        pos[j] = ok[j] ? p : 0;
    }
    // every K and V row of the group is requested before any is used
    float kv[kPer][8], vv[kPer][8];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        load8(K + ((int64_t)u * cap + pos[j]) * kD + 8 * l16, kv[j]);
        load8(V + ((int64_t)u * cap + pos[j]) * kD + 8 * l16, vv[j]);
    }
    // scores
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int kk = wave * 4 + grp + j * (kBlock / 16);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) d = fmaf(qv[g][r], kv[j][r], d);
            d = sum16(d);
            if (l16 == 0 && kk < nk) s_p[g][kk] = ok[j] ? d : -INFINITY;
        }
    }
    lds_sync();
    // softmax statistics of the split, one wave per head (strided)
    for (int g = wave; g < G; g += kBlock / 64) {
        const float a = (lane < nk) ? s_p[g][lane] : -INFINITY;
        float m = a;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        const float e = (lane < nk && m != -INFINITY) ? __expf(a - m) : 0.0f;
        float l = e;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
        if (lane < nk) s_p[g][lane] = e;
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
        const int kk = wave * 4 + grp + j * (kBlock / 16);
        if (kk < nk) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pg = s_p[g][kk];
#pragma unroll
                for (int r = 0; r < 8; ++r) acc[g][r] = fmaf(pg, vv[j][r], acc[g][r]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            float a = acc[g][r];
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            acc[g][r] = a;
        }
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

// merge of the split partials: one 1024-thread block per unit.  All (m, l)
// pairs are read at once; wave g folds head g's; each thread then sums one
// output over the splits with the loads of 32 splits in flight.
constexpr int kCBlock = 1024;

__global__ __launch_bounds__(kCBlock) void combine_kernel(const float* __restrict__ part, int G,
                                                           int n_splits, float* __restrict__ out) {
    const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ float s_m[8][kMaxSplits];
    __shared__ float s_f[8][kMaxSplits];
    const float* up = part + (int64_t)u * n_splits * G * (kD + 2);
    for (int i = tid; i < G * n_splits; i += kCBlock) {
        const int s = i / G, g = i - s * G;
        s_m[g][s] = up[(s * G + g) * (kD + 2)];
        s_f[g][s] = up[(s * G + g) * (kD + 2) + 1];
    }
    lds_sync();
    for (int g = wave; g < G; g += kCBlock / 64) {
        float M = -INFINITY;
        for (int s = lane; s < n_splits; s += 64) M = fmaxf(M, s_m[g][s]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
        float L = 0.0f;
        for (int s = lane; s < n_splits; s += 64) {
            const float ms = s_m[g][s];
            const float f = (ms == -INFINITY) ? 0.0f : __expf(ms - M);
            s_m[g][s] = f;                 // reuse: weight before normalisation
            L = fmaf(s_f[g][s], f, L);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
        const float invL = 1.0f / L;
        for (int s = lane; s < n_splits; s += 64) s_f[g][s] = s_m[g][s] * invL;
    }
    lds_sync();
    constexpr int kUnroll = 32;
    for (int i = tid; i < G * kD; i += kCBlock) {
        const int g = i / kD, d = i - g * kD;
        float o = 0.0f;
        for (int s0 = 0; s0 < n_splits; s0 += kUnroll) {
            float v[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const int s = s0 + k < n_splits ? s0 + k : n_splits - 1;
                v[k] = up[(s * G + g) * (kD + 2) + 2 + d];
            }
#pragma unroll
            for (int k = 0; k < kUnroll; ++k)
                if (s0 + k < n_splits) o = fmaf(v[k], s_f[g][s0 + k], o);
        }
        out[((int64_t)u * G + g) * kD + d] = o;
    }
}

template <typename T>
static hipError_t launch_attend_t(int G, const T* K, const T* V, int64_t cap, int units,
                                  const T* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                                  const int32_t* sel, const int32_t* sel_n, int top_k,
                                  int n_splits, float* part, hipStream_t st) {
    const dim3 grid(n_splits, units), blk(kBlock);
#define PK_ATT(GG)                                                                              \
    attend_kernel<T, GG><<<grid, blk, 0, st>>>(K, V, cap, q, sink_end, r_end, n_tok, sel, sel_n, \
                                               top_k, n_splits, part)
    switch (G) {
        case 1: PK_ATT(1); break;
        case 2: PK_ATT(2); break;
        case 4: PK_ATT(4); break;
        case 8: PK_ATT(8); break;
        default: return hipErrorInvalidValue;
    }
#undef PK_ATT
    return hipGetLastError();
}

int attend_split() { return kSplit; }

hipError_t launch_combine(const float* part, int units, int G, int n_splits, float* out,
                          hipStream_t st) {
    combine_kernel<<<dim3(units), dim3(kCBlock), 0, st>>>(part, G, n_splits, out);
    return hipGetLastError();
}
int attend_max_splits() { return kMaxSplits; }

hipError_t launch_attend(bool bf16, int G, const void* K, const void* V, int64_t cap, int units,
                         const void* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                         const int32_t* sel, const int32_t* sel_n, int top_k, int n_splits,
                         float* part, hipStream_t st) {
    if (bf16)
        return launch_attend_t<uint16_t>(G, (const uint16_t*)K, (const uint16_t*)V, cap, units,
                                         (const uint16_t*)q, sink_end, r_end, n_tok, sel, sel_n,
                                         top_k, n_splits, part, st);
    return launch_attend_t<float>(G, (const float*)K, (const float*)V, cap, units, (const float*)q,
                                  sink_end, r_end, n_tok, sel, sel_n, top_k, n_splits, part, st);
}

}  // namespace pk
