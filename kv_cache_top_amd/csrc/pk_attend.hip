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
// writes its partial (max, sum, unnormalised output) per query head; the
// unit's last block merges them.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

constexpr int kSplit = 64;

template <typename T, int G>
__global__ __launch_bounds__(kBlock) void attend_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int64_t cap, const T* __restrict__ q,
    int64_t sink_end, int64_t r_end, int64_t n_tok, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_n, int top_k, int n_splits, float* __restrict__ part,
    uint32_t* __restrict__ tickets, float* __restrict__ out) {
    const int u = blockIdx.y, sp = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, l16 = lane & 15;
    __shared__ float s_p[G][kSplit];
    __shared__ float s_red[kBlock / 64][G][kD];
    __shared__ float s_m[G], s_l[G];
    __shared__ int s_last;

    const int64_t n_hot = sink_end + (n_tok - r_end);
    int nsel = sel_n[u];
    nsel = nsel < 0 ? 0 : (nsel > top_k ? top_k : nsel);
    const int64_t total = n_hot + nsel;
    const int64_t i0 = (int64_t)sp * kSplit;
    const int nk = (int)((total - i0) < kSplit ? (total - i0 > 0 ? total - i0 : 0) : kSplit);

    // this lane's 8 coordinates of every query head of the group, pre-scaled by 1/sqrt(d)
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        load8(q + ((int64_t)u * G + g) * kD + 8 * l16, qv[g]);
#pragma unroll
        for (int r = 0; r < 8; ++r) qv[g][r] *= 0.08838834764831845f;
    }

    auto position = [&](int kk, bool* ok) -> int64_t {
        const int64_t i = i0 + kk;
        int64_t p;
        if (i < n_hot) {
            p = (i < sink_end) ? i : r_end + (i - sink_end);
        } else {
            p = sel[(int64_t)u * top_k + (i - n_hot)];
        }
        *ok = (p >= 0 && p < n_tok);
        return *ok ? p : 0;
    };

    // scores
    for (int kk = wave * 4 + grp; kk < nk; kk += kBlock / 16) {
        bool ok;
        const int64_t p = position(kk, &ok);
        float kv[8];
        load8(K + ((int64_t)u * cap + p) * kD + 8 * l16, kv);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) d = fmaf(qv[g][r], kv[r], d);
            d = sum16(d);
            if (l16 == 0) s_p[g][kk] = ok ? d : -INFINITY;
        }
    }
    __syncthreads();
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
    __syncthreads();
    // weighted values
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < 8; ++r) acc[g][r] = 0.0f;
    for (int kk = wave * 4 + grp; kk < nk; kk += kBlock / 16) {
        bool ok;
        const int64_t p = position(kk, &ok);
        float vv[8];
        load8(V + ((int64_t)u * cap + p) * kD + 8 * l16, vv);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float pg = s_p[g][kk];
#pragma unroll
            for (int r = 0; r < 8; ++r) acc[g][r] = fmaf(pg, vv[r], acc[g][r]);
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
    __syncthreads();
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

    // ---- ticket: the unit's last block merges the splits
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&tickets[u], 1u) == (uint32_t)(n_splits - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const float* up = part + (int64_t)u * n_splits * G * (kD + 2);
    for (int i = tid; i < G * kD; i += kBlock) {
        const int g = i / kD, d = i - g * kD;
        float M = -INFINITY;
        for (int s = 0; s < n_splits; ++s) M = fmaxf(M, up[(s * G + g) * (kD + 2)]);
        float L = 0.0f, O = 0.0f;
        for (int s = 0; s < n_splits; ++s) {
            const float* rp = up + (s * G + g) * (kD + 2);
            const float m = rp[0];
            if (m == -INFINITY) continue;
            const float f = __expf(m - M);
            L = fmaf(rp[1], f, L);
            O = fmaf(rp[2 + d], f, O);
        }
        out[((int64_t)u * G + g) * kD + d] = O / L;
    }
    if (tid == 0) tickets[u] = 0;
}

template <typename T>
static hipError_t launch_attend_t(int G, const T* K, const T* V, int64_t cap, int units,
                                  const T* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                                  const int32_t* sel, const int32_t* sel_n, int top_k,
                                  int n_splits, float* part, uint32_t* tickets, float* out,
                                  hipStream_t st) {
    const dim3 grid(n_splits, units), blk(kBlock);
#define PK_ATT(GG)                                                                              \
    attend_kernel<T, GG><<<grid, blk, 0, st>>>(K, V, cap, q, sink_end, r_end, n_tok, sel, sel_n, \
                                               top_k, n_splits, part, tickets, out)
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

hipError_t launch_attend(bool bf16, int G, const void* K, const void* V, int64_t cap, int units,
                         const void* q, int64_t sink_end, int64_t r_end, int64_t n_tok,
                         const int32_t* sel, const int32_t* sel_n, int top_k, int n_splits,
                         float* part, uint32_t* tickets, float* out, hipStream_t st) {
    if (bf16)
        return launch_attend_t<uint16_t>(G, (const uint16_t*)K, (const uint16_t*)V, cap, units,
                                         (const uint16_t*)q, sink_end, r_end, n_tok, sel, sel_n,
                                         top_k, n_splits, part, tickets, out, st);
    return launch_attend_t<float>(G, (const float*)K, (const float*)V, cap, units, (const float*)q,
                                  sink_end, r_end, n_tok, sel, sel_n, top_k, n_splits, part,
                                  tickets, out, st);
}

}  // namespace pk
