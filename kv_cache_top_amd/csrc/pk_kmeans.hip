// Comparison coarse stage with learned centroids (gfx950): per unit and
// subspace, 256 centroids fitted by k-means to the keys stored at prefill, in
// place of the analytic sign-pattern centroids.
//
// ParisKV page, "Problem definition" and "Drift-robust analytic centroids":
// centroids fitted to the prefill keys are the design the page argues
// against, since their buckets stop matching keys whose distribution drifts
// during decoding.  The page does not define the fitting; the one used here:
//  * similarity of centroid c and rotated subspace vector x_b: the fp32
//    pairwise tree of fl32(c_j x_j) (the same tree as every other score of
//    the path); bucket = most similar centroid, ties to the lower index;
//  * initial centroids: the normalised subspace vectors of 256 given keys;
//  * Lloyd iterations: assign, then c = S / ||S|| with S the exact integer sum
//    of the assigned vectors in fixed point (coordinates rounded to multiples
//    of 2^-20, added with 64-bit integer atomics, so the result does not depend
//    on the order of the additions), norm and quotient in float64, rounded to
//    fp32; a centroid with a zero sum keeps its value.
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

constexpr int kCent = 256;
constexpr int kKmThreads = 1024;                // 64 keys per pass, 16 lanes per key
constexpr int kTabStride = kCent * 8 + 4;       // floats per subspace table in LDS (+16 B:
                                                // the 16 subspaces of a wave hit distinct banks)
constexpr double kFix = 1048576.0;              // 2^20

__device__ __forceinline__ long long fixed_point(float x) {
    return (long long)rint((double)x * kFix);
}

// rotated subspace l16 of key `row` (16 lanes per key)
template <typename T>
__device__ __forceinline__ void rotated_subspace(const T* K, int64_t row, int l16, uint32_t sbits,
                                                 float v[8]) {
    load8(K + row * kD + 8 * l16, v);
    apply_signs(v, sbits);
    fwht128_g16(v, l16);
}

// S[u][b][i] = fixed point of subspace b of key init_pos[u][i]: one 16-lane
// group per (unit, i), 16 groups per block
template <typename T>
__global__ __launch_bounds__(kBlock) void km_seed_kernel(const T* __restrict__ K, int64_t cap,
                                                          const int32_t* __restrict__ init_pos,
                                                          int units, uint64_t sign_lo,
                                                          uint64_t sign_hi,
                                                          long long* __restrict__ S) {
    const int l16 = threadIdx.x & 15;
    const int g = blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4);
    if (g >= units * kCent) return;                       // whole 16-lane groups
    const int u = g / kCent, i = g - u * kCent;
    float v[8];
    rotated_subspace(K, (int64_t)u * cap + init_pos[g], l16, lane_sign_byte(sign_lo, sign_hi, l16), v);
    long long* s = S + (((int64_t)u * kSub + l16) * kCent + i) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = fixed_point(v[j]);
}

// centroid = S / ||S|| (float64, rounded to fp32) where S != 0; S cleared for
// the next accumulation.  One thread per (unit, subspace, centroid).
__global__ __launch_bounds__(kBlock) void km_normalise_kernel(long long* __restrict__ S,
                                                               float* __restrict__ cents,
                                                               int64_t n) {
    const int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (t >= n) return;
    long long* s = S + t * 8;
    double d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = (double)s[j];
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = ss + d[j] * d[j];   // coordinate order, no contraction
    if (ss > 0.0) {
        const double nrm = sqrt(ss);
        float* c = cents + t * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (float)(d[j] / nrm);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = 0;
}

// Most similar centroid of every subspace of keys [p0, p0 + count) of unit
// blockIdx.y.  ACC: add the key's fixed-point subspace vector to its
// centroid's sum; else: store the bucket ids.  The unit's 16 tables (128 KB)
// sit in LDS; lane l16 of a group scans table l16 for its key.
template <typename T, bool ACC>
__global__ __launch_bounds__(kKmThreads) void km_assign_kernel(
    const T* __restrict__ K, int64_t cap, int64_t p0, int64_t count, uint64_t sign_lo,
    uint64_t sign_hi, const float* __restrict__ cents, long long* __restrict__ S,
    uint8_t* __restrict__ ids) {
    __shared__ __align__(16) float s_tab[kSub * kTabStride];
    const int u = blockIdx.y, tid = threadIdx.x, l16 = tid & 15;
    const float* ct = cents + (int64_t)u * kSub * kCent * 8;
    for (int i = tid; i < kSub * kCent * 2; i += kKmThreads) {   // float4 units
        const int b = i / (kCent * 2), r = i - b * (kCent * 2);
        *reinterpret_cast<float4*>(&s_tab[b * kTabStride + 4 * r]) =
            reinterpret_cast<const float4*>(ct)[i];
    }
    lds_sync();
    const uint32_t sbits = lane_sign_byte(sign_lo, sign_hi, l16);
    const float* tab = s_tab + l16 * kTabStride;
    const int64_t step = (int64_t)gridDim.x * (kKmThreads / 16);
    for (int64_t k = (int64_t)blockIdx.x * (kKmThreads / 16) + (tid >> 4); k < count; k += step) {
        const int64_t row = (int64_t)u * cap + p0 + k;
        float v[8];
        rotated_subspace(K, row, l16, sbits, v);
        float best = -INFINITY;
        int arg = 0;
        for (int c = 0; c < kCent; ++c) {
            const float4 c0 = *reinterpret_cast<const float4*>(tab + 8 * c);
            const float4 c1 = *reinterpret_cast<const float4*>(tab + 8 * c + 4);
            const float t[8] = {__fmul_rn(c0.x, v[0]), __fmul_rn(c0.y, v[1]),
                                __fmul_rn(c0.z, v[2]), __fmul_rn(c0.w, v[3]),
                                __fmul_rn(c1.x, v[4]), __fmul_rn(c1.y, v[5]),
                                __fmul_rn(c1.z, v[6]), __fmul_rn(c1.w, v[7])};
            const float s = tree8(t);
            if (s > best) {                      // strict: the lower index keeps a tie
                best = s;
                arg = c;
            }
        }
        if constexpr (ACC) {
            long long* s = S + (((int64_t)u * kSub + l16) * kCent + arg) * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                atomicAdd(reinterpret_cast<unsigned long long*>(s + j),
                          (unsigned long long)fixed_point(v[j]));
        } else {
            ids[row * kSub + l16] = (uint8_t)arg;
        }
    }
}

namespace {
template <typename T>
hipError_t km_fit_t(const void* Kv, int64_t cap, int units, int64_t n_fit, const int32_t* init_pos,
                    int iters, const uint64_t sign[2], float* cents, long long* S, hipStream_t st) {
    const T* K = (const T*)Kv;
    const int64_t nc = (int64_t)units * kSub * kCent;
    const int seed_blocks = (units * kCent + kBlock / 16 - 1) / (kBlock / 16);
    const int norm_blocks = (int)((nc + kBlock - 1) / kBlock);
    hipError_t e = launch(km_seed_kernel<T>, dim3(seed_blocks), dim3(kBlock), 0, st, K, cap,
                          init_pos, units, sign[0], sign[1], S);
    if (e != hipSuccess) return e;
    e = launch(km_normalise_kernel, dim3(norm_blocks), dim3(kBlock), 0, st, S, cents, nc);
    if (e != hipSuccess) return e;
    const int64_t per = (n_fit + kKmThreads / 16 - 1) / (kKmThreads / 16);
    const dim3 grid((unsigned)(per < 64 ? per : 64), units);
    for (int it = 0; it < iters && e == hipSuccess; ++it) {
        e = launch(km_assign_kernel<T, true>, grid, dim3(kKmThreads), 0, st, K, cap, (int64_t)0,
                   n_fit, sign[0], sign[1], (const float*)cents, S, (uint8_t*)nullptr);
        if (e == hipSuccess)
            e = launch(km_normalise_kernel, dim3(norm_blocks), dim3(kBlock), 0, st, S, cents, nc);
    }
    return e;
}
}  // namespace

hipError_t launch_km_fit(bool bf16, const void* K, int64_t cap, int units, int64_t n_fit,
                         const int32_t* init_pos, int iters, const uint64_t sign[2], float* cents,
                         long long* S, hipStream_t st) {
    if (n_fit < 1 || units < 1 || iters < 0) return hipErrorInvalidValue;
    return bf16 ? km_fit_t<uint16_t>(K, cap, units, n_fit, init_pos, iters, sign, cents, S, st)
                : km_fit_t<float>(K, cap, units, n_fit, init_pos, iters, sign, cents, S, st);
}

hipError_t launch_km_ids(bool bf16, const void* K, int64_t cap, int units, int64_t p0,
                         int64_t count, const uint64_t sign[2], const float* cents, uint8_t* ids,
                         hipStream_t st) {
    if (count <= 0) return hipSuccess;
    const int64_t per = (count + kKmThreads / 16 - 1) / (kKmThreads / 16);
    const dim3 grid((unsigned)(per < 64 ? per : 64), units), blk(kKmThreads);
    if (bf16)
        return launch(km_assign_kernel<uint16_t, false>, grid, blk, 0, st, (const uint16_t*)K, cap,
                      p0, count, sign[0], sign[1], cents, (long long*)nullptr, ids);
    return launch(km_assign_kernel<float, false>, grid, blk, 0, st, (const float*)K, cap, p0, count,
                  sign[0], sign[1], cents, (long long*)nullptr, ids);
}

}  // namespace pk
