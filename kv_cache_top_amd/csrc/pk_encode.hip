// Per-key encode, per-query preparation and the decode append (gfx950).
//
// ParisKV page, "Drift-robust analytic centroids" (normalisation and shared
// SRHT rotation; sign-pattern centroids), "Coarse candidate generation"
// (nearest centroid per subspace; top-rho centroids per query subspace with
// rank weights), "Candidate reranking (RSQ-IP)" (sign + 3-bit magnitude code,
// calibration scale w computed when the key is stored).
#include "pk_device.hpp"
#include "pk_launch.hpp"

namespace pk {

// ---------------------------------------------------------------------------
// encode: one 16-lane group per key.  Reads the key row once (256 B bf16 /
// 512 B fp32) and writes 16 B of ids and a record (64 B of codes + 4 B of w
// per subspace).  Lane l holds rotated coordinates 8l..8l+7: one subspace of
// m = 8, the two subspaces 2l, 2l+1 of m = 4, or half of subspace l/2 of
// m = 16 (even lane: its coordinates 0..7).  Either way the lane's id byte is
// the sign bits of its 8 coordinates (bit r = [x_{8l+r} < 0]) and its nibble
// word their 8 codes; the magnitudes are coded against the squared norm of
// their own subspace, and each subspace gets one w.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double xor1_f64(double x) {
    const int2 v = *reinterpret_cast<int2*>(&x);
    const int2 o = make_int2(xor16<1>(v.x), xor16<1>(v.y));
    return *reinterpret_cast<const double*>(&o);
}

template <typename T, int M>
__global__ __launch_bounds__(kBlock) void encode_kernel(const T* __restrict__ K, int64_t cap,
                                                         int64_t p0, int64_t count, int64_t total,
                                                         uint8_t* __restrict__ ids,
                                                         uint8_t* __restrict__ rec, uint64_t sign_lo,
                                                         uint64_t sign_hi, CodeTables tab) {
    constexpr int kHalves = M == 4 ? 2 : 1;    // subspaces coded per lane
    constexpr int kCoords = M == 4 ? 4 : 8;    // of the lane's coordinates each
    __shared__ float s_lev[8];
    if (threadIdx.x < 8) s_lev[threadIdx.x] = tab.levels[threadIdx.x];
    lds_sync();

    const int l16 = threadIdx.x & 15;
    const uint32_t sbits = lane_sign_byte(sign_lo, sign_hi, l16);
    const int64_t ngroups = (int64_t)gridDim.x * (kBlock / 16);
    for (int64_t key = (int64_t)blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4); key < total;
         key += ngroups) {
        const int64_t u = key / count;
        const int64_t pos = p0 + (key - u * count);
        const int64_t row = u * cap + pos;
        float v[8];
        load8(K + row * kD + 8 * l16, v);
        apply_signs(v, sbits);
        fwht128_g16(v, l16);

        uint32_t id = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r) id |= (v[r] < 0.0f ? 1u : 0u) << r;

        float sq[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) sq[r] = __fmul_rn(v[r], v[r]);
        // squared norm of each subspace: the spec's pairwise tree
        float ss[kHalves];
        if constexpr (M == 8) {
            ss[0] = tree8(sq);
        } else if constexpr (M == 16) {
            // tree of coordinates 0..7 (even lane) plus tree of 8..15 (odd lane)
            const float own = tree8(sq), oth = xor16<1>(own);
            ss[0] = (l16 & 1) ? (oth + own) : (own + oth);
        } else {
            ss[0] = (sq[0] + sq[1]) + (sq[2] + sq[3]);
            ss[1] = (sq[4] + sq[5]) + (sq[6] + sq[7]);
        }
        uint32_t packed = 0;
        float w[kHalves];
#pragma unroll
        for (int h = 0; h < kHalves; ++h) {
            float bound[7];
#pragma unroll
            for (int l = 0; l < 7; ++l) bound[l] = __fmul_rn(tab.sq_thr[l], ss[h]);
            uint32_t part = 0;
            double s2 = 0.0, s1 = 0.0;
#pragma unroll
            for (int j = 0; j < kCoords; ++j) {
                const int r = h * kCoords + j;
                // mag = #{l : sq >= bound[l]}; the bounds ascend (squared
                // thresholds times ss >= 0, rounded monotonically), so three
                // levels of a binary search give the same count, ties and NaN
                // included
                const float x = sq[r];
                const bool c1 = x >= bound[3];
                const bool c2 = x >= (c1 ? bound[5] : bound[1]);
                const bool c3 = x >= (c1 ? (c2 ? bound[6] : bound[4]) : (c2 ? bound[2] : bound[0]));
                const uint32_t mag = (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (c3 ? 1u : 0u);
                part |= ((((id >> r) & 1u) << 3) | mag) << (4 * r);
                const double ax = fabs((double)v[r]);
                s2 += ax * ax;
                s1 += (double)s_lev[mag] * ax;
            }
            if constexpr (M == 16) {   // both halves of the subspace (same sums on both lanes)
                s2 += xor1_f64(s2);
                s1 += xor1_f64(s1);
            }
            // ss = 0: all codes of the subspace 0 and w = 0; otherwise
            // w = ||x_b|| / sqrt(d) / <v_b, x_b / ||x_b||> = ||x_b||^2 / (sqrt(d) <v_b, x_b>)
            w[h] = 0.0f;
            if (ss[h] != 0.0f) {
                packed |= part;
                w[h] = (float)(s2 / (11.313708498984761 * s1));
            }
        }
        ids[row * kSub + l16] = (uint8_t)id;
        uint8_t* r = rec + row * rec_bytes<M>();
        reinterpret_cast<uint32_t*>(r)[l16] = packed;
        if constexpr (M == 8)
            reinterpret_cast<float*>(r + 64)[l16] = w[0];
        else if constexpr (M == 4)
            reinterpret_cast<float2*>(r + 64)[l16] = make_float2(w[0], w[1]);
        else if ((l16 & 1) == 0)
            reinterpret_cast<float*>(r + 64)[l16 >> 1] = w[0];
    }
}

// ---------------------------------------------------------------------------
// query preparation: one block of G waves per (id byte b, unit).
//   y_g = H D q_g (spec arithmetic); wave g rotates query head g (the four
//   16-lane groups of the wave compute the same transform) and reads the 8
//   coordinates 8b..8b+7 from lane b, so they are wave-uniform.
//   m = 8 (subspace b): lane l scores the centroids c = l + 64 t, t < 4, as
//   the pairwise fp32 tree ((t0+t1)+(t2+t3)) + ((t4+t5)+(t6+t7)) of the
//   signed coordinates; top-rho by (score desc, c asc): rho rounds of a wave
//   maximum of the order keys, the lowest index among the lanes holding it by
//   ballot, and removal; vote table row L[b][c] = sum_g weight(rank of c in
//   head g's picks).
//   m = 4 (subspaces 2b, 2b+1): lanes 0..15 score the 16 centroids of 2b from
//   coordinates 0..3 with the tree (t0+t1)+(t2+t3), lanes 16..31 those of
//   2b+1 from coordinates 4..7; top-rho in each half the same way; the row the
//   scan reads for id byte b is L[2b][c & 15] + L[2b+1][c >> 4].
// Block (0, u) also writes Ysum = sum_g y_g (for the rerank) and may copy the
// step's new K/V token into the store.
// ---------------------------------------------------------------------------
struct VoteWeights {
    uint32_t w[kRhoMax];
};

// The 4 spec-tree scores ((t0+t1)+(t2+t3)) + ((t4+t5)+(t6+t7)) of the 8-bit
// sign patterns c = lane + 64 t (t < 4) against the wave-uniform y
// (t_j = -y_j where bit j of c is set).
__device__ __forceinline__ void pattern_scores(const float y[8], int lane, float s[4]) {
    const float t0 = (lane & 1) ? -y[0] : y[0], t1 = (lane & 2) ? -y[1] : y[1];
    const float t2 = (lane & 4) ? -y[2] : y[2], t3 = (lane & 8) ? -y[3] : y[3];
    const float t4 = (lane & 16) ? -y[4] : y[4], t5 = (lane & 32) ? -y[5] : y[5];
    const float lo = (t0 + t1) + (t2 + t3);
    const float p45 = t4 + t5;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float t6 = (t & 1) ? -y[6] : y[6], t7 = (t & 2) ? -y[7] : y[7];
        s[t] = lo + (p45 + (t6 + t7));
    }
}

// The rho largest of a wave's 256 values (4 per lane), with multiplicity,
// descending, wave-uniform; out[r] for r >= rho is 0.
__device__ __forceinline__ void top_values(const float s[4], int rho, int lane,
                                           float out[kRhoMax]) {
    uint32_t k[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) k[t] = f32_order_key(s[t]);   // > 0: 0 marks a removed value
#pragma unroll
    for (int r = 0; r < kRhoMax; ++r) {
        out[r] = 0.0f;
        if (r < rho) {
            const uint32_t m = wave_max(max(max(k[0], k[1]), max(k[2], k[3])));
            out[r] = order_key_f32(m);
            int tt = 0;
            uint64_t bal = 0;
#pragma unroll
            for (int t = 3; t >= 0; --t) {
                const uint64_t bt = __ballot(k[t] == m);
                if (bt != 0) {
                    tt = t;
                    bal = bt;
                }
            }
            if (lane == __ffsll((unsigned long long)bal) - 1) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (t == tt) k[t] = 0;
            }
        }
    }
}

// m = 16, subspace b (rotated coordinates 16b..16b+15) of query head g, one
// wave per head.  Centroid c = lo + 256 hi scores S = fl(A[lo] + B[hi]), with
// A and B the 8-coordinate trees of the two halves: that is the spec's
// 16-term tree.  fp32 addition is monotone in each operand, so with tau = the
// rho-th largest of the rho x rho sums of the rho largest A and B values (at
// least rho centroids score >= tau), every centroid scoring >= tau has
// fl(A[lo] + max B) >= tau and fl(max A + B[hi]) >= tau.  The top-rho by
// (score desc, c asc) are therefore found among the pairs of those lo and hi
// values (typically a few dozen pairs; exact score ties widen the set up to
// all 65536 pairs, still exact but slower).  The votes of the G heads' picks
// are merged per centroid and written into a 256-slot linear-probing hash
// table (vote << 16 | c, 0 = empty), which the scan probes.
__device__ void qprep16(const float v[8], int b, int g, int G, int lane, int rho,
                        const VoteWeights& wts, uint32_t* s_tab, uint8_t* out) {
    __shared__ float s_av[8][256], s_bv[8][256];
    __shared__ uint8_t s_ai[8][256], s_bi[8][256];
    __shared__ uint32_t s_pick[8][kRhoMax];
    float ya[8], yb[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        ya[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[r]), 2 * b));
        yb[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[r]), 2 * b + 1));
    }
    float A[4], Bs[4], av[kRhoMax], bv[kRhoMax];
    pattern_scores(ya, lane, A);
    pattern_scores(yb, lane, Bs);
    top_values(A, rho, lane, av);
    top_values(Bs, rho, lane, bv);

    // tau: lane 8x + z holds fl(av[x] + bv[z])
    const int x = lane >> 3, z = lane & 7;
    float ax = av[0], bz = bv[0];
#pragma unroll
    for (int r = 1; r < kRhoMax; ++r) {
        ax = (x == r) ? av[r] : ax;
        bz = (z == r) ? bv[r] : bz;
    }
    uint32_t kk = (x < rho && z < rho) ? f32_order_key(ax + bz) : 0u;
    uint32_t tau = 0;
    for (int r = 0; r < rho; ++r) {
        tau = wave_max(kk);
        const uint64_t bal = __ballot(kk == tau);
        if (lane == __ffsll((unsigned long long)bal) - 1) kk = 0u;
    }

    // the lo (I) and hi (J) values that can reach tau
    uint32_t nI = 0, nJ = 0;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bool inI = f32_order_key(A[t] + bv[0]) >= tau;
        const bool inJ = f32_order_key(av[0] + Bs[t]) >= tau;
        const uint64_t bi = __ballot(inI), bj = __ballot(inJ);
        if (inI) {
            const uint32_t at = nI + (uint32_t)__popcll(bi & below);
            s_av[g][at] = A[t];
            s_ai[g][at] = (uint8_t)(lane + 64 * t);
        }
        if (inJ) {
            const uint32_t at = nJ + (uint32_t)__popcll(bj & below);
            s_bv[g][at] = Bs[t];
            s_bi[g][at] = (uint8_t)(lane + 64 * t);
        }
        nI += (uint32_t)__popcll(bi);
        nJ += (uint32_t)__popcll(bj);
    }
    lds_sync();

    // rho rounds over the candidate pairs: each lane's best order key below the
    // previous pick, then the wave maximum (64-bit: score key, then 0xffff - c)
    const uint32_t P = nI * nJ;
    uint64_t last = ~0ull;
    for (int r = 0; r < rho; ++r) {
        uint64_t best = 0;
        for (uint32_t p = (uint32_t)lane; p < P; p += 64u) {
            const uint32_t ii = p / nJ, jj = p - ii * nJ;
            const uint32_t ks = f32_order_key(s_av[g][ii] + s_bv[g][jj]);
            const uint32_t c = (uint32_t)s_ai[g][ii] | ((uint32_t)s_bi[g][jj] << 8);
            const uint64_t key = ((uint64_t)ks << 32) | (0xffffu - c);
            if (ks >= tau && key < last && key > best) best = key;
        }
        const uint32_t hi = wave_max((uint32_t)(best >> 32));
        const uint32_t lo = wave_max((uint32_t)(best >> 32) == hi ? (uint32_t)best : 0u);
        last = ((uint64_t)hi << 32) | lo;
        if (lane == 0) s_pick[g][r] = 0xffffu - lo;
    }
    lds_sync();

    // wave 0: merge the G * rho picks per centroid, insert each once
    if (g == 0) {
        const int P2 = G * rho;
        uint32_t c = 0, w = 0;
        if (lane < P2) {
            const int gg = lane / rho, rr = lane - gg * rho;
            c = s_pick[gg][rr];
#pragma unroll
            for (int r = 0; r < kRhoMax; ++r) w = (rr == r) ? wts.w[r] : w;
        }
        uint32_t vote = 0;
        bool owner = lane < P2;
        for (int q = 0; q < P2; ++q) {
            const uint32_t cq = (uint32_t)__builtin_amdgcn_readlane((int)c, q);
            const uint32_t wq = (uint32_t)__builtin_amdgcn_readlane((int)w, q);
            if (lane < P2 && cq == c) {
                vote += wq;
                if (q < lane) owner = false;
            }
        }
        if (owner) {
            uint32_t slot = hash16(c);
            for (int k = 0; k < 256; ++k) {
                if (atomicCAS(&s_tab[slot], 0u, (vote << 16) | c) == 0u) break;
                slot = (slot + 1u) & 255u;
            }
        }
    }
    lds_sync();
    if (g == 0) reinterpret_cast<uint4*>(out)[lane] = reinterpret_cast<const uint4*>(s_tab)[lane];
}


constexpr int kQMaxBlock = 512;  // G <= 8 waves

template <typename T, int M>
__global__ __launch_bounds__(kQMaxBlock) void qprep_kernel(
    const T* __restrict__ q, int G, uint64_t sign_lo, uint64_t sign_hi, int rho, VoteWeights wts,
    const float* __restrict__ cents, uint8_t* __restrict__ lut, float* __restrict__ ysum,
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, uint8_t* __restrict__ K,
    uint8_t* __restrict__ V, int64_t row_bytes, int64_t cap, int64_t new_pos, uint4* __restrict__ rk,
    uint4* __restrict__ rv, int64_t ring_rows, int64_t ring_slot) {
    const int b = blockIdx.x, u = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, g = tid >> 6, l16 = lane & 15;
    __shared__ uint32_t s_row[256];
    __shared__ float s_y[8][kD];

    float v[8];
    load8(q + ((int64_t)u * G + g) * kD + 8 * l16, v);
    if (b == 0 && k_new != nullptr) {
        const int per_row = (int)(row_bytes / 16);
        if (tid < per_row) {
            const int64_t dst = ((u * cap + new_pos) * row_bytes) / 16 + tid;
            const uint4 kx = k_new[(int64_t)u * per_row + tid], vx = v_new[(int64_t)u * per_row + tid];
            reinterpret_cast<uint4*>(K)[dst] = kx;
            reinterpret_cast<uint4*>(V)[dst] = vx;
            if (rk != nullptr) {
                const int64_t rd = ((int64_t)u * ring_rows + ring_slot) * per_row + tid;
                rk[rd] = kx;
                rv[rd] = vx;
            }
        }
    }
    for (int i = tid; i < 256; i += 64 * G) s_row[i] = 0;
    apply_signs(v, lane_sign_byte(sign_lo, sign_hi, l16));
    fwht128_g16(v, l16);
    if (b == 0 && lane < 16) {
#pragma unroll
        for (int r = 0; r < 8; ++r) s_y[g][8 * l16 + r] = v[r];
    }

    if constexpr (M == 16) {
        lds_sync();   // s_row zeroed
        qprep16(v, b, g, G, lane, rho, wts, s_row, lut + ((int64_t)u * 8 + b) * 1024);
    } else {
        // subspace b of head g, wave-uniform
        float y[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) y[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[r]), b));
        uint32_t key[4];
        if constexpr (M == 4) {
            // lane l < 32 holds centroid l & 15 of subspace 2b + (l >> 4)
            const int h = (lane >> 4) & 1;
            const float a0 = h ? y[4] : y[0], a1 = h ? y[5] : y[1];
            const float a2 = h ? y[6] : y[2], a3 = h ? y[7] : y[3];
            const float t0 = (lane & 1) ? -a0 : a0, t1 = (lane & 2) ? -a1 : a1;
            const float t2 = (lane & 4) ? -a2 : a2, t3 = (lane & 8) ? -a3 : a3;
            key[0] = lane < 32 ? f32_order_key((t0 + t1) + (t2 + t3)) : 0u;
            key[1] = key[2] = key[3] = 0u;
        } else if (cents == nullptr) {
            float sc[4];
            pattern_scores(y, lane, sc);
#pragma unroll
            for (int t = 0; t < 4; ++t) key[t] = f32_order_key(sc[t]);  // > 0 for every finite score
        } else {
            // learned centroids (comparison stage): the fp32 tree of fl32(c_j y_j)
            const float4* ct = reinterpret_cast<const float4*>(cents + ((int64_t)u * kSub + b) * 256 * 8);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float4 c0 = ct[2 * (64 * t + lane)], c1 = ct[2 * (64 * t + lane) + 1];
                const float p[8] = {__fmul_rn(c0.x, y[0]), __fmul_rn(c0.y, y[1]), __fmul_rn(c0.z, y[2]),
                                    __fmul_rn(c0.w, y[3]), __fmul_rn(c1.x, y[4]), __fmul_rn(c1.y, y[5]),
                                    __fmul_rn(c1.z, y[6]), __fmul_rn(c1.w, y[7])};
                key[t] = f32_order_key(tree8(p));
            }
        }
        lds_sync();

        // the vote weights as wave-uniform values (an indexed argument read
        // inside the rounds is a scalar load and a wait per round)
        uint32_t wv[kRhoMax];
#pragma unroll
        for (int k = 0; k < kRhoMax; ++k) wv[k] = (uint32_t)__builtin_amdgcn_readfirstlane((int)wts.w[k]);
        auto weight = [&](int r) {
            uint32_t w = wv[0];
#pragma unroll
            for (int k = 1; k < kRhoMax; ++k) w = (r == k) ? wv[k] : w;
            return w;
        };
        if constexpr (M == 4) {
            // each half separately; s_row[16 h + c] = vote of centroid c of subspace 2b + h
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t kk = ((lane >> 4) == h) ? key[0] : 0u;
                for (int r = 0; r < rho; ++r) {
                    const uint32_t m = wave_max(kk);
                    const uint64_t bal = __ballot(kk == m);
                    const int c = __ffsll((unsigned long long)bal) - 1;   // lane 16 h + centroid
                    if (lane == c) kk = 0;  // removed
                    if (lane == 0) atomicAdd(&s_row[c], weight(r));
                }
            }
        } else {
            for (int r = 0; r < rho; ++r) {
                const uint32_t m = wave_max(max(max(key[0], key[1]), max(key[2], key[3])));
                int c = 256;
#pragma unroll
                for (int t = 3; t >= 0; --t) {
                    const uint64_t bal = __ballot(key[t] == m);
                    if (bal != 0) c = 64 * t + (__ffsll((unsigned long long)bal) - 1);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (c == 64 * t + lane) key[t] = 0;  // removed
                if (lane == 0) atomicAdd(&s_row[c], weight(r));
            }
        }
        lds_sync();
        if (tid < 64) {
            // vote of id-byte value c (at most 255: checked on the host)
            auto entry = [&](int c) -> uint32_t {
                if constexpr (M == 4) return s_row[c & 15] + s_row[16 + (c >> 4)];
                return s_row[c];
            };
            uint32_t* out = reinterpret_cast<uint32_t*>(lut + ((int64_t)u * kSub + b) * 256);
            out[tid] = (entry(4 * tid) & 0xffu) | ((entry(4 * tid + 1) & 0xffu) << 8) |
                       ((entry(4 * tid + 2) & 0xffu) << 16) | ((entry(4 * tid + 3) & 0xffu) << 24);
        }
    }
    if (b == 0) {
        for (int i = tid; i < kD; i += 64 * G) {
            float a = s_y[0][i];
            for (int h = 1; h < G; ++h) a += s_y[h][i];
            ysum[(int64_t)u * kD + i] = a;
        }
    }
}

// ---------------------------------------------------------------------------
// decode append: copy one token per unit into the store at position pos
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void append_kernel(const uint4* __restrict__ k_new,
                                                         const uint4* __restrict__ v_new,
                                                         uint8_t* __restrict__ K,
                                                         uint8_t* __restrict__ V, int64_t row_bytes,
                                                         int64_t cap, int64_t pos, int units,
                                                         uint4* __restrict__ rk,
                                                         uint4* __restrict__ rv, int64_t ring_rows,
                                                         int64_t ring_slot) {
    const int per_row = (int)(row_bytes / 16);
    const int64_t n = (int64_t)units * per_row;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t u = i / per_row, j = i - u * per_row;
        const int64_t dst = ((u * cap + pos) * row_bytes) / 16 + j;
        reinterpret_cast<uint4*>(K)[dst] = k_new[i];
        reinterpret_cast<uint4*>(V)[dst] = v_new[i];
        if (rk != nullptr) {
            const int64_t rd = (u * ring_rows + ring_slot) * per_row + j;
            rk[rd] = k_new[i];
            rv[rd] = v_new[i];
        }
    }
}

// ---------------------------------------------------------------------------
// ring fill (prefill of a host-memory store): the sink rows [0, sink_end) and
// the local rows [r_end, n) of every unit, read over the host link once
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void ring_fill_kernel(const uint4* __restrict__ K,
                                                            const uint4* __restrict__ V,
                                                            uint4* __restrict__ rk,
                                                            uint4* __restrict__ rv, int per_row,
                                                            int64_t cap, int units,
                                                            int64_t sink_end, int64_t r_end,
                                                            int64_t n, int64_t ring_rows,
                                                            int64_t n_sink, int64_t span) {
    const int64_t hot = sink_end + (n - r_end);
    const int64_t total = (int64_t)units * hot * per_row;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kBlock) {
        const int64_t j = i % per_row, t = i / per_row;
        const int64_t u = t / hot, h = t - u * hot;
        const int64_t p = h < sink_end ? h : r_end + (h - sink_end);
        const int64_t slot = p < sink_end ? p : n_sink + p % span;   // as ring_slot()
        const int64_t src = (u * cap + p) * per_row + j, dst = (u * ring_rows + slot) * per_row + j;
        rk[dst] = K[src];
        rv[dst] = V[src];
    }
}

// ---------------------------------------------------------------------------
// streaming read of a buffer (measurement reference), in the pattern that read
// fastest here for launches of tens of MB: block b reads the contiguous
// 32 KB [b * 2048, b * 2048 + 2048) of 16-byte pieces, eight nontemporal loads
// per thread all in flight (indices clamped to the last piece), folded into a
// checksum that is stored only if it matches an improbable value (so the loads
// are kept)
// ---------------------------------------------------------------------------
constexpr int kStreamPer = 8;   // pieces per thread

__global__ __launch_bounds__(kBlock) void stream_read_kernel(const uint4* __restrict__ src,
                                                              int64_t n, uint32_t* __restrict__ sink) {
    const int64_t start = (int64_t)blockIdx.x * (kStreamPer * kBlock) + threadIdx.x;
    uint4 v[kStreamPer];
#pragma unroll
    for (int j = 0; j < kStreamPer; ++j) {
        const int64_t i = start + j * kBlock;
        v[j] = load_nt(src + (i < n ? i : n - 1));
    }
    uint32_t acc = 0;
#pragma unroll
    for (int j = 0; j < kStreamPer; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// ---------------------------------------------------------------------------
// random gather of records (measurement reference): lane t reads the 16-byte
// piece t % per of record t / per, record i at row idx[i] (clamped to the
// array); four pieces per thread in flight, folded into a checksum stored only
// if it matches an improbable value
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void gather_read_kernel(const uint4* __restrict__ src,
                                                              int64_t n_rows, int per,
                                                              const int32_t* __restrict__ idx,
                                                              int64_t total,
                                                              uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t t0 = (int64_t)blockIdx.x * kBlock + threadIdx.x; t0 < total; t0 += 4 * stride) {
        int64_t off[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t t = t0 + k * stride < total ? t0 + k * stride : total - 1;
            const int64_t rec = t / per;
            int64_t row = idx[rec];
            row = row < 0 ? 0 : (row >= n_rows ? n_rows - 1 : row);
            off[k] = row * per + (t - rec * per);
        }
        uint4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = src[off[k]];
#pragma unroll
        for (int k = 0; k < 4; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_encode(bool bf16, const void* K, int64_t cap, int units, int64_t p0,
                         int64_t count, uint8_t* ids, uint8_t* rec, const uint64_t sign[2],
                         const CodeTables& tab, hipStream_t st) {
    const int64_t total = (int64_t)units * count;
    if (total <= 0) return hipSuccess;
    const int64_t groups_needed = total;
    int64_t blocks = (groups_needed + (kBlock / 16) - 1) / (kBlock / 16);
    if (blocks > 65536) blocks = 65536;
    const dim3 grid((unsigned)blocks), blk(kBlock);
#define PK_ENC(TY, MM)                                                                        \
    return launch(encode_kernel<TY, MM>, grid, blk, 0, st, (const TY*)K, cap, p0, count, total, \
                  ids, rec, sign[0], sign[1], tab)
    if (tab.sub_dim == 4) {
        if (bf16) PK_ENC(uint16_t, 4);
        PK_ENC(float, 4);
    }
    if (tab.sub_dim == 16) {
        if (bf16) PK_ENC(uint16_t, 16);
        PK_ENC(float, 16);
    }
    if (tab.sub_dim != 8) return hipErrorInvalidValue;
    if (bf16) PK_ENC(uint16_t, 8);
    PK_ENC(float, 8);
#undef PK_ENC
}

hipError_t launch_qprep(bool bf16, const void* q, int units, int G, const uint64_t sign[2],
                        int rho, const uint8_t* weights, const float* cents, uint8_t* lut, float* ysum, int sub_dim,
                        const void* k_new, const void* v_new, void* K, void* V, int64_t row_bytes,
                        int64_t cap, int64_t new_pos, int64_t slot, const HotRing& ring,
                        hipStream_t st) {
    VoteWeights w;
    for (int i = 0; i < kRhoMax; ++i) w.w[i] = (i < rho) ? weights[i] : 0u;
    const dim3 grid(sub_dim == 16 ? 8 : kSub, units), blk(64 * G);
    if (sub_dim != 8 && ((sub_dim != 4 && sub_dim != 16) || cents != nullptr))
        return hipErrorInvalidValue;
#define PK_QP(TY, MM)                                                                            \
    return launch(qprep_kernel<TY, MM>, grid, blk, 0, st, (const TY*)q, G, sign[0], sign[1], rho, \
                  w, cents, lut, ysum, (const uint4*)k_new, (const uint4*)v_new, (uint8_t*)K,      \
                  (uint8_t*)V, row_bytes, cap, new_pos, (uint4*)ring.k, (uint4*)ring.v, ring.rows, \
                  slot)
    if (sub_dim == 4) {
        if (bf16) PK_QP(uint16_t, 4);
        PK_QP(float, 4);
    }
    if (sub_dim == 16) {
        if (bf16) PK_QP(uint16_t, 16);
        PK_QP(float, 16);
    }
    if (bf16) PK_QP(uint16_t, 8);
    PK_QP(float, 8);
#undef PK_QP
}

hipError_t launch_append(const void* k_new, const void* v_new, void* K, void* V,
                         int64_t row_bytes, int64_t cap, int64_t pos, int64_t slot, int units,
                         const HotRing& ring, hipStream_t st) {
    const int64_t n = (int64_t)units * (row_bytes / 16);
    const int blocks = (int)((n + kBlock - 1) / kBlock);
    return launch(append_kernel, dim3(blocks), dim3(kBlock), 0, st, (const uint4*)k_new,
                  (const uint4*)v_new, (uint8_t*)K, (uint8_t*)V, row_bytes, cap, pos, units,
                  (uint4*)ring.k, (uint4*)ring.v, ring.rows, slot);
}

hipError_t launch_gather_read(const void* src, int64_t n_rows, int rec_bytes, const int32_t* idx,
                              int64_t count, uint32_t* sink, hipStream_t st) {
    const int per = rec_bytes / 16;
    const int64_t total = count * per;
    int64_t blocks = (total + 4 * kBlock - 1) / (4 * kBlock);
    if (blocks > 16384) blocks = 16384;
    return launch(gather_read_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                  (const uint4*)src, n_rows, per, idx, total, sink);
}

hipError_t launch_stream_read(const void* src, int64_t n16, uint32_t* sink, hipStream_t st) {
    const int64_t blocks = (n16 + kStreamPer * kBlock - 1) / (kStreamPer * kBlock);
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    return launch(stream_read_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st,
                  (const uint4*)src, n16, sink);
}

hipError_t launch_ring_fill(const void* K, const void* V, int64_t row_bytes, int64_t cap,
                            int units, int64_t sink_end, int64_t r_end, int64_t n,
                            const HotRing& ring, hipStream_t st) {
    if (ring.k == nullptr) return hipSuccess;
    const int per_row = (int)(row_bytes / 16);
    const int64_t total = (int64_t)units * (sink_end + (n - r_end)) * per_row;
    if (total <= 0) return hipSuccess;
    int64_t blocks = (total + kBlock - 1) / kBlock;
    if (blocks > 8192) blocks = 8192;
    return launch(ring_fill_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, st, (const uint4*)K,
                  (const uint4*)V, (uint4*)ring.k, (uint4*)ring.v, per_row, cap, units, sink_end,
                  r_end, n, ring.rows, ring.n_sink, ring.span);
}

}  // namespace pk
