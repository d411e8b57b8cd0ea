// Magnitude codebook of the 4-bit RSQ-IP code (host only).
//
// ParisKV page, "Candidate reranking (RSQ-IP) > Quantization": each coordinate
// of a rotated, normalised subspace direction gets a sign bit and a 3-bit
// magnitude whose codebook follows from the Beta prior the rotation induces.
//
// For u uniform on the unit sphere of R^m, a = |u_j| has density
// proportional to (1 - a^2)^((m-3)/2) on [0, 1] (u_j^2 ~ Beta(1/2, (m-1)/2)).
// The codebook is the Lloyd-Max quantiser of a: levels are the conditional
// means of their bins, thresholds the midpoints between levels.  Both
// integrals have closed forms:
//   mass:    with a = sin(theta), integral of (1-a^2)^((m-3)/2) da is the
//            integral of cos^(m-2)(theta) d(theta), by the reduction formula;
//   moment:  integral of a (1-a^2)^k da = -(1-a^2)^(k+1) / (2(k+1)).
#include <cmath>
#include <cstdint>

#include "pariskv.h"

namespace {

// integral_0^theta cos^n(t) dt
double cos_power_integral(int n, double theta) {
    if (n == 0) return theta;
    if (n == 1) return std::sin(theta);
    const double c = std::cos(theta), s = std::sin(theta);
    return std::pow(c, n - 1) * s / n + (double)(n - 1) / n * cos_power_integral(n - 2, theta);
}

struct AbsCoordLaw {
    int m;
    double total;  // unnormalised mass of [0, 1]
    explicit AbsCoordLaw(int m_) : m(m_) { total = cos_power_integral(m - 2, M_PI / 2); }
    double cdf(double a) const {
        if (a >= 1.0) return 1.0;
        return cos_power_integral(m - 2, std::asin(a)) / total;
    }
    // E[a ; a < x] (unnormalised antiderivative difference / total)
    double partial_moment(double x) const {
        const double k1 = (m - 3) / 2.0 + 1.0;
        const double one = 1.0 / (2.0 * k1);
        const double r = (x >= 1.0) ? 0.0 : std::pow(1.0 - x * x, k1);
        return (one - r / (2.0 * k1)) / total;
    }
};

// thresholds t[0..n-2] at the l/n quantiles of the law (bisection)
void quantile_thresholds(const AbsCoordLaw& law, int n, double* t) {
    for (int i = 0; i < n - 1; ++i) {
        const double target = (i + 1.0) / n;
        double lo = 0.0, hi = 1.0;
        for (int it = 0; it < 200 && hi - lo > 0.0; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (mid <= lo || mid >= hi) break;   // adjacent doubles
            (law.cdf(mid) < target ? lo : hi) = mid;
        }
        t[i] = 0.5 * (lo + hi);
    }
}

}  // namespace

// Alternative reading: equal-probability bins (threshold l = the l/n quantile of
// a, found by bisection on the closed-form law) with conditional-mean levels.
extern "C" pk_status pk_codebook_quantile(int32_t sub_dim, int32_t n_levels, float* levels,
                                          float* sq_thresholds) {
    if (sub_dim < 2 || n_levels != 8 || !levels || !sq_thresholds) return PK_ERR_INVALID;
    const AbsCoordLaw law(sub_dim);
    const int n = n_levels;
    double t[8];
    quantile_thresholds(law, n, t);
    double lo = 0.0;
    for (int i = 0; i < n; ++i) {
        const double hi = (i == n - 1) ? 1.0 : t[i];
        levels[i] = (float)((law.partial_moment(hi) - law.partial_moment(lo)) /
                            (law.cdf(hi) - law.cdf(lo)));
        lo = hi;
    }
    for (int i = 0; i < n - 1; ++i) sq_thresholds[i] = (float)(t[i] * t[i]);
    return PK_OK;
}

extern "C" pk_status pk_codebook(int32_t sub_dim, int32_t n_levels, float* levels,
                                 float* sq_thresholds) {
    if (sub_dim < 2 || n_levels != 8 || !levels || !sq_thresholds) return PK_ERR_INVALID;
    const AbsCoordLaw law(sub_dim);
    const int n = n_levels;
    double t[8], c[8];
    // start from the equal-probability thresholds: every bin then has mass
    // 1/n (from a uniform start on [0, 1] the top bins of a large-m law hold
    // no mass in double precision, and their levels would be 0/0); the law
    // is log-concave for m >= 3, so the Lloyd fixed point is unique
    quantile_thresholds(law, n, t);
    for (int iter = 0; iter < 200000; ++iter) {
        double lo = 0.0;
        for (int i = 0; i < n; ++i) {
            const double hi = (i == n - 1) ? 1.0 : t[i];
            const double mass = law.cdf(hi) - law.cdf(lo);
            c[i] = (law.partial_moment(hi) - law.partial_moment(lo)) / mass;
            lo = hi;
        }
        double moved = 0.0;
        for (int i = 0; i < n - 1; ++i) {
            const double nt = 0.5 * (c[i] + c[i + 1]);
            moved = std::fmax(moved, std::fabs(nt - t[i]));
            t[i] = nt;
        }
        if (moved < 1e-15) break;
    }
    double lo = 0.0;
    for (int i = 0; i < n; ++i) {
        const double hi = (i == n - 1) ? 1.0 : t[i];
        c[i] = (law.partial_moment(hi) - law.partial_moment(lo)) / (law.cdf(hi) - law.cdf(lo));
        lo = hi;
        levels[i] = (float)c[i];
    }
    for (int i = 0; i < n - 1; ++i) sq_thresholds[i] = (float)(t[i] * t[i]);
    return PK_OK;
}
