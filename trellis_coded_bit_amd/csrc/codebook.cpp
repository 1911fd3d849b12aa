// tcq_make_codebook: the closed-form Gaussian quantile table in a seeded order
// (the CurveTQ abstract on the aqora listing names a closed-form quantile table; the
// QTIP abstract names lookup-only trellis codes).  Host code, no GPU involvement.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "tcq.h"

namespace tcq {
void set_error(const char *fmt, ...);
}

namespace {

// Wichura, "Algorithm AS 241: The percentage points of the normal distribution",
// Applied Statistics 37 (1988), PPND16.  Three rational approximations in nested
// (Horner) form: a central one in r = 0.180625 - q^2 for |q| <= 0.425, and two tail
// ones in r = sqrt(-log(min(p, 1-p))) split at r = 5.
struct Rational8 {
    double num[8];  // coefficients of r^0 .. r^7
    double den[8];
    // numerator and denominator polynomials at r, each in nested form
    void eval(double r, double &a, double &b) const {
        a = num[7];
        b = den[7];
        for (int i = 6; i >= 0; --i) {
            a = a * r + num[i];
            b = b * r + den[i];
        }
    }
};

constexpr Rational8 kCentral = {
    {3.3871328727963666080e0, 1.3314166789178437745e+2, 1.9715909503065514427e+3,
     1.3731693765509461125e+4, 4.5921953931549871457e+4, 6.7265770927008700853e+4,
     3.3430575583588128105e+4, 2.5090809287301226727e+3},
    {1.0, 4.2313330701600911252e+1, 6.8718700749205790830e+2, 5.3941960214247511077e+3,
     2.1213794301586595867e+4, 3.9307895800092710610e+4, 2.8729085735721942674e+4,
     5.2264952788528545610e+3}};
constexpr Rational8 kNearTail = {
    {1.42343711074968357734e0, 4.63033784615654529590e0, 5.76949722146069140550e0,
     3.64784832476320460504e0, 1.27045825245236838258e0, 2.41780725177450611770e-1,
     2.27238449892691845833e-2, 7.74545014278341407640e-4},
    {1.0, 2.05319162663775882187e0, 1.67638483018380384940e0, 6.89767334985100004550e-1,
     1.48103976427480074590e-1, 1.51986665636164571966e-2, 5.47593808499534494600e-4,
     1.05075007164441684324e-9}};
constexpr Rational8 kFarTail = {
    {6.65790464350110377720e0, 5.46378491116411436990e0, 1.78482653991729133580e0,
     2.96560571828504891230e-1, 2.65321895265761230930e-2, 1.24266094738807843860e-3,
     2.71155556874348757815e-5, 2.01033439929228813265e-7},
    {1.0, 5.99832206555887937690e-1, 1.36929880922735805310e-1, 1.48753612908506148525e-2,
     7.86869131145613259100e-4, 1.84631831751005468180e-5, 1.42151175831644588870e-7,
     2.04426310338993978564e-15}};

double normal_quantile(double p) {
    const double q = p - 0.5;
    double a, b;
    if (std::fabs(q) <= 0.425) {
        kCentral.eval(0.180625 - q * q, a, b);
        return q * a / b;  // (q * num) / den, left to right as in the published routine
    }
    const double r = std::sqrt(-std::log(q < 0.0 ? p : 1.0 - p));
    if (r <= 5.0)
        kNearTail.eval(r - 1.6, a, b);
    else
        kFarTail.eval(r - 5.0, a, b);
    const double x = a / b;
    return q < 0.0 ? -x : x;
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): Weyl step by the golden gamma, then
// the "variant 13" 64-bit finalizer.
struct SplitMix64 {
    uint64_t x;
    uint64_t operator()() {
        x += 0x9E3779B97F4A7C15ull;
        uint64_t z = x;
        z ^= z >> 30;
        z *= 0xBF58476D1CE4E5B9ull;
        z ^= z >> 27;
        z *= 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

// 2^bits quantiles Phi^-1((a + 1/2) / 2^bits), ascending, with the upper half the exact
// negation of the lower half.
std::vector<float> quantiles(int bits) {
    const int64_t m = int64_t{1} << bits;
    std::vector<float> g(static_cast<size_t>(m), 0.0f);
    for (int64_t a = 0, b = m - 1; a < b; ++a, --b) {
        const float v = static_cast<float>(normal_quantile((static_cast<double>(a) + 0.5) /
                                                           static_cast<double>(m)));
        g[a] = v;
        g[b] = -v;
    }
    return g;
}

}  // namespace

extern "C" int tcq_make_codebook(int L, int V, uint64_t seed, float *out_host) {
    if (L < 1 || L > 24 || V < 1 || V > 8 || V > L) {
        tcq::set_error("tcq_make_codebook: need 1 <= L <= 24 and 1 <= V <= min(L, 8) (L=%d V=%d)",
                       L, V);
        return TCQ_EINVAL;
    }
    if (!out_host) {
        tcq::set_error("tcq_make_codebook: out_host is NULL");
        return TCQ_EINVAL;
    }
    const int64_t rows = int64_t{1} << L;
    // field widths, most significant field first
    std::vector<int> width(V);
    for (int v = 0; v < V; ++v) width[v] = L / V + (v < L % V ? 1 : 0);
    std::vector<std::vector<float>> grid(V);
    for (int v = 0; v < V; ++v) grid[v] = quantiles(width[v]);

    for (int64_t e = 0; e < rows; ++e) {
        int lo = L;
        for (int v = 0; v < V; ++v) {
            lo -= width[v];
            const int64_t field = (e >> lo) & ((int64_t{1} << width[v]) - 1);
            out_host[e * V + v] = grid[v][static_cast<size_t>(field)];
        }
    }
    // Fisher-Yates, last row first
    SplitMix64 rng{seed};
    std::vector<float> tmp(V);
    for (int64_t i = rows - 1; i > 0; --i) {
        const int64_t j = static_cast<int64_t>(rng() % static_cast<uint64_t>(i + 1));
        if (j == i) continue;
        std::memcpy(tmp.data(), out_host + i * V, sizeof(float) * V);
        std::memcpy(out_host + i * V, out_host + j * V, sizeof(float) * V);
        std::memcpy(out_host + j * V, tmp.data(), sizeof(float) * V);
    }
    return TCQ_OK;
}
