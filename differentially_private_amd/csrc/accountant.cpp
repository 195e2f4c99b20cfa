// Privacy accounting on the host: the Renyi-DP of the Poisson-subsampled Gaussian mechanism,
// its composition and conversion to (epsilon, delta) ("Privacy-Preserving Machine Learning",
// section on privacy accounting: RDP bounds add over steps; the unsampled Gaussian has per-step
// RDP alpha / (2 sigma^2); subsampling mixes the inclusion and non-inclusion cases), and the
// exact one-step Gaussian pair of "Sensitivity Inflation from Cross-Record Precision Routing in
// Private Quantized Fine-Tuning", Sec. 3.2 Eq. 5.
//
// Sampled Gaussian (sensitivity 1, noise multiplier sigma, sampling probability q): the order-
// alpha divergence of (1 - q) N(0, s^2) + q N(1, s^2) from N(0, s^2) is log(A) / (alpha - 1) with
//   A = E_{z ~ N(0, s^2)} [(1 - q + q e^u)^alpha],  u = (2z - 1) / (2 s^2)
// (Mironov, Talwar and Zhang, "Renyi differential privacy of the sampled Gaussian mechanism").
// Integer alpha: binomial expansion, A = sum_k C(alpha, k) (1-q)^(alpha-k) q^k e^((k^2-k)/(2s^2)).
// Other alpha: split the expectation at z0 = s^2 log((1-q)/q) + 1/2, where the two summands are
// equal; below z0 expand (1 - q)^alpha (1 + x)^alpha, x = q e^u / (1 - q) < 1, above it
// (q e^u)^alpha (1 + 1/x)^alpha, each as a binomial series; every term integrates to a Gaussian
// tail:
//   A = sum_i C(alpha, i) [ (1-q)^(alpha-i) q^i e^((i^2-i)/(2s^2)) erfc((i - z0)/(sqrt2 s)) / 2
//                         + q^(alpha-i) (1-q)^i e^((j^2-j)/(2s^2)) erfc((z0 - j)/(sqrt2 s)) / 2 ],
// j = alpha - i.  Past i = alpha the coefficients alternate in sign and the terms decrease, so the
// sum stops once both terms are below 1e-16 of the running total.  Everything is summed in log
// space with the signs kept apart.
#include <cmath>
#include <cstdint>
#include <limits>

namespace dpsgd {

namespace {

constexpr double kNegInf = -std::numeric_limits<double>::infinity();

// log(erfc(x)), finite far into the tail (erfc underflows past x ~ 26.5)
double log_erfc(double x) {
    if (x < 25.0) return std::log(std::erfc(x));
    // erfc(x) = e^(-x^2) / (x sqrt(pi)) (1 - 1/(2x^2) + 3/(4x^4) - 15/(8x^6) + 105/(16x^8) - ...)
    const double r = 1.0 / (x * x);
    const double series = 1.0 - r / 2 + 3 * r * r / 4 - 15 * r * r * r / 8 + 105 * r * r * r * r / 16;
    return -x * x - std::log(x) - 0.5 * std::log(M_PI) + std::log(series);
}

// log(e^a + e^b)
double log_add(double a, double b) {
    if (a == kNegInf) return b;
    if (b == kNegInf) return a;
    const double m = a > b ? a : b;
    return m + std::log1p(std::exp(-std::fabs(a - b)));
}

double log_a_integer(double q, double sigma, int64_t alpha) {
    double acc = kNegInf;
    for (int64_t k = 0; k <= alpha; ++k) {
        const double log_coef = std::lgamma((double)alpha + 1) - std::lgamma((double)k + 1) -
                                std::lgamma((double)(alpha - k) + 1);
        const double t = log_coef + (double)(alpha - k) * std::log1p(-q) + (double)k * std::log(q) +
                         ((double)k * k - k) / (2 * sigma * sigma);
        acc = log_add(acc, t);
    }
    return acc;
}

double log_a_fractional(double q, double sigma, double alpha) {
    const double s2 = sigma * sigma;
    const double z0 = s2 * std::log((1 - q) / q) + 0.5;
    const double lq = std::log(q), l1q = std::log1p(-q);
    double pos = kNegInf, neg = kNegInf;     // log of the positive and of the negative part
    double log_c = 0.0;                      // log |C(alpha, i)|
    bool c_pos = true;                       // sign of C(alpha, i)
    for (int64_t i = 0; i < 100000000; ++i) {
        const double di = (double)i, dj = alpha - di;
        const double t0 = log_c + dj * l1q + di * lq + (di * di - di) / (2 * s2) +
                          log_erfc((di - z0) / (std::sqrt(2.0) * sigma)) - std::log(2.0);
        const double t1 = log_c + dj * lq + di * l1q + (dj * dj - dj) / (2 * s2) +
                          log_erfc((z0 - dj) / (std::sqrt(2.0) * sigma)) - std::log(2.0);
        const double t = log_add(t0, t1);
        if (c_pos) pos = log_add(pos, t);
        else neg = log_add(neg, t);
        if (di > alpha + 1 && t < pos - 16 * std::log(10.0)) break;
        // C(alpha, i + 1) = C(alpha, i) (alpha - i) / (i + 1)
        const double f = alpha - di;
        if (f == 0.0) break;                 // (integer alpha: the series ends)
        log_c += std::log(std::fabs(f)) - std::log(di + 1);
        if (f < 0) c_pos = !c_pos;
    }
    if (neg == kNegInf) return pos;
    return pos + std::log1p(-std::exp(neg - pos));
}

// standard normal CDF times e^a, as a log: log(e^a Phi(y))
double log_exp_phi(double a, double y) { return a + log_erfc(-y / std::sqrt(2.0)) - std::log(2.0); }

}  // namespace

double rdp_sampled_gaussian(double q, double sigma, double alpha) {
    if (q == 0.0) return 0.0;
    if (q == 1.0) return alpha / (2 * sigma * sigma);
    double log_a;
    if (alpha == std::floor(alpha) && alpha <= 1e6)
        log_a = log_a_integer(q, sigma, (int64_t)alpha);
    else
        log_a = log_a_fractional(q, sigma, alpha);
    return log_a / (alpha - 1);
}

double rdp_epsilon(const double* orders, const double* rdp, int n, double delta, bool tight,
                   double* best_order) {
    double best = std::numeric_limits<double>::infinity();
    double arg = 0.0;
    for (int k = 0; k < n; ++k) {
        const double a = orders[k];
        const double e = tight ? rdp[k] + std::log((a - 1) / a) - (std::log(delta) + std::log(a)) / (a - 1)
                               : rdp[k] + std::log(1 / delta) / (a - 1);
        if (e < best) {
            best = e;
            arg = a;
        }
    }
    if (best_order) *best_order = arg;
    return best;
}

double gaussian_pair_delta(double eps, double mu) {
    // Phi(mu/2 - eps/mu) - e^eps Phi(-mu/2 - eps/mu)
    const double a = std::exp(log_exp_phi(0.0, mu / 2 - eps / mu));
    const double b = std::exp(log_exp_phi(eps, -mu / 2 - eps / mu));
    return a - b;
}

double gaussian_pair_epsilon(double delta, double mu) {
    // delta(eps) decreases in eps: bisection
    double lo = 0.0, hi = 1.0;
    while (gaussian_pair_delta(hi, mu) > delta && hi < 1e6) hi *= 2;
    for (int it = 0; it < 200 && hi - lo > 1e-13 * hi; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (gaussian_pair_delta(mid, mu) > delta) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}

}  // namespace dpsgd
