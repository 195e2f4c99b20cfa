"""Privacy accounting and Poisson sampling for the DP-SGD step, written from the definitions.

TEST INFRASTRUCTURE ONLY: this module is the reference the library's accountant and sampler are
checked against; only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline may use it.
It shares no code with the library: the Renyi divergence is integrated numerically from its
definition (the library sums a series), Eq. 5 is solved by bisection in 30-digit arithmetic, and
the sampler's draws come from the oracle's own Philox4x32-10.

- rdp_sampled_gaussian(q, sigma, alpha): per-step RDP of the Poisson-subsampled Gaussian
  mechanism ("Privacy-Preserving Machine Learning", section "Privacy accounting": RDP bounds add
  over steps; subsampling mixes the inclusion and non-inclusion cases), i.e. the Renyi divergence
  of order alpha between the mixture (1 - q) N(0, sigma^2) + q N(1, sigma^2) and N(0, sigma^2)
  (sensitivity 1, noise multiplier sigma):
      (1 / (alpha - 1)) log E_{z ~ N(0, sigma^2)} [(1 - q + q exp((2z - 1) / (2 sigma^2)))^alpha].
- epsilon_conservative / epsilon_tight: (epsilon, delta) from RDP over a set of orders: the
  conversion of Mironov's Renyi-DP paper (rdp + log(1/delta) / (alpha - 1)) and the tighter one of
  Balle, Barthe, Gaboardi, Hsu and Sato, "Hypothesis testing interpretations and Renyi
  differential privacy" (rdp + log((alpha - 1) / alpha) - (log delta + log alpha) / (alpha - 1)).
- gaussian_pair_delta / gaussian_pair_epsilon: Eq. 5 of "Sensitivity Inflation from Cross-Record
  Precision Routing in Private Quantized Fine-Tuning" (Sec. 3.2): the exact hockey-stick
  divergence of a one-step Gaussian release at mu = Delta / (sigma C).
- poisson_sample(seed, step, q, n): each record of n included independently with probability q
  ("Privacy-Preserving Machine Learning", DP-SGD phase 1): record i draws word i mod 4 of
  Philox4x32-10 block 2^63 + floor(i / 4) under key = seed, counter words 2-3 = step (the top
  bit of the block index keeps the sampler's words apart from the noise stream's), and is
  included iff that word < floor(q 2^32).
"""
from __future__ import annotations

import math

import mpmath as mp
import numpy as np

DIGITS = 30
# orders analysed by default: 1.1 .. 10.9 in steps of 0.1, then 12 .. 63
DEFAULT_ORDERS = [1 + x / 10 for x in range(1, 100)] + list(range(12, 64))


def rdp_sampled_gaussian(q: float, sigma: float, alpha: float) -> float:
    """Per-step RDP of order alpha > 1 of the sampled Gaussian mechanism, by quadrature."""
    if q == 0:
        return 0.0
    with mp.workdps(DIGITS):
        s = mp.mpf(sigma)
        qq = mp.mpf(q)
        a = mp.mpf(alpha)

        def integrand(z):
            ratio = 1 - qq + qq * mp.exp((2 * z - 1) / (2 * s * s))
            return mp.npdf(z, 0, s) * ratio ** a

        # the integrand's mass sits near z ~ alpha (the tilted Gaussian): split there
        # (increasing for alpha > 1)
        pts = [-mp.inf, -10 * s, 0, mp.mpf(0.5), a / 2, a, 2 * a + 10 * s, mp.inf]
        A = mp.quad(integrand, pts)
        return float(mp.log(A) / (a - 1))


def rdp_curve(q: float, sigma: float, steps: int, orders=DEFAULT_ORDERS):
    """RDP of `steps` composed steps (RDP adds over steps) at each order."""
    return [steps * rdp_sampled_gaussian(q, sigma, a) for a in orders]


def epsilon_conservative(rdp, orders, delta: float):
    """min over orders of rdp + log(1/delta) / (alpha - 1); returns (epsilon, order)."""
    vals = [(r + math.log(1 / delta) / (a - 1), a) for r, a in zip(rdp, orders)]
    return min(vals)


def epsilon_tight(rdp, orders, delta: float):
    """min over orders of rdp + log((alpha - 1) / alpha) - (log delta + log alpha) / (alpha - 1)."""
    vals = [(r + math.log((a - 1) / a) - (math.log(delta) + math.log(a)) / (a - 1), a)
            for r, a in zip(rdp, orders)]
    return min(vals)


def gaussian_pair_delta(eps: float, mu: float) -> float:
    """Eq. 5: Phi(mu/2 - eps/mu) - e^eps Phi(-mu/2 - eps/mu)."""
    with mp.workdps(DIGITS):
        e, m = mp.mpf(eps), mp.mpf(mu)
        return float(mp.ncdf(m / 2 - e / m) - mp.exp(e) * mp.ncdf(-m / 2 - e / m))


def gaussian_pair_epsilon(delta: float, mu: float) -> float:
    """The epsilon at which Eq. 5's delta equals `delta` (delta decreases in epsilon), by
    bisection in 30-digit arithmetic."""
    with mp.workdps(DIGITS):
        m = mp.mpf(mu)

        def d(e):
            return mp.ncdf(m / 2 - e / m) - mp.exp(e) * mp.ncdf(-m / 2 - e / m)
        lo, hi = mp.mpf(0), mp.mpf(1)
        while d(hi) > delta:
            hi *= 2
        for _ in range(200):
            mid = (lo + hi) / 2
            if d(mid) > delta:
                lo = mid
            else:
                hi = mid
        return float((lo + hi) / 2)


def poisson_sample(seed: int, step: int, q: float, n: int) -> np.ndarray:
    """Inclusion mask (bool, length n) of the Poisson sampler."""
    from . import philox_words
    nb = (n + 3) // 4
    words = philox_words(seed, step, (1 << 63), nb).reshape(-1)[:n].astype(np.uint64)
    threshold = int(math.floor(q * 4294967296.0))
    return words < np.uint64(threshold)
