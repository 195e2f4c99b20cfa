"""Pins of the oracle's accountant and Poisson sampler (oracle/accountant.py) against the pages and
closed forms.  CPU only."""
import json
import math
import os

import numpy as np
import pytest

from oracle import accountant as acc


def test_page_rdp_accountant_epsilons(golden_dir):
    """300 and 600 Poisson-sampled Gaussian steps at q = 0.01, sigma = 1, delta = 1e-5: the page
    prints epsilon 1.451 and 1.748.  Reproduced with the tighter RDP conversion over the default
    orders; the conservative conversion is larger, as a valid bound must be."""
    g = json.load(open(os.path.join(golden_dir, "p1_accountant.json")))
    per_step = [acc.rdp_sampled_gaussian(g["q"], g["sigma"], a) for a in acc.DEFAULT_ORDERS]
    for steps, want in g["epsilon_3dp"].items():
        rdp = [int(steps) * r for r in per_step]
        eps, order = acc.epsilon_tight(rdp, acc.DEFAULT_ORDERS, g["delta"])
        assert round(eps, 3) == want, (steps, eps, order)
        assert acc.epsilon_conservative(rdp, acc.DEFAULT_ORDERS, g["delta"])[0] > eps


@pytest.mark.parametrize("alpha,sigma", [(1.5, 1.0), (2, 0.7), (10, 2.0), (33.3, 4.0)])
def test_unsampled_gaussian_rdp(alpha, sigma):
    """q = 1 is the unsampled Gaussian: the page states the per-step RDP alpha / (2 sigma^2)."""
    assert abs(acc.rdp_sampled_gaussian(1.0, sigma, alpha) - alpha / (2 * sigma ** 2)) < 1e-12


@pytest.mark.parametrize("q,sigma,alpha", [(0.01, 1.0, 2), (0.01, 1.0, 7), (0.05, 0.8, 12),
                                           (0.3, 1.5, 40), (0.001, 1.0, 63)])
def test_integer_order_binomial_closed_form(q, sigma, alpha):
    """For integer orders the expectation expands binomially: A = sum_k C(alpha, k) (1-q)^(alpha-k)
    q^k exp((k^2 - k) / (2 sigma^2)) (E exp(k z / sigma^2) = exp(k^2 / (2 sigma^2)) for
    z ~ N(0, sigma^2)); the oracle's quadrature must agree with this independent form."""
    terms = [math.log(math.comb(alpha, k)) + (alpha - k) * math.log1p(-q) + k * math.log(q)
             + (k * k - k) / (2 * sigma ** 2) for k in range(alpha + 1)]
    top = max(terms)
    want = (top + math.log(sum(math.exp(t - top) for t in terms))) / (alpha - 1)
    assert abs(acc.rdp_sampled_gaussian(q, sigma, alpha) - want) <= 1e-10 * max(1.0, abs(want))


def test_rdp_properties():
    """RDP of the sampled mechanism: 0 at q = 0, increasing in q and in alpha, below the
    unsampled value."""
    assert acc.rdp_sampled_gaussian(0.0, 1.0, 5) == 0.0
    r = [acc.rdp_sampled_gaussian(q, 1.0, 5) for q in (0.01, 0.02, 0.1, 1.0)]
    assert all(a < b for a, b in zip(r, r[1:]))
    ra = [acc.rdp_sampled_gaussian(0.02, 1.0, a) for a in (1.5, 3, 8, 20)]
    assert all(a < b for a, b in zip(ra, ra[1:]))


def test_eq5_gaussian_pair_values(golden_dir):
    """Eq. 5 at the advertised mu = 1 and the measured mu = 1.065: the printed one-step epsilons
    at delta = 1e-3, 1e-5, 1e-6 (3.14 / 4.38 / 4.89 and 3.39 / 4.71 / 5.25)."""
    g = json.load(open(os.path.join(golden_dir, "p5_gaussian_pair.json")))
    for mu, want in g["epsilon_2dp"].items():
        for d, w in zip(g["delta"], want):
            e = acc.gaussian_pair_epsilon(d, float(mu))
            assert round(e, 2) == w, (mu, d, e)
            assert abs(acc.gaussian_pair_delta(e, float(mu)) - d) < 1e-12


def test_eq5_closed_forms():
    """At epsilon = 0 Eq. 5 is the total variation distance of N(0,1) and N(mu,1), 2 Phi(mu/2) - 1;
    delta decreases in epsilon and increases in mu."""
    for mu in (0.1, 1.0, 3.0):
        tv = math.erf(mu / 2 / math.sqrt(2))
        assert abs(acc.gaussian_pair_delta(0.0, mu) - tv) < 1e-15
    d = [acc.gaussian_pair_delta(e, 1.0) for e in (0.5, 1, 2, 4)]
    assert all(a > b for a, b in zip(d, d[1:]))
    assert acc.gaussian_pair_delta(2.0, 1.2) > acc.gaussian_pair_delta(2.0, 1.0)


def test_poisson_sampler_statistics():
    """Inclusion count over n records is Binomial(n, q): within 5 standard deviations of q n over
    several steps; q = 0 includes nothing, q = 1 everything; different steps draw different sets."""
    n = 1_000_000
    for step in range(3):
        m = acc.poisson_sample(7, step, 0.01, n)
        assert abs(m.sum() - 0.01 * n) < 5 * math.sqrt(0.01 * 0.99 * n)
    assert not acc.poisson_sample(7, 0, 0.0, 1000).any()
    assert acc.poisson_sample(7, 0, 1.0, 1000).all()
    a, b = acc.poisson_sample(7, 0, 0.5, 4096), acc.poisson_sample(7, 1, 0.5, 4096)
    assert 0.4 < (a != b).mean() < 0.6
