"""The library's host-side accountant (series evaluation of the sampled Gaussian's RDP, RDP
conversions, Eq. 5) against the oracle (numerical integration of the definition, 30-digit
bisection), the page's printed values, and its argument checks.  CPU only."""
import json
import os

import pytest

import differentially_private_amd as dp
from oracle import accountant as acc


@pytest.mark.parametrize("q,sigma", [(0.01, 1.0), (0.001, 0.8), (0.05, 2.0), (0.3, 1.2), (0.9, 0.7),
                                     (1e-5, 0.5)])
def test_rdp_matches_oracle(q, sigma):
    orders = [1.05, 1.5, 2, 2.7, 3.3, 5, 8.5, 12, 20.25, 33, 63]
    lib = dp.rdp_sampled_gaussian(q, sigma, orders)
    for a, v in zip(orders, lib):
        want = acc.rdp_sampled_gaussian(q, sigma, a)
        # relative 1e-9, plus 1e-14 absolute: log(A) for A near 1 (tiny q) keeps ~1e-16 of A
        assert abs(v - want) <= 1e-9 * abs(want) + 1e-14, (q, sigma, a, v, want)


def test_rdp_edge_orders_and_rates():
    o = [1.5, 4, 30.5]
    assert dp.rdp_sampled_gaussian(0.0, 1.0, o) == [0.0, 0.0, 0.0]
    assert all(abs(v - a / 2) < 1e-15 for v, a in zip(dp.rdp_sampled_gaussian(1.0, 1.0, o), o))


def test_page_epsilons_from_library(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_accountant.json")))
    per = dp.rdp_sampled_gaussian(g["q"], g["sigma"], acc.DEFAULT_ORDERS)
    for steps, want in g["epsilon_3dp"].items():
        rdp = [int(steps) * r for r in per]
        eps, order = dp.rdp_to_epsilon(acc.DEFAULT_ORDERS, rdp, g["delta"], tight=True)
        assert round(eps, 3) == want
        e_or, o_or = acc.epsilon_tight(rdp, acc.DEFAULT_ORDERS, g["delta"])
        assert abs(eps - e_or) < 1e-9 and order == o_or
        e_c, _ = dp.rdp_to_epsilon(acc.DEFAULT_ORDERS, rdp, g["delta"], tight=False)
        assert abs(e_c - acc.epsilon_conservative(rdp, acc.DEFAULT_ORDERS, g["delta"])[0]) < 1e-9


def test_gaussian_pair_matches_oracle(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p5_gaussian_pair.json")))
    for mu, want in g["epsilon_2dp"].items():
        for d, w in zip(g["delta"], want):
            e = dp.gaussian_pair_epsilon(d, float(mu))
            assert round(e, 2) == w
            assert abs(e - acc.gaussian_pair_epsilon(d, float(mu))) < 1e-9
    for eps, mu in [(0.0, 0.5), (1.0, 1.0), (3.0, 2.0), (8.0, 1.0), (0.3, 0.05)]:
        assert abs(dp.gaussian_pair_delta(eps, mu) - acc.gaussian_pair_delta(eps, mu)) < 1e-13


@pytest.mark.parametrize("call", [
    lambda: dp.rdp_sampled_gaussian(1.5, 1.0, [2]),
    lambda: dp.rdp_sampled_gaussian(0.1, 0.0, [2]),
    lambda: dp.rdp_sampled_gaussian(0.1, 1.0, [1.0]),
    lambda: dp.rdp_sampled_gaussian(0.1, 1.0, [float("nan")]),
    lambda: dp.rdp_to_epsilon([2.0], [0.1], 0.0),
    lambda: dp.rdp_to_epsilon([2.0], [0.1], 1.0),
    lambda: dp.rdp_to_epsilon([2.0], [-0.1], 1e-5),
    lambda: dp.gaussian_pair_delta(-1.0, 1.0),
    lambda: dp.gaussian_pair_delta(1.0, 0.0),
    lambda: dp.gaussian_pair_epsilon(0.0, 1.0),
    lambda: dp.gaussian_pair_epsilon(1e-5, float("inf")),
])
def test_accountant_argument_errors(call):
    with pytest.raises(dp.DpsgdError) as e:
        call()
    assert e.value.code == dp.ERR_INVALID_ARG


class _Fake:
    def __init__(self, v):
        self.v = v

    def data_ptr(self):
        return self.v


@pytest.mark.parametrize("kw", [dict(q=-0.1), dict(q=1.01), dict(q=float("nan")), dict(population=-1),
                                dict(population=(1 << 36) + 1), dict(count=None), dict(indices=None),
                                dict(ws=None), dict(ws=_Fake((1 << 20) + 4)), dict(mask=_Fake((1 << 22) + 2))])
def test_sampler_rejects_before_launch(kw):
    a = dict(seed=1, step=2, q=0.1, population=1000, indices=_Fake(1 << 21), count=_Fake(1 << 23),
             ws=_Fake(1 << 20), mask=None)
    a.update(kw)
    with pytest.raises(dp.DpsgdError) as e:
        dp.poisson_sample(a["seed"], a["step"], a["q"], a["population"], a["indices"], a["count"],
                          a["ws"], mask=a["mask"], stream=0)
    assert e.value.code == dp.ERR_INVALID_ARG
    assert dp.poisson_ws_bytes(-1) == -1 and dp.poisson_ws_bytes(0) == 16
    # two int64 per workgroup of 8,192 records, then 4 bytes of inclusion bits per 32 records
    # (rounded up to 8 bytes)
    def ws(n):
        return 16 * -(-n // 8192) + 8 * -(-(-(-n // 32) * 4) // 8)
    for n in (1, 31, 32, 33, 1024, 1025, 8192, 8193, 1 << 27, (1 << 36)):
        assert dp.poisson_ws_bytes(n) == ws(n), n
    assert dp.poisson_ws_bytes(1024) == 144 and dp.poisson_ws_bytes(8193) == 1064
