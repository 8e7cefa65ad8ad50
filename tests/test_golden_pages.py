"""The oracle against the values the pages print (tests/golden/page_values.json).

Each fixture entry names the page and passage it comes from; the checks
below compute the same quantity with the oracle and compare it at the
precision the page prints."""

import json
import math
import os

import numpy as np
import pytest

from oracle import tq_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


def test_dmse_small_bits_rounds_to_printed_values():
    g = GOLDEN["dmse_small_bits"]
    for b, printed, dec in zip(g["b"], g["printed"], g["decimals"]):
        dm = O.lloyd_max(4096, b)[2]
        assert round(dm, dec) == printed, (b, dm)


def test_gap_ratio_is_sqrt3_pi_over_2_not_sqrt_3pi_over_2():
    g = GOLDEN["gap_to_lower_bound"]
    # the distortion ratio D_mse * 4^b climbs with b towards the high-rate
    # constant sqrt(3) * pi / 2, the ~2.7 gap the page prints; the garbled
    # sqrt(3 pi) / 2 = 1.53 is already exceeded at b = 2
    ratios = [O.lloyd_max(4096, b)[2] * 4.0 ** b for b in range(1, 7)]
    steps = np.diff(ratios)
    assert np.all(steps > 0) and np.all(np.diff(steps) < 0)
    assert ratios[-1] < math.sqrt(3) * math.pi / 2 < g["printed_ratio"] + 0.01
    # Aitken extrapolation of the last three terms estimates the limit
    limit = ratios[-1] - steps[-1] ** 2 / (steps[-1] - steps[-2])
    assert abs(limit - math.sqrt(3) * math.pi / 2) < 0.02
    assert round(math.sqrt(3) * math.pi / 2, 1) == g["printed_overview_ratio"]
    assert ratios[1] > math.sqrt(3 * math.pi) / 2


def test_b1_bias_and_dequant_level():
    g = GOLDEN["mse_inner_product_bias_b1"]
    d = 4096
    c, _, dmse, _ = O.lloyd_max(d, 1)
    # slope of the b = 1 mse estimate = d * c^2 = 1 - D_mse(1) -> 2/pi
    assert abs(d * c[1] ** 2 - (1 - dmse)) < 1e-10   # quadrature accuracy at d = 4096
    assert round(1 - dmse, g["decimals"]) == g["printed"]
    assert abs(c[1] - math.sqrt(2 / (math.pi * d))) < 1e-3 * c[1]


def test_index_entropy_b4_and_prefix_code_saving():
    g = GOLDEN["index_entropy_b4"]
    d = 128
    _, t, _, _ = O.lloyd_max(d, 4)
    e = np.concatenate(([0.0], t[8:], [1.0]))
    p_half = O.beta_upper_tail(e[:-1], d) - O.beta_upper_tail(e[1:], d)
    h = -2 * np.sum(p_half * np.log2(p_half))
    assert round(h, 1) == g["printed_bits"]
    assert abs((4 - h) / 4 - g["printed_saving"]) < 0.01          # 5.65 %: "about 5 %"


def test_storage_and_split_arithmetic():
    s = GOLDEN["rotation_storage"]
    assert round(s["d"] ** 2 * 4 / 2 ** 20) == s["printed_mb"]
    o = GOLDEN["outlier_split_2p5"]
    eff = (o["outlier_channels"] * o["outlier_bits"]
           + (o["channels"] - o["outlier_channels"]) * o["other_bits"]) / o["channels"]
    # The printed split does not add up: 32 x 3 + 96 x 2 bits over 128
    # channels is 2.25 bits, not the 2.5 printed beside it.  The outlier split
    # is not on the built path; the discrepancy is recorded as a reading.
    assert eff == 2.25 and eff != o["printed_effective_bits"]
    r = GOLDEN["rotorquant_parameters"]
    assert r["turbo"] == r["d"] ** 2          # a dense d x d rotation's parameter count


def test_one_hot_energy_spreads_over_all_coordinates():
    g = GOLDEN["one_hot_spread"]
    d = g["d"]
    rs = np.random.default_rng(0)
    signs = np.where(rs.integers(0, 2, d) == 1, 1, -1).astype(np.int8)
    for j in (0, 17, d - 1):
        e = np.zeros((1, d))
        e[0, j] = 1.0
        y = O.rht(e, signs)
        assert np.allclose(np.abs(y), 1 / math.sqrt(d), atol=1e-15)
        assert np.count_nonzero(np.abs(y) > 0.5 / math.sqrt(d)) == g["printed_dims"]


@pytest.mark.parametrize("d", [64, 1024])
def test_lemma1_variance_is_one_over_d(d):
    assert GOLDEN["lemma1_gaussian_limit"]["variance"] == "1/d"
    from scipy import integrate
    var = integrate.quad(lambda x: x * x * O.beta_pdf(np.array([x]), d)[0], -1, 1,
                         points=[-5 / math.sqrt(d), 0, 5 / math.sqrt(d)], epsabs=1e-14)[0]
    assert abs(var * d - 1) < 1e-9
