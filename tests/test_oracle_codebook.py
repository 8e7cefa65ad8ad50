"""Pins of the oracle's codebook (Lemma 1 density and Lloyd-Max) against
what the TurboQuant paper summary (Jump2Paper Archive) and mathematics fix:
normalisation and variance of the Lemma 1 density, quadrature of the cell
moments, the closed-form 1-bit centroid, the uniform d = 3 case, the
Gaussian limit, a brute-force search of the optimum, Theorem D_mse's printed
numerics and bounds, and the b = 4 index entropy from the limitations
section."""

import math

import numpy as np
import pytest
from scipy import integrate, optimize, stats
from scipy.special import gammaln

from oracle import tq_oracle as O


@pytest.mark.parametrize("d", [3, 5, 16, 128, 2048])
def test_beta_density_is_normalised_with_variance_one_over_d(d):
    # A coordinate of a uniform point on S^{d-1} has E[X] = 0, E[X^2] = 1/d.
    f = lambda x: O.beta_pdf(np.array([x]), d)[0]
    pts = [-6 / math.sqrt(d), 6 / math.sqrt(d)] if d > 50 else None
    mass = integrate.quad(f, -1, 1, points=pts, limit=200)[0]
    mean = integrate.quad(lambda x: x * f(x), -1, 1, points=pts, limit=200)[0]
    var = integrate.quad(lambda x: x * x * f(x), -1, 1, points=pts, limit=200)[0]
    assert abs(mass - 1) < 1e-10
    assert abs(mean) < 1e-12
    assert abs(var - 1 / d) < 1e-10 / d


@pytest.mark.parametrize("d", [3, 7, 128, 2048])
def test_cell_moments_match_quadrature(d):
    g = np.random.default_rng(1)
    scale = min(1.0, 5 / math.sqrt(d))
    for _ in range(8):
        lo, hi = np.sort(g.uniform(0, scale, size=2))
        m0, m1, m2 = O.cell_moments(np.array([lo]), np.array([hi]), d)
        f = lambda x: O.beta_pdf(np.array([x]), d)[0]
        q0 = integrate.quad(f, lo, hi, epsabs=0, epsrel=1e-13)[0]
        q1 = integrate.quad(lambda x: x * f(x), lo, hi, epsabs=0, epsrel=1e-13)[0]
        q2 = integrate.quad(lambda x: x * x * f(x), lo, hi, epsabs=0, epsrel=1e-13)[0]
        assert abs(m0[0] - q0) <= 1e-11 * max(q0, 1e-300) + 1e-15
        assert abs(m1[0] - q1) <= 1e-11 * max(q1, 1e-300) + 1e-15
        assert abs(m2[0] - q2) <= 1e-11 * max(q2, 1e-300) + 1e-15
    # The upper tail goes through 1/2 at 0 and to 0 at 1.
    assert abs(O.beta_upper_tail(0.0, d) - 0.5) < 1e-15
    assert O.beta_upper_tail(1.0, d) == 0.0


@pytest.mark.parametrize("d", [3, 16, 128, 2048])
def test_one_bit_centroid_closed_form(d):
    # b = 1: the centroid is E[X | X > 0] = Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2))
    # and D_mse = d (E[X^2] - c^2) = 1 - d c^2.
    c, t, dmse, _ = O.lloyd_max(d, 1)
    exact = math.exp(gammaln(d / 2) - 0.5 * math.log(math.pi) - gammaln((d + 1) / 2))
    assert abs(c[1] - exact) < 1e-11 * exact
    assert c[0] == -c[1] and t[0] == 0.0
    assert abs(dmse - (1 - d * exact * exact)) < 1e-11


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_d3_density_is_uniform_so_quantiser_is_uniform(m):
    # d = 3: f_X = 1/2 on [-1, 1]; the optimal quantiser is uniform and
    # D_mse = 3 * (2/K)^2 / 12 = 4^-m, the lower bound.
    c, t, dmse, _ = O.lloyd_max(3, m, tol=1e-15)
    k = 1 << m
    assert np.allclose(c, -1 + (2 * np.arange(k) + 1) / k, atol=1e-12)
    assert np.allclose(t, -1 + 2 * np.arange(1, k) / k, atol=1e-12)
    assert abs(dmse - 4.0 ** (-m)) < 1e-12


@pytest.mark.parametrize("d,m", [(128, 1), (128, 2), (128, 3), (128, 4), (2048, 3), (37, 3)])
def test_codebook_structure(d, m):
    c, t, dmse, _ = O.lloyd_max(d, m)
    k = 1 << m
    assert c.shape == (k,) and t.shape == (k - 1,)
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    assert np.array_equal(c, -c[::-1]) and np.array_equal(t, -t[::-1])
    assert t[k // 2 - 1] == 0.0
    # thresholds are midpoints and every centroid is the mean of its cell
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-16)
    edges = np.concatenate(([0.0], t[k // 2:], [1.0]))
    m0, m1, _ = O.cell_moments(edges[:-1], edges[1:], d)
    assert np.allclose(m1 / m0, c[k // 2:], rtol=1e-12, atol=0)


def _gaussian_lloyd(k, iters=20000):
    """Independent Lloyd-Max for N(0, 1) with closed-form normal moments."""
    half = k // 2
    c = (np.arange(half) + 0.5) * 3.0 / half
    for _ in range(iters):
        e = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        mass = stats.norm.sf(e[:-1]) - stats.norm.sf(e[1:])
        first = stats.norm.pdf(e[:-1]) - stats.norm.pdf(e[1:])
        c_new = first / mass
        if np.max(np.abs(c_new - c)) < 1e-15:
            c = c_new
            break
        c = c_new
    e = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    mass = stats.norm.sf(e[:-1]) - stats.norm.sf(e[1:])
    first = stats.norm.pdf(e[:-1]) - stats.norm.pdf(e[1:])
    xpdf = lambda v: np.where(np.isfinite(v), v * stats.norm.pdf(np.where(np.isfinite(v), v, 0.0)), 0.0)
    ex2 = mass + xpdf(e[:-1]) - xpdf(e[1:])
    mse = 2 * np.sum(ex2 - 2 * c * first + c * c * mass)
    return c, mse


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_large_d_tends_to_gaussian_lloyd_max(m):
    # Lemma 1: the marginal tends to N(0, 1/d), so sqrt(d) * c_k tends to the
    # Lloyd-Max levels of N(0, 1); the error is O(1/d).
    gc, gmse = _gaussian_lloyd(1 << m)
    if m == 1:
        assert abs(gc[0] - math.sqrt(2 / math.pi)) < 1e-14
        assert abs(gmse - (1 - 2 / math.pi)) < 1e-14
    d = 4096
    c, _, dmse, _ = O.lloyd_max(d, m)
    k = 1 << m
    assert np.allclose(math.sqrt(d) * c[k // 2:], gc, rtol=3 / d * 4, atol=0)
    assert abs(dmse - gmse) < 3 * gmse / d * 4


def test_theorem_dmse_printed_numerics():
    # Theorem D_mse prints 0.36, 0.117, 0.03, 0.009 for b = 1..4.  They are
    # the large-d values rounded; at d = 128 the exact values are
    # 0.3609 / 0.1160 / 0.03397 / 0.009315.
    big = [O.lloyd_max(4096, b)[2] for b in (1, 2, 3, 4)]
    assert round(big[0], 2) == 0.36
    assert round(big[1], 3) == 0.117
    assert round(big[2], 2) == 0.03
    assert round(big[3], 3) == 0.009
    d128 = [O.lloyd_max(128, b)[2] for b in (1, 2, 3, 4)]
    assert np.allclose(d128, [0.360889, 0.116000, 0.033966, 0.009315], atol=5e-7)


@pytest.mark.parametrize("d", [128, 2048])
def test_theorem_dmse_bounds(d):
    # Lower bound 4^-b (Shannon lower bound + Yao); upper bound read as
    # sqrt(3)*pi/2 * 4^-b (the printed constant is garbled; sqrt(3*pi)/2 is
    # violated by the page's own numerics, while sqrt(3)*pi/2 ~ 2.72 is the
    # ~2.7x gap the summary quotes).
    for b in range(1, 6):
        dm = O.lloyd_max(d, b)[2]
        assert 4.0 ** -b <= dm <= math.sqrt(3) * math.pi / 2 * 4.0 ** -b
        if b >= 2:
            assert dm > math.sqrt(3 * math.pi) / 2 * 4.0 ** -b


def test_brute_force_optimum_m2():
    # Grid + bounded search over the single positive threshold of a 2-bit
    # symmetric quantiser; centroids = cell means; cost by quadrature.
    d = 128
    f = lambda x: O.beta_pdf(np.array([x]), d)[0]

    def cost(t):
        lo_mass = integrate.quad(f, 0, t, epsrel=1e-13)[0]
        hi_mass = integrate.quad(f, t, 1, epsrel=1e-13, points=[0.6])[0]
        c1 = integrate.quad(lambda x: x * f(x), 0, t, epsrel=1e-13)[0] / lo_mass
        c2 = integrate.quad(lambda x: x * f(x), t, 1, epsrel=1e-13, points=[0.6])[0] / hi_mass
        return (integrate.quad(lambda x: (x - c1) ** 2 * f(x), 0, t, epsrel=1e-13)[0]
                + integrate.quad(lambda x: (x - c2) ** 2 * f(x), t, 1, epsrel=1e-13, points=[0.6])[0])

    grid = np.linspace(0.02, 0.25, 47)
    t0 = grid[np.argmin([cost(t) for t in grid])]
    res = optimize.minimize_scalar(cost, bounds=(t0 - 0.01, t0 + 0.01), method="bounded",
                                   options={"xatol": 1e-9})
    c, t, dmse, _ = O.lloyd_max(d, 2)
    assert abs(res.x - t[2]) < 1e-6
    assert abs(2 * d * res.fun - dmse) < 1e-9


def test_b4_index_entropy_about_3_8_bits():
    # Limitations section: a prefix code on b = 4 indices would need about
    # 3.8 bits (entropy of the cell probabilities).
    for d, expect in ((128, 3.774), (2048, 3.766)):
        c, t, _, _ = O.lloyd_max(d, 4)
        e = np.concatenate(([0.0], t[8:], [1.0]))
        p_half = O.beta_upper_tail(e[:-1], d) - O.beta_upper_tail(e[1:], d)
        h = -2 * np.sum(p_half * np.log2(p_half))
        assert abs(2 * np.sum(p_half) - 1) < 1e-12
        assert round(h, 1) == 3.8
        assert abs(h - expect) < 0.02


def test_storage_arithmetic():
    # Limitations section: a d x d float32 matrix at d = 1536 is ~9 MB; the
    # forum post's 16,384 parameters are 128^2.
    assert abs(1536 * 1536 * 4 / 2**20 - 9.0) < 0.05
    assert 128 * 128 == 16384
