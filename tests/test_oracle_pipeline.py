"""Pins of the oracle's rotation, quantiser, packing, encode/decode and
inner-product estimator.

Sources: the TurboQuant paper summary (Jump2Paper Archive) -- definitions
table, Lemma 1, MSE decomposition, Theorem D_mse, the 1-bit 2/pi bias
paragraph, Definition 1 / Lemma 4 (QJL), Theorem D_prod; the AI Trends video
summary chapters 04:24 and 06:06 (normalise, RHT, transpose to undo); the
forum post's one-hot worst case (damoang RotorQuant post)."""

import math

import numpy as np
import pytest
from scipy import linalg, stats

import synth
from oracle import tq_oracle as O


# ----------------------------------------------------------------- rotation

@pytest.mark.parametrize("d", [2, 4, 8, 32, 128, 256])
def test_sylvester_is_scipy_hadamard(d):
    h = O.sylvester(d)
    assert np.array_equal(h, linalg.hadamard(d).astype(np.float64))
    assert np.array_equal(h @ h.T, d * np.eye(d))


def test_rht_is_orthogonal_and_inverted_by_its_transpose():
    g = synth.rng(3)
    d = 128
    s = synth.rht_signs(g, d)
    u = g.standard_normal((50, d))
    y = O.rht(u, s)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(u, axis=1), rtol=1e-14)
    assert np.allclose(O.rht_inverse(y, s), u, atol=1e-13)
    # explicit matrix: Pi = H diag(s) / sqrt(d)
    pi = O.sylvester(d) * s[None, :].astype(np.float64) / math.sqrt(d)
    assert np.allclose(y, u @ pi.T, atol=1e-13)
    assert np.allclose(pi @ pi.T, np.eye(d), atol=1e-13)
    # a basis vector spreads to +-1/sqrt(d) in every coordinate
    e = np.zeros((1, d)); e[0, 5] = 1
    assert np.allclose(np.abs(O.rht(e, s)), 1 / math.sqrt(d), atol=1e-15)


# ---------------------------------------------------------------- quantiser

def _nearest_bruteforce(y32, c):
    """argmin_k |y - c_k|; exact ties go to the larger |c_k|, and at y = 0
    to the positive centroid."""
    out = np.empty(y32.shape, dtype=np.int64)
    for i, v in enumerate(y32.ravel()):
        dist = np.abs(v - c)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:
            mags = np.abs(c[best])
            best = best[mags == mags.max()]
            best = best[c[best] >= 0] if len(best) > 1 else best
        out.ravel()[i] = best[0]
    return out


@pytest.mark.parametrize("d,m", [(128, 1), (128, 2), (128, 3), (128, 4), (8, 3), (2048, 2)])
def test_quantize_is_nearest_centroid(d, m):
    c, t, _, _ = O.lloyd_max(d, m)
    c32, t32 = O.codebook_f32(c, t)
    g = synth.rng(7)
    y = g.standard_normal(4000) / math.sqrt(d)
    # plus the thresholds themselves, their negatives, zero and -0
    y = np.concatenate([y, t32, -t32, [0.0, -0.0, 1.0, -1.0]])
    got = O.quantize(y, t32)
    # the threshold rule equals the nearest centroid (brute force over all
    # centroids, on the float64 y) wherever the float32 thresholds are the
    # midpoints of the float32 centroids, i.e. away from a 1e-7 band
    ref = _nearest_bruteforce(y, c32)
    mid_ok = np.abs(0.5 * (c32[:-1] + c32[1:]) - t32) <= 2 * np.spacing(np.abs(t32).astype(np.float32)).astype(np.float64) + 1e-30
    assert mid_ok.all()
    near = np.min(np.abs(y[:, None] - t32[None, :]), axis=1) < 1e-7
    assert np.array_equal(got[~near], ref[~near])
    # on exact thresholds the rule is: larger magnitude
    for k, tk in enumerate(t32):
        idx = O.quantize(np.array([tk]), t32)[0]
        if tk > 0:
            assert idx == k + 1
        elif tk < 0:
            assert idx == k
        else:
            assert idx == k + 1          # zero goes to the positive side


@pytest.mark.parametrize("m", [1, 2, 3])
def test_pack_unpack_bijection_all_patterns(m):
    # every pattern of the first 4 coordinates of an 8-coordinate row (the
    # other 4 fixed) packs to a distinct record and unpacks back
    k = 1 << m
    grids = np.stack(np.meshgrid(*[np.arange(k)] * 4, indexing="ij"), -1).reshape(-1, 4)
    rest = np.tile(np.array([[k - 1, 0, k // 2, 1 % k]]), (grids.shape[0], 1))
    rows = np.concatenate([grids, rest], axis=1)
    packed = O.pack_bits(rows, m)
    assert packed.shape == (k ** 4, m)
    assert len({p.tobytes() for p in packed}) == k ** 4
    assert np.array_equal(O.unpack_bits(packed, m, 8), rows)


@pytest.mark.parametrize("m,d", [(3, 8), (3, 32), (2, 64), (4, 128), (1, 128)])
def test_pack_is_little_endian_dense_stream(m, d):
    # The record, read as one little-endian integer, is sum_j idx_j 2^(m j).
    g = synth.rng(11)
    idx = g.integers(0, 1 << m, size=(5, d))
    packed = O.pack_bits(idx, m)
    for row, p in zip(idx, packed):
        value = sum(int(v) << (m * j) for j, v in enumerate(row))
        assert int.from_bytes(p.tobytes(), "little") == value
    # three 3-bit codes 1, 2, 3 ... 7, 0 in 24 bits
    assert list(O.pack_bits(np.array([[1, 2, 3, 4, 5, 6, 7, 0]]), 3)[0]) == [209, 88, 31]


# ------------------------------------------------------------ encode/decode

def _config1(seed=0, n=4096, d=128):
    g = synth.rng(seed)
    x = synth.gaussian(g, n, d)
    s = synth.rht_signs(g, d)
    return x, s


def test_rotated_coordinates_follow_lemma1():
    # Lemma 1 / video 05:32: after normalising and rotating, one coordinate
    # follows the Beta-type density; Kolmogorov-Smirnov against its CDF.
    x, s = _config1()
    c, t, _, _ = O.lloyd_max(128, 3)
    enc = O.encode_mse(x, 128, s, *O.codebook_f32(c, t))
    for j in (0, 77):
        ks = stats.kstest(enc["y"][:, j], lambda v: 1 - O.beta_upper_tail(v, 128))
        assert ks.pvalue > 0.01


def test_config1_distortion_matches_theorem():
    # Inputs i.i.d. N(0,1): Pi u is exactly uniform on the sphere, so the mean
    # ||u - u~||^2 equals d * C(f_X, b) (the MSE decomposition) up to
    # sampling error; it lies between the bounds of Theorem D_mse.
    d, b = 128, 3
    x, s = _config1()
    c, t, dmse, _ = O.lloyd_max(d, b)
    c32, t32 = O.codebook_f32(c, t)
    enc = O.encode_mse(x, d, s, c32, t32)
    xt = O.decode(enc["codes"], enc["norms"], d, d, s, c32)
    n = enc["norms"].astype(np.float64)
    u = x / n[:, None]
    err = np.sum((u - xt / n[:, None]) ** 2, axis=1)
    se = err.std() / math.sqrt(len(err))
    assert abs(err.mean() - dmse) < 4 * se
    assert 4.0 ** -b < err.mean() < math.sqrt(3) * math.pi / 2 * 4.0 ** -b
    # norms are kept exactly (float32 of ||x||)
    assert np.allclose(n, np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-7)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_one_hot_worst_case(b):
    # Forum post: a one-hot input is the RHT's worst case.  Every rotated
    # coordinate is +-1/sqrt(d), so ||u - u~||^2 = (1 - sqrt(d) c*)^2 with c*
    # the float32 centroid nearest 1/sqrt(d).
    d = 128
    g = synth.rng(5)
    s = synth.rht_signs(g, d)
    c, t, _, _ = O.lloyd_max(d, b)
    c32, t32 = O.codebook_f32(c, t)
    x = np.zeros((3, d), dtype=np.float32)
    x[0, 0] = 1.0; x[1, 100] = -2.5; x[2, 127] = 7.0
    enc = O.encode_mse(x, d, s, c32, t32)
    xt = O.decode(enc["codes"], enc["norms"], d, d, s, c32)
    n = np.abs(x).sum(axis=1)
    err = np.sum((x / n[:, None] - xt / n[:, None]) ** 2, axis=1)
    cstar = c32[np.argmin(np.abs(c32 - 1 / math.sqrt(d)))]
    assert np.allclose(err, (1 - math.sqrt(d) * cstar) ** 2, atol=1e-12)


def test_padding_and_zero_vector():
    d_in, d = 100, 128
    g = synth.rng(9)
    x = synth.gaussian(g, 6, d_in)
    x[2] = 0.0
    s = synth.rht_signs(g, d)
    c, t, _, _ = O.lloyd_max(d, 2)
    c32, t32 = O.codebook_f32(c, t)
    enc = O.encode_mse(x, d, s, c32, t32)
    assert enc["norms"][2] == 0.0
    assert np.all(enc["idx"][2] == 2)                 # y = 0 -> positive side
    xt = O.decode(enc["codes"], enc["norms"], d, d_in, s, c32)
    assert xt.shape == (6, d_in) and np.all(xt[2] == 0.0)
    # the pad is part of the rotation: zero-padding then rotating equals
    # rotating the padded vector
    xp = np.zeros((6, d)); xp[:, :d_in] = x
    enc2 = O.encode_mse(xp, d, s, c32, t32)
    assert np.array_equal(enc2["codes"], enc["codes"])


# ----------------------------------------------------------------- estimator

def test_estimator_equals_inner_product_with_decoded_vector():
    # <q, Q^-1(Q(x))> computed by rotating the query once equals the inner
    # product with the decoded (un-rotated) vector, for mse and prod.
    d, d_in = 128, 120
    g = synth.rng(21)
    x = synth.gaussian(g, 64, d_in)
    s = synth.rht_signs(g, d)
    _, sm = synth.qjl_matrix(g, d)
    q = synth.gaussian(g, 5, d_in).astype(np.float64)
    for mode in ("mse", "prod"):
        b = 3
        m = b if mode == "mse" else b - 1
        c, t, _, _ = O.lloyd_max(d, m)
        c32, t32 = O.codebook_f32(c, t)
        if mode == "mse":
            e = O.encode_mse(x, d, s, c32, t32)
            xt = O.decode(e["codes"], e["norms"], d, d_in, s, c32)
            est = O.score(q, e["codes"], e["norms"], d, s, c32)
        else:
            e = O.encode_prod(x, d, s, c32, t32, sm)
            xt = O.decode(e["codes"], e["norms"], d, d_in, s, c32, e["qjl"], e["rnorms"], sm)
            est = O.score(q, e["codes"], e["norms"], d, s, c32, e["qjl"], e["rnorms"], sm)
        assert np.allclose(est, q @ xt.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_mse_inner_product_bias_slope(b):
    # 2/pi paragraph: TurboQuant_mse shrinks inner products.  For isotropic
    # keys the regression slope of the estimate on <q, x> is
    # d * sum_k p_k c_k^2 = 1 - D_mse(b) (centroid condition + symmetry);
    # at b = 1 and large d this is 2/pi.
    d = 128
    g = synth.rng(30 + b)
    x = synth.gaussian(g, 20000, d)
    s = synth.rht_signs(g, d)
    q = g.standard_normal((1, d))
    c, t, dmse, _ = O.lloyd_max(d, b)
    c32, t32 = O.codebook_f32(c, t)
    e = O.encode_mse(x, d, s, c32, t32)
    est = O.score(q, e["codes"], e["norms"], d, s, c32)[0]
    true = x.astype(np.float64) @ q[0]
    slope = np.dot(est, true) / np.dot(true, true)
    resid = est - slope * true
    se = math.sqrt(np.dot(resid, resid) / (len(true) - 1) / np.dot(true, true))
    assert abs(slope - (1 - dmse)) < 5 * se + 2e-3
    if b == 1:
        assert abs((1 - O.lloyd_max(1 << 14, 1)[2]) - 2 / math.pi) < 1e-4


@pytest.mark.parametrize("b", [1, 2, 3])
def test_prod_is_unbiased_over_random_draws(b):
    # Theorem D_prod: E[<y, x~>] = <y, x> over the randomness (signs and S
    # redrawn), for a fixed pair; also the variance stays below the
    # Lemma 4 / Theorem D_prod scale (pi/(2d)) ||y||^2 D_mse(b-1).
    d = 128
    g = synth.rng(40 + b)
    x = synth.gaussian(g, 1, d)
    q = g.standard_normal((1, d))
    true = float(x.astype(np.float64)[0] @ q[0])
    m = b - 1
    if m:
        c, t, dm1, _ = O.lloyd_max(d, m)
        c32, t32 = O.codebook_f32(c, t)
    else:
        c32 = t32 = np.zeros(0)
        dm1 = 1.0
    reps = 600
    ests = np.empty(reps)
    for r in range(reps):
        s = synth.rht_signs(g, d)
        _, sm = synth.qjl_matrix(g, d)
        e = O.encode_prod(x, d, s, c32 if m else None, t32 if m else None, sm)
        ests[r] = O.score(q, e["codes"], e["norms"], d, s, c32 if m else None,
                          e["qjl"], e["rnorms"], sm)[0, 0]
    se = ests.std() / math.sqrt(reps)
    assert abs(ests.mean() - true) < 4.5 * se
    nx2 = float(np.sum(x.astype(np.float64) ** 2))
    bound = math.pi / (2 * d) * float(q[0] @ q[0]) * nx2 * dm1
    assert ests.var() < 1.3 * bound
    # Theorem D_prod's bound, with the garbled constant read as sqrt(3)*pi^2
    assert ests.var() < math.sqrt(3) * math.pi ** 2 * float(q[0] @ q[0]) * nx2 / d * 4.0 ** -b


def test_prod_slope_is_one_on_many_pairs():
    # Same statement over many keys under one draw of (signs, S): the OLS
    # slope of est on <q, x> is 1 (while mse at equal total bits is < 1).
    d = 128
    g = synth.rng(50)
    x = synth.gaussian(g, 8000, d)
    s = synth.rht_signs(g, d)
    _, sm = synth.qjl_matrix(g, d)
    q = g.standard_normal((1, d))
    c, t, _, _ = O.lloyd_max(d, 2)
    c32, t32 = O.codebook_f32(c, t)
    e = O.encode_prod(x, d, s, c32, t32, sm)
    est = O.score(q, e["codes"], e["norms"], d, s, c32, e["qjl"], e["rnorms"], sm)[0]
    true = x.astype(np.float64) @ q[0]
    slope = np.dot(est, true) / np.dot(true, true)
    resid = est - slope * true
    se = math.sqrt(np.dot(resid, resid) / (len(true) - 1) / np.dot(true, true))
    assert abs(slope - 1) < 5 * se


def test_qjl_lemma4_expectation():
    # Lemma 4: E_S[ sqrt(pi/2)/d * S^T sign(S r) ] = r / ||r|| for Gaussian S
    # (E[s sign<s, r>] = sqrt(2/pi) r/||r||); Monte Carlo over S.
    d = 32
    g = synth.rng(60)
    r = g.standard_normal(d)
    acc = np.zeros(d)
    reps = 4000
    for _ in range(reps):
        sm = g.standard_normal((d, d))
        z = np.where(sm @ r >= 0, 1.0, -1.0)
        acc += math.sqrt(math.pi / 2) / d * (sm.T @ z)
    acc /= reps
    assert np.allclose(acc, r / np.linalg.norm(r), atol=5 * math.sqrt(math.pi / 2 / d / reps))


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_rows_encode_as_the_zero_row(bad):
    # The pages leave non-finite input open; the reading taken is that a row
    # holding a NaN or an infinity has no norm: it is stored as the zero
    # row's record with the norm NaN, so it decodes to NaN and scores NaN,
    # while the other rows of the batch are untouched.
    d, m = 128, 2
    g = synth.rng(5)
    x = g.standard_normal((4, d))
    x[1] = 0.0
    x[2, 17] = bad
    signs = synth.rht_signs(g, d)
    _, s64 = synth.qjl_matrix(g, d)
    c, t, _, _ = O.lloyd_max(d, m)
    c32, t32 = O.codebook_f32(c, t)
    clean = np.delete(x, 2, axis=0)
    for enc in (lambda a: O.encode_mse(a, d, signs, c32, t32), lambda a: O.encode_prod(a, d, signs, c32, t32, s64)):
        r, ref = enc(x), enc(clean)
        assert np.isnan(r["norms"][2]) and np.all(np.isfinite(np.delete(r["norms"], 2)))
        assert np.array_equal(r["codes"][2], r["codes"][1])                    # the zero row's codes
        assert np.all(O.unpack_bits(r["codes"][2:3], m, d) == (1 << m) // 2)   # y = 0: positive side
        assert np.array_equal(np.delete(r["codes"], 2, axis=0), ref["codes"])
        if "qjl" in r:
            assert np.array_equal(r["qjl"][2], r["qjl"][1]) and r["rnorms"][2] == r["rnorms"][1]
    dec = O.decode(r["codes"], r["norms"], d, d, signs, c32, r["qjl"], r["rnorms"], s64)
    assert np.all(np.isnan(dec[2])) and np.all(np.isfinite(np.delete(dec, 2, axis=0)))
    est = O.score(g.standard_normal((2, d)), r["codes"], r["norms"], d, signs, c32, r["qjl"], r["rnorms"], s64)
    assert np.all(np.isnan(est[:, 2])) and np.all(np.isfinite(np.delete(est, 2, axis=1)))
