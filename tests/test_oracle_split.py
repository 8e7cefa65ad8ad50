"""Pins of the oracle's outlier-channel split (the paper summary's KV-cache
setting: outlier channels quantised at more bits, each channel set by its
own instance)."""

import numpy as np

import synth
from oracle import tq_oracle as O


def _cb(d, m):
    c, t, _, _ = O.lloyd_max(d, m)
    return O.codebook_f32(c, t)


def _part(g, c0, d_in, b):
    d = max(32, 1 << (d_in - 1).bit_length())
    c, t = _cb(d, b)
    return {"c0": c0, "d_in": d_in, "d": d, "rot": synth.rht_signs(g, d), "centroids": c, "thresholds": t}


def _dist(x, xt):
    return float(np.mean(np.sum((x - xt) ** 2, axis=1) / np.sum(x ** 2, axis=1)))


def test_one_part_is_the_plain_quantiser():
    g = synth.rng(1)
    x = synth.gaussian(g, 50, 128).astype(np.float64)
    p = _part(g, 0, 128, 3)
    enc = O.split_encode(x, [p])
    plain = O.encode_mse(x, 128, p["rot"], p["centroids"], p["thresholds"])
    assert np.array_equal(enc[0]["codes"], plain["codes"])
    q = g.standard_normal((3, 128))
    assert np.allclose(O.split_score(q, enc, [p]),
                       O.score(q, plain["codes"], plain["norms"], 128, p["rot"], p["centroids"]), atol=1e-12)


def test_split_estimate_is_the_inner_product_with_the_split_reconstruction():
    g = synth.rng(2)
    x = synth.with_outliers(synth.gaussian(g, 40, 128)).astype(np.float64)
    parts = [_part(g, 0, 32, 3), _part(g, 32, 96, 2)]
    enc = O.split_encode(x, parts)
    xt = O.split_decode(enc, parts)
    q = g.standard_normal((4, 128))
    assert np.allclose(O.split_score(q, enc, parts), q @ xt.T, atol=1e-10)


def test_outlier_split_beats_uniform_bits_on_outlier_channels():
    # four channels x 20 dominate the norm; giving the 32 channels that hold
    # them one more bit (2.25 bits on average) more than halves the uniform
    # 2-bit distortion, and 32 x 4 + 96 x 3 bits more than halves 3 bits
    g = synth.rng(3)
    x = synth.with_outliers(synth.gaussian(g, 2000, 128)).astype(np.float64)
    uni = {}
    for b in (2, 3):
        p = _part(g, 0, 128, b)
        uni[b] = _dist(x, O.split_decode(O.split_encode(x, [p]), [p]))
    for b_out, b_rest, ref in ((3, 2, 2), (4, 3, 3)):
        parts = [_part(g, 0, 32, b_out), _part(g, 32, 96, b_rest)]
        dist = _dist(x, O.split_decode(O.split_encode(x, parts), parts))
        assert dist < uni[ref] / 2, (b_out, b_rest, dist, uni[ref])
