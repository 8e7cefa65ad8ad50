"""Pins of the oracle's block-diagonal rotations (the 2-D Givens and 4-D
quaternion rotations of the RotorQuant forum post) used in place of the
randomised Hadamard transform at equal bits."""

import math

import numpy as np
import pytest

import synth
from oracle import tq_oracle as O

D = 128


def _quat_mul(p, q):
    # Hamilton product (w, x, y, z), from i^2 = j^2 = k^2 = ijk = -1
    w1, x1, y1, z1 = p
    w2, x2, y2, z2 = q
    return np.array([w1 * w2 - x1 * x2 - y1 * y2 - z1 * z2,
                     w1 * x2 + x1 * w2 + y1 * z2 - z1 * y2,
                     w1 * y2 - x1 * z2 + y1 * w2 + z1 * x2,
                     w1 * z2 + x1 * y2 - y1 * x2 + z1 * w2])


def test_quaternion_block_is_the_left_hamilton_product():
    one, i, j, k = np.eye(4)
    r = O.block_rotation("quat", np.tile(i, (1, 1)), 4)
    assert np.allclose(r @ j, k) and np.allclose(r @ i, -one)       # i j = k, i i = -1
    rj = O.block_rotation("quat", j[None], 4)
    assert np.allclose(rj @ k, i) and np.allclose(rj @ i, -k)       # j k = i, j i = -k
    rng = np.random.default_rng(0)
    p, v = rng.standard_normal(4), rng.standard_normal(4)
    p /= np.linalg.norm(p)
    assert np.allclose(O.block_rotation("quat", p[None], 4) @ v, _quat_mul(p, v), atol=1e-15)


def test_givens_block_and_identities():
    r = O.block_rotation("givens", np.array([[0.0, 1.0]]), 2)         # 90 degrees
    assert np.allclose(r @ [1.0, 0.0], [0.0, 1.0]) and np.allclose(r @ [0.0, 1.0], [-1.0, 0.0])
    assert np.allclose(O.block_rotation("givens", np.tile([1.0, 0.0], (D // 2, 1)), D), np.eye(D))
    assert np.allclose(O.block_rotation("quat", np.tile([1.0, 0, 0, 0], (D // 4, 1)), D), np.eye(D))


@pytest.mark.parametrize("kind", ["givens", "quat"])
def test_block_rotations_are_orthogonal_and_inverted_by_the_transpose(kind):
    g = synth.rng(1)
    prm = synth.givens_params(g, D) if kind == "givens" else synth.quaternion_params(g, D)
    r = O.block_rotation(kind, prm, D)
    assert np.allclose(r.T @ r, np.eye(D), atol=1e-6)      # float32 parameters
    u = g.standard_normal((5, D))
    y = O.rht(u, (kind, prm))
    assert np.allclose(O.rht_inverse(y, (kind, prm)), u @ (r.T @ r), atol=1e-12)


@pytest.mark.parametrize("kind", ["rht", "givens", "quat"])
def test_isotropic_distortion_is_rotation_invariant(kind):
    # for i.i.d. Gaussian rows y = Pi x/||x|| is uniform on the sphere for any
    # orthogonal Pi, so the b = 3 distortion is D_mse(128, 3) within sampling error
    g = synth.rng(2)
    x = g.standard_normal((4000, D))
    spec = synth.rht_signs(g, D) if kind == "rht" else (
        kind, synth.givens_params(g, D) if kind == "givens" else synth.quaternion_params(g, D))
    c, t, dmse, _ = O.lloyd_max(D, 3)
    c32, t32 = O.codebook_f32(c, t)
    e = O.encode_mse(x, D, spec, c32, t32)
    xt = O.decode(e["codes"], e["norms"], D, D, spec, c32)
    n = np.linalg.norm(x, axis=1)
    err = np.sum(((x - xt) / n[:, None]) ** 2, axis=1)
    assert abs(err.mean() - dmse) < 4 * err.std() / math.sqrt(len(err)) + 2e-4


def test_one_hot_worst_case_favours_the_hadamard_rotation():
    # one-hot rows: the RHT spreads the energy over all 128 coordinates
    # (each +-1/sqrt d); a Givens pair keeps it in 2, a quaternion in 4, far
    # outside the codebook's range, so their distortion is much larger
    g = synth.rng(3)
    c, t, _, _ = O.lloyd_max(D, 3)
    c32, t32 = O.codebook_f32(c, t)
    x = np.eye(D)
    dist = {}
    for kind in ("rht", "givens", "quat"):
        spec = synth.rht_signs(g, D) if kind == "rht" else (
            kind, synth.givens_params(g, D) if kind == "givens" else synth.quaternion_params(g, D))
        e = O.encode_mse(x, D, spec, c32, t32)
        xt = O.decode(e["codes"], e["norms"], D, D, spec, c32)
        dist[kind] = float(np.mean(np.sum((x - xt) ** 2, axis=1)))
    assert dist["rht"] < 0.07
    assert dist["givens"] > 5 * dist["rht"] and dist["quat"] > 5 * dist["rht"]
