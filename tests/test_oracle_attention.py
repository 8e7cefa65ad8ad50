"""Pins of the oracle's decode attention (PolarQuant paper review, step 9:
softmax(K^ q / sqrt d) V^ on reconstructed keys and values) in cases whose
answer is fixed without the softmax code path: one token, equal scores,
one dominant key, and the GQA grouping."""

import math

import numpy as np

import synth
from oracle import tq_oracle as O

D = 128


def _setup(n, groups, seed, mode="mse", bk=2, bv=2):
    g = synth.rng(seed)
    k = synth.gaussian(g, groups * n, D).astype(np.float64)
    v = synth.gaussian(g, groups * n, D).astype(np.float64)
    ks, vs = synth.rht_signs(g, D), synth.rht_signs(g, D)
    s_bits, s64 = synth.qjl_matrix(g, D)
    mk = bk if mode == "mse" else bk - 1
    ck, tk = O.codebook_f32(*O.lloyd_max(D, mk)[:2])
    cv, tv = O.codebook_f32(*O.lloyd_max(D, bv)[:2])
    if mode == "mse":
        ek = O.encode_mse(k, D, ks, ck, tk)
        keys = {"codes": ek["codes"], "norms": ek["norms"], "signs": ks, "centroids": ck}
    else:
        ek = O.encode_prod(k, D, ks, ck, tk, s64)
        keys = {"codes": ek["codes"], "norms": ek["norms"], "qjl": ek["qjl"], "rnorms": ek["rnorms"],
                "signs": ks, "centroids": ck, "s": s64}
    ev = O.encode_mse(v, D, vs, cv, tv)
    values = {"codes": ev["codes"], "norms": ev["norms"], "signs": vs, "centroids": cv}
    return g, keys, values


def test_single_token_returns_its_reconstructed_value():
    g, keys, values = _setup(1, 3, seed=1)
    q = g.standard_normal((3 * 2, D))
    out = O.decode_attention(q, 3, keys, values, D, D, 1 / math.sqrt(D))
    xv = O.decode(values["codes"], values["norms"], D, D, values["signs"], values["centroids"])
    for gi in range(3):
        assert np.allclose(out[2 * gi:2 * gi + 2], xv[gi], atol=1e-12)


def test_zero_scale_is_the_mean_of_the_reconstructed_values():
    g, keys, values = _setup(37, 2, seed=2, mode="prod", bk=3)
    q = g.standard_normal((2 * 4, D))
    out = O.decode_attention(q, 2, keys, values, D, D, 0.0)
    xv = O.decode(values["codes"], values["norms"], D, D, values["signs"], values["centroids"])
    assert np.allclose(out[:4], xv[:37].mean(axis=0), atol=1e-12)
    assert np.allclose(out[4:], xv[37:].mean(axis=0), atol=1e-12)


def test_dominant_key_takes_all_the_weight():
    # a query parallel to one key's reconstruction and a large scale: the
    # softmax weight concentrates on that key (the limit of the definition)
    g, keys, values = _setup(50, 1, seed=3, bk=4)
    xk = O.decode(keys["codes"], keys["norms"], D, D, keys["signs"], keys["centroids"])
    est = xk @ xk[17]
    assert np.argmax(est) == 17
    out = O.decode_attention(xk[17:18], 1, keys, values, D, D, 1e4)
    xv = O.decode(values["codes"], values["norms"], D, D, values["signs"], values["centroids"])
    assert np.allclose(out[0], xv[17], atol=1e-9)


def test_weights_follow_the_estimator_and_groups_are_independent():
    # two tokens: out = p0 v0 + p1 v1 with p1 / p0 = exp(scale * (e1 - e0)),
    # e the inner product with the reconstructed key (estimator identity);
    # shuffling another group's tokens leaves a group's output unchanged
    g, keys, values = _setup(2, 2, seed=4)
    q = g.standard_normal((2, D))
    out = O.decode_attention(q, 2, keys, values, D, D, 0.3)
    xk = O.decode(keys["codes"], keys["norms"], D, D, keys["signs"], keys["centroids"])
    xv = O.decode(values["codes"], values["norms"], D, D, values["signs"], values["centroids"])
    e = np.array([q[0] @ xk[0], q[0] @ xk[1]])
    p1 = 1.0 / (1.0 + math.exp(-0.3 * (e[1] - e[0])))
    assert np.allclose(out[0], (1 - p1) * xv[0] + p1 * xv[1], atol=1e-10)
    per_token = ("codes", "norms", "qjl", "rnorms")
    perm = {k: (v[[0, 1, 3, 2]] if k in per_token else v) for k, v in keys.items()}
    permv = {k: (v[[0, 1, 3, 2]] if k in per_token else v) for k, v in values.items()}
    out2 = O.decode_attention(q, 2, perm, permv, D, D, 0.3)
    assert np.allclose(out2, out, atol=1e-12)
