"""Helpers for the GPU parity tests: the oracle side of each comparison and
the acceptance rules.

Rules (from the accuracy target of the hot path):
  * codes and QJL sign bits are bit-exact except where the oracle's float64
    value lies within EPS = 1e-5 of a decision boundary (|y_j - t_k| for a
    code, |(S r)_i| / gamma for a QJL bit); such flips are counted and must
    stay below 1e-4 of all codes;
  * norms within 1e-6 relative; gamma within 1e-5 relative;
  * decoded vectors and scores within 1e-4 * (|ref| + floor) element-wise,
    floor = n / sqrt(d) for decoded coordinates and n ||q|| / sqrt(d) for
    scores, with the oracle evaluated on the GPU's records (so allowed
    boundary flips do not count twice).
"""

from __future__ import annotations

import functools
import math
import sys

import numpy as np

from oracle import tq_oracle as O

EPS = 1e-5
MAX_FLIP_FRACTION = 1e-4


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def codebook32(d: int, m: int):
    """The oracle's codebook for (d, m), rounded to float32 (as float64)."""
    # plain Lloyd needs ~1e5 iterations at m = 8; 1e-10 is far below the
    # float32 rounding the kernels use
    c, t, _, _ = O.lloyd_max(d, m, tol=1e-14 if m <= 6 else 1e-10)
    return O.codebook_f32(c, t)


def check_codes(gpu_codes: np.ndarray, y64: np.ndarray, ref_idx: np.ndarray, t32: np.ndarray, m: int,
                count_limit: bool = True):
    """Returns (gpu_idx, flips, near) after asserting the code rule.  The
    flip budget is statistical: inputs built to put many coordinates exactly
    on a boundary (constant rows rotate to exact zeros) pass count_limit=False
    and are held to the eps rule alone."""
    d = y64.shape[1]
    gi = O.unpack_bits(gpu_codes, m, d)
    diff = gi != ref_idx
    dist = np.full(y64.shape, np.inf)
    for tk in np.concatenate([t32, [0.0]]):
        dist = np.minimum(dist, np.abs(y64 - tk))
    near = int(np.sum(dist < EPS))
    flips = int(diff.sum())
    assert np.all(dist[diff] < EPS), f"{flips} code flips, {int(np.sum(dist[diff] >= EPS))} outside the eps band"
    if count_limit:
        assert flips <= MAX_FLIP_FRACTION * gi.size, f"{flips} flips of {gi.size} codes"
    return gi, flips, near


def check_norms(gpu: np.ndarray, ref: np.ndarray, rtol=1e-6):
    ref = np.asarray(ref, np.float64)
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    assert np.all(err <= rtol * np.abs(ref) + 1e-30), f"max rel err {np.max(err / np.maximum(np.abs(ref), 1e-30)):.3e}"


def check_qjl(gpu_qjl: np.ndarray, gpu_rnorms: np.ndarray, y64: np.ndarray, gpu_idx, c32, s64: np.ndarray):
    """QJL bits and gamma against r = y - c[idx] on the GPU's (checked) codes."""
    d = y64.shape[1]
    ymse = O.centroid_values(gpu_idx, c32) if c32 is not None and len(c32) else np.zeros_like(y64)
    r = y64 - ymse
    gamma = np.sqrt(np.sum(r * r, axis=1))
    sr = r @ s64.T
    zref = (sr >= 0.0).astype(np.int64)
    zg = O.unpack_bits(gpu_qjl, 1, d)
    diff = zg != zref
    rel = np.abs(sr) / np.maximum(gamma, 1e-30)[:, None]
    flips = int(diff.sum())
    assert np.all(rel[diff] < EPS), f"{flips} qjl flips, {int(np.sum(rel[diff] >= EPS))} outside the eps band"
    assert flips <= MAX_FLIP_FRACTION * zg.size
    err = np.abs(gpu_rnorms.astype(np.float64) - gamma)
    assert np.all(err <= 1e-5 * gamma + 1e-7), f"gamma max err {err.max():.3e}"
    return flips


def check_close(gpu: np.ndarray, ref: np.ndarray, floor, rtol=1e-4, what="values"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = rtol * (np.abs(ref) + floor)
    err = np.abs(gpu - ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"worst excess {np.max(err / np.maximum(bound, 1e-300)):.3f}x")


def decode_floor(norms: np.ndarray, d: int):
    return (np.asarray(norms, np.float64) / math.sqrt(d))[:, None]


def score_floor(norms: np.ndarray, q: np.ndarray, d: int):
    qn = np.linalg.norm(np.asarray(q, np.float64), axis=1)
    return qn[:, None] * np.asarray(norms, np.float64)[None, :] / math.sqrt(d)
