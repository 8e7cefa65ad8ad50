"""CPU oracle for the TurboQuant online vector quantiser.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
constants with the HIP library; random inputs (signs, S, data) are passed in.

Everything is plain numpy/scipy in float64 with scalar-style steps in the
order the sources give them.  Sources (cited by title and section):

* [TQ-sum]  "TurboQuant: Online Vector Quantization" paper summary
  (Jump2Paper Archive, arXiv 2504.19874): Lemma 1 (Beta marginal), the
  definitions table (Q, Q^-1, B = b*d bits), the MSE decomposition into a
  1-D k-means problem, Theorem "D_mse" (bound and the numerics
  0.36/0.117/0.03/0.009), Definition 1 (QJL map) and the QJL dequantiser
  with Lemma 4, Theorem "D_prod" (unbiasedness, residual QJL), the 1-bit
  2/pi bias paragraph, the experiment-setup table (precomputed Max-Lloyd
  codebooks for b = 1..8).
* [TQ-video] AI Trends summary of the TurboQuant video: chapter 04:24
  (L2 normalise, then multiply by the RHT matrix), 05:32 (Beta
  distribution), 06:06 (quantise in the transformed domain, undo by the
  transpose and the stored norm).
* [HN] GeekNews translation of the Hacker News thread: the SRHT remark
  (O(d log d) rotation) and the remark that queries are un-rotated.
* [RQ] damoang forum post on RotorQuant: block-diagonal 2-D Givens
  (PlanarQuant) and 4-D quaternion (IsoQuant) rotations in place of the
  Hadamard butterflies; on a one-hot input they keep the energy in a few
  coordinates where the RHT spreads it over all of them.
* [PQ-rev] 모두의 AI review of PolarQuant, step 9 (into attention): the
  reconstructed keys and values go into the usual scaled attention
  softmax(K^ q / sqrt d) V^.

Readings of points the sources leave open (each one is listed in the
design notes of the repository):

* Rotation: Pi = (1/sqrt d) * H * D with H the natural-order Sylvester
  Hadamard matrix and D = diag(signs); Pi^-1 = Pi^T = (1/sqrt d) * D * H.
* Inputs of dimension d_in < d are zero-padded to d (a power of two).
* The norm is kept separately in float32; the zero vector encodes u = 0.
  A row holding a NaN or an infinity is encoded as the zero row with the
  norm NaN (so it decodes to NaN and scores NaN).
* The codebook is the Lloyd-Max quantiser of the Lemma 1 density at the
  padded d, exactly symmetric.  The quantiser in use is its float32
  rounding (an input here, as the random parameters are).
* Bucket rule: nearest centroid; a coordinate that sits exactly on a
  threshold goes to the centroid of larger magnitude, and y = 0 goes to the
  positive side (the quantiser is an odd function).  Decisions are taken on
  the float64 y itself.
* TurboQuant_prod: m = b - 1 bits of mse code, residual r = y - c[idx] in the
  rotated domain, gamma = ||r||, QJL bit i = [(S r)_i >= 0] (sign(0) = +1),
  dequantised as gamma * sqrt(pi/2)/d * S^T z.  S is an input; the library
  stores it as bfloat16, so callers pass S already rounded to bfloat16.
* Record layout: dense m-bit codes, coordinate j's code in bits
  [m*j, m*j + m) of a little-endian bit stream (bit s is bit s%8 of byte
  s//8); the QJL plane holds bit i at stream position i.
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import betainc, gammaln

__all__ = [
    "beta_log_norm", "beta_pdf", "beta_upper_tail", "cell_moments",
    "lloyd_max", "codebook_f32", "sylvester", "block_rotation", "rht", "rht_inverse",
    "quantize", "centroid_values", "pack_bits", "unpack_bits",
    "encode_mse", "encode_prod", "decode", "score", "rotate_query",
    "decode_attention", "topk", "split_encode", "split_decode", "split_score", "QJL_SCALE",
]

# sqrt(pi/2): the QJL dequantiser scale of Definition 1 / Lemma 4 [TQ-sum].
QJL_SCALE = math.sqrt(math.pi / 2.0)


# --------------------------------------------------------------------------
# Lemma 1 [TQ-sum]: one coordinate of a uniform point on S^{d-1} has density
#   f_X(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2).
# --------------------------------------------------------------------------

def beta_log_norm(d: int) -> float:
    """log of the Lemma 1 normaliser Gamma(d/2)/(sqrt(pi) Gamma((d-1)/2))."""
    return gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)


def beta_pdf(x, d: int):
    """Lemma 1 density f_X at x (zero outside (-1, 1)); needs d >= 3."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    inside = np.abs(x) < 1.0
    xi = x[inside]
    out[inside] = np.exp(beta_log_norm(d) + 0.5 * (d - 3) * np.log1p(-xi * xi))
    return out


def beta_upper_tail(x, d: int):
    """P(X > x) for the Lemma 1 density.

    (1 + X)/2 follows Beta((d-1)/2, (d-1)/2), so P(X > x) equals the
    regularised incomplete beta function at (1 - x)/2.
    """
    a = 0.5 * (d - 1)
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    return betainc(a, a, 0.5 * (1.0 - x))


def _pow_one_minus_sq(x, e):
    """(1 - x^2)^e, computed in log space (0 at |x| = 1)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    inside = np.abs(x) < 1.0
    xi = x[inside]
    out[inside] = np.exp(e * np.log1p(-xi * xi))
    return out


def cell_moments(lo, hi, d: int):
    """Zeroth, first and second moments of f_X over the cells [lo, hi].

    M0 = int f,  M1 = int x f,  M2 = int x^2 f, with 0 <= lo < hi <= 1.
    M1 follows from d/dx (1-x^2)^((d-1)/2) = -(d-1) x (1-x^2)^((d-3)/2);
    M2 from one more integration by parts, which leaves the Lemma 1 density
    of dimension d+2 (exponent (d-1)/2).
    """
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    c_d = math.exp(beta_log_norm(d))
    c_d2 = math.exp(beta_log_norm(d + 2))
    m0 = beta_upper_tail(lo, d) - beta_upper_tail(hi, d)
    p_lo = _pow_one_minus_sq(lo, 0.5 * (d - 1))
    p_hi = _pow_one_minus_sq(hi, 0.5 * (d - 1))
    m1 = c_d / (d - 1) * (p_lo - p_hi)
    mass_d2 = beta_upper_tail(lo, d + 2) - beta_upper_tail(hi, d + 2)
    m2 = c_d / (d - 1) * (lo * p_lo - hi * p_hi + mass_d2 / c_d2)
    return m0, m1, m2


# --------------------------------------------------------------------------
# Lloyd-Max codebook: the MSE decomposition of [TQ-sum] reduces D_mse to
# d * C(f_X, b), the 1-D continuous k-means cost on f_X; the setup table
# says the codebooks are found by numerical Max-Lloyd optimisation.
# --------------------------------------------------------------------------

def lloyd_max(d: int, m: int, tol: float = 1e-14, max_iter: int = 2_000_000):
    """Lloyd-Max quantiser with 2^m levels for the Lemma 1 density.

    Returns (centroids[2^m], thresholds[2^m - 1], D_mse, iterations), all
    float64.  f_X is even, so the optimum is odd-symmetric: the iteration
    runs on the positive half (cells [t_k, t_{k+1}] with t_0 = 0, last edge
    1) and the negative half is its mirror.  One iteration = thresholds at
    midpoints of neighbouring centroids, then centroids = conditional means.
    D_mse = d * sum_k int_cell (x - c_k)^2 f_X.
    """
    if d < 3:
        raise ValueError("the Lemma 1 density needs d >= 3")
    if not 1 <= m <= 8:
        raise ValueError("m must be in 1..8")
    half = 1 << (m - 1)
    # Start from equal-mass cells on the positive half.
    grid = np.linspace(0.0, 1.0, 200001)
    tail = beta_upper_tail(grid, d)          # decreasing from 0.5 to 0
    targets = 0.5 * (1.0 - np.arange(1, half) / half)
    inner = np.interp(-targets, -tail, grid) if half > 1 else np.zeros(0)
    edges = np.concatenate(([0.0], inner, [1.0]))
    m0, m1, _ = cell_moments(edges[:-1], edges[1:], d)
    c = m1 / m0
    it = 0
    prev = None
    for it in range(1, max_iter + 1):
        edges = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
        m0, m1, _ = cell_moments(edges[:-1], edges[1:], d)
        c_new = m1 / m0
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        # The iteration converges linearly; with rho = delta/prev the error
        # left after this step is about delta * rho / (1 - rho).
        if delta <= 4e-17:
            break
        if prev is not None and prev > 0.0:
            rho = min(delta / prev, 1.0 - 1e-12)
            if delta * rho / (1.0 - rho) < tol:
                break
        prev = delta
    edges = np.concatenate(([0.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
    m0, m1, m2 = cell_moments(edges[:-1], edges[1:], d)
    cost_half = np.sum(m2 - 2.0 * c * m1 + c * c * m0)
    dmse = d * 2.0 * cost_half
    centroids = np.concatenate((-c[::-1], c))
    thresholds = np.concatenate((-edges[1:-1][::-1], [0.0], edges[1:-1]))
    return centroids, thresholds, float(dmse), it


def codebook_f32(centroids, thresholds):
    """The float32 rounding of a codebook, as float64 arrays (what the
    kernels hold)."""
    return (np.asarray(centroids, np.float32).astype(np.float64),
            np.asarray(thresholds, np.float32).astype(np.float64))


# --------------------------------------------------------------------------
# Randomised Hadamard rotation [TQ-video 04:24, 06:06], [HN SRHT remark].
# --------------------------------------------------------------------------

def sylvester(d: int) -> np.ndarray:
    """Natural-order Sylvester Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d, dtype=np.int64)
    both = np.bitwise_and.outer(i, i)
    parity = np.zeros_like(both)
    for bit in range(d.bit_length()):
        parity ^= (both >> bit) & 1
    return np.where(parity == 1, -1.0, 1.0)


_H_CACHE: dict[int, np.ndarray] = {}


def _h(d: int) -> np.ndarray:
    if d not in _H_CACHE:
        _H_CACHE[d] = sylvester(d)
    return _H_CACHE[d]


def block_rotation(kind, params, d):
    """The block-diagonal rotations the RotorQuant forum post describes
    [RQ]: "givens" -- one 2-D rotation [[c, -s], [s, c]] per coordinate pair
    (2i, 2i+1), params [d/2, 2] = (cos, sin); "quat" -- per coordinate quad
    4i..4i+3 the left product p * v with the unit quaternion p = (w, x, y, z)
    (params [d/4, 4]), written as its 4 x 4 matrix.  Returns R [d, d]."""
    prm = np.asarray(params, dtype=np.float64)
    r = np.zeros((d, d))
    if kind == "givens":
        for i, (c, s) in enumerate(prm.reshape(-1, 2)):
            r[2 * i:2 * i + 2, 2 * i:2 * i + 2] = [[c, -s], [s, c]]
    elif kind == "quat":
        for i, (w, x, y, z) in enumerate(prm.reshape(-1, 4)):
            r[4 * i:4 * i + 4, 4 * i:4 * i + 4] = [[w, -x, -y, -z],
                                                   [x, w, -z, y],
                                                   [y, z, w, -x],
                                                   [z, -y, x, w]]
    else:
        raise ValueError(kind)
    return r


def _is_block(spec):
    return isinstance(spec, tuple) and len(spec) == 2 and isinstance(spec[0], str)


def rht(u, signs):
    """y = Pi u for each row of u ([n, d] float64).  signs: the RHT sign
    vector, Pi = (1/sqrt d) * H * diag(signs); or a block rotation
    (kind, params) of ``block_rotation``."""
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    if _is_block(signs):
        return u @ block_rotation(signs[0], signs[1], d).T
    s = np.asarray(signs, dtype=np.float64)
    return (u * s) @ _h(d).T / math.sqrt(d)


def rht_inverse(y, signs):
    """u = Pi^T y: for the RHT (1/sqrt d) * signs * (H * y) (H symmetric);
    for a block rotation the transpose of its matrix."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    if _is_block(signs):
        return y @ block_rotation(signs[0], signs[1], d)
    s = np.asarray(signs, dtype=np.float64)
    return (y @ _h(d).T) / math.sqrt(d) * s


def _pad(x, d):
    x = np.asarray(x).astype(np.float64)
    if x.ndim == 1:
        x = x[None, :]
    n, d_in = x.shape
    if d_in > d:
        raise ValueError("d_in > d")
    out = np.zeros((n, d), dtype=np.float64)
    out[:, :d_in] = x
    return out


def _normalise(xp):
    """n = ||x||_2 (rounded to float32, as stored) and u = x / n (u = 0 when
    n = 0) [TQ-video 04:24].  A row holding a NaN or an infinity has no
    norm: it is stored with n = NaN and encoded as the zero row (u = 0)."""
    finite = np.all(np.isfinite(xp), axis=1)
    safe = np.where(finite[:, None], xp, 0.0)
    n64 = np.sqrt(np.sum(safe * safe, axis=1))
    u = np.zeros_like(xp)
    nz = n64 > 0
    u[nz] = safe[nz] / n64[nz, None]
    n64[~finite] = np.nan
    return n64.astype(np.float32), u


# --------------------------------------------------------------------------
# Scalar quantiser and bit packing [TQ-sum definitions table: Q maps R^d to
# {0,1}^{b*d}].
# --------------------------------------------------------------------------

def quantize(y, thresholds):
    """Bucket index of each coordinate of y (any shape), nearest centroid.

    ``thresholds`` are the 2^m - 1 ascending (float32-valued) midpoints of a
    symmetric codebook.  The decision is taken on y as given (float64).  With
    K = 2^m and L = #{positive thresholds t : |y| >= t}:
    idx = K/2 + L for y >= 0 and idx = K/2 - 1 - L for y < 0, i.e. ties go
    to the centroid of larger magnitude and y = 0 to the positive side.
    """
    t = np.asarray(thresholds, dtype=np.float64)
    k = t.size + 1
    half = k // 2
    tpos = t[half:]                       # thresholds above the middle one
    y64 = np.asarray(y, dtype=np.float64)
    mag = np.abs(y64)
    level = np.zeros(y64.shape, dtype=np.int64)
    for tk in tpos:
        level += (mag >= tk)
    return np.where(y64 >= 0.0, half + level, half - 1 - level)


def centroid_values(idx, centroids):
    return np.asarray(centroids, dtype=np.float64)[np.asarray(idx)]


def pack_bits(fields, width: int) -> np.ndarray:
    """Pack rows of non-negative ints, ``width`` bits each, as a dense
    little-endian bit stream: field j of a row occupies stream bits
    [width*j, width*j + width), bit p of the field at stream bit width*j+p,
    stream bit s at bit s % 8 of byte s // 8.  Returns uint8 [n, bytes]."""
    fields = np.asarray(fields, dtype=np.int64)
    if fields.ndim == 1:
        fields = fields[None, :]
    n, cnt = fields.shape
    nbits = width * cnt
    if nbits % 8:
        raise ValueError("row does not fill whole bytes")
    out = np.zeros((n, nbits // 8), dtype=np.uint8)
    for j in range(cnt):
        for p in range(width):
            s = width * j + p
            bit = ((fields[:, j] >> p) & 1).astype(np.uint8)
            out[:, s >> 3] |= bit << (s & 7)
    return out


def unpack_bits(packed, width: int, cnt: int) -> np.ndarray:
    """Inverse of pack_bits: uint8 [n, bytes] -> int64 [n, cnt]."""
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.ndim == 1:
        packed = packed[None, :]
    n = packed.shape[0]
    out = np.zeros((n, cnt), dtype=np.int64)
    for j in range(cnt):
        for p in range(width):
            s = width * j + p
            bit = (packed[:, s >> 3] >> (s & 7)) & 1
            out[:, j] |= bit.astype(np.int64) << p
    return out


# --------------------------------------------------------------------------
# TurboQuant_mse and TurboQuant_prod [TQ-sum: the two variants, Theorem
# D_mse, Definition 1, Theorem D_prod; TQ-video 04:24..06:06].
# --------------------------------------------------------------------------

def encode_mse(x, d, signs, centroids, thresholds):
    """TurboQuant_mse encode.

    x: [n, d_in] (any float dtype, widened exactly).  Returns a dict with
    codes (uint8 [n, m*d/8]), norms (float32 [n]), and the diagnostics the
    parity harness needs: y (float64 rotated unit vectors) and idx.
    """
    m = int(round(math.log2(len(centroids))))
    xp = _pad(x, d)
    norms, u = _normalise(xp)
    y = rht(u, signs)
    idx = quantize(y, thresholds)
    return {"codes": pack_bits(idx, m), "norms": norms, "y": y, "idx": idx}


def encode_prod(x, d, signs, centroids, thresholds, s_matrix):
    """TurboQuant_prod encode with m = b - 1 mse bits (centroids of 2^m
    levels; m = 0 means an empty codebook and a pure QJL code).

    r = y - c[idx] (rotated domain), gamma = ||r||_2, z_i = [(S r)_i >= 0].
    Returns codes, qjl (uint8 [n, d/8]), norms, rnorms (float32) and the
    diagnostics y, idx, sr (= S r, float64).
    """
    xp = _pad(x, d)
    norms, u = _normalise(xp)
    y = rht(u, signs)
    if centroids is None or len(centroids) == 0:
        m = 0
        idx = np.zeros(y.shape, dtype=np.int64)
        ymse = np.zeros_like(y)
        codes = np.zeros((y.shape[0], 0), dtype=np.uint8)
    else:
        m = int(round(math.log2(len(centroids))))
        idx = quantize(y, thresholds)
        ymse = centroid_values(idx, centroids)
        codes = pack_bits(idx, m)
    r = y - ymse
    gamma = np.sqrt(np.sum(r * r, axis=1))
    s = np.asarray(s_matrix, dtype=np.float64)
    sr = r @ s.T
    z = (sr >= 0.0).astype(np.int64)
    return {"codes": codes, "qjl": pack_bits(z, 1), "norms": norms,
            "rnorms": gamma.astype(np.float32), "y": y, "idx": idx, "sr": sr}


def decode(codes, norms, d, d_in, signs, centroids, qjl=None, rnorms=None,
           s_matrix=None):
    """Q^-1: y~ = c[idx] (+ gamma * sqrt(pi/2)/d * S^T z for prod), then
    x~ = n * Pi^T y~ truncated to d_in [TQ-sum Q^-1 and QJL dequantiser;
    TQ-video 06:06]."""
    norms = np.asarray(norms, dtype=np.float64)
    n = norms.shape[0]
    if centroids is not None and len(centroids) > 0:
        m = int(round(math.log2(len(centroids))))
        idx = unpack_bits(codes, m, d)
        yt = centroid_values(idx, centroids)
    else:
        yt = np.zeros((n, d), dtype=np.float64)
    if qjl is not None:
        z = 2.0 * unpack_bits(qjl, 1, d) - 1.0
        s = np.asarray(s_matrix, dtype=np.float64)
        g = np.asarray(rnorms, dtype=np.float64)
        yt = yt + (g * QJL_SCALE / d)[:, None] * (z @ s)
    xt = rht_inverse(yt, signs) * norms[:, None]
    return xt[:, :d_in]


def rotate_query(q, d, signs):
    """q' = Pi q_pad: the query is rotated once instead of un-rotating every
    key ([HN]: queries are un-rotated; Pi orthogonal)."""
    return rht(_pad(q, d), signs)


def score(q, codes, norms, d, signs, centroids, qjl=None, rnorms=None,
          s_matrix=None):
    """Inner-product estimates <q, Q^-1(Q(x))> for every (query, key).

    est = n * ( sum_j q'_j c[idx_j]
                + gamma * sqrt(pi/2)/d * sum_i (S q')_i z_i )
    with q' = Pi q.  Returns float64 [nq, n]."""
    qr = rotate_query(q, d, signs)
    norms = np.asarray(norms, dtype=np.float64)
    n = norms.shape[0]
    if centroids is not None and len(centroids) > 0:
        m = int(round(math.log2(len(centroids))))
        idx = unpack_bits(codes, m, d)
        est = qr @ centroid_values(idx, centroids).T
    else:
        est = np.zeros((qr.shape[0], n), dtype=np.float64)
    if qjl is not None:
        z = 2.0 * unpack_bits(qjl, 1, d) - 1.0
        s = np.asarray(s_matrix, dtype=np.float64)
        sq = qr @ s.T
        g = np.asarray(rnorms, dtype=np.float64)
        est = est + (sq @ z.T) * (g * QJL_SCALE / d)[None, :]
    return est * norms[None, :]


def decode_attention(q, groups, keys, values, d, d_in, scale):
    """Scaled attention over reconstructed keys and values [PQ-rev step 9]
    with grouped query heads: query row g*nq + i attends over the n tokens of
    KV group g,
        s_t = scale * <q, Q^-1(key_t)>   (the estimator of ``score``),
        p = softmax(s),   out = sum_t p_t Q^-1(value_t)   (``decode``).
    keys: dict with codes, norms, signs, centroids (+ qjl, rnorms, s for
    TurboQuant_prod keys); values: dict with codes, norms, signs, centroids
    (TurboQuant_mse).  Returns float64 [groups*nq, d_in]."""
    q = np.asarray(q, dtype=np.float64)
    nq = q.shape[0] // groups
    n = np.asarray(keys["norms"]).shape[0] // groups
    out = np.zeros((groups * nq, d_in), dtype=np.float64)
    for g in range(groups):
        ks = slice(g * n, (g + 1) * n)
        qs = q[g * nq:(g + 1) * nq]
        est = score(qs, keys["codes"][ks] if keys.get("codes") is not None else None,
                    keys["norms"][ks], d, keys["signs"], keys["centroids"],
                    keys["qjl"][ks] if keys.get("qjl") is not None else None,
                    keys["rnorms"][ks] if keys.get("rnorms") is not None else None,
                    keys.get("s"))
        sc = scale * est
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        p = w / w.sum(axis=1, keepdims=True)
        xv = decode(values["codes"][ks], values["norms"][ks], d, d_in, values["signs"],
                    values["centroids"])
        out[g * nq:(g + 1) * nq] = p @ xv
    return out


def topk(est, k):
    """Nearest-neighbour search on the estimates [TQ-sum, search
    application]: per row the k largest values, larger first, equal values
    by smaller key index, NaN never selected; rows with fewer than k
    candidates end in index -1, value -inf.  Returns (idx int64 [rows, k],
    vals float64 [rows, k])."""
    est = np.asarray(est, dtype=np.float64)
    rows, n = est.shape
    idx = np.full((rows, k), -1, dtype=np.int64)
    vals = np.full((rows, k), -np.inf)
    keys = np.arange(n)
    for r in range(rows):
        ok = ~np.isnan(est[r])
        cand = keys[ok]
        order = cand[np.lexsort((cand, -est[r][ok]))][:k]
        idx[r, :len(order)] = order
        vals[r, :len(order)] = est[r][order]
    return idx, vals


# --------------------------------------------------------------------------
# Outlier-channel split [TQ-sum experiment setup: a set of outlier channels
# quantised at more bits than the rest, as two independent instances].
# parts: list of dicts with "c0" (first column), "d_in", "d", "rot" (RHT
# signs or a block rotation), "centroids", "thresholds"; TurboQuant_mse.
# --------------------------------------------------------------------------

def split_encode(x, parts):
    x = np.asarray(x, dtype=np.float64)
    return [encode_mse(x[:, p["c0"]:p["c0"] + p["d_in"]], p["d"], p["rot"], p["centroids"], p["thresholds"])
            for p in parts]


def split_decode(encs, parts):
    cols = [decode(e["codes"], e["norms"], p["d"], p["d_in"], p["rot"], p["centroids"])
            for e, p in zip(encs, parts)]
    return np.concatenate(cols, axis=1)


def split_score(q, encs, parts):
    """The split estimate: the sum of every part's estimate on its columns."""
    q = np.asarray(q, dtype=np.float64)
    return sum(score(q[:, p["c0"]:p["c0"] + p["d_in"]], e["codes"], e["norms"], p["d"], p["rot"],
                     p["centroids"]) for e, p in zip(encs, parts))
