"""Seeded synthetic inputs shared by the tests and the benchmark.

This module only draws random numbers; it holds none of the quantiser's
arithmetic.  Both the HIP path and the CPU oracle receive the arrays drawn
here, including the random parameters of the method (the RHT sign vector and
the QJL matrix S), so the two sides never need a common random generator.

Draw order within one workload: data, then signs, then S, then queries.

Workload shapes follow the configurations the library is measured on:
  * gaussian rows N(0, 1) (the d = 128 mse case),
  * keys with four fixed outlier channels {0, 1, 2, 3} scaled by 20,
  * a KV cache whose channels carry scales drawn log-uniformly in [0.1, 10]
    per (tensor, head, channel),
  * clustered unit-norm database rows (centres g/||g||, per-coordinate noise
    sigma/sqrt(d_in) with sigma = 0.1, renormalised).
"""

from __future__ import annotations

import numpy as np

OUTLIER_CHANNELS = (0, 1, 2, 3)
OUTLIER_SCALE = 20.0


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def gaussian(g: np.random.Generator, n: int, d: int, dtype=np.float32):
    """[n, d] i.i.d. N(0, 1) in float32, then cast to ``dtype``."""
    return g.standard_normal((n, d), dtype=np.float32).astype(dtype)


def with_outliers(x: np.ndarray) -> np.ndarray:
    """Scale the fixed outlier channels by 20 (in float32, then cast back)."""
    y = x.astype(np.float32)
    y[..., list(OUTLIER_CHANNELS)] *= OUTLIER_SCALE
    return y.astype(x.dtype)


def rht_signs(g: np.random.Generator, d: int) -> np.ndarray:
    """int8 [d] of independent fair +-1 draws (the RHT diagonal)."""
    return np.where(g.integers(0, 2, size=d) == 1, 1, -1).astype(np.int8)


def givens_params(g: np.random.Generator, d: int) -> np.ndarray:
    """float32 [d/2, 2]: (cos, sin) of an angle drawn uniformly in [0, 2 pi)
    per coordinate pair."""
    th = g.uniform(0.0, 2.0 * np.pi, size=d // 2)
    return np.stack([np.cos(th), np.sin(th)], axis=1).astype(np.float32)


def quaternion_params(g: np.random.Generator, d: int) -> np.ndarray:
    """float32 [d/4, 4]: a uniform unit quaternion (w, x, y, z) per
    coordinate quad (a normalised 4-D Gaussian draw)."""
    p = g.standard_normal((d // 4, 4))
    return (p / np.linalg.norm(p, axis=1, keepdims=True)).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, round to nearest
    even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def qjl_matrix(g: np.random.Generator, d: int):
    """The d x d QJL matrix with i.i.d. N(0, 1) entries, stored as bfloat16.

    Returns (bits uint16 [d, d] row-major, values float64 [d, d])."""
    s = g.standard_normal((d, d), dtype=np.float32)
    bits = f32_to_bf16_bits(s)
    return bits, bf16_bits_to_f64(bits)


def kv_cache(g: np.random.Generator, heads: int, tokens: int, d: int):
    """K and V [heads, tokens, d] float32 with per-(tensor, head, channel)
    scales exp(U(ln 0.1, ln 10))."""
    out = []
    for _ in range(2):
        base = g.standard_normal((heads, tokens, d), dtype=np.float32)
        scale = np.exp(g.uniform(np.log(0.1), np.log(10.0), size=(heads, 1, d))).astype(np.float32)
        out.append(base * scale)
    return out[0], out[1]


def clustered_unit(g: np.random.Generator, n: int, d_in: int, centres: int,
                   sigma: float = 0.1, centre_vectors=None):
    """Unit-norm rows around ``centres`` random unit centres.  Returns
    (rows float32 [n, d_in], centre vectors float32 [centres, d_in])."""
    if centre_vectors is None:
        c = g.standard_normal((centres, d_in))
        centre_vectors = (c / np.linalg.norm(c, axis=1, keepdims=True)).astype(np.float32)
    pick = g.integers(0, centre_vectors.shape[0], size=n)
    pts = centre_vectors[pick].astype(np.float64)
    pts += (sigma / np.sqrt(d_in)) * g.standard_normal((n, d_in))
    pts /= np.linalg.norm(pts, axis=1, keepdims=True)
    return pts.astype(np.float32), centre_vectors


# --------------------------------------------------------------------------
# Device-side draws for benchmark-size inputs (torch on the GPU, seeded).
# --------------------------------------------------------------------------

def torch_gaussian(n: int, d: int, seed: int, device, dtype=None, outliers=False):
    """[n, d] N(0, 1) drawn on ``device`` with a seeded torch generator, in
    float32, optional outlier channels, then cast to ``dtype``."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    x = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
    if outliers:
        x[:, list(OUTLIER_CHANNELS)] *= OUTLIER_SCALE
    if dtype is not None and dtype != torch.float32:
        x = x.to(dtype)
    return x


def torch_clustered_unit(n: int, d_in: int, centres: int, seed: int, device,
                         sigma: float = 0.1, chunk: int = 1 << 17):
    """Device-side version of clustered_unit for large n (float32 rows)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    c = torch.randn((centres, d_in), generator=gen, device=device, dtype=torch.float32)
    c = c / c.norm(dim=1, keepdim=True)
    out = torch.empty((n, d_in), device=device, dtype=torch.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        pick = torch.randint(0, centres, (e - s,), generator=gen, device=device)
        pts = c[pick] + (sigma / d_in ** 0.5) * torch.randn((e - s, d_in), generator=gen, device=device)
        out[s:e] = pts / pts.norm(dim=1, keepdim=True)
    return out, c


def torch_kv_cache(heads: int, tokens: int, d: int, seed: int, device):
    """K, V [heads, tokens, d] bfloat16 on the device: N(0, 1) times per
    (tensor, head, channel) scales exp(U(ln 0.1, ln 10))."""
    import math
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for _ in range(2):
        base = torch.randn((heads, tokens, d), generator=gen, device=device, dtype=torch.float32)
        u = torch.rand((heads, 1, d), generator=gen, device=device, dtype=torch.float32)
        scale = torch.exp(math.log(0.1) + u * (math.log(10.0) - math.log(0.1)))
        out.append((base * scale).to(torch.bfloat16))
    return out[0], out[1]
