"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Every case prints its parameters before touching the GPU.  Inputs come from
synth (seeded); expected values come from oracle/ only, evaluated on the
same inputs (and, for dequantisation and scores, on the GPU's checked
records).  Acceptance rules are in tests/parity.py."""

import math

import numpy as np
import pytest
import torch

import parity as P
import synth
from embedding_vector_quantization_amd import binding as B
from oracle import tq_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _to_device(x32: np.ndarray, dtype: str, ld_pad: int = 0):
    """Device tensor of `dtype` (a view with row stride d_in + ld_pad) and
    the exact float64 widening of its values for the oracle."""
    n, d_in = x32.shape
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(TORCH_DT[dtype])
    host64 = t.float().numpy().astype(np.float64)
    full = torch.zeros((n, d_in + ld_pad), dtype=TORCH_DT[dtype])
    full[:, :d_in] = t
    dev = full.to(DEV)
    return dev[:, :d_in], host64


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


def run_case(n, d_in, d, b, mode, dtype="f32", seed=0, ld_pad=0, outliers=False, special_rows=None,
             nq=0, decode=True, count_limit=True):
    P.say(f"[case] n={n} d_in={d_in} d={d} b={b} mode={mode} dtype={dtype} seed={seed} "
          f"ld_pad={ld_pad} nq={nq}")
    g = synth.rng(seed)
    x32 = synth.gaussian(g, n, d_in)
    if outliers:
        x32 = synth.with_outliers(x32)
    if special_rows:
        for r, row in special_rows.items():
            x32[r] = row
    signs = synth.rht_signs(g, d)
    s_bits, s64 = synth.qjl_matrix(g, d) if mode == "prod" else (None, None)
    qh = g.standard_normal((nq, d_in)).astype(np.float32) if nq else None
    m = b if mode == "mse" else b - 1
    c32, t32 = P.codebook32(d, m) if m > 0 else (None, None)

    q = B.Quantizer.create(d_in, d, b, mode, signs, s_bits, centroids=c32, thresholds=t32)
    xd, x64 = _to_device(x32, dtype, ld_pad)
    out = B.encode(q, xd)
    torch.cuda.synchronize()
    rec = {k: _np(v) for k, v in out.items()}

    n64 = np.sqrt(np.sum(x64 * x64, axis=1))
    P.check_norms(rec["norms"], n64)
    if mode == "mse":
        ref = O.encode_mse(x64, d, signs, c32, t32)
    else:
        ref = O.encode_prod(x64, d, signs, c32, t32, s64)
    gi = None
    if m > 0:
        gi, flips, near = P.check_codes(rec["codes"], ref["y"], ref["idx"], t32, m, count_limit)
        P.say(f"    codes ok: flips={flips} near-boundary={near} of {gi.size}")
    if mode == "prod":
        qf = P.check_qjl(rec["qjl"], rec["rnorms"], ref["y"], gi if gi is not None else np.zeros_like(ref["idx"]),
                         c32, s64)
        P.say(f"    qjl ok: flips={qf}")
    result = {"rec": rec, "x64": x64, "signs": signs, "s64": s64, "c32": c32, "q": q, "out": out}
    if decode:
        dec = _np(B.decode(q, out))
        torch.cuda.synchronize()
        ref_dec = O.decode(rec["codes"], rec["norms"], d, d_in, signs, c32,
                           rec.get("qjl"), rec.get("rnorms"), s64)
        P.check_close(dec, ref_dec, P.decode_floor(rec["norms"], d), what="decode")
        result["dec"] = dec
    if nq:
        qd = torch.from_numpy(qh).to(DEV)
        sc = _np(B.score(q, qd, out))
        torch.cuda.synchronize()
        ref_sc = O.score(qh.astype(np.float64), rec["codes"], rec["norms"], d, signs, c32,
                         rec.get("qjl"), rec.get("rnorms"), s64)
        P.check_close(sc, ref_sc, P.score_floor(rec["norms"], qh, d), what="score")
        result["scores"] = sc
    return result


# ------------------------------------------------------------------ mse

def test_config1_mse_b3_and_distortion():
    # 4,096 x 128 float32 N(0,1), b = 3: parity, then the decoded distortion
    # reproduces Theorem D_mse's value for d = 128 (0.033966) within 4 SE.
    r = run_case(4096, 128, 128, 3, "mse", nq=4)
    x = r["x64"]
    n = np.linalg.norm(x, axis=1)
    err = np.sum((x / n[:, None] - r["dec"] / n[:, None]) ** 2, axis=1)
    dmse = O.lloyd_max(128, 3)[2]
    assert abs(err.mean() - dmse) < 4 * err.std() / math.sqrt(len(err))


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("n", [1, 17, 1000])
def test_mse_bits_dtypes_ragged(b, dtype, n):
    run_case(n, 128, 128, b, "mse", dtype=dtype, seed=100 + b, nq=3)


@pytest.mark.parametrize("d_in,d", [(20, 32), (64, 64), (100, 128), (200, 256), (512, 512),
                                    (1000, 1024), (1536, 2048), (3000, 4096), (4096, 4096)])
@pytest.mark.parametrize("b", [2, 4])
def test_mse_dimensions(d_in, d, b):
    run_case(300, d_in, d, b, "mse", seed=7, nq=2)


@pytest.mark.parametrize("b", [5, 6, 7, 8])
def test_mse_high_bits(b):
    run_case(500, 128, 128, b, "mse", seed=11, nq=2)


@pytest.mark.parametrize("dtype,d_in,ld_pad", [("f32", 128, 8), ("f32", 100, 3), ("bf16", 100, 0),
                                               ("f16", 120, 8), ("bf16", 128, 4)])
def test_strided_and_unaligned_rows(dtype, d_in, ld_pad):
    run_case(333, d_in, 128, 3, "mse", dtype=dtype, seed=13, ld_pad=ld_pad, nq=2)


def test_zero_onehot_and_wide_range_rows():
    d = 128
    rows = {0: np.zeros(d, np.float32), 5: np.eye(d, dtype=np.float32)[3] * 7.0,
            9: np.full(d, 1e-15, np.float32), 10: np.full(d, 1e17, np.float32),
            63: -np.eye(d, dtype=np.float32)[127]}
    r = run_case(64, d, d, 3, "mse", seed=17, special_rows=rows, nq=2, count_limit=False)
    assert r["rec"]["norms"][0] == 0.0
    assert np.all(r["dec"][0] == 0.0)
    assert np.all(r["scores"][:, 0] == 0.0)


@pytest.mark.parametrize("mode", ["mse", "prod"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_16bit_special_rows(dtype, mode):
    # 16-bit rows at d = 128 never go through a float32 copy of each element
    # (packed dot products give the signed pairs, the first two butterfly
    # stages and n^2): zero and negative-zero rows, one-hot rows, rows far
    # below and above unit scale (float16: subnormal elements) and a
    # constant row, whose transform has exact zeros.
    d = 128
    g = synth.rng(19)
    tiny = 1e-15 if dtype == "bf16" else 2e-6
    big = 1e17 if dtype == "bf16" else 1000.0
    rows = {0: np.zeros(d, np.float32), 1: np.full(d, -0.0, np.float32),
            5: np.eye(d, dtype=np.float32)[3] * 7.0, 63: -np.eye(d, dtype=np.float32)[127],
            9: (tiny * g.standard_normal(d)).astype(np.float32),
            10: (big * g.standard_normal(d)).astype(np.float32), 11: np.full(d, tiny, np.float32)}
    r = run_case(64, d, d, 3, mode, dtype=dtype, seed=23, special_rows=rows, nq=2, count_limit=False)
    assert r["rec"]["norms"][0] == 0.0 and r["rec"]["norms"][1] == 0.0
    assert np.all(r["dec"][:2] == 0.0)


@pytest.mark.parametrize("mode", ["mse", "prod"])
@pytest.mark.parametrize("dtype,d_in,d", [("f32", 128, 128), ("bf16", 128, 128), ("f16", 128, 128),
                                          ("f32", 200, 256), ("bf16", 100, 128), ("f32", 3000, 4096),
                                          ("bf16", 4096, 4096)])
def test_nonfinite_rows(mode, dtype, d_in, d):
    # Rows holding a NaN, +inf or -inf (alone, or with the rest of the row
    # finite) are stored as the zero row's record with norm NaN; they decode
    # to NaN and score NaN; the other rows of their wave are untouched.
    n, b = 40, 3
    P.say(f"[case] non-finite rows mode={mode} dtype={dtype} d_in={d_in} d={d}")
    g = synth.rng(29)
    x32 = synth.gaussian(g, n, d_in)
    x32[3, 5] = np.nan
    x32[7, :] = np.inf
    x32[8, d_in - 1] = -np.inf
    x32[20] = np.nan
    x32[21] = 0.0
    x32[39, 0] = np.inf
    bad = np.array([3, 7, 8, 20, 39])
    signs = synth.rht_signs(g, d)
    s_bits, s64 = synth.qjl_matrix(g, d) if mode == "prod" else (None, None)
    m = b if mode == "mse" else b - 1
    c32, t32 = P.codebook32(d, m)
    q = B.Quantizer.create(d_in, d, b, mode, signs, s_bits, centroids=c32, thresholds=t32)
    xd, x64 = _to_device(x32, dtype)
    out = B.encode(q, xd)
    qh = g.standard_normal((2, d_in)).astype(np.float32)
    dec = _np(B.decode(q, out))
    sc = _np(B.score(q, torch.from_numpy(qh).to(DEV), out))
    torch.cuda.synchronize()
    rec = {k: _np(v) for k, v in out.items()}
    ref = O.encode_mse(x64, d, signs, c32, t32) if mode == "mse" else O.encode_prod(x64, d, signs, c32, t32, s64)
    good = np.setdiff1d(np.arange(n), bad)
    assert np.all(np.isnan(rec["norms"][bad]))
    P.check_norms(rec["norms"][good], np.sqrt(np.sum(x64[good] ** 2, axis=1)))
    assert np.array_equal(rec["codes"][bad], ref["codes"][bad])
    assert np.array_equal(rec["codes"][bad], np.repeat(rec["codes"][21:22], len(bad), axis=0))
    gi, flips, near = P.check_codes(rec["codes"][good], ref["y"][good], ref["idx"][good], t32, m)
    if mode == "prod":
        assert np.array_equal(rec["qjl"][bad], np.repeat(rec["qjl"][21:22], len(bad), axis=0))
        assert np.all(rec["rnorms"][bad] == rec["rnorms"][21])
        P.check_qjl(rec["qjl"][good], rec["rnorms"][good], ref["y"][good], gi, c32, s64)
    assert np.all(np.isnan(dec[bad])) and np.all(np.isfinite(dec[good]))
    assert np.all(np.isnan(sc[:, bad])) and np.all(np.isfinite(sc[:, good]))


def test_qjl_matrix_with_tiny_entries():
    # S entries far below unit scale (bfloat16 1e-7, 3e-6, 2^-20, -5e-8):
    # the QJL bits still agree with the oracle's float64 S r outside the
    # eps band
    d, n, b = 128, 2000, 3
    P.say(f"[case] prod b={b} d={d} n={n} with tiny S entries")
    g = synth.rng(37)
    x = torch.from_numpy(synth.gaussian(g, n, d)).to(torch.bfloat16)
    signs = synth.rht_signs(g, d)
    s_bits, _ = synth.qjl_matrix(g, d)
    s_bits = s_bits.copy()
    tiny = synth.f32_to_bf16_bits(np.array([1e-7, 3e-6, 2.0 ** -20, -5e-8, -1e-6], np.float32))
    pos = g.choice(d * d, size=200, replace=False)
    s_bits.reshape(-1)[pos] = tiny[np.arange(200) % len(tiny)]
    s64 = synth.bf16_bits_to_f64(s_bits)
    c32, t32 = P.codebook32(d, b - 1)
    q = B.Quantizer.create(d, d, b, "prod", signs, s_bits, c32, t32)
    out = B.encode(q, x.to(DEV))
    torch.cuda.synchronize()
    rec = {k: _np(v) for k, v in out.items()}
    x64 = x.float().numpy().astype(np.float64)
    ref = O.encode_prod(x64, d, signs, c32, t32, s64)
    gi, flips, _ = P.check_codes(rec["codes"], ref["y"], ref["idx"], t32, b - 1)
    qf = P.check_qjl(rec["qjl"], rec["rnorms"], ref["y"], gi, c32, s64)
    P.say(f"    codes flips={flips}, qjl flips={qf}")


def test_n_zero_is_a_noop():
    q = B.Quantizer.create(128, 128, 3, "mse", synth.rht_signs(synth.rng(1), 128),
                           centroids=P.codebook32(128, 3)[0], thresholds=P.codebook32(128, 3)[1])
    x = torch.zeros((0, 128), device=DEV)
    out = q.alloc_codes(0)
    B.tq_encode_mse(q, x, out)
    torch.cuda.synchronize()


def test_encode_is_deterministic():
    P.say("[case] determinism n=5000 d=128 b=3 prod")
    g = synth.rng(21)
    x = torch.from_numpy(synth.gaussian(g, 5000, 128)).to(DEV)
    s_bits, _ = synth.qjl_matrix(g, 128)
    c32, t32 = P.codebook32(128, 2)
    q = B.Quantizer.create(128, 128, 3, "prod", synth.rht_signs(g, 128), s_bits, c32, t32)
    a, b = B.encode(q, x), B.encode(q, x)
    torch.cuda.synchronize()
    for k in ("codes", "qjl", "norms", "rnorms"):
        assert torch.equal(a[k], b[k]), k


# ------------------------------------------------------------------ prod

@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_prod_bits_dtypes(b, dtype):
    run_case(1000, 128, 128, b, "prod", dtype=dtype, seed=200 + b, outliers=(dtype == "f16"), nq=3)


@pytest.mark.parametrize("dtype,ld_pad,n", [("bf16", 8, 333), ("f16", 64, 1001), ("bf16", 0, 16), ("f16", 0, 15)])
def test_prod_strided_16bit_rows(dtype, ld_pad, n):
    # 16-bit rows at d = 128 (the matrix-core transform path) with a row
    # stride beyond d_in, whole and ragged last groups
    run_case(n, 128, 128, 3, "prod", dtype=dtype, seed=33, ld_pad=ld_pad, outliers=True, nq=2)


@pytest.mark.parametrize("d_in,d", [(32, 32), (60, 64), (256, 256), (400, 512), (1536, 2048), (3000, 4096)])
def test_prod_dimensions(d_in, d):
    run_case(200, d_in, d, 3, "prod", seed=31, nq=2)


# d = 4096: one vector over a pair of waves (the last butterfly stage and
# the sums through LDS); 16-bit inputs, a ragged d_in (the unvectorised row
# loads), a row stride past d_in, an odd row count (the second pair of the
# last workgroup idle) and the prod path with 1 and 4 bits
@pytest.mark.parametrize("mode,b,dtype,d_in,ld_pad,n", [("mse", 3, "bf16", 4096, 0, 65), ("mse", 2, "f16", 3001, 5, 33),
                                                        ("mse", 4, "f32", 2049, 3, 7), ("prod", 1, "bf16", 4000, 8, 9),
                                                        ("prod", 4, "f32", 4096, 0, 5)])
def test_d4096_paired_waves(mode, b, dtype, d_in, ld_pad, n):
    run_case(n, d_in, 4096, b, mode, dtype=dtype, seed=77 + b, ld_pad=ld_pad, nq=3)


def test_d4096_many_queries():
    # 20 queries: TurboQuant_mse scores on the matrix cores
    run_case(100, 4096, 4096, 2, "mse", seed=83, nq=20)


# ------------------------------------------------------------------ rotation

@pytest.mark.parametrize("d_in,d", [(128, 128), (100, 128), (32, 32), (1536, 2048), (3000, 4096), (4096, 4096)])
def test_rht_forward_inverse(d_in, d):
    P.say(f"[case] rht d_in={d_in} d={d}")
    g = synth.rng(41)
    x = synth.gaussian(g, 257, d_in)
    signs = synth.rht_signs(g, d)
    q = B.Quantizer(d_in=d_in, d=d, m=0, mode="mse")
    q.signs = torch.from_numpy(signs).to(DEV)
    xd = torch.from_numpy(x).to(DEV)
    y = torch.empty((257, d), device=DEV)
    B.tq_rht(q, xd, y)
    back = torch.empty((257, d_in), device=DEV)
    B.tq_rht(q, y, back, inverse=True)
    torch.cuda.synchronize()
    ref = O.rht(np.pad(x.astype(np.float64), ((0, 0), (0, d - d_in))), signs)
    nx = np.linalg.norm(x.astype(np.float64), axis=1)[:, None]
    # P4: forward and round trip within 1e-6 element-wise (relative to the
    # element plus ||x|| / sqrt d) and in norm
    P.check_close(_np(y), ref, nx / math.sqrt(d), rtol=1e-6, what="rht")
    P.check_close(_np(back), x, nx / math.sqrt(d), rtol=1e-6, what="rht round trip")
    rt = np.linalg.norm(_np(back).astype(np.float64) - x, axis=1) / nx[:, 0]
    P.say(f"    round trip max relative norm error {rt.max():.2e}")
    assert rt.max() <= 1e-6


# ------------------------------------------------------------------ grouped scores

@pytest.mark.parametrize("mode,b,d,nq", [("mse", 3, 128, 5), ("prod", 3, 128, 4), ("mse", 2, 256, 3),
                                         ("prod", 4, 128, 1), ("mse", 7, 128, 2), ("prod", 2, 64, 3)])
def test_score_grouped_matches_per_group_oracle(mode, b, d, nq):
    groups, n = 3, 700
    P.say(f"[case] grouped scores mode={mode} b={b} d={d} groups={groups} nq={nq} n={n}")
    g = synth.rng(77)
    x = synth.gaussian(g, groups * n, d)
    signs = synth.rht_signs(g, d)
    s_bits, s64 = synth.qjl_matrix(g, d) if mode == "prod" else (None, None)
    qh = g.standard_normal((groups * nq, d)).astype(np.float32)
    m = b if mode == "mse" else b - 1
    c32, t32 = P.codebook32(d, m)
    q = B.Quantizer.create(d, d, b, mode, signs, s_bits, c32, t32)
    rec = B.encode(q, torch.from_numpy(x).to(DEV))
    ld = n + 3
    scores = torch.full((groups * nq, ld), float("nan"), device=DEV)
    ws = torch.empty(B.tq_score_workspace(q, groups * nq), dtype=torch.uint8, device=DEV)
    B.tq_score_grouped(q, torch.from_numpy(qh).to(DEV), groups, rec, scores, ws)
    torch.cuda.synchronize()
    r = {k: _np(v) for k, v in rec.items()}
    sc = _np(scores)
    assert np.all(np.isnan(sc[:, n:]))                      # nothing written past n
    for gi in range(groups):
        ks = slice(gi * n, (gi + 1) * n)
        qs = slice(gi * nq, (gi + 1) * nq)
        sub = {k: (None if v is None else v[ks]) for k, v in r.items()}
        ref = O.score(qh[qs].astype(np.float64), sub["codes"], sub["norms"], d, signs, c32,
                      sub.get("qjl"), sub.get("rnorms"), s64)
        P.check_close(sc[qs, :n], ref, P.score_floor(sub["norms"], qh[qs], d), what=f"group {gi}")


# ------------------------------------------------------------------ one query per group, d = 128

@pytest.mark.parametrize("mode,b,n", [("mse", 3, 600_001), ("mse", 2, 262_145), ("mse", 1, 5000),
                                      ("mse", 4, 200_003), ("prod", 4, 300_007), ("prod", 3, 4099),
                                      ("prod", 3, 262_147), ("prod", 2, 5003), ("prod", 1, 5005),
                                      ("mse", 3, 37)])
def test_score_one_query_d128(mode, b, n):
    # one query: enough keys that each workgroup walks several key tiles,
    # and a ragged last tile
    run_case(n, 128, 128, b, mode, seed=300 + b, nq=1, decode=False, count_limit=n >= 1000)


@pytest.mark.parametrize("mode,b", [("mse", 3), ("mse", 2), ("prod", 4)])
def test_score_one_query_grouped_and_accumulated(mode, b):
    # 5 groups of 3,001 keys, one query each; a second call adds the same
    # estimates to what the first wrote
    groups, n, d = 5, 3001, 128
    P.say(f"[case] one query per group mode={mode} b={b} groups={groups} n={n}")
    g = synth.rng(310 + b)
    x = synth.gaussian(g, groups * n, d)
    signs = synth.rht_signs(g, d)
    s_bits, s64 = synth.qjl_matrix(g, d) if mode == "prod" else (None, None)
    qh = g.standard_normal((groups, d)).astype(np.float32)
    m = b if mode == "mse" else b - 1
    c32, t32 = P.codebook32(d, m)
    q = B.Quantizer.create(d, d, b, mode, signs, s_bits, c32, t32)
    rec = B.encode(q, torch.from_numpy(x).to(DEV))
    scores = torch.full((groups, n + 5), float("nan"), device=DEV)
    ws = torch.empty(B.tq_score_workspace(q, groups), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(qh).to(DEV)
    B.tq_score_grouped(q, qd, groups, rec, scores, ws)
    first = scores.clone()
    B.tq_score_accumulate(q, qd, groups, rec, scores, ws)
    torch.cuda.synchronize()
    r = {k: _np(v) for k, v in rec.items()}
    sc1, sc2 = _np(first), _np(scores)
    assert np.all(np.isnan(sc2[:, n:]))
    for gi in range(groups):
        ks = slice(gi * n, (gi + 1) * n)
        sub = {k: (None if v is None else v[ks]) for k, v in r.items()}
        ref = O.score(qh[gi:gi + 1].astype(np.float64), sub["codes"], sub["norms"], d, signs, c32,
                      sub.get("qjl"), sub.get("rnorms"), s64)
        floor = P.score_floor(sub["norms"], qh[gi:gi + 1], d)
        P.check_close(sc1[gi:gi + 1, :n], ref, floor, what=f"group {gi}")
        P.check_close(sc2[gi:gi + 1, :n], 2 * ref, 2 * floor, what=f"group {gi} accumulated")


@pytest.mark.parametrize("mode,b,nq", [("prod", 3, 4), ("mse", 2, 4), ("prod", 4, 3), ("mse", 3, 6),
                                       ("mse", 1, 2), ("prod", 1, 5), ("prod", 2, 3), ("prod", 3, 7)])
def test_score_few_queries_grouped_accumulated(mode, b, nq):
    # up to four queries per block (a full block of four, a block of three, and
    # six queries: a block of four and a ragged block of two); 3 groups of
    # 2,500 keys, so the last key tile of each group is ragged; a second call
    # adds the same estimates to what the first wrote
    groups, n, d = 3, 2500, 128
    P.say(f"[case] few queries grouped mode={mode} b={b} groups={groups} nq={nq} n={n}")
    g = synth.rng(350 + b + nq)
    x = synth.gaussian(g, groups * n, d)
    signs = synth.rht_signs(g, d)
    s_bits, s64 = synth.qjl_matrix(g, d) if mode == "prod" else (None, None)
    qh = g.standard_normal((groups * nq, d)).astype(np.float32)
    m = b if mode == "mse" else b - 1
    c32, t32 = P.codebook32(d, m) if m > 0 else (None, None)
    q = B.Quantizer.create(d, d, b, mode, signs, s_bits, c32, t32)
    rec = B.encode(q, torch.from_numpy(x).to(DEV))
    scores = torch.full((groups * nq, n + 3), float("nan"), device=DEV)
    ws = torch.empty(B.tq_score_workspace(q, groups * nq), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(qh).to(DEV)
    B.tq_score_grouped(q, qd, groups, rec, scores, ws)
    first = scores.clone()
    B.tq_score_accumulate(q, qd, groups, rec, scores, ws)
    torch.cuda.synchronize()
    r = {k: _np(v) for k, v in rec.items()}
    sc1, sc2 = _np(first), _np(scores)
    assert np.all(np.isnan(sc2[:, n:]))
    for gi in range(groups):
        ks = slice(gi * n, (gi + 1) * n)
        qs = slice(gi * nq, (gi + 1) * nq)
        sub = {k: (None if v is None else v[ks]) for k, v in r.items()}
        ref = O.score(qh[qs].astype(np.float64), sub["codes"], sub["norms"], d, signs, c32,
                      sub.get("qjl"), sub.get("rnorms"), s64)
        floor = P.score_floor(sub["norms"], qh[qs], d)
        P.check_close(sc1[qs, :n], ref, floor, what=f"group {gi}")
        P.check_close(sc2[qs, :n], 2 * ref, 2 * floor, what=f"group {gi} accumulated")


# ------------------------------------------------------------------ many queries (matrix cores)

@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_score_many_queries_d128(b):
    # 37 queries: one 64-query block, ragged; 3,001 keys: six 512-key tiles,
    # the last ragged (its waves past the end store nothing, the one across
    # it column by column)
    run_case(3001, 128, 128, b, "mse", seed=320 + b, nq=37, decode=False)


def exact_fit_takes(c, d):
    """Whether the many-query kernel multiplies an odd-symmetric codebook of
    1 or 2 bits with float16-exact code values (outer value P in
    [1024, 2047], inner q 2^-k with q <= 2047, unit u = b / P in float32):
    two products instead of three when delta sqrt(d) <= b / 150000, delta
    the largest |v u - c|.  A host replica of the rule, used to say which
    path a case takes."""
    return exact_fit_delta(c) * np.sqrt(d) * 150000.0 <= np.float64(c[-1])


def exact_fit_delta(c):
    c = np.asarray(c, np.float64)
    b = c[-1]
    if len(c) == 2:
        u = float(np.float32(b / 1024))
        return abs(1024 * u - b)
    a, alpha = c[2], c[2] / c[3]
    best = None
    for pp in range(1024, 2048):
        x, k = alpha * pp, 0
        while k < 24 and round(x * 2.0 ** (k + 1)) <= 2047:
            k += 1
        key = (np.float32(abs(round(x * 2.0 ** k) * 2.0 ** -k / pp - alpha)), pp, k)
        best = key if best is None or key < best else best
    _, pp, k = best
    qv = round(alpha * pp * 2.0 ** k) * 2.0 ** -k
    u = float(np.float32(b / pp))
    return max(abs(pp * u - b), abs(qv * u - a))


@pytest.mark.parametrize("b,d_in,d", [(2, 1536, 2048), (4, 1536, 2048), (3, 200, 256), (1, 512, 512),
                                      (2, 400, 512)])
def test_score_many_queries_wide(b, d_in, d):
    if b <= 2:
        # b = 1 (one magnitude) and b = 2 at d = 2048 take the two-product
        # path, b = 2 at d = 512 (its codebook's inner/outer ratio has no
        # close float16 fit) the three-product one
        assert exact_fit_takes(P.codebook32(d, b)[0], d) == (b == 1 or d != 512)
    run_case(700, d_in, d, b, "mse", seed=330 + b, nq=16, decode=False)


def test_score_many_queries_exact_custom_codebook():
    # an odd-symmetric 2-bit codebook with inner / outer = 1/3 exactly in
    # float32: the two-product path, its fit off only by the float32 unit
    n, d, nq = 1500, 256, 24
    P.say(f"[case] many queries custom codebook n={n} nq={nq}")
    g = synth.rng(352)
    x = synth.gaussian(g, n, d)
    signs = synth.rht_signs(g, d)
    qh = g.standard_normal((nq, d)).astype(np.float32)
    c32 = np.array([-3, -1, 1, 3], np.float32) / np.float32(64)
    t32 = np.array([-2, 0, 2], np.float32) / np.float32(64)
    assert exact_fit_takes(c32, d)
    q = B.Quantizer.create(d, d, 2, "mse", signs, None, c32, t32)
    rec = B.encode(q, torch.from_numpy(x).to(DEV))
    sc = _np(B.score(q, torch.from_numpy(qh).to(DEV), rec))
    torch.cuda.synchronize()
    r = {k: _np(v) for k, v in rec.items()}
    ref = O.score(qh.astype(np.float64), r["codes"], r["norms"], d, signs, c32)
    P.check_close(sc, ref, P.score_floor(r["norms"], qh, d), what="scores")


@pytest.mark.parametrize("b", [2, 3])
def test_score_many_queries_grouped_accumulated(b):
    # 3 groups of 1,000 keys, 20 queries each; a second call adds the same
    # estimates to what the first wrote
    groups, n, nq, d = 3, 1000, 20, 128
    P.say(f"[case] many queries grouped b={b} groups={groups} nq={nq} n={n}")
    g = synth.rng(340 + b)
    x = synth.gaussian(g, groups * n, d)
    signs = synth.rht_signs(g, d)
    qh = g.standard_normal((groups * nq, d)).astype(np.float32)
    c32, t32 = P.codebook32(d, b)
    q = B.Quantizer.create(d, d, b, "mse", signs, None, c32, t32)
    rec = B.encode(q, torch.from_numpy(x).to(DEV))
    scores = torch.full((groups * nq, n + 3), float("nan"), device=DEV)
    ws = torch.empty(B.tq_score_workspace(q, groups * nq), dtype=torch.uint8, device=DEV)
    qd = torch.from_numpy(qh).to(DEV)
    B.tq_score_grouped(q, qd, groups, rec, scores, ws)
    first = scores.clone()
    B.tq_score_accumulate(q, qd, groups, rec, scores, ws)
    torch.cuda.synchronize()
    r = {k: _np(v) for k, v in rec.items()}
    sc1, sc2 = _np(first), _np(scores)
    assert np.all(np.isnan(sc2[:, n:]))
    for gi in range(groups):
        ks = slice(gi * n, (gi + 1) * n)
        qs = slice(gi * nq, (gi + 1) * nq)
        ref = O.score(qh[qs].astype(np.float64), r["codes"][ks], r["norms"][ks], d, signs, c32)
        floor = P.score_floor(r["norms"][ks], qh[qs], d)
        P.check_close(sc1[qs, :n], ref, floor, what=f"group {gi}")
        P.check_close(sc2[qs, :n], 2 * ref, 2 * floor, what=f"group {gi} accumulated")


@pytest.mark.parametrize("b", [2, 3])
def test_score_many_queries_large_and_tiny_query_scales(b):
    # query rows scaled by 1e6 and 1e-6: the per-row power-of-two scaling keeps
    # the float16 split in range (b = 2: exact code values, two products;
    # b = 3: three)
    n, d, nq = 2000, 128, 16
    P.say(f"[case] many queries extreme scales n={n} nq={nq} b={b}")
    g = synth.rng(350 + 10 * (b - 3))
    x = synth.gaussian(g, n, d)
    signs = synth.rht_signs(g, d)
    qh = g.standard_normal((nq, d)).astype(np.float32)
    qh[:8] *= 1e6
    qh[8:] *= 1e-6
    c32, t32 = P.codebook32(d, b)
    q = B.Quantizer.create(d, d, b, "mse", signs, None, c32, t32)
    rec = B.encode(q, torch.from_numpy(x).to(DEV))
    sc = _np(B.score(q, torch.from_numpy(qh).to(DEV), rec))
    torch.cuda.synchronize()
    r = {k: _np(v) for k, v in rec.items()}
    ref = O.score(qh.astype(np.float64), r["codes"], r["norms"], d, signs, c32)
    P.check_close(sc, ref, P.score_floor(r["norms"], qh, d), what="scores")
