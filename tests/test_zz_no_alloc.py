"""GPU test of tq_attend_noalloc, the variant of tq_attend that takes no
workspace (its partials live in a fixed device array inside the library):
through the C ABI, its output equals tq_attend's on the same inputs
bit for bit (the same kernels), on two calls in a row, the second one
smaller than the first; a request beyond the array's size is refused."""

import math

import numpy as np
import pytest
import torch

import parity as P
import synth
from embedding_vector_quantization_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 128


def _case(groups, nq, n, kmode, bk, bv, d_in, seed):
    g = synth.rng(seed)
    kd = torch.from_numpy(synth.gaussian(g, groups * n, d_in)).to(DEV)
    vd = torch.from_numpy(synth.gaussian(g, groups * n, d_in)).to(DEV)
    ks, vs = synth.rht_signs(g, D), synth.rht_signs(g, D)
    s_bits, _ = synth.qjl_matrix(g, D) if kmode == "prod" else (None, None)
    qh = torch.from_numpy(g.standard_normal((groups * nq, d_in)).astype(np.float32)).to(DEV)
    mk = bk if kmode == "mse" else bk - 1
    ck, tk = P.codebook32(D, mk) if mk > 0 else (None, None)
    cv, tv = P.codebook32(D, bv)
    qk = B.Quantizer.create(d_in, D, bk, kmode, ks, s_bits, ck, tk)
    qv = B.Quantizer.create(d_in, D, bv, "mse", vs, None, cv, tv)
    return qk, B.encode(qk, kd), qv, B.encode(qv, vd), qh


def _both(case, groups):
    qk, krec, qv, vrec, qh = case
    n = krec["norms"].shape[0] // groups
    ref = torch.empty((qh.shape[0], qk.d_in), device=DEV)
    ws = torch.empty(B.tq_attend_workspace(qk, groups, qh.shape[0] // groups, n), dtype=torch.uint8, device=DEV)
    B.tq_attend(qk, krec, qv, vrec, qh, groups, ref, ws)
    got = torch.full_like(ref, float("nan"))
    B.tq_attend_noalloc(qk, krec, qv, vrec, qh, groups, got)
    torch.cuda.synchronize()
    return got, ref


def test_attend_noalloc_matches_attend_on_two_calls():
    # first call: one layer of 8 KV heads x 32,768 tokens, 32 query heads
    # (prod keys b = 3, mse values b = 3; 2.1 MiB of partials); second call:
    # smaller, ragged (3 groups x 3 queries x 1,000 tokens, d_in = 100)
    P.say("[case] attend_noalloc: 8 x 4 queries x 32768 tokens, then 3 x 3 x 1000")
    big = _case(8, 4, 32768, "prod", 3, 3, D, seed=71)
    got, ref = _both(big, 8)
    assert torch.equal(got, ref)
    small = _case(3, 3, 1000, "mse", 2, 4, 100, seed=72)
    got, ref = _both(small, 3)
    assert torch.equal(got, ref)
    assert bool(torch.isfinite(got).all())


def test_attend_noalloc_refuses_beyond_its_array():
    # 64 KV groups x 4 queries x 131,072 tokens need 64 MiB of partials
    P.say("[case] attend_noalloc size limit")
    qk, krec, qv, vrec, qh = _case(1, 4, 256, "mse", 2, 2, D, seed=73)
    groups, nq, n = 64, 4, 131072
    assert B.tq_attend_workspace(qk, groups, nq, n) > B.ATTEND_NOALLOC_MAX_WORKSPACE
    pk, pv = qk.params(), qv.params()
    ck, cv = B._codes_struct(krec), B._codes_struct(vrec)
    import ctypes
    out = torch.empty((groups * nq, D), device=DEV)
    st = B.lib().tq_attend_noalloc(ctypes.byref(pk), qk.mode_code, ctypes.byref(ck), ctypes.byref(pv),
                                   ctypes.byref(cv), qh.data_ptr(), qh.stride(0), groups, nq, n,
                                   1.0 / math.sqrt(D), out.data_ptr(), out.stride(0), None)
    assert st == B.TQ_ERR_WORKSPACE
