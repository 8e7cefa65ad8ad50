"""GPU parity of the outlier-channel split (one library call per channel
range, scores accumulated with tq_score_accumulate) against the oracle's
split functions, evaluated on the GPU's records."""

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


def _np(t):
    return None if t is None else t.detach().cpu().numpy()


@pytest.mark.parametrize("layout", [((0, 32, 3), (32, 96, 2)), ((0, 32, 4), (32, 96, 3)),
                                    ((0, 64, 4), (64, 64, 3))])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_encode_decode_score(layout, dtype):
    P.say(f"[case] split {layout} dtype={dtype}")
    g = synth.rng(100)
    n, nq = 3000, 5
    x32 = synth.with_outliers(synth.gaussian(g, n, 128))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xt = torch.from_numpy(x32).to(tdt)
    x64 = xt.float().numpy().astype(np.float64)
    qh = g.standard_normal((nq, 128)).astype(np.float32)
    parts, oparts = [], []
    for c0, d_in, b in layout:
        d = max(32, 1 << (d_in - 1).bit_length())
        signs = synth.rht_signs(g, d)
        c32, t32 = P.codebook32(d, b)
        parts.append((c0, B.Quantizer.create(d_in, d, b, "mse", signs, None, c32, t32)))
        oparts.append({"c0": c0, "d_in": d_in, "d": d, "rot": signs, "centroids": c32, "thresholds": t32})
    sq = B.SplitQuantizer(parts)
    recs = sq.encode(xt.to(DEV))
    dec = _np(sq.decode(recs))
    sc = _np(sq.score(torch.from_numpy(qh).to(DEV), recs))
    torch.cuda.synchronize()
    ref = O.split_encode(x64, oparts)
    encs = []
    for r, e, p in zip(recs, ref, oparts):
        rr = {k: _np(v) for k, v in r.items()}
        xs = x64[:, p["c0"]:p["c0"] + p["d_in"]]
        P.check_norms(rr["norms"], np.sqrt(np.sum(xs * xs, axis=1)))
        P.check_codes(rr["codes"], e["y"], e["idx"], p["thresholds"], int(round(math.log2(len(p["centroids"])))))
        encs.append({"codes": rr["codes"], "norms": rr["norms"]})
    ref_dec = O.split_decode(encs, oparts)
    floor = np.max([e["norms"] / math.sqrt(p["d"]) for e, p in zip(encs, oparts)], axis=0)[:, None]
    P.check_close(dec, ref_dec, floor, what="split decode")
    ref_sc = O.split_score(qh.astype(np.float64), encs, oparts)
    nsum = sum(e["norms"].astype(np.float64) for e in encs)
    P.check_close(sc, ref_sc, np.linalg.norm(qh, axis=1)[:, None] * nsum[None, :] / math.sqrt(32),
                  what="split score")
