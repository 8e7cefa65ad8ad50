"""Benchmark of the TurboQuant hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu]

A step is one pass of the whole hot path over one batch: TurboQuant_prod
b = 3 (2-bit mse code + 1-bit QJL) encode of a KV-cache key batch
(8 KV heads x 131,072 tokens x d = 128, bfloat16, outlier channels
{0,1,2,3} x 20), decode of every key (float32 out), and the inner-product
scores of 32 query heads (GQA 4:1: each KV head against its 4 queries).
value = keys per second through the step.  The same run also times the
TurboQuant_mse b = 3 kernels on their own (encode of 2^22 float32 rows,
score of 2^24 keys for one query), the fused decode attention over one
layer's KV cache (b = 2 and 4), a top-10 search of 1,000 queries over
1,000,000 rows (b = 2 and 4), the RHT / Givens / quaternion rotation
comparison and the outlier-channel split on the key batch, reports each kernel's HBM bandwidth against
the 8 TB/s peak, and times the CPU oracle on a bounded sample.

--profile-kernel NAME --reps R runs only that kernel R times, each call after
the same cache flush the timed loops use (for rocprofv3); NAME = encode_prod |
decode | score | encode_mse | score_mse | attend2 | attend4 | attend2x32 |
attend4x32 | search2 | search4 | probes (the bandwidth probes) | copy (a
plain device copy of known size, to calibrate FETCH_SIZE / WRITE_SIZE).

Per-kernel times of the step kernels and the TurboQuant_mse headline kernels
are averages over back-to-back calls between one pair of HIP events, the
calls cycling over enough copies of their buffers (or moving enough bytes)
that their inputs come from HBM, not the Infinity Cache; ms_flushed_call is
the average of a HIP event pair around single calls with the Infinity Cache
and L2s flushed before each (a 2 GiB read-only stream outside the pair),
which adds the launch latency.  Attention, search, probes and the
comparisons use the flushed single calls.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "encoded vectors/s + score-kernel GB/s (% HBM peak), d=128 b=3"
HEADS, TOKENS, D, B_BITS, QHEADS = 8, 131072, 128, 3, 32
N_KEYS = HEADS * TOKENS
MENC_N = 1 << 22
MSCORE_N = 1 << 24
KERNEL_SOURCES = ["tq_encode.hip", "tq_decode.hip", "tq_score.hip", "tq_lut.h", "tq_device.h", "tq_internal.h",
                  "tq_attend.hip", "tq_scorem.hip", "tq_topk.hip"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--profile-kernel", default=None)
    ap.add_argument("--reps", type=int, default=5)
    return ap.parse_args()


_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)


def _code_only(text: str) -> str:
    """A C++ source without its comments, whitespace runs collapsed (string
    and character literals kept), so that comment edits leave it unchanged."""
    def keep(m):
        t = m.group(0)
        return " " if t.startswith("/") else t
    return " ".join(_TOKENS.sub(keep, text).split())


def source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout excluded): the
    committed counter summary applies while it matches."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "embedding_vector_quantization_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ setup

def make_workload(torch, tq, synth, library_codebook):
    dev = "cuda"
    g = synth.rng(4)
    x = synth.torch_gaussian(N_KEYS, D, seed=4, device=dev, dtype=torch.bfloat16, outliers=True)
    signs = synth.rht_signs(g, D)
    s_bits, s64 = synth.qjl_matrix(g, D)
    qh = g.standard_normal((QHEADS, D)).astype("float32")
    c32, t32 = library_codebook(D, B_BITS - 1)
    q = tq.Quantizer.create(D, D, B_BITS, "prod", signs, s_bits, c32, t32, device=dev)
    rec = q.alloc_codes(N_KEYS)
    dec = torch.empty((N_KEYS, D), dtype=torch.float32, device=dev)
    queries = torch.from_numpy(qh).to(dev)
    scores = torch.empty((QHEADS, TOKENS), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_score_workspace(q, QHEADS), dtype=torch.uint8, device=dev)
    host = {"signs": signs, "s_bits": s_bits, "s64": s64, "q": qh, "c32": c32, "t32": t32}
    return {"x": x, "q": q, "rec": rec, "dec": dec, "queries": queries, "scores": scores, "ws": ws,
            "host": host}


def run_encode(tq, w):
    tq.tq_encode_prod(w["q"], w["x"], w["rec"])


def run_decode(tq, w):
    tq.tq_decode(w["q"], w["rec"], w["dec"])


def run_score(tq, w):
    # one launch: query heads 4h..4h+3 against KV head h's keys
    tq.tq_score_grouped(w["q"], w["queries"], HEADS, w["rec"], w["scores"], w["ws"])


def run_step(tq, w):
    run_encode(tq, w)
    run_decode(tq, w)
    run_score(tq, w)


class CacheFlush:
    """Evicts the 256 MB Infinity Cache (MALL) and the L2s between timed
    calls: a read-only stream over 2 GiB (eight times the MALL) with the
    probe library's read kernel, issued outside the timed event pair.  It
    writes nothing, so it leaves only clean lines behind, and the dirty
    lines of the previous call are written back while it runs.  Every
    per-kernel figure is therefore taken with its inputs in HBM, not in a
    cache that a back-to-back repetition of the same call would hit, and
    without another kernel's write-backs in its time."""

    BYTES = 1 << 31

    def __init__(self, torch):
        self.lib = probe_lib()
        self.buf = torch.ones(self.BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
        self.torch = torch

    def __call__(self):
        rc = self.lib.tqp_read(self.buf.data_ptr(), self.BYTES, self.sink.data_ptr(),
                               self.torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"cache flush failed: hip error {rc}")


def time_region(torch, fn, reps, flush):
    """Average milliseconds of one fn() call over reps calls, each bracketed
    by its own pair of HIP events on the current stream (the one every
    library call is issued on), with the caches flushed before each call
    (outside the pair): for a single-launch call this is the kernel's
    duration on cold inputs."""
    return time_interleaved(torch, [fn], reps, flush)[0]


def time_interleaved(torch, fns, reps, flush):
    """As time_region for several calls at once: each repetition times every
    fn in turn, so slow drifts of clock or memory state hit all of them
    alike.  Returns the average milliseconds of each."""
    stream = torch.cuda.current_stream()
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(reps)]
    for row in ev:
        for fn, (start, end) in zip(fns, row):
            flush()
            start.record(stream)
            fn()
            end.record(stream)
    torch.cuda.synchronize()
    return [sum(row[i][0].elapsed_time(row[i][1]) for row in ev) / reps for i in range(len(fns))]


def time_rotating(torch, fns, reps):
    """Average milliseconds per call of back-to-back calls cycling over fns,
    each fn working on its own copy of the buffers, between one pair of HIP
    events.  With enough copies each call's inputs were last touched several
    calls (and more than the Infinity Cache's 256 MB) earlier, so they come
    from HBM, while the launch latency overlaps the previous call as in a
    serving loop: the average is the kernel's own duration on cold inputs."""
    stream = torch.cuda.current_stream()
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls = max(reps, len(fns)) // len(fns) * len(fns)
    start.record(stream)
    for i in range(calls):
        fns[i % len(fns)]()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / calls


def step_copies(torch, w, sets):
    """`sets` copies of the step's buffers: key rows and records cloned,
    outputs fresh (the queries and the quantiser are shared)."""
    out = []
    for _ in range(sets):
        c = dict(w)
        c["x"] = w["x"].clone()
        c["rec"] = {k: (None if v is None else v.clone()) for k, v in w["rec"].items()}
        c["dec"] = torch.empty_like(w["dec"])
        c["scores"] = torch.empty_like(w["scores"])
        out.append(c)
    return out


# Working-set copies for the rotating timings: about 1.2 GB, 1.8 GB and
# 0.6 GB per cycle (encode 312 MB, decode 600 MB, score 75 MB per call).
ROTATE_SETS = {"encode_prod": 4, "decode": 3, "score": 8}


# Algorithmic bytes per unit (what the method must move, padding excluded).
def bytes_encode_prod():   # per key: bf16 in, 2-bit codes, QJL plane, two norms
    return D * 2 + (B_BITS - 1) * D // 8 + D // 8 + 4 + 4


def bytes_decode_prod():   # per key: record in, float32 row out
    return (B_BITS - 1) * D // 8 + D // 8 + 8 + D * 4


def bytes_score_prod(nq):  # per key: record in, nq float32 scores out
    return (B_BITS - 1) * D // 8 + D // 8 + 8 + 4 * nq


def bytes_encode_mse_f32():
    return D * 4 + B_BITS * D // 8 + 4


def bytes_score_mse(nq):
    return B_BITS * D // 8 + 4 + 4 * nq


def kernel_entry(name, units, unit_bytes, ms, unit="vectors/s"):
    gbs = units * unit_bytes / (ms * 1e-3) / 1e9
    return {"kernel": name, "units": units, "bytes_per_unit": unit_bytes, "ms": round(ms, 4),
            "rate": units / (ms * 1e-3), "rate_unit": unit, "GB/s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


# ------------------------------------------------------------------ headline mse kernels

def mse_quantizer(tq, synth, library_codebook):
    g = synth.rng(1)
    signs = synth.rht_signs(g, D)
    c32, t32 = library_codebook(D, B_BITS)
    q = tq.Quantizer.create(D, D, B_BITS, "mse", signs, None, c32, t32, device="cuda")
    return q, g


def mse_encode_setup(torch, tq, synth, library_codebook):
    """TurboQuant_mse b = 3 encode of 2^22 float32 rows; returns the call."""
    q, _ = mse_quantizer(tq, synth, library_codebook)
    x = synth.torch_gaussian(MENC_N, D, seed=1, device="cuda")
    rec = q.alloc_codes(MENC_N)
    return lambda: tq.tq_encode_mse(q, x, rec)


def mse_score_setup(torch, tq, synth, library_codebook, nq=1):
    """nq queries against 2^24 TurboQuant_mse b = 3 keys (one key group);
    returns the call."""
    q, g = mse_quantizer(tq, synth, library_codebook)
    keys_src = synth.torch_gaussian(MSCORE_N, D, seed=2, device="cuda", dtype=torch.bfloat16)
    keys = q.alloc_codes(MSCORE_N)
    tq.tq_encode_mse(q, keys_src, keys)
    del keys_src
    query = torch.from_numpy(g.standard_normal((nq, D)).astype("float32")).to("cuda")
    scores = torch.empty((nq, MSCORE_N), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_score_workspace(q, nq), dtype=torch.uint8, device="cuda")
    return lambda: tq.tq_score(q, query, keys, scores, ws)


def prod_score_setup(torch, tq, synth, library_codebook, nq=1):
    """nq queries against 2^24 TurboQuant_prod b = 3 keys (2 code bits and
    the QJL plane; one key group); returns the call."""
    g = synth.rng(5)
    signs = synth.rht_signs(g, D)
    s_bits, _ = synth.qjl_matrix(g, D)
    c32, t32 = library_codebook(D, B_BITS - 1)
    q = tq.Quantizer.create(D, D, B_BITS, "prod", signs, s_bits, c32, t32, device="cuda")
    keys_src = synth.torch_gaussian(MSCORE_N, D, seed=6, device="cuda", dtype=torch.bfloat16)
    keys = q.alloc_codes(MSCORE_N)
    tq.tq_encode_prod(q, keys_src, keys)
    del keys_src
    query = torch.from_numpy(g.standard_normal((nq, D)).astype("float32")).to("cuda")
    scores = torch.empty((nq, MSCORE_N), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_score_workspace(q, nq), dtype=torch.uint8, device="cuda")
    return lambda: tq.tq_score(q, query, keys, scores, ws)


def mse_headline(torch, tq, synth, library_codebook, reps, flush):
    """Each call moves 2.4 GB (encode) or 0.94 / 1.14 / 3.0 GB (score with 1,
    4 or 32 queries; 1.0 GB for the one-query prod score), several times the
    Infinity Cache, so back-to-back calls on the same buffers read HBM.  With
    32 queries the estimates run on the matrix cores and the 2.1 GB of score
    rows written dominate."""
    out = []
    for setup, name, units, unit_bytes, unit in (
            (mse_encode_setup, "encode_mse b=3 f32 (2^22 rows)", MENC_N, bytes_encode_mse_f32(), "vectors/s"),
            (mse_score_setup, "score_mse b=3 Q=1 (2^24 keys)", MSCORE_N, bytes_score_mse(1), "keys/s"),
            (lambda *a: mse_score_setup(*a, nq=4), "score_mse b=3 Q=4 (2^24 keys)", MSCORE_N, bytes_score_mse(4),
             "keys/s"),
            (lambda *a: mse_score_setup(*a, nq=32), "score_mse b=3 Q=32 (2^24 keys, matrix cores)", MSCORE_N,
             bytes_score_mse(32), "keys/s"),
            (prod_score_setup, "score_prod b=3 Q=1 (2^24 keys)", MSCORE_N, bytes_score_prod(1), "keys/s")):
        fn = setup(torch, tq, synth, library_codebook)
        ms = time_rotating(torch, [fn], reps)
        ms_call = time_region(torch, fn, reps, flush)
        del fn
        torch.cuda.empty_cache()
        e = kernel_entry(name, units, unit_bytes, ms, unit)
        e["ms_flushed_call"] = round(ms_call, 4)
        out.append(e)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ decode attention

ATT_HEADS, ATT_TOKENS = 8, 32768


ATT_LAYERS = 32


def attend_setup(torch, tq, synth, library_codebook, b, layers=1):
    """Decode attention over a KV cache of `layers` layers, each 8 KV heads x
    32,768 tokens x d = 128 bfloat16 (per-channel scales), TurboQuant_mse
    b-bit keys and values, 32 query heads (4 per KV head).  One layer is
    encoded and its records copied to the other layers (distinct memory,
    same content).  Returns the call that runs attention over every layer in
    turn, one layer after the other on the stream."""
    g = synth.rng(40 + b)
    k, v = synth.torch_kv_cache(ATT_HEADS, ATT_TOKENS, D, seed=3, device="cuda")
    c32, t32 = library_codebook(D, b)
    qk = tq.Quantizer.create(D, D, b, "mse", synth.rht_signs(g, D), None, c32, t32, device="cuda")
    qv = tq.Quantizer.create(D, D, b, "mse", synth.rht_signs(g, D), None, c32, t32, device="cuda")
    krec = tq.encode(qk, k.reshape(-1, D))
    vrec = tq.encode(qv, v.reshape(-1, D))
    del k, v

    def copy(rec):
        return {key: (None if t is None else t.clone()) for key, t in rec.items()}

    kl = [krec] + [copy(krec) for _ in range(layers - 1)]
    vl = [vrec] + [copy(vrec) for _ in range(layers - 1)]
    q = torch.from_numpy(g.standard_normal((QHEADS, D)).astype("float32")).to("cuda")
    out = torch.empty((layers, QHEADS, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_attend_workspace(qk, ATT_HEADS, QHEADS // ATT_HEADS, ATT_TOKENS),
                     dtype=torch.uint8, device="cuda")

    def run():
        for i in range(layers):
            tq.tq_attend(qk, kl[i], qv, vl[i], q, ATT_HEADS, out[i], ws)
    return run


def bytes_attend(b):   # per (token, KV head): key and value records with their norms
    return 2 * (b * D // 8 + 4)


def attend_headline(torch, tq, synth, library_codebook, reps, flush):
    """One layer per call, and a pass over 32 layers (1.2 GB of records at
    b = 4, far above the MALL) as one timed region."""
    out = []
    for b in (2, 4):
        for layers in (1, ATT_LAYERS):
            fn = attend_setup(torch, tq, synth, library_codebook, b, layers)
            ms = time_region(torch, fn, reps if layers == 1 else max(3, reps // 8), flush)
            del fn
            torch.cuda.empty_cache()
            e = kernel_entry(f"attend mse b={b} K+V, {layers} layer(s) x 8 KV heads x 32768 tokens, 32 q heads",
                             layers * ATT_HEADS * ATT_TOKENS, bytes_attend(b), ms, "tokens/s")
            e["layers"] = layers
            e["ms_per_layer"] = round(ms / layers, 4)
            out.append(e)
    return out


# ------------------------------------------------------------------ rotation variants

def rotation_comparison(torch, tq, synth, library_codebook, reps, flush):
    """The prefill-scale key batch (8 x 131,072 bfloat16 rows, outlier
    channels) with the RHT, 2-D Givens and 4-D quaternion rotations at equal
    bits: TurboQuant_prod b = 3 encode time, and the relative distortion
    ||x - x~||^2 / ||x||^2 of b = 3 TurboQuant_mse on those keys and on
    one-hot rows (the worst case the Hadamard transform guards against)."""
    x = synth.torch_gaussian(N_KEYS, D, seed=4, device="cuda", dtype=torch.bfloat16, outliers=True)
    xf = x.float()
    onehot = torch.eye(D, device="cuda").repeat(64, 1)
    g = synth.rng(6)
    s_bits, _ = synth.qjl_matrix(g, D)
    c2, t2 = library_codebook(D, B_BITS - 1)
    c3, t3 = library_codebook(D, B_BITS)
    kinds = ("rht", "givens", "quat")
    qps, dists = [], []
    for kind in kinds:
        signs = synth.rht_signs(g, D)
        rot = None if kind == "rht" else (synth.givens_params(g, D) if kind == "givens"
                                          else synth.quaternion_params(g, D))
        qps.append(tq.Quantizer.create(D, D, B_BITS, "prod", signs, s_bits, c2, t2, device="cuda",
                                       rotation=kind, rot=rot))
        qm = tq.Quantizer.create(D, D, B_BITS, "mse", signs, None, c3, t3, device="cuda", rotation=kind, rot=rot)
        dist = []
        for rows in (xf, onehot):
            dec = tq.decode(qm, tq.encode(qm, rows))
            dist.append(((rows - dec).pow(2).sum(1) / rows.pow(2).sum(1)).mean().item())
        dists.append(dist)
    # the three encoders timed call by call in turn, so that all of them see
    # the same clock and memory state
    recs = [qp.alloc_codes(N_KEYS) for qp in qps]
    fns = [(lambda qp=qp, rec=rec: tq.tq_encode_prod(qp, x, rec)) for qp, rec in zip(qps, recs)]
    ms_all = time_interleaved(torch, fns, reps, flush)
    out = []
    for kind, ms, dist in zip(kinds, ms_all, dists):
        out.append({"rotation": kind, "encode_prod_b3_ms": round(ms, 4),
                    "encode_prod_b3_GB/s": round(N_KEYS * bytes_encode_prod() / (ms * 1e-3) / 1e9, 1),
                    "mse_b3_distortion_keys": round(dist[0], 5), "mse_b3_distortion_onehot": round(dist[1], 5)})
    del recs, x, xf
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ outlier-channel split

def split_comparison(torch, tq, synth, library_codebook, reps, flush):
    """The key batch (outlier channels 0..3 x 20) quantised with an
    outlier-channel split -- channels [0, 32) at one more bit than [32, 128),
    each range its own TurboQuant_mse instance -- against uniform bits:
    encode time (one call per range) and relative distortion."""
    x = synth.torch_gaussian(N_KEYS, D, seed=4, device="cuda", dtype=torch.bfloat16, outliers=True)
    xf = x.float()
    g = synth.rng(7)

    def quant(d_in, b):
        d = max(32, 1 << (d_in - 1).bit_length())
        c, t = library_codebook(d, b)
        return tq.Quantizer.create(d_in, d, b, "mse", synth.rht_signs(g, d), None, c, t, device="cuda")

    layouts = (("uniform b=2", [(0, 128, 2)]), ("split 32x3 + 96x2 (2.25 bits)", [(0, 32, 3), (32, 96, 2)]),
               ("uniform b=3", [(0, 128, 3)]), ("split 32x4 + 96x3 (3.25 bits)", [(0, 32, 4), (32, 96, 3)]),
               ("uniform b=4", [(0, 128, 4)]))
    sqs, dists = [], []
    for name, layout in layouts:
        sq = tq.SplitQuantizer([(c0, quant(w, b)) for c0, w, b in layout])
        recs = sq.encode(x)
        dec = sq.decode(recs)
        dists.append(((xf - dec).pow(2).sum(1) / xf.pow(2).sum(1)).mean().item())
        sqs.append(sq)
        del recs, dec
    # the layouts timed call by call in turn (same clock and memory state)
    ms_all = time_interleaved(torch, [(lambda sq=sq: sq.encode(x)) for sq in sqs], reps, flush)
    out = []
    for (name, layout), ms, dist in zip(layouts, ms_all, dists):
        bits = sum(w * b for _, w, b in layout) / D
        out.append({"layout": name, "bits": bits, "encode_ms": round(ms, 4), "distortion": round(dist, 5)})
    del x, xf
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ nearest-neighbour search

SEARCH_N, SEARCH_DIN, SEARCH_D, SEARCH_Q, SEARCH_K = 1_000_000, 1536, 2048, 1000, 10


def search_rows(torch, synth):
    """1,000,000 clustered unit rows (d_in = 1,536) and 1,000 queries drawn the
    same way; returns (rows, queries) on the device."""
    x, cvec = synth.torch_clustered_unit(SEARCH_N, SEARCH_DIN, 1000, seed=5, device="cuda")
    g = synth.rng(5)
    qh, _ = synth.clustered_unit(g, SEARCH_Q, SEARCH_DIN, 1000, centre_vectors=cvec.cpu().numpy())
    return x, torch.from_numpy(qh).to("cuda")


def search_setup(torch, tq, synth, library_codebook, b, x, qd):
    """TurboQuant_mse b-bit database of the rows (padded to d = 2,048) and the
    top-10 call for all queries; returns (call, idx)."""
    c32, t32 = library_codebook(SEARCH_D, b)
    q = tq.Quantizer.create(SEARCH_DIN, SEARCH_D, b, "mse", synth.rht_signs(synth.rng(50 + b), SEARCH_D),
                            None, c32, t32, device="cuda")
    rec = tq.encode(q, x)
    idx = torch.empty((SEARCH_Q, SEARCH_K), dtype=torch.int64, device="cuda")
    vals = torch.empty((SEARCH_Q, SEARCH_K), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_topk_workspace(q, SEARCH_Q, SEARCH_N, SEARCH_K), dtype=torch.uint8, device="cuda")
    return (lambda: tq.tq_topk(q, qd, rec, SEARCH_K, idx, vals, ws)), idx


def search_headline(torch, tq, synth, library_codebook, reps, flush):
    """Top-10 search of 1,000 queries over 1,000,000 clustered unit rows
    (d_in = 1,536 padded to 2,048), TurboQuant_mse b = 2 and 4; reports
    queries/s, recall@10 against float32 brute force on the unquantised rows,
    and the estimator's arithmetic rate (2 Q N d flops per search)."""
    x, qd = search_rows(torch, synth)
    exact = torch.topk(qd @ x.T, SEARCH_K, dim=1).indices
    out = []
    for b in (2, 4):
        fn, idx = search_setup(torch, tq, synth, library_codebook, b, x, qd)
        ms = time_region(torch, fn, reps, flush)
        recall = (idx[:, :, None] == exact[:, None, :]).any(-1).float().mean().item()
        out.append({"kernel": f"search mse b={b}: 1000 queries x 1M rows (1536->2048), top-10",
                    "ms": round(ms, 3), "queries/s": round(SEARCH_Q / (ms * 1e-3), 1),
                    "recall@10": round(recall, 4),
                    "estimate_TFLOP/s": round(2.0 * SEARCH_Q * SEARCH_N * SEARCH_D / (ms * 1e-3) / 1e12, 1)})
        del fn, idx
        torch.cuda.empty_cache()
    del x, exact
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ CPU oracle baseline

def _host_threads():
    """(os.cpu_count(), the CPU affinity mask, the BLAS thread count)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    try:
        mask = sorted(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        mask = list(range(os.cpu_count() or 1))
    return os.cpu_count(), mask, blas


def _mask_text(mask):
    """Compact text of a CPU list (0-7,16-23)."""
    runs, start = [], None
    for i, c in enumerate(mask):
        if start is None:
            start = c
        if i + 1 == len(mask) or mask[i + 1] != c + 1:
            runs.append(f"{start}" if start == c else f"{start}-{c}")
            start = None
    return ",".join(runs)


def _blas_limit(threads):
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=threads)


def _oracle_step_rate(O, x, h, seconds):
    """Keys/s of the oracle over the step's sample (encode_prod + decode +
    the 4 query heads' scores, chunks of 4,096 keys), cycled for `seconds`."""
    c32, t32, s64, signs = h["c32"], h["t32"], h["s64"], h["signs"]
    qh = h["q"][:4].astype("float64")
    done, t0, chunk = 0, time.time(), 4096
    while time.time() - t0 < seconds:
        off = done % x.shape[0]
        xs = x[off:off + chunk]
        e = O.encode_prod(xs, D, signs, c32, t32, s64)
        O.decode(e["codes"], e["norms"], D, D, signs, c32, e["qjl"], e["rnorms"], s64)
        O.score(qh, e["codes"], e["norms"], D, signs, c32, e["qjl"], e["rnorms"], s64)
        done += chunk
    dt = time.time() - t0
    return done / dt, done, dt


def _oracle_configs(O, synth, np):
    """The oracle on every measured configuration, in full (4,096 x 128
    TurboQuant_mse b = 3 encode + decode) or on a fixed subset: 4,096 float16
    keys with outliers, TurboQuant_prod b = 4, 32 queries' scores; one KV
    head x 4,096 tokens of the KV cache, decode attention for its 4 query
    heads (b = 2 and 4); 8,192 bfloat16 keys with outliers, TurboQuant_prod
    b = 3 encode; 10,000 clustered rows (1,536 -> 2,048), TurboQuant_mse b = 2
    encode, then 10 queries' scores and top-10.  Returns per-unit rates."""
    out = {}

    def timed(fn):
        t0 = time.time()
        fn()
        return time.time() - t0

    def cb(d, m):
        c, t, _, _ = O.lloyd_max(d, m)
        return O.codebook_f32(c, t)

    g = synth.rng(0)
    x = synth.gaussian(g, 4096, D).astype(np.float64)
    s = synth.rht_signs(g, D)
    c3, t3 = cb(D, 3)

    def c1():
        e = O.encode_mse(x, D, s, c3, t3)
        O.decode(e["codes"], e["norms"], D, D, s, c3)
    dt = timed(c1)
    out["C1 mse b=3 encode+decode, 4,096 x 128 f32 (full)"] = {"vectors/s": round(4096 / dt, 1), "s": round(dt, 2)}

    g = synth.rng(2)
    x = synth.with_outliers(synth.gaussian(g, 4096, D)).astype(np.float16).astype(np.float64)
    s = synth.rht_signs(g, D)
    _, s64 = synth.qjl_matrix(g, D)
    qh = g.standard_normal((32, D))
    c, t = cb(D, 3)

    def c2():
        e = O.encode_prod(x, D, s, c, t, s64)
        O.score(qh, e["codes"], e["norms"], D, s, c, e["qjl"], e["rnorms"], s64)
    dt = timed(c2)
    out["C2 prod b=4 encode + 32 queries' scores, 4,096 f16 keys"] = {"keys/s": round(4096 / dt, 1),
                                                                     "s": round(dt, 2)}

    k, v = synth.kv_cache(synth.rng(3), 1, 4096, D)
    k, v = k[0].astype(np.float64), v[0].astype(np.float64)
    g = synth.rng(43)
    qh = g.standard_normal((4, D))
    for b in (2, 4):
        sk, sv = synth.rht_signs(g, D), synth.rht_signs(g, D)
        c, t = cb(D, b)

        def c3f():
            ek = O.encode_mse(k, D, sk, c, t)
            ev = O.encode_mse(v, D, sv, c, t)
            O.decode_attention(qh, 1, dict(ek, signs=sk, centroids=c), dict(ev, signs=sv, centroids=c), D, D,
                               1.0 / math.sqrt(D))
        dt = timed(c3f)
        out[f"C3 mse b={b} K+V encode + attention, 1 KV head x 4,096 tokens, 4 q heads"] = {
            "tokens/s": round(4096 / dt, 1), "s": round(dt, 2)}

    g = synth.rng(4)
    x = synth.with_outliers(synth.gaussian(g, 8192, D))
    import torch
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    s = synth.rht_signs(g, D)
    _, s64 = synth.qjl_matrix(g, D)
    c, t = cb(D, 2)
    dt = timed(lambda: O.encode_prod(x, D, s, c, t, s64))
    out["C4 prod b=3 encode, 8,192 bf16 keys"] = {"vectors/s": round(8192 / dt, 1), "s": round(dt, 2)}

    g = synth.rng(5)
    x, cv = synth.clustered_unit(g, 10000, SEARCH_DIN, 1000)
    qh, _ = synth.clustered_unit(g, 10, SEARCH_DIN, 1000, centre_vectors=cv)
    s = synth.rht_signs(g, SEARCH_D)
    c, t = cb(SEARCH_D, 2)

    def c5():
        e = O.encode_mse(x.astype(np.float64), SEARCH_D, s, c, t)
        est = O.score(qh.astype(np.float64), e["codes"], e["norms"], SEARCH_D, s, c)
        O.topk(est, SEARCH_K)
    dt = timed(c5)
    out["C5 mse b=2 encode + 10 queries' scores + top-10, 10,000 rows 1,536 -> 2,048"] = {
        "rows/s": round(10000 / dt, 1), "s": round(dt, 2)}
    return out


def cpu_baseline(w, synth):
    """The oracle (test infrastructure, as it stands) timed on the host.
    value: keys/s of the step (encode_prod + decode + the GQA scores) on the
    first 65,536 keys of KV head 0 with its 4 query heads, cycled in chunks of
    4,096 for ~10 s with every host core available to BLAS; the same sample
    again with BLAS held to one thread; then every configuration's full run
    or subset (all cores)."""
    import numpy as np
    from oracle import tq_oracle as O
    ncpu, mask, blas = _host_threads()
    h = w["host"]
    x = w["x"][:65536].float().cpu().numpy().astype(np.float64)
    rate_all, done, dt = _oracle_step_rate(O, x, h, 10.0)
    with _blas_limit(1):
        rate_one, done1, dt1 = _oracle_step_rate(O, x, h, 8.0)
    configs = _oracle_configs(O, synth, np)
    return {"value": round(rate_all, 1), "unit": "keys/s", "cores": int(blas or ncpu), "kind": "oracle",
            "sample": f"first 65,536 keys of KV head 0 cycled in chunks of 4,096 (encode_prod + decode + "
                      f"its 4 query heads' scores): {done} keys in {dt:.1f} s",
            "host": {"os_cpu_count": ncpu, "affinity": _mask_text(mask), "affinity_cpus": len(mask),
                     "blas_threads": blas},
            "single_thread": {"value": round(rate_one, 1), "unit": "keys/s", "cores": 1,
                              "sample": f"same sample, BLAS limited to 1 thread: {done1} keys in {dt1:.1f} s"},
            "configs": configs}


# ------------------------------------------------------------------ bandwidth probes

def probe_lib():
    """libtqprobe.so: streaming read, write and read/write-mix kernels of
    known byte counts (built beside libtq.so)."""
    import ctypes
    path = os.path.join(ROOT, "embedding_vector_quantization_amd", "libtqprobe.so")
    L = ctypes.CDLL(path)
    vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
    L.tqp_read.argtypes = [vp, i64, vp, vp]
    L.tqp_write.argtypes = [vp, i64, u32, vp]
    L.tqp_mixed.argtypes = [vp, i64, vp, i64, i64, ctypes.c_int32, vp]
    L.tqp_write_once.argtypes = [vp, i64, u32, vp]
    L.tqp_mixed_once.argtypes = [vp, i64, vp, i64, i64, vp]
    L.tqp_issue.argtypes = [ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32, vp]
    for f in (L.tqp_read, L.tqp_write, L.tqp_mixed, L.tqp_write_once, L.tqp_mixed_once, L.tqp_issue):
        f.restype = ctypes.c_int
    return L


# name, bytes read per unit, bytes written per unit, units, row-wise stores,
# one-shot workgroups (else persistent ones striding over the buffer)
PROBES = (
    ("read only, 1 GiB", 1 << 30, 0, 1, 0, 0),
    ("write only, 1 GiB", 0, 1 << 30, 1, 0, 0),
    ("read 64 B + write 512 B per unit, 2^20 units (decode to float32)", 64, 512, 1 << 20, 0, 0),
    ("read 64 B + write 512 B per unit, 2^20 units, stores of 64 B in each of 16 rows", 64, 512, 1 << 20, 1, 0),
    ("read 256 B + write 64 B per unit, 2^20 units (16-bit rows to records)", 256, 64, 1 << 20, 0, 0),
    ("read 512 B + write 64 B per unit, 2^21 units (float32 rows to records)", 512, 64, 1 << 21, 0, 0),
    ("write only, 1 GiB, one-shot workgroups", 0, 1 << 30, 1, 0, 1),
    ("read 64 B + write 512 B per unit, 2^20 units, one-shot 16-wave workgroups", 64, 512, 1 << 20, 0, 1),
)
DECODE_PROBE, DECODE_PROBE_ONCE = PROBES[2][0], PROBES[7][0]


def probe_calls(torch):
    """[(name, bytes moved, call)] over two 1 GiB device buffers."""
    L = probe_lib()
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"bandwidth probe failed: hip error {rc}")

    calls = []
    for name, rd, wr, units, rows, once in PROBES:
        if wr == 0:
            fn = (lambda: check(L.tqp_read(a.data_ptr(), 1 << 30, sink.data_ptr(), stream)))
        elif rd == 0:
            write = L.tqp_write_once if once else L.tqp_write
            fn = (lambda write=write: check(write(b.data_ptr(), 1 << 30, 7, stream)))
        elif once:
            fn = (lambda rd=rd, wr=wr, units=units: check(L.tqp_mixed_once(a.data_ptr(), rd, b.data_ptr(), wr, units,
                                                                            stream)))
        else:
            fn = (lambda rd=rd, wr=wr, units=units, rows=rows: check(L.tqp_mixed(a.data_ptr(), rd, b.data_ptr(), wr,
                                                                                 units, rows, stream)))
        calls.append((name, (rd + wr) * units, fn))
    return calls, (a, b, sink)


def bandwidth_probes(torch, reps, flush):
    """Rates the memory system reaches for pure read and write streams and
    for the read/write mixes of the kernels, cold caches, HIP events."""
    calls, keep = probe_calls(torch)
    ms_all = time_interleaved(torch, [fn for _, _, fn in calls], reps, flush)
    out = []
    for (name, nbytes, _), ms in zip(calls, ms_all):
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.append({"probe": name, "bytes": nbytes, "ms": round(ms, 4), "GB/s": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
    del keep
    torch.cuda.empty_cache()
    return out


ISSUE_MODES = ("MFMA only", "FMA only", "both in every wave")
ISSUE_ITERS = 20000


def issue_calls(torch, L=None):
    """[(waves per SIMD, mode, call)] for the issue probe: 4 MFMAs or 64
    FMAs per loop trip, 1,024 or 2,048 workgroups of four waves."""
    L = L or probe_lib()
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def call(mode, blocks):
        rc = L.tqp_issue(mode, out.data_ptr(), blocks, ISSUE_ITERS, stream)
        if rc != 0:
            raise RuntimeError(f"issue probe failed: hip error {rc}")

    calls = []
    for blocks in (1024, 2048):
        for mode in range(3):
            calls.append((blocks * 4 // 1024, mode, lambda mode=mode, blocks=blocks: call(mode, blocks)))
    return calls, out


def issue_probe(torch, reps):
    """How much matrix-core work a SIMD overlaps with vector work of the
    same wave: loop time per wave and trip (ns) of the issue probe's three
    modes, and the fraction of the MFMA body's time that disappears when
    both bodies share a wave (0: the two add up; 1: full overlap)."""
    calls, keep = issue_calls(torch)
    ms_all = time_interleaved(torch, [fn for _, _, fn in calls], reps, lambda: None)
    res = {}
    for (wps, mode, _), ms in zip(calls, ms_all):
        res.setdefault(wps, {})[mode] = ms * 1e6 / ISSUE_ITERS / wps     # ns per wave-trip
    out = []
    for wps, t in sorted(res.items()):
        out.append({"waves_per_simd": wps,
                    "ns_per_wave_trip": {ISSUE_MODES[m]: round(t[m], 2) for m in range(3)},
                    "mfma_hidden_same_wave": round((t[0] + t[1] - t[2]) / t[0], 3)})
    del keep
    return out


# ------------------------------------------------------------------ traffic from rocprofv3

def traffic_for(kernel: str):
    """HBM bytes per launch and VALU instructions per launch from the
    committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE scaled by
    the copy-kernel calibration; SQ_INSTS_VALU), or None when missing or when
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("source_sha") != source_hash():
        return None
    return data.get("kernels", {}).get(kernel)


# VALU issue peak: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one 64-lane
# instruction per SIMD every 4 cycles), in lane-operations per second.
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9


def add_valu(entry, name, launches=1):
    """The VALU roofline fraction of a kernel entry: SQ_INSTS_VALU per launch
    (from the committed counter summary, while the kernel sources match) x 64
    lane-operations x launches / the entry's time / the VALU issue peak."""
    prof = traffic_for(name)
    if prof and prof.get("valu_insts_per_launch"):
        ops = prof["valu_insts_per_launch"] * 64 * launches
        entry["valu_lane_ops_per_unit"] = round(ops / entry["units"], 1)
        entry["valu_frac"] = round(ops / (entry["ms"] * 1e-3) / VALU_PEAK_LANE_OPS, 4)


# ------------------------------------------------------------------ main

def profile_only(args, torch, tq, synth, library_codebook):
    """One kernel (or the probes) R times with the cache flush before each
    call, as the timed loops of the full run do, for rocprofv3."""
    name = args.profile_kernel
    flush = CacheFlush(torch)
    if name == "copy":
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(args.reps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "copy", "bytes_each_way": a.numel() * 4, "reps": args.reps}))
        return
    if name == "probes":
        calls, keep = probe_calls(torch)
        icalls, ikeep = issue_calls(torch)
        fns = [fn for _, _, fn in calls] + [fn for _, _, fn in icalls]
    elif name in ("attend2", "attend4", "attend2x32", "attend4x32"):
        fns = [attend_setup(torch, tq, synth, library_codebook, int(name[6]), 32 if name.endswith("x32") else 1)]
    elif name in ("search2", "search4"):
        x, qd = search_rows(torch, synth)
        fns = [search_setup(torch, tq, synth, library_codebook, int(name[-1]), x, qd)[0]]
    elif name in ("encode_mse", "score_mse", "score_prod_q1"):
        setup = {"encode_mse": mse_encode_setup, "score_mse": mse_score_setup,
                 "score_prod_q1": prod_score_setup}[name]
        fns = [setup(torch, tq, synth, library_codebook)]
    else:
        w = make_workload(torch, tq, synth, library_codebook)
        run_step(tq, w)
        step_fn = {"encode_prod": run_encode, "decode": run_decode, "score": run_score}[name]
        fns = [lambda: step_fn(tq, w)]
    for _ in range(args.reps):
        for call in fns:
            flush()
            call()
    torch.cuda.synchronize()
    print(json.dumps({"profile": name, "reps": args.reps}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the quantiser shards by rows with no communication, see the design notes)",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import torch

    import numpy as np

    import synth
    import embedding_vector_quantization_amd as tq

    def library_codebook(d, m):
        c, t, _ = tq.tq_make_codebook(d, m)
        return c.astype(np.float32), t.astype(np.float32)

    tq.lib()
    if args.profile_kernel:
        profile_only(args, torch, tq, synth, library_codebook)
        return

    w = make_workload(torch, tq, synth, library_codebook)
    for _ in range(args.warmup):
        run_step(tq, w)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        run_step(tq, w)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    print(f"[bench] step {ms_step:.4f} ms over {args.steps} steps", file=sys.stderr, flush=True)

    flush = CacheFlush(torch)
    reps = max(5, args.steps)
    ms_enc, ms_dec, ms_sc = time_interleaved(
        torch, [lambda: run_encode(tq, w), lambda: run_decode(tq, w), lambda: run_score(tq, w)], reps, flush)
    # the same kernels back to back over rotating buffer copies (the primary
    # figure: the kernel's own duration with inputs from HBM)
    copies = step_copies(torch, w, max(ROTATE_SETS.values()))
    ms_rot = [time_rotating(torch, [(lambda c=c: fn(tq, c)) for c in copies[:ROTATE_SETS[nm]]], reps)
              for nm, fn in (("encode_prod", run_encode), ("decode", run_decode), ("score", run_score))]
    del copies
    torch.cuda.empty_cache()
    kernels = [kernel_entry("encode_prod b=3 bf16", N_KEYS, bytes_encode_prod(), ms_rot[0]),
               kernel_entry("decode_prod b=3 -> f32", N_KEYS, bytes_decode_prod(), ms_rot[1]),
               kernel_entry("score_prod b=3 GQA 4 q/head (grouped)", N_KEYS, bytes_score_prod(4), ms_rot[2],
                            "keys/s")]
    for k, ms_call in zip(kernels, (ms_enc, ms_dec, ms_sc)):
        k["ms_flushed_call"] = round(ms_call, 4)
        k["hbm_frac_flushed_call"] = round(k["units"] * k["bytes_per_unit"] / (ms_call * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    names = ["encode_prod", "decode", "score"]
    for k, nm in zip(kernels, names):
        add_valu(k, nm)
    dom = max(range(3), key=lambda i: kernels[i]["ms"])
    dominant, dom_name = kernels[dom], names[dom]
    print("[bench] step kernels done", file=sys.stderr, flush=True)
    headline = mse_headline(torch, tq, synth, library_codebook, reps, flush)
    for k, nm in zip(headline, ("encode_mse", "score_mse")):
        add_valu(k, nm)
    add_valu(headline[4], "score_prod_q1")
    probes = bandwidth_probes(torch, reps, flush)
    issue = issue_probe(torch, 5)
    print("[bench] mse headline and probes done", file=sys.stderr, flush=True)
    attend = attend_headline(torch, tq, synth, library_codebook, reps, flush)
    for k in attend:
        if k["kernel"].startswith("attend mse b=2"):
            add_valu(k, "attend2x32", launches=k["layers"])
    print("[bench] attention done", file=sys.stderr, flush=True)
    search = search_headline(torch, tq, synth, library_codebook, max(3, reps // 4), flush)
    print("[bench] search done", file=sys.stderr, flush=True)
    rotations = rotation_comparison(torch, tq, synth, library_codebook, reps, flush)
    split = split_comparison(torch, tq, synth, library_codebook, reps, flush)
    prof = traffic_for(dom_name)
    mixed = {p["probe"]: p for p in probes}
    dec_probe = mixed[DECODE_PROBE]["GB/s"]
    dec_probe_once = mixed[DECODE_PROBE_ONCE]["GB/s"]

    line = {
        "metric": METRIC,
        "value": round(N_KEYS / (ms_step * 1e-3), 1),
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kv-keys prod b=3 d=128: 8 KV heads x 131072 tokens bf16, outlier channels x20; "
                               "step = encode_prod + decode (f32) + scores of 32 query heads (GQA 4:1)",
                   "keys": N_KEYS, "d": D, "b": B_BITS, "mode": "prod", "input_dtype": "bf16",
                   "query_heads": QHEADS},
        "roofline": {"bound": "hbm", "achieved": dominant["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": dominant["hbm_frac"], "traffic": (prof or {}).get("bytes_per_launch"),
                     "kernel": dom_name, "bytes_per_unit": dominant["bytes_per_unit"], "units_per_launch": N_KEYS,
                     "timing": "HIP event pair around back-to-back calls cycling over "
                               f"{ROTATE_SETS[dom_name]} copies of the buffers (inputs from HBM); "
                               "ms_flushed_call: event pair per call after a 2 GiB read flush"},
        "targets_d128_b3": {"encode_prod_hbm_frac": kernels[0]["hbm_frac"],
                            "score_grouped_prod_hbm_frac": kernels[2]["hbm_frac"],
                            "encode_mse_f32_hbm_frac": headline[0]["hbm_frac"],
                            "score_mse_q1_hbm_frac": headline[1]["hbm_frac"],
                            "score_prod_q1_hbm_frac": headline[4]["hbm_frac"],
                            "decode_vs_same_mix_probe": round(kernels[1]["hbm_frac_flushed_call"] * HBM_PEAK_GBS / dec_probe, 4),
                            "decode_vs_one_shot_mix_probe": round(
                                kernels[1]["hbm_frac_flushed_call"] * HBM_PEAK_GBS / dec_probe_once, 4)},
        "kernels": kernels,
        "mse_headline": headline,
        "bandwidth_probes": probes,
        "issue_probe": issue,
        "attend": attend,
        "search": search,
        "rotations": rotations,
        "outlier_split": split,
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.skip_cpu:
        print("[bench] cpu baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, synth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
