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

--profile-kernel NAME --reps R runs only that kernel R times (for rocprofv3
counter collection); NAME = encode_prod | decode | score | encode_mse |
score_mse | attend2 | attend4 | search2 | search4 | copy (a plain device copy
of known size, to calibrate FETCH_SIZE / WRITE_SIZE).
"""

from __future__ import annotations

import argparse
import hashlib
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
KERNEL_SOURCES = ["tq_encode.hip", "tq_decode.hip", "tq_score.hip", "tq_lut.h", "tq_device.h", "tq_internal.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--profile-kernel", default=None)
    ap.add_argument("--reps", type=int, default=5)
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "embedding_vector_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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


def time_region(torch, fn, reps):
    """Average milliseconds of one fn() call over reps calls, each bracketed
    by its own pair of HIP events on the current stream (the one every
    library call is issued on), so the idle gaps between calls are not
    counted: for a single-launch call this is the kernel's duration."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for start, end in ev:
        start.record(stream)
        fn()
        end.record(stream)
    torch.cuda.synchronize()
    return sum(start.elapsed_time(end) for start, end in ev) / reps


def time_interleaved(torch, fns, reps):
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
            start.record(stream)
            fn()
            end.record(stream)
    torch.cuda.synchronize()
    return [sum(row[i][0].elapsed_time(row[i][1]) for row in ev) / reps for i in range(len(fns))]


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


def mse_score_setup(torch, tq, synth, library_codebook):
    """One query against 2^24 TurboQuant_mse b = 3 keys; returns the call."""
    q, g = mse_quantizer(tq, synth, library_codebook)
    keys_src = synth.torch_gaussian(MSCORE_N, D, seed=2, device="cuda", dtype=torch.bfloat16)
    keys = q.alloc_codes(MSCORE_N)
    tq.tq_encode_mse(q, keys_src, keys)
    del keys_src
    query = torch.from_numpy(g.standard_normal((1, D)).astype("float32")).to("cuda")
    scores = torch.empty((1, MSCORE_N), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_score_workspace(q, 1), dtype=torch.uint8, device="cuda")
    return lambda: tq.tq_score(q, query, keys, scores, ws)


def mse_headline(torch, tq, synth, library_codebook, reps):
    enc = mse_encode_setup(torch, tq, synth, library_codebook)
    ms_enc = time_region(torch, enc, reps)
    del enc
    torch.cuda.empty_cache()
    sc = mse_score_setup(torch, tq, synth, library_codebook)
    ms_sc = time_region(torch, sc, reps)
    del sc
    torch.cuda.synchronize()
    return [kernel_entry("encode_mse b=3 f32 (2^22 rows)", MENC_N, bytes_encode_mse_f32(), ms_enc),
            kernel_entry("score_mse b=3 Q=1 (2^24 keys)", MSCORE_N, bytes_score_mse(1), ms_sc, "keys/s")]


# ------------------------------------------------------------------ decode attention

ATT_HEADS, ATT_TOKENS = 8, 32768


def attend_setup(torch, tq, synth, library_codebook, b):
    """Decode attention over one layer's KV cache: 8 KV heads x 32,768 tokens
    x d = 128 bfloat16 (per-channel scales), TurboQuant_mse b-bit keys and
    values, 32 query heads (4 per KV head); returns the call."""
    g = synth.rng(40 + b)
    k, v = synth.torch_kv_cache(ATT_HEADS, ATT_TOKENS, D, seed=3, device="cuda")
    c32, t32 = library_codebook(D, b)
    qk = tq.Quantizer.create(D, D, b, "mse", synth.rht_signs(g, D), None, c32, t32, device="cuda")
    qv = tq.Quantizer.create(D, D, b, "mse", synth.rht_signs(g, D), None, c32, t32, device="cuda")
    krec = tq.encode(qk, k.reshape(-1, D))
    vrec = tq.encode(qv, v.reshape(-1, D))
    del k, v
    q = torch.from_numpy(g.standard_normal((QHEADS, D)).astype("float32")).to("cuda")
    out = torch.empty((QHEADS, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_attend_workspace(qk, ATT_HEADS, QHEADS // ATT_HEADS, ATT_TOKENS),
                     dtype=torch.uint8, device="cuda")
    return lambda: tq.tq_attend(qk, krec, qv, vrec, q, ATT_HEADS, out, ws)


def bytes_attend(b):   # per (token, KV head): key and value records with their norms
    return 2 * (b * D // 8 + 4)


def attend_headline(torch, tq, synth, library_codebook, reps):
    out = []
    for b in (2, 4):
        fn = attend_setup(torch, tq, synth, library_codebook, b)
        ms = time_region(torch, fn, reps)
        del fn
        torch.cuda.empty_cache()
        out.append(kernel_entry(f"attend mse b={b} K+V, 8 KV heads x 32768 tokens, 32 q heads",
                                ATT_HEADS * ATT_TOKENS, bytes_attend(b), ms, "tokens/s"))
    return out


# ------------------------------------------------------------------ rotation variants

def rotation_comparison(torch, tq, synth, library_codebook, reps):
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
    ms_all = time_interleaved(torch, fns, reps)
    out = []
    for kind, ms, dist in zip(kinds, ms_all, dists):
        out.append({"rotation": kind, "encode_prod_b3_ms": round(ms, 4),
                    "encode_prod_b3_GB/s": round(N_KEYS * bytes_encode_prod() / (ms * 1e-3) / 1e9, 1),
                    "mse_b3_distortion_keys": round(dist[0], 5), "mse_b3_distortion_onehot": round(dist[1], 5)})
    del recs, x, xf
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ outlier-channel split

def split_comparison(torch, tq, synth, library_codebook, reps):
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
    ms_all = time_interleaved(torch, [(lambda sq=sq: sq.encode(x)) for sq in sqs], reps)
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


def search_headline(torch, tq, synth, library_codebook, reps):
    """Top-10 search of 1,000 queries over 1,000,000 clustered unit rows
    (d_in = 1,536 padded to 2,048), TurboQuant_mse b = 2 and 4; reports
    queries/s, recall@10 against float32 brute force on the unquantised rows,
    and the estimator's arithmetic rate (2 Q N d flops per search)."""
    x, qd = search_rows(torch, synth)
    exact = torch.topk(qd @ x.T, SEARCH_K, dim=1).indices
    out = []
    for b in (2, 4):
        fn, idx = search_setup(torch, tq, synth, library_codebook, b, x, qd)
        ms = time_region(torch, fn, reps)
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

def cpu_baseline(w):
    """The oracle (test infrastructure) on a bounded sample of the same
    workload: encode_prod + decode + GQA scores for chunks of 4,096 keys of
    KV head 0 with its 4 queries, cycling over 65,536 keys for ~12 s."""
    import numpy as np
    from oracle import tq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    h = w["host"]
    x = w["x"][:65536].float().cpu().numpy().astype(np.float64)
    c32, t32, s64, signs = h["c32"], h["t32"], h["s64"], h["signs"]
    qh = h["q"][:4].astype(np.float64)
    done, t0, chunk = 0, time.time(), 4096
    while time.time() - t0 < 12.0:   # cycle over the sample for about 12 s
        off = done % x.shape[0]
        xs = x[off:off + chunk]
        e = O.encode_prod(xs, D, signs, c32, t32, s64)
        O.decode(e["codes"], e["norms"], D, D, signs, c32, e["qjl"], e["rnorms"], s64)
        O.score(qh, e["codes"], e["norms"], D, signs, c32, e["qjl"], e["rnorms"], s64)
        done += chunk
    dt = time.time() - t0
    return {"value": round(done / dt, 1), "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first 65,536 keys of KV head 0 cycled in chunks of 4,096 (encode_prod + decode + "
                      f"its 4 query heads' scores): {done} keys in {dt:.1f} s"}


# ------------------------------------------------------------------ traffic from rocprofv3

def traffic_for(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel calibration), or None
    when it is missing or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        return None
    if data.get("source_sha") != source_hash():
        return None
    entry = data.get("kernels", {}).get(kernel)
    return None if entry is None else entry.get("bytes_per_launch")


# ------------------------------------------------------------------ main

def profile_only(args, torch, tq, synth, library_codebook):
    name = args.profile_kernel
    if name == "copy":
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        b = torch.empty_like(a)
        for _ in range(args.reps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "copy", "bytes_each_way": a.numel() * 4, "reps": args.reps}))
        return
    if name in ("attend2", "attend4"):
        fn = attend_setup(torch, tq, synth, library_codebook, int(name[-1]))
        for _ in range(args.reps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"profile": name, "reps": args.reps}))
        return
    if name in ("search2", "search4"):
        x, qd = search_rows(torch, synth)
        fn, _ = search_setup(torch, tq, synth, library_codebook, int(name[-1]), x, qd)
        for _ in range(args.reps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"profile": name, "reps": args.reps}))
        return
    if name in ("encode_mse", "score_mse"):
        setup = mse_encode_setup if name == "encode_mse" else mse_score_setup
        fn = setup(torch, tq, synth, library_codebook)
        for _ in range(args.reps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"profile": name, "reps": args.reps}))
        return
    w = make_workload(torch, tq, synth, library_codebook)
    run_step(tq, w)
    fn = {"encode_prod": run_encode, "decode": run_decode, "score": run_score}[name]
    for _ in range(args.reps):
        fn(tq, w)
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

    reps = max(5, args.steps)
    ms_enc = time_region(torch, lambda: run_encode(tq, w), reps)
    ms_dec = time_region(torch, lambda: run_decode(tq, w), reps)
    ms_sc = time_region(torch, lambda: run_score(tq, w), reps)
    kernels = [kernel_entry("encode_prod b=3 bf16", N_KEYS, bytes_encode_prod(), ms_enc),
               kernel_entry("decode_prod b=3 -> f32", N_KEYS, bytes_decode_prod(), ms_dec),
               kernel_entry("score_prod b=3 GQA 4 q/head (grouped)", N_KEYS, bytes_score_prod(4), ms_sc,
                            "keys/s")]
    dominant = max(kernels, key=lambda k: k["ms"])
    dom_name = {kernels[0]["kernel"]: "encode_prod", kernels[1]["kernel"]: "decode",
                kernels[2]["kernel"]: "score"}[dominant["kernel"]]
    headline = mse_headline(torch, tq, synth, library_codebook, reps)
    attend = attend_headline(torch, tq, synth, library_codebook, reps)
    search = search_headline(torch, tq, synth, library_codebook, max(3, reps // 4))
    rotations = rotation_comparison(torch, tq, synth, library_codebook, reps)
    split = split_comparison(torch, tq, synth, library_codebook, reps)
    traffic = traffic_for(dom_name)

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
                     "frac": dominant["hbm_frac"], "traffic": traffic, "kernel": dom_name,
                     "bytes_per_unit": dominant["bytes_per_unit"], "units_per_launch": N_KEYS},
        "kernels": kernels,
        "mse_headline": headline,
        "attend": attend,
        "search": search,
        "rotations": rotations,
        "outlier_split": split,
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.skip_cpu:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
