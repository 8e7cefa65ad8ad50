"""ctypes binding of libtq (include/tq.h).  Argument marshalling only: every
step of the quantiser runs in the HIP kernels of libtq.so.  PyTorch supplies
device memory and the current stream.

The functions carry the C names (tq_make_codebook, tq_encode_mse,
tq_encode_prod, tq_decode, tq_score_workspace, tq_score, tq_rht) and take
torch tensors; `Quantizer` holds the device-side parameters of one quantiser
(codebook, RHT signs, QJL matrix) and allocates outputs for convenience.
"""

from __future__ import annotations

import contextlib
import ctypes
import math
import os
from dataclasses import dataclass

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK, TQ_ERR_ARG, TQ_ERR_DIM, TQ_ERR_BITS = 0, -1, -2, -3
TQ_ERR_ALIGN, TQ_ERR_WORKSPACE, TQ_ERR_HIP, TQ_ERR_NOCONV = -4, -5, -6, -7
TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2
TQ_MSE, TQ_PROD = 0, 1
TQ_ROT_RHT, TQ_ROT_GIVENS, TQ_ROT_QUAT = 0, 1, 2

EXPORTED = ("tq_make_codebook", "tq_encode_mse", "tq_encode_prod", "tq_decode",
            "tq_score_workspace", "tq_score", "tq_score_grouped", "tq_score_accumulate", "tq_topk_workspace",
            "tq_topk",
            "tq_attend_workspace", "tq_attend", "tq_attend_noalloc",
            "tq_rht", "tq_status_string", "tq_version")


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class TqParams(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("d", ctypes.c_int32), ("m", ctypes.c_int32),
                ("rotation", ctypes.c_int32), ("centroids", ctypes.c_void_p),
                ("thresholds", ctypes.c_void_p), ("signs", ctypes.c_void_p),
                ("qjl_s", ctypes.c_void_p), ("rot", ctypes.c_void_p)]


class TqCodes(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("qjl", ctypes.c_void_p),
                ("norms", ctypes.c_void_p), ("rnorms", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libtq.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python embedding_vector_quantization_amd/csrc/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        pp, pc = ctypes.POINTER(TqParams), ctypes.POINTER(TqCodes)
        dp = ctypes.POINTER(ctypes.c_double)
        L.tq_make_codebook.argtypes = [i32, i32, dp, dp, dp]
        L.tq_make_codebook.restype = ctypes.c_int
        for name in ("tq_encode_mse", "tq_encode_prod"):
            f = getattr(L, name)
            f.argtypes = [pp, vp, i32, i64, i64, pc, vp]
            f.restype = ctypes.c_int
        L.tq_decode.argtypes = [pp, i32, pc, i64, vp, i64, vp]
        L.tq_decode.restype = ctypes.c_int
        L.tq_score_workspace.argtypes = [pp, i32, i64]
        L.tq_score_workspace.restype = sz
        L.tq_score.argtypes = [pp, i32, vp, i64, i64, pc, i64, vp, i64, vp, sz, vp]
        L.tq_score.restype = ctypes.c_int
        L.tq_score_grouped.argtypes = [pp, i32, vp, i64, i64, i64, pc, i64, vp, i64, vp, sz, vp]
        L.tq_score_grouped.restype = ctypes.c_int
        L.tq_score_accumulate.argtypes = L.tq_score_grouped.argtypes
        L.tq_score_accumulate.restype = ctypes.c_int
        L.tq_topk_workspace.argtypes = [pp, i32, i64, i64, i32]
        L.tq_topk_workspace.restype = sz
        L.tq_topk.argtypes = [pp, i32, vp, i64, i64, pc, i64, i32, vp, vp, vp, sz, vp]
        L.tq_topk.restype = ctypes.c_int
        L.tq_attend_workspace.argtypes = [pp, i32, i64, i64, i64]
        L.tq_attend_workspace.restype = sz
        L.tq_attend.argtypes = [pp, i32, pc, pp, pc, vp, i64, i64, i64, i64, ctypes.c_float, vp, i64, vp,
                                sz, vp]
        L.tq_attend.restype = ctypes.c_int
        L.tq_attend_noalloc.argtypes = [pp, i32, pc, pp, pc, vp, i64, i64, i64, i64, ctypes.c_float, vp, i64, vp]
        L.tq_attend_noalloc.restype = ctypes.c_int
        L.tq_rht.argtypes = [pp, vp, i64, vp, i64, i64, i32, vp]
        L.tq_rht.restype = ctypes.c_int
        L.tq_status_string.argtypes = [i32]
        L.tq_status_string.restype = ctypes.c_char_p
        L.tq_version.argtypes = []
        L.tq_version.restype = i32
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().tq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _on_stream(stream):
    """Context for the temporaries of a convenience call: inside it torch's
    caching allocator files new blocks under `stream`, the stream the library
    launches on, so a workspace freed when the call returns is not handed to
    work queued on another stream while the kernels still read it."""
    if stream is None:
        return contextlib.nullcontext()
    import torch
    return torch.cuda.stream(stream)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.float16: TQ_F16, torch.bfloat16: TQ_BF16}[t.dtype]


# --------------------------------------------------------------- parameters

def tq_make_codebook(d: int, m: int):
    """Host Lloyd-Max codebook: (centroids[2^m], thresholds[2^m-1], dmse),
    float64 numpy arrays."""
    c = np.zeros(1 << m, dtype=np.float64)
    t = np.zeros((1 << m) - 1, dtype=np.float64)
    dm = ctypes.c_double(0.0)
    st = lib().tq_make_codebook(int(d), int(m),
                                c.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                t.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                ctypes.byref(dm))
    _check(st, "tq_make_codebook")
    return c, t, dm.value


@dataclass
class Quantizer:
    """Device-side parameters of one quantiser (caller-owned torch tensors).

    mode: "mse" (m = b bits) or "prod" (m = b - 1 bits + the QJL plane)."""
    d_in: int
    d: int
    m: int
    mode: str
    centroids: object = None      # torch float32 [2^m] on the device
    thresholds: object = None     # torch float32 [2^m - 1]
    signs: object = None          # torch int8 [d]
    qjl_s: object = None          # torch int16 [d, d] (bfloat16 bit patterns)
    rotation: int = 0             # TQ_ROT_*
    rot: object = None            # torch float32 block rotation parameters

    @classmethod
    def create(cls, d_in, d, b, mode, signs, qjl_s_bits=None, centroids=None, thresholds=None,
               device="cuda", rotation="rht", rot=None):
        """Uploads the parameters.  `signs` int8 [d] (RHT), `qjl_s_bits`
        uint16 [d, d] bfloat16 patterns (prod), optional float codebook arrays
        (default: tq_make_codebook(d, m) rounded to float32); rotation "rht",
        "givens" (rot float32 [d/2, 2] of cos, sin) or "quat" (rot float32
        [d/4, 4] unit quaternions)."""
        import torch
        m = b if mode == "mse" else b - 1
        if m > 0 and centroids is None:
            centroids, thresholds, _ = tq_make_codebook(d, m)
        q = cls(d_in=d_in, d=d, m=m, mode=mode)
        if m > 0:
            q.centroids = torch.tensor(np.asarray(centroids, np.float32), device=device)
            q.thresholds = torch.tensor(np.asarray(thresholds, np.float32), device=device)
        if signs is not None:
            q.signs = torch.tensor(np.asarray(signs, np.int8), device=device)
        if qjl_s_bits is not None:
            q.qjl_s = torch.tensor(np.asarray(qjl_s_bits, np.uint16).view(np.int16), device=device)
        q.rotation = {"rht": TQ_ROT_RHT, "givens": TQ_ROT_GIVENS, "quat": TQ_ROT_QUAT}[rotation]
        if rot is not None:
            q.rot = torch.tensor(np.ascontiguousarray(rot, np.float32).reshape(-1), device=device)
        return q

    def params(self) -> TqParams:
        return TqParams(self.d_in, self.d, self.m, self.rotation, _ptr(self.centroids), _ptr(self.thresholds),
                        _ptr(self.signs), _ptr(self.qjl_s), _ptr(self.rot))

    @property
    def mode_code(self) -> int:
        return TQ_PROD if self.mode == "prod" else TQ_MSE

    @property
    def record_bytes(self) -> int:
        return self.m * self.d // 8

    def alloc_codes(self, n: int, device="cuda") -> dict:
        import torch
        out = {"codes": torch.empty((n, self.record_bytes), dtype=torch.uint8, device=device)
               if self.m > 0 else None,
               "norms": torch.empty(n, dtype=torch.float32, device=device)}
        if self.mode == "prod":
            out["qjl"] = torch.empty((n, self.d // 8), dtype=torch.uint8, device=device)
            out["rnorms"] = torch.empty(n, dtype=torch.float32, device=device)
        else:
            out["qjl"] = out["rnorms"] = None
        return out


def _codes_struct(c: dict) -> TqCodes:
    return TqCodes(_ptr(c.get("codes")), _ptr(c.get("qjl")), _ptr(c.get("norms")), _ptr(c.get("rnorms")))


# --------------------------------------------------------------- entry points

def tq_encode_mse(q: Quantizer, x, out: dict, n: int | None = None, stream=None) -> dict:
    """x: [n, ld_x] float32/float16/bfloat16 on the device (rows contiguous)."""
    return _encode(lib().tq_encode_mse, "tq_encode_mse", q, x, out, n, stream)


def tq_encode_prod(q: Quantizer, x, out: dict, n: int | None = None, stream=None) -> dict:
    return _encode(lib().tq_encode_prod, "tq_encode_prod", q, x, out, n, stream)


def _encode(fn, name, q, x, out, n, stream):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name}: x must be a 2-D tensor with unit column stride")
    n = x.shape[0] if n is None else n
    p, c = q.params(), _codes_struct(out)
    _check(fn(ctypes.byref(p), x.data_ptr(), _dtype_code(x), x.stride(0), n, ctypes.byref(c),
              _stream(stream)), name)
    return out


def tq_decode(q: Quantizer, codes: dict, out, n: int | None = None, stream=None):
    """out: float32 [n, ld_out] with ld_out >= d_in."""
    n = codes["norms"].shape[0] if n is None else n
    p, c = q.params(), _codes_struct(codes)
    _check(lib().tq_decode(ctypes.byref(p), q.mode_code, ctypes.byref(c), n, out.data_ptr(),
                           out.stride(0), _stream(stream)), "tq_decode")
    return out


def tq_score_workspace(q: Quantizer, nq: int) -> int:
    p = q.params()
    return int(lib().tq_score_workspace(ctypes.byref(p), q.mode_code, nq))


def tq_score(q: Quantizer, queries, keys: dict, scores, workspace, n: int | None = None, stream=None):
    """queries float32 [nq, ldq]; scores float32 [nq, ld_scores]; workspace a
    uint8 device tensor of at least tq_score_workspace(q, nq) bytes."""
    n = keys["norms"].shape[0] if n is None else n
    p, c = q.params(), _codes_struct(keys)
    _check(lib().tq_score(ctypes.byref(p), q.mode_code, queries.data_ptr(), queries.stride(0),
                          queries.shape[0], ctypes.byref(c), n, scores.data_ptr(), scores.stride(0),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream(stream)), "tq_score")
    return scores


def tq_score_accumulate(q: Quantizer, queries, groups: int, keys: dict, scores, workspace, stream=None):
    """As tq_score_grouped, adding the estimates to `scores`."""
    return tq_score_grouped(q, queries, groups, keys, scores, workspace, stream, _fn="tq_score_accumulate")


def tq_score_grouped(q: Quantizer, queries, groups: int, keys: dict, scores, workspace, stream=None,
                     _fn="tq_score_grouped"):
    """queries float32 [groups * nq, ldq]; keys: groups * n records;
    scores float32 [groups * nq, ld_scores >= n]."""
    nq_all = queries.shape[0]
    n_all = keys["norms"].shape[0]
    if nq_all % groups or n_all % groups:
        raise ValueError("queries and keys must split into `groups` equal blocks")
    p, c = q.params(), _codes_struct(keys)
    _check(getattr(lib(), _fn)(ctypes.byref(p), q.mode_code, queries.data_ptr(), queries.stride(0),
                               groups, nq_all // groups, ctypes.byref(c), n_all // groups,
                               scores.data_ptr(), scores.stride(0), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(stream)), _fn)
    return scores


def tq_topk_workspace(q: Quantizer, nq: int, n: int, k: int) -> int:
    p = q.params()
    return int(lib().tq_topk_workspace(ctypes.byref(p), q.mode_code, nq, n, k))


def tq_topk(q: Quantizer, queries, keys: dict, k: int, idx, vals, workspace, n: int | None = None, stream=None):
    """queries float32 [nq, ldq]; idx int64 [nq, k]; vals float32 [nq, k]
    (contiguous); workspace >= tq_topk_workspace(q, nq, n, k) bytes."""
    n = keys["norms"].shape[0] if n is None else n
    p, c = q.params(), _codes_struct(keys)
    _check(lib().tq_topk(ctypes.byref(p), q.mode_code, queries.data_ptr(), queries.stride(0), queries.shape[0],
                         ctypes.byref(c), n, k, idx.data_ptr(), vals.data_ptr(), workspace.data_ptr(),
                         workspace.numel() * workspace.element_size(), _stream(stream)), "tq_topk")
    return idx, vals


def tq_attend_workspace(qk: Quantizer, groups: int, nq_per_group: int, n_per_group: int) -> int:
    p = qk.params()
    return int(lib().tq_attend_workspace(ctypes.byref(p), qk.mode_code, groups, nq_per_group, n_per_group))


def tq_attend(qk: Quantizer, keys: dict, qv: Quantizer, values: dict, queries, groups: int, out,
              workspace, scale: float | None = None, stream=None):
    """Decode attention: queries float32 [groups * nq, ldq]; keys / values:
    groups * n records each (values TurboQuant_mse); out float32
    [groups * nq, ld_out]; workspace >= tq_attend_workspace(qk, groups, nq, n)
    bytes.  scale defaults to 1/sqrt(128)."""
    nq_all = queries.shape[0]
    n_all = keys["norms"].shape[0]
    if nq_all % groups or n_all % groups or values["norms"].shape[0] != n_all:
        raise ValueError("queries, keys and values must split into `groups` equal blocks")
    if qv.mode != "mse":
        raise ValueError("values must be TurboQuant_mse codes")
    pk, pv = qk.params(), qv.params()
    ck, cv = _codes_struct(keys), _codes_struct(values)
    sc = 1.0 / math.sqrt(128.0) if scale is None else float(scale)
    _check(lib().tq_attend(ctypes.byref(pk), qk.mode_code, ctypes.byref(ck), ctypes.byref(pv),
                           ctypes.byref(cv), queries.data_ptr(), queries.stride(0), groups, nq_all // groups,
                           n_all // groups, sc, out.data_ptr(), out.stride(0), workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), _stream(stream)), "tq_attend")
    return out


# Size of the fixed device array tq_attend_noalloc uses for its partials.
ATTEND_NOALLOC_MAX_WORKSPACE = 16 << 20


def tq_attend_noalloc(qk: Quantizer, keys: dict, qv: Quantizer, values: dict, queries, groups: int, out,
                      scale: float | None = None, stream=None):
    """tq_attend with the library's fixed scratch instead of a workspace
    (allocates nothing): tq_attend_workspace(...) must be at most
    ATTEND_NOALLOC_MAX_WORKSPACE bytes; calls that overlap on one GPU race."""
    nq_all = queries.shape[0]
    n_all = keys["norms"].shape[0]
    if nq_all % groups or n_all % groups or values["norms"].shape[0] != n_all:
        raise ValueError("queries, keys and values must split into `groups` equal blocks")
    if qv.mode != "mse":
        raise ValueError("values must be TurboQuant_mse codes")
    pk, pv = qk.params(), qv.params()
    ck, cv = _codes_struct(keys), _codes_struct(values)
    sc = 1.0 / math.sqrt(128.0) if scale is None else float(scale)
    _check(lib().tq_attend_noalloc(ctypes.byref(pk), qk.mode_code, ctypes.byref(ck), ctypes.byref(pv),
                                   ctypes.byref(cv), queries.data_ptr(), queries.stride(0), groups,
                                   nq_all // groups, n_all // groups, sc, out.data_ptr(), out.stride(0),
                                   _stream(stream)), "tq_attend_noalloc")
    return out


def tq_rht(q: Quantizer, inp, out, inverse: bool = False, stream=None):
    p = q.params()
    _check(lib().tq_rht(ctypes.byref(p), inp.data_ptr(), inp.stride(0), out.data_ptr(),
                        out.stride(0), inp.shape[0], 1 if inverse else 0, _stream(stream)), "tq_rht")
    return out


# --------------------------------------------------------------- conveniences

# Outputs and temporaries are allocated on `stream` (the current stream when
# None); outputs are ready once that stream has been synchronised.

def encode(q: Quantizer, x, stream=None) -> dict:
    with _on_stream(stream):
        out = q.alloc_codes(x.shape[0], device=x.device)
        fn = tq_encode_prod if q.mode == "prod" else tq_encode_mse
        return fn(q, x, out, stream=stream)


def decode(q: Quantizer, codes: dict, stream=None):
    import torch
    with _on_stream(stream):
        n = codes["norms"].shape[0]
        out = torch.empty((n, q.d_in), dtype=torch.float32, device=codes["norms"].device)
        return tq_decode(q, codes, out, stream=stream)


def score(q: Quantizer, queries, keys: dict, stream=None):
    import torch
    with _on_stream(stream):
        dev = keys["norms"].device
        nq, n = queries.shape[0], keys["norms"].shape[0]
        scores = torch.empty((nq, n), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, tq_score_workspace(q, nq)), dtype=torch.uint8, device=dev)
        return tq_score(q, queries, keys, scores, ws, stream=stream)


# --------------------------------------------------------------- channel split

@dataclass
class SplitQuantizer:
    """Outlier-channel split: contiguous channel ranges, each quantised by
    its own Quantizer (its own bits, rotation, codebook and norm).  Every
    step is one library call per range (see tq_score_accumulate in tq.h)."""
    parts: list                    # [(first column, Quantizer)], ranges in order

    @property
    def d_in(self) -> int:
        c0, q = self.parts[-1]
        return c0 + q.d_in

    def encode(self, x, stream=None) -> list:
        return [encode(q, x[:, c0:c0 + q.d_in], stream=stream) for c0, q in self.parts]

    def decode(self, recs: list, stream=None):
        import torch
        with _on_stream(stream):
            n = recs[0]["norms"].shape[0]
            out = torch.empty((n, self.d_in), dtype=torch.float32, device=recs[0]["norms"].device)
            for (c0, q), r in zip(self.parts, recs):
                tq_decode(q, r, out[:, c0:], stream=stream)
            return out

    def score(self, queries, recs: list, groups: int = 1, stream=None):
        import torch
        with _on_stream(stream):
            n_all = recs[0]["norms"].shape[0]
            scores = torch.empty((queries.shape[0], n_all // groups), dtype=torch.float32, device=queries.device)
            for i, ((c0, q), r) in enumerate(zip(self.parts, recs)):
                ws = torch.empty(tq_score_workspace(q, queries.shape[0]), dtype=torch.uint8, device=queries.device)
                fn = tq_score_grouped if i == 0 else tq_score_accumulate
                fn(q, queries[:, c0:], groups, r, scores, ws, stream=stream)
            return scores
