"""CPU test of the binding's stream handling: when a caller passes a stream,
the convenience calls allocate their outputs and workspaces while that
stream is torch's current stream, so torch's caching allocator ties the
blocks to the stream the kernels run on.  No GPU and no library call is
involved (the C entry points are replaced by stubs)."""

import contextlib

import torch

from embedding_vector_quantization_amd import binding as B


class _Recorder:
    def __init__(self):
        self.active = None
        self.allocs = []

    @contextlib.contextmanager
    def stream(self, s):
        prev, self.active = self.active, s
        try:
            yield
        finally:
            self.active = prev

    def empty(self, *args, **kwargs):
        kwargs.pop("device", None)
        self.allocs.append(self.active)
        return torch.zeros(*args, **kwargs)


def _patch(monkeypatch, rec):
    monkeypatch.setattr(torch.cuda, "stream", rec.stream)
    monkeypatch.setattr(torch, "empty", rec.empty)
    monkeypatch.setattr(B, "tq_score_workspace", lambda q, nq: 64)
    for name in ("tq_score", "tq_score_grouped", "tq_score_accumulate", "tq_decode", "tq_encode_mse",
                 "tq_encode_prod"):
        monkeypatch.setattr(B, name, lambda *a, **k: None)


def test_convenience_calls_allocate_on_the_callers_stream(monkeypatch):
    rec = _Recorder()
    _patch(monkeypatch, rec)
    side = object()                       # stands for a torch.cuda.Stream
    q = B.Quantizer(d_in=8, d=32, m=2, mode="mse")
    keys = {"norms": torch.zeros(5), "codes": torch.zeros((5, 8), dtype=torch.uint8)}
    B.score(q, torch.zeros((3, 8)), keys, stream=side)
    B.decode(q, keys, stream=side)
    B.encode(q, torch.zeros((5, 8)), stream=side)
    sq = B.SplitQuantizer(parts=[(0, q), (8, B.Quantizer(d_in=8, d=32, m=3, mode="mse"))])
    sq.score(torch.zeros((3, 16)), [keys, keys], stream=side)
    sq.decode([keys, keys], stream=side)
    assert rec.allocs and all(a is side for a in rec.allocs), rec.allocs


def test_without_a_stream_nothing_is_redirected(monkeypatch):
    rec = _Recorder()
    _patch(monkeypatch, rec)
    q = B.Quantizer(d_in=8, d=32, m=2, mode="mse")
    keys = {"norms": torch.zeros(5), "codes": torch.zeros((5, 8), dtype=torch.uint8)}
    B.score(q, torch.zeros((3, 8)), keys)
    assert rec.allocs and all(a is None for a in rec.allocs)
