"""The Python wrappers on a side stream (CPU only, torch.cuda mocked): the
library enqueues on the stream it is given, while the wrappers allocate
scratch, outputs and workspaces from torch's caching allocator on the current
stream; those tensors must then be marked as used by the side stream
(record_stream), or their memory could be handed out again while the kernels
still run."""

import torch

import lsh_sampled_sparse_amd as mp


class FakeStream:
    def __init__(self, h):
        self.cuda_stream = h


class FakeTensor:
    def __init__(self):
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)


def _mock_streams(monkeypatch, cur):
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: cur)
    monkeypatch.setattr(torch.cuda, "ExternalStream", lambda h, device=None: FakeStream(h))


def test_side_stream_detection(monkeypatch):
    cur = FakeStream(0)
    _mock_streams(monkeypatch, cur)
    assert mp._side_stream(None, "cuda:0") is None
    assert mp._side_stream(cur, "cuda:0") is None
    assert mp._side_stream(0, "cuda:0") is None            # the raw handle of the current stream
    side = FakeStream(1234)
    assert mp._side_stream(side, "cuda:0") is side
    assert mp._side_stream(5678, "cuda:0").cuda_stream == 5678
    t1, t2 = FakeTensor(), FakeTensor()
    mp._keep_alive_on(side, t1, None, t2)
    assert t1.recorded == [side] and t2.recorded == [side]
    mp._keep_alive_on(None, t1)
    assert t1.recorded == [side]


def test_decode_marks_its_buffers_on_a_side_stream(monkeypatch):
    cur = FakeStream(0)
    _mock_streams(monkeypatch, cur)
    kept = []
    monkeypatch.setattr(mp, "_keep_alive_on",
                        lambda side, *ts: kept.append((side, [t for t in ts if t is not None])))
    monkeypatch.setattr(mp, "kv_view", lambda t: None)
    calls = []
    monkeypatch.setattr(mp.capi, "mp_decode_attn", lambda *a: calls.append(a))

    class Index:
        workspace = torch.empty(8, dtype=torch.uint8)
        tables = None
        handle = 1

        def scratch_bytes(self, H_q, tables=False):
            return 64

    q = torch.zeros(1, 4, 128)
    side = FakeStream(99)
    out = mp.decode_attn(q, Index(), None, None, 4, 64, stream=side)
    assert calls and calls[0][-1] == 99                 # enqueued on the side stream
    s, ts = kept[0]
    assert s is side
    assert any(t is out for t in ts)                    # the output made here
    assert any(t.numel() == 64 for t in ts)             # the scratch made here
    assert any(t is Index.workspace for t in ts)        # the index it reads
    kept.clear()
    mp.decode_attn(q, Index(), None, None, 4, 64)        # current stream: nothing to mark
    assert kept[0][0] is None
