"""Host logic of the Python binding that runs without a GPU.

The workspace a binding call allocates for itself is created on torch's
current stream and dropped when the call returns; when the call runs on
another stream, that stream must be recorded on the allocation, or the caching
allocator could hand the memory to a new allocation while the library's
kernels on that stream still use it.
"""
import types

import pytest
import torch

import mlp_prefill_amd as m


class _Buf:
    def __init__(self, n):
        self.n = n
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)

    def numel(self):
        return self.n


class _ExtStream:
    def __init__(self, ptr):
        self.cuda_stream = ptr


@pytest.fixture
def fake_torch(monkeypatch):
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *a, **k: types.SimpleNamespace(cuda_stream=0x10))
    monkeypatch.setattr(torch, "empty", lambda n, dtype=None, device=None: _Buf(n))
    monkeypatch.setattr(torch.cuda, "ExternalStream", _ExtStream)


def test_callers_workspace_is_used_as_is(fake_torch):
    mine = _Buf(4096)
    assert m._scratch(1000, mine, "cuda", 0x20) is mine
    assert mine.recorded == []


def test_own_workspace_on_the_current_stream_records_nothing(fake_torch):
    for s in (None, 0x10, types.SimpleNamespace(cuda_stream=0x10)):
        ws = m._scratch(1000, None, "cuda", s)
        assert ws.n == 1000 and ws.recorded == []


def test_own_workspace_on_another_stream_records_that_stream(fake_torch):
    ws = m._scratch(100, None, "cuda", 0x20)                       # raw hipStream_t
    assert ws.n == 256                                              # never a zero-size buffer
    assert len(ws.recorded) == 1 and ws.recorded[0].cuda_stream == 0x20
    ws = m._scratch(100, None, "cuda", _ExtStream(0x30))           # an object with .cuda_stream
    assert len(ws.recorded) == 1 and ws.recorded[0].cuda_stream == 0x30


def test_workspace_query_path_records_the_stream(fake_torch):
    def query(wsp, szp):
        szp._obj.value = 5000
        return m.OK
    ws, sz = m._workspace(query, None, "cuda", 0x40)
    assert sz.value == 5000 and ws.recorded[0].cuda_stream == 0x40
