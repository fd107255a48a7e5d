"""CPU checks of the Python binding's workspace handling (no GPU: torch's stream and
allocation calls are replaced by stand-ins that record what the binding asks for)."""
import pytest
import torch

import block_drafting_verification_amd as dsp


class FakeStream:
    def __init__(self, h):
        self.cuda_stream = h


class FakeBuf:
    def __init__(self, n):
        self.n = n
        self.recorded = []

    def numel(self):
        return self.n

    def record_stream(self, s):
        self.recorded.append(s.cuda_stream)


@pytest.fixture
def fake(monkeypatch):
    state = {"cur": FakeStream(11)}
    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: state["cur"])
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    monkeypatch.setattr(torch, "empty", lambda n, dtype=None, device=None: FakeBuf(n))
    dsp._ws_cache.clear()
    yield state
    dsp._ws_cache.clear()


def test_one_shot_calls_share_a_buffer_per_device_and_stream(fake):
    dev = torch.device("cuda", 0)
    a = dsp._workspace(1000, dev)
    b = dsp._workspace(500, dev)
    assert a is b and not a.recorded
    c = dsp._workspace(5000, dev)  # grows: a new buffer replaces the entry
    assert c is not a and c.numel() >= 5000
    fake["cur"] = FakeStream(22)    # another current stream: its own entry
    d = dsp._workspace(100, dev)
    assert d is not c
    assert set(dsp._ws_cache) == {(0, 11), (0, 22)}


def test_a_call_on_another_stream_gets_its_own_recorded_buffer(fake):
    dev = torch.device("cuda", 0)
    shared = dsp._workspace(1000, dev)
    other = FakeStream(33)
    p = dsp._workspace(1000, dev, stream=other)
    q = dsp._workspace(1000, dev, stream=other)
    assert p is not shared and q is not p
    assert p.recorded == [33] and q.recorded == [33]
    assert set(dsp._ws_cache) == {(0, 11)}
    # the current stream passed explicitly is the shared case
    assert dsp._workspace(10, dev, stream=FakeStream(11)) is shared


def test_prepared_calls_get_private_buffers(fake):
    dev = torch.device("cuda", 0)
    a = dsp._workspace(1000, dev, private=True)
    b = dsp._workspace(1000, dev, private=True)
    assert a is not b and not dsp._ws_cache
