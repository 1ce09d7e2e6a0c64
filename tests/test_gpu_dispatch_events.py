"""kvc_set_dispatch_events: the timing hook attaches caller events to the
first and last kernels of the next decode call.  Results must not change,
the dispatch-event time must be positive and no longer than stream markers
around the same call, and the hook must be used by exactly one call."""
import numpy as np
import pytest
import torch

from harness import Built, bits
from workloads import DecodeWorkload

pytestmark = pytest.mark.gpu


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()                                     # creates the underlying event
    torch.cuda.synchronize()
    return evs


@pytest.mark.parametrize("dtype,splits", [("bf16", 0), ("fp8", 0), ("int4", 0), ("bf16", 3),
                                          ("f32", 1), ("f32", 4)])
def test_dispatch_events_time_the_decode_kernels(dtype, splits):
    print(f"dispatch events: {dtype} splits={splits}", flush=True)
    w = DecodeWorkload("dispatch" + dtype, 5, 8, 2, 128 if dtype != "f32" else 64, dtype,
                       (200, 3000))
    b = Built(w)
    q = torch.from_numpy(w.q()).to(b.io).cuda()
    ref = b.c.attn_decode(0, b.seqs, q, num_splits=splits)
    torch.cuda.synchronize()
    d0, d1, s0, s1 = _events(4)
    s0.record()
    b.c.set_dispatch_events(d0, d1)
    out = b.c.attn_decode(0, b.seqs, q, num_splits=splits)
    s1.record()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref)), "same results with the hook set"
    t_disp, t_mark = d0.elapsed_time(d1), s0.elapsed_time(s1)
    assert 0.0 < t_disp <= t_mark * 1.01 + 1e-3, (t_disp, t_mark)
    # used by one call only: a second call leaves both events where they were
    again = b.c.attn_decode(0, b.seqs, q, num_splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits(again), bits(ref))
    assert d0.elapsed_time(d1) == t_disp


def test_dispatch_events_on_append_and_noalloc():
    w = DecodeWorkload("dispatchapp", 4, 8, 2, 128, "bf16", (100, 900))
    b = Built(w)
    q = torch.from_numpy(w.q()).to(b.io).cuda()
    rng = np.random.default_rng(7)
    k = torch.from_numpy(rng.standard_normal((4, 2, 128), dtype=np.float32)).to(b.io).cuda()
    v = torch.from_numpy(rng.standard_normal((4, 2, 128), dtype=np.float32)).to(b.io).cuda()
    b.c.seq_grow(list(range(4)))
    d0, d1 = _events(2)
    b.c.set_dispatch_events(d0, d1)
    out = b.c.attn_decode_append(0, b.seqs, k, v, q)
    torch.cuda.synchronize()
    assert d0.elapsed_time(d1) > 0.0
    ref = b.c.attn_decode(0, b.seqs, q)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref))
    b.c.set_dispatch_events(d0, d1)
    out2 = b.c.attn_decode_noalloc(0, b.seqs, q)
    torch.cuda.synchronize()
    assert d0.elapsed_time(d1) > 0.0
    assert np.array_equal(bits(out2), bits(ref))


def test_dispatch_events_cleared_by_a_failing_call():
    w = DecodeWorkload("dispatchfail", 2, 8, 2, 128, "bf16", 300)
    b = Built(w)
    q = torch.from_numpy(w.q()).to(b.io).cuda()
    d0, d1 = _events(2)
    t0 = d0.elapsed_time(d1)
    b.c.set_dispatch_events(d0, d1)
    with pytest.raises(Exception):
        b.c.attn_decode(0, b.seqs, q, scale=-1.0)      # refused before any launch
    b.c.attn_decode(0, b.seqs, q)                      # not timed: the hook went with the refusal
    torch.cuda.synchronize()
    assert d0.elapsed_time(d1) == t0
