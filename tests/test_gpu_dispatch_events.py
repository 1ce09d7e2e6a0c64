"""kvc_set_dispatch_events: the timing hook attaches caller events to the
first and last kernels of the next attention call, or both to its main
kernel.  Results must not change, the dispatch-event times must be positive,
the main kernel no longer than the call and the call no longer than stream
markers around it, and the hook must be used by exactly one call."""
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
    d0, d1, s0, s1, k0, k1 = _events(6)
    s0.record()
    b.c.set_dispatch_events(d0, d1)
    out = b.c.attn_decode(0, b.seqs, q, num_splits=splits)
    s1.record()
    b.c.set_dispatch_events(k0, k1, main_kernel=True)
    out_k = b.c.attn_decode(0, b.seqs, q, num_splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ref)), "same results with the hook set"
    assert np.array_equal(bits(out_k), bits(ref))
    t_disp, t_mark, t_main = d0.elapsed_time(d1), s0.elapsed_time(s1), k0.elapsed_time(k1)
    assert 0.0 < t_disp <= t_mark * 1.01 + 1e-3, (t_disp, t_mark)
    assert 0.0 < t_main <= t_disp * 1.05 + 2e-3, (t_main, t_disp)
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


def test_dispatch_events_on_prefill_and_extend():
    import kv_cache_flashattention_amd as kv
    rng = np.random.default_rng(11)
    B, T, nq, nkv, d = 2, 300, 8, 2, 128
    q, k, v = (torch.from_numpy(rng.standard_normal((B, T, h, d), dtype=np.float32))
               .to(torch.bfloat16).cuda() for h in (nq, nkv, nkv))
    nb = -(-T // 16)
    c = kv.KvCache(1, nq, nkv, d, B * nb + 2, B, nb, "bf16")
    for s_ in range(B):
        c.seq_alloc(s_, T)
    seqs = torch.arange(B, dtype=torch.int32, device="cuda")
    ref = c.attn_prefill(0, q, k, v, seqs=seqs)
    torch.cuda.synchronize()
    for main in (False, True):
        d0, d1 = _events(2)
        c.set_dispatch_events(d0, d1, main_kernel=main)
        out = c.attn_prefill(0, q, k, v, seqs=seqs)
        torch.cuda.synchronize()
        assert d0.elapsed_time(d1) > 0.0
        assert np.array_equal(bits(out), bits(ref))
    qe = q[:, -64:].contiguous()
    ref_e = c.attn_extend(0, seqs, qe)
    torch.cuda.synchronize()
    d0, d1 = _events(2)
    c.set_dispatch_events(d0, d1, main_kernel=True)
    out_e = c.attn_extend(0, seqs, qe)
    torch.cuda.synchronize()
    assert d0.elapsed_time(d1) > 0.0
    assert np.array_equal(bits(out_e), bits(ref_e))


def test_dispatch_events_unknown_scope_refused():
    import kv_cache_flashattention_amd as kv
    w = DecodeWorkload("dispatchscope", 2, 8, 2, 128, "bf16", 100)
    b = Built(w)
    d0, d1 = _events(2)
    rc = kv.lib().kvc_set_dispatch_events(b.c._h, d0.cuda_event, d1.cuda_event, 7)
    assert rc != 0
    t0 = d0.elapsed_time(d1)
    q = torch.from_numpy(w.q()).to(b.io).cuda()
    b.c.attn_decode(0, b.seqs, q)                      # the refused hook left nothing behind
    torch.cuda.synchronize()
    assert d0.elapsed_time(d1) == t0
