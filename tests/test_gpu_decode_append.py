"""kvc_attn_decode_append (kv_append + attn_decode in one call) against the
two calls it replaces: identical outputs bit for bit and identical cache
bytes, for every storage type, with windows, several split counts, GQA
groups wider than 16 query heads, and invalid device entries."""
import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import Built, assert_close, bits, f64
from workloads import DecodeWorkload

pytestmark = pytest.mark.gpu


def _pair(dtype, n_q, n_kv, d, lengths, batch=6, tag="dapp"):
    w = DecodeWorkload(tag + dtype + str(n_q) + str(d), batch, n_q, n_kv, d, dtype, lengths,
                       outliers=(dtype in ("fp8", "int4")))
    return w, Built(w), Built(w)


def _new_rows(w, io, seed=7):
    rng = np.random.default_rng(seed)
    k = torch.from_numpy(rng.standard_normal((w.batch, w.n_kv, w.d), dtype=np.float32)).to(io)
    v = torch.from_numpy(rng.standard_normal((w.batch, w.n_kv, w.d), dtype=np.float32)).to(io)
    q = torch.from_numpy(rng.standard_normal((w.batch, w.n_q, w.d), dtype=np.float32)).to(io)
    return k.cuda(), v.cuda(), q.cuda()


def _same_pools(a, b):
    ok = torch.equal(a.c.k_pool.view(torch.uint8), b.c.k_pool.view(torch.uint8)) and \
        torch.equal(a.c.v_pool.view(torch.uint8), b.c.v_pool.view(torch.uint8))
    if a.c.k_scale is not None:
        ok = ok and torch.equal(a.c.k_scale.view(torch.int32), b.c.k_scale.view(torch.int32)) \
            and torch.equal(a.c.v_scale.view(torch.int32), b.c.v_scale.view(torch.int32))
    return ok


@pytest.mark.parametrize("dtype,n_q,n_kv,d", [("bf16", 32, 8, 128), ("fp16", 12, 4, 64),
                                              ("bf16", 32, 1, 128), ("fp8", 64, 8, 128),
                                              ("int4", 16, 4, 64), ("f32", 8, 2, 128)])
def test_decode_append_equals_append_then_decode(dtype, n_q, n_kv, d):
    w, A, B = _pair(dtype, n_q, n_kv, d, (1, 300))
    io = A.io
    for step in range(3):                              # crosses block boundaries for some
        k, v, q = _new_rows(w, io, seed=step)
        A.c.seq_grow(list(range(w.batch)))
        B.c.seq_grow(list(range(w.batch)))
        A.c.append(0, A.seqs, k, v)
        ya = A.c.attn_decode(0, A.seqs, q, num_splits=step)
        yb = B.c.attn_decode_append(0, B.seqs, k, v, q, num_splits=step)
        torch.cuda.synchronize()
        assert torch.equal(bits_t(ya), bits_t(yb)), f"{dtype} step {step}: outputs differ"
        assert _same_pools(A, B), f"{dtype} step {step}: cache bytes differ"


def bits_t(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_decode_append_with_window_and_vs_oracle():
    w, A, B = _pair("bf16", 32, 8, 128, (200, 700), tag="dappw")
    k, v, q = _new_rows(w, A.io)
    for X in (A, B):
        X.c.seq_grow(list(range(w.batch)))
        X.m.grow(list(range(w.batch)))
    A.c.append(0, A.seqs, k, v)
    ya = A.c.attn_decode(0, A.seqs, q, window=100, sinks=4)
    yb = B.c.attn_decode_append(0, B.seqs, k, v, q, window=100, sinks=4)
    torch.cuda.synchronize()
    assert torch.equal(bits_t(ya), bits_t(yb)) and _same_pools(A, B)
    # against the oracle on the model holding the same rows
    from oracle import attention as Aor
    import math
    for b in range(w.batch):
        B.m.write_rows(0, b, int(B.m.length[b]) - 1, bits(k[b:b + 1]), bits(v[b:b + 1]))
        K, V = B.m.logical_values(0, b)
        r = Aor.decode_attention(f64(q[b]), K, V, 1 / math.sqrt(w.d), window=100, sinks=4)
        assert_close(f64(yb[b]), r, what=f"seq {b}")


def test_decode_append_invalid_entries_match_two_calls():
    w, A, B = _pair("bf16", 32, 8, 128, (5, 90), batch=4, tag="dappi")
    k, v, q = _new_rows(w, A.io)
    seqs = torch.tensor([0, 99, 2, -1], dtype=torch.int32, device="cuda")
    for X in (A, B):
        X.c.seq_grow(list(range(w.batch)))
    A.c.append(0, seqs, k, v)
    ya = A.c.attn_decode(0, seqs, q)
    yb = B.c.attn_decode_append(0, seqs, k, v, q)
    torch.cuda.synchronize()
    assert _same_pools(A, B)
    assert torch.equal(torch.isnan(ya.float()), torch.isnan(yb.float()))
    assert torch.all(torch.isnan(yb[1].float())) and torch.all(torch.isnan(yb[3].float()))
    ok = torch.tensor([0, 2], device="cuda")
    assert torch.equal(bits_t(ya[ok]), bits_t(yb[ok]))


def test_decode_append_rejects_bad_arguments():
    w, A, _ = _pair("bf16", 8, 2, 64, (3, 20), batch=2, tag="dappe")
    k, v, q = _new_rows(w, A.io)
    rc = kv.lib().kvc_attn_decode_append(A.c._h, 0, 2, A.seqs.data_ptr(), None, None,
                                         q.data_ptr(), q.data_ptr(), 0.125, 0, 0, 0, None, 0, None)
    assert rc == kv.KVC_E_INVAL
    with pytest.raises(kv.KvcError) as e:                       # misaligned k_new
        kb = torch.empty(k.numel() * 2 + 8, dtype=torch.uint8, device="cuda")[8:].view(-1)
        kv._check(kv.lib().kvc_attn_decode_append(A.c._h, 0, 2, A.seqs.data_ptr(), kb.data_ptr(),
                                                  v.data_ptr(), q.data_ptr(), q.data_ptr(), 0.125,
                                                  0, 0, 0, None, 0, None))
    assert e.value.code == kv.KVC_E_INVAL
