"""Degenerate and empty inputs on the GPU.

* Empty calls (no sequences, no prompt rows) return without error and leave
  the cache untouched.
* Equal keys, or a zero query, make every visible key equally likely: each
  output row is the mean of the visible V rows (decode: all L rows; prefill
  row t: rows 0..t; extend row t: rows 0..L-T+t).  Checked against that
  closed form and the float64 oracle, for bf16 and fp8 caches."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import assert_close, bits, f64
from oracle import attention as A
from oracle.paged import PagedCacheModel

pytestmark = pytest.mark.gpu


def test_empty_calls_do_nothing():
    n_q, n_kv, d = 8, 2, 128
    c = kv.KvCache(1, n_q, n_kv, d, 8, 2, 4, "bf16", poison=True)
    c.seq_alloc(0, 20)
    before_k, before_v = bits(c.k_pool).copy(), bits(c.v_pool).copy()
    e_seqs = torch.zeros(0, dtype=torch.int32, device="cuda")
    e_q = torch.zeros(0, n_q, d, dtype=torch.bfloat16, device="cuda")
    e_kv = torch.zeros(0, n_kv, d, dtype=torch.bfloat16, device="cuda")
    assert c.attn_decode(0, e_seqs, e_q).shape == (0, n_q, d)
    c.append(0, e_seqs, e_kv, e_kv)
    qp = torch.zeros(1, 0, n_q, d, dtype=torch.bfloat16, device="cuda")
    kp = torch.zeros(1, 0, n_kv, d, dtype=torch.bfloat16, device="cuda")
    assert c.attn_prefill(0, qp, kp, kp).shape == (1, 0, n_q, d)
    assert c.attn_extend(0, e_seqs, torch.zeros(0, 4, n_q, d, dtype=torch.bfloat16,
                                                device="cuda")).shape == (0, 4, n_q, d)
    torch.cuda.synchronize()
    assert np.array_equal(bits(c.k_pool), before_k) and np.array_equal(bits(c.v_pool), before_v)


def _mean_rows(v, upto):
    """mean of rows 0..upto[t] of v [L, n_kv, d] for each t -> [len(upto), n_kv, d]"""
    cs = np.cumsum(v, axis=0)
    return np.stack([cs[u] / (u + 1) for u in upto])


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("kind", ["equal_keys", "zero_query"])
def test_decode_uniform_weights_give_mean_of_v(dtype, kind):
    n_q, n_kv, d = 16, 4, 128
    lengths = [1, 19, 260]
    G = n_q // n_kv
    rng = np.random.default_rng(31)
    io = kv.IO_TORCH[dtype]
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 2
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max(nbs), dtype, poison=True)
    m = PagedCacheModel(1, n_kv, d, dtype, n_blocks, len(lengths), max(nbs), poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    o = 0
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        m.set_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        if kind == "equal_keys":
            k1 = rng.standard_normal((1, 1, n_kv, d)).astype(np.float32)
            kf = np.repeat(k1, L, axis=1)
        else:
            kf = rng.standard_normal((1, L, n_kv, d)).astype(np.float32)
        k = torch.from_numpy(kf).to(io).cuda()
        v = torch.from_numpy(rng.standard_normal((1, L, n_kv, d)).astype(np.float32)).to(io).cuda()
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        if dtype == "fp8":
            m.write_rows(0, b, 0, k[0].float().cpu().numpy(), v[0].float().cpu().numpy())
        else:
            m.write_rows(0, b, 0, bits(k[0]), bits(v[0]))
    if kind == "zero_query":
        q = torch.zeros(len(lengths), n_q, d, dtype=io, device="cuda")
    else:
        q = torch.from_numpy(rng.standard_normal((len(lengths), n_q, d)).astype(np.float32)).to(io).cuda()
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    y = f64(c.attn_decode(0, seqs, q, num_splits=2))
    for b, L in enumerate(lengths):
        K, V = m.logical_values(0, b)
        mean = V.mean(axis=0)                          # [n_kv, d]
        closed = np.repeat(mean, G, axis=0)            # query head h uses kv head h // G
        ref = A.decode_attention(f64(q[b]), K, V, 1 / math.sqrt(d))
        assert np.allclose(ref, closed, atol=1e-12), "oracle must reduce to the mean of V"
        assert_close(y[b], closed, what=f"{dtype} {kind} decode seq {b} vs mean of V")


def test_prefill_and_extend_equal_keys_give_running_mean():
    n_q, n_kv, d, T = 8, 2, 64, 200
    G = n_q // n_kv
    rng = np.random.default_rng(32)
    k1 = rng.standard_normal((1, n_kv, d)).astype(np.float32)
    kf = np.repeat(k1[None], T, axis=1)                # [1, T, n_kv, d], every key equal
    k = torch.from_numpy(kf).to(torch.bfloat16).cuda()
    v = torch.from_numpy(rng.standard_normal((1, T, n_kv, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    q = torch.from_numpy(rng.standard_normal((1, T, n_q, d)).astype(np.float32)).to(torch.bfloat16).cuda()
    nb = -(-T // 16)
    c = kv.KvCache(1, n_q, n_kv, d, nb + 1, 1, nb, "bf16", poison=True)
    c.seq_alloc(0, T)
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = f64(c.attn_prefill(0, q, k, v, seqs=seqs))[0]
    vd = f64(v[0])
    closed = np.repeat(_mean_rows(vd, range(T)), G, axis=1)    # [T, n_q, d]
    ref = A.prefill_attention(f64(q[0]), f64(k[0]), vd, 1 / math.sqrt(d))
    assert np.allclose(ref, closed, atol=1e-12)
    assert_close(out, closed, what="equal-key prefill vs running mean of V")
    # the last 64 rows again as an extend chunk against the cache the prefill filled
    Tc = 64
    ext = f64(c.attn_extend(0, seqs, q[:, T - Tc:].contiguous()))[0]
    assert_close(ext, closed[T - Tc:], what="equal-key extend vs running mean of V")
