"""GPU parity of kvc_attn_extend: T new query rows per sequence against the
whole paged context (positions len-T .. len-1), against the float64 oracle's
extend_attention on the same rows.  Chunked prefill through the cache must
reproduce the whole-prompt prefill."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import assert_close, f64
from oracle import attention as A

pytestmark = pytest.mark.gpu


def _rows(rng, shape, io):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(io).cuda()


def _cache_with_contexts(dtype, n_q, n_kv, d, lengths, seed):
    """A cache whose sequence b holds lengths[b] rows behind a shuffled table;
    returns the cache and the io-typed rows of every sequence."""
    rng = np.random.default_rng(seed)
    io = kv.IO_TORCH[dtype]
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 5
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max(nbs) + 1, dtype, poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    o, rows = 0, []
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        k, v = _rows(rng, (1, L, n_kv, d), io), _rows(rng, (1, L, n_kv, d), io)
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        rows.append((k[0], v[0]))
    return c, rows


@pytest.mark.parametrize("dtype,n_q,n_kv,d,T,lengths", [
    ("bf16", 32, 8, 128, 1, [1, 40, 513]),
    ("bf16", 32, 8, 128, 7, [7, 100, 1000]),
    ("bf16", 8, 2, 128, 64, [64, 65, 700]),
    ("bf16", 4, 4, 128, 257, [257, 300, 1201]),
    ("f16", 8, 2, 64, 100, [100, 131, 555]),
    ("bf16", 6, 1, 64, 33, [33, 34, 99, 1030]),
])
def test_extend_vs_oracle(dtype, n_q, n_kv, d, T, lengths):
    c, rows = _cache_with_contexts(dtype, n_q, n_kv, d, lengths, seed=T)
    rng = np.random.default_rng([T, d])
    q = _rows(rng, (len(lengths), T, n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    out = c.attn_extend(0, seqs, q)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    for b, (k, v) in enumerate(rows):
        ref = A.extend_attention(f64(q[b]), f64(k), f64(v), scale)
        assert_close(f64(out[b]), ref, what=f"extend {dtype} T={T} L={lengths[b]}", io=dtype)


def test_chunked_prefill_through_the_cache_equals_whole_prefill():
    """A 700-token prompt in chunks of 100, 256, 1 and 343 rows: grow the
    sequence by the chunk, write the chunk's K/V at its offset, then
    attn_extend its queries; every row matches the oracle's whole-prompt
    prefill, as does attn_prefill."""
    dtype, n_q, n_kv, d, T = "bf16", 32, 8, 128, 700
    rng = np.random.default_rng(7)
    io = kv.IO_TORCH[dtype]
    q, k, v = (_rows(rng, (1, T, h, d), io) for h in (n_q, n_kv, n_kv))
    nb = -(-T // 16)
    c = kv.KvCache(1, n_q, n_kv, d, nb + 4, 1, nb, dtype, poison=True)
    table = rng.permutation(nb + 4)[:nb].astype(np.int32)
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    cuts = [0, 100, 356, 357, 700]
    for a, b in zip(cuts[:-1], cuts[1:]):
        if a == 0:
            c.set_block_table(0, table[:-(-b // 16)], b)    # first chunk: shuffled blocks
        else:
            c.seq_grow_by(0, b - a)                          # later chunks: from the free list
        c.write(0, seqs, a, k[:, a:b].contiguous(), v[:, a:b].contiguous())
        out[:, a:b] = c.attn_extend(0, seqs, q[:, a:b].contiguous())
    whole = c.attn_prefill(0, q, k, v)
    torch.cuda.synchronize()
    ref = A.prefill_attention(f64(q[0]), f64(k[0]), f64(v[0]), 1 / math.sqrt(d))
    assert_close(f64(out[0]), ref, what="chunked prefill")
    assert_close(f64(whole[0]), ref, what="whole prefill")


def test_extend_invalid_entries_give_nan_rows():
    """Out-of-range ids and sequences holding fewer than T rows give NaN
    rows; the valid sequences in the same call are unaffected."""
    dtype, n_q, n_kv, d, T = "bf16", 8, 2, 128, 20
    c, rows = _cache_with_contexts(dtype, n_q, n_kv, d, [50, 10, 90], seed=3)
    rng = np.random.default_rng(4)
    q = _rows(rng, (4, T, n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.tensor([0, 1, 99, 2], dtype=torch.int32, device="cuda")
    out = c.attn_extend(0, seqs, q)
    torch.cuda.synchronize()
    y = f64(out)
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    scale = 1 / math.sqrt(d)
    for i, b in ((0, 0), (3, 2)):
        k, v = rows[b]
        assert_close(y[i], A.extend_attention(f64(q[i]), f64(k), f64(v), scale),
                     what=f"valid entry {i}")


def test_extend_llama8b_chunk_sampled_rows():
    """A 512-row chunk at the end of 4 contexts of up to 8,192 rows (32 q /
    8 kv heads of 128): sampled rows against the oracle, computed one query
    row at a time at its absolute position."""
    dtype, n_q, n_kv, d, T = "bf16", 32, 8, 128, 512
    lengths = [8192, 4000, 513, 6000]
    c, rows = _cache_with_contexts(dtype, n_q, n_kv, d, lengths, seed=11)
    rng = np.random.default_rng(12)
    q = _rows(rng, (len(lengths), T, n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    out = c.attn_extend(0, seqs, q)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    for b, (k, v) in enumerate(rows):
        L = lengths[b]
        sample = np.unique(np.concatenate([[0, 1, 255, 256, T - 1], rng.integers(0, T, 6)]))
        ref = A.gqa_attention(f64(q[b])[sample], f64(k), f64(v), scale, q_pos=L - T + sample)
        assert_close(f64(out[b])[sample], ref, what=f"chunk of 512 at L={L}")


@pytest.mark.parametrize("dtype", ["fp8", "int4"])
@pytest.mark.parametrize("n_q,n_kv,d,T,lengths,window,sinks", [
    (32, 8, 128, 64, [64, 100, 700], 0, 0),
    (8, 2, 64, 33, [33, 290, 1030], 0, 0),
    (32, 8, 128, 100, [100, 400, 900], 128, 4),
])
def test_extend_scaled_cache_vs_dequantised_oracle(dtype, n_q, n_kv, d, T, lengths, window,
                                                   sinks):
    """fp8 / int4 cache: codes are staged exactly and the block scales applied
    to scores and probabilities; the result matches the oracle on the exactly
    dequantised values the cache holds (the oracle's paged model fed the same
    rows) within the bf16 tolerances."""
    from oracle.paged import PagedCacheModel
    rng = np.random.default_rng([T, d, window])
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 5
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max(nbs) + 1, dtype, poison=True)
    m = PagedCacheModel(1, n_kv, d, dtype, n_blocks, len(lengths), max(nbs) + 1, poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    o = 0
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        m.set_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        k = _rows(rng, (1, L, n_kv, d), torch.bfloat16)
        v = _rows(rng, (1, L, n_kv, d), torch.bfloat16)
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        m.write_rows(0, b, 0, k[0].float().cpu().numpy(), v[0].float().cpu().numpy())
    q = _rows(rng, (len(lengths), T, n_q, d), torch.bfloat16)
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    out = c.attn_extend(0, seqs, q, window=window, sinks=sinks)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    for b in range(len(lengths)):
        K, V = m.logical_values(0, b)
        ref = A.extend_attention(f64(q[b]), K, V, scale, window=window, sinks=sinks)
        assert_close(f64(out[b]), ref, what=f"{dtype} extend T={T} L={lengths[b]} w={window}")
