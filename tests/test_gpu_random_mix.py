"""Seeded random configurations against the float64 oracle.

Each case draws its whole configuration from its seed, so a failure names a
reproducible shape:
  * decode: every storage type, d 64 and 128, 1 to 8 kv heads with query
    groups of 1 to 24 heads (groups above 16 take two 16-column passes),
    ragged lengths drawn on and around the 16-row block and 32-row unit
    edges, the work list or a fixed split count, windows with sinks;
  * causal prefill (16-bit types): ragged prompt lengths, windows, and the
    prompt rows written to the cache checked bit for bit;
  * extend: every cache type, T new rows after contexts of T or more rows.
Oracle: the materialised float64 definitions of decode, prefill and extend
attention ("KV Cache & Flash Attention.", Flash Attention and
PagedAttention sections), on the values the cache holds (fp8 and int4:
exactly dequantised by the oracle's own codec model fed the same rows)."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import assert_close, bits, f64
from oracle import attention as A
from oracle.paged import PagedCacheModel

pytestmark = pytest.mark.gpu

EDGE_LENGTHS = (1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513)
DTYPES = ("bf16", "f16", "fp8", "int4")


def _rows(rng, shape, io):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(io).cuda()


def _lengths(rng, n, lo=1, hi=1500):
    """n lengths, each an edge length or uniform in [lo, hi], at least lo."""
    out = []
    for _ in range(n):
        if rng.random() < 0.5:
            out.append(int(rng.choice([L for L in EDGE_LENGTHS if L >= lo] or [lo])))
        else:
            out.append(int(rng.integers(lo, hi, endpoint=True)))
    return out


def _cache(rng, dtype, n_q, n_kv, d, lengths):
    """A cache holding lengths[b] random rows for sequence b behind a shuffled
    table, and the oracle's paged model fed the same rows."""
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 3
    max_bps = max(nbs) + 1
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max_bps, dtype, poison=True)
    m = PagedCacheModel(1, n_kv, d, dtype, n_blocks, len(lengths), max_bps, poison=True)
    io = kv.IO_TORCH[dtype]
    perm = rng.permutation(n_blocks).astype(np.int32)
    o = 0
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        m.set_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        k, v = _rows(rng, (1, L, n_kv, d), io), _rows(rng, (1, L, n_kv, d), io)
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        if dtype in ("fp8", "int4"):
            m.write_rows(0, b, 0, k[0].float().cpu().numpy(), v[0].float().cpu().numpy())
        else:
            m.write_rows(0, b, 0, bits(k[0]), bits(v[0]))
    return c, m


def _draw_decode(seed):
    rng = np.random.default_rng([101, seed])
    dtype = DTYPES[seed % 4]
    d = (64, 128)[(seed // 4) % 2]
    n_kv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 24]))
    lengths = _lengths(rng, int(rng.integers(1, 9, endpoint=True)))
    window = sinks = splits = 0
    if rng.random() < 0.4:
        window = int(rng.integers(1, 600, endpoint=True))
        sinks = int(rng.choice([0, 1, 4, 37]))
    else:
        splits = int(rng.choice([0, 0, 2, 5]))
    return rng, dtype, d, n_kv * G, n_kv, lengths, window, sinks, splits


@pytest.mark.parametrize("seed", range(128))
def test_random_decode(seed):
    rng, dtype, d, n_q, n_kv, lengths, window, sinks, splits = _draw_decode(seed)
    what = (f"seed {seed}: {dtype} d={d} n_q={n_q} n_kv={n_kv} lengths={lengths} "
            f"window={window} sinks={sinks} splits={splits}")
    print(what, flush=True)
    c, m = _cache(rng, dtype, n_q, n_kv, d, lengths)
    q = _rows(rng, (len(lengths), n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    out = c.attn_decode(0, seqs, q, num_splits=splits, window=window, sinks=sinks)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    io = "f16" if dtype == "f16" else "bf16"
    for b in range(len(lengths)):
        K, V = m.logical_values(0, b)
        ref = A.decode_attention(f64(q[b]), K, V, scale, window, sinks)
        assert_close(f64(out[b]), ref, io=io, what=f"{what}, sequence {b}")


@pytest.mark.parametrize("seed", range(32))
def test_random_prefill_writes_and_attends(seed):
    rng = np.random.default_rng([202, seed])
    dtype = ("bf16", "f16")[seed % 2]
    d = (64, 128)[(seed // 2) % 2]
    n_kv = int(rng.choice([1, 2, 4, 8]))
    n_q = n_kv * int(rng.choice([1, 2, 4, 5, 8]))
    batch = int(rng.integers(1, 3, endpoint=True))
    T = int(rng.choice([1, 2, 63, 64, 65, 255, 256, 257])) if rng.random() < 0.5 \
        else int(rng.integers(1, 700, endpoint=True))
    window = sinks = 0
    if rng.random() < 0.4:
        window = int(rng.integers(1, 400, endpoint=True))
        sinks = int(rng.choice([0, 1, 4, 37]))
    what = f"seed {seed}: {dtype} d={d} n_q={n_q} n_kv={n_kv} batch={batch} T={T} window={window} sinks={sinks}"
    print(what, flush=True)
    io = kv.IO_TORCH[dtype]
    q, k, v = (_rows(rng, (batch, T, h, d), io) for h in (n_q, n_kv, n_kv))
    nb = -(-T // 16)
    c = kv.KvCache(1, n_q, n_kv, d, batch * nb + 3, batch, nb, dtype, poison=True)
    for s in range(batch):
        c.seq_alloc(s, T)
    seqs = torch.arange(batch, dtype=torch.int32, device="cuda")
    out = c.attn_prefill(0, q, k, v, seqs=seqs, window=window, sinks=sinks)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    for s in range(batch):
        ref = A.prefill_attention(f64(q[s]), f64(k[s]), f64(v[s]), scale, window, sinks)
        assert_close(f64(out[s]), ref, io=dtype, what=f"{what}, sequence {s}")
        gk, gv = c.gather(0, s, 0, T)
        assert np.array_equal(bits(gk), bits(k[s])) and np.array_equal(bits(gv), bits(v[s])), \
            f"{what}: cache rows of sequence {s}"


@pytest.mark.parametrize("seed", range(32))
def test_random_extend(seed):
    rng = np.random.default_rng([303, seed])
    dtype = DTYPES[seed % 4]
    d = (64, 128)[(seed // 4) % 2]
    n_kv = int(rng.choice([1, 2, 4, 8]))
    n_q = n_kv * int(rng.choice([1, 2, 4, 8]))
    T = int(rng.choice([1, 7, 64, 65, 200]))
    lengths = _lengths(rng, int(rng.integers(1, 4, endpoint=True)), lo=T, hi=1200)
    window = sinks = 0
    if rng.random() < 0.4:
        window = int(rng.integers(1, 400, endpoint=True))
        sinks = int(rng.choice([0, 1, 4]))
    what = (f"seed {seed}: {dtype} d={d} n_q={n_q} n_kv={n_kv} T={T} lengths={lengths} "
            f"window={window} sinks={sinks}")
    print(what, flush=True)
    c, m = _cache(rng, dtype, n_q, n_kv, d, lengths)
    q = _rows(rng, (len(lengths), T, n_q, d), kv.IO_TORCH[dtype])
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    out = c.attn_extend(0, seqs, q, window=window, sinks=sinks)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    io = "f16" if dtype == "f16" else "bf16"
    for b in range(len(lengths)):
        K, V = m.logical_values(0, b)
        ref = A.extend_attention(f64(q[b]), K, V, scale, window=window, sinks=sinks)
        assert_close(f64(out[b]), ref, io=io, what=f"{what}, sequence {b}")
