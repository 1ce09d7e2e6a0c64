"""kvc_seq_grow_append against kvc_seq_grow followed by kvc_append.

Two caches start from the same state (same tables, same rows written).
Each step grows a batch of sequences by one token and appends its rows:
one cache through the fused call, the other through the two calls. After
every step the two hold bit-identical pools and scales, equal device tables
and lengths, and equal host bookkeeping.  The cases cover new blocks (lengths
on block edges), copy-on-write of a shared, partly filled last block, batches
split over several launches, and refused calls that change nothing.  The two
calls it is compared with are themselves checked against the oracle's paged
model (test_gpu_cache.py, test_gpu_prefix.py)."""
import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv

pytestmark = pytest.mark.gpu

DTYPES = ("bf16", "f16", "f32", "fp8", "int4")


def _rows(rng, n, n_kv, d, io):
    return torch.from_numpy(rng.standard_normal((n, n_kv, d), dtype=np.float32) * 3).to(io).cuda()


def _twins(dtype, lengths, n_kv=2, d=128, n_layers=2, spare=64):
    """Two caches holding the same rows for sequences 0..len(lengths)-1."""
    rng = np.random.default_rng([7, len(lengths), d])
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + spare
    max_bps = max(nbs) + 8
    io = kv.IO_TORCH[dtype]
    caches = [kv.KvCache(n_layers, 4 * n_kv, n_kv, d, n_blocks, len(lengths) + 4, max_bps, dtype,
                         poison=True) for _ in range(2)]
    for s, L in enumerate(lengths):
        k = torch.from_numpy(rng.standard_normal((1, L, n_kv, d), dtype=np.float32)).to(io).cuda()
        v = torch.from_numpy(rng.standard_normal((1, L, n_kv, d), dtype=np.float32)).to(io).cuda()
        for c in caches:
            c.seq_alloc(s, L)
            for layer in range(n_layers):
                c.write(layer, torch.tensor([s], dtype=torch.int32, device="cuda"), 0, k, v)
    torch.cuda.synchronize()
    return caches, rng, io


def _same(a, b, what):
    torch.cuda.synchronize()
    for name in ("k_pool", "v_pool", "k_scale", "v_scale", "block_table", "seq_len_dev"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            assert y is None
            continue
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"{what}: {name} differs"


def _host_state(c, seqs):
    return [(c.seq_len(s), list(c.seq_blocks(s))) for s in seqs], c.free_blocks()


@pytest.mark.parametrize("dtype", DTYPES)
def test_grow_append_equals_grow_then_append(dtype):
    # lengths on and around block edges, so steps start new blocks
    lengths = [1, 15, 16, 17, 31, 32, 47, 100]
    (a, b), rng, io = _twins(dtype, lengths)
    seqs_host = list(range(len(lengths)))
    seqs = torch.tensor(seqs_host, dtype=torch.int32, device="cuda")
    for step in range(20):
        layer = step % 2
        sub = [s for s in seqs_host if (s + step) % 3 != 0]    # a changing subset
        k, v = _rows(rng, len(sub), a.n_kv, a.d, io), _rows(rng, len(sub), a.n_kv, a.d, io)
        a.seq_grow_append(layer, sub, k, v)
        b.seq_grow(sub)
        b.append(layer, torch.tensor(sub, dtype=torch.int32, device="cuda"), k, v)
        _same(a, b, f"{dtype} step {step}")
        assert _host_state(a, seqs_host) == _host_state(b, seqs_host)
    del seqs


@pytest.mark.parametrize("dtype", ("bf16", "fp8", "int4"))
def test_grow_append_copies_a_shared_partial_block(dtype):
    """dst shares src's first 40 rows (block 2 half full): its first grow
    must copy that block before the row lands, exactly as grow + append."""
    (a, b), rng, io = _twins(dtype, [64])
    for c in (a, b):
        c.seq_share_prefix(0, 1, 40)
    for step in range(3):
        k, v = _rows(rng, 2, a.n_kv, a.d, io), _rows(rng, 2, a.n_kv, a.d, io)
        a.seq_grow_append(0, [1, 0], k, v)
        b.seq_grow([1, 0])
        b.append(0, torch.tensor([1, 0], dtype=torch.int32, device="cuda"), k, v)
        _same(a, b, f"{dtype} shared step {step}")
        assert _host_state(a, [0, 1]) == _host_state(b, [0, 1])
    assert a.seq_blocks(1)[2] != a.seq_blocks(0)[2]       # the copy happened


@pytest.mark.parametrize("dtype", ("bf16", "fp8"))
def test_grow_append_batches_over_several_launches(dtype):
    lengths = [int(x) for x in np.random.default_rng(3).integers(1, 60, size=230)]
    (a, b), rng, io = _twins(dtype, lengths, n_kv=1, d=64, n_layers=1, spare=300)
    seqs_host = list(range(len(lengths)))
    for step in range(3):
        k, v = _rows(rng, len(seqs_host), 1, 64, io), _rows(rng, len(seqs_host), 1, 64, io)
        a.seq_grow_append(0, seqs_host, k, v)
        b.seq_grow(seqs_host)
        b.append(0, torch.tensor(seqs_host, dtype=torch.int32, device="cuda"), k, v)
        _same(a, b, f"{dtype} 230 sequences, step {step}")
    assert _host_state(a, seqs_host) == _host_state(b, seqs_host)


def test_grow_append_refusals_change_nothing():
    (a, _), rng, io = _twins("bf16", [16, 20])
    before = _host_state(a, [0, 1])
    pools = (a.k_pool.clone(), a.v_pool.clone(), a.block_table.clone(), a.seq_len_dev.clone())
    k, v = _rows(rng, 2, a.n_kv, a.d, io), _rows(rng, 2, a.n_kv, a.d, io)
    for seqs, layer in (([0, 0], 0),          # duplicate id
                        ([0, 5], 0),          # sequence not live
                        ([0, 1], 2)):         # layer out of range
        with pytest.raises(kv.KvcError):
            a.seq_grow_append(layer, seqs, k, v)
    torch.cuda.synchronize()
    assert _host_state(a, [0, 1]) == before
    for x, y in zip(pools, (a.k_pool, a.v_pool, a.block_table, a.seq_len_dev)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))   # bits (the pools hold NaN)
