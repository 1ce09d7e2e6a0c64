"""Prefill that fills the cache (kvc_attn_prefill with sequences) on 16-bit
caches.  The whole pool must equal the oracle's paged model byte for byte
(rows written once, slots past the prompt still holding the poison pattern,
unusable entries and too-short sequences untouched), for ragged prompt
lengths, both head sizes, windows, and a layer other than 0; the attention
rows must match the oracle."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import assert_close, bits, f64, pools_match
from oracle import attention as A
from oracle.paged import PagedCacheModel

pytestmark = pytest.mark.gpu

IO = {"bf16": torch.bfloat16, "f16": torch.float16}


def _case(dtype, d, T, window=0, sinks=0, seed=11):
    n_q, n_kv, n_layers, layer = 8, 2, 2, 1
    rng = np.random.default_rng(seed)
    # entry 0, 1: prompts of T rows; entry 2: a sequence holding fewer rows
    # than the prompt (not written); entry 3: an id outside the table
    nbT = -(-T // 16)
    short = max(T - 17, 1)
    nbs = -(-short // 16)
    n_blocks = 2 * nbT + nbs + 5
    c = kv.KvCache(n_layers, n_q, n_kv, d, n_blocks, 3, nbT + 1, dtype, poison=True)
    m = PagedCacheModel(n_layers, n_kv, d, dtype, n_blocks, 3, nbT + 1, poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    tabs = [perm[:nbT], perm[nbT:2 * nbT], perm[2 * nbT:2 * nbT + nbs]]
    for s, (tab, L) in enumerate(zip(tabs, (T, T, short))):
        c.set_block_table(s, tab, L)
        m.set_table(s, tab, L)
    q = torch.from_numpy(rng.standard_normal((4, T, n_q, d), dtype=np.float32)).to(IO[dtype]).cuda()
    k = torch.from_numpy(rng.standard_normal((4, T, n_kv, d), dtype=np.float32)).to(IO[dtype]).cuda()
    v = torch.from_numpy(rng.standard_normal((4, T, n_kv, d), dtype=np.float32)).to(IO[dtype]).cuda()
    seqs = torch.tensor([1, 0, 2, 99], dtype=torch.int32, device="cuda")
    out = c.attn_prefill(layer, q, k, v, seqs=seqs, window=window, sinks=sinks)
    torch.cuda.synchronize()
    m.write_rows(layer, 1, 0, bits(k[0]), bits(v[0]))
    m.write_rows(layer, 0, 0, bits(k[1]), bits(v[1]))
    return c, m, q, k, v, out


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [77, 301, 515])
def test_prefill_writes_cache_bit_exact(dtype, d, T):
    c, m, q, k, v, out = _case(dtype, d, T)
    assert pools_match(c, m), f"{dtype} d={d} T={T}: pools differ from the oracle model"
    scale = 1 / math.sqrt(d)
    for s in (0, 3):                                   # a written and an unwritten entry
        ref = A.prefill_attention(f64(q[s]), f64(k[s]), f64(v[s]), scale)
        assert_close(f64(out[s]), ref, what=f"prefill {dtype} d={d} T={T} entry {s}", io=dtype)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
def test_windowed_prefill_writes_cache_bit_exact(dtype, d):
    T, window, sinks = 700, 100, 4
    c, m, q, k, v, out = _case(dtype, d, T, window=window, sinks=sinks, seed=5)
    assert pools_match(c, m)
    ref = A.prefill_attention(f64(q[1]), f64(k[1]), f64(v[1]), 1 / math.sqrt(d),
                              window=window, sinks=sinks)
    assert_close(f64(out[1]), ref, what=f"windowed prefill {dtype}", io=dtype)
