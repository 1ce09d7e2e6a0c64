"""The algorithmic figures the bench divides by, pinned on the CPU.

The rooflines in bench.py are algorithmic bytes (decode) or FLOPs (prefill,
extend) per call over the kernel's time, so a wrong count would misstate
every fraction of peak.  Each count is checked here against a brute-force
count over the oracle's visibility mask ("KV Cache & Flash Attention.",
Flash Attention section: every visible (query, key) pair costs one QK^T dot
product and one PV accumulation of d multiply-adds each) or against the
cache layout written out element by element, and the headline prefill figure
against the closed form quoted with the measurements."""
import numpy as np
import pytest

import bench
from oracle.attention import visible_keys


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 64, 100])
def test_prefill_flops_counts_every_visible_pair(T):
    batch, n_q, d = 2, 3, 64
    pairs = int(visible_keys(np.arange(T), T).sum())
    assert bench.prefill_flops(batch, T, n_q, d) == batch * n_q * pairs * 4 * d


def test_prefill_flops_headline_shape():
    # 4 sequences of 8,192 tokens, 32 query heads of 128
    assert bench.prefill_flops(4, 8192, 32, 128) == 2_199_291_691_008


@pytest.mark.parametrize("ctx,chunk", [(0, 5), (7, 1), (16, 16), (40, 9)])
def test_extend_flops_counts_every_visible_pair(ctx, chunk):
    batch, n_q, d = 3, 2, 128
    # chunk queries at positions ctx .. ctx+chunk-1 against ctx+chunk keys
    pairs = int(visible_keys(np.arange(ctx, ctx + chunk), ctx + chunk).sum())
    assert bench.extend_flops(batch, ctx, chunk, n_q, d) == batch * n_q * pairs * 4 * d


@pytest.mark.parametrize("L,window,sinks", [(1, 0, 0), (50, 0, 0), (50, 16, 0), (50, 16, 4),
                                            (50, 49, 4), (50, 60, 4), (100, 33, 20),
                                            (100, 1, 0)])
def test_window_rows_match_the_oracle_mask(L, window, sinks):
    vis = visible_keys([L - 1], L, window, sinks)[0]
    rows, blocks = bench.window_rows(L, window, sinks)
    assert rows == int(vis.sum())
    assert blocks == len(np.unique(np.nonzero(vis)[0] // 16))


class _W:
    def __init__(self, batch, n_q, n_kv, d):
        self.batch, self.n_q, self.n_kv, self.d = batch, n_q, n_kv, d


@pytest.mark.parametrize("kv_elem,scaled", [(2, False), (1, True), (0.5, True)])
def test_decode_bytes_element_by_element(kv_elem, scaled):
    w = _W(batch=3, n_q=8, n_kv=2, d=64)
    lengths = np.array([1, 16, 33])
    total = 0.0
    for L in lengths:
        total += 2 * L * w.n_kv * w.d * kv_elem          # every K and V element once
        nblk = -(-L // 16)
        total += nblk * 4                                 # one int32 table entry per block
        if scaled:
            total += 2 * nblk * w.n_kv * 4                # a float K and V scale per block and head
    total += 2 * w.batch * w.n_q * w.d * 2               # 16-bit query and output rows
    assert bench.decode_bytes(w, lengths, kv_elem) == int(total)
