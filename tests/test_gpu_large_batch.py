"""Decode of batches wider than one launch's share (more than 2,048
sequences are run as consecutive sub-batches): every row against the
oracle, then an append + decode step (one call) across the sub-batch boundary."""
import math

import numpy as np
import pytest
import torch

from harness import Built, assert_close, bits, f64
from oracle import attention as A
from workloads import DecodeWorkload

pytestmark = pytest.mark.gpu


def test_decode_more_than_2048_sequences():
    w = DecodeWorkload("big", 2500, 8, 2, 64, "bf16", (1, 40))
    b = Built(w)
    q = torch.from_numpy(w.q()).to(torch.bfloat16).cuda()
    y = f64(b.c.attn_decode(0, b.seqs, q))
    scale = 1 / math.sqrt(w.d)
    qd = f64(q)
    for s in range(w.batch):
        K, V = b.m.logical_values(0, s)
        assert_close(y[s], A.decode_attention(qd[s], K, V, scale), what=f"seq {s}")
    # one append + decode step (one call) over the same batch
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((w.batch, w.n_kv, w.d), dtype=np.float32)).to(
        torch.bfloat16).cuda()
    v = torch.from_numpy(rng.standard_normal((w.batch, w.n_kv, w.d), dtype=np.float32)).to(
        torch.bfloat16).cuda()
    b.c.seq_grow(list(range(w.batch)))
    b.m.grow(list(range(w.batch)))
    y2 = f64(b.c.attn_decode_append(0, b.seqs, k, v, q))
    checked = set(range(0, 40)) | set(range(2030, 2070)) | set(range(2460, 2500))
    for s in range(w.batch):
        b.m.write_rows(0, s, int(b.m.length[s]) - 1, bits(k[s:s + 1]), bits(v[s:s + 1]))
        if s in checked:
            K, V = b.m.logical_values(0, s)
            assert_close(y2[s], A.decode_attention(qd[s], K, V, scale), what=f"append+decode seq {s}")
    assert b.pools_equal()


@pytest.mark.parametrize("batch", [1, 64, 65, 256, 257, 700, 2048 + 40])
def test_decode_batches_around_the_prologue_layouts(batch):
    """The work list's prologue lets every wave scan a batch of up to 64
    entries on its own, gives each thread one batch entry up to 256 entries
    and eight contiguous ones above; the wave's first entry is found 64
    entries at a time; 2,088 sequences run as a 2,048-entry sub-batch and a
    40-entry one.  Every row against the oracle on both sides of those
    edges."""
    print(f"batch {batch}", flush=True)
    w = DecodeWorkload(f"edge{batch}", batch, 8, 2, 64, "bf16", (1, 200))
    b = Built(w)
    q = torch.from_numpy(w.q()).to(torch.bfloat16).cuda()
    y = f64(b.c.attn_decode(0, b.seqs, q))
    scale = 1 / math.sqrt(w.d)
    qd = f64(q)
    for s in range(w.batch):
        K, V = b.m.logical_values(0, s)
        assert_close(y[s], A.decode_attention(qd[s], K, V, scale), what=f"batch {batch}, seq {s}")
