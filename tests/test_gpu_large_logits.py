"""Large logits: queries and keys scaled by 4, so scores (q . k / sqrt(d))
have a standard deviation of about 16 and a row's running maximum grows by
far more than the kernels' lazy-rescale threshold (2^8 in the base-2 domain)
many times along the row.  Decode (bf16, f16 and fp8 caches), prefill and
extend must still match the float64 oracle (fp8 against the dequantised
cache values).  The softmax stays exact under any schedule of rescales, so
the bounds are the ordinary ones."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import assert_close, f64
from oracle import attention as A
from oracle.paged import PagedCacheModel

pytestmark = pytest.mark.gpu

SCALE_UP = 4.0


def _rows(rng, shape, io, s=1.0):
    return torch.from_numpy((s * rng.standard_normal(shape)).astype(np.float32)).to(io).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f16", "fp8"])
def test_decode_large_logits(dtype):
    n_q, n_kv, d = 16, 2, 128
    lengths = [1, 37, 300, 777]
    rng = np.random.default_rng(21)
    io = kv.IO_TORCH[dtype]
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 4
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max(nbs) + 1, dtype, poison=True)
    m = PagedCacheModel(1, n_kv, d, dtype, n_blocks, len(lengths), max(nbs) + 1, poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    o = 0
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        m.set_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        k = _rows(rng, (1, L, n_kv, d), io, SCALE_UP)
        v = _rows(rng, (1, L, n_kv, d), io)
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        if dtype == "fp8":
            m.write_rows(0, b, 0, k[0].float().cpu().numpy(), v[0].float().cpu().numpy())
        else:
            m.write_rows(0, b, 0, k[0].cpu().view(torch.int16).numpy().view(np.uint16),
                         v[0].cpu().view(torch.int16).numpy().view(np.uint16))
    q = _rows(rng, (len(lengths), n_q, d), io, SCALE_UP)
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(d)
    for splits in (0, 3):
        y = f64(c.attn_decode(0, seqs, q, num_splits=splits))
        for b in range(len(lengths)):
            K, V = m.logical_values(0, b)
            ref = A.decode_attention(f64(q[b]), K, V, scale)
            assert_close(y[b], ref, what=f"{dtype} large-logit decode seq {b} splits {splits}",
                         io="f16" if dtype == "f16" else "bf16")


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_large_logits(d):
    n_q, n_kv, T = 8, 2, 300
    rng = np.random.default_rng(22)
    io = torch.bfloat16
    q = _rows(rng, (2, T, n_q, d), io, SCALE_UP)
    k = _rows(rng, (2, T, n_kv, d), io, SCALE_UP)
    v = _rows(rng, (2, T, n_kv, d), io)
    c = kv.KvCache(1, n_q, n_kv, d, 4, 1, 1, "bf16")
    out = c.attn_prefill(0, q, k, v)
    torch.cuda.synchronize()
    for s in range(2):
        ref = A.prefill_attention(f64(q[s]), f64(k[s]), f64(v[s]), 1 / math.sqrt(d))
        assert_close(f64(out[s]), ref, what=f"large-logit prefill d={d} seq {s}")


def test_extend_large_logits():
    n_q, n_kv, d, T = 8, 2, 128, 96
    lengths = [T + 400, T + 5]
    rng = np.random.default_rng(23)
    io = torch.bfloat16
    nbs = [-(-L // 16) for L in lengths]
    n_blocks = sum(nbs) + 3
    c = kv.KvCache(1, n_q, n_kv, d, n_blocks, len(lengths), max(nbs) + 1, "bf16", poison=True)
    perm = rng.permutation(n_blocks).astype(np.int32)
    o, rows = 0, []
    for b, L in enumerate(lengths):
        c.set_block_table(b, perm[o:o + nbs[b]], L)
        o += nbs[b]
        k = _rows(rng, (1, L, n_kv, d), io, SCALE_UP)
        v = _rows(rng, (1, L, n_kv, d), io)
        c.write(0, torch.tensor([b], dtype=torch.int32, device="cuda"), 0, k, v)
        rows.append((k[0], v[0]))
    q = _rows(rng, (len(lengths), T, n_q, d), io, SCALE_UP)
    seqs = torch.arange(len(lengths), dtype=torch.int32, device="cuda")
    out = c.attn_extend(0, seqs, q)
    torch.cuda.synchronize()
    for b in range(len(lengths)):
        ref = A.extend_attention(f64(q[b]), f64(rows[b][0]), f64(rows[b][1]), 1 / math.sqrt(d))
        assert_close(f64(out[b]), ref, what=f"large-logit extend seq {b}")
