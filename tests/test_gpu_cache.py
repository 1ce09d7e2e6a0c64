"""Cache writes on the GPU are bit-exact against the oracle's paged model:
bulk writes, kv_append, the block-table gather, fp8 codes and scales."""
import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import Built, bits
from oracle.paged import PagedCacheModel
from workloads import DecodeWorkload

pytestmark = pytest.mark.gpu


def small(dtype, d=128, n_q=8, n_kv=2, lengths=(1, 70), batch=5, outliers=False, tag="cache"):
    return DecodeWorkload(tag + dtype, batch, n_q, n_kv, d, dtype, lengths, outliers=outliers)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "f32", "fp8"])
@pytest.mark.parametrize("d", [64, 128])
def test_write_append_pools_bit_exact(dtype, d):
    w = small(dtype, d=d, outliers=(dtype == "fp8"))
    b = Built(w, n_layers=2, layer=1)
    assert b.pools_equal()


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
def test_gather_returns_logical_rows(dtype):
    w = small(dtype, lengths=(20, 90), outliers=(dtype == "fp8"))
    b = Built(w)
    for s in range(w.batch):
        L = int(w.lengths[s])
        for start, count in ((0, L), (L // 3, L - L // 3), (L - 1, 1)):
            k, v = b.c.gather(0, s, start, count)
            mk, mv = b.m.logical_raw(0, s, start, count)
            assert np.array_equal(bits(k), mk) and np.array_equal(bits(v), mv)


def test_fp8_append_requantises_growing_block():
    """Rows appended one at a time into one block with growing magnitudes:
    codes and scales follow the oracle's slab rule bit for bit."""
    c = kv.KvCache(1, 4, 1, 128, 4, 1, 4, "fp8", poison=True)
    m = PagedCacheModel(1, 1, 128, "fp8", 4, 1, 4, poison=True)
    c.seq_alloc(0, 0)
    m.alloc(0, 0)
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(0)
    for r in range(40):
        mag = [0.0, 1e-3, 1.0, 0.5, 7.0, 3.0, 300.0, 1e4][r % 8] * (1 + r // 8)
        row = (rng.standard_normal((1, 1, 128)) * mag).astype(np.float32)
        k = torch.from_numpy(row).to(torch.bfloat16).cuda()
        v = torch.from_numpy(row[:, :, ::-1].copy()).to(torch.bfloat16).cuda()
        c.seq_grow([0])
        m.grow([0])
        c.append(0, seqs, k[0:1].reshape(1, 1, 128).contiguous(), v.reshape(1, 1, 128).contiguous())
        m.write_rows(0, 0, r, k.float().cpu().numpy().reshape(1, 1, 128),
                     v.float().cpu().numpy().reshape(1, 1, 128))
        torch.cuda.synchronize()
        assert np.array_equal(bits(c.k_pool), m.K), f"row {r}"
        assert np.array_equal(bits(c.v_pool), m.V), f"row {r}"
        assert np.array_equal(bits(c.k_scale.view(torch.int32)).view(np.uint32),
                              m.Ks.view(np.uint32)), f"row {r}"


def test_fp8_write_mid_block_matches_slab_rule():
    """Bulk writes that start and stop inside blocks, on top of earlier rows."""
    c = kv.KvCache(1, 8, 2, 64, 12, 2, 8, "fp8", poison=True)
    m = PagedCacheModel(1, 2, 64, "fp8", 12, 2, 8, poison=True)
    c.set_block_table(0, [7, 2, 9, 4], 60)
    m.set_table(0, [7, 2, 9, 4], 60)
    seqs = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(1)
    for start, T, mag in ((0, 5, 1.0), (5, 20, 3.0), (25, 3, 0.1), (28, 32, 50.0)):
        rows = (rng.standard_normal((1, T, 2, 64)) * mag).astype(np.float32)
        k = torch.from_numpy(rows).to(torch.bfloat16).cuda()
        v = torch.from_numpy(-rows).to(torch.bfloat16).cuda()
        c.write(0, seqs, start, k, v)
        m.write_rows(0, 0, start, k[0].float().cpu().numpy(), v[0].float().cpu().numpy())
    torch.cuda.synchronize()
    assert np.array_equal(bits(c.k_pool), m.K) and np.array_equal(bits(c.v_pool), m.V)
    assert np.array_equal(bits(c.v_scale.view(torch.int32)).view(np.uint32), m.Vs.view(np.uint32))


def test_invalid_device_entries_are_skipped():
    """Sequence ids outside the table or sequences of length 0 are not
    written and produce NaN decode rows; valid entries are unaffected."""
    w = small("bf16", batch=3, lengths=(5, 40))
    b = Built(w)
    before_k = bits(b.c.k_pool).copy()
    seqs = torch.tensor([0, 99, -1], dtype=torch.int32, device="cuda")
    k = torch.randn(3, w.n_kv, w.d, device="cuda").to(torch.bfloat16)
    b.c.append(0, seqs, k, k)
    torch.cuda.synchronize()
    after = bits(b.c.k_pool)
    changed = np.argwhere(before_k != after)
    blk_of_0 = b.m.physical(0, int(w.lengths[0]) - 1)[0]
    assert all(int(i[1]) == blk_of_0 for i in changed)
    q = torch.randn(3, w.n_q, w.d, device="cuda").to(torch.bfloat16)
    out = b.c.attn_decode(0, seqs, q).float().cpu().numpy()
    assert np.all(np.isfinite(out[0])) and np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
