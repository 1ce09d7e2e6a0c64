"""Prefix sharing with copy-on-write on the GPU: after shares, copies and
appends, both pools equal the oracle model's byte for byte (poisoned slots,
fp8 and int4 scales included), every sequence gathers its own rows, and decode of
every sequence matches the oracle on its rows."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import FP8_ABS_TOL, SCALED, assert_close, bits, f64, pools_match, stored_rows
from oracle import attention as A
from oracle.paged import PagedCacheModel

pytestmark = pytest.mark.gpu


class Pair:
    """A GPU cache and the oracle's model driven by the same operations."""

    def __init__(self, dt, n_q=8, n_kv=2, d=128, n_blocks=24, max_seqs=4, max_bps=8):
        self.dt, self.n_q, self.n_kv, self.d = dt, n_q, n_kv, d
        self.c = kv.KvCache(1, n_q, n_kv, d, n_blocks, max_seqs, max_bps, dt, poison=True)
        self.m = PagedCacheModel(1, n_kv, d, dt, n_blocks, max_seqs, max_bps, poison=True)
        self.io = kv.IO_TORCH[dt]
        self.rng = np.random.default_rng(0)

    def rows(self, n):
        r = lambda: torch.from_numpy(
            self.rng.standard_normal((n, self.n_kv, self.d), dtype=np.float32)).to(self.io).cuda()
        return r(), r()

    def _mirror(self, seq, start, k, v):
        if self.dt in SCALED:
            self.m.write_rows(0, seq, start, k.float().cpu().numpy(), v.float().cpu().numpy())
        else:
            self.m.write_rows(0, seq, start, bits(k), bits(v))

    def write(self, seq, start, k, v):
        sel = torch.tensor([seq], dtype=torch.int32, device="cuda")
        self.c.write(0, sel, start, k[None].contiguous(), v[None].contiguous())
        self._mirror(seq, start, k, v)

    def set_table(self, seq, blocks, L):
        self.c.set_block_table(seq, blocks, L)
        self.m.set_table(seq, blocks, L)

    def share(self, src, dst, plen):
        self.c.seq_share_prefix(src, dst, plen)
        self.m.share_prefix(src, dst, plen)

    def grow_append(self, seqs):
        self.c.seq_grow(seqs)
        self.m.grow(seqs)
        k, v = self.rows(len(seqs))
        self.c.append(0, torch.tensor(seqs, dtype=torch.int32, device="cuda"), k, v)
        for i, s in enumerate(seqs):
            self._mirror(s, self.m.length[s] - 1, k[i:i + 1], v[i:i + 1])

    def grow_by_write(self, seq, n):
        start = self.m.length[seq]
        self.c.seq_grow_by(seq, n)
        self.m.grow_by(seq, n)
        k, v = self.rows(n)
        self.write(seq, start, k, v)

    def pools_equal(self):
        return pools_match(self.c, self.m)


@pytest.mark.parametrize("dt", ["bf16", "fp8", "f16", "int4"])
def test_share_copy_on_write_append(dt):
    P = Pair(dt)
    perm = P.rng.permutation(24).astype(np.int32)
    P.set_table(0, perm[:3], 40)
    k, v = P.rows(40)
    P.write(0, 0, k, v)
    P.share(0, 1, 36)                  # block 2 shared, partly filled for seq 1
    P.grow_append([1])                 # seq 1 writes row 36: copy of block 2 first
    P.grow_append([0, 1])              # seq 0 row 40 (its own block now), seq 1 row 37
    P.share(1, 2, 32)                  # whole blocks only
    P.grow_by_write(2, 20)             # rows 32..51 of seq 2 into fresh blocks
    P.share(0, 3, 41)
    P.grow_append([3, 0])              # both need a copy?  seq 3 copies; seq 0 then owns alone
    torch.cuda.synchronize()
    assert P.pools_equal()
    for s in range(4):
        gk, gv = P.c.gather(0, s, 0, P.m.length[s])
        mk, mv = stored_rows(P.m, 0, s)
        assert np.array_equal(bits(gk), mk) and np.array_equal(bits(gv), mv)
    q = torch.from_numpy(P.rng.standard_normal((4, P.n_q, P.d), dtype=np.float32)).to(
        P.io).cuda()
    out = P.c.attn_decode(0, torch.arange(4, dtype=torch.int32, device="cuda"), q)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(P.d)
    io = "bf16" if dt in SCALED else dt
    for s in range(4):
        K, V = P.m.logical_values(0, s)
        ref = A.decode_attention(f64(q[s]), K, V, scale)
        tol = dict(abs_tol=FP8_ABS_TOL) if dt == "fp8" else {}
        assert_close(f64(out[s]), ref, io=io, what=f"{dt} seq {s}", **tol)


def test_release_keeps_blocks_other_sequences_hold():
    P = Pair("bf16")
    P.set_table(0, np.arange(3, dtype=np.int32), 48)
    k, v = P.rows(48)
    P.write(0, 0, k, v)
    P.share(0, 1, 48)
    P.c.seq_release(0)
    P.m.release(0)
    P.grow_append([1])
    torch.cuda.synchronize()
    assert P.pools_equal()
    gk, _ = P.c.gather(0, 1, 0, 49)
    assert np.array_equal(bits(gk)[:48], bits(k))
