"""Seeded random sequences of cache operations on the GPU against the oracle's
paged model ("KV Cache & Flash Attention.", PagedAttention section: blocks
taken on demand, prefixes shared through the table, blocks returned when a
sequence ends; copy-on-write when a shared, partly filled block would
change).

Each step draws one operation on a small paged cache and applies it to the
library and to the model: a new sequence with its rows written in bulk, one
token for a subset of the live sequences (grow and append in one launch, or
grow then append), a prompt chunk, a shared prefix, a release.  An operation
the free list cannot serve is refused by both sides and changes neither.
After every step both pools (and fp8/int4 scales) are equal byte for byte;
at the end every live sequence is decoded and compared with the float64
oracle on the values the model holds."""
import math

import numpy as np
import pytest
import torch

import kv_cache_flashattention_amd as kv
from harness import assert_close, f64
from oracle import attention as A
from test_gpu_prefix import Pair

pytestmark = pytest.mark.gpu


def _refused(fn):
    try:
        fn()
    except kv.KvcError as e:
        assert e.code == kv.KVC_E_NO_BLOCKS, e
        return True
    return False


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dt", ["bf16", "f16", "fp8", "int4"])
def test_random_cache_operations(dt, seed):
    P = Pair(dt, n_blocks=12, max_seqs=6, max_bps=12)      # small: the free list runs out
    rng = np.random.default_rng([404, seed])
    P.rng = np.random.default_rng([405, seed])
    live = []
    history = []
    seen = {"refused": 0, "copy": 0, "grow_append": 0, "share": 0}
    for step in range(80):
        free_ids = [s for s in range(6) if s not in live]
        ops = ["new"] if not live else ["grow_append", "grow_then_append", "chunk", "release"]
        if live and free_ids:
            ops += ["new", "share"]
        op = str(rng.choice(ops))
        what = f"{dt} seed {seed} step {step}: {op}"
        if op == "new" and free_ids:
            s, L = int(rng.choice(free_ids)), int(rng.integers(1, 60, endpoint=True))
            need = -(-L // 16)
            if need > len(P.m.free):
                seen["refused"] += 1
                assert _refused(lambda: P.c.seq_alloc(s, L)), what
            else:
                P.c.seq_alloc(s, L)
                P.m.alloc(s, L)
                k, v = P.rows(L)
                P.write(s, 0, k, v)
                live.append(s)
            what += f" seq {s} len {L}"
        elif op in ("grow_append", "grow_then_append"):
            sub = [int(x) for x in rng.permutation(live)[:int(rng.integers(1, len(live), endpoint=True))]]
            sub = [s for s in sub if P.m.length[s] < 12 * 16]
            if not sub:
                continue
            need = sum(1 for s in sub if P.m.length[s] % 16 == 0 or P.m._shared_partial(s))
            k, v = P.rows(len(sub))
            seen["copy"] += any(P.m._shared_partial(s) for s in sub)
            if need > len(P.m.free):
                seen["refused"] += 1
                if op == "grow_append":
                    assert _refused(lambda: P.c.seq_grow_append(0, sub, k, v)), what
                else:
                    assert _refused(lambda: P.c.seq_grow(sub)), what
            elif op == "grow_append":
                seen["grow_append"] += 1
                P.c.seq_grow_append(0, sub, k, v)
                P.m.grow(sub)
                for i, s in enumerate(sub):
                    P._mirror(s, P.m.length[s] - 1, k[i:i + 1], v[i:i + 1])
            else:
                P.grow_append(sub)
            what += f" seqs {sub}"
        elif op == "chunk":
            s, n = int(rng.choice(live)), int(rng.integers(1, 20, endpoint=True))
            if P.m.length[s] + n > 12 * 16:
                continue
            need = -(-(P.m.length[s] + n) // 16) - -(-P.m.length[s] // 16)
            need += 1 if P.m._shared_partial(s) else 0
            if need > len(P.m.free):
                seen["refused"] += 1
                assert _refused(lambda: P.c.seq_grow_by(s, n)), what
            else:
                P.grow_by_write(s, n)
            what += f" seq {s} +{n}"
        elif op == "share":
            src, dst = int(rng.choice(live)), int(rng.choice(free_ids))
            plen = int(rng.integers(0, P.m.length[src], endpoint=True))
            P.share(src, dst, plen)
            seen["share"] += 1
            live.append(dst)
            what += f" {src} -> {dst} prefix {plen}"
        elif op == "release":
            s = int(rng.choice(live))
            P.c.seq_release(s)
            P.m.release(s)
            live.remove(s)
            what += f" seq {s}"
        history.append(what)
        assert P.pools_equal(), "\n".join(history)
        for s in live:
            assert P.c.seq_len(s) == P.m.length[s], what
            assert list(P.c.seq_blocks(s)) == P.m.table[s], what
    # the draw covered every kind of step this test is for
    assert all(seen.values()), seen
    # every live sequence with rows, decoded against the oracle
    rows = [s for s in live if P.m.length[s] > 0]
    if rows:
        seqs = torch.tensor(rows, dtype=torch.int32, device="cuda")
        q = torch.from_numpy(P.rng.standard_normal((len(rows), P.n_q, P.d),
                                                   dtype=np.float32)).to(P.io).cuda()
        out = P.c.attn_decode(0, seqs, q)
        torch.cuda.synchronize()
        io = "f16" if dt == "f16" else "bf16"
        for i, s in enumerate(rows):
            K, V = P.m.logical_values(0, s)
            ref = A.decode_attention(f64(q[i]), K, V, 1 / math.sqrt(P.d))
            assert_close(f64(out[i]), ref, io=io, what=f"{dt} seed {seed}: sequence {s}")
