"""Shared helpers for the GPU parity tests: build a cache from a seeded
workload through the C ABI, replay the same writes in the oracle's paged
model, and compare results to the oracle's tolerances."""
import math

import numpy as np
import torch

import kv_cache_flashattention_amd as kv
from oracle import attention as A
from oracle.codecs import int4_pack
from oracle.paged import PagedCacheModel

# Attention tolerances: max |y - r| <= 2e-2 and, per output row (one token
# and one query head), max|y - r| / max|r| <= 1e-2 for bf16/fp16 data; fp8
# caches: max |y - r| <= 6e-2 against the unquantised inputs.
ABS_TOL, REL_TOL, FP8_ABS_TOL = 2e-2, 1e-2, 6e-2


def bits(t):
    """Storage bit patterns of a CPU copy of a torch tensor, as numpy."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy().view(np.uint8)


def f64(t):
    return t.detach().cpu().double().numpy()


SCALED = ("fp8", "int4")


def stored_pools(m):
    """The model's pools as the library lays them out (int4: two codes per byte)."""
    return m.packed_pools() if m.dtype == "int4" else (m.K, m.V)


def pools_match(c, m):
    """GPU pools (and scales) equal the model's, byte for byte."""
    K, V = stored_pools(m)
    ok = np.array_equal(bits(c.k_pool), K) and np.array_equal(bits(c.v_pool), V)
    if m.dtype in SCALED:
        ok &= np.array_equal(bits(c.k_scale.view(torch.int32)).view(np.uint32),
                             m.Ks.view(np.uint32))
        ok &= np.array_equal(bits(c.v_scale.view(torch.int32)).view(np.uint32),
                             m.Vs.view(np.uint32))
    return bool(ok)


def stored_rows(m, layer, seq, start=0, count=None):
    """Rows of one sequence as kvc_gather returns them (int4: packed along d)."""
    K, V = m.logical_raw(layer, seq, start, count)
    if m.dtype == "int4":
        return int4_pack(K, -1), int4_pack(V, -1)
    return K, V


# Mantissa bits of each output type: a correctly rounded output differs from
# the exact value by up to half a unit in its last place, which for bf16
# exceeds 2e-2 once |y| >= 8.  The absolute bound is therefore applied on top
# of that unavoidable rounding of the output itself.
MANT_BITS = {"bf16": 8, "f16": 11, "f32": 24}


def half_ulp(r, io):
    r = np.abs(np.asarray(r, np.float64))
    e = np.floor(np.log2(np.maximum(r, 2.0 ** -126)))
    return np.exp2(e - MANT_BITS[io])


def errors(y, r, io=None):
    """(max abs error beyond the output rounding, max row-normwise relative
    error) over [..., d] rows; io=None counts the whole difference."""
    y, r = np.asarray(y, np.float64), np.asarray(r, np.float64)
    diff = np.abs(y - r)
    excess = diff if io is None else np.maximum(diff - half_ulp(r, io), 0.0)
    denom = np.maximum(np.abs(r).max(axis=-1), 1e-30)
    return float(excess.max()), float((diff.max(axis=-1) / denom).max())


def assert_close(y, r, abs_tol=ABS_TOL, rel_tol=REL_TOL, what="", io="bf16"):
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    a, rel = errors(y, r, io)
    assert a <= abs_tol and rel <= rel_tol, f"{what}: abs {a:.3e} rel {rel:.3e}"
    return a, rel


class Built:
    """A cache on the GPU and its oracle model, holding the same rows."""

    @property
    def io_name(self):
        return {"bf16": "bf16", "f16": "f16", "fp8": "bf16", "int4": "bf16", "f32": "f32"}[self.dt]

    def __init__(self, w, n_layers=1, layer=0, poison=True, identity_tables=False):
        """Populate every sequence of workload w in `layer`: its first L-1
        rows by one bulk write, then a grow of every sequence by one token
        and one kv_append of the last row for all of them together."""
        self.w, self.layer = w, layer
        dt = {"bf16": "bf16", "fp16": "f16", "fp8": "fp8", "int4": "int4", "f32": "f32"}[w.kv_dtype]
        self.dt = dt
        L = w.lengths
        max_bps = int(w.blocks_per_seq.max()) + 1
        n_blocks = w.n_blocks + w.batch        # spare blocks for growth
        self.c = kv.KvCache(n_layers, w.n_q, w.n_kv, w.d, n_blocks, w.batch, max_bps, dt,
                            poison=poison)
        self.m = PagedCacheModel(n_layers, w.n_kv, w.d, dt, n_blocks, w.batch, max_bps,
                                 poison=poison)
        tables = w.block_tables()
        if identity_tables:
            o, tables = 0, []
            for nb in w.blocks_per_seq:
                tables.append(np.arange(o, o + nb, dtype=np.int32))
                o += nb
        self.seqs = torch.arange(w.batch, dtype=torch.int32, device="cuda")
        io = kv.IO_TORCH[dt]
        self.io = io
        self.src_k, self.src_v = [], []          # io-typed source rows (fp8 check)
        for b in range(w.batch):
            pre = int(L[b]) - 1
            nb = -(-pre // 16)
            self.c.set_block_table(b, tables[b][:nb], pre)
            self.m.set_table(b, tables[b][:nb], pre)
            k, v = w.kv_rows(b, 0, int(L[b]))
            kt = torch.from_numpy(k).to(io).cuda()
            vt = torch.from_numpy(v).to(io).cuda()
            self.src_k.append(kt)
            self.src_v.append(vt)
            if pre:
                sel = torch.tensor([b], dtype=torch.int32, device="cuda")
                self.c.write(layer, sel, 0, kt[None, :pre].contiguous(),
                             vt[None, :pre].contiguous())
                self._mirror(layer, b, 0, kt[:pre], vt[:pre])
        self.c.seq_grow(list(range(w.batch)))
        self.m.grow(list(range(w.batch)))
        ks = torch.stack([self.src_k[b][int(L[b]) - 1] for b in range(w.batch)]).contiguous()
        vs = torch.stack([self.src_v[b][int(L[b]) - 1] for b in range(w.batch)]).contiguous()
        self.c.append(layer, self.seqs, ks, vs)
        for b in range(w.batch):
            self._mirror(layer, b, int(L[b]) - 1, ks[b:b + 1], vs[b:b + 1])
        torch.cuda.synchronize()

    def _mirror(self, layer, b, start, kt, vt):
        if self.dt in SCALED:
            self.m.write_rows(layer, b, start, kt.float().cpu().numpy(), vt.float().cpu().numpy())
        else:
            self.m.write_rows(layer, b, start, bits(kt), bits(vt))

    def pools_equal(self):
        return pools_match(self.c, self.m)

    def oracle_decode(self, q_io, b=None):
        """Oracle decode rows for every sequence (or one) from the model's
        stored values (dequantised for fp8 and int4)."""
        qd = f64(q_io)
        scale = 1 / math.sqrt(self.w.d)
        bs = range(self.w.batch) if b is None else [b]
        out = []
        for bb in bs:
            K, V = self.m.logical_values(self.layer, bb)
            out.append(A.decode_attention(qd[bb], K, V, scale))
        return np.array(out)

    def oracle_decode_source(self, q_io):
        """fp8 only: the oracle on the unquantised bf16 source rows."""
        qd = f64(q_io)
        scale = 1 / math.sqrt(self.w.d)
        return np.array([A.decode_attention(qd[b], f64(self.src_k[b]), f64(self.src_v[b]), scale)
                         for b in range(self.w.batch)])
