"""Seeded synthetic inputs for the five attention workloads.

This module only draws random numbers and arranges them into arrays of the
workloads' shapes.  It holds none of the attention arithmetic and imports
neither the library nor the oracle; both sides are fed from it.

Recipe (float32 draws from numpy's PCG64; every array is reproducible from
its seed and, for the large caches, from the chunk it lives in):

* GPT-2 small, one layer (``gpt2_small``): x [261, 768] ~ N(0,1);
  W_q, W_k, W_v [768, 768] ~ N(0,1)/sqrt(768), drawn in that order;
  Q = x W_q (likewise K, V) in float64, rounded to float32, heads split as
  12 x 64 columns.  Decode step t then draws k_t, v_t, q_t [12, 64] ~ N(0,1).
* Paged decode (``decode_workload``): per-sequence K/V rows ~ N(0,1), drawn
  in chunks of 1024 rows seeded by (seed, tag, sequence, chunk); optional
  outliers: each element independently, with probability 1/100, times 8
  (separate draws for K and V); queries [B, n_q, d] ~ N(0,1).
  Context lengths either fixed or integer-uniform on [lo, hi] inclusive.
* Causal prefill (``prefill_workload``): q [B, T, n_q, d], k, v
  [B, T, n_kv, d] ~ N(0,1).
* Block tables: a random permutation of the whole pool, cut into
  consecutive runs of ceil(L/16) blocks per sequence, so that no kernel can
  rely on a sequence's blocks being adjacent.
"""
import zlib

import numpy as np

CHUNK = 1024
BLOCK = 16


def _rng(*key):
    """Generator seeded by a tuple of ints and strings (strings by CRC-32)."""
    ints = [zlib.crc32(k.encode()) if isinstance(k, str) else int(k) for k in key]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(ints)))


# ------------------------------------------------------------------ GPT-2 small
class GPT2Small:
    """One attention layer of GPT-2 small: 12 heads of 64, fp32, seed 0."""

    def __init__(self, prompt_len=261, n_new=200, seed=0, n_heads=12, d_head=64):
        self.prompt_len, self.n_new, self.seed = prompt_len, n_new, seed
        self.n_heads, self.d = n_heads, d_head
        width = n_heads * d_head
        rng = np.random.Generator(np.random.PCG64(seed))
        x = rng.standard_normal((prompt_len, width))
        Wq = rng.standard_normal((width, width)) / np.sqrt(width)
        Wk = rng.standard_normal((width, width)) / np.sqrt(width)
        Wv = rng.standard_normal((width, width)) / np.sqrt(width)
        shape = (prompt_len, n_heads, d_head)
        self.q_prompt = (x @ Wq).astype(np.float32).reshape(shape)
        self.k_prompt = (x @ Wk).astype(np.float32).reshape(shape)
        self.v_prompt = (x @ Wv).astype(np.float32).reshape(shape)
        self.steps = []
        for _ in range(n_new):
            k = rng.standard_normal((n_heads, d_head)).astype(np.float32)
            v = rng.standard_normal((n_heads, d_head)).astype(np.float32)
            q = rng.standard_normal((n_heads, d_head)).astype(np.float32)
            self.steps.append((k, v, q))


# ------------------------------------------------------------------ paged decode
class DecodeWorkload:
    """Paged decode: B sequences with cached contexts and one new token each."""

    def __init__(self, tag, batch, n_q, n_kv, d, kv_dtype, lengths, outliers=False,
                 seed=0, spare_blocks=0):
        self.tag, self.batch, self.n_q, self.n_kv, self.d = tag, batch, n_q, n_kv, d
        self.kv_dtype, self.outliers, self.seed = kv_dtype, outliers, seed
        if isinstance(lengths, tuple):
            lo, hi = lengths
            self.lengths = _rng(seed, tag, 1 << 20).integers(lo, hi, size=batch, endpoint=True)
        else:
            self.lengths = np.full(batch, int(lengths))
        self.lengths = self.lengths.astype(np.int64)
        self.blocks_per_seq = -(-self.lengths // BLOCK)
        self.n_blocks = int(self.blocks_per_seq.sum()) + spare_blocks

    def q(self):
        return _rng(self.seed, self.tag, 1 << 21).standard_normal(
            (self.batch, self.n_q, self.d), dtype=np.float32)

    def _chunk(self, b, c):
        rng = _rng(self.seed, self.tag, b, c)
        shape = (CHUNK, self.n_kv, self.d)
        k = rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        if self.outliers:
            k = np.where(rng.random(shape) < 0.01, k * np.float32(8), k)
            v = np.where(rng.random(shape) < 0.01, v * np.float32(8), v)
        return k, v

    def kv_rows(self, b, start, count):
        """float32 K, V rows [count, n_kv, d] of sequence b at positions start.."""
        ks, vs = [], []
        p, end = start, start + count
        while p < end:
            c = p // CHUNK
            k, v = self._chunk(b, c)
            lo, hi = p - c * CHUNK, min(end, (c + 1) * CHUNK) - c * CHUNK
            ks.append(k[lo:hi])
            vs.append(v[lo:hi])
            p = (c + 1) * CHUNK
        if not ks:
            z = np.zeros((0, self.n_kv, self.d), dtype=np.float32)
            return z, z.copy()
        return np.concatenate(ks), np.concatenate(vs)

    def block_tables(self):
        """Shuffled tables: a permutation of the pool cut per sequence."""
        perm = _rng(self.seed, self.tag, 1 << 22).permutation(self.n_blocks).astype(np.int32)
        out, o = [], 0
        for nb in self.blocks_per_seq:
            out.append(perm[o:o + nb])
            o += nb
        return out


def decode_workload(name, small=False, seed=0):
    """The paged-decode workloads at full size, or shrunk for quick parity tests.

    name: 'llama8b_decode' (40 sequences, 32 q / 8 kv heads, d 128, bf16,
    lengths uniform in [512, 4096]); 'llama70b_decode_bf16' / '_fp8' / '_int4'
    (8 x 32,768 tokens, 64 q / 8 kv heads, outliers); 'long_mha_decode' (one
    128,000-token sequence, 32 / 32 heads, fp16).
    """
    if name == "llama8b_decode":
        return DecodeWorkload(name, 40 if not small else 6, 32, 8, 128, "bf16",
                              (512, 4096) if not small else (1, 300), seed=seed)
    if name in ("llama70b_decode_bf16", "llama70b_decode_fp8", "llama70b_decode_int4"):
        dt = name.rsplit("_", 1)[1]
        return DecodeWorkload("llama70b_decode", 8 if not small else 3, 64, 8, 128, dt,
                              32768 if not small else 531, outliers=True, seed=seed)
    if name == "long_mha_decode":
        return DecodeWorkload(name, 1, 32, 32, 128, "fp16",
                              128000 if not small else 2085, seed=seed)
    raise KeyError(name)


# ------------------------------------------------------------------ causal prefill
class PrefillWorkload:
    def __init__(self, tag, batch, T, n_q, n_kv, d, seed=0):
        self.tag, self.batch, self.T, self.n_q, self.n_kv, self.d = tag, batch, T, n_q, n_kv, d
        self.seed = seed

    def qkv(self):
        rng = _rng(self.seed, self.tag, 0)
        q = rng.standard_normal((self.batch, self.T, self.n_q, self.d), dtype=np.float32)
        k = rng.standard_normal((self.batch, self.T, self.n_kv, self.d), dtype=np.float32)
        v = rng.standard_normal((self.batch, self.T, self.n_kv, self.d), dtype=np.float32)
        return q, k, v


def prefill_workload(name="llama8b_prefill", small=False, seed=0):
    """4 sequences x 8,192 tokens, 32 q / 8 kv heads, d 128, bf16 (or shrunk)."""
    if small:
        return PrefillWorkload(name, 2, 333, 32, 8, 128, seed=seed)
    return PrefillWorkload(name, 4, 8192, 32, 8, 128, seed=seed)
