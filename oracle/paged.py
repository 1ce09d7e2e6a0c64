"""Host model of the paged KV cache, byte for byte (test infrastructure only).

Allocation follows the paged-cache data structure of [KVFA] (PagedAttention
section): HBM is cut into fixed blocks of 16 token rows; each sequence owns a
page table listing its blocks in logical order; a new block is taken from the
free list only when the sequence's length is a multiple of 16 before the new
token, i.e. when its last block is full; releasing a sequence puts all of its
blocks back on the free list; the physical place of logical position p is
(table[p // 16], p % 16).  [KPF] ("Paged attention: stop reserving empty
tables") describes the same block table.  The free list is the page's plain
Python list: initially 0 .. n_blocks-1, ``pop()`` takes from the end and a
release appends the sequence's blocks in table order.

Prefix sharing follows [KVFA] ``share_prefix`` (a second sequence's table
starts with the first ceil(prefix_len/16) blocks of the first) with the rule
[KVFA] and [KPF] state in prose: sequences with a common beginning point at
the same blocks and a block is copied only when one of them would change it.
Each block counts the sequences holding it; a release frees only blocks no
one holds any more (appended in table order); a grow whose new row lands in a
partly filled last block held by another sequence first moves the growing
sequence to a fresh copy of that block (taken from the free list like any
other block, all layers copied).

Physical layout of one layer's pools (the library's documented layout):
  K[block][kv_head][slot 0..15][d]      (a token's d values contiguous)
  V[block][kv_head][d][slot 0..15]      (a d-column's 16 tokens contiguous)
  Kscale, Vscale[block][kv_head]        float32, fp8 and int4 caches only
An int4 cache holds its codes here unpacked (int8, -7..7); the library stores
them two per byte along the last axis (K rows: d/2 bytes, V columns: 8 bytes
of 16 tokens), which ``codecs.int4_pack`` reproduces.
Stored elements are raw storage-format bit patterns.  Unwritten slots keep
whatever was there (tests fill the pools with a poison pattern first), and
this model keeps the same poison so whole pools can be compared.
"""
import numpy as np

from .codecs import (bf16_bits_to_f64, e4m3_decode, f16_bits_to_f64,
                     fp8_slab_write, int4_slab_write)

BLOCK = 16
STORAGE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
           "int4": np.int8}
POISON = {"f32": 0xFFFFFFFF, "f16": 0xFFFF, "bf16": 0xFFFF, "fp8": 0xFF,
          "int4": -1}                                 # 0xF nibbles
SCALED = ("fp8", "int4")


class PagedCacheModel:
    def __init__(self, n_layers, n_kv, d, dtype, n_blocks, max_seqs, max_blocks_per_seq,
                 poison=True):
        assert dtype in STORAGE
        self.n_layers, self.n_kv, self.d, self.dtype = n_layers, n_kv, d, dtype
        self.n_blocks, self.max_seqs, self.max_bps = n_blocks, max_seqs, max_blocks_per_seq
        st = STORAGE[dtype]
        fill = POISON[dtype] if poison else 0
        self.K = np.full((n_layers, n_blocks, n_kv, BLOCK, d), fill, dtype=st)
        self.V = np.full((n_layers, n_blocks, n_kv, d, BLOCK), fill, dtype=st)
        if dtype in SCALED:
            nanbits = np.uint32(0xFFFFFFFF) if poison else np.uint32(0)
            self.Ks = np.full((n_layers, n_blocks, n_kv), nanbits, dtype=np.uint32).view(np.float32)
            self.Vs = np.full((n_layers, n_blocks, n_kv), nanbits, dtype=np.uint32).view(np.float32)
        self.free = list(range(n_blocks))
        self.refs = [0] * n_blocks
        self.table = {}
        self.length = {}

    # ------------------------------------------------------------ allocation
    def _take(self):
        b = self.free.pop()
        self.refs[b] = 1
        return b

    def alloc(self, seq, n_tokens):
        """Make seq live with n_tokens rows: as many blocks as it takes to
        hold them, i.e. the least count c with 16 c >= n_tokens."""
        count = (n_tokens + BLOCK - 1) // BLOCK
        if count > len(self.free):
            raise MemoryError("no free blocks")
        blocks = []
        while len(blocks) < count:
            blocks.append(self._take())
        self.table[seq] = blocks
        self.length[seq] = n_tokens

    def _shared_partial(self, s):
        return self.length[s] % BLOCK != 0 and self.refs[self.table[s][-1]] > 1

    def _copy_block(self, src, dst):
        self.K[:, dst] = self.K[:, src]
        self.V[:, dst] = self.V[:, src]
        if self.dtype in SCALED:
            self.Ks[:, dst] = self.Ks[:, src]
            self.Vs[:, dst] = self.Vs[:, src]

    def grow(self, seqs):
        need = sum(1 for s in seqs if self.length[s] % BLOCK == 0 or self._shared_partial(s))
        if need > len(self.free):
            raise MemoryError("no free blocks")
        for s in seqs:
            if self.length[s] % BLOCK == 0:
                self.table[s].append(self._take())
            elif self._shared_partial(s):               # copy before writing
                old = self.table[s][-1]
                new = self._take()
                self._copy_block(old, new)
                self.refs[old] -= 1
                self.table[s][-1] = new
            self.length[s] += 1

    def grow_by(self, seq, n):
        """n single-token grows of one sequence (a prompt chunk)."""
        need = -(-(self.length[seq] + n) // BLOCK) - -(-self.length[seq] // BLOCK)
        need += 1 if n > 0 and self._shared_partial(seq) else 0
        if need > len(self.free):
            raise MemoryError("no free blocks")
        for _ in range(n):
            self.grow([seq])

    def share_prefix(self, src, dst, prefix_len):
        """dst holds the first prefix_len rows of src through the same blocks:
        its table lists the blocks of src that hold positions 0 .. prefix_len-1,
        and each of them gains one holder."""
        assert dst not in self.table and 0 <= prefix_len <= self.length[src]
        held = [self.physical(src, p)[0] for p in range(0, prefix_len, BLOCK)]
        for b in held:
            self.refs[b] += 1
        self.table[dst] = held
        self.length[dst] = prefix_len

    def release(self, seq):
        for b in self.table.pop(seq):
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.free.append(b)
        del self.length[seq]

    def set_table(self, seq, blocks, length):
        """Install an explicit block list (tests use shuffled tables)."""
        blocks = [int(b) for b in blocks]
        assert len(blocks) == -(-length // BLOCK)
        for b in blocks:
            self.free.remove(b)
            self.refs[b] = 1
        self.table[seq] = blocks
        self.length[seq] = length

    def physical(self, seq, pos):
        return self.table[seq][pos // BLOCK], pos % BLOCK

    # ---------------------------------------------------------------- writes
    def write_rows(self, layer, seq, start, k_rows, v_rows):
        """Store rows for positions start .. start+T-1 of one sequence.

        k_rows, v_rows: [T, n_kv, d].  For 16/32-bit caches they are the
        storage bit patterns (uint16 / uint32) and are copied bit for bit; for
        an fp8 or int4 cache they are float32 values (bf16 inputs widened
        exactly) and go through that format's per-slab scale rule, one slab
        write per (block, head) covering all of the new rows that land in that
        block.
        """
        T = k_rows.shape[0]
        assert start + T <= self.length[seq]
        if self.dtype not in SCALED:
            st = STORAGE[self.dtype]
            for i in range(T):
                b, r = self.physical(seq, start + i)
                self.K[layer, b, :, r, :] = np.asarray(k_rows[i]).view(st)
                self.V[layer, b, :, :, r] = np.asarray(v_rows[i]).view(st)
            return
        slab_write = fp8_slab_write if self.dtype == "fp8" else int4_slab_write
        p = start
        while p < start + T:
            b, r0 = self.physical(seq, p)
            n = min(BLOCK - r0, start + T - p)
            i0 = p - start
            for h in range(self.n_kv):
                kc, ks = slab_write(self.K[layer, b, h], self.Ks[layer, b, h], r0,
                                        k_rows[i0:i0 + n, h, :])
                self.K[layer, b, h] = kc
                self.Ks[layer, b, h] = ks
                vc, vs = slab_write(self.V[layer, b, h].T, self.Vs[layer, b, h], r0,
                                        v_rows[i0:i0 + n, h, :])
                self.V[layer, b, h] = vc.T
                self.Vs[layer, b, h] = vs
            p += n

    # ----------------------------------------------------------------- reads
    def _widen(self, raw):
        if self.dtype == "f32":
            return raw.view(np.float32).astype(np.float64)
        if self.dtype == "f16":
            return f16_bits_to_f64(raw)
        if self.dtype == "bf16":
            return bf16_bits_to_f64(raw)
        if self.dtype == "int4":
            return raw.astype(np.float64)
        return e4m3_decode(raw)

    def logical_raw(self, layer, seq, start=0, count=None):
        """Stored bit patterns of rows start..start+count-1: K, V [count, n_kv, d]."""
        L = self.length[seq]
        count = L - start if count is None else count
        Kr = np.empty((count, self.n_kv, self.d), dtype=self.K.dtype)
        Vr = np.empty((count, self.n_kv, self.d), dtype=self.V.dtype)
        for i in range(count):
            b, r = self.physical(seq, start + i)
            Kr[i] = self.K[layer, b, :, r, :]
            Vr[i] = self.V[layer, b, :, :, r]
        return Kr, Vr

    def packed_pools(self, layer=None):
        """int4: the K and V pools as the library stores them, two codes per byte."""
        from .codecs import int4_pack
        assert self.dtype == "int4"
        K = self.K if layer is None else self.K[layer]
        V = self.V if layer is None else self.V[layer]
        return int4_pack(K, axis=-1), int4_pack(V, axis=-1)

    def logical_values(self, layer, seq):
        """Dequantised K, V of the whole sequence as exact float64 [L, n_kv, d]."""
        L = self.length[seq]
        Kr, Vr = self.logical_raw(layer, seq)
        K, V = self._widen(Kr), self._widen(Vr)
        if self.dtype in SCALED:
            for i in range(L):
                b, _ = self.physical(seq, i)
                K[i] *= self.Ks[layer, b, :].astype(np.float64)[:, None]
                V[i] *= self.Vs[layer, b, :].astype(np.float64)[:, None]
        return K, V
