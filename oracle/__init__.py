"""CPU oracle for paged-KV-cache causal attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may import,
call, link or execute anything in this package: only the tests,
``__graft_entry__.smoke()`` and the bench's CPU-baseline leg use it.  It shares
no code with the HIP library (no kernels, headers, helpers, tables or
constant generators) and imports nothing from it.

Everything here is plain and slow on purpose, written so that a reader can
check it against the three source pages by eye:

* ``attention``  -- the definition: materialised softmax(Q K^T * scale) V with a
  causal mask, in float64; the page's tiled flash loop and online softmax; the
  split-context (m, l) merge.
* ``codecs``     -- reference encoders/decoders for the storage formats
  (bf16, fp16, OCP fp8 e4m3fn) and the per-block fp8 scale rule.
* ``paged``      -- a host model of the paged cache (free list, block tables,
  16-token blocks) that replays every write byte for byte.
* ``sizes``      -- the closed forms the pages print (bytes per token,
  triangular operation counts).

Pages cited (by title and section):
  [KVFA]  "KV Cache & Flash Attention." (kvcache-7e2.pages.dev)
  [DF]    "KV Cache & FlashAttention" (deepforge.srivtx.xyz)
  [KPF]   "KV cache, paged, flash and sparse attention" (abhishekpatel.co)

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against a value the pages print, a closed form, an invariant, a library
routine or brute force; none is "parity unpinned".
"""
