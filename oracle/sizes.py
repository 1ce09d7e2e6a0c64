"""Closed forms the pages print (test infrastructure only).

* Bytes of K/V cache per token: two vectors (K and V) per layer per kv head,
  each d_head numbers of a given byte width ([DF] cache-size formula; [KPF]
  "Opening the hood: how big is the notebook?"; [KVFA] memory-cost section,
  whose gqa_kv_bytes also multiplies by tokens and batch).
* The MLA variant stores one latent of (kv_lora_rank + rope dim) numbers per
  layer per token ([KVFA] memory-cost section).  Size arithmetic only.
* Attention rows computed while emitting N tokens without a cache:
  1 + 2 + ... + N = N(N+1)/2 ([KVFA] naive decoding section); with a cache,
  one row per token.
"""


def kv_bytes_per_token(n_layers, n_kv_heads, d_head, bytes_per_elem):
    return 2 * n_layers * n_kv_heads * d_head * bytes_per_elem


def gqa_kv_bytes(n_tokens, n_layers, n_kv_heads, d_head, dtype_b=2, batch=1):
    return batch * n_tokens * kv_bytes_per_token(n_layers, n_kv_heads, d_head, dtype_b)


def mla_kv_bytes(n_tokens, n_layers, kv_lora_rank, qk_rope_dim, dtype_b=2, batch=1):
    return batch * n_tokens * n_layers * (kv_lora_rank + qk_rope_dim) * dtype_b


def naive_attention_rows(n):
    """Rows computed when every step recomputes the whole prefix: sum 1..n."""
    return n * (n + 1) // 2


def naive_prefix_rows(prompt_len, n_new):
    """Token passes without a cache: prompt_len + (prompt_len+1) + ... over n_new steps."""
    return sum(prompt_len + i for i in range(n_new))


def cached_prefix_rows(prompt_len, n_new):
    """Token passes with a cache: the prompt once, then each new token once."""
    return prompt_len + n_new
