/*
 * kvfa -- paged KV cache and exact causal softmax attention for AMD MI355X
 * (gfx950).  C ABI.
 *
 * What is computed.  Decoder attention against a growing key/value cache:
 * each layer keeps one K row and one V row per kv head for every token seen
 * so far, a new token appends its own rows, and its query then attends over
 * all rows of its sequence ("KV Cache & Flash Attention." (kvcache-7e2),
 * KV cache section; "KV Cache & FlashAttention" (deepforge), first section;
 * "KV cache, paged, flash and sparse attention" (abhishekpatel), "Following
 * one new token through the cache").  The attention is the exact
 * softmax(q K^T * scale) V with a causal mask, evaluated tile by tile with the
 * online softmax (running max m, running sum l, rescale by exp(m_old-m_new))
 * so the score matrix never reaches device memory (kvcache-7e2, Flash
 * Attention and online softmax sections).  Query head h reads kv head
 * h / (n_q_heads / n_kv_heads) (grouped-query attention, kvcache-7e2
 * memory-cost section).
 *
 * Paged storage (kvcache-7e2, PagedAttention section; abhishekpatel, "Paged
 * attention: stop reserving empty tables").  Each layer's K and V live in
 * pools of fixed 16-token blocks; every sequence has a block table listing
 * its blocks in logical order, so logical position p lives in block
 * table[p / 16], slot p % 16.  Blocks come from a free list and go back to
 * it when a sequence is released.  Physical layout of the caller-owned pools
 * (elements of the storage type, row-major, innermost last):
 *
 *   k_pool  [n_layers][n_blocks][n_kv_heads][16][d_head]
 *   v_pool  [n_layers][n_blocks][n_kv_heads][d_head][16]   (slot innermost)
 *   k_scale, v_scale [n_layers][n_blocks][n_kv_heads]  float, fp8 and int4 only
 *   block_table [max_seqs][max_blocks_per_seq]  int32, -1 where unused
 *   seq_len     [max_seqs]                       int32 tokens stored
 *
 * Storage types.  f32, f16, bf16: K/V rows are stored bit for bit.  fp8: the
 * OCP E4M3FN format (max 448, round to nearest even, saturating), one float
 * scale per (layer, block, kv head) for K and one for V, equal to
 * absmax/448 over the rows written so far to that block (0 for an all-zero
 * block); a code holds round(x / scale); when a new row raises the absmax of
 * a partly filled block, the rows already there are re-encoded as
 * encode(fl(decode(code) * s_old) / s_new), all in IEEE float32.  Queries and
 * outputs use the storage type, except that an fp8 cache takes bf16 queries,
 * keys, values and outputs ("io type").
 *
 * int4 (kvcache-7e2 names an int4 cache in its memory-cost section and
 * fixes nothing else, so the format below is this library's): codes are
 * signed integers -7 .. 7 (two's complement nibbles; -8 is never written),
 * two per byte with the element of even index in the low nibble, so a K
 * slab is [16][d_head / 2] bytes and a V slab [d_head][8] bytes (tokens 2i
 * and 2i+1 of a column share byte i).  Scales follow the fp8 rule with 7 in
 * place of 448: absmax/7 per (layer, block, kv head), a code holds
 * rint(x / scale) (ties to even) clamped to +-7, and a growing absmax
 * re-encodes the block's earlier rows as encode(fl(code * s_old) / s_new).
 * The io type is bf16.
 *
 * Conventions.  Every function returns KVC_OK (0) or a negative status and
 * never throws; kvc_last_error() gives a message for the calling thread.
 * The caller owns all device memory (pools, tables, inputs, outputs,
 * workspace) and all streams it passes; a handle owns host metadata and,
 * when it has device buffers, one internal stream and two events (made by
 * kvc_create, released by kvc_destroy) on which kvc_attn_prefill runs its
 * cache write beside the attention kernel.  Pointers
 * named *_dev are device pointers, *_host host pointers.  Work is enqueued
 * asynchronously on the given stream (0 = the default stream); argument
 * errors are detected before anything is enqueued, launch failures give
 * KVC_E_HIP, and faults inside kernels surface at the caller's next
 * synchronisation.  A handle is not thread-safe.  Sequence ids passed in
 * device arrays are checked by the kernels themselves: an id outside
 * [0, max_seqs), a length of zero or beyond the table, or a block id outside
 * the pool makes the kernel skip that entry (attention rows come back NaN,
 * cache writes are not made); the kernels never read or write outside the
 * buffers they are given.
 */
#ifndef KVFA_H
#define KVFA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define KVC_OK             0
#define KVC_E_INVAL       -1  /* null or out-of-range argument                         */
#define KVC_E_UNSUPPORTED -2  /* d_head not 64/128, n_q % n_kv != 0, block != 16, ...  */
#define KVC_E_NO_BLOCKS   -3  /* free list too short; nothing was changed               */
#define KVC_E_STATE       -4  /* unknown/released/live sequence, host-only handle, ...  */
#define KVC_E_WORKSPACE   -5  /* workspace smaller than kvc_decode_workspace_bytes      */
#define KVC_E_HIP         -6  /* a HIP launch or runtime call failed                    */

typedef enum kvc_dtype {
  KVC_F32 = 0,
  KVC_F16 = 1,
  KVC_BF16 = 2,
  KVC_FP8_E4M3FN = 3,
  KVC_INT4 = 4
} kvc_dtype;

typedef struct kvc_config {
  int32_t n_layers;           /* >= 1                                              */
  int32_t n_q_heads;          /* multiple of n_kv_heads                            */
  int32_t n_kv_heads;         /* >= 1 (1 = multi-query attention)                  */
  int32_t d_head;             /* 64 or 128                                         */
  int32_t block_size;         /* tokens per block; must be 16                      */
  int32_t n_blocks;           /* blocks per layer pool                             */
  int32_t max_seqs;           /* sequence ids are 0 .. max_seqs-1                  */
  int32_t max_blocks_per_seq; /* table width; a sequence holds <= 16x this tokens  */
  int32_t kv_dtype;           /* a kvc_dtype                                       */
} kvc_config;

typedef struct kvc_sizes {    /* bytes the caller must allocate on the device      */
  uint64_t k_pool, v_pool, k_scale, v_scale, block_table, seq_len;
} kvc_sizes;

typedef struct kvc_buffers {  /* caller-owned device buffers, sized by kvc_sizes   */
  void* k_pool;
  void* v_pool;
  float* k_scale;             /* NULL unless kv_dtype is fp8 or int4               */
  float* v_scale;
  int32_t* block_table;
  int32_t* seq_len;
} kvc_buffers;

typedef struct kvc_cache kvc_cache;

/* Cache bytes per token over all layers: 2 (K and V) x n_layers x n_kv_heads
 * x d_head x element bytes (kvcache-7e2 memory-cost section; deepforge
 * cache-size formula; abhishekpatel "Opening the hood").  fp8 counts one
 * byte per element, int4 half a byte; the per-block scales are not
 * included. */
int kvc_bytes_per_token(const kvc_config* cfg, uint64_t* out);

/* Device bytes for every buffer of a cache with this configuration. */
int kvc_required_sizes(const kvc_config* cfg, kvc_sizes* out);

/* Create a cache handle over caller-allocated device buffers (kv_cache_create).
 * All n_blocks blocks start on the free list, which is the list 0..n_blocks-1
 * used as a stack (kvcache-7e2 PagedAttention section).  Enqueues on `stream`
 * a fill of block_table with -1 and seq_len with 0.  dev == NULL creates a
 * host-only handle: the allocator works, and every call that needs the device
 * returns KVC_E_STATE. */
int kvc_create(const kvc_config* cfg, const kvc_buffers* dev, hipStream_t stream,
               kvc_cache** out);
int kvc_destroy(kvc_cache* cache);

/* Make `seq` live with n_tokens tokens: ceil(n_tokens / 16) blocks popped from
 * the free list (kvcache-7e2, PagedAttention section: `allocate` takes
 * ceil(n / 16) blocks for a new sequence).  The rows themselves are written later
 * (kvc_write, kvc_attn_prefill).  KVC_E_STATE if seq is already live,
 * KVC_E_NO_BLOCKS if the free list is too short (state unchanged). */
int kvc_seq_alloc(kvc_cache* cache, int32_t seq, int32_t n_tokens, hipStream_t stream);

/* Grow each of n live sequences by one token (kvcache-7e2, PagedAttention
 * section: `append_token` takes a new block only when the sequence's length
 * is a multiple of 16, i.e. its last block is full): a sequence whose length
 * is a multiple of 16 first takes one block from the free list.  Ids must be distinct.  All-or-nothing: KVC_E_NO_BLOCKS leaves
 * every sequence as it was.  The device copy of the table and lengths is
 * updated on `stream`. */
int kvc_seq_grow(kvc_cache* cache, int32_t n, const int32_t* seqs_host, hipStream_t stream);

/* Grow one live sequence by n_tokens at once (a prompt chunk): the same
 * blocks, in the same order, as n_tokens single-token grows of that sequence
 * (kvcache-7e2 PagedAttention: a block is taken when a token starts one).
 * All or nothing: KVC_E_NO_BLOCKS or KVC_E_INVAL leave the state unchanged. */
int kvc_seq_grow_by(kvc_cache* cache, int32_t seq, int32_t n_tokens, hipStream_t stream);

/* Return all blocks of `seq` to the free list, in table order (kvcache-7e2,
 * PagedAttention section: `release` hands every block of a finished sequence
 * back), and mark it not live (device length 0, table entries -1). */
int kvc_seq_release(kvc_cache* cache, int32_t seq, hipStream_t stream);

/* Prefix sharing (kvcache-7e2, PagedAttention section, `share_prefix`;
 * abhishekpatel, "Paged attention: stop reserving empty tables": sequences
 * that start alike refer to the same physical blocks, and a block is
 * duplicated only when a write would alter it).
 * `dst` (not live) becomes live holding the first prefix_len rows of `src`
 * (live, 0 <= prefix_len <= len(src)) by sharing its first
 * ceil(prefix_len/16) blocks; no data moves.  Every block counts the
 * sequences holding it: kvc_seq_release returns a block to the free list
 * only when the last holder releases it.  Copy-on-write: when a grow would
 * put new rows into a partly filled last block that another sequence also
 * holds, the growing sequence first gets its own copy of that block (one
 * free block, all layers, K, V and fp8 scales, copied on the stream before
 * the grow's table update).  Rows below a sequence's length at its last
 * grow must not be rewritten while their block is shared. */
int kvc_seq_share_prefix(kvc_cache* cache, int32_t src, int32_t dst, int32_t prefix_len,
                         hipStream_t stream);

/* Number of sequences holding `block` (0 = free). */
int kvc_block_refs(const kvc_cache* cache, int32_t block, int32_t* out);

/* Make `seq` live with an explicit block list (each block must be free) and
 * length `len` (nblk must equal ceil(len/16)).  For tests and callers that
 * manage placement themselves. */
int kvc_set_block_table(kvc_cache* cache, int32_t seq, const int32_t* blocks_host,
                        int32_t nblk, int32_t len, hipStream_t stream);

/* Host-side queries of the handle's own state. */
int kvc_seq_len(const kvc_cache* cache, int32_t seq, int32_t* out);
int kvc_seq_blocks(const kvc_cache* cache, int32_t seq, int32_t* blocks_host, int32_t cap,
                   int32_t* n_out);
int kvc_free_blocks(const kvc_cache* cache, int32_t* out);

/* kv_append: store the newest token's K and V rows of one layer for each of n
 * sequences, at position seq_len[seq] - 1 (call kvc_seq_grow first).  Each
 * decoded token adds exactly one K row and one V row per layer to its
 * sequence's cache before its query attends (kvcache-7e2, KV cache section;
 * deepforge, first section; abhishekpatel, "Following one new token through
 * the cache").  The row lands in slot (len-1) % 16 of block
 * table[(len-1) / 16] (kvcache-7e2, PagedAttention section, `physical`).
 * k_dev, v_dev: [n][n_kv_heads][d_head] in the io type.  16/32-bit caches
 * store the bits unchanged; fp8 and int4 caches apply their scale rule. */
int kvc_append(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
               const void* k_dev, const void* v_dev, hipStream_t stream);

/* kvc_seq_grow followed by kvc_append of the grown rows of one layer, in one
 * launch (the same two steps of a decoded token: the block manager places
 * the new position, kvcache-7e2 PagedAttention section, `append_token`; its
 * K and V rows are stored there, KV cache section).  The host's block
 * manager already knows where each new row goes, so the launch carries each
 * entry's block and slot along with the grow's table and length writes, and
 * the kernel reads no table or length.  seqs_host: n distinct live sequence
 * ids; k_dev, v_dev: [n][n_kv_heads][d_head] in the io type, row i for
 * seqs_host[i].  The resulting pools, tables and lengths equal those of
 * kvc_seq_grow then kvc_append.  Checks as kvc_seq_grow (all-or-nothing:
 * nothing changes on an error it reports), plus the layer range and
 * non-NULL k_dev, v_dev.  Copy-on-write block copies run first, as in
 * kvc_seq_grow.  Batches above 96 entries take one launch per 96. */
int kvc_seq_grow_append(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_host,
                        const void* k_dev, const void* v_dev, hipStream_t stream);

/* Bulk store of T consecutive rows per sequence (prefill, population):
 * positions start .. start+T-1 of each of n sequences, which must all lie
 * below the sequence's length.  k_dev, v_dev: [n][T][n_kv_heads][d_head] in
 * the io type.  For fp8 and int4 each (block, kv head) is written once with
 * all of its new rows (the scale rule applied to the rows together). */
int kvc_write(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
              int32_t start, int32_t T, const void* k_dev, const void* v_dev,
              hipStream_t stream);

/* attn_prefill: causal attention of whole prompts, query t seeing keys
 * 0..t, computed tile by tile with the online softmax (kvcache-7e2 Flash
 * Attention section; deepforge: a prompt is processed all at once and the
 * score table never leaves on-chip memory).  q_dev [n][T][n_q_heads][d_head],
 * k_dev, v_dev [n][T][n_kv_heads][d_head], out_dev [n][T][n_q_heads][d_head],
 * all in the io type.  When seqs_dev is not NULL the prompt's K/V rows are
 * also stored as positions 0..T-1 of those sequences (as kvc_write with
 * start 0; each sequence needs length >= T), by a write that runs on the
 * handle's internal stream beside the attention kernel and is joined back
 * into `stream` before the call returns (later work on `stream` sees the
 * rows).  seqs_dev == NULL: attention only.  scale is the score multiplier (1/sqrt(d_head) in the pages); it
 * must be finite and > 0 (KVC_E_INVAL otherwise): the kernels take each row
 * maximum on unscaled scores. */
int kvc_attn_prefill(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                     int32_t T, const void* q_dev, const void* k_dev, const void* v_dev,
                     void* out_dev, float scale, hipStream_t stream);

/* attn_extend: T new query rows per sequence against everything the cache
 * holds for it, the new rows' own K/V included (written before the call,
 * e.g. by kvc_write at start = len - T).  Query t of sequence s sits at
 * position len(s) - T + t and sees cached rows 0 .. len(s) - T + t: one chunk
 * of a prompt processed against the chunks before it (kvcache-7e2
 * continuous-batching section: chunked prefill; abhishekpatel.co: long
 * prefills split into chunks), or the target's pass over T drafted tokens
 * (kvcache-7e2 speculative-decoding section).  q_dev, out_dev:
 * [n][T][n_q_heads][d_head] in the io type, 16-byte aligned.  bf16, f16,
 * fp8 and int4 caches (KVC_E_UNSUPPORTED for f32).  For fp8 and int4 the
 * stored codes are used exactly (every E4M3FN value and every int4 code is
 * a bf16 value); each block's K scale multiplies the scores of that block's
 * keys, its V scale multiplies their probabilities before they are rounded
 * to bf16 for the PV product, and the row sum adds the unscaled
 * probabilities in fp32.  scale finite and > 0.
 * A device
 * entry that is out of range, has len < T, or whose table holds an invalid
 * block id among its first ceil(len/16) entries gets NaN rows.  No
 * workspace. */
int kvc_attn_extend(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                    int32_t T, const void* q_dev, void* out_dev, float scale,
                    hipStream_t stream);

/* Workspace bytes kvc_attn_decode needs for a batch of n sequences with this
 * num_splits (0 = automatic), given the longest live sequence of the cache
 * at the time of the call.  0 when the plan needs no workspace. */
int kvc_decode_workspace_bytes(const kvc_cache* cache, int32_t n, int32_t num_splits,
                               uint64_t* out);

/* attn_decode: one query row per sequence against all of its cached rows
 * (every row visible: the newest token's own row was appended first), the
 * step the cache exists for: the new token's query against the stored K and
 * V instead of recomputing them (kvcache-7e2, naive decoding and KV cache
 * sections; abhishekpatel, "Following one new token through the cache").
 * The rows are read through the block table (kvcache-7e2, PagedAttention
 * section: the kernel gathers K and V from the physical blocks when it
 * attends), once per group of query heads sharing a kv head; the pass is
 * bound by how fast the cache can be read (deepforge: decoding is
 * memory-bound).
 * q_dev, out_dev: [n][n_q_heads][d_head] in the io type.  Long contexts are
 * cut into splits swept in parallel, each keeping its own (m, l, O), and
 * merged afterwards with weights exp(m_s - max m) -- the online softmax's
 * rescale applied across splits.  num_splits: 0 = automatic, else the
 * number of splits of the longest sequence.  ws_dev: caller-owned workspace
 * of at least kvc_decode_workspace_bytes bytes (may be NULL if that is 0).
 * scale: finite and > 0, as for kvc_attn_prefill. */
int kvc_attn_decode(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                    const void* q_dev, void* out_dev, float scale, int32_t num_splits,
                    void* ws_dev, uint64_t ws_bytes, hipStream_t stream);

/* Sliding-window / attention-sink variants of the three attention calls
 * (abhishekpatel.co "Sparse attention": each token sees only the previous w
 * tokens; kvcache-7e2 eviction paragraph: a sliding window drops the oldest
 * tokens, attention sinks always keep the first few).  With window > 0 the
 * query at position p sees key j iff p - window < j <= p or j < sinks;
 * window = 0 is full causal attention (sinks then change nothing).  Same
 * arguments, layouts and errors as the calls above; window, sinks >= 0
 * (KVC_E_INVAL otherwise); f32 caches have no windowed kernel
 * (KVC_E_UNSUPPORTED when window > 0).  The decode reads only the blocks a
 * query can see, so its cost follows min(len, window + sinks). */
int kvc_attn_prefill_window(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                            int32_t T, const void* q_dev, const void* k_dev, const void* v_dev,
                            void* out_dev, float scale, int32_t window, int32_t sinks,
                            hipStream_t stream);
int kvc_attn_decode_window(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                           const void* q_dev, void* out_dev, float scale, int32_t window,
                           int32_t sinks, int32_t num_splits, void* ws_dev, uint64_t ws_bytes,
                           hipStream_t stream);
int kvc_attn_extend_window(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                           int32_t T, const void* q_dev, void* out_dev, float scale,
                           int32_t window, int32_t sinks, hipStream_t stream);

/* kv_append followed by attn_decode in one call (kvcache-7e2 KV cache
 * section: the new token's K and V rows join the cache, then its query
 * attends over every row of its sequence).  Same contract as kvc_append
 * (call kvc_seq_grow first; k_new_dev, v_new_dev [n][n_kv_heads][d_head] in
 * the io type, 16-byte aligned) and as kvc_attn_decode_window (window = 0:
 * full attention).  Outputs and cache contents equal those of kvc_append
 * then kvc_attn_decode_window: the call enqueues the append kernel, then the
 * decode, on the same stream.  The workspace is sized by
 * kvc_decode_workspace_bytes as for kvc_attn_decode. */
int kvc_attn_decode_append(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                           const void* k_new_dev, const void* v_new_dev, const void* q_dev,
                           void* out_dev, float scale, int32_t window, int32_t sinks,
                           int32_t num_splits, void* ws_dev, uint64_t ws_bytes,
                           hipStream_t stream);

/* kvc_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory around the call (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments,
 * layouts, results and errors as kvc_attn_decode with window 0, except that
 * the split partials live in a fixed 64 MiB array in device memory owned by
 * the library: each device it runs on holds one such array from the first
 * kvc_create on that device until the process ends.  The call allocates
 * nothing.  A call whose plan needs more than 64 MiB (the bytes
 * kvc_decode_workspace_bytes reports; about 8,000 (sequence, kv-head group)
 * segments plus the chip's waves at d_head 128) returns KVC_E_WORKSPACE and
 * enqueues nothing.  Every call on one device shares that device's array and
 * nothing in it needs clearing (each call writes every entry it reads before
 * reading it), so calls that may overlap on one device -- on different
 * streams, or from different threads -- race and must be serialised by the
 * caller; calls ordered on one stream are safe. */
int kvc_attn_decode_noalloc(kvc_cache* cache, int32_t layer, int32_t n, const int32_t* seqs_dev,
                            const void* q_dev, void* out_dev, float scale, int32_t num_splits,
                            hipStream_t stream);

/* Block-table gather (kvcache-7e2, PagedAttention section: `physical` maps
 * a logical position p to (table[p / 16], p % 16), and attention gathers K
 * and V from those physical blocks): copy the stored bit patterns of
 * positions start .. start+count-1 of `seq` in logical order into
 * k_out_dev, v_out_dev, each
 * [count][n_kv_heads][d_head] of the storage type (fp8: raw codes; int4:
 * [count][n_kv_heads][d_head / 2] bytes, codes packed along d_head as in
 * the pools' K rows, for V as well). */
int kvc_gather(const kvc_cache* cache, int32_t layer, int32_t seq, int32_t start, int32_t count,
               void* k_out_dev, void* v_out_dev, hipStream_t stream);

/* Scopes of kvc_set_dispatch_events. */
enum {
  KVC_TIME_CALL = 0,          /* first kernel's start to last kernel's end */
  KVC_TIME_MAIN_KERNEL = 1    /* the call's main kernel only */
};

/* Timing hook, for callers that measure the kernels against their roofline
 * (a profiler-free benchmark, a serving loop's own telemetry); no page
 * defines it.  It times a call's kernels without stream-marker overhead.
 * The next attention call on this cache (kvc_attn_decode,
 * _window, _append, _noalloc, kvc_attn_prefill, _window, kvc_attn_extend,
 * _window) attaches start_event and stop_event to kernel dispatches of its
 * own (hipExtLaunchKernel records them as those kernels begin and end):
 *   KVC_TIME_CALL: start at the call's first kernel, stop at its last;
 *   KVC_TIME_MAIN_KERNEL: both at the call's main kernel, the one that reads
 *     the cache or the prompt (decode: the work-list kernel, or the split
 *     kernel of an f32 cache, from its first to its last launch when a large
 *     batch runs in sub-batches; the merge and the append kernel stay
 *     outside).
 * Prefill and extend time their attention kernel in both scopes (a prompt's
 * cache write runs beside it on the handle's side stream, outside the
 * events).  Both handles are hipEvent_t created by the caller with timing
 * enabled on the cache's device; either may be NULL; the caller keeps
 * ownership.  The events are used by that one call, whether it launches or
 * fails, and then forgotten; two NULLs clear them.  A call that launches
 * nothing (n = 0 or T = 0) records neither.  KVC_E_INVAL for a NULL cache or
 * an unknown scope (which also clears them). */
int kvc_set_dispatch_events(kvc_cache* cache, void* start_event, void* stop_event,
                            int32_t scope);

/* Message describing the last failure on the calling thread ("" if none). */
const char* kvc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVFA_H */
