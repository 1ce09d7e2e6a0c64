// C ABI and host-side cache manager.
//
// The manager keeps the authoritative host copy of the paged cache's
// metadata: a free list used as a stack (initially 0..n_blocks-1, blocks are
// popped from the end and released blocks are pushed back in table order),
// one block table per sequence and its length ("KV Cache & Flash Attention."
// (kvcache-7e2), PagedAttention section: fixed 16-token blocks, a per-sequence
// table, a new block only when the last one is full, release returns every
// block).  Sequences may share the blocks of a common prefix
// (kvcache-7e2 PagedAttention `share_prefix`); each block counts the
// sequences holding it, and a release returns only the blocks nobody holds
// any more.  A shared block is copied before a sequence writes into it
// ("KV cache, paged, flash and sparse attention" (abhishekpatel), "Paged
// attention: stop reserving empty tables": sharing stays safe because a block
// is duplicated only when a write would alter it): a grow whose new rows land
// in a shared, partly filled last block first gives the growing sequence its
// own copy.  Every change
// is mirrored to the caller's device tables by a small
// kernel whose arguments carry the changed entries, enqueued on the caller's
// stream, so attention kernels later on that stream see it.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvfa_internal.h"

using namespace kvfa;

struct kvc_cache {
  kvc_config cfg;
  bool has_dev = false;
  kvc_buffers dev{};
  std::vector<int32_t> free_list;               // stack: back() is popped first
  std::vector<std::vector<int32_t>> table;      // per sequence
  std::vector<int32_t> len;                     // per sequence
  std::vector<uint8_t> live;                    // per sequence
  std::vector<int32_t> refs;                    // per block: sequences holding it (0 = free)
  int32_t cu_count = 256;                       // compute units of the device (decode plan)
  // A prompt's cache write runs on `side`, beside the attention kernel on the
  // caller's stream: fork / join events order it after the caller's earlier
  // work and before its later work.  Created with the handle (not during a
  // call, which may be under graph capture).
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // Device address of the library-owned decode scratch on the device the
  // handle was created on (kvc_attn_decode_noalloc).
  void* scratch = nullptr;
  // Dispatch events for the next decode call (kvc_set_dispatch_events).
  DispatchEvents timing{};
  ~kvc_cache() {
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
    if (side) (void)hipStreamDestroy(side);
  }
  CacheView view() const {
    CacheView v{};
    v.k = dev.k_pool;
    v.v = dev.v_pool;
    v.ks = dev.k_scale;
    v.vs = dev.v_scale;
    v.bt = dev.block_table;
    v.len = dev.seq_len;
    v.n_layers = cfg.n_layers;
    v.n_q = cfg.n_q_heads;
    v.n_kv = cfg.n_kv_heads;
    v.d = cfg.d_head;
    v.n_blocks = cfg.n_blocks;
    v.max_seqs = cfg.max_seqs;
    v.max_bps = cfg.max_blocks_per_seq;
    v.dtype = cfg.kv_dtype;
    return v;
  }
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVC_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int check_config(const kvc_config* c) {
  if (!c) return fail(KVC_E_INVAL, "config is NULL");
  if (c->n_layers < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_blocks < 1 ||
      c->max_seqs < 1 || c->max_blocks_per_seq < 1)
    return fail(KVC_E_INVAL, "config counts must be positive");
  if (c->kv_dtype < KVC_F32 || c->kv_dtype > KVC_INT4)
    return fail(KVC_E_INVAL, "unknown kv_dtype");
  if (c->block_size != kBlock) return fail(KVC_E_UNSUPPORTED, "block_size must be 16");
  if (c->d_head != 64 && c->d_head != 128) return fail(KVC_E_UNSUPPORTED, "d_head must be 64 or 128");
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(KVC_E_UNSUPPORTED, "n_q_heads must be a multiple of n_kv_heads");
  if ((int64_t)c->max_blocks_per_seq * kBlock > INT32_MAX)
    return fail(KVC_E_UNSUPPORTED, "max_blocks_per_seq too large");
  return KVC_OK;
}

uint64_t pool_bytes(const kvc_config* c) {
  return (uint64_t)c->n_layers * c->n_blocks * c->n_kv_heads * slab_bytes(c->kv_dtype, c->d_head);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Collects (index, value) writes and flushes them in launches of at most
// kTableUpdateMax entries each -- or, with a sink, only collects them for a
// launch that carries them with other work.
struct Uploader {
  kvc_cache* c;
  hipStream_t s;
  TableUpdate u{};
  hipError_t err = hipSuccess;
  std::vector<std::pair<int32_t, int32_t>>* sink = nullptr;
  Uploader(kvc_cache* c_, hipStream_t s_) : c(c_), s(s_) {}
  void put(int32_t idx, int32_t val) {
    if (!c->has_dev) return;
    if (sink) {
      sink->emplace_back(idx, val);
      return;
    }
    u.idx[u.n] = idx;
    u.val[u.n] = val;
    if (++u.n == kTableUpdateMax) flush();
  }
  void bt(int32_t seq, int32_t i, int32_t blk) { put(seq * c->cfg.max_blocks_per_seq + i, blk); }
  void len(int32_t seq, int32_t l) { put(-seq - 1, l); }
  void flush() {
    if (u.n == 0) return;
    hipError_t e = launch_table_update(c->view(), u, s);
    if (e != hipSuccess && err == hipSuccess) err = e;
    u.n = 0;
  }
  int finish() {
    flush();
    return err == hipSuccess ? KVC_OK : hip_fail(err, "table update launch");
  }
};

// Collects copy-on-write block copies and launches them (before the table
// updates of the same call) in batches of at most kCopyMax pairs.
struct Copier {
  kvc_cache* c;
  hipStream_t s;
  BlockCopy u{};
  hipError_t err = hipSuccess;
  Copier(kvc_cache* c_, hipStream_t s_) : c(c_), s(s_) {}
  void put(int32_t src, int32_t dst) {
    if (!c->has_dev) return;
    u.src[u.n] = src;
    u.dst[u.n] = dst;
    if (++u.n == kCopyMax) flush();
  }
  void flush() {
    if (u.n == 0) return;
    hipError_t e = launch_copy_blocks(c->view(), u, s);
    if (e != hipSuccess && err == hipSuccess) err = e;
    u.n = 0;
  }
  int finish() {
    flush();
    return err == hipSuccess ? KVC_OK : hip_fail(err, "block copy launch");
  }
};

int32_t take_block(kvc_cache* c) {
  int32_t b = c->free_list.back();
  c->free_list.pop_back();
  c->refs[b] = 1;
  return b;
}

// Before new rows are written at position len of `seq`: if they land in a
// partly filled last block that another sequence also holds, give `seq` its
// own copy of that block.  Returns whether a copy was made.
bool unshare_last(kvc_cache* c, int32_t seq, Copier& cp, Uploader& up) {
  const int32_t len = c->len[seq];
  if (len % kBlock == 0) return false;                 // the next row starts a new block
  auto& t = c->table[seq];
  const int32_t old = t.back();
  if (c->refs[old] <= 1) return false;
  const int32_t nb = take_block(c);
  cp.put(old, nb);
  c->refs[old] -= 1;
  t.back() = nb;
  up.bt(seq, (int32_t)t.size() - 1, nb);
  return true;
}

bool needs_copy(const kvc_cache* c, int32_t seq) {
  return c->len[seq] % kBlock != 0 && c->refs[c->table[seq].back()] > 1;
}

int check_seq(const kvc_cache* c, int32_t seq) {
  if (seq < 0 || seq >= c->cfg.max_seqs) return fail(KVC_E_INVAL, "sequence id out of range");
  return KVC_OK;
}

int need_dev(const kvc_cache* c) {
  if (!c->has_dev) return fail(KVC_E_STATE, "host-only handle has no device buffers");
  return KVC_OK;
}

int32_t live_max_len(const kvc_cache* c) {
  int32_t m = 0;
  for (int32_t s = 0; s < c->cfg.max_seqs; ++s)
    if (c->live[s]) m = std::max(m, c->len[s]);
  return m;
}

}  // namespace

extern "C" {

const char* kvc_last_error(void) { return g_err.c_str(); }

int kvc_bytes_per_token(const kvc_config* cfg, uint64_t* out) {
  int r = check_config(cfg);
  if (r) return r;
  if (!out) return fail(KVC_E_INVAL, "out is NULL");
  *out = 2ull * cfg->n_layers * cfg->n_kv_heads * cfg->d_head * storage_bits(cfg->kv_dtype) / 8;
  return KVC_OK;
}

int kvc_required_sizes(const kvc_config* cfg, kvc_sizes* out) {
  int r = check_config(cfg);
  if (r) return r;
  if (!out) return fail(KVC_E_INVAL, "out is NULL");
  out->k_pool = out->v_pool = pool_bytes(cfg);
  uint64_t sc = (uint64_t)cfg->n_layers * cfg->n_blocks * cfg->n_kv_heads * sizeof(float);
  out->k_scale = out->v_scale = has_scales(cfg->kv_dtype) ? sc : 0;
  out->block_table = (uint64_t)cfg->max_seqs * cfg->max_blocks_per_seq * sizeof(int32_t);
  out->seq_len = (uint64_t)cfg->max_seqs * sizeof(int32_t);
  return KVC_OK;
}

int kvc_create(const kvc_config* cfg, const kvc_buffers* dev, hipStream_t stream,
               kvc_cache** out) {
  int r = check_config(cfg);
  if (r) return r;
  if (!out) return fail(KVC_E_INVAL, "out is NULL");
  if (dev) {
    if (!dev->k_pool || !dev->v_pool || !dev->block_table || !dev->seq_len)
      return fail(KVC_E_INVAL, "device buffer is NULL");
    if (has_scales(cfg->kv_dtype) && (!dev->k_scale || !dev->v_scale))
      return fail(KVC_E_INVAL, "fp8 and int4 caches need k_scale and v_scale");
    if (!aligned16(dev->k_pool) || !aligned16(dev->v_pool))
      return fail(KVC_E_INVAL, "pools must be 16-byte aligned");
  }
  kvc_cache* c = new (std::nothrow) kvc_cache();
  if (!c) return fail(KVC_E_INVAL, "out of host memory");
  c->cfg = *cfg;
  c->free_list.resize(cfg->n_blocks);
  for (int32_t i = 0; i < cfg->n_blocks; ++i) c->free_list[i] = i;
  c->table.resize(cfg->max_seqs);
  c->len.assign(cfg->max_seqs, 0);
  c->live.assign(cfg->max_seqs, 0);
  c->refs.assign(cfg->n_blocks, 0);
  if (dev) {
    c->has_dev = true;
    c->dev = *dev;
    int device = 0, cus = 0;
    if (hipGetDevice(&device) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess &&
        cus > 0)
      c->cu_count = cus;
    hipError_t e = scratch_address(&c->scratch);
    if (e != hipSuccess) {
      delete c;
      return hip_fail(e, "decode scratch address");
    }
    e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->join, hipEventDisableTiming);
    if (e != hipSuccess) {
      delete c;
      return hip_fail(e, "side stream / events");
    }
    e = launch_fill_tables(c->view(), stream);
    if (e != hipSuccess) {
      delete c;
      return hip_fail(e, "table fill launch");
    }
  }
  *out = c;
  return KVC_OK;
}

int kvc_destroy(kvc_cache* cache) {
  delete cache;
  return KVC_OK;
}

int kvc_seq_alloc(kvc_cache* c, int32_t seq, int32_t n_tokens, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = check_seq(c, seq);
  if (r) return r;
  if (c->live[seq]) return fail(KVC_E_STATE, "sequence is already live");
  if (n_tokens < 0) return fail(KVC_E_INVAL, "n_tokens < 0");
  int64_t nb = ((int64_t)n_tokens + kBlock - 1) / kBlock;
  if (nb > c->cfg.max_blocks_per_seq) return fail(KVC_E_INVAL, "n_tokens exceeds the table width");
  if (nb > (int64_t)c->free_list.size()) return fail(KVC_E_NO_BLOCKS, "free list exhausted");
  Uploader up(c, stream);
  auto& t = c->table[seq];
  t.clear();
  for (int64_t i = 0; i < nb; ++i) {
    int32_t b = take_block(c);
    t.push_back(b);
    up.bt(seq, (int32_t)i, b);
  }
  c->len[seq] = n_tokens;
  c->live[seq] = 1;
  up.len(seq, n_tokens);
  return up.finish();
}

namespace {
// Everything kvc_seq_grow checks before it changes any state.
int check_grow(const kvc_cache* c, int32_t n, const int32_t* seqs) {
  if (n < 0 || (n > 0 && !seqs)) return fail(KVC_E_INVAL, "bad sequence list");
  std::vector<uint8_t> seen(c->cfg.max_seqs, 0);
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    int r = check_seq(c, seqs[i]);
    if (r) return r;
    int32_t s = seqs[i];
    if (!c->live[s]) return fail(KVC_E_STATE, "sequence is not live");
    if (seen[s]) return fail(KVC_E_INVAL, "duplicate sequence id");
    seen[s] = 1;
    if ((int64_t)c->len[s] + 1 > (int64_t)c->cfg.max_blocks_per_seq * kBlock)
      return fail(KVC_E_INVAL, "sequence would exceed its table width");
    if (c->len[s] % kBlock == 0 || needs_copy(c, s)) ++need;
  }
  if (need > (int64_t)c->free_list.size()) return fail(KVC_E_NO_BLOCKS, "free list exhausted");
  return KVC_OK;
}

// One more row for sequence s: a fresh block when the row starts one, a
// private copy of a shared partly filled last block, then the length.
void grow_one(kvc_cache* c, int32_t s, Copier& cp, Uploader& up) {
  if (c->len[s] % kBlock == 0) {
    int32_t b = take_block(c);
    up.bt(s, (int32_t)c->table[s].size(), b);
    c->table[s].push_back(b);
  } else {
    unshare_last(c, s, cp, up);
  }
  c->len[s] += 1;
  up.len(s, c->len[s]);
}
}  // namespace

int kvc_seq_grow(kvc_cache* c, int32_t n, const int32_t* seqs, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = check_grow(c, n, seqs);
  if (r) return r;
  Copier cp(c, stream);
  Uploader up(c, stream);
  for (int32_t i = 0; i < n; ++i) grow_one(c, seqs[i], cp, up);
  int rc = cp.finish();
  int ru = up.finish();
  return rc ? rc : ru;
}

int kvc_seq_grow_append(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs,
                        const void* k, const void* v, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = need_dev(c);
  if (r) return r;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  r = check_grow(c, n, seqs);
  if (r) return r;
  if (n == 0) return KVC_OK;
  if (!k || !v) return fail(KVC_E_INVAL, "NULL device pointer");
  // Bookkeeping first, exactly as kvc_seq_grow; the table and length writes
  // are kept to ride with the appends.  Copy-on-write block copies are
  // launched before them, so the appended rows land on the copies.
  Copier cp(c, stream);
  Uploader up(c, stream);
  std::vector<std::pair<int32_t, int32_t>> writes;
  writes.reserve(2 * (size_t)n);
  up.sink = &writes;
  std::vector<int32_t> wend(n);                        // writes made up to entry i
  for (int32_t i = 0; i < n; ++i) {
    grow_one(c, seqs[i], cp, up);
    wend[i] = (int32_t)writes.size();
  }
  int rc = cp.finish();
  if (rc) return rc;
  hipError_t e = hipSuccess;
  const CacheView cv = c->view();
  for (int32_t i0 = 0; i0 < n && e == hipSuccess; i0 += kGrowAppendMax) {
    const int32_t m = std::min<int32_t>(kGrowAppendMax, n - i0);
    GrownRows g{};
    g.n = m;
    g.first = i0;
    const int32_t w0 = i0 == 0 ? 0 : wend[i0 - 1], w1 = wend[i0 + m - 1];
    g.nup = w1 - w0;                                   // at most two per entry
    for (int32_t j = 0; j < g.nup; ++j) {
      g.idx[j] = writes[w0 + j].first;
      g.val[j] = writes[w0 + j].second;
    }
    for (int32_t j = 0; j < m; ++j) {
      const int32_t s = seqs[i0 + j], pos = c->len[s] - 1;
      g.pos[j] = pos;
      g.blk[j] = c->table[s][pos / kBlock];
    }
    e = launch_grow_append(cv, layer, g, k, v, stream);
  }
  return e == hipSuccess ? KVC_OK : hip_fail(e, "grow + append launch");
}

int kvc_seq_grow_by(kvc_cache* c, int32_t seq, int32_t n_tokens, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = check_seq(c, seq);
  if (r) return r;
  if (!c->live[seq]) return fail(KVC_E_STATE, "sequence is not live");
  if (n_tokens < 0) return fail(KVC_E_INVAL, "negative token count");
  const int64_t len = c->len[seq], to = len + n_tokens;
  if (to > (int64_t)c->cfg.max_blocks_per_seq * kBlock)
    return fail(KVC_E_INVAL, "sequence would exceed its table width");
  // one block per token that starts a block: the blocks n single-token
  // grows would take, in the same (last-freed-first) order
  const int64_t fresh = (to + kBlock - 1) / kBlock - (len + kBlock - 1) / kBlock;
  const bool copy = n_tokens > 0 && needs_copy(c, seq);
  if (fresh + (copy ? 1 : 0) > (int64_t)c->free_list.size())
    return fail(KVC_E_NO_BLOCKS, "free list exhausted");
  Copier cp(c, stream);
  Uploader up(c, stream);
  if (copy) unshare_last(c, seq, cp, up);
  for (int64_t i = 0; i < fresh; ++i) {
    int32_t b = take_block(c);
    up.bt(seq, (int32_t)c->table[seq].size(), b);
    c->table[seq].push_back(b);
  }
  c->len[seq] = (int32_t)to;
  up.len(seq, c->len[seq]);
  int rc = cp.finish();
  int ru = up.finish();
  return rc ? rc : ru;
}

int kvc_seq_release(kvc_cache* c, int32_t seq, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = check_seq(c, seq);
  if (r) return r;
  if (!c->live[seq]) return fail(KVC_E_STATE, "sequence is not live");
  Uploader up(c, stream);
  auto& t = c->table[seq];
  for (size_t i = 0; i < t.size(); ++i) {
    if (--c->refs[t[i]] == 0) c->free_list.push_back(t[i]);
    up.bt(seq, (int32_t)i, -1);
  }
  t.clear();
  c->len[seq] = 0;
  c->live[seq] = 0;
  up.len(seq, 0);
  return up.finish();
}

int kvc_set_block_table(kvc_cache* c, int32_t seq, const int32_t* blocks, int32_t nblk,
                        int32_t len, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = check_seq(c, seq);
  if (r) return r;
  if (c->live[seq]) return fail(KVC_E_STATE, "sequence is already live");
  if (len < 0 || nblk != (len + kBlock - 1) / kBlock || (nblk > 0 && !blocks))
    return fail(KVC_E_INVAL, "nblk must equal ceil(len / 16)");
  if (nblk > c->cfg.max_blocks_per_seq) return fail(KVC_E_INVAL, "table too long");
  std::vector<uint8_t> seen(c->cfg.n_blocks, 0);
  for (int32_t i = 0; i < nblk; ++i) {
    int32_t b = blocks[i];
    if (b < 0 || b >= c->cfg.n_blocks) return fail(KVC_E_INVAL, "block id out of range");
    if (c->refs[b] || seen[b]) return fail(KVC_E_STATE, "block is not free");
    seen[b] = 1;
  }
  // Remove the chosen blocks from the free list, keeping the order of the rest.
  std::vector<int32_t> rest;
  rest.reserve(c->free_list.size());
  for (int32_t b : c->free_list)
    if (!seen[b]) rest.push_back(b);
  c->free_list.swap(rest);
  Uploader up(c, stream);
  auto& t = c->table[seq];
  t.assign(blocks, blocks + nblk);
  for (int32_t i = 0; i < nblk; ++i) {
    c->refs[blocks[i]] = 1;
    up.bt(seq, i, blocks[i]);
  }
  c->len[seq] = len;
  c->live[seq] = 1;
  up.len(seq, len);
  return up.finish();
}

int kvc_seq_share_prefix(kvc_cache* c, int32_t src, int32_t dst, int32_t prefix_len,
                         hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = check_seq(c, src);
  if (!r) r = check_seq(c, dst);
  if (r) return r;
  if (!c->live[src]) return fail(KVC_E_STATE, "source sequence is not live");
  if (c->live[dst] || src == dst) return fail(KVC_E_STATE, "destination sequence is already live");
  if (prefix_len < 0 || prefix_len > c->len[src])
    return fail(KVC_E_INVAL, "prefix_len must lie in 0 .. len(src)");
  const int32_t n = (prefix_len + kBlock - 1) / kBlock;
  Uploader up(c, stream);
  auto& t = c->table[dst];
  t.assign(c->table[src].begin(), c->table[src].begin() + n);
  for (int32_t i = 0; i < n; ++i) {
    c->refs[t[i]] += 1;
    up.bt(dst, i, t[i]);
  }
  c->len[dst] = prefix_len;
  c->live[dst] = 1;
  up.len(dst, prefix_len);
  return up.finish();
}

int kvc_block_refs(const kvc_cache* c, int32_t block, int32_t* out) {
  if (!c || !out) return fail(KVC_E_INVAL, "NULL argument");
  if (block < 0 || block >= c->cfg.n_blocks) return fail(KVC_E_INVAL, "block id out of range");
  *out = c->refs[block];
  return KVC_OK;
}

int kvc_seq_len(const kvc_cache* c, int32_t seq, int32_t* out) {
  if (!c || !out) return fail(KVC_E_INVAL, "NULL argument");
  int r = check_seq(c, seq);
  if (r) return r;
  if (!c->live[seq]) return fail(KVC_E_STATE, "sequence is not live");
  *out = c->len[seq];
  return KVC_OK;
}

int kvc_seq_blocks(const kvc_cache* c, int32_t seq, int32_t* blocks, int32_t cap,
                   int32_t* n_out) {
  if (!c || !n_out) return fail(KVC_E_INVAL, "NULL argument");
  int r = check_seq(c, seq);
  if (r) return r;
  if (!c->live[seq]) return fail(KVC_E_STATE, "sequence is not live");
  const auto& t = c->table[seq];
  *n_out = (int32_t)t.size();
  if (blocks) {
    if (cap < (int32_t)t.size()) return fail(KVC_E_INVAL, "cap too small");
    std::copy(t.begin(), t.end(), blocks);
  }
  return KVC_OK;
}

int kvc_free_blocks(const kvc_cache* c, int32_t* out) {
  if (!c || !out) return fail(KVC_E_INVAL, "NULL argument");
  *out = (int32_t)c->free_list.size();
  return KVC_OK;
}

int kvc_append(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs, const void* k,
               const void* v, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = need_dev(c);
  if (r) return r;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  if (n < 0) return fail(KVC_E_INVAL, "n < 0");
  if (n == 0) return KVC_OK;
  if (!seqs || !k || !v) return fail(KVC_E_INVAL, "NULL device pointer");
  hipError_t e = launch_append(c->view(), layer, n, seqs, k, v, stream);
  return e == hipSuccess ? KVC_OK : hip_fail(e, "append launch");
}

int kvc_write(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs, int32_t start,
              int32_t T, const void* k, const void* v, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = need_dev(c);
  if (r) return r;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  if (n < 0 || T < 0 || start < 0) return fail(KVC_E_INVAL, "negative size");
  if ((int64_t)start + T > (int64_t)c->cfg.max_blocks_per_seq * kBlock)
    return fail(KVC_E_INVAL, "rows beyond the table width");
  if (n == 0 || T == 0) return KVC_OK;
  if (!seqs || !k || !v) return fail(KVC_E_INVAL, "NULL device pointer");
  if (!aligned16(k) || !aligned16(v)) return fail(KVC_E_INVAL, "k/v must be 16-byte aligned");
  hipError_t e = launch_write(c->view(), layer, n, seqs, start, T, k, v, stream);
  return e == hipSuccess ? KVC_OK : hip_fail(e, "write launch");
}

namespace {
// window >= 0 (0: full causal attention), sinks >= 0; the VALU (f32) kernels
// have no window.
int check_window(const kvc_cache* c, int32_t window, int32_t sinks) {
  if (window < 0 || sinks < 0) return fail(KVC_E_INVAL, "window and sinks must be >= 0");
  if (window > 0 && c->cfg.kv_dtype == KVC_F32)
    return fail(KVC_E_UNSUPPORTED, "sliding windows need a bf16, f16, fp8 or int4 cache");
  return KVC_OK;
}
}  // namespace

int kvc_attn_prefill(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs, int32_t T,
                     const void* q, const void* k, const void* v, void* out, float scale,
                     hipStream_t stream) {
  return kvc_attn_prefill_window(c, layer, n, seqs, T, q, k, v, out, scale, 0, 0, stream);
}

int kvc_attn_prefill_window(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs,
                            int32_t T, const void* q, const void* k, const void* v, void* out,
                            float scale, int32_t window, int32_t sinks, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  const DispatchEvents ev = c->timing;                 // this call's, whatever its outcome
  c->timing = DispatchEvents{};
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(KVC_E_INVAL, "scale must be finite and positive");
  int rw = check_window(c, window, sinks);
  if (rw) return rw;
  int r = need_dev(c);
  if (r) return r;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  if (n < 0 || T < 0) return fail(KVC_E_INVAL, "negative size");
  if (n == 0 || T == 0) return KVC_OK;
  if (!q || !k || !v || !out) return fail(KVC_E_INVAL, "NULL device pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(KVC_E_INVAL, "q/k/v/out must be 16-byte aligned");
  if (seqs && (int64_t)T > (int64_t)c->cfg.max_blocks_per_seq * kBlock)
    return fail(KVC_E_INVAL, "prompt longer than the table width");
  // The cache write (HBM-bound) and the attention (matrix-core-bound) read the
  // same inputs and write disjoint outputs, so they run side by side: the
  // write on the handle's side stream, forked from and joined back into the
  // caller's stream.
  hipError_t e = hipSuccess;
  bool forked = false;
  if (seqs) {
    e = hipEventRecord(c->fork, stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(c->side, c->fork, 0);
    if (e == hipSuccess) {
      forked = true;
      e = launch_write(c->view(), layer, n, seqs, 0, T, k, v, c->side);
    }
  }
  if (e == hipSuccess)
    e = launch_prefill(c->view(), n, T, q, k, v, out, scale, window, sinks, stream, ev);
  if (forked) {
    // Whatever failed above, the caller's stream waits for everything enqueued
    // on the side stream, which may still read k and v.
    hipError_t j = hipEventRecord(c->join, c->side);
    if (j == hipSuccess) j = hipStreamWaitEvent(stream, c->join, 0);
    if (j != hipSuccess) j = hipStreamSynchronize(c->side);
    if (e == hipSuccess) e = j;
  }
  return e == hipSuccess ? KVC_OK : hip_fail(e, "prefill launch");
}

int kvc_attn_extend(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs, int32_t T,
                    const void* q, void* out, float scale, hipStream_t stream) {
  return kvc_attn_extend_window(c, layer, n, seqs, T, q, out, scale, 0, 0, stream);
}

int kvc_attn_extend_window(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs,
                           int32_t T, const void* q, void* out, float scale, int32_t window,
                           int32_t sinks, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  const DispatchEvents ev = c->timing;                 // this call's, whatever its outcome
  c->timing = DispatchEvents{};
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(KVC_E_INVAL, "scale must be finite and positive");
  if (window < 0 || sinks < 0) return fail(KVC_E_INVAL, "window and sinks must be >= 0");
  if (c->cfg.kv_dtype == KVC_F32)
    return fail(KVC_E_UNSUPPORTED, "attn_extend needs a bf16, f16, fp8 or int4 cache");
  int r = need_dev(c);
  if (r) return r;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  if (n < 0 || T < 0) return fail(KVC_E_INVAL, "negative size");
  if (n == 0 || T == 0) return KVC_OK;
  if ((int64_t)T > (int64_t)c->cfg.max_blocks_per_seq * kBlock)
    return fail(KVC_E_INVAL, "more query rows than a sequence can hold");
  if (!seqs || !q || !out) return fail(KVC_E_INVAL, "NULL device pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(KVC_E_INVAL, "q/out must be 16-byte aligned");
  bool handled = false;
  hipError_t e = launch_extend(c->view(), layer, n, seqs, T, q, out, scale, window, sinks, stream,
                               &handled, ev);
  if (e == hipSuccess && !handled) return fail(KVC_E_UNSUPPORTED, "no extend kernel for this shape");
  return e == hipSuccess ? KVC_OK : hip_fail(e, "extend launch");
}

int kvc_decode_workspace_bytes(const kvc_cache* c, int32_t n, int32_t num_splits, uint64_t* out) {
  if (!c || !out) return fail(KVC_E_INVAL, "NULL argument");
  if (n < 0 || num_splits < 0) return fail(KVC_E_INVAL, "negative size");
  DecodePlan p = make_decode_plan(c->view(), n, live_max_len(c), num_splits, c->cu_count);
  *out = p.ws_bytes;
  return KVC_OK;
}

int kvc_attn_decode(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs, const void* q,
                    void* out, float scale, int32_t num_splits, void* ws, uint64_t ws_bytes,
                    hipStream_t stream) {
  return kvc_attn_decode_window(c, layer, n, seqs, q, out, scale, 0, 0, num_splits, ws, ws_bytes,
                                stream);
}

namespace {
int decode_impl(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs, const void* knew,
                const void* vnew, const void* q, void* out, float scale, int32_t window,
                int32_t sinks, int32_t num_splits, void* ws, uint64_t ws_bytes,
                hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  const DispatchEvents ev = c->timing;                 // this call's, whatever its outcome
  c->timing = DispatchEvents{};
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(KVC_E_INVAL, "scale must be finite and positive");
  int rw = check_window(c, window, sinks);
  if (rw) return rw;
  int r = need_dev(c);
  if (r) return r;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  if (n < 0 || num_splits < 0) return fail(KVC_E_INVAL, "negative size");
  if (n == 0) return KVC_OK;
  if (!seqs || !q || !out) return fail(KVC_E_INVAL, "NULL device pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(KVC_E_INVAL, "q/out must be 16-byte aligned");
  if (knew && (!vnew || !aligned16(knew) || !aligned16(vnew)))
    return fail(KVC_E_INVAL, "k_new/v_new must be non-NULL and 16-byte aligned");
  int32_t max_len = live_max_len(c);
  if (max_len <= 0) return fail(KVC_E_STATE, "no live sequence holds any token");
  DecodePlan p = make_decode_plan(c->view(), n, max_len, num_splits, c->cu_count);
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes))
    return fail(KVC_E_WORKSPACE, "workspace too small: need " + std::to_string(p.ws_bytes) +
                                     " bytes");
  if (p.ws_bytes > 0 && !aligned16(ws)) return fail(KVC_E_INVAL, "workspace must be 16-byte aligned");
  hipError_t e = launch_decode(c->view(), layer, n, seqs, q, out, scale, p, ws, window, sinks,
                               knew, vnew, stream, ev);
  return e == hipSuccess ? KVC_OK : hip_fail(e, "decode launch");
}
}  // namespace

int kvc_attn_decode_window(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs,
                           const void* q, void* out, float scale, int32_t window, int32_t sinks,
                           int32_t num_splits, void* ws, uint64_t ws_bytes, hipStream_t stream) {
  return decode_impl(c, layer, n, seqs, nullptr, nullptr, q, out, scale, window, sinks,
                     num_splits, ws, ws_bytes, stream);
}

int kvc_attn_decode_append(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs,
                           const void* k_new, const void* v_new, const void* q, void* out,
                           float scale, int32_t window, int32_t sinks, int32_t num_splits,
                           void* ws, uint64_t ws_bytes, hipStream_t stream) {
  if (!k_new || !v_new) {
    if (c) c->timing = DispatchEvents{};
    return fail(KVC_E_INVAL, "k_new/v_new is NULL");
  }
  return decode_impl(c, layer, n, seqs, k_new, v_new, q, out, scale, window, sinks, num_splits,
                     ws, ws_bytes, stream);
}

int kvc_attn_decode_noalloc(kvc_cache* c, int32_t layer, int32_t n, const int32_t* seqs,
                            const void* q, void* out, float scale, int32_t num_splits,
                            hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = need_dev(c);
  if (r || n < 0 || num_splits < 0) {
    c->timing = DispatchEvents{};
    return r ? r : fail(KVC_E_INVAL, "negative size");
  }
  if (n > 0) {
    DecodePlan p = make_decode_plan(c->view(), n, live_max_len(c), num_splits, c->cu_count);
    if (p.ws_bytes > kScratchBytes) {
      c->timing = DispatchEvents{};
      return fail(KVC_E_WORKSPACE, "the call needs " + std::to_string(p.ws_bytes) +
                                       " bytes of workspace, more than the library scratch (" +
                                       std::to_string(kScratchBytes) +
                                       " bytes): use kvc_attn_decode with a workspace");
    }
  }
  return decode_impl(c, layer, n, seqs, nullptr, nullptr, q, out, scale, 0, 0, num_splits,
                     c->scratch, kScratchBytes, stream);
}

int kvc_set_dispatch_events(kvc_cache* c, void* start_event, void* stop_event, int32_t scope) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  if (scope != KVC_TIME_CALL && scope != KVC_TIME_MAIN_KERNEL) {
    c->timing = DispatchEvents{};
    return fail(KVC_E_INVAL, "scope must be KVC_TIME_CALL or KVC_TIME_MAIN_KERNEL");
  }
  c->timing.start = (hipEvent_t)start_event;
  c->timing.stop = (hipEvent_t)stop_event;
  c->timing.main_only = scope == KVC_TIME_MAIN_KERNEL;
  return KVC_OK;
}

int kvc_gather(const kvc_cache* c, int32_t layer, int32_t seq, int32_t start, int32_t count,
               void* k_out, void* v_out, hipStream_t stream) {
  if (!c) return fail(KVC_E_INVAL, "cache is NULL");
  int r = need_dev(c);
  if (r) return r;
  r = check_seq(c, seq);
  if (r) return r;
  if (!c->live[seq]) return fail(KVC_E_STATE, "sequence is not live");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(KVC_E_STATE, "layer out of range");
  if (start < 0 || count < 0 || (int64_t)start + count > c->len[seq])
    return fail(KVC_E_INVAL, "rows outside the sequence");
  if (count == 0) return KVC_OK;
  if (!k_out || !v_out) return fail(KVC_E_INVAL, "NULL device pointer");
  hipError_t e = launch_gather(c->view(), layer, seq, start, count, k_out, v_out, stream);
  return e == hipSuccess ? KVC_OK : hip_fail(e, "gather launch");
}

}  // extern "C"
