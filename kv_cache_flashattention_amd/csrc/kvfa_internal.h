// Internal declarations shared by the host manager and the kernel launchers.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <tuple>
#include <utility>

#include "kvfa.h"

namespace kvfa {

constexpr int kBlock = 16;          // tokens per physical block
constexpr int kTableUpdateMax = 240; // (index, value) pairs carried per update launch

// Everything a kernel needs to address the cache, passed by value.
struct CacheView {
  void* k;            // k_pool
  void* v;            // v_pool
  float* ks;          // k_scale (fp8 and int4 only)
  float* vs;          // v_scale (fp8 and int4 only)
  int32_t* bt;        // block_table [max_seqs][max_bps]
  int32_t* len;       // seq_len [max_seqs]
  int32_t n_layers, n_q, n_kv, d, n_blocks, max_seqs, max_bps;
  int32_t dtype;      // kvc_dtype of the storage
};

// Table/length writes enqueued as kernel arguments (no host staging buffer
// whose lifetime would have to outlive the copy).  idx >= 0 addresses
// block_table[idx]; idx < 0 addresses seq_len[-idx - 1].
struct TableUpdate {
  int32_t n;
  int32_t idx[kTableUpdateMax];
  int32_t val[kTableUpdateMax];
};

// One launch of a grow followed by the append of the grown rows.  The host's
// block manager has just placed each entry's new row, so the launch carries
// where it goes (its position in the sequence and the block holding it); the
// kernel reads no table or length for it.  The grow's table and length writes
// (TableUpdate form, at most two per entry) ride in the same launch.
constexpr int kGrowAppendMax = 96;
struct GrownRows {
  int32_t n;                        // entries in this launch
  int32_t first;                    // batch index of entry 0 (its row in k_new / v_new)
  int32_t nup;                      // table / length writes
  int32_t pos[kGrowAppendMax];      // position of the entry's new row
  int32_t blk[kGrowAppendMax];      // block holding that position
  int32_t idx[2 * kGrowAppendMax];  // as TableUpdate
  int32_t val[2 * kGrowAppendMax];
};

// Copy-on-write block copies: block src -> dst, every layer, K and V slabs of
// all kv heads and (fp8, int4) their scales.
constexpr int kCopyMax = 120;
struct BlockCopy {
  int32_t n;
  int32_t src[kCopyMax];
  int32_t dst[kCopyMax];
};

// How one decode call divides its work.
//  * Matrix-core path (16-bit and fp8 caches): a work list.  The batch's
//    32-token units, over every (sequence, kv-head group), are cut into
//    `waves` equal contiguous ranges, one per wave; each wave leaves one
//    (m, l, O) partial per piece of a (sequence, group) segment it covers and
//    a merge combines the pieces.  Batches larger than kMaxBatch are run in
//    sub-batches of at most kMaxBatch sequences.
//  * VALU path (f32 caches): a grid of `splits` fixed-length splits per
//    (sequence, query head), merged when splits > 1.
constexpr int kMaxBatch = 2048;

struct DecodePlan {
  int32_t work_list;  // 1: matrix-core work list, 0: VALU splits
  int32_t splits;     // VALU: splits per sequence
  int32_t split_len;  // VALU: tokens per split, a multiple of 64
  int32_t waves;      // work list: waves sharing the work of one (sub-)batch
  uint64_t ws_bytes;  // workspace bytes the call needs
};

__host__ __device__ inline int storage_bits(int dtype) {
  return dtype == KVC_F32 ? 32 : dtype == KVC_FP8_E4M3FN ? 8 : dtype == KVC_INT4 ? 4 : 16;
}
// Bytes of one (block, kv head) slab of K or V: 16 rows of d elements.
__host__ __device__ inline int64_t slab_bytes(int dtype, int d) {
  return (int64_t)kBlock * d * storage_bits(dtype) / 8;
}
__host__ __device__ inline bool has_scales(int dtype) {
  return dtype == KVC_FP8_E4M3FN || dtype == KVC_INT4;
}
inline int io_dtype(int dtype) { return has_scales(dtype) ? KVC_BF16 : dtype; }

// Size of the library-owned decode scratch used by kvc_attn_decode_noalloc
// (one copy per device, alive until the process ends).
constexpr uint64_t kScratchBytes = 64ull << 20;
// Device address of the current device's scratch (looked up once per device).
hipError_t scratch_address(void** addr);

DecodePlan make_decode_plan(const CacheView& cv, int32_t n, int32_t max_len, int32_t num_splits,
                            int32_t cu_count);
uint64_t work_list_ws_bytes(const CacheView& cv, int32_t nb, int32_t waves);
int work_list_waves_per_cu(const CacheView& cv);

// Dispatch events of one call (kvc_set_dispatch_events): `start` is recorded
// as the call's first kernel begins and `stop` as its last kernel ends, or,
// with main_only, both on the call's main kernel (decode: the work-list or
// VALU kernel; prefill and extend: the attention kernel in either case).
struct DispatchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool main_only = false;
};

// Launch of kernel k, optionally with dispatch events (hipExtLaunchKernel
// records them from the kernel's own dispatch, not as separate stream
// markers).  The arguments are converted to the kernel's parameter types.
template <typename... P, size_t... I>
hipError_t launch_args(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                       hipEvent_t stop, std::tuple<P...>& t, std::index_sequence<I...>) {
  void* args[] = {(void*)&std::get<I>(t)..., nullptr};
  if (!start && !stop) return hipLaunchKernel((const void*)k, grid, block, args, 0, s);
  return hipExtLaunchKernel((const void*)k, grid, block, args, 0, s, start, stop, 0);
}
template <typename... P, typename... A>
hipError_t launch_ev(void (*k)(P...), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                     hipEvent_t stop, A... a) {
  std::tuple<P...> t(a...);
  return launch_args(k, grid, block, s, start, stop, t, std::index_sequence_for<P...>{});
}

// Launchers: return hipSuccess or the launch error.
hipError_t launch_fill_tables(const CacheView& cv, hipStream_t s);
hipError_t launch_table_update(const CacheView& cv, const TableUpdate& u, hipStream_t s);
hipError_t launch_copy_blocks(const CacheView& cv, const BlockCopy& u, hipStream_t s);
// start: dispatch event recorded as the append kernel begins (or null).
hipError_t launch_append(const CacheView& cv, int layer, int n, const int32_t* seqs,
                         const void* k, const void* v, hipStream_t s,
                         hipEvent_t start = nullptr);
hipError_t launch_grow_append(const CacheView& cv, int layer, const GrownRows& g, const void* k,
                              const void* v, hipStream_t s, hipEvent_t start = nullptr);
hipError_t launch_write(const CacheView& cv, int layer, int n, const int32_t* seqs, int start,
                        int T, const void* k, const void* v, hipStream_t s);
hipError_t launch_gather(const CacheView& cv, int layer, int seq, int start, int count,
                         void* k_out, void* v_out, hipStream_t s);
// knew / vnew non-null: append those rows (kv_append) as part of the call.
// ev: dispatch events of the call's first and last kernels (or nulls).
hipError_t launch_decode(const CacheView& cv, int layer, int n, const int32_t* seqs,
                         const void* q, void* out, float scale, const DecodePlan& plan,
                         void* ws, int window, int sinks, const void* knew, const void* vnew,
                         hipStream_t s, DispatchEvents ev = {});
// window > 0: key j visible to position p iff p - window < j <= p or
// j < sinks; window = 0: full causal attention.
hipError_t launch_prefill(const CacheView& cv, int n, int T, const void* q, const void* k,
                          const void* v, void* out, float scale, int window, int sinks,
                          hipStream_t s, DispatchEvents ev = {});
// T query rows per sequence against the paged cache (bf16 / f16 caches);
// *handled = false when the cache type has no such kernel.
hipError_t launch_extend(const CacheView& cv, int layer, int n, const int32_t* seqs, int T,
                         const void* q, void* out, float scale, int window, int sinks,
                         hipStream_t s, bool* handled, DispatchEvents ev = {});

}  // namespace kvfa
