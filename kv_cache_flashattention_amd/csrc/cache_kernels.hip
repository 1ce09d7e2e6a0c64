// Cache maintenance kernels: table fills and updates, kv_append (one row per
// sequence), bulk row writes (prefill / population) and the block-table
// gather.
//
// Addressing follows the paged layout: logical position p of a sequence is
// slot p % 16 of block table[p / 16] ("KV Cache & Flash Attention."
// (kvcache-7e2), PagedAttention section).  K slabs are [16][d] (a token's
// row contiguous), V slabs are [d][16] (one head-dimension column of the
// block's 16 tokens contiguous), which is the order the attention kernels'
// matrix-core operands consume.
#include <algorithm>

#include "kvfa_internal.h"
#include "fp8_e4m3.h"

namespace kvfa {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Validates a device-side sequence entry; returns its length or -1.
__device__ __forceinline__ int seq_length(const CacheView& cv, int seq) {
  if (seq < 0 || seq >= cv.max_seqs) return -1;
  int L = cv.len[seq];
  if (L <= 0 || L > cv.max_bps * kBlock) return -1;
  return L;
}

__device__ __forceinline__ int block_of(const CacheView& cv, int seq, int pos) {
  int b = cv.bt[(int64_t)seq * cv.max_bps + pos / kBlock];
  return (b < 0 || b >= cv.n_blocks) ? -1 : b;
}

// Element offset of slab (layer, block, head) in a pool.
__device__ __forceinline__ int64_t slab_elems(const CacheView& cv, int layer, int blk, int h) {
  return (((int64_t)layer * cv.n_blocks + blk) * cv.n_kv + h) * (int64_t)(kBlock * cv.d);
}

__device__ __forceinline__ int64_t scale_idx(const CacheView& cv, int layer, int blk, int h) {
  return ((int64_t)layer * cv.n_blocks + blk) * cv.n_kv + h;
}

// ---------------------------------------------------------------- tables
__global__ void k_fill_tables(CacheView cv) {
  int64_t nbt = (int64_t)cv.max_seqs * cv.max_bps;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nbt;
       i += (int64_t)gridDim.x * blockDim.x)
    cv.bt[i] = -1;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < cv.max_seqs;
       i += (int64_t)gridDim.x * blockDim.x)
    cv.len[i] = 0;
}

// One table or length write: idx >= 0 is block_table[idx], idx < 0 is
// seq_len[-idx - 1]; indices outside the tables are dropped.
__device__ __forceinline__ void table_write(const CacheView& cv, int32_t idx, int32_t val) {
  if (idx >= 0) {
    if ((int64_t)idx < (int64_t)cv.max_seqs * cv.max_bps) cv.bt[idx] = val;
  } else {
    const int32_t s = -idx - 1;
    if (s < cv.max_seqs) cv.len[s] = val;
  }
}

__global__ void k_table_update(CacheView cv, TableUpdate u) {
  const int i = threadIdx.x;
  if (i < u.n) table_write(cv, u.idx[i], u.val[i]);
}

// ---------------------------------------------------------------- block copy
// Copy-on-write of a shared block: workgroup (pair p, layer l) copies the
// K and V data of block src[p] to block dst[p] in layer l (all kv heads,
// contiguous in both pools) and, for fp8 and int4, their per-head scales.  Block ids
// come from the host manager, which only hands out ids below n_blocks.
__global__ __launch_bounds__(256) void k_copy_blocks(CacheView cv, BlockCopy u) {
  const int p = blockIdx.x, layer = blockIdx.y;
  if (p >= u.n) return;
  const int64_t src = u.src[p], dst = u.dst[p];
  if (src < 0 || src >= cv.n_blocks || dst < 0 || dst >= cv.n_blocks) return;
  const int64_t bytes = cv.n_kv * slab_bytes(cv.dtype, cv.d);
  const int64_t so = ((int64_t)layer * cv.n_blocks + src) * bytes;
  const int64_t dof = ((int64_t)layer * cv.n_blocks + dst) * bytes;
  const uint4* ks = (const uint4*)((const uint8_t*)cv.k + so);
  const uint4* vs = (const uint4*)((const uint8_t*)cv.v + so);
  uint4* kd = (uint4*)((uint8_t*)cv.k + dof);
  uint4* vd = (uint4*)((uint8_t*)cv.v + dof);
  // eight 16-byte chunks of K and of V in flight per thread before the stores
  const int64_t n16 = bytes / 16;
  for (int64_t i0 = threadIdx.x; i0 < n16; i0 += 8 * (int64_t)blockDim.x) {
    uint4 a[8], c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + u * (int64_t)blockDim.x;
      if (i < n16) {
        a[u] = ks[i];
        c[u] = vs[i];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + u * (int64_t)blockDim.x;
      if (i < n16) {
        kd[i] = a[u];
        vd[i] = c[u];
      }
    }
  }
  if (has_scales(cv.dtype)) {
    for (int h = threadIdx.x; h < cv.n_kv; h += blockDim.x) {
      const int64_t s0 = ((int64_t)layer * cv.n_blocks + src) * cv.n_kv + h;
      const int64_t d0 = ((int64_t)layer * cv.n_blocks + dst) * cv.n_kv + h;
      cv.ks[d0] = cv.ks[s0];
      cv.vs[d0] = cv.vs[s0];
    }
  }
}

// ---------------------------------------------------------------- append
// One wave per (sequence, kv head): the new row goes to slot (L-1) % 16 of
// block table[(L-1) / 16].  16/32-bit storage copies the bits.
template <typename E>
__device__ void append_row_copy(const CacheView& cv, int layer, int b, int h, int blk, int slot,
                                const E* knew, const E* vnew) {
  const int d = cv.d, lane = threadIdx.x;
  const int64_t base = slab_elems(cv, layer, blk, h);
  E* K = (E*)cv.k + base;
  E* V = (E*)cv.v + base;
  const E* kr = knew + ((int64_t)b * cv.n_kv + h) * d;
  const E* vr = vnew + ((int64_t)b * cv.n_kv + h) * d;
  for (int j = lane; j < d; j += 64) {
    K[slot * d + j] = kr[j];
    V[j * kBlock + slot] = vr[j];
  }
}

template <typename E>
__global__ __launch_bounds__(64) void k_append_copy(CacheView cv, int layer, const int32_t* seqs,
                                                    const E* knew, const E* vnew) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int seq = seqs[b];
  const int L = seq_length(cv, seq);
  if (L < 0) return;
  const int pos = L - 1;
  const int blk = block_of(cv, seq, pos);
  if (blk < 0) return;
  append_row_copy(cv, layer, b, h, blk, pos % kBlock, knew, vnew);
}

// fp8 append of one slab column set.  Every lane owns the head-dimension
// indices lane, lane+64; the slab's scale is kept equal to absmax/448 over the
// rows written so far; when it grows, rows 0..slot-1 are re-encoded from
// their decoded values.  `row_stride` / `col_stride` place element (r, j)
// of the slab at r*row_stride + j*col_stride (K: d, 1; V: 1, 16).
__device__ void fp8_append_slab(uint8_t* slab, float* scale, int slot, int d, int row_stride,
                                int col_stride, const uint16_t* row_bf16) {
  const int lane = threadIdx.x;
  float x[2] = {0.f, 0.f};
  float amax = 0.f;
  for (int t = 0, j = lane; j < d; j += 64, ++t) {
    x[t] = bf16_to_f32(row_bf16[j]);
    amax = fmaxf(amax, fabsf(x[t]));
  }
  amax = wave_max(amax);
  const float s_new = amax / 448.0f;
  float s = s_new;
  if (slot > 0) {
    const float s_old = *scale;
    s = fmaxf(s_old, s_new);
    if (s > s_old) {
      for (int r = 0; r < slot; ++r)
        for (int j = lane; j < d; j += 64) {
          uint8_t* p = slab + r * row_stride + j * col_stride;
          float y = e4m3_decode(*p) * s_old;
          *p = (uint8_t)e4m3_encode(y / s);
        }
    }
  }
  for (int t = 0, j = lane; j < d; j += 64, ++t) {
    float y = s > 0.f ? x[t] / s : x[t];
    slab[slot * row_stride + j * col_stride] = (uint8_t)e4m3_encode(y);
  }
  if (lane == 0) *scale = s;
}

__device__ void append_row_fp8(const CacheView& cv, int layer, int b, int h, int blk, int slot,
                               const uint16_t* knew, const uint16_t* vnew) {
  const int d = cv.d;
  const int64_t base = slab_elems(cv, layer, blk, h);
  const int64_t si = scale_idx(cv, layer, blk, h);
  const int64_t row = ((int64_t)b * cv.n_kv + h) * d;
  fp8_append_slab((uint8_t*)cv.k + base, cv.ks + si, slot, d, d, 1, knew + row);
  fp8_append_slab((uint8_t*)cv.v + base, cv.vs + si, slot, d, 1, kBlock, vnew + row);
}

__global__ __launch_bounds__(64) void k_append_fp8(CacheView cv, int layer, const int32_t* seqs,
                                                   const uint16_t* knew, const uint16_t* vnew) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int seq = seqs[b];
  const int L = seq_length(cv, seq);
  if (L < 0) return;
  const int pos = L - 1;
  const int blk = block_of(cv, seq, pos);
  if (blk < 0) return;
  append_row_fp8(cv, layer, b, h, blk, pos % kBlock, knew, vnew);
}

// ---------------------------------------------------------------- bulk write
// One workgroup per (logical block touched, kv head, sequence) writes the
// block's rows that fall in [start, start+T).  Input rows are
// [n][T][n_kv][d].  The block's rows are staged in LDS so that V can be
// written column by column in the [d][16] order.
template <typename E>
__global__ __launch_bounds__(256) void k_write_copy(CacheView cv, int layer, const int32_t* seqs,
                                                    int start, int T, const E* kin, const E* vin) {
  __shared__ E vt[kBlock * 128];
  const int lb = start / kBlock + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int seq = seqs[b];
  const int L = seq_length(cv, seq);
  if (L < 0 || start + T > L) return;
  const int blk = block_of(cv, seq, lb * kBlock);
  if (blk < 0) return;
  const int d = cv.d;
  const int p0 = max(start, lb * kBlock), p1 = min(start + T, lb * kBlock + kBlock);
  const int64_t base = slab_elems(cv, layer, blk, h);
  E* K = (E*)cv.k + base;
  E* V = (E*)cv.v + base;
  if constexpr (sizeof(E) == 2) {
    // 16-bit rows move in 16-byte chunks (8 values): K straight to its slab
    // rows, V into a padded LDS tile, then out as 16-byte columns of 8 tokens
    // (element by element where the 8 tokens straddle the written range).
    __shared__ __attribute__((aligned(16))) uint16_t vt2[kBlock][128 + 8];
    const int G8 = d / 8;
    for (int i = threadIdx.x; i < kBlock * G8; i += blockDim.x) {
      const int r = i / G8, gk = i % G8, p = lb * kBlock + r;
      if (p >= p0 && p < p1) {
        const int64_t src = (((int64_t)b * T + (p - start)) * cv.n_kv + h) * d + 8 * gk;
        *(uint4*)(K + r * d + 8 * gk) = *(const uint4*)(kin + src);
        *(uint4*)&vt2[r][8 * gk] = *(const uint4*)(vin + src);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < d * 2; i += blockDim.x) {
      const int j = i >> 1, r0 = 8 * (i & 1), pr = lb * kBlock + r0;
      if (pr >= p0 && pr + 8 <= p1) {
        uint4 x;
        x.x = (uint32_t)vt2[r0][j] | ((uint32_t)vt2[r0 + 1][j] << 16);
        x.y = (uint32_t)vt2[r0 + 2][j] | ((uint32_t)vt2[r0 + 3][j] << 16);
        x.z = (uint32_t)vt2[r0 + 4][j] | ((uint32_t)vt2[r0 + 5][j] << 16);
        x.w = (uint32_t)vt2[r0 + 6][j] | ((uint32_t)vt2[r0 + 7][j] << 16);
        *(uint4*)(V + j * kBlock + r0) = x;
      } else {
        for (int e = 0; e < 8; ++e)
          if (pr + e >= p0 && pr + e < p1) V[j * kBlock + r0 + e] = vt2[r0 + e][j];
      }
    }
  } else {
    for (int i = threadIdx.x; i < (p1 - p0) * d; i += blockDim.x) {
      const int p = p0 + i / d, j = i % d;
      const int64_t src = (((int64_t)b * T + (p - start)) * cv.n_kv + h) * d + j;
      K[(p % kBlock) * d + j] = kin[src];
      vt[(p % kBlock) * d + j] = vin[src];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < d * kBlock; i += blockDim.x) {
      const int j = i / kBlock, r = i % kBlock, p = lb * kBlock + r;
      if (p >= p0 && p < p1) V[j * kBlock + r] = vt[r * d + j];
    }
  }
}

// fp8 bulk write: the new rows of a slab are encoded together with one scale
// update (absmax over all of them), after re-encoding older rows if the
// scale grew.
__global__ __launch_bounds__(256) void k_write_fp8(CacheView cv, int layer, const int32_t* seqs,
                                                   int start, int T, const uint16_t* kin,
                                                   const uint16_t* vin) {
  __shared__ float red[2][4];
  const int lb = start / kBlock + blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int seq = seqs[b];
  const int L = seq_length(cv, seq);
  if (L < 0 || start + T > L) return;
  const int blk = block_of(cv, seq, lb * kBlock);
  if (blk < 0) return;
  const int d = cv.d;
  const int p0 = max(start, lb * kBlock), p1 = min(start + T, lb * kBlock + kBlock);
  const int r0 = p0 - lb * kBlock, nnew = p1 - p0;
  const int64_t base = slab_elems(cv, layer, blk, h);
  const int64_t si = scale_idx(cv, layer, blk, h);
  uint8_t* K = (uint8_t*)cv.k + base;
  uint8_t* V = (uint8_t*)cv.v + base;
  // Old scales are read by every thread before the barrier below; thread 0
  // overwrites them only after it.
  const float sk_old = r0 > 0 ? cv.ks[si] : 0.f, sv_old = r0 > 0 ? cv.vs[si] : 0.f;
  float ka = 0.f, va = 0.f;
  for (int i = threadIdx.x; i < nnew * d; i += blockDim.x) {
    const int64_t src = (((int64_t)b * T + (p0 - start + i / d)) * cv.n_kv + h) * d + i % d;
    ka = fmaxf(ka, fabsf(bf16_to_f32(kin[src])));
    va = fmaxf(va, fabsf(bf16_to_f32(vin[src])));
  }
  ka = wave_max(ka);
  va = wave_max(va);
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = ka;
    red[1][w] = va;
  }
  __syncthreads();
  ka = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  va = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  float sk = ka / 448.0f, sv = va / 448.0f;
  if (r0 > 0) {
    const float skn = fmaxf(sk_old, sk), svn = fmaxf(sv_old, sv);
    for (int i = threadIdx.x; i < r0 * d; i += blockDim.x) {
      const int r = i / d, j = i % d;
      if (skn > sk_old) {
        uint8_t* p = K + r * d + j;
        *p = (uint8_t)e4m3_encode((e4m3_decode(*p) * sk_old) / skn);
      }
      if (svn > sv_old) {
        uint8_t* p = V + j * kBlock + r;
        *p = (uint8_t)e4m3_encode((e4m3_decode(*p) * sv_old) / svn);
      }
    }
    sk = skn;
    sv = svn;
  }
  for (int i = threadIdx.x; i < nnew * d; i += blockDim.x) {
    const int r = r0 + i / d, j = i % d;
    const int64_t src = (((int64_t)b * T + (p0 - start + i / d)) * cv.n_kv + h) * d + j;
    const float xk = bf16_to_f32(kin[src]), xv = bf16_to_f32(vin[src]);
    K[r * d + j] = (uint8_t)e4m3_encode(sk > 0.f ? xk / sk : xk);
    V[j * kBlock + r] = (uint8_t)e4m3_encode(sv > 0.f ? xv / sv : xv);
  }
  if (threadIdx.x == 0) {
    cv.ks[si] = sk;
    cv.vs[si] = sv;
  }
}

// ---------------------------------------------------------------- int4
// Codes are signed nibbles, two per byte (even element low).  K slabs are
// [16][d/2] bytes, V slabs [d][8] bytes (tokens 2i, 2i+1 of a column in
// byte i).  A code is rint(x / s) clamped to +-7 with s = absmax/7 of the
// slab's rows; a growing scale re-encodes the older rows from
// fl(code * s_old).
__device__ __forceinline__ uint32_t int4_encode(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -7.0f), 7.0f);
  return (uint32_t)(int)r & 0xFu;
}
__device__ __forceinline__ float int4_value(uint32_t nib) {
  return (float)(((int)(nib << 28)) >> 28);
}
// New nibble of a slot: `old` re-encoded when the scale grew (rows < r0),
// the new value x encoded (rows r0 .. r0+nnew-1), else unchanged.
__device__ __forceinline__ uint32_t int4_update(uint32_t old, int r, int r0, int nnew, float s_old,
                                                float s, float x) {
  if (r < r0) return s > s_old ? int4_encode((int4_value(old) * s_old) / s) : old;
  if (r < r0 + nnew) return int4_encode(s > 0.f ? x / s : x);
  return old;
}

// One workgroup per (logical block touched, kv head, sequence), like the
// bulk writes above; start < 0 selects append mode: one row per sequence,
// at position seq_len - 1, inputs [n][n_kv][d].  Every thread owns whole
// bytes, so the two nibbles of a byte are written together.
// Rows [start, start + T) of batch entry b that fall in logical block lb
// (physical block blk), kv head h; input rows are [n][T][n_kv][d].  Called
// by whole workgroups of 256 threads.
__device__ void int4_write_rows(const CacheView& cv, int layer, int b, int h, int blk, int lb,
                                int start, int T, const uint16_t* kin, const uint16_t* vin) {
  __shared__ float red[2][4];
  const int d = cv.d, hb = d / 2;
  const int p0 = max(start, lb * kBlock), p1 = min(start + T, lb * kBlock + kBlock);
  const int r0 = p0 - lb * kBlock, nnew = p1 - p0;
  const int64_t si = scale_idx(cv, layer, blk, h);
  uint8_t* K = (uint8_t*)cv.k + si * slab_bytes(KVC_INT4, d);
  uint8_t* V = (uint8_t*)cv.v + si * slab_bytes(KVC_INT4, d);
  auto in_idx = [&](int r, int j) -> int64_t {     // slab row r (new), column j
    return (((int64_t)b * T + (lb * kBlock + r - start)) * cv.n_kv + h) * d + j;
  };
  // Old scales are read by every thread before the barrier below; thread 0
  // overwrites them only after it.
  const float sk_old = r0 > 0 ? cv.ks[si] : 0.f, sv_old = r0 > 0 ? cv.vs[si] : 0.f;
  float ka = 0.f, va = 0.f;
  for (int i = threadIdx.x; i < nnew * d; i += blockDim.x) {
    const int64_t src = in_idx(r0 + i / d, i % d);
    ka = fmaxf(ka, fabsf(bf16_to_f32(kin[src])));
    va = fmaxf(va, fabsf(bf16_to_f32(vin[src])));
  }
  ka = wave_max(ka);
  va = wave_max(va);
  const int w = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = ka;
    red[1][w] = va;
  }
  __syncthreads();
  ka = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  va = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  float sk = ka / 7.0f, sv = va / 7.0f;
  if (r0 > 0) {
    sk = fmaxf(sk_old, sk);
    sv = fmaxf(sv_old, sv);
  }
  // K: bytes (row r, pair jb) of the rows that change (older rows only when
  // the scale grew).
  const int kr_lo = sk > sk_old || r0 == 0 ? 0 : r0;
  for (int i = kr_lo * hb + threadIdx.x; i < (r0 + nnew) * hb; i += blockDim.x) {
    const int r = i / hb, jb = i % hb;
    const uint32_t old = K[i];
    float x0 = 0.f, x1 = 0.f;
    if (r >= r0) {
      x0 = bf16_to_f32(kin[in_idx(r, 2 * jb)]);
      x1 = bf16_to_f32(kin[in_idx(r, 2 * jb + 1)]);
    }
    const uint32_t lo = int4_update(old & 0xFu, r, r0, nnew, sk_old, sk, x0);
    const uint32_t hi = int4_update(old >> 4, r, r0, nnew, sk_old, sk, x1);
    K[i] = (uint8_t)(lo | (hi << 4));
  }
  // V: bytes (column j, token pair rb).
  const int vr_lo = sv > sv_old || r0 == 0 ? 0 : r0;
  const int rb_lo = vr_lo / 2, rb_hi = (r0 + nnew + 1) / 2, nrb = rb_hi - rb_lo;
  for (int i = threadIdx.x; i < d * nrb; i += blockDim.x) {
    const int j = i / nrb, rb = rb_lo + i % nrb;
    uint8_t* p = V + j * (kBlock / 2) + rb;
    const uint32_t old = *p;
    const int ra = 2 * rb, rc = 2 * rb + 1;
    const float x0 = ra >= r0 && ra < r0 + nnew ? bf16_to_f32(vin[in_idx(ra, j)]) : 0.f;
    const float x1 = rc >= r0 && rc < r0 + nnew ? bf16_to_f32(vin[in_idx(rc, j)]) : 0.f;
    const uint32_t lo = int4_update(old & 0xFu, ra, r0, nnew, sv_old, sv, x0);
    const uint32_t hi = int4_update(old >> 4, rc, r0, nnew, sv_old, sv, x1);
    *p = (uint8_t)(lo | (hi << 4));
  }
  if (threadIdx.x == 0) {
    cv.ks[si] = sk;
    cv.vs[si] = sv;
  }
}

__global__ __launch_bounds__(256) void k_write_int4(CacheView cv, int layer, const int32_t* seqs,
                                                    int start, int T, const uint16_t* kin,
                                                    const uint16_t* vin) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int seq = seqs[b];
  const int L = seq_length(cv, seq);
  if (L < 0) return;
  int lb;
  if (start < 0) {
    start = L - 1;
    T = 1;
    lb = start / kBlock;
  } else {
    if (start + T > L) return;
    lb = start / kBlock + blockIdx.x;
  }
  const int blk = block_of(cv, seq, lb * kBlock);
  if (blk < 0) return;
  int4_write_rows(cv, layer, b, h, blk, lb, start, T, kin, vin);
}

// ---------------------------------------------------------------- grow + append
// The grow's table and length writes, by workgroup (0, 0, 0) of a launch.
__device__ __forceinline__ void grown_tables(const CacheView& cv, const GrownRows& g) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < g.nup; i += blockDim.x) table_write(cv, g.idx[i], g.val[i]);
}

// One wave per (entry, kv head), as the append above, with the row's place
// taken from the launch.
template <typename E>
__global__ __launch_bounds__(64) void k_grow_append_copy(CacheView cv, int layer, GrownRows g,
                                                         const E* knew, const E* vnew) {
  grown_tables(cv, g);
  const int i = blockIdx.x;
  if (i >= g.n) return;
  append_row_copy(cv, layer, g.first + i, blockIdx.y, g.blk[i], g.pos[i] % kBlock, knew, vnew);
}

__global__ __launch_bounds__(64) void k_grow_append_fp8(CacheView cv, int layer, GrownRows g,
                                                        const uint16_t* knew,
                                                        const uint16_t* vnew) {
  grown_tables(cv, g);
  const int i = blockIdx.x;
  if (i >= g.n) return;
  append_row_fp8(cv, layer, g.first + i, blockIdx.y, g.blk[i], g.pos[i] % kBlock, knew, vnew);
}

__global__ __launch_bounds__(256) void k_grow_append_int4(CacheView cv, int layer, GrownRows g,
                                                         const uint16_t* knew,
                                                         const uint16_t* vnew) {
  grown_tables(cv, g);
  const int i = blockIdx.z;
  if (i >= g.n) return;
  const int pos = g.pos[i];
  int4_write_rows(cv, layer, g.first + i, blockIdx.y, g.blk[i], pos / kBlock, pos, 1, knew, vnew);
}

// Gather of an int4 cache: K and V rows [count][n_kv][d/2] bytes, codes
// packed along d like the K slabs.  One thread per output byte.
__global__ __launch_bounds__(256) void k_gather_int4(CacheView cv, int layer, int seq, int start,
                                                     int count, uint8_t* kout, uint8_t* vout) {
  const int hb = cv.d / 2;
  const int64_t total = (int64_t)count * cv.n_kv * hb;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int jb = (int)(i % hb);
    const int h = (int)((i / hb) % cv.n_kv);
    const int p = start + (int)(i / ((int64_t)hb * cv.n_kv));
    const int blk = block_of(cv, seq, p);
    if (blk < 0) continue;
    const int64_t base = scale_idx(cv, layer, blk, h) * slab_bytes(KVC_INT4, cv.d);
    const uint8_t* K = (const uint8_t*)cv.k + base;
    const uint8_t* V = (const uint8_t*)cv.v + base;
    const int r = p % kBlock, sh = 4 * (r & 1);
    kout[i] = K[r * hb + jb];
    const uint32_t lo = (V[(2 * jb) * (kBlock / 2) + r / 2] >> sh) & 0xFu;
    const uint32_t hi = (V[(2 * jb + 1) * (kBlock / 2) + r / 2] >> sh) & 0xFu;
    vout[i] = (uint8_t)(lo | (hi << 4));
  }
}

// ---------------------------------------------------------------- gather
template <typename E>
__global__ __launch_bounds__(256) void k_gather(CacheView cv, int layer, int seq, int start,
                                                int count, E* kout, E* vout) {
  const int d = cv.d;
  const int64_t total = (int64_t)count * cv.n_kv * d;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(i % d);
    const int h = (int)((i / d) % cv.n_kv);
    const int p = start + (int)(i / ((int64_t)d * cv.n_kv));
    const int blk = block_of(cv, seq, p);
    if (blk < 0) continue;
    const int64_t base = slab_elems(cv, layer, blk, h);
    kout[i] = ((const E*)cv.k)[base + (p % kBlock) * d + j];
    vout[i] = ((const E*)cv.v)[base + j * kBlock + (p % kBlock)];
  }
}

}  // namespace

hipError_t launch_fill_tables(const CacheView& cv, hipStream_t s) {
  int64_t nbt = (int64_t)cv.max_seqs * cv.max_bps;
  int grid = (int)std::min<int64_t>((nbt + 255) / 256 + 1, 4096);
  hipLaunchKernelGGL(k_fill_tables, dim3(grid), dim3(256), 0, s, cv);
  return hipGetLastError();
}

hipError_t launch_table_update(const CacheView& cv, const TableUpdate& u, hipStream_t s) {
  hipLaunchKernelGGL(k_table_update, dim3(1), dim3(256), 0, s, cv, u);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CacheView& cv, const BlockCopy& u, hipStream_t s) {
  if (u.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_copy_blocks, dim3(u.n, cv.n_layers), dim3(256), 0, s, cv, u);
  return hipGetLastError();
}

hipError_t launch_append(const CacheView& cv, int layer, int n, const int32_t* seqs,
                         const void* k, const void* v, hipStream_t s, hipEvent_t start) {
  dim3 grid(n, cv.n_kv);
  switch (cv.dtype) {
    case KVC_F32:
      return launch_ev(k_append_copy<uint32_t>, grid, dim3(64), s, start, nullptr, cv, layer,
                       seqs, (const uint32_t*)k, (const uint32_t*)v);
    case KVC_F16:
    case KVC_BF16:
      return launch_ev(k_append_copy<uint16_t>, grid, dim3(64), s, start, nullptr, cv, layer,
                       seqs, (const uint16_t*)k, (const uint16_t*)v);
    case KVC_INT4:
      return launch_ev(k_write_int4, dim3(1, cv.n_kv, n), dim3(256), s, start, nullptr, cv, layer,
                       seqs, -1, 1, (const uint16_t*)k, (const uint16_t*)v);
    default:
      return launch_ev(k_append_fp8, grid, dim3(64), s, start, nullptr, cv, layer, seqs,
                       (const uint16_t*)k, (const uint16_t*)v);
  }
}

hipError_t launch_grow_append(const CacheView& cv, int layer, const GrownRows& g, const void* k,
                              const void* v, hipStream_t s, hipEvent_t start) {
  if (g.n <= 0 && g.nup <= 0) return hipSuccess;
  const int n = g.n > 0 ? g.n : 1;                     // table writes alone: one workgroup row
  dim3 grid(n, cv.n_kv);
  switch (cv.dtype) {
    case KVC_F32:
      return launch_ev(k_grow_append_copy<uint32_t>, grid, dim3(64), s, start, nullptr, cv, layer,
                       g, (const uint32_t*)k, (const uint32_t*)v);
    case KVC_F16:
    case KVC_BF16:
      return launch_ev(k_grow_append_copy<uint16_t>, grid, dim3(64), s, start, nullptr, cv, layer,
                       g, (const uint16_t*)k, (const uint16_t*)v);
    case KVC_INT4:
      return launch_ev(k_grow_append_int4, dim3(1, cv.n_kv, n), dim3(256), s, start, nullptr, cv,
                       layer, g, (const uint16_t*)k, (const uint16_t*)v);
    default:
      return launch_ev(k_grow_append_fp8, grid, dim3(64), s, start, nullptr, cv, layer, g,
                       (const uint16_t*)k, (const uint16_t*)v);
  }
}

hipError_t launch_write(const CacheView& cv, int layer, int n, const int32_t* seqs, int start,
                        int T, const void* k, const void* v, hipStream_t s) {
  const int nlb = (start + T - 1) / kBlock - start / kBlock + 1;
  dim3 grid(nlb, cv.n_kv, n);
  switch (cv.dtype) {
    case KVC_F32:
      hipLaunchKernelGGL(k_write_copy<uint32_t>, grid, dim3(256), 0, s, cv, layer, seqs, start, T,
                         (const uint32_t*)k, (const uint32_t*)v);
      break;
    case KVC_F16:
    case KVC_BF16:
      hipLaunchKernelGGL(k_write_copy<uint16_t>, grid, dim3(256), 0, s, cv, layer, seqs, start, T,
                         (const uint16_t*)k, (const uint16_t*)v);
      break;
    case KVC_INT4:
      hipLaunchKernelGGL(k_write_int4, grid, dim3(256), 0, s, cv, layer, seqs, start, T,
                         (const uint16_t*)k, (const uint16_t*)v);
      break;
    default:
      hipLaunchKernelGGL(k_write_fp8, grid, dim3(256), 0, s, cv, layer, seqs, start, T,
                         (const uint16_t*)k, (const uint16_t*)v);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const CacheView& cv, int layer, int seq, int start, int count,
                         void* k_out, void* v_out, hipStream_t s) {
  int64_t total = (int64_t)count * cv.n_kv * cv.d;
  int grid = (int)std::min<int64_t>((total + 255) / 256, 8192);
  switch (storage_bits(cv.dtype)) {
    case 4:
      hipLaunchKernelGGL(k_gather_int4, dim3(grid), dim3(256), 0, s, cv, layer, seq, start,
                         count, (uint8_t*)k_out, (uint8_t*)v_out);
      break;
    case 32:
      hipLaunchKernelGGL(k_gather<uint32_t>, dim3(grid), dim3(256), 0, s, cv, layer, seq, start,
                         count, (uint32_t*)k_out, (uint32_t*)v_out);
      break;
    case 16:
      hipLaunchKernelGGL(k_gather<uint16_t>, dim3(grid), dim3(256), 0, s, cv, layer, seq, start,
                         count, (uint16_t*)k_out, (uint16_t*)v_out);
      break;
    default:
      hipLaunchKernelGGL(k_gather<uint8_t>, dim3(grid), dim3(256), 0, s, cv, layer, seq, start,
                         count, (uint8_t*)k_out, (uint8_t*)v_out);
  }
  return hipGetLastError();
}

}  // namespace kvfa
