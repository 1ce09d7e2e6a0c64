// Small device helpers shared by the attention kernels.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "kvfa_internal.h"

namespace kvfa {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Storage/io element <-> float for the three element kinds the attention
// kernels read: float (f32), half (f16), bf16 bit patterns (uint16_t tag).
struct BF16 { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(BF16 x) { return bf16_bits_to_f32(x.bits); }

template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ BF16 from_f32<BF16>(float x) { return BF16{f32_to_bf16_bits(x)}; }

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Length of a device-side sequence entry, or -1 if the entry is unusable.
__device__ __forceinline__ int valid_len(const CacheView& cv, int seq) {
  if (seq < 0 || seq >= cv.max_seqs) return -1;
  int L = cv.len[seq];
  if (L <= 0 || L > cv.max_bps * kBlock) return -1;
  return L;
}

__device__ __forceinline__ int table_block(const CacheView& cv, int seq, int pos) {
  int b = cv.bt[(int64_t)seq * cv.max_bps + pos / kBlock];
  return (b < 0 || b >= cv.n_blocks) ? -1 : b;
}

__device__ __forceinline__ int64_t slab_offset(const CacheView& cv, int layer, int blk, int h) {
  return (((int64_t)layer * cv.n_blocks + blk) * cv.n_kv + h) * (int64_t)(kBlock * cv.d);
}

__device__ __forceinline__ int64_t scale_offset(const CacheView& cv, int layer, int blk, int h) {
  return ((int64_t)layer * cv.n_blocks + blk) * cv.n_kv + h;
}

}  // namespace kvfa
