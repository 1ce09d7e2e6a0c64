// Causal prefill attention over whole prompts.
//
// The prompt's queries are cut into row tiles and its keys/values into
// column tiles; each query row keeps (m, l, O) while the key tiles stream
// through on-chip memory, and only O/l is written back ("KV Cache & Flash
// Attention." (kvcache-7e2), Flash Attention section; "KV Cache &
// FlashAttention" (deepforge): the score table is never stored).  Query t
// sees keys 0..t.
//
// This file holds the portable VALU kernel (f32 and any shape the
// matrix-core kernel does not cover) and the dispatch.
#include "common.h"

namespace kvfa {

hipError_t launch_prefill_mfma(const CacheView& cv, int n, int T, const void* q, const void* k,
                               const void* v, void* out, float scale_log2, int window, int sinks,
                               hipStream_t s, DispatchEvents ev, bool* handled);
hipError_t launch_extend_mfma(const CacheView& cv, int layer, int n, const int32_t* seqs, int T,
                              const void* q, void* out, float scale_log2, int window, int sinks,
                              hipStream_t s, DispatchEvents ev, bool* handled);

namespace {

constexpr int kKeyTile = 32;

// One wave per (64-query tile, q head, sequence); lane i owns query row
// tile*64 + i with its q and O in registers.  Key/value tiles of 32 rows are
// staged in LDS as float and read by all lanes (broadcast reads).
template <typename IO, int D>
__global__ __launch_bounds__(64) void k_prefill_valu(int n_q, int n_kv, int T, const IO* q,
                                                     const IO* k, const IO* v, IO* out,
                                                     float scale_log2) {
  __shared__ float ks[kKeyTile][D];
  __shared__ float vs[kKeyTile][D];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int g = h / (n_q / n_kv);
  const int t = tile * 64 + lane;
  const bool row_ok = t < T;
  float qr[D], o[D];
  const IO* qrow = q + (((int64_t)b * T + (row_ok ? t : 0)) * n_q + h) * D;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    qr[j] = to_f32(qrow[j]);
    o[j] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int last = min(T - 1, tile * 64 + 63);               // last key any row of the tile sees
  for (int j0 = 0; j0 <= last; j0 += kKeyTile) {
    for (int i = lane; i < kKeyTile * D; i += 64) {
      const int jj = i / D, c = i % D, key = j0 + jj;
      float kk = 0.f, vv = 0.f;
      if (key < T) {
        const int64_t src = (((int64_t)b * T + key) * n_kv + g) * D + c;
        kk = to_f32(k[src]);
        vv = to_f32(v[src]);
      }
      ks[jj][c] = kk;
      vs[jj][c] = vv;
    }
    __syncthreads();
    float s2[kKeyTile];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kKeyTile; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc += qr[c] * ks[jj][c];
      const int key = j0 + jj;
      s2[jj] = (key <= t && key < T) ? acc * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s2[jj]);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new != -INFINITY) {                               // some key of the tile is visible
      const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
      float psum = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kKeyTile; ++jj) {
        const float p = exp2f(s2[jj] - m_new);
        psum += p;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] += p * vs[jj][c];
      }
      l = l * alpha + psum;
      m = m_new;
    }
    __syncthreads();
  }
  if (row_ok) {
    IO* orow = out + (((int64_t)b * T + t) * n_q + h) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) orow[c] = from_f32<IO>(o[c] * inv);
  }
}

template <typename IO>
hipError_t run_valu(const CacheView& cv, int n, int T, const void* q, const void* k,
                    const void* v, void* out, float sl2, hipStream_t s, DispatchEvents ev) {
  dim3 grid((T + 63) / 64, cv.n_q, n);
  if (cv.d == 128)
    return launch_ev(k_prefill_valu<IO, 128>, grid, dim3(64), s, ev.start, ev.stop, cv.n_q,
                     cv.n_kv, T, (const IO*)q, (const IO*)k, (const IO*)v, (IO*)out, sl2);
  return launch_ev(k_prefill_valu<IO, 64>, grid, dim3(64), s, ev.start, ev.stop, cv.n_q, cv.n_kv,
                   T, (const IO*)q, (const IO*)k, (const IO*)v, (IO*)out, sl2);
}

}  // namespace

hipError_t launch_prefill(const CacheView& cv, int n, int T, const void* q, const void* k,
                          const void* v, void* out, float scale, int window, int sinks,
                          hipStream_t s, DispatchEvents ev) {
  const float sl2 = scale * kLog2e;
  bool handled = false;
  hipError_t e = launch_prefill_mfma(cv, n, T, q, k, v, out, sl2, window, sinks, s, ev, &handled);
  if (handled) return e;
  if (window > 0) return hipErrorInvalidValue;          // the VALU kernel has no window
  switch (io_dtype(cv.dtype)) {
    case KVC_F32: return run_valu<float>(cv, n, T, q, k, v, out, sl2, s, ev);
    case KVC_F16: return run_valu<_Float16>(cv, n, T, q, k, v, out, sl2, s, ev);
    default: return run_valu<BF16>(cv, n, T, q, k, v, out, sl2, s, ev);
  }
}

hipError_t launch_extend(const CacheView& cv, int layer, int n, const int32_t* seqs, int T,
                         const void* q, void* out, float scale, int window, int sinks,
                         hipStream_t s, bool* handled, DispatchEvents ev) {
  return launch_extend_mfma(cv, layer, n, seqs, T, q, out, scale * kLog2e, window, sinks, s, ev,
                            handled);
}

}  // namespace kvfa
