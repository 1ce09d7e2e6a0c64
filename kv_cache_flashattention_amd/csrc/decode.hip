// Decode attention: one query row per sequence against its paged K/V.
//
// Each workgroup sweeps one split of one sequence's context with the online
// softmax -- running max m, running sum l, output rescaled by
// exp(m_old - m_new) when the max grows ("KV Cache & Flash Attention."
// (kvcache-7e2), Flash Attention and online softmax sections; "KV Cache &
// FlashAttention" (deepforge), running-summary paragraphs) -- and gathers
// K/V through the block table (kvcache-7e2, PagedAttention section).  With
// one split the result O/l is written directly; with several, each split
// leaves (m, l, O) in the workspace and a merge kernel combines them with
// weights exp(m_s - max m), the same rescale applied across splits.
//
// Scores are kept in the base-2 domain: s2 = (q . k) * scale * log2(e), so
// exp(s - m) = exp2(s2 - m2) and the hardware exp2 is used directly.
//
// This file holds the plan and the portable VALU kernel (with its merge) used
// for f32 caches; the matrix-core path for 16-bit and fp8 caches lives in
// mfma_decode.hip.
#include <algorithm>

#include "common.h"
#include "fp8_e4m3.h"

namespace kvfa {

hipError_t launch_decode_mfma(const CacheView& cv, int layer, int n, const int32_t* seqs,
                              const void* q, void* out, float scale_log2, const DecodePlan& plan,
                              void* ws, int window, int sinks, hipStream_t s, DispatchEvents ev,
                              bool* handled);

DecodePlan make_decode_plan(const CacheView& cv, int32_t n, int32_t max_len, int32_t num_splits,
                            int32_t cu_count) {
  DecodePlan p{0, 1, 64, 0, 0};
  if (max_len <= 0 || n <= 0) return p;
  if (cv.dtype != KVC_F32) {
    // Work list: every wave of a full chip gets an equal share; with an
    // explicit num_splits, about that many pieces per (sequence, group).
    const int nb = n < kMaxBatch ? n : kMaxBatch;
    const int64_t groups = (int64_t)nb * cv.n_kv * ((cv.n_q / cv.n_kv + 15) / 16);
    int64_t waves = num_splits > 0
                        ? groups * num_splits
                        : (int64_t)std::max(cu_count, 1) * work_list_waves_per_cu(cv);
    waves = std::max<int64_t>(4, std::min<int64_t>(waves, (int64_t)1 << 24));
    p.work_list = 1;
    p.waves = (int32_t)waves;
    p.ws_bytes = work_list_ws_bytes(cv, nb, p.waves);
    return p;
  }
  // VALU splits: whole multiples of 64 tokens.
  const int64_t chunks = (max_len + 63) / 64;
  int64_t splits;
  if (num_splits > 0) {
    splits = std::min<int64_t>(num_splits, chunks);
  } else {
    const int64_t heads = (int64_t)n * cv.n_q;
    splits = std::max<int64_t>(1, std::min<int64_t>((2048 + heads - 1) / heads, chunks));
  }
  const int64_t per = (chunks + splits - 1) / splits;
  p.split_len = (int32_t)(per * 64);
  p.splits = (int32_t)((max_len + p.split_len - 1) / p.split_len);
  if (p.splits > 1)
    p.ws_bytes = (uint64_t)n * cv.n_q * p.splits * (cv.d + 2) * sizeof(float);
  return p;
}

namespace {

template <typename E> __device__ __forceinline__ float kv_to_f32(E x) { return to_f32(x); }
template <> __device__ __forceinline__ float kv_to_f32<uint8_t>(uint8_t x) { return e4m3_decode(x); }

// Workspace layout: O [n][n_q][splits][d], then m [n][n_q][splits], l [...].
struct Partials {
  float* O;
  float* m;
  float* l;
};

__device__ __forceinline__ Partials partials(void* ws, int n, int n_q, int splits, int d) {
  Partials P;
  P.O = (float*)ws;
  P.m = P.O + (int64_t)n * n_q * splits * d;
  P.l = P.m + (int64_t)n * n_q * splits;
  return P;
}

// Portable decode: one wave per (split, q head, sequence).  Lane t scores
// token c+t of each 64-token chunk (its K row read whole); the head-dimension
// columns j = lane, lane+64 of O are owned by the lanes, which read the V
// slab's [d][16] columns one block at a time.
template <typename E, typename IO, int D>
__global__ __launch_bounds__(64) void k_decode_valu(CacheView cv, int layer, const int32_t* seqs,
                                                    const IO* q, IO* out, void* ws, int n,
                                                    int splits, int split_len, float scale_log2) {
  constexpr int J = D / 64;
  __shared__ float qs[D];
  __shared__ float ps[64];
  __shared__ int blks[64];
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  const int G = cv.n_q / cv.n_kv, g = h / G;
  const int seq = seqs[b];
  const int L = valid_len(cv, seq);
  IO* orow = out + ((int64_t)b * cv.n_q + h) * D;
  if (L < 0) {
    if (splits == 1)
      for (int j = lane; j < D; j += 64) orow[j] = from_f32<IO>(__builtin_nanf(""));
    return;
  }
  const int t0 = s * split_len;
  if (t0 >= L) return;
  const int t1 = min(t0 + split_len, L);
  for (int j = lane; j < D; j += 64) qs[j] = to_f32(q[((int64_t)b * cv.n_q + h) * D + j]);
  __syncthreads();

  const bool fp8 = cv.dtype == KVC_FP8_E4M3FN;
  float m = -INFINITY, l = 0.f, o[J];
#pragma unroll
  for (int i = 0; i < J; ++i) o[i] = 0.f;

  for (int c = t0; c < t1; c += 64) {
    const int t = c + lane;
    float s2 = -INFINITY;
    int blk = -1;
    if (t < t1) {
      blk = table_block(cv, seq, t);
      if (blk < 0) {
        s2 = __builtin_nanf("");
      } else {
        const E* kr = (const E*)cv.k + slab_offset(cv, layer, blk, g) + (t % kBlock) * D;
        float acc = 0.f;
#pragma unroll 8
        for (int j = 0; j < D; ++j) acc += qs[j] * kv_to_f32(kr[j]);
        if (fp8) acc *= cv.ks[scale_offset(cv, layer, blk, g)];
        s2 = acc * scale_log2;
      }
    }
    const float cm = wave_max64(s2);
    const float m_new = fmaxf(m, cm);
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
    const float p = t < t1 ? exp2f(s2 - m_new) : 0.f;
    l = l * alpha + wave_sum64(p);
#pragma unroll
    for (int i = 0; i < J; ++i) o[i] *= alpha;
    m = m_new;
    ps[lane] = p;
    blks[lane] = blk;
    __syncthreads();
    for (int bi = 0; bi < 4 && c + bi * kBlock < t1; ++bi) {
      const int bb = blks[bi * kBlock];
      const int nslot = min(kBlock, t1 - (c + bi * kBlock));
      if (bb < 0) {
#pragma unroll
        for (int i = 0; i < J; ++i) o[i] = __builtin_nanf("");
        continue;
      }
      const E* vs = (const E*)cv.v + slab_offset(cv, layer, bb, g);
      const float vsc = fp8 ? cv.vs[scale_offset(cv, layer, bb, g)] : 1.f;
#pragma unroll
      for (int i = 0; i < J; ++i) {
        const E* col = vs + (lane + 64 * i) * kBlock;
        float acc = 0.f;
        for (int r = 0; r < nslot; ++r) acc += ps[bi * kBlock + r] * kv_to_f32(col[r]);
        o[i] += acc * vsc;
      }
    }
    __syncthreads();
  }

  if (splits == 1) {
    const float inv = 1.f / l;
#pragma unroll
    for (int i = 0; i < J; ++i) orow[lane + 64 * i] = from_f32<IO>(o[i] * inv);
  } else {
    Partials P = partials(ws, n, cv.n_q, splits, D);
    const int64_t r = ((int64_t)b * cv.n_q + h) * splits + s;
#pragma unroll
    for (int i = 0; i < J; ++i) P.O[r * D + lane + 64 * i] = o[i];
    if (lane == 0) {
      P.m[r] = m;
      P.l[r] = l;
    }
  }
}

// Merge of split partials: M = max_s m_s, w_s = exp2(m_s - M),
// out = sum_s w_s O_s / sum_s w_s l_s.  One wave per (q head, sequence);
// only the splits that hold tokens of this sequence are read.
template <typename IO, int D>
__global__ __launch_bounds__(64) void k_decode_merge(CacheView cv, const int32_t* seqs, IO* out,
                                                     const void* ws, int n, int splits,
                                                     int split_len) {
  constexpr int J = D / 64;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  IO* orow = out + ((int64_t)b * cv.n_q + h) * D;
  const int L = valid_len(cv, seqs[b]);
  if (L < 0) {
    for (int j = lane; j < D; j += 64) orow[j] = from_f32<IO>(__builtin_nanf(""));
    return;
  }
  const int ns = min(splits, (L + split_len - 1) / split_len);
  Partials P = partials((void*)ws, n, cv.n_q, splits, D);
  const int64_t r0 = ((int64_t)b * cv.n_q + h) * splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, P.m[r0 + s]);
  float den = 0.f, acc[J];
#pragma unroll
  for (int i = 0; i < J; ++i) acc[i] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2f(P.m[r0 + s] - M);
    den += w * P.l[r0 + s];
#pragma unroll
    for (int i = 0; i < J; ++i) acc[i] += w * P.O[(r0 + s) * D + lane + 64 * i];
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < J; ++i) orow[lane + 64 * i] = from_f32<IO>(acc[i] * inv);
}

template <typename E, typename IO, int D>
hipError_t run_valu(const CacheView& cv, int layer, int n, const int32_t* seqs, const void* q,
                    void* out, float scale_log2, const DecodePlan& p, void* ws, hipStream_t st,
                    DispatchEvents ev) {
  hipError_t e = launch_ev(k_decode_valu<E, IO, D>, dim3(p.splits, cv.n_q, n), dim3(64), st,
                           ev.start, p.splits == 1 || ev.main_only ? ev.stop : nullptr, cv, layer,
                           seqs, (const IO*)q, (IO*)out, ws, n, p.splits, p.split_len, scale_log2);
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_ev(k_decode_merge<IO, D>, dim3(cv.n_q, n), dim3(64), st, nullptr,
                   ev.main_only ? nullptr : ev.stop, cv, seqs, (IO*)out, (const void*)ws, n,
                   p.splits, p.split_len);
}

template <int D>
hipError_t run_valu_d(const CacheView& cv, int layer, int n, const int32_t* seqs, const void* q,
                      void* out, float sl2, const DecodePlan& p, void* ws, hipStream_t st,
                      DispatchEvents ev) {
#define KVFA_RUN(E, IO) run_valu<E, IO, D>(cv, layer, n, seqs, q, out, sl2, p, ws, st, ev)
  switch (cv.dtype) {
    case KVC_F32: return KVFA_RUN(float, float);
    case KVC_F16: return KVFA_RUN(_Float16, _Float16);
    case KVC_BF16: return KVFA_RUN(BF16, BF16);
    case KVC_FP8_E4M3FN: return KVFA_RUN(uint8_t, BF16);
    default: return hipErrorInvalidValue;                // int4 runs on the matrix cores only
  }
#undef KVFA_RUN
}

}  // namespace

hipError_t launch_decode(const CacheView& cv, int layer, int n, const int32_t* seqs,
                         const void* q, void* out, float scale, const DecodePlan& plan,
                         void* ws, int window, int sinks, const void* knew, const void* vnew,
                         hipStream_t s, DispatchEvents ev) {
  const float sl2 = scale * kLog2e;
  // The newest rows go in by the append kernel, ordered before the decode on
  // the stream.  (A decode kernel that took position L-1 from knew / vnew and
  // stored the row itself saved that launch but ran its unit loop slower:
  // 89.6 against 87.9 us per Llama-8B-shaped decode step.)
  if (knew != nullptr) {
    hipError_t e = launch_append(cv, layer, n, seqs, knew, vnew, s,
                                 ev.main_only ? nullptr : ev.start);
    if (e != hipSuccess) return e;
    if (!ev.main_only) ev.start = nullptr;              // the append kernel opened the call
  }
  bool handled = false;
  hipError_t e = launch_decode_mfma(cv, layer, n, seqs, q, out, sl2, plan, ws, window, sinks, s,
                                    ev, &handled);
  if (handled) return e;
  if (window > 0) return hipErrorInvalidValue;          // the VALU kernel has no window
  if (cv.d == 128) return run_valu_d<128>(cv, layer, n, seqs, q, out, sl2, plan, ws, s, ev);
  return run_valu_d<64>(cv, layer, n, seqs, q, out, sl2, plan, ws, s, ev);
}

}  // namespace kvfa
