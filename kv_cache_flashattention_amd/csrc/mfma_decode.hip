// Decode attention on the matrix cores (bf16 / fp16 / fp8 / int4 caches, d 64
// or 128).
//
// Work list.  The unit of work is 32 tokens (two 16-token blocks) of one
// (sequence, kv-head group) segment, where a group is up to 16 query heads
// sharing one kv head, so each K/V byte is read once for the whole query
// group (grouped-query attention, "KV Cache & Flash Attention." (kvcache-7e2)
// memory-cost section).  Every workgroup first turns the batch's lengths into
// prefix sums of unit counts (in LDS); the W units of the batch are then cut
// into `waves` equal contiguous ranges, one per wave, whatever the mix of
// lengths.  A wave sweeps its range segment piece by segment piece; per unit
// it
//   1. computes S^T = K Q^T with 16x16x32 MFMAs: the 16 M-rows are tokens,
//      the 16 N-columns are the query rows (padded with zeros), K = head dim;
//   2. updates the running max m and sum l of each query row and rescales
//      its output by exp(m_old - m_new) (kvcache-7e2, online softmax
//      section), all in fp32;
//   3. computes O^T += V^T P^T with MFMAs over the unit's 32 tokens.
// Units are double-buffered in registers: the next unit's K/V loads are
// issued before the current unit is computed, so a wave keeps HBM reads in
// flight while it computes.  At the end of each piece the wave writes its
// (m, l, O) to workspace slot (segment + wave), so the pieces of a segment
// occupy consecutive slots; a merge kernel combines them with weights
// exp(m_s - max m) -- the online softmax's rescale applied across pieces --
// and writes O / l.
//
// Operand placement.  A 16x16x32 MFMA lane l holds, for its operand, row (or
// column) l % 16 and a group of 8 reduction indices chosen by l / 16; the
// reduction indices may be assigned in any order as long as both operands
// agree.  K slabs are [16][d], so a lane loads 16 bytes of one token's row
// for QK^T.  For PV the reduction runs over tokens, and the V slabs are
// [d][16], so a lane loads 8 consecutive tokens of one head-dimension column.
// Which token each S^T row holds is chosen so that the probabilities a lane
// ends up with are exactly the tokens its V operand covers: no data moves
// between lanes except the row max/sum.
//
// fp8: codes are widened to bf16 exactly (every E4M3FN value is a bf16
// value); the block's K scale multiplies its scores and its V scale the
// probabilities before they are rounded to bf16; the running sum l uses the
// unscaled probabilities.
//
// int4: a dword of 8 codes becomes 8 bf16 operands with two bit operations
// per pair: the sign bit of every nibble is flipped (offset binary, n = c + 8)
// and each nibble is placed in the low mantissa bits of 128.0, giving the
// exact bf16 value c + 136.  The operands therefore carry a constant offset
// of 136, removed after the products: the scores lose 136 * sum(q) (per
// query row, computed once per segment) and the output loses 136 * sum of
// the rounded probabilities fed to the PV products (accumulated beside O
// with the same rescaling).  The conversion pairs nibbles k and k+4, so the
// reduction indices come in the order 0,4,1,5,2,6,3,7; the query operand and
// the probability operand are permuted to match.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace kvfa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

enum { KV_BF16 = 0, KV_F16 = 1, KV_FP8 = 2, KV_INT4 = 3 };

// K/V loads.  Every cached byte is read exactly once per call, so the loads
// carry the non-temporal hint: the stream is not kept in L2 or the Infinity
// Cache, where it would only displace lines that are reused (queries, block
// tables, partials).  The Llama-8B-, 70B- and 128,000-token-shaped calls run
// 9-10 % faster with it (same-box A/B, bit-identical outputs).
typedef __attribute__((ext_vector_type(4))) uint32_t ntu4;
typedef __attribute__((ext_vector_type(2))) uint32_t ntu2;
__device__ __forceinline__ uint4 ld_stream4(const void* p) {
  const ntu4 v = __builtin_nontemporal_load((const ntu4*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_stream2(const void* p) {
  const ntu2 v = __builtin_nontemporal_load((const ntu2*)p);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t ld_stream1(const void* p) {
  return __builtin_nontemporal_load((const uint32_t*)p);
}

template <int KV> struct Op { typedef bf16x8 T; };
template <> struct Op<KV_F16> { typedef f16x8 T; };

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 fp8 codes (two dwords) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 int4 codes (code k in nibble k of x, two's complement) -> 8 bf16 holding
// code + 136 exactly, in the order of codes 0,4,1,5,2,6,3,7.
constexpr float kInt4Offset = 136.0f;
// The sign flip and the exponent bits are one XOR with 0x4308 per half
// (bits disjoint from the masked nibble except bit 3, which it flips), so a
// pair costs a shift and one three-input bit operation.
__device__ __forceinline__ bf16x8 int4x8_to_bf16_off(uint32_t x) {
  const uint32_t m = 0x000F000Fu, e = 0x43084308u;
  uint4 r;
  r.x = (x & m) ^ e;
  r.y = ((x >> 4) & m) ^ e;
  r.z = ((x >> 8) & m) ^ e;
  r.w = ((x >> 12) & m) ^ e;
  return __builtin_bit_cast(bf16x8, r);
}
// Dword i of a uint4 (i a compile-time constant after unrolling).
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
// 8 bf16 (a dword per pair, value k at half k) reordered to 0,4,1,5,2,6,3,7.
__device__ __forceinline__ uint4 interleave_halves(uint4 a) {
  return make_uint4((a.x & 0xFFFFu) | (a.z << 16), (a.x >> 16) | (a.z & 0xFFFF0000u),
                    (a.y & 0xFFFFu) | (a.w << 16), (a.y >> 16) | (a.w & 0xFFFF0000u));
}
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float sum8_bf16(bf16x8 a) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x2 t = {a[2 * j], a[2 * j + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(t, one, s, false);
  }
  return s;
}

template <typename T> __device__ __forceinline__ T pack8(const float* p);
template <> __device__ __forceinline__ bf16x8 pack8<bf16x8>(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)p[j];
  return r;
}
template <> __device__ __forceinline__ f16x8 pack8<f16x8>(const float* p) {
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (_Float16)p[j];
  return r;
}

// Head-dimension offset of the 8 reduction indices of k-step ks, lane group g.
// 16-bit data: 8 consecutive values per k-step.  fp8: one 16-byte load covers
// k-steps 2a and 2a+1.  int4: one load of D/8 bytes covers every k-step
// (dword ks of it), so lane group g holds dims D/4*g .. D/4*g + D/4 - 1.
template <int KV, int D> __device__ __forceinline__ int dmap(int ks, int g) {
  if (KV == KV_INT4) return (D / 4) * g + 8 * ks;
  if (KV == KV_FP8) return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1);
  return 32 * ks + 8 * g;
}

// Token of a 32-token unit held by row r of S^T tile t (t = 0, 1): block
// r >> 3 and slot 8*((r >> 2) & 1) + 4t + (r & 3).  After the MFMA, lane
// group g holds rows 4g..4g+3 of both tiles, i.e. block g >> 1, slots
// 8*(g & 1) + 4t + i: exactly the 8 consecutive slots its PV operand covers
// (slot j = 4t + i of the k-step).
__device__ __forceinline__ int tok_block(int r) { return r >> 3; }
__device__ __forceinline__ int tok_slot(int t, int r) { return 8 * ((r >> 2) & 1) + 4 * t + (r & 3); }

// One unit's loaded K/V operands (registers).
template <int KV, int D> struct Unit {
  static constexpr int KS = D / 32;                    // k-steps of QK^T
  static constexpr int DT = D / 16;                    // 16-row tiles of O^T
  // 16-byte K loads per tile (int4: one load of D/8 bytes)
  static constexpr int KL = KV == KV_FP8 ? KS / 2 : KV == KV_INT4 ? 1 : KS;
  // V registers: fp8 two 8-byte loads per uint4, int4 four 4-byte loads
  static constexpr int VL = KV == KV_FP8 ? DT / 2 : KV == KV_INT4 ? DT / 4 : DT;
  uint4 k[2][KL];
  uint4 v[VL];
  float ksc, vsc;                                      // fp8/int4: this lane's block scales
  int sj;                                              // the lane's slot in its table chunk
};

// Units a wave keeps loaded (ring depth).  Deeper rings cost registers and
// with them resident waves; on the 70B-shaped workloads a depth of 3 gained
// nothing for fp8 and int4 and a depth of 4 lost 14% for int4.
template <int KV> struct DecodeDepth { static constexpr int value = 2; };

// Workspace of one (sub-)batch: O [slots][16][D] f32, m [slots][16],
// l [slots][16], then the batch's unit prefix sums [nb+1] (int64) and unit
// counts [nb] (int32) for the merge.
struct WorkWs {
  float* O;
  float* m;
  float* l;
  int64_t* units;
  int32_t* counts;
};

constexpr int kUnit = 32;   // tokens per work unit
constexpr int kTabUnits = 32;   // units per block-table chunk (64 lanes, two blocks each)
constexpr float kStale = 8.0f;   // lazy-rescale threshold of the running max (log2 units)

// Units of one segment that a query at position L-1 can see.  Without a
// window: all ceil(L/32) units.  With a window w: the units holding sink
// positions 0 .. sinks-1, then the units from the one holding position L-w
// on; when the two ranges meet, all units.  unit(i) maps the segment's i-th
// visible unit to its unit index in the sequence.
struct UnitMap {
  int count, ns, gap;
  __device__ UnitMap(int L, int window, int sinks) {
    const int nu = (L + kUnit - 1) / kUnit;
    count = nu, ns = nu, gap = 0;
    if (window > 0 && L > window) {
      const int w0 = (L - window) / kUnit;
      const int s1 = (min(sinks, L) + kUnit - 1) / kUnit;
      if (w0 > s1) {
        ns = s1;
        gap = w0 - s1;
        count = nu - gap;
      }
    }
  }
  __device__ int unit(int i) const { return i < ns ? i : i + gap; }
};

__host__ __device__ inline int64_t work_slots(int nb, int nkvg, int waves) {
  return (int64_t)nb * nkvg + waves;
}

__device__ __forceinline__ WorkWs work_ws(void* ws, int64_t slots, int D, int nb) {
  WorkWs w;
  w.O = (float*)ws;
  w.m = w.O + slots * 16 * D;
  w.l = w.m + slots * 16;
  w.units = (int64_t*)(w.l + slots * 16);   // slots*16*(D+2) floats: 8-byte aligned
  w.counts = (int32_t*)(w.units + nb + 1);
  return w;
}

// Wave-uniform values read from LDS or memory, moved to scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// floor(a * W / P) without overflow: W = qP + r.
__device__ __forceinline__ int64_t share(int64_t a, int64_t W, int64_t P) {
  if ((W >> 31) == 0 && (P >> 16) == 0) {              // the common sizes: 32-bit divisions
    const uint32_t w = (uint32_t)W, p = (uint32_t)P, x = (uint32_t)a;
    return (int64_t)(x * (w / p) + (x * (w % p)) / p);
  }
  return a * (W / P) + (a * (W % P)) / P;
}


template <int KV, int D>
__global__ __launch_bounds__(256, 2) void k_decode_work(CacheView cv, int layer,
                                                        const int32_t* seqs, const uint16_t* q,
                                                        void* ws, int nb, int qgroups, int waves,
                                                        float sl2, int window, int sinks) {
  typedef typename Op<KV>::T OpT;
  typedef Unit<KV, D> U;
  constexpr int KS = U::KS, DT = U::DT, KL = U::KL;
  constexpr int NB = DecodeDepth<KV>::value;
  static_assert(NB == 2, "the block-scale shuffles assume one unit in flight");
  constexpr int EB = KV == KV_FP8 ? 1 : 2;            // bytes per element (not int4)
  constexpr int64_t SB = KV == KV_INT4 ? kBlock * D / 2 : kBlock * D * EB;   // slab bytes
  __shared__ int64_t s_units[kMaxBatch + 1];
  __shared__ int32_t s_counts[kMaxBatch];
  __shared__ int32_t s_seq[kMaxBatch], s_len[kMaxBatch];   // each entry's sequence and length
  // batches of at most 64 entries: each wave's own copy of the four arrays
  __shared__ int64_t w_units[4][65];
  __shared__ int32_t w_counts[4][64], w_seq[4][64], w_len[4][64];
  __shared__ int64_t s_wsum[4];
  constexpr int kLenCache = 4096;
  __shared__ int32_t s_lenall[kLenCache];               // every sequence's length (small caches)

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int G = cv.n_q / cv.n_kv;
  const int nkvg = cv.n_kv * qgroups;
  const int64_t slots = work_slots(nb, nkvg, waves);
  WorkWs W_ = work_ws(ws, slots, D, nb);

  // ---- unit counts and their prefix sums: up to 8 contiguous entries per
  // thread (nb <= 2048), one per thread when nb <= 256 so that no wave works
  // through the entries alone.  Batches of at most 64 entries are scanned by
  // every wave on its own (lane b: entry b) into its own copy of the arrays,
  // which takes no barrier after the lengths are in.  The batch's sequence
  // ids and, when the cache has at most kLenCache sequences, all of their
  // lengths are loaded together, so the lengths do not wait for the ids.
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool small = nb <= 64;                           // the same for every wave
  int64_t* const su = small ? w_units[wv] : s_units;
  int32_t* const sc = small ? w_counts[wv] : s_counts;
  int32_t* const ss = small ? w_seq[wv] : s_seq;
  int32_t* const sl = small ? w_len[wv] : s_len;
  {
    const bool lens_in_lds = cv.max_seqs <= kLenCache;
    const int per = nb <= 256 ? 1 : 8;                   // wave-uniform
    const int first = small ? lane : tid * per;          // this thread's first entry
    int sqv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int b = first + i;
      sqv[i] = i < per && b < nb ? seqs[b] : -1;
    }
    if (lens_in_lds)
      for (int i = tid; i < cv.max_seqs; i += 256) s_lenall[i] = cv.len[i];
    __syncthreads();
    int64_t loc[8], tsum = 0;
    int lv[8];                                          // LDS lengths, read before any branch
#pragma unroll
    for (int i = 0; i < 8; ++i)
      lv[i] = lens_in_lds ? s_lenall[sqv[i] >= 0 && sqv[i] < cv.max_seqs ? sqv[i] : 0] : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int b = first + i;
      int c = 0;
      if (i < per && b < nb) {
        const int sq = sqv[i];
        int L;
        if (lens_in_lds) {
          L = sq >= 0 && sq < cv.max_seqs ? lv[i] : -1;
          if (L <= 0 || L > cv.max_bps * kBlock) L = -1;
        } else {
          L = valid_len(cv, sq);
        }
        c = L > 0 ? UnitMap(L, window, sinks).count : 0;
        sc[b] = c;
        ss[b] = sq;
        sl[b] = L;
      }
      loc[i] = (int64_t)c * nkvg;
      tsum += loc[i];
    }
    // inclusive scan of the threads' sums over the wave: 32-bit when the
    // batch's unit count is bounded below 2^31 (each segment holds at most
    // max_bps / 2 + 1 units)
    int64_t x = tsum;
    if ((int64_t)nb * (cv.max_bps / 2 + 1) * nkvg < (1ll << 31)) {
      int32_t x32 = (int32_t)tsum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x32, o, 64);
        if (lane >= o) x32 += y;
      }
      x = x32;
    } else {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
    }
    if (small) {
      // lanes nb.. hold no units: lane 63 holds the batch's total
      const int64_t ex = x - tsum;
      const int64_t total = uni64(__shfl(x, 63, 64));
      if (lane < nb) su[lane] = ex;
      if (lane == 0) su[nb] = total;
      if (blockIdx.x == 0 && wv == 0) {
        if (lane < nb) {
          W_.units[lane] = ex;
          W_.counts[lane] = sc[lane];
        }
        if (lane == 0) W_.units[nb] = total;
      }
    } else {
      if (lane == 63) s_wsum[tid >> 6] = x;
      __syncthreads();
      int64_t ex = x - tsum;
      for (int i = 0; i < (tid >> 6); ++i) ex += s_wsum[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int b = tid * per + i;
        if (i < per && b < nb) s_units[b] = ex;
        ex += loc[i];
      }
      if (tid == 0) s_units[nb] = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
      __syncthreads();
      if (blockIdx.x == 0) {
        for (int b = tid; b <= nb; b += 256) W_.units[b] = s_units[b];
        for (int b = tid; b < nb; b += 256) W_.counts[b] = s_counts[b];
      }
    }
  }

  const int gw = blockIdx.x * 4 + wv;
  const int64_t Wt = su[nb];
  if (gw >= waves || Wt == 0) return;
  int64_t u = share(gw, Wt, waves);
  const int64_t u1 = share(gw + 1, Wt, waves);

  // entry holding unit u: the last b with su[b] <= u (entries without
  // units share their offset with the next entry and are skipped this way).
  // The offsets do not decrease, so the entries at or below u are a prefix:
  // count them 64 at a time with one LDS read and a ballot per chunk.
  int b = 0;
  {
    int k = 0;
    for (int c0 = 0; c0 < nb; c0 += 64) {              // wave-uniform
      const int e = c0 + lane;
      const uint64_t m = __builtin_amdgcn_ballot_w64(e < nb && su[e < nb ? e : 0] <= u);
      k += __builtin_popcountll(m);
      if (m != ~0ull) break;
    }
    b = uni(k - 1);                                     // su[0] = 0 <= u: k >= 1
  }

  const uint8_t* kpool = (const uint8_t*)cv.k;
  const uint8_t* vpool = (const uint8_t*)cv.v;
  const int64_t layer_blocks = (int64_t)layer * cv.n_blocks;

  while (u < u1) {
    while (uni64(su[b + 1]) <= u) ++b;                // skip to the entry holding u
    const int cb = uni(sc[b]);
    const int64_t sb = uni64(su[b]);
    const int64_t rem = u - sb;
    int kvg, c0;
    if ((rem >> 31) == 0) {                             // the common sizes: 32-bit division
      kvg = (int)((uint32_t)rem / (uint32_t)cb);
      c0 = (int)((uint32_t)rem - (uint32_t)kvg * (uint32_t)cb);
    } else {
      kvg = (int)(rem / cb);
      c0 = (int)(rem % cb);
    }
    const int64_t segend = sb + (int64_t)(kvg + 1) * cb;
    const int64_t pend = u1 < segend ? u1 : segend;
    const int c1 = c0 + (int)(pend - u);
    const int kvh = kvg / qgroups, qg = kvg % qgroups;
    const int seq = uni(ss[b]);
    const int L = uni(sl[b]);                          // > 0: the entry has units
    const UnitMap umap(L, window, sinks);
    // Query operand (B of S^T = K Q^T): column r16 = query row qg*16 + r16,
    // loaded after the piece's first block-table load (below).
    const int qi = qg * 16 + r16;
    const bool qrow = qi < G;
    OpT qop[KS];
    float qoff = 0.f;                                 // int4: -136 * sum of the query row
    f32x4 o[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, lpart = 0.f;
    float pvs = 0.f;                                  // int4: sum of the PV probabilities
    bool bad = false;
    const int32_t* btrow = cv.bt + (int64_t)seq * cv.max_bps;
    const int last_blk = (L - 1) / kBlock;

    // Block table of the piece, 32 units at a time: lane l holds the block of
    // unit tab0 + l/2, slot l&1 (entries past the sequence's end clamped to
    // its last block, whose extra tokens are masked), and for fp8/int4 that
    // block's scales.  Units then read their block ids with readlane, so the
    // data loads do not wait on a table load and addresses are scalar.
    constexpr bool SCALED = KV == KV_FP8 || KV == KV_INT4;
    int tab = 0, tab0 = c0;
    float tks = 1.f, tvs = 1.f;
    auto load_tab = [&](int cs0) {
      tab0 = cs0;
      const int cs = cs0 + (lane >> 1);
      int x = 0;
      if (cs < c1) {
        x = btrow[min(2 * umap.unit(cs) + (lane & 1), last_blk)];
        if (x < 0 || x >= cv.n_blocks) {
          bad = true;
          x = -1;
        }
      }
      tab = x;
      if constexpr (SCALED) {
        const int64_t si = (layer_blocks + max(x, 0)) * cv.n_kv + kvh;
        tks = cv.ks[si];
        tvs = cv.vs[si];
      }
    };
    load_tab(c0);
    {
      const uint16_t* qr = q + ((int64_t)b * cv.n_q + kvh * G + (qrow ? qi : 0)) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 raw = qrow ? *(const uint4*)(qr + dmap<KV, D>(ks, g)) : make_uint4(0, 0, 0, 0);
        if (KV == KV_INT4) raw = interleave_halves(raw);
        qop[ks] = __builtin_bit_cast(OpT, raw);
      }
    }


    // Issue every load of unit cs into buffer B.
    auto issue = [&](U& B, int cs) {
      if (cs - tab0 >= kTabUnits) load_tab(cs);       // wave-uniform
      const int j = 2 * (cs - tab0);
      int64_t sbase[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int x = max(__builtin_amdgcn_readlane(tab, j + i), 0);   // invalid: NaN rows later
        sbase[i] = ((layer_blocks + x) * cv.n_kv + kvh) * SB;
      }
      const uint8_t* krow = kpool + (tok_block(r16) ? sbase[1] : sbase[0]);
      if constexpr (KV == KV_INT4) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint8_t* kp = krow + tok_slot(t, r16) * (D / 2) + (D / 8) * g;
          if (D == 128) {
            B.k[t][0] = ld_stream4(kp);
          } else {
            const uint2 x = ld_stream2(kp);
            B.k[t][0] = make_uint4(x.x, x.y, 0u, 0u);
          }
        }
        // V column j = 16 dt + r16: tokens 8 (g & 1) .. +7 of block g >> 1
        // are the dword at byte 4 (g & 1) of the column's 8 bytes.
        const uint8_t* vcol = vpool + ((g >> 1) ? sbase[1] : sbase[0]) + 4 * (g & 1);
        uint32_t w[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) w[dt] = ld_stream1(vcol + (16 * dt + r16) * 8);
#pragma unroll
        for (int i = 0; i < DT / 4; ++i)
          B.v[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint8_t* rp = krow + (int64_t)tok_slot(t, r16) * D * EB;
#pragma unroll
          for (int a = 0; a < KL; ++a) {
            const int off = KV == KV_FP8 ? 64 * a + 16 * g : 2 * dmap<KV, D>(a, g);
            B.k[t][a] = ld_stream4(rp + off);
          }
        }
        const uint8_t* vslab = vpool + ((g >> 1) ? sbase[1] : sbase[0]) + 8 * (g & 1) * EB;
        if constexpr (KV == KV_FP8) {
#pragma unroll
          for (int dt = 0; dt < DT; dt += 2) {
            const uint2 lo = ld_stream2(vslab + (16 * dt + r16) * kBlock);
            const uint2 hi = ld_stream2(vslab + (16 * (dt + 1) + r16) * kBlock);
            B.v[dt / 2] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            B.v[dt] = ld_stream4(vslab + 2 * (16 * dt + r16) * kBlock);
        }
      }
      B.sj = j + (g >> 1);                            // this lane's block: table lane
    };
    // The unit's block scales, read from the table chunk it was issued from:
    // called before the next issue, which may load the next chunk.  Their
    // loads are then older than the unit's own K/V loads, so the shuffles do
    // not wait on the loads in flight.
    auto scales = [&](U& B) {
      if constexpr (SCALED) {
        B.ksc = __shfl(tks, B.sj, 64);
        B.vsc = __shfl(tvs, B.sj, 64);
      }
    };

    // Fold unit c (loaded in B) into (m, l, O).
    auto compute = [&](const U& B, int cs) {
      const int c = umap.unit(cs);
      const int nvalid = min(kUnit, L - c * kUnit);
      const bool tail = nvalid < kUnit;
      // window: positions before L - window that are not sinks are hidden
      const int wlo = window > 0 ? L - window : 0;
      const bool wedge = c * kUnit < wlo && c * kUnit + kUnit > sinks;
      // ---- S^T = K Q^T, two 16-token tiles
      f32x4 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int a = 0; a < KL; ++a) {
          if constexpr (KV == KV_INT4) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              sacc[t] = mfma(int4x8_to_bf16_off(word(B.k[t][0], ks)), qop[ks], sacc[t]);
          } else if constexpr (KV == KV_FP8) {
            sacc[t] = mfma(__builtin_bit_cast(OpT, fp8x8_to_bf16(B.k[t][a].x, B.k[t][a].y)),
                           qop[2 * a], sacc[t]);
            sacc[t] = mfma(__builtin_bit_cast(OpT, fp8x8_to_bf16(B.k[t][a].z, B.k[t][a].w)),
                           qop[2 * a + 1], sacc[t]);
          } else {
            sacc[t] = mfma(__builtin_bit_cast(OpT, B.k[t][a]), qop[a], sacc[t]);
          }
        }
      }
      // ---- online softmax (this lane's S^T column: query r16; its values
      // are tokens 16*(g>>1) + 8*(g&1) + 4t + i of the unit)
      float ksc = 1.f, vsc = 1.f;
      if constexpr (SCALED) {
        ksc = B.ksc;
        vsc = B.vsc;
      }
      const int pos0 = 16 * (g >> 1) + 8 * (g & 1);
      // A score enters the exponent as p = s a + b, with a = scale log2(e)
      // times the block's K scale (kept above zero, so that a hidden
      // position's -inf stays -inf) and b the int4 offset term.  a and b
      // belong to the lane's block, so within the lane the map is increasing:
      // the lane's max is taken on the raw scores s and mapped once, the
      // lanes' maxima are combined, and exp2(p - m) is exp2(fma(s, a, b - m)).
      const float a = vmax(sl2 * ksc, 1e-30f);        // (a NaN scale stays NaN)
      const float b = KV == KV_INT4 ? qoff * a : 0.f;
      float sc[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[t][i] = sacc[t][i];
      if (tail || wedge) {                            // wave-uniform: masked units only
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = c * kUnit + pos0 + 4 * t + i;
            if (pos0 + 4 * t + i >= nvalid || (pos < wlo && pos >= sinks)) sc[t][i] = -INFINITY;
          }
      }
      // (maximum, not fmaxf: no canonicalising of the selected values)
      const float smax = vmax(vmax(vmax(sc[0][0], sc[0][1]), vmax(sc[0][2], sc[0][3])),
                              vmax(vmax(sc[1][0], sc[1][1]), vmax(sc[1][2], sc[1][3])));
      float cmax = fmaf(smax, a, b);
      cmax = vmax(cmax, __shfl_xor(cmax, 16, 64));
      cmax = vmax(cmax, __shfl_xor(cmax, 32, 64));
      // Lazy rescale: the running max m moves only when a row's new max
      // exceeds it by more than kStale (log2 units), so most units skip the
      // rescale of O; probabilities stay below 2^kStale.  (m, l, O) remain a
      // consistent triple for the merge whatever m is.
      // (written so that a NaN max -- NaN scores or scales -- also takes the
      // branch and makes m NaN: the merge then propagates it instead of
      // taking the piece for an empty one)
      if (__any(!(cmax <= m + kStale))) {
        const float m_new = vmax(m, cmax);
        const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        lpart *= alpha;
        pvs *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i) o[i] *= alpha;
      }
      const float bm = b - m;
      float psum = 0.f, pv[8];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sc[t][i], a, bm));
          psum += e;
          pv[4 * t + i] = e * vsc;
        }
      lpart += psum;
      // ---- O^T += V^T P^T over the unit's 32 tokens; in a sequence's last
      // unit, V slots past its end are zeroed (they may hold stale or
      // poisoned bytes, and 0 * NaN would poison O).  int4 codes are always
      // finite, so there the zero probabilities suffice.
      if constexpr (KV == KV_INT4) {
        const float pvp[8] = {pv[0], pv[4], pv[1], pv[5], pv[2], pv[6], pv[3], pv[7]};
        const bf16x8 pop = pack8<bf16x8>(pvp);
        pvs += sum8_bf16(pop);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          o[dt] = mfma(int4x8_to_bf16_off(word(B.v[dt / 4], dt & 3)), pop, o[dt]);
      } else {
        const OpT pop = pack8<OpT>(pv);
        const int nok = tail ? nvalid - pos0 : 8;       // valid slots among the lane's 8
        uint32_t keep[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (KV == KV_FP8) {
            uint32_t mk = 0;
#pragma unroll
            for (int y = 0; y < 4; ++y) mk |= ((4 * (e & 1) + y) < nok ? 0xFFu : 0u) << (8 * y);
            keep[e] = mk;
          } else {
            keep[e] = (2 * e < nok ? 0xFFFFu : 0u) | (2 * e + 1 < nok ? 0xFFFF0000u : 0u);
          }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          OpT vop;
          if constexpr (KV == KV_FP8) {
            const uint4 w4 = B.v[dt / 2];
            const uint32_t lo = ((dt & 1) ? w4.z : w4.x) & keep[0];
            const uint32_t hi = ((dt & 1) ? w4.w : w4.y) & keep[1];
            vop = __builtin_bit_cast(OpT, fp8x8_to_bf16(lo, hi));
          } else {
            const uint4 raw = B.v[dt];
            vop = __builtin_bit_cast(OpT, make_uint4(raw.x & keep[0], raw.y & keep[1],
                                                     raw.z & keep[2], raw.w & keep[3]));
          }
          o[dt] = mfma(vop, pop, o[dt]);
        }
      }
    };

    // NB register buffers in a ring: the loads of unit c+NB-1 go out before
    // unit c is computed, so NB-1 units are in flight while the wave computes.
    U buf[NB];
    issue(buf[0], c0);
    // The query rows were loaded before the first unit's loads: wait for them
    // here, once, so that the unit loop below never waits on them (and with
    // them on every load issued since).
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ntu4 x = __builtin_bit_cast(ntu4, qop[ks]);
      asm volatile("" : "+v"(x));
      qop[ks] = __builtin_bit_cast(OpT, x);
    }
    // int4: -136 * sum of the query row's values (the K operands' offset)
    if (KV == KV_INT4) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qoff += sum8_bf16(__builtin_bit_cast(bf16x8, qop[ks]));
      qoff += __shfl_xor(qoff, 16, 64);
      qoff += __shfl_xor(qoff, 32, 64);
      qoff *= -kInt4Offset;
    }
    // Two units per step with no conditions in the steady state, so that the
    // compiler's wait counts see one fixed order of loads: unit c+1's loads
    // go out while unit c is computed.  A piece holds at least one unit.
    int c = c0;
    for (; c + 2 < c1; c += 2) {
      scales(buf[0]);
      issue(buf[1], c + 1);
      compute(buf[0], c);
      scales(buf[1]);
      issue(buf[0], c + 2);
      compute(buf[1], c + 1);
    }
    scales(buf[0]);
    if (c + 1 < c1) {
      issue(buf[1], c + 1);
      compute(buf[0], c);
      scales(buf[1]);
      compute(buf[1], c + 1);
    } else {
      compute(buf[0], c);
    }

    // ---- piece done: (m, l, O) of this wave's query rows to slot (segment + wave)
    float l = lpart + __shfl_xor(lpart, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if constexpr (KV == KV_INT4) {                   // remove the V operands' offset
      float ps = pvs + __shfl_xor(pvs, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[dt][i] = fmaf(-kInt4Offset, ps, o[dt][i]);
    }
    if (__any(bad)) l = __builtin_nanf("");
    const int64_t slot = (int64_t)b * nkvg + kvg + gw;
    if (qrow) {
      float* Orow = W_.O + (slot * 16 + r16) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *(float4*)(Orow + 16 * dt + 4 * g) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (g == 0) {
        W_.m[slot * 16 + r16] = m;
        W_.l[slot * 16 + r16] = l;
      }
    }
    u = pend;
  }
}

// Merge of the pieces of every (sequence, query head): the pieces of segment
// s are in slots s + w for the waves w whose ranges meet the segment.
// M = max m, weights exp2(m - M), out = sum w O / sum w l.  One workgroup of
// four waves per (query head, sequence): each wave folds every fourth piece
// into its own running (M, den, acc) -- the same online rescale, four pieces
// per step so their loads are in flight together -- and the four waves are
// combined through LDS.  An entry without units (invalid) gets NaN.  The
// maxima are taken NaN-propagating, so a piece made NaN by a NaN input (a
// score or a block scale) makes its row NaN instead of counting as empty.
template <bool F16, int D>
__global__ __launch_bounds__(256) void k_decode_work_merge(CacheView cv, const void* ws_,
                                                           uint16_t* out, int nb, int qgroups,
                                                           int waves) {
  constexpr int J = D / 64;
  constexpr int UN = 4;
  __shared__ float sM[4], sDen[4], sAcc[4][D];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wv = tid >> 6;
  const int G = cv.n_q / cv.n_kv;
  const int nkvg = cv.n_kv * qgroups;
  const int kvh = h / G, qi = h % G, kvg = kvh * qgroups + qi / 16, r = qi % 16;
  const int64_t slots = work_slots(nb, nkvg, waves);
  WorkWs W_ = work_ws((void*)ws_, slots, D, nb);
  uint16_t* orow = out + ((int64_t)b * cv.n_q + h) * D;
  const int cb = W_.counts[b];
  const int64_t Wt = W_.units[nb];
  if (cb == 0 || Wt == 0) {
    for (int j = tid; j < D; j += 256) orow[j] = F16 ? 0x7E00 : 0x7FC0;   // NaN
    return;
  }
  const int64_t q_ = Wt / waves, r_ = Wt % waves;
  auto start_of = [&](int64_t w) -> int64_t { return w * q_ + (w * r_) / waves; };
  // wave holding unit x: the largest w with floor(w W / P) <= x, which is
  // floor(((x + 1) P - 1) / W)
  auto wave_of = [&](int64_t x) -> int64_t { return ((x + 1) * waves - 1) / Wt; };
  const int64_t s0 = W_.units[b] + (int64_t)kvg * cb;             // first unit
  const int64_t w0 = wave_of(s0), w1 = wave_of(s0 + cb - 1);
  const bool some_empty = q_ == 0;                                 // fewer units than waves
  const int64_t seg = (int64_t)b * nkvg + kvg;

  float M = -INFINITY, den = 0.f, acc[J];
#pragma unroll
  for (int i = 0; i < J; ++i) acc[i] = 0.f;
  for (int64_t w = w0 + wv; w <= w1; w += 4 * UN) {
    float pm[UN], pl[UN], po[UN][J];
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const int64_t ww = w + 4 * k;
      // waves whose range is empty wrote nothing
      const bool ok = ww <= w1 && (!some_empty || start_of(ww) != start_of(ww + 1));
      const int64_t sl = ok ? seg + ww : 0;
      pm[k] = ok ? W_.m[sl * 16 + r] : -INFINITY;
      pl[k] = ok ? W_.l[sl * 16 + r] : 0.f;
#pragma unroll
      for (int i = 0; i < J; ++i) po[k][i] = ok ? W_.O[(sl * 16 + r) * D + lane + 64 * i] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int k = 0; k < UN; ++k) Mn = vmax(Mn, pm[k]);     // a NaN piece makes Mn NaN
    if (Mn == -INFINITY) continue;
    const float a = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    den *= a;
#pragma unroll
    for (int i = 0; i < J; ++i) acc[i] *= a;
#pragma unroll
    for (int k = 0; k < UN; ++k) {
      const float f = pm[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm[k] - Mn);
      den += f * pl[k];
#pragma unroll
      for (int i = 0; i < J; ++i) acc[i] += f * po[k][i];
    }
    M = Mn;
  }
  if (lane == 0) {
    sM[wv] = M;
    sDen[wv] = den;
  }
#pragma unroll
  for (int i = 0; i < J; ++i) sAcc[wv][lane + 64 * i] = acc[i];
  __syncthreads();
  const float Mt = vmax(vmax(sM[0], sM[1]), vmax(sM[2], sM[3]));
  float f[4], dt = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f[k] = sM[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sM[k] - Mt);
    dt += f[k] * sDen[k];
  }
  const float inv = 1.f / dt;
  for (int j = tid; j < D; j += 256) {
    const float y = (f[0] * sAcc[0][j] + f[1] * sAcc[1][j] + f[2] * sAcc[2][j] +
                     f[3] * sAcc[3][j]) * inv;
    orow[j] = F16 ? __builtin_bit_cast(uint16_t, (_Float16)y) : f32_to_bf16_bits(y);
  }
}

template <int KV, int D>
hipError_t run(const CacheView& cv, int layer, int n, const int32_t* seqs, const void* q,
               void* out, float sl2, const DecodePlan& p, void* ws, int window, int sinks,
               hipStream_t st, DispatchEvents ev) {
  const int G = cv.n_q / cv.n_kv;
  const int qgroups = (G + 15) / 16;
  const int grid = (p.waves + 3) / 4;
  for (int b0 = 0; b0 < n; b0 += kMaxBatch) {
    const int nb = n - b0 < kMaxBatch ? n - b0 : kMaxBatch;
    const uint16_t* qb = (const uint16_t*)q + (int64_t)b0 * cv.n_q * D;
    uint16_t* ob = (uint16_t*)out + (int64_t)b0 * cv.n_q * D;
    const bool last = b0 + nb == n;
    hipError_t e = launch_ev(k_decode_work<KV, D>, dim3(grid), dim3(256), st,
                             b0 == 0 ? ev.start : nullptr, last && ev.main_only ? ev.stop : nullptr,
                             cv, layer, seqs + b0, qb, ws, nb, qgroups, p.waves, sl2, window,
                             sinks);
    if (e != hipSuccess) return e;
    e = launch_ev(k_decode_work_merge<KV == KV_F16, D>, dim3(cv.n_q, nb), dim3(256), st, nullptr,
                  last && !ev.main_only ? ev.stop : nullptr, cv, (const void*)ws, ob, nb, qgroups,
                  p.waves);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KV, int D>
int occupancy_waves() {
  static int waves = 0;
  if (waves == 0) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks,
                                                     (const void*)k_decode_work<KV, D>,
                                                     256, 0) != hipSuccess || blocks < 1)
      blocks = 2;
    waves = 4 * blocks;
  }
  return waves;
}

}  // namespace

// Waves per CU the work list is cut for, by storage type (at most the
// kernel's occupancy).  With two units in flight per wave, one wave per SIMD
// keeps enough bytes in flight for 16 KiB (16-bit) and 8 KiB (fp8) units, and
// fewer waves mean fewer pieces to start and merge; int4's 4 KiB units run at
// the same speed with four or eight waves.
constexpr int kWaves16 = 4, kWavesFp8 = 4, kWavesInt4 = 8;

uint64_t work_list_ws_bytes(const CacheView& cv, int32_t nb, int32_t waves) {
  const int nkvg = cv.n_kv * ((cv.n_q / cv.n_kv + 15) / 16);
  const int64_t slots = work_slots(nb, nkvg, waves);
  return (uint64_t)slots * 16 * (cv.d + 2) * 4 + (uint64_t)(nb + 1) * 8 + (uint64_t)nb * 4 + 16;
}

// Waves one compute unit keeps resident for this cache's decode kernel (the
// work list is cut for a full chip).  Host-only handles have no device to
// ask and use 8.
int work_list_waves_per_cu(const CacheView& cv) {
  if (cv.k == nullptr) return 8;
  int occ;
  if (cv.d == 128) {
    occ = cv.dtype == KVC_BF16   ? occupancy_waves<KV_BF16, 128>()
          : cv.dtype == KVC_F16  ? occupancy_waves<KV_F16, 128>()
          : cv.dtype == KVC_INT4 ? occupancy_waves<KV_INT4, 128>()
                                 : occupancy_waves<KV_FP8, 128>();
  } else {
    occ = cv.dtype == KVC_BF16   ? occupancy_waves<KV_BF16, 64>()
          : cv.dtype == KVC_F16  ? occupancy_waves<KV_F16, 64>()
          : cv.dtype == KVC_INT4 ? occupancy_waves<KV_INT4, 64>()
                                 : occupancy_waves<KV_FP8, 64>();
  }
  const int want = cv.dtype == KVC_INT4 ? kWavesInt4 : cv.dtype == KVC_FP8_E4M3FN ? kWavesFp8
                                                                                  : kWaves16;
  return std::min(occ, want);
}

hipError_t launch_decode_mfma(const CacheView& cv, int layer, int n, const int32_t* seqs,
                              const void* q, void* out, float sl2, const DecodePlan& p, void* ws,
                              int window, int sinks, hipStream_t st, DispatchEvents ev,
                              bool* handled) {
  *handled = p.work_list != 0;
  if (!*handled) return hipSuccess;
#define KVFA_RUN(KVT, DD) run<KVT, DD>(cv, layer, n, seqs, q, out, sl2, p, ws, window, sinks, st, ev)
  if (cv.d == 128) {
    if (cv.dtype == KVC_BF16) return KVFA_RUN(KV_BF16, 128);
    if (cv.dtype == KVC_F16) return KVFA_RUN(KV_F16, 128);
    if (cv.dtype == KVC_INT4) return KVFA_RUN(KV_INT4, 128);
    return KVFA_RUN(KV_FP8, 128);
  }
  if (cv.dtype == KVC_BF16) return KVFA_RUN(KV_BF16, 64);
  if (cv.dtype == KVC_F16) return KVFA_RUN(KV_F16, 64);
  if (cv.dtype == KVC_INT4) return KVFA_RUN(KV_INT4, 64);
  return KVFA_RUN(KV_FP8, 64);
#undef KVFA_RUN
}

}  // namespace kvfa
