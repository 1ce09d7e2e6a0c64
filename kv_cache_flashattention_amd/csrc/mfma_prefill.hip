// Causal prefill attention on the matrix cores (bf16 / fp16, d 64 or 128).
//
// Tiling ("KV Cache & Flash Attention." (kvcache-7e2), Flash Attention
// section): a workgroup owns 256 consecutive query rows of one query head
// (eight waves x 32 rows) and streams the prompt's keys/values through LDS in
// tiles of 64 rows.  Per tile each wave
//   1. computes S^T = K Q^T (32 keys x 32 queries per 32x32x16 MFMA, d as
//      the reduction), so a lane holds 16 keys of one query column;
//   2. applies the causal mask on tiles that touch the diagonal and runs the
//      online softmax in fp32 (kvcache-7e2, online softmax section): row max
//      = in-lane max + one swap with the partner lane 32 away;
//   3. accumulates O^T += V^T P^T with P in registers (no LDS round trip).
// The score tile never leaves registers; only O / l is written.
//
// Two wave groups per SIMD, offset by half a tile ("ping-pong").  Waves w and
// w+4 share a SIMD.  The kernel runs in slots of half a tile; in each slot
// one group issues its matrix-core work (the PV product of tile i-1, S of
// tile i, and the short VALU work that needs S: row max and rescale) while
// the other group computes the exponentials of its last score tile and
// stages the next K or V tile into LDS.  The matrix core of each SIMD stays
// busy while the VALU serves the other wave.  Group 1 stages K tiles, group
// 0 stages V tiles, each in its own exponent slot, through registers (loads
// issued two slots ahead).  Every LDS write and the reads it must follow or
// precede lie on either side of the barrier at the end of every second
// slot, so whole-prompt tiles take that one barrier per tile; paged tiles
// keep a barrier at the end of every slot, which measured faster there.
//
// Running max.  The rescale factor exp(m_old - m_new) is applied only when
// the row max has grown by more than 8 (base-2 units) since the last
// rescale; otherwise the stale max is kept.  The result is the same exact
// softmax -- every term and the final sum use the one max in force -- and
// the terms stay below 2^8, far inside fp32/bf16 range.  Scores stay raw
// until the exponent: p = exp2(s * scale * log2(e) - m) is one FMA and one
// v_exp_f32 (terms below 2^-126 of the max flush to zero).  The row sum adds
// the probabilities as rounded to the 16-bit type the PV product uses.
//
// Layout choices.  K tiles sit in LDS as rows [key][d]; V tiles are written
// transposed, [d][key], during staging so that the PV operand (8
// consecutive keys of one d) is a single 16-byte LDS read.  Which key each
// S^T row holds is permuted so that the 8 probabilities a lane holds for a
// PV k-step are 8 consecutive keys.  Rows of both tiles are padded by 16
// bytes, which puts the 16 rows one operand read touches on 16 different
// bank groups and keeps every operand address a per-lane base plus an
// immediate offset; staging writes fill whole rows.
//
// Scheduling.  Query tiles near the end of the prompt see the most keys;
// each XCD walks its (sequence, kv head) tiles from the last to the first
// so the heaviest workgroups start first.  Consecutive workgroups go to
// different XCDs; the work list gives each XCD a contiguous run of one kv
// head's work, so its L2 serves the K/V tiles that its workgroups share.
#include "common.h"

namespace kvfa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int BM = 256;   // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr float kStale = 8.0f;

template <bool F16> struct Op { typedef bf16x8 T; };
template <> struct Op<true> { typedef f16x8 T; };

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// Sum of the 8 rounded probabilities of one PV operand, two per dot product.
__device__ __forceinline__ float sum8(bf16x8 p, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x2 t = {p[2 * j], p[2 * j + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(t, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float sum8(f16x8 p, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f16x2 t = {p[2 * j], p[2 * j + 1]};
    acc = __builtin_amdgcn_fdot2(t, one, acc, false);
  }
  return acc;
}

// The value held by the lane 32 away: one v_permlane32_swap, no LDS.
__device__ __forceinline__ float half_swap(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                            __builtin_bit_cast(uint32_t, x), false, false);
  // lanes 0-31 find the partner's value in r[1], lanes 32-63 in r[0]; the
  // other element holds the lane's own value.
  return __builtin_bit_cast(float, (__lane_id() < 32) ? r[1] : r[0]);
}

// Scheduling pattern for a run of N MFMAs, each fed by one 16-byte LDS
// operand read: the reads run at most AHEAD instructions ahead of the MFMAs
// that consume them, which bounds the registers holding operands in flight.
template <int N, int AHEAD>
__device__ __forceinline__ void interleave_lds_mfma() {
#pragma unroll
  for (int n = 0; n < AHEAD; ++n) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
  for (int n = 0; n < N - AHEAD; ++n) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int n = 0; n < AHEAD; ++n) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// The thread index, hidden from the optimizer so that per-lane addresses are
// recomputed where they are used (a few VALU ops in slots with spare VALU
// issue) instead of being hoisted out of the tile loop into registers that
// would stay live across it.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Key (0..31 within a 32-key S^T tile) held by MFMA row r = 8*jj + 4*h + i.
// Lane half h then holds keys 8h..8h+7 (jj = 0, 1) and 16+8h..16+8h+7
// (jj = 2, 3).
__device__ __forceinline__ int row_key(int r) {
  const int jj = r >> 3, h = (r >> 2) & 1, i = r & 3;
  return (jj < 2) ? 8 * h + 4 * jj + i : 16 + 8 * h + 4 * (jj - 2) + i;
}

// PAGED = false: whole prompts, K/V rows [n][T][n_kv][d] beside the queries,
// query t at position t.  PAGED = true: T new query rows per sequence
// against the len(s) rows the paged cache holds for it (the new rows'
// K/V included), query t at position len(s) - T + t; K/V tiles are staged
// straight from the (block, kv head) slabs through the block table.
// SC (paged only): a scaled cache, KVC_FP8_E4M3FN or KVC_INT4, whose slabs
// hold codes with one float scale per (block, kv head).  Staging widens each
// code exactly to bf16 (every E4M3FN value and every int4 code is a bf16
// value); the tile's four K scales multiply the scores of their blocks'
// keys and its four V scales the probabilities before they are rounded for
// the PV products, while the row sum l adds the unscaled probabilities.
template <int D, bool F16, bool PAGED, bool WIN, int SC = 0>
__global__ __launch_bounds__(512, 1) void k_prefill_mfma(int n_q, int n_kv, int T,
                                                         const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         uint16_t* __restrict__ out, float sl2,
                                                         int ntiles, int n_seq, int n_units,
                                                         int xcd_split, CacheView cv, int layer,
                                                         const int32_t* __restrict__ seqs,
                                                         int window, int sinks) {
  typedef typename Op<F16>::T OpT;
  constexpr int KS = D / 16;        // k-steps of QK^T
  constexpr int DT = D / 32;        // 32-row tiles of O^T
  constexpr int KG = D / 8;         // 16-byte granules per K row
  constexpr int KP = D + 8;         // padded row lengths (elements)
  constexpr int VP = BN + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VP];
  __shared__ float Ssc[2][8];       // scaled caches: K scales [0..3], V scales [4..7] of a tile

  // ---- work assignment.  Workgroup L runs on XCD L % 8; the work list is
  // cut into 8 contiguous parts, one per XCD, ordered (kv head, sequence,
  // query tile from the last, query head of the group).  An XCD thus works
  // through one (sequence, kv head) at a time and its L2 holds the K/V rows
  // that all of its resident workgroups read.
  const int G = n_q / n_kv;
  int u = blockIdx.x;
  if (xcd_split) u = (u % 8) * (n_units / 8) + u / 8;
  const int hg = u % G;
  int r = u / G;
  const int tile = ntiles - 1 - r % ntiles;
  r /= ntiles;
  const int b = r % n_seq;
  const int g = r / n_seq;
  const int head = g * G + hg;
  const int q0 = tile * BM;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2;                              // SIMD w & 3 hosts waves w, w ^ 4
  const int rq0 = q0 + 32 * (2 * (w & 3) + grp);       // first query row of this wave
  const int qrow = rq0 + col;                          // this lane's query position
  const int64_t qstride = (int64_t)n_q * D, kvstride = (int64_t)n_kv * D;

  // ---- keys: L rows; query row t sits at position qoff + t
  int L = T, seq = 0;
  if constexpr (PAGED) {
    seq = seqs[b];
    bool bad = seq < 0 || seq >= cv.max_seqs;
    L = bad ? 0 : cv.len[seq];
    bad = bad || L < T || L > cv.max_bps * kBlock;
    if (!bad) {
      const int32_t* bt = cv.bt + (int64_t)seq * cv.max_bps;
      for (int j = tid; j < (L + kBlock - 1) / kBlock; j += 512) {
        const int e = bt[j];
        bad = bad || e < 0 || e >= cv.n_blocks;
      }
    }
    if (__syncthreads_or(bad)) {                       // invalid entry: NaN rows
      const uint16_t nan = F16 ? 0x7E00 : 0x7FC0;
      for (int e = tid; e < BM * D; e += 512) {
        const int row = q0 + e / D;
        if (row < T) out[((int64_t)b * T + row) * qstride + (int64_t)head * D + e % D] = nan;
      }
      return;
    }
  }
  const int qoff = L - T;
  const int kend = min(L, qoff + q0 + BM);             // keys any row of the workgroup sees
  const int nkc = (kend + BN - 1) / BN;                // key tiles up to the causal limit
  // Tile list.  Without a window: tiles 0 .. nkc-1.  With a window w: the
  // tiles holding sink keys, then the tiles from the one holding the
  // workgroup's first windowed key (position qoff + q0 - w + 1) on.
  int nst = 0, wt0 = 0;
  if constexpr (WIN) {
    nst = min((sinks + BN - 1) / BN, nkc);
    wt0 = max(nst, max(0, qoff + q0 - window + 1) / BN);
  }
  const int nkt = nst + (nkc - wt0);                   // tiles in the list
  auto tile_of = [&](int i) { return WIN ? (i < nst ? i : wt0 + (i - nst)) : i; };
  // Does this wave need list entry i: a key of the tile visible to one of its
  // rows (positions pw .. pw + 31)?  Without a window: the tiles up to the
  // one holding its last row's position.
  const int pw = qoff + rq0;
  const int wn = rq0 < T ? min(nkt, (pw + 31) / BN + 1) : 0;
  auto need = [&](int i) {
    if constexpr (!WIN) {
      return i < wn;
    } else {
      if (rq0 >= T || i >= nkt) return false;
      const int k0 = BN * tile_of(i);
      if (k0 > pw + 31) return false;                  // after every row
      return k0 < sinks || k0 + BN - 1 > pw - window;
    }
  };

  // ---- query operand (B of S^T = K Q^T)
  OpT qop[KS];
  {
    const uint16_t* qp = q + ((int64_t)b * T + min(qrow, T - 1)) * qstride + (int64_t)head * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = __builtin_bit_cast(OpT, *(const u32x4*)(qp + 16 * ks + 8 * half));
  }

  // ---- staging through registers.  Rows past the last key load row L-1
  // instead: their scores are masked (the key is after every query), so
  // they contribute exp(-inf) * finite = 0.
  constexpr int KCH = BN * D / 8 / 256;                // 16-byte K chunks per group thread
  constexpr int VBL = (BN / 4) * (D / 8);              // prompt: 4x8 V blocks per tile
  constexpr int VCH = D * BN / 8 / 256;                // paged: 16-byte V^T chunks per thread
  u32x4 sreg[4];                                       // plain vectors: stay in registers
  const uint16_t* kbase = k + (int64_t)b * T * kvstride + (int64_t)g * D;
  const uint16_t* vbase = v + (int64_t)b * T * kvstride + (int64_t)g * D;
  // paged: slab (block e, kv head g) of this layer starts at pool + e * slab
  const int64_t slab = (int64_t)n_kv * kBlock * D;
  const uint16_t* kpool = (const uint16_t*)cv.k + ((int64_t)layer * cv.n_blocks * n_kv + g) * kBlock * D;
  const uint16_t* vpool = (const uint16_t*)cv.v + ((int64_t)layer * cv.n_blocks * n_kv + g) * kBlock * D;
  const int32_t* btab = cv.bt + (int64_t)seq * cv.max_bps;
  // scaled caches: byte pools (fp8 one byte per code, int4 two codes per
  // byte) and the scale index base
  constexpr bool FP8 = SC == KVC_FP8_E4M3FN, I4 = SC == KVC_INT4;
  constexpr int CB = I4 ? 2 : 1;                       // codes per byte
  const int64_t slab8 = slab / CB;                     // slab bytes
  const uint8_t* kpool8 = (const uint8_t*)cv.k + ((int64_t)layer * cv.n_blocks * n_kv + g) * slab8 / n_kv;
  const uint8_t* vpool8 = (const uint8_t*)cv.v + ((int64_t)layer * cv.n_blocks * n_kv + g) * slab8 / n_kv;
  const int64_t sc0 = (int64_t)layer * cv.n_blocks * n_kv + g;   // + block * n_kv
  // 8 fp8 codes (two dwords) times a scale, rounded to 8 bf16 (four dwords)
  // 8 fp8 codes (two dwords) -> 8 bf16, exactly
  auto widen8 = [&](uint32_t lo, uint32_t hi) {
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    const b2 x[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false),
                     __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)};
    u32x4 r;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) r[w2] = __builtin_bit_cast(uint32_t, x[w2]);
    return r;
  };
  // 8 int4 codes (one dword, code k in nibble k) -> 8 bf16, exactly
  auto widen8_i4 = [&](uint32_t x) {
    u32x4 r;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      // the builtin is typed unsigned: the signed field goes through int
      const float lo = (float)(int)__builtin_amdgcn_sbfe((int)x, 8 * w2, 4);
      const float hi = (float)(int)__builtin_amdgcn_sbfe((int)x, 8 * w2 + 4, 4);
      r[w2] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
              ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
    }
    return r;
  };
  // scaled caches: the K and V scales of the tile's four blocks, loaded by
  // group threads 0..3 with the K tile and written to LDS beside it
  float scK = 1.f, scV = 1.f;
  // Prompt staging: this thread's element offsets within a K or V tile
  // (row t / KG, granule t % KG; V rows 4 kg, granule dg), computed once;
  // the other chunks of a tile lie a uniform number of rows further on.
  const int tg = tid & 255;
  const int koff = (tg / KG) * (int)kvstride + 8 * (tg % KG);
  const int voff = 4 * (tg % (BN / 4)) * (int)kvstride + 8 * (tg / (BN / 4));
  // Paged staging: a tile's block ids are read (ktab / vtab) before the
  // staging group writes its previous tile into LDS, so the table round
  // trip overlaps those writes and the data loads (load_k / load_v) start
  // without waiting for it.  Slab offsets: block id times the slab size,
  // both below 2^32, as one 32 x 32 -> 64-bit product.
  int kblk[KCH], sblk = 0, vblk = 0;
  auto slab_off = [](int e, int64_t n) { return (int64_t)((uint64_t)(uint32_t)e * (uint32_t)n); };
  auto ktab = [&](int li) {
    if constexpr (PAGED) {
      const int i = tile_of(li);
      const int lim = L - 1 - BN * i;
      const int t = opaque_tid() & 255;
#pragma unroll
      for (int c0 = 0; c0 < KCH; ++c0) kblk[c0] = btab[(BN * i + min(t / KG + c0 * (256 / KG), lim)) >> 4];
      if constexpr (SC != 0) {
        if (t < 4) sblk = btab[min(BN * i + kBlock * t, L - 1) >> 4];
      }
    }
  };
  auto vtab = [&](int li) {
    if constexpr (PAGED) {
      const int i = tile_of(li);
      const int t = opaque_tid() & 255;
      vblk = btab[min(BN * i + kBlock * ((t >> 1) & 3), L - 1) >> 4];   // block (c / 2) % 4 of every chunk
    }
  };
  auto load_k = [&](int li) {
    const int i = tile_of(li);
    const int lim = L - 1 - BN * i;                    // last valid row of the tile
    const int t = opaque_tid() & 255;
    if constexpr (PAGED) {
#pragma unroll
      for (int c0 = 0; c0 < KCH; ++c0) {
        const int kp = BN * i + min(t / KG + c0 * (256 / KG), lim);
        const int e = kblk[c0];
        if constexpr (FP8) {
          const uint2 x = *(const uint2*)(kpool8 + slab_off(e, slab8) + (kp & (kBlock - 1)) * D + 8 * (t % KG));
          sreg[c0] = u32x4{x.x, x.y, 0u, 0u};
        } else if constexpr (I4) {
          const uint32_t x = *(const uint32_t*)(kpool8 + slab_off(e, slab8) + (kp & (kBlock - 1)) * (D / 2) +
                                                4 * (t % KG));
          sreg[c0] = u32x4{x, 0u, 0u, 0u};
        } else {
          const uint16_t* sl = kpool + slab_off(e, slab);
          sreg[c0] = *(const u32x4*)(sl + (kp & (kBlock - 1)) * D + 8 * (t % KG));
        }
      }
      if constexpr (SC != 0) {
        if (t < 4) {
          scK = cv.ks[sc0 + (int64_t)sblk * n_kv];
          scV = cv.vs[sc0 + (int64_t)sblk * n_kv];
        }
      }
    } else {
      const uint16_t* tb = kbase + (int64_t)(BN * i) * kvstride;
      if (lim >= BN - 1) {                             // whole tile: no row clamps
#pragma unroll
        for (int c0 = 0; c0 < KCH; ++c0)
          sreg[c0] = *(const u32x4*)(tb + koff + c0 * (256 / KG) * (int)kvstride);
      } else {
#pragma unroll
        for (int c0 = 0; c0 < KCH; ++c0) {
          const int row = min(t / KG + c0 * (256 / KG), lim);
          sreg[c0] = *(const u32x4*)(tb + row * kvstride + 8 * (t % KG));
        }
      }
    }
  };
  auto store_k = [&](int buf) {
    const int t = opaque_tid() & 255;
#pragma unroll
    for (int c0 = 0; c0 < KCH; ++c0) {
      u32x4 x = sreg[c0];
      if constexpr (FP8) x = widen8(x[0], x[1]);
      if constexpr (I4) x = widen8_i4(x[0]);
      *(u32x4*)&Ks[buf][(t / KG + c0 * (256 / KG)) * KP + 8 * (t % KG)] = x;
    }
    if constexpr (SC != 0) {
      if (t < 4) {
        Ssc[buf][t] = scK;
        Ssc[buf][4 + t] = scV;
      }
    }
  };
  // Prompt V: thread (kg, dg) moves keys 4kg..4kg+3 of d-granule dg,
  // transposing them; the 16 lanes of one LDS write pass cover one whole
  // V^T row.  Paged V: the slabs are already [d][16], so chunk c = (d row
  // c / 8, block (c / 2) % 4 of the tile, half c % 2) is a plain 16-byte
  // copy; keys at or past L (stale slots of the last block, blocks past the
  // end) are zeroed, since 0 * NaN would poison the PV product.
  auto load_v = [&](int li) {
    const int i = tile_of(li);
    const int t = opaque_tid() & 255;
    if constexpr (PAGED) {
#pragma unroll
      for (int c0 = 0; c0 < VCH; ++c0) {
        const int c = t + 256 * c0, rr = c >> 3, h = c & 1;
        const int e = vblk;
        if constexpr (FP8) {
          const uint2 x = *(const uint2*)(vpool8 + slab_off(e, slab8) + rr * kBlock + 8 * h);
          sreg[c0] = u32x4{x.x, x.y, 0u, 0u};
        } else if constexpr (I4) {
          const uint32_t x = *(const uint32_t*)(vpool8 + slab_off(e, slab8) + rr * (kBlock / 2) + 4 * h);
          sreg[c0] = u32x4{x, 0u, 0u, 0u};
        } else {
          const uint16_t* sl = vpool + slab_off(e, slab);
          sreg[c0] = *(const u32x4*)(sl + rr * kBlock + 8 * h);
        }
      }
    } else if (t < VBL) {
      const int kg = t % (BN / 4), dg = t / (BN / 4);
      const uint16_t* tb = vbase + (int64_t)(BN * i) * kvstride;
      const int lim = L - 1 - BN * i;
      if (lim >= BN - 1) {                             // whole tile: no row clamps
#pragma unroll
        for (int r = 0; r < 4; ++r) sreg[r] = *(const u32x4*)(tb + voff + r * (int)kvstride);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = min(4 * kg + r, lim);
          sreg[r] = *(const u32x4*)(tb + row * kvstride + 8 * dg);
        }
      }
    }
  };
  auto store_v = [&](int buf, int li) {
    const int i = tile_of(li);
    const int t = opaque_tid() & 255;
    if constexpr (PAGED) {
#pragma unroll
      for (int c0 = 0; c0 < VCH; ++c0) {
        const int c = t + 256 * c0, rr = c >> 3, j = (c >> 1) & 3, h = c & 1;
        const int nvalid = L - (BN * i + kBlock * j + 8 * h);   // keys of the chunk below L
        u32x4 x = sreg[c0];
        if constexpr (FP8) x = widen8(x[0], x[1]);
        if constexpr (I4) x = widen8_i4(x[0]);
        if (nvalid < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep = (2 * e + 1 < nvalid) ? 0xFFFFFFFFu
                                : (2 * e < nvalid) ? 0x0000FFFFu : 0u;
            x[e] &= keep;
          }
        }
        *(u32x4*)&Vt[buf][rr * VP + kBlock * j + 8 * h] = x;
      }
    } else if (t < VBL) {
      const int kg = t % (BN / 4), dg = t / (BN / 4);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wd = dd >> 1;
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint2 pk;   // keys 0..3 of column dd
        pk.x = __builtin_amdgcn_perm(sreg[1][wd], sreg[0][wd], sel);
        pk.y = __builtin_amdgcn_perm(sreg[3][wd], sreg[2][wd], sel);
        *(uint2*)&Vt[buf][(8 * dg + dd) * VP + 4 * kg] = pk;
      }
    }
  };

  // ---- per-wave state
  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  f32x16 sacc[2];
  OpT pop[4];

  // S^T of tile i (buffer i & 1)
  auto qk = [&](int i) {
    const int buf = i & 1, t = opaque_tid(), c = t & 31, h = (t >> 5) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[st][e] = 0.f;
      const uint16_t* krow = &Ks[buf][(32 * st + row_key(c)) * KP + 8 * h];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        OpT a = __builtin_bit_cast(OpT, *(const u32x4*)(krow + 16 * ks));
        sacc[st] = mfma32(a, qop[ks], sacc[st]);
      }
    }
    interleave_lds_mfma<2 * KS, 3>();
  };
  // online softmax of tile i, first half: mask, row max, rescale of O and l
  float vsc_r[4] = {1.f, 1.f, 1.f, 1.f};             // scaled caches: V scales of tile i
  auto rowmax = [&](int i) {
    const int k0 = BN * tile_of(i);
    if constexpr (SC != 0) {
      // scores of the keys of block j (elements jj < 2 of sacc[st]: block
      // 2 st, jj >= 2: block 2 st + 1) times that block's K scale
      const float* sc = Ssc[i & 1];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[st][e] *= sc[2 * st + ((e >> 2) >= 2 ? 1 : 0)];
#pragma unroll
      for (int j = 0; j < 4; ++j) vsc_r[j] = sc[4 + j];
    }
    // the tile reaches past the wave's first row, or (window) holds a
    // non-sink key at or before the last row's window start
    const bool diag = k0 + BN - 1 > pw;
    const bool wedge = WIN && k0 <= pw + 31 - window && k0 + BN > sinks;
    if (diag || wedge) {
      // element e of sacc[st] holds key k0 + 32 st + 8 half + kofs(e)
      const int t = opaque_tid();
      const int rel = pw + (t & 31) - k0 - 8 * ((t >> 5) & 1);   // query position - key base
      const int kbase = k0 + 8 * ((t >> 5) & 1);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int jj = e >> 2, kofs = 32 * st + (jj < 2 ? 4 * jj : 16 + 4 * (jj - 2)) + (e & 3);
          bool hide = kofs > rel;                                  // key after the query
          if (WIN)                                                // outside window, not a sink
            hide = hide || (kofs <= rel - window && kbase + kofs >= sinks);
          if (hide) sacc[st][e] = -INFINITY;
        }
    }
    float rmax = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) rmax = fmaxf(rmax, sacc[st][e]);
    rmax = fmaxf(rmax, half_swap(rmax)) * sl2;         // base-2 domain (sl2 > 0)
    const float m_new = fmaxf(m, rmax);
    const bool grow = m_new > m + kStale;              // also true when m = -inf and m_new finite
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new)) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[d][e] *= alpha;
    }
    if (grow) m = m_new;
  };
  // probabilities of tile i under the running max -> pop
  auto expo = [&](int i) {
    const float msub = m == -INFINITY ? 0.f : m;       // fully masked rows so far: p = 0
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = __builtin_amdgcn_exp2f(fmaf(sacc[st][8 * kb + e], sl2, -msub));
        if constexpr (SC != 0) {                       // l: unscaled; PV: times the V scale
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lsum += p[e];
            p[e] *= vsc_r[2 * st + kb];
          }
        }
        pop[2 * st + kb] = pack8<OpT>(p);
      }
  };
  // l += row sums of P_i; O^T += V^T P^T of tile i over 4 k-steps of 16 keys
  auto pv = [&](int i) {
    if constexpr (SC == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) lsum = sum8(pop[j], lsum);
    }
    const int buf = i & 1, t = opaque_tid(), c = t & 31, h = (t >> 5) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* vr = &Vt[buf][(32 * dt + c) * VP + 32 * st + 16 * kb + 8 * h];
          OpT a = __builtin_bit_cast(OpT, *(const u32x4*)vr);
          o[dt] = mfma32(a, pop[2 * st + kb], o[dt]);
        }
      }
    interleave_lds_mfma<4 * DT, 3>();
  };

  // ---- prologue: K_0 into LDS; loads of K_1 (group 1) and V_0 (group 0)
  if (grp == 1) {
    ktab(0);
    load_k(0);
    if (1 < nkt) ktab(1);
    store_k(0);
    if (1 < nkt) load_k(1);
  } else {
    vtab(0);
    load_v(0);
  }
  __syncthreads();

  // ---- slots.  Every wave runs the same sequence, per tile i: a matrix
  // phase (row sums and PV of P_{i-1}, then S_i, its row max and the
  // rescale of O and l) and an exponent phase (its group's staging duty,
  // then P_i), each closed by a barrier.  Group 1 starts one slot late, so
  // in slot 2i+g group g runs the matrix phase of tile i and in slot 2i+1+g
  // its exponent phase.  Staging: group 1 writes K_{i+2} in its exponent
  // phase of tile i (slot 2i+2), group 0 writes V_i in its exponent phase
  // of tile i (slot 2i+1); in both cases the buffer's previous tile was last
  // read in slot 2i+1 or earlier, and the new tile is first read two or
  // more slots later.  Loads are issued two slots before their LDS write.
  // The matrix phase runs at a raised wave priority: its MFMAs issue first
  // and the other wave's VALU work fills the remaining issue cycles.
  // Whole prompts: one barrier per tile (every LDS write and read it orders
  // lies on either side of the barrier that ends a group's matrix phase for
  // group 1 and its exponent phase for group 0); the groups offset each
  // other by half a tile.  Paged tiles: a barrier after each phase.
  constexpr bool ONE = !PAGED;
  if (grp == 1) {
    if (1 < nkt) {
      if (2 < nkt) ktab(2);
      store_k(1);
      if (2 < nkt) load_k(2);
    }
    if (!ONE) __syncthreads();
  }
  for (int i = 0; i <= nkt; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
    if (i >= 1 && need(i - 1)) pv(i - 1);            // P_{i-1} dies before S_i is born
    if (need(i)) {
      qk(i);
      rowmax(i);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if (!ONE || grp == 1) __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // staging first: its LDS writes drain while the exponentials run
    if (grp == 1) {
      if (i + 2 < nkt) {
        if (i + 3 < nkt) ktab(i + 3);
        store_k(i & 1);
        if (i + 3 < nkt) load_k(i + 3);
      }
    } else if (i < nkt) {
      if (i + 1 < nkt) vtab(i + 1);
      store_v(i & 1, i);
      if (i + 1 < nkt) load_v(i + 1);
    }
    if (need(i)) expo(i);
    __builtin_amdgcn_sched_barrier(0);
    if (!ONE || grp == 0) __syncthreads();
  }
  if (!ONE && grp == 0) __syncthreads();             // same barrier count for both groups

  // ---- epilogue: O / l for this lane's query column
  if (rq0 >= T || qrow >= T) return;
  const float l = lsum + half_swap(lsum);
  const float inv = 1.f / l;
  uint16_t* orow = out + ((int64_t)b * T + qrow) * qstride + (int64_t)head * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 32 * dt + 8 * jj + 4 * half;
      uint16_t hv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float y = o[dt][4 * jj + i] * inv;
        hv[i] = F16 ? __builtin_bit_cast(uint16_t, (_Float16)y)
                    : __builtin_bit_cast(uint16_t, (__bf16)y);
      }
      uint2 pk = make_uint2((uint32_t)hv[0] | ((uint32_t)hv[1] << 16),
                            (uint32_t)hv[2] | ((uint32_t)hv[3] << 16));
      *(uint2*)(orow + d0) = pk;
    }
}

template <int D, bool F16, bool PAGED, int SC = 0>
hipError_t run(const CacheView& cv, int layer, int n, const int32_t* seqs, int T, const void* q,
               const void* k, const void* v, void* out, float sl2, int window, int sinks,
               hipStream_t s, DispatchEvents ev) {
  const int ntiles = (T + BM - 1) / BM;
  const int64_t units = (int64_t)cv.n_q * n * ntiles;
  if (units > INT32_MAX) return hipErrorInvalidValue;
  const int xcd_split = units % 8 == 0 ? 1 : 0;
  const dim3 grid((uint32_t)units), block(512);
  if (window > 0)
    return launch_ev(k_prefill_mfma<D, F16, PAGED, true, SC>, grid, block, s, ev.start, ev.stop,
                     cv.n_q, cv.n_kv, T, (const uint16_t*)q, (const uint16_t*)k,
                     (const uint16_t*)v, (uint16_t*)out, sl2, ntiles, n, (int)units, xcd_split,
                     cv, layer, seqs, window, sinks);
  return launch_ev(k_prefill_mfma<D, F16, PAGED, false, SC>, grid, block, s, ev.start, ev.stop,
                   cv.n_q, cv.n_kv, T, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                   (uint16_t*)out, sl2, ntiles, n, (int)units, xcd_split, cv, layer, seqs, 0, 0);
}

template <bool PAGED>
hipError_t dispatch(const CacheView& cv, int layer, int n, const int32_t* seqs, int T,
                    const void* q, const void* k, const void* v, void* out, float sl2,
                    int window, int sinks, hipStream_t s, DispatchEvents ev, bool* handled) {
  *handled = true;
  const int io = io_dtype(cv.dtype);
  if (io == KVC_BF16 && (!PAGED || cv.dtype == KVC_BF16)) {
    if (cv.d == 128) return run<128, false, PAGED>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
    if (cv.d == 64) return run<64, false, PAGED>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
  } else if (PAGED && cv.dtype == KVC_FP8_E4M3FN) {
    if (cv.d == 128) return run<128, false, true, KVC_FP8_E4M3FN>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
    if (cv.d == 64) return run<64, false, true, KVC_FP8_E4M3FN>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
  } else if (PAGED && cv.dtype == KVC_INT4) {
    if (cv.d == 128) return run<128, false, true, KVC_INT4>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
    if (cv.d == 64) return run<64, false, true, KVC_INT4>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
  } else if (io == KVC_F16) {
    if (cv.d == 128) return run<128, true, PAGED>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
    if (cv.d == 64) return run<64, true, PAGED>(cv, layer, n, seqs, T, q, k, v, out, sl2, window, sinks, s, ev);
  }
  *handled = false;
  return hipSuccess;
}

}  // namespace

hipError_t launch_prefill_mfma(const CacheView& cv, int n, int T, const void* q, const void* k,
                               const void* v, void* out, float sl2, int window, int sinks,
                               hipStream_t s, DispatchEvents ev, bool* handled) {
  return dispatch<false>(cv, 0, n, nullptr, T, q, k, v, out, sl2, window, sinks, s, ev, handled);
}

hipError_t launch_extend_mfma(const CacheView& cv, int layer, int n, const int32_t* seqs, int T,
                              const void* q, void* out, float sl2, int window, int sinks,
                              hipStream_t s, DispatchEvents ev, bool* handled) {
  return dispatch<true>(cv, layer, n, seqs, T, q, nullptr, nullptr, out, sl2, window, sinks, s,
                        ev, handled);
}

}  // namespace kvfa
