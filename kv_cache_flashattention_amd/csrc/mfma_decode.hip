// Decode attention on the matrix cores (bf16 / fp16 / fp8 caches, d 64 or 128).
//
// Work unit: one workgroup of four waves per (split, kv head, group of up to
// 16 query heads sharing that kv head, sequence), so each K/V byte of the
// split is read once for the whole query group (grouped-query attention,
// "KV Cache & Flash Attention." (kvcache-7e2) memory-cost section).  The
// waves take 64-token chunks (four 16-token blocks) of the split in turn; per
// chunk a wave
//   1. computes S^T = K Q^T with 16x16x32 MFMAs: the 16 M-rows are tokens,
//      the 16 N-columns are the query rows (padded with zeros), K = head dim;
//   2. updates the running max m and sum l of each query row and rescales
//      its output by exp(m_old - m_new) (kvcache-7e2, online softmax
//      section), all in fp32;
//   3. computes O^T += V^T P^T with MFMAs over the chunk's tokens.
// The waves' (m, l, O) are combined through LDS at the end; with one split
// the workgroup writes O / l, otherwise it leaves (m, l, O) for the merge.
//
// Operand placement.  A 16x16x32 MFMA lane l holds, for its operand, row (or
// column) l % 16 and a group of 8 reduction indices chosen by l / 16; the
// reduction indices may be assigned in any order as long as both operands
// agree.  K slabs are [16][d], so a lane loads 16 bytes of one token's row
// for QK^T.  For PV the reduction runs over tokens, and the V slabs are
// [d][16], so a lane loads 8 (or, for fp8, 16) consecutive tokens of one
// head-dimension column.  Which token each S^T row holds is chosen so that
// the probabilities a lane ends up with are exactly the tokens its V
// operand covers: no data moves between lanes except the row max/sum.
//
// fp8: codes are widened to bf16 exactly (every E4M3FN value is a bf16
// value); the block's K scale multiplies its scores and its V scale the
// probabilities before they are rounded to bf16; the running sum l uses the
// unscaled probabilities.
#include "common.h"

namespace kvfa {

hipError_t launch_decode_merge(const CacheView& cv, int n, const int32_t* seqs, void* out,
                               const DecodePlan& p, const void* ws, hipStream_t st);

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

enum { KV_BF16 = 0, KV_F16 = 1, KV_FP8 = 2 };

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
// k-steps 2a and 2a+1.
template <int KV> __device__ __forceinline__ int dmap(int ks, int g) {
  if (KV == KV_FP8) return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1);
  return 32 * ks + 8 * g;
}

// Token held by row r of S^T tile t (t = 0..3) within a 64-token chunk:
// block (0..3) and slot (0..15).  After the MFMA, lane group g holds rows
// 4g..4g+3 of every tile; the PV k-step s takes tiles 2s and 2s+1, and its
// operand slot j = 4u + i of lane group g is row 4g+i of tile 2s+u.
template <int KV> __device__ __forceinline__ int tok_block(int t, int r) {
  if (KV == KV_FP8) return r >> 2;                        // group g <-> block g
  return 2 * (t >> 1) + (r >> 3);                         // group g <-> block 2s+(g>>1)
}
template <int KV> __device__ __forceinline__ int tok_slot(int t, int r) {
  if (KV == KV_FP8) return 4 * t + (r & 3);               // slots 8s..8s+7 per k-step
  return 8 * ((r >> 2) & 1) + 4 * (t & 1) + (r & 3);      // slots 8(g&1)..+7
}

template <int KV, int D>
__global__ __launch_bounds__(256, 2) void k_decode_mfma(CacheView cv, int layer,
                                                        const int32_t* seqs, const uint16_t* q,
                                                        uint16_t* out, void* ws, int n,
                                                        int splits, int split_len, float sl2,
                                                        int qgroups) {
  typedef typename Op<KV>::T OpT;
  constexpr int KS = D / 32;     // k-steps of QK^T
  constexpr int DT = D / 16;     // 16-row tiles of O^T
  constexpr int EB = KV == KV_FP8 ? 1 : 2;
  __shared__ float sO[4][16][D + 1];
  __shared__ float sm[4][16], sl[4][16];

  const int s = blockIdx.x, kvh = blockIdx.y / qgroups, qg = blockIdx.y % qgroups;
  const int b = blockIdx.z;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int G = cv.n_q / cv.n_kv;
  const int seq = seqs[b];
  const int L = valid_len(cv, seq);
  if (L < 0) {
    if (splits == 1) {
      for (int e = threadIdx.x; e < 16 * D; e += 256) {
        const int qi = qg * 16 + e / D;
        if (qi < G)
          out[((int64_t)b * cv.n_q + kvh * G + qi) * D + e % D] = 0x7FC0;   // NaN
      }
    }
    return;
  }
  const int t0 = s * split_len;
  if (t0 >= L) return;
  const int t1 = min(t0 + split_len, L);

  // Query operand (B of S^T = K Q^T): column r16 = query row qg*16 + r16.
  const int qi = qg * 16 + r16;
  const bool qrow = qi < G;
  OpT qop[KS];
  {
    const uint16_t* qr = q + ((int64_t)b * cv.n_q + kvh * G + (qrow ? qi : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 raw = qrow ? *(const uint4*)(qr + dmap<KV>(ks, g)) : make_uint4(0, 0, 0, 0);
      qop[ks] = __builtin_bit_cast(OpT, raw);
    }
  }

  f32x4 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lpart = 0.f;
  bool bad = false;

  const int32_t* btrow = cv.bt + (int64_t)seq * cv.max_bps;
  const uint8_t* kpool = (const uint8_t*)cv.k;
  const uint8_t* vpool = (const uint8_t*)cv.v;
  const int64_t slab_bytes = (int64_t)kBlock * D * EB;
  const int64_t layer_blocks = (int64_t)layer * cv.n_blocks;
  const int nchunks = (t1 - t0 + 63) / 64;
  const int last_blk = (L - 1) / kBlock;             // last table entry of the sequence
  const int wu = __builtin_amdgcn_readfirstlane(w);   // wave index as a scalar

  for (int ci = wu; ci < nchunks; ci += 4) {
    const int c = t0 + ci * 64;
    const int nvalid = min(64, t1 - c);
    const bool tail = nvalid < 64;
    // Table entries of the chunk's four blocks (entries past the sequence's
    // end are clamped to its last block; their tokens are masked below).
    int64_t sbase[4];
    int64_t sidx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int x = btrow[min(c / kBlock + i, last_blk)];
      if (x < 0 || x >= cv.n_blocks) {
        bad = true;
        x = 0;
      }
      sidx[i] = (layer_blocks + x) * cv.n_kv + kvh;
      sbase[i] = sidx[i] * slab_bytes;
    }
    auto pick = [&](const int64_t* a, int i) -> int64_t {
      return i == 0 ? a[0] : i == 1 ? a[1] : i == 2 ? a[2] : a[3];
    };

    // ---- issue every K and V load of the chunk before using any
    constexpr int KL = KV == KV_FP8 ? KS / 2 : KS;      // 16-byte K loads per tile
    constexpr int VL = KV == KV_FP8 ? DT : 2 * DT;      // 16-byte V loads per chunk
    uint4 kraw[4][KL];
    uint4 vraw[VL];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* krow = kpool + pick(sbase, tok_block<KV>(t, r16)) +
                            (int64_t)tok_slot<KV>(t, r16) * D * EB;
#pragma unroll
      for (int a = 0; a < KL; ++a) {
        const int off = KV == KV_FP8 ? 64 * a + 16 * g : 2 * dmap<KV>(a, g);
        kraw[t][a] = *(const uint4*)(krow + off);
      }
    }
    if (KV == KV_FP8) {
      const uint8_t* vslab = vpool + pick(sbase, g);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) vraw[dt] = *(const uint4*)(vslab + (16 * dt + r16) * kBlock);
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint8_t* vslab = vpool + pick(sbase, 2 * st + (g >> 1));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          vraw[st * DT + dt] =
              *(const uint4*)(vslab + 2 * ((16 * dt + r16) * kBlock + 8 * (g & 1)));
      }
    }

    // ---- S^T = K Q^T for four 16-token tiles
    f32x4 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < KL; ++a) {
        if (KV == KV_FP8) {
          sacc[t] = mfma(__builtin_bit_cast(OpT, fp8x8_to_bf16(kraw[t][a].x, kraw[t][a].y)),
                         qop[2 * a], sacc[t]);
          sacc[t] = mfma(__builtin_bit_cast(OpT, fp8x8_to_bf16(kraw[t][a].z, kraw[t][a].w)),
                         qop[2 * a + 1], sacc[t]);
        } else {
          sacc[t] = mfma(__builtin_bit_cast(OpT, kraw[t][a]), qop[a], sacc[t]);
        }
      }
    }

    // ---- online softmax over the chunk (this lane's S^T column: query r16)
    float ksc = 1.f, vsc = 1.f;
    if (KV == KV_FP8) {
      const int64_t si = pick(sidx, g);
      ksc = cv.ks[si];
      vsc = cv.vs[si];
    }
    float p[4][4];
    float cmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[t][i] * (sl2 * ksc);
        if (tail) {
          const int r = 4 * g + i;
          const int pos = 16 * tok_block<KV>(t, r) + tok_slot<KV>(t, r);
          if (pos >= nvalid) x = -INFINITY;
        }
        p[t][i] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m, cmax);
    const float alpha = m == -INFINITY ? 0.f : exp2f(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = exp2f(p[t][i] - m_new);
        psum += p[t][i];
      }
    lpart = lpart * alpha + psum;
    m = m_new;
#pragma unroll
    for (int i = 0; i < DT; ++i) o[i] *= alpha;

    // ---- O^T += V^T P^T, two k-steps of 32 tokens
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = p[2 * st + (j >> 2)][j & 3] * vsc;
      const OpT pop = pack8<OpT>(pv);
      // This lane's V operand covers block bi, slots s0..s0+7 of the chunk;
      // in the chunk holding the split's end, slots past it are zeroed (they
      // may hold stale or poisoned bytes, and 0 * NaN would poison O).
      const int bi = KV == KV_FP8 ? g : 2 * st + (g >> 1);
      const int s0 = KV == KV_FP8 ? 8 * st : 8 * (g & 1);
      const int nok = tail ? nvalid - 16 * bi - s0 : 8;  // valid slots among the 8
      uint32_t keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (KV == KV_FP8) {        // 4 one-byte slots per dword, dwords 0..1 used
          const int base = 4 * e;
          uint32_t mk = 0;
#pragma unroll
          for (int y = 0; y < 4; ++y) mk |= (base + y < nok ? 0xFFu : 0u) << (8 * y);
          keep[e] = mk;
        } else {                   // 2 two-byte slots per dword
          keep[e] = (2 * e < nok ? 0xFFFFu : 0u) | (2 * e + 1 < nok ? 0xFFFF0000u : 0u);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        OpT vop;
        if (KV == KV_FP8) {
          const uint32_t lo = (st == 0 ? vraw[dt].x : vraw[dt].z) & keep[0];
          const uint32_t hi = (st == 0 ? vraw[dt].y : vraw[dt].w) & keep[1];
          vop = __builtin_bit_cast(OpT, fp8x8_to_bf16(lo, hi));
        } else {
          const uint4 raw = vraw[st * DT + dt];
          vop = __builtin_bit_cast(OpT, make_uint4(raw.x & keep[0], raw.y & keep[1],
                                                   raw.z & keep[2], raw.w & keep[3]));
        }
        o[dt] = mfma(vop, pop, o[dt]);
      }
    }
  }

  // ---- combine the four waves
  float l = lpart + __shfl_xor(lpart, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (bad) l = __builtin_nanf("");
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) sO[w][r16][16 * dt + 4 * g + i] = o[dt][i];
  if (g == 0) {
    sm[w][r16] = m;
    sl[w][r16] = l;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * D; e += 256) {
    const int qq = e / D, d = e % D;
    const int qi2 = qg * 16 + qq;
    if (qi2 >= G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm[ww][qq]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float f = sm[ww][qq] == -INFINITY ? 0.f : exp2f(sm[ww][qq] - M);
      acc += f * sO[ww][qq][d];
      lsum += f * sl[ww][qq];
    }
    const int h = kvh * G + qi2;
    if (splits == 1) {
      const float y = acc / lsum;
      out[((int64_t)b * cv.n_q + h) * D + d] =
          KV == KV_F16 ? __builtin_bit_cast(uint16_t, (_Float16)y) : f32_to_bf16_bits(y);
    } else {
      float* PO = (float*)ws;
      float* Pm = PO + (int64_t)n * cv.n_q * splits * D;
      float* Pl = Pm + (int64_t)n * cv.n_q * splits;
      const int64_t r = ((int64_t)b * cv.n_q + h) * splits + s;
      PO[r * D + d] = acc;
      if (d == 0) {
        Pm[r] = M;
        Pl[r] = lsum;
      }
    }
  }
}

template <int KV, int D>
hipError_t run(const CacheView& cv, int layer, int n, const int32_t* seqs, const void* q,
               void* out, float sl2, const DecodePlan& p, void* ws, hipStream_t st) {
  const int G = cv.n_q / cv.n_kv;
  const int qgroups = (G + 15) / 16;
  hipLaunchKernelGGL((k_decode_mfma<KV, D>), dim3(p.splits, cv.n_kv * qgroups, n), dim3(256), 0,
                     st, cv, layer, seqs, (const uint16_t*)q, (uint16_t*)out, ws, n, p.splits,
                     p.split_len, sl2, qgroups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_decode_merge(cv, n, seqs, out, p, ws, st);
}

}  // namespace

hipError_t launch_decode_mfma(const CacheView& cv, int layer, int n, const int32_t* seqs,
                              const void* q, void* out, float sl2, const DecodePlan& p, void* ws,
                              hipStream_t st, bool* handled) {
  *handled = true;
  if (cv.d == 128) {
    if (cv.dtype == KVC_BF16) return run<KV_BF16, 128>(cv, layer, n, seqs, q, out, sl2, p, ws, st);
    if (cv.dtype == KVC_F16) return run<KV_F16, 128>(cv, layer, n, seqs, q, out, sl2, p, ws, st);
    if (cv.dtype == KVC_FP8_E4M3FN) return run<KV_FP8, 128>(cv, layer, n, seqs, q, out, sl2, p, ws, st);
  } else if (cv.d == 64) {
    if (cv.dtype == KVC_BF16) return run<KV_BF16, 64>(cv, layer, n, seqs, q, out, sl2, p, ws, st);
    if (cv.dtype == KVC_F16) return run<KV_F16, 64>(cv, layer, n, seqs, q, out, sl2, p, ws, st);
    if (cv.dtype == KVC_FP8_E4M3FN) return run<KV_FP8, 64>(cv, layer, n, seqs, q, out, sl2, p, ws, st);
  }
  *handled = false;
  return hipSuccess;
}

}  // namespace kvfa
