// Causal prefill attention on the matrix cores (bf16 / fp16, d 64 or 128).
//
// Tiling ("KV Cache & Flash Attention." (kvcache-7e2), Flash Attention
// section): a workgroup owns 128 consecutive query rows of one query head
// (four waves x 32 rows) and streams the prompt's keys/values through LDS in
// tiles of 64 rows, double-buffered: while a tile is consumed the next one is
// already on its way from HBM.  Per tile each wave
//   1. computes S^T = K Q^T (32 keys x 32 queries per 32x32x16 MFMA, d as
//      the reduction), so a lane holds 16 keys of one query column;
//   2. applies the causal mask on tiles that touch the diagonal and runs the
//      online softmax in fp32 (kvcache-7e2, online softmax section): row max
//      = in-lane max + one exchange with the partner lane 32 away;
//   3. accumulates O^T += V^T P^T with P in registers (no LDS round trip).
// The score tile never leaves registers; only O / l is written.
//
// Running max.  The rescale factor exp(m_old - m_new) is applied only when
// the row max has grown by more than 8 (base-2 units) since the last
// rescale; otherwise the stale max is kept.  The result is the same exact
// softmax -- every term and the final sum use the one max in force -- and
// the terms stay below 2^8, far inside fp32/bf16 range.  Scores stay raw
// until the exponent: p = exp2(s * scale * log2(e) - m) is one FMA and one
// v_exp_f32 (terms below 2^-126 of the max flush to zero).
//
// Layout choices.  K tiles sit in LDS as rows [key][d]; V tiles are written
// transposed, [d][key], during staging so that the PV operand (8
// consecutive keys of one d) is a single 16-byte LDS read.  Which key each
// S^T row holds is permuted so that the 8 probabilities a lane holds for a
// PV k-step are 8 consecutive keys.
//
// Scheduling.  Query tiles near the end of the prompt see the most keys;
// the grid's slowest dimension walks the tiles from the last to the first so
// the heaviest workgroups start first.  On 8-XCD parts consecutive
// workgroups go to different XCDs; query heads are numbered so that the
// heads sharing one kv head land on the same XCD (and its L2).
#include "common.h"

namespace kvfa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int BM = 128;   // query rows per workgroup
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

// Key (0..31 within a 32-key S^T tile) held by MFMA row r = 8*jj + 4*h + i.
// Lane half h then holds keys 8h..8h+7 (jj = 0, 1) and 16+8h..16+8h+7
// (jj = 2, 3).
__device__ __forceinline__ int row_key(int r) {
  const int jj = r >> 3, h = (r >> 2) & 1, i = r & 3;
  return (jj < 2) ? 8 * h + 4 * jj + i : 16 + 8 * h + 4 * (jj - 2) + i;
}

// LDS tiles are stored without padding, with 16-byte granules XOR-swizzled
// per row so that the lanes of one LDS access hit distinct banks, both when
// the tiles are written during staging and when the MFMA operands are read.
// K tile [key][d]: granule g of row r lives at g ^ ksw(r); the operand read
// touches rows {0..3, 8..11} (+32) at one granule, which ksw spreads over 8
// granules.  V^T tile [d][key]: granule g of row r lives at g ^ vsw(r);
// operand reads touch 8 consecutive rows, staging writes rows 8 apart.
__device__ __forceinline__ int ksw(int r) { return (r & 3) | ((r >> 1) & 4); }
__device__ __forceinline__ int vsw(int r) { return (r & 7) ^ ((r >> 3) & 7); }

template <int D, bool F16>
__global__ __launch_bounds__(256, 2) void k_prefill_mfma(int n_q, int n_kv, int T,
                                                         const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         uint16_t* __restrict__ out, float sl2,
                                                         int ntiles, int xcd_heads) {
  typedef typename Op<F16>::T OpT;
  constexpr int KS = D / 16;        // k-steps of QK^T
  constexpr int DT = D / 32;        // 32-row tiles of O^T
  constexpr int KG = D / 8;         // 16-byte granules per K row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * BN];

  // ---- work assignment
  const int bx = blockIdx.x;
  const int head = xcd_heads ? (bx % 8) * (n_q / 8) + bx / 8 : bx;
  const int b = blockIdx.y;
  const int tile = ntiles - 1 - (int)blockIdx.z;
  const int q0 = tile * BM;
  const int g = head / (n_q / n_kv);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int qrow = q0 + 32 * w + col;                 // this lane's query position
  const bool wave_live = q0 + 32 * w < T;
  const int64_t qstride = (int64_t)n_q * D, kvstride = (int64_t)n_kv * D;

  // ---- query operand (B of S^T = K Q^T)
  OpT qop[KS];
  {
    const uint16_t* qp = q + ((int64_t)b * T + min(qrow, T - 1)) * qstride + (int64_t)head * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = __builtin_bit_cast(OpT, *(const u32x4*)(qp + 16 * ks + 8 * half));
  }

  // ---- staging of one K/V tile: global -> registers -> LDS.  Rows past
  // the prompt's end load row T-1 instead: their scores are masked (the key
  // is after every query), so they contribute exp(-inf) * finite = 0.
  constexpr int KCH = BN * D / 8 / 256;               // 16-byte K chunks per thread
  constexpr int VBL = (BN / 4) * (D / 8);             // 4x8 V blocks per tile
  u32x4 kreg[KCH], vreg[4];   // plain vectors: stay in registers
  const uint16_t* kbase = k + (int64_t)b * T * kvstride + (int64_t)g * D;
  const uint16_t* vbase = v + (int64_t)b * T * kvstride + (int64_t)g * D;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, row = c / KG, c8 = c % KG;
      const int key = min(k0 + row, T - 1);
      kreg[i] = *(const u32x4*)(kbase + (int64_t)key * kvstride + 8 * c8);
    }
    if (tid < VBL) {
      const int kg = tid / (D / 8), dg = tid % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(k0 + 4 * kg + r, T - 1);
        vreg[r] = *(const u32x4*)(vbase + (int64_t)key * kvstride + 8 * dg);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, row = c / KG, c8 = c % KG;
      *(u32x4*)&Ks[buf][row * D + 8 * (c8 ^ ksw(row))] = kreg[i];
    }
    if (tid < VBL) {
      const int kg = tid / (D / 8), dg = tid % (D / 8);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wd = dd >> 1, row = 8 * dg + dd;
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint2 pk;   // keys 0..3 of column dd
        pk.x = __builtin_amdgcn_perm(vreg[1][wd], vreg[0][wd], sel);
        pk.y = __builtin_amdgcn_perm(vreg[3][wd], vreg[2][wd], sel);
        *(uint2*)&Vt[buf][row * BN + 8 * ((kg >> 1) ^ vsw(row)) + 4 * (kg & 1)] = pk;
      }
    }
  };

  f32x16 o[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;

  const int kend = min(T, q0 + BM);                   // keys any row of the tile sees
  const int nkt = (kend + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1, k0 = j * BN;
    if (j + 1 < nkt) load_tile(k0 + BN);

    // wave-level causal skip: every key of the tile is after every query of the wave
    if (wave_live && k0 <= q0 + 32 * w + 31) {
      f32x16 sacc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[st][e] = 0.f;
        const int row = 32 * st + row_key(col);
        const uint16_t* krow = &Ks[buf][row * D];
        const int sw = ksw(row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          OpT a = __builtin_bit_cast(OpT, *(const u32x4*)(krow + 8 * ((2 * ks + half) ^ sw)));
          sacc[st] = mfma32(a, qop[ks], sacc[st]);
        }
      }
      // causal mask on tiles that reach past the wave's first query
      if (k0 + BN - 1 > q0 + 32 * w) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int r = 8 * (e >> 2) + 4 * half + (e & 3);
            if (k0 + 32 * st + row_key(r) > qrow) sacc[st][e] = -INFINITY;
          }
      }
      float rmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) rmax = fmaxf(rmax, sacc[st][e]);
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64)) * sl2;   // base-2 domain (sl2 > 0)
      // stale-max online softmax update
      const float m_new = fmaxf(m, rmax);
      const bool grow = m_new > m + kStale;           // also true when m = -inf and m_new finite
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - m_new)) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      }
      if (grow) m = m_new;
      const float msub = m == -INFINITY ? 0.f : m;   // fully masked rows so far: p = 0
      float p[2][16];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[st][e] = __builtin_amdgcn_exp2f(fmaf(sacc[st][e], sl2, -msub));
          lsum += p[st][e];
        }
      // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const OpT pop = pack8<OpT>(&p[st][8 * kb]);
          const int gr = 4 * st + 2 * kb + half;       // logical granule of the keys
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int row = 32 * dt + col;
            const uint16_t* vr = &Vt[buf][row * BN + 8 * (gr ^ vsw(row))];
            OpT a = __builtin_bit_cast(OpT, *(const u32x4*)vr);
            o[dt] = mfma32(a, pop, o[dt]);
          }
        }
    }
    if (j + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l for this lane's query column
  if (!wave_live || qrow >= T) return;
  const float l = lsum + __shfl_xor(lsum, 32, 64);
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

template <int D, bool F16>
hipError_t run(const CacheView& cv, int n, int T, const void* q, const void* k, const void* v,
               void* out, float sl2, hipStream_t s) {
  const int ntiles = (T + BM - 1) / BM;
  const int xcd_heads = (cv.n_q % 8 == 0 && (cv.n_q / 8) % (cv.n_q / cv.n_kv) == 0) ? 1 : 0;
  hipLaunchKernelGGL((k_prefill_mfma<D, F16>), dim3(cv.n_q, n, ntiles), dim3(256), 0, s, cv.n_q,
                     cv.n_kv, T, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                     (uint16_t*)out, sl2, ntiles, xcd_heads);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_mfma(const CacheView& cv, int n, int T, const void* q, const void* k,
                               const void* v, void* out, float sl2, hipStream_t s,
                               bool* handled) {
  *handled = true;
  const int io = io_dtype(cv.dtype);
  if (io == KVC_BF16) {
    if (cv.d == 128) return run<128, false>(cv, n, T, q, k, v, out, sl2, s);
    if (cv.d == 64) return run<64, false>(cv, n, T, q, k, v, out, sl2, s);
  } else if (io == KVC_F16) {
    if (cv.d == 128) return run<128, true>(cv, n, T, q, k, v, out, sl2, s);
    if (cv.d == 64) return run<64, true>(cv, n, T, q, k, v, out, sl2, s);
  }
  *handled = false;
  return hipSuccess;
}

}  // namespace kvfa
