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
// the terms stay below 2^8, far inside fp32/bf16 range.
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
  constexpr int KP = D + 8;         // padded K row (elements)
  constexpr int VP = BN + 8;        // padded V^T row (elements)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN][KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D][VP];

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
    const bool ok = qrow < T;
    const uint16_t* qp = q + ((int64_t)b * T + (ok ? qrow : 0)) * qstride + (int64_t)head * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 raw = ok ? *(const uint4*)(qp + 16 * ks + 8 * half) : make_uint4(0, 0, 0, 0);
      qop[ks] = __builtin_bit_cast(OpT, raw);
    }
  }

  // ---- staging of one K/V tile: global -> registers -> LDS
  constexpr int KCH = BN * D / 8 / 256;               // 16-byte K chunks per thread
  constexpr int VBL = (BN / 4) * (D / 8);             // 4x8 V blocks per tile
  uint4 kreg[KCH], vreg[4];
  const uint16_t* kbase = k + (int64_t)b * T * kvstride + (int64_t)g * D;
  const uint16_t* vbase = v + (int64_t)b * T * kvstride + (int64_t)g * D;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, row = c / (D / 8), c8 = c % (D / 8);
      const int key = k0 + row;
      kreg[i] = key < T ? *(const uint4*)(kbase + (int64_t)key * kvstride + 8 * c8)
                        : make_uint4(0, 0, 0, 0);
    }
    if (tid < VBL) {
      const int kg = tid / (D / 8), dg = tid % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * kg + r;
        vreg[r] = key < T ? *(const uint4*)(vbase + (int64_t)key * kvstride + 8 * dg)
                          : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i, row = c / (D / 8), c8 = c % (D / 8);
      *(uint4*)&Ks[buf][row][8 * c8] = kreg[i];
    }
    if (tid < VBL) {
      const int kg = tid / (D / 8), dg = tid % (D / 8);
      const uint32_t* r0 = (const uint32_t*)&vreg[0];
      const uint32_t* r1 = (const uint32_t*)&vreg[1];
      const uint32_t* r2 = (const uint32_t*)&vreg[2];
      const uint32_t* r3 = (const uint32_t*)&vreg[3];
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wd = dd >> 1;
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint2 pk;
        pk.x = __builtin_amdgcn_perm(r1[wd], r0[wd], sel);   // keys 0,1 of column dd
        pk.y = __builtin_amdgcn_perm(r3[wd], r2[wd], sel);   // keys 2,3
        *(uint2*)&Vt[buf][8 * dg + dd][4 * kg] = pk;
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
        const uint16_t* krow = &Ks[buf][32 * st + row_key(col)][8 * half];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          OpT a = __builtin_bit_cast(OpT, *(const uint4*)(krow + 16 * ks));
          sacc[st] = mfma32(a, qop[ks], sacc[st]);
        }
      }
      // scores -> base-2 domain, causal mask on diagonal tiles
      const bool diag = k0 + BN - 1 > q0 + 32 * w;
      float p[2][16];
      float rmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float x = sacc[st][e] * sl2;
          if (diag) {
            const int r = 8 * (e >> 2) + 4 * half + (e & 3);
            if (k0 + 32 * st + row_key(r) > qrow) x = -INFINITY;
          }
          p[st][e] = x;
          rmax = fmaxf(rmax, x);
        }
      rmax = fmaxf(rmax, __shfl_xor(rmax, 32, 64));
      // stale-max online softmax update
      const float m_new = fmaxf(m, rmax);
      const bool grow = m_new > m + kStale;           // also true when m = -inf and m_new finite
      const float m_use = grow ? m_new : m;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? (m == -INFINITY ? 0.f : exp2f(m - m_new)) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int i = 0; i < DT; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      }
      m = m_use;
      const float msub = m == -INFINITY ? 0.f : m;   // fully masked rows so far: p = 0
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[st][e] = exp2f(p[st][e] - msub);
          lsum += p[st][e];
        }
      // O^T += V^T P^T over 4 k-steps of 16 keys
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const OpT pop = pack8<OpT>(&p[st][8 * kb]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint16_t* vr = &Vt[buf][32 * dt + col][32 * st + 16 * kb + 8 * half];
            OpT a = __builtin_bit_cast(OpT, *(const uint4*)vr);
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
        hv[i] = F16 ? __builtin_bit_cast(uint16_t, (_Float16)y) : f32_to_bf16_bits(y);
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
