// Shared tail of the two GEMM kernels (int4 and MXFP4): adds the low-rank
// branch's up projection T L2^T (Terminology Entry, section 2.3, E4 second
// term) and the bias to a finished fp32 output tile, optionally applies the
// MLP activation, rounds to bf16 and stores the tile through LDS as 16-byte
// row segments.
#pragma once

#include "svdq_internal.h"

namespace svdq {
namespace tail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// acc[tm][tn] holds the 16x16 tile (wr + 16 tm, wc + 16 tn) of the block's
// BM x BN output in the MFMA result layout (lane l: column l % 16, rows
// 4 (l / 16) + i).  T holds t_slices partial sums of M x r floats, t_stride
// floats apart, added in slice order.  T (times `scale`, a power of two) is
// split into a bf16 hi/lo pair and enters bf16 MFMAs whose accumulator input
// is the tile, so the branch keeps ~16 significant bits of T.
template <int TM, int TN>
__device__ inline void lowrank_accumulate(f32x4 (&acc)[TM][TN], const float* __restrict__ T,
                                          int t_slices, long t_stride, int r,
                                          const uint16_t* __restrict__ L2, int m0, int n0,
                                          int row1, int col1, int wr, int wc, int lane,
                                          float scale) {
  const int fr = lane & 15;
  const int fk = lane >> 4;
  for (int j0 = 0; j0 < r; j0 += 32) {
    const int j = j0 + 8 * fk;
    const bool j_ok = j < r;
    bf16x8 thi[TM], tlo[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int m = m0 + wr + 16 * t + fr;
      float tv[8];
      if (j_ok && m < row1) {
        const float* tp = T + (size_t)m * r + j;
        float4 a = *reinterpret_cast<const float4*>(tp);
        float4 b = *reinterpret_cast<const float4*>(tp + 4);
        for (int sl = 1; sl < t_slices; ++sl) {
          const float4 a2 = *reinterpret_cast<const float4*>(tp + sl * t_stride);
          const float4 b2 = *reinterpret_cast<const float4*>(tp + sl * t_stride + 4);
          a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
          b.x += b2.x; b.y += b2.y; b.z += b2.z; b.w += b2.w;
        }
        tv[0] = a.x * scale; tv[1] = a.y * scale; tv[2] = a.z * scale; tv[3] = a.w * scale;
        tv[4] = b.x * scale; tv[5] = b.y * scale; tv[6] = b.z * scale; tv[7] = b.w * scale;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) tv[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)tv[e];
        thi[t][e] = h;
        tlo[t][e] = (__bf16)(tv[e] - (float)h);
      }
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n0 + wc + 16 * tn + fr;
      const bf16x8 lf = (j_ok && n < col1)
                            ? as_bf16x8(*reinterpret_cast<const uint4*>(L2 + (size_t)n * r + j))
                            : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(thi[tm], lf, acc[tm][tn], 0, 0, 0);
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tlo[tm], lf, acc[tm][tn], 0, 0, 0);
      }
    }
  }
}

// GELU in its tanh form (Hendrycks and Gimpel, "Gaussian Error Linear Units",
// section 2), the activation between a DiT MLP's up and down projections:
//   gelu(v) = 0.5 v (1 + tanh(u)),  u = sqrt(2/pi) (v + 0.044715 v^3).
// Since 0.5 (1 + tanh u) = 1 / (1 + e^(-2u)), it is evaluated as
// v / (1 + 2^z) with z = -2 u log2(e): one exp2 and one reciprocal on the
// transcendental unit.  Large negative v gives 2^z = inf and -0; large
// positive v gives v.
__device__ inline float gelu_tanh(float v) {
  constexpr float c0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float c1 = c0 * 0.044715f;
  const float z = v * __builtin_fmaf(v * v, c1, c0);
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// Bias, the activation (act == kActGeluTanh: gelu_tanh of the float32 sum),
// bf16 rounding and the store of the tile through LDS as 16-byte row
// segments.  lds must hold BM * BN * 2 bytes; the caller has synchronized the
// block so that the space is free.
template <int TM, int TN, int BM, int BN, int THREADS>
__device__ inline void bias_store(f32x4 (&acc)[TM][TN], const uint16_t* __restrict__ bias,
                                  uint16_t* __restrict__ Y, int ldy, int m0, int n0, int row1,
                                  int col1, int wr, int wc, int lane, int tid, uint8_t* lds,
                                  int act) {
  const int fr = lane & 15;
  const int fk = lane >> 4;

  // bias, bf16, then the tile goes through LDS (columns swizzled by 16 elements
  // per group of 4 rows, so that the 4 row groups of a write hit distinct banks)
  // and leaves as 16-byte row segments.
  uint16_t* otile = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int col = wc + 16 * tn + fr;
    const int n = n0 + col;
    const float bv = (bias && n < col1) ? __uint_as_float(uint32_t(bias[n]) << 16) : 0.f;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wr + 16 * tm + 4 * fk + i;
        float v = acc[tm][tn][i] + bv;
        if (act == kActGeluTanh) v = gelu_tanh(v);
        otile[row * BN + (col ^ (16 * ((row >> 2) & 3)))] = __builtin_bit_cast(uint16_t, (__bf16)v);
      }
  }
  __syncthreads();
  constexpr int CPR = BN / 8;   // 16-byte chunks per output row
  for (int c = tid; c < BM * CPR; c += THREADS) {
    const int row = c / CPR, ch = c - (c / CPR) * CPR;
    const int m = m0 + row, n = n0 + 8 * ch;
    if (m < row1 && n < col1) {
      const uint4 v = *reinterpret_cast<const uint4*>(otile + row * BN + 8 * (ch ^ (2 * ((row >> 2) & 3))));
      *reinterpret_cast<uint4*>(Y + (size_t)m * ldy + n) = v;
    }
  }
}

}  // namespace tail
}  // namespace svdq

namespace svdq {
namespace tail {

template <int TM, int TN, int BM, int BN, int THREADS>
__device__ inline void lowrank_bias_store(f32x4 (&acc)[TM][TN], const float* __restrict__ T,
                                          int t_slices, long t_stride, int r,
                                          const uint16_t* __restrict__ L2,
                                          const uint16_t* __restrict__ bias,
                                          uint16_t* __restrict__ Y, int ldy, int m0, int n0,
                                          int row1, int col1, int wr, int wc, int lane, int tid,
                                          uint8_t* lds, int act) {
  lowrank_accumulate<TM, TN>(acc, T, t_slices, t_stride, r, L2, m0, n0, row1, col1, wr, wc, lane,
                             1.0f);
  bias_store<TM, TN, BM, BN, THREADS>(acc, bias, Y, ldy, m0, n0, row1, col1, wr, wc, lane, tid,
                                      lds, act);
}

}  // namespace tail
}  // namespace svdq
