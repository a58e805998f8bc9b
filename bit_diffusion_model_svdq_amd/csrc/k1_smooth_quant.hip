// k1: fused smoothing + per-group activation quantization + lora_down, gfx950.
//
// Computes the first factors of the SVDQuant dual-path forward (Terminology
// Entry, section 2.3, equation E4): x_hat = X diag(s)^-1 (the activation side
// of the outlier migration E1), its 4-bit quantization Q(x_hat) with one
// float32 scale per 64 channels, and the low-rank branch's down projection
// T = x_hat L1^T.  The abstract of the SVDQuant paper motivates the fusion:
// running the low-rank branch as a separate kernel re-reads the activations.
// Here X is read from HBM exactly once.
//
// Work split: one workgroup owns 16 rows (one MFMA row tile) and all of K;
// its 8 waves take every 8th 64-channel group.  In a wave, lane l holds row
// (l % 16) and the 16 consecutive channels 16 * (l / 16) .. +15 of the group,
// so the group's absmax is a 16-element local max plus two cross-lane steps,
// and the same registers are already the A operand of the bf16 MFMA (any
// channel order that A and B share leaves the dot product unchanged).
// x_hat enters the MFMA as a bf16 hi/lo pair, so T keeps ~16 significant bits.
// The 8 waves' T partials are summed in LDS in a fixed order (deterministic).
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kRows = 16;
constexpr int kThreads = kWaves * 64;

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <int RT>  // RT = r / 16 column tiles of T
__global__ __launch_bounds__(kThreads) void smooth_quant_lora_down_kernel(
    const uint16_t* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ L1, int r, uint8_t* __restrict__ qx, float* __restrict__ sx,
    float* __restrict__ T) {
  extern __shared__ float lds[];  // inv_s [K] | T partials [kWaves][16][r]
  float* inv_s = lds;
  float* tpart = lds + K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m0 = blockIdx.x * kRows;
  const int G = K / kGroup;

  // fl32(1 / s[k]): IEEE division, computed once per workgroup.
  for (int k = tid; k < K; k += kThreads) inv_s[k] = 1.0f / smooth[k];
  __syncthreads();

  const int row = m0 + (lane & 15);
  const bool row_ok = row < M;
  const int kseg = lane >> 4;
  f32x4 acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = wave; g < G; g += kWaves) {
    const int k0 = g * kGroup + kseg * 16;
    uint4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
    if (row_ok) {
      const uint4* p = reinterpret_cast<const uint4*>(X + (size_t)row * K + k0);
      xa = p[0];
      xb = p[1];
    }
    const uint32_t w[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    const float4* isp = reinterpret_cast<const float4*>(inv_s + k0);
    float is[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = isp[i];
      is[4 * i + 0] = v.x;
      is[4 * i + 1] = v.y;
      is[4 * i + 2] = v.z;
      is[4 * i + 3] = v.w;
    }
    float xh[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xh[2 * i] = bf16_lo(w[i]) * is[2 * i];
      xh[2 * i + 1] = bf16_hi(w[i]) * is[2 * i + 1];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float scale = amax / 7.0f;
    const float inv = amax > 0.f ? 7.0f / amax : 0.f;
    uint32_t pk[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float q = __builtin_rintf(xh[i] * inv);
      q = fminf(fmaxf(q, -7.0f), 7.0f);
      pk[i >> 3] |= (uint32_t(int(q)) & 0xFu) << (4 * (i & 7));
    }
    if (row_ok) {
      *reinterpret_cast<uint2*>(qx + (size_t)row * (K / 2) + k0 / 2) = make_uint2(pk[0], pk[1]);
      if (kseg == 0) sx[(size_t)row * G + g] = scale;
    }
    if constexpr (RT > 0) {
      bf16x8 ahi[2], alo[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = xh[8 * c + i];
          const __bf16 h = (__bf16)v;
          ahi[c][i] = h;
          alo[c][i] = (__bf16)(v - (float)h);
        }
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int n = t * 16 + (lane & 15);
        const uint4* lp = reinterpret_cast<const uint4*>(L1 + (size_t)n * K + k0);
        const bf16x8 b0 = as_bf16x8(lp[0]);
        const bf16x8 b1 = as_bf16x8(lp[1]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[0], b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[0], b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[1], b1, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[1], b1, acc[t], 0, 0, 0);
      }
    }
  }

  if constexpr (RT > 0) {
    // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + i.
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        tpart[(wave * 16 + 4 * (lane >> 4) + i) * r + t * 16 + (lane & 15)] = acc[t][i];
    __syncthreads();
    for (int e = tid; e < 16 * r; e += kThreads) {
      const int rr = e / r, c = e - (e / r) * r;
      float s = 0.f;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) s += tpart[(wv * 16 + rr) * r + c];
      if (m0 + rr < M) T[(size_t)(m0 + rr) * r + c] = s;
    }
  }
}

template <int RT>
hipError_t launch_rt(const uint16_t* X, int M, int K, int r, const float* smooth,
                     const uint16_t* L1, uint8_t* qx, float* sx, float* T, hipStream_t stream) {
  const size_t lds = (size_t)K * 4 + (size_t)kWaves * 16 * r * 4;
  auto kern = smooth_quant_lora_down_kernel<RT>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int blocks = (M + kRows - 1) / kRows;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, stream, X, M, K, smooth, L1, r, qx,
                     sx, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_smooth_quant_lora_down(const uint16_t* X, int M, int K, int r,
                                         const float* smooth, const uint16_t* L1, uint8_t* qx,
                                         float* sx, float* T, hipStream_t stream) {
  switch (r / 16) {
    case 0: return launch_rt<0>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 1: return launch_rt<1>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 2: return launch_rt<2>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 3: return launch_rt<3>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 4: return launch_rt<4>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 5: return launch_rt<5>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 6: return launch_rt<6>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 7: return launch_rt<7>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    case 8: return launch_rt<8>(X, M, K, r, smooth, L1, qx, sx, T, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace svdq
