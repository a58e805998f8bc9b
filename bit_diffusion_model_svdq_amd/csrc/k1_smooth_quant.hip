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
// each of its 8 waves takes a contiguous run of 64-channel groups and issues
// the loads of up to 6 groups at once (the whole run for K <= 3072), so
// that a workgroup has its entire slice of X in flight.  Lane
// l holds row (l % 16) and, of each group, channels 8 * (l / 16) + 0..7 and
// 32 + 8 * (l / 16) + 0..7: exactly the A operand layout of two 16x16x32 bf16
// MFMAs, and two 16-byte loads that cover 64 contiguous bytes per row.  The
// group absmax is a local max plus two cross-lane steps.
//
// Rounding to the integer code uses the float32 adder: for |y| <= 7.0000005,
// fl32(y + 1.5 * 2^23) = 1.5 * 2^23 + rne(y) exactly, so the low byte of its
// bit pattern is the code as an int8 and its low nibble is the packed code.
// |y| cannot exceed 7 * (1 + 2^-24) because inv = fl32(7 / amax), so no clamp
// is needed.  x_hat enters the MFMA as a bf16 hi/lo pair (hi = x_hat with the
// low 16 bits cleared, lo = bf16(x_hat - hi), an exact difference), so T keeps
// ~16 significant bits.  The 8 waves' T partials are summed in LDS in a fixed
// order (deterministic).
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kRows = 16;
constexpr int kThreads = kWaves * 64;
constexpr float kRound = 12582912.0f;  // 1.5 * 2^23

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t cvt_bf16x2(float a, float b) {  // round-to-nearest-even pair
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// Two codes per byte from the rounding adder's results (low nibble = even channel).
__device__ inline uint32_t nib2(float ze, float zo) {
  const uint32_t e = __float_as_uint(ze), o = __float_as_uint(zo);
  return (e & 0x0Fu) | ((o << 4) & 0xF0u);
}

__device__ inline uint32_t pack8(const float* z) {  // 8 codes -> one dword
  const uint32_t b0 = nib2(z[0], z[1]), b1 = nib2(z[2], z[3]);
  const uint32_t b2 = nib2(z[4], z[5]), b3 = nib2(z[6], z[7]);
  return __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
}

template <int RT>  // RT = r / 16 column tiles of T
__global__ __launch_bounds__(kThreads) void smooth_quant_lora_down_kernel(
    const uint16_t* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ L1, int r, uint8_t* __restrict__ qx, float* __restrict__ sx,
    float* __restrict__ T) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // inv_s [K] | T partials [kWaves][16][r]
  float* inv_s = lds;
  float* tpart = lds + K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int m0 = blockIdx.x * kRows;
  const int G = K / kGroup;
  const int per_wave = (G + kWaves - 1) / kWaves;
  const int g_begin = min(G, wave * per_wave);
  const int g_end = min(G, g_begin + per_wave);

  // fl32(1 / s[k]): IEEE division, once per workgroup.
  for (int k = tid; k < K; k += kThreads) inv_s[k] = 1.0f / smooth[k];

  const int row = m0 + (lane & 15);
  const bool row_ok = row < M;
  const int fk = lane >> 4;
  // rows past M read row M-1 (never stored): every load is unconditional, so
  // the compiler issues them back to back instead of draining at branch joins
  const uint16_t* xrow = X + (size_t)min(row, M - 1) * K + 8 * fk;
  f32x4 acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  __syncthreads();  // inv_s ready

  // Process one group whose X pieces (xa: channels 8fk..+7, xb: 32+8fk..+7) are in registers.
  // The codes and the scale come back in registers: stores share the in-order
  // vector-memory counter with loads, so a store issued here would make the
  // next group's wait for its prefetched L1 fragments wait for the store too.
  auto process = [&](int g, uint4 xa, uint4 xb, const uint4* lb, uint2& out, float& out_scale) {
    const int k0 = g * kGroup + 8 * fk;
    const uint32_t w[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    float xh[16];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f32x4 i0 = *reinterpret_cast<const f32x4*>(inv_s + k0 + 32 * c);
      const f32x4 i1 = *reinterpret_cast<const f32x4*>(inv_s + k0 + 32 * c + 4);
      const float is[8] = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xh[8 * c + 2 * i] = __uint_as_float(w[4 * c + i] << 16) * is[2 * i];
        xh[8 * c + 2 * i + 1] = __uint_as_float(w[4 * c + i] & 0xFFFF0000u) * is[2 * i + 1];
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const float scale = amax / 7.0f;
    const float inv = amax > 0.f ? 7.0f / amax : 0.f;
    float z[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = xh[i] * inv + kRound;  // two roundings: product, then code
    out.x = pack8(z);
    out.y = pack8(z + 8);
    out_scale = scale;
    if constexpr (RT > 0) {
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b0 = __float_as_uint(xh[2 * i]), b1 = __float_as_uint(xh[2 * i + 1]);
        hi[i] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // upper halves: truncated bf16 pair
        lo[i] = cvt_bf16x2(xh[2 * i] - __uint_as_float(b0 & 0xFFFF0000u),
                           xh[2 * i + 1] - __uint_as_float(b1 & 0xFFFF0000u));
      }
      const bf16x8 ahi0 = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
      const bf16x8 ahi1 = as_bf16x8(make_uint4(hi[4], hi[5], hi[6], hi[7]));
      const bf16x8 alo0 = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
      const bf16x8 alo1 = as_bf16x8(make_uint4(lo[4], lo[5], lo[6], lo[7]));
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const bf16x8 b0 = as_bf16x8(lb[2 * t]), b1 = as_bf16x8(lb[2 * t + 1]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi0, b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo0, b0, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi1, b1, acc[t], 0, 0, 0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo1, b1, acc[t], 0, 0, 0);
      }
    }
  };
  constexpr int NL = RT > 0 ? 2 * RT : 1;
  constexpr int kChunk = RT > 4 ? 3 : 6;  // groups whose X loads are in flight together
  auto load_l1 = [&](int g, uint4* lb) {
    if constexpr (RT > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const uint16_t* lp = L1 + (size_t)(t * 16 + (lane & 15)) * K + g * kGroup + 8 * fk;
        lb[2 * t] = *reinterpret_cast<const uint4*>(lp);
        lb[2 * t + 1] = *reinterpret_cast<const uint4*>(lp + 32);
      }
    }
  };

  for (int c0 = g_begin; c0 < g_end; c0 += kChunk) {
    // all X loads of the chunk first
    uint4 xa[kChunk], xb[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int gj = min(c0 + j, g_end - 1);   // groups past the run re-read its last one (unused)
      xa[j] = *reinterpret_cast<const uint4*>(xrow + gj * kGroup);
      xb[j] = *reinterpret_cast<const uint4*>(xrow + gj * kGroup + 32);
    }
    uint4 lbc[NL], lbn[NL];
#pragma unroll
    for (int e = 0; e < NL; ++e) lbn[e] = make_uint4(0u, 0u, 0u, 0u);
    load_l1(c0, lbc);
    uint2 codes[kChunk];
    float scales[kChunk];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      codes[j] = make_uint2(0u, 0u);
      scales[j] = 0.f;
      if (c0 + j < g_end) {
        if (j + 1 < kChunk && c0 + j + 1 < g_end) load_l1(c0 + j + 1, lbn);
        process(c0 + j, xa[j], xb[j], lbc, codes[j], scales[j]);
#pragma unroll
        for (int e = 0; e < NL; ++e) lbc[e] = lbn[e];
      }
    }
    if (row_ok) {
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (c0 + j < g_end) {
          uint8_t* qrow = qx + (size_t)row * (K / 2) + (c0 + j) * 32 + 4 * fk;
          *reinterpret_cast<uint32_t*>(qrow) = codes[j].x;
          *reinterpret_cast<uint32_t*>(qrow + 16) = codes[j].y;
          if (fk == 0) sx[(size_t)row * G + c0 + j] = scales[j];
        }
      }
    }
  }

  if constexpr (RT > 0) {
    // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + i.
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        tpart[(wave * 16 + 4 * fk + i) * r + t * 16 + (lane & 15)] = acc[t][i];
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
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
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
