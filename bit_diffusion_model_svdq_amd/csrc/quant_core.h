// The activation quantizers' arithmetic (int4 and MXFP4), shared by every
// kernel that produces activation codes (the standalone quantize kernel and
// the fused small-K forwards), so that their codes and scales agree bit for bit.
//
// SVDQuant (Terminology Entry, section 2.3, equations E2-E4): the smoothed
// activation x_hat = x * fl32(1 / s) is cut into groups of 64 channels along
// K; a group's scale is amax / 7 and its codes are round(x_hat * (7 / amax)),
// both in float32.  A group whose absmax is below 2^-100 (zero included) is a
// zero group: scale 0, codes 0.
//
// Lane layout: the four lanes l, l ^ 16, l ^ 32, l ^ 48 of a wave hold one row
// of a group between them (16 channels each), so the group absmax is a local
// max plus two cross-lane steps.
//
// Rounding uses the float32 adder: for |y| <= 7.0000005,
// fl32(y + 1.5 * 2^23) = 1.5 * 2^23 + rne(y) exactly, so the low nibble of the
// sum's bit pattern is the code in two's complement.  |y| cannot exceed
// 7 * (1 + 2^-24) because inv = fl32(7 / amax), so no clamp is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {
namespace quant {

constexpr float kRound = 12582912.0f;   // 1.5 * 2^23
constexpr float kTinyGroup = 0x1p-100f;

// The row's group absmax from this lane's local max (lanes l ^ 16, l ^ 32 hold
// the rest of the row).
__device__ inline float row_group_absmax(float local) {
  local = fmaxf(local, __shfl_xor(local, 16));
  return fmaxf(local, __shfl_xor(local, 32));
}

// N smoothed values of one group row -> the scale's float32 bits and the
// rounding adder's results z (code = low nibble of the bits of z).
template <int N>
__device__ inline void int4_codes(const float* xh, float amax, uint32_t& scale_bits, float* z) {
  const bool coded = amax >= kTinyGroup;
  scale_bits = coded ? __float_as_uint(amax / 7.0f) : 0u;
  const float inv = coded ? 7.0f / amax : 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) z[i] = xh[i] * inv + kRound;  // two roundings: product, then code
}

// Two codes per byte from the rounding adder's results (low nibble = even channel).
__device__ inline uint32_t nib2(float ze, float zo) {
  const uint32_t e = __float_as_uint(ze), o = __float_as_uint(zo);
  return (e & 0x0Fu) | ((o << 4) & 0xF0u);
}

// 8 consecutive channels' codes -> one dword of packed nibbles.
__device__ inline uint32_t pack8(const float* z) {
  const uint32_t b0 = nib2(z[0], z[1]), b1 = nib2(z[2], z[3]);
  const uint32_t b2 = nib2(z[4], z[5]), b3 = nib2(z[6], z[7]);
  return __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
}

// MXFP4 (the OCP microscaling format): a block of 32 channels shares one E8M0
// scale byte, 2^(byte - 127), with byte = max(exponent field of the block
// absmax - 2, 0), i.e. the shared exponent floor(log2 amax) - 2 clamped at
// -127; each value becomes an FP4 E2M1 code of value / scale, rounded to
// nearest even with saturation at +-6, the sign kept for a value that rounds
// to zero.
__device__ inline uint32_t mx_scale_byte(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return (uint32_t)(ef - 2 > 0 ? ef - 2 : 0);
}

// 8 values of one block under its scale byte -> 8 FP4 codes in one dword
// (channel 2i in the low nibble of byte i).  v_cvt_scalef32_pk_fp4_f32 divides
// by the power-of-two scale and rounds, two values per instruction.  A block
// whose scale would be the subnormal 2^-127 (byte 0: absmax < 2^-125) is
// converted as v * 2^127 with scale 1 instead, which is exact.
__device__ inline uint32_t mx_codes8(const float* v, uint32_t byte) {
  float sc = __uint_as_float(byte << 23);
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v[i];
  if (byte == 0u) {
    sc = 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = v[i] * 0x1p127f;
  }
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[0], f[1], sc, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[2], f[3], sc, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[4], f[5], sc, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f[6], f[7], sc, 3);
  return w;
}

}  // namespace quant
}  // namespace svdq
