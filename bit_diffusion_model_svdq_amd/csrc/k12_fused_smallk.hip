// The whole SVDQuant forward in one kernel, for small K (K <= 1280).
//
// Terminology Entry, section 2.3, equation E4: Y = Q(x_hat) Q(R) + x_hat L1^T
// L2^T + b with x_hat = X diag(s)^-1 (E1) and Q the per-64-channel int4
// quantizer (E2, E3).  At small K the two-kernel forward (quantize, then GEMM)
// is latency-bound: each kernel is a short dependent chain of loads, and qx,
// sx and T make a round trip through HBM.  Here one workgroup takes 16 token
// rows and 128 NT output columns and does everything in one launch: X is read
// once, the codes never leave LDS.  Every workgroup streams its whole column
// slice of W through its compute unit (W is reused over 16 rows only), so the
// path pays off while the layer's work is small: measured on MI355X, one
// latency-bound launch of about 9 us against 14-21 us for the two kernels up
// to about 100 group-tiles (16 x 16 x 64 MFMA blocks) per compute unit, and a
// tie at 400.  The host plan takes it up to 256 per compute unit.
//
// Phases of a workgroup (8 waves):
//   1. every load issued up front, in the order the values are used: s, the
//      wave's groups of X and their L1 rows, the workgroup's weight scales and
//      bias (coalesced, for LDS), the L2 rows of the tail, then the first
//      kDepth pairs of groups of the wave's W fragments.  A wave's loads complete in issue order (one in-order counter),
//      so a value used before an earlier-issued one would wait for it; and a
//      load issued right before its use would expose its whole latency.  The
//      loads are unconditional (clamped addresses; NULL L1, L2 or bias read a
//      valid dummy address and are masked), so none sits behind a branch;
//   2. fl32(1 / s) into LDS, then each wave quantizes groups wave, wave + 8,
//      ... of the 16 rows with quant_core.h's arithmetic (bit-identical to
//      the standalone quantize kernel) into MFMA-ready int8 fragments in LDS,
//      and accumulates its partial T = x_hat L1^T (bf16 hi/lo MFMAs);
//   3. the waves' partial T summed in a fixed order;
//   4. the int4 GEMM: per group, one A fragment from LDS against each wave's
//      NT column tiles of W, read straight from L2 kDepth pairs of groups
//      ahead, and the exact scale epilogue of the W4A4 GEMM kernel;
//   5. 1/256, bias, T L2^T (bf16 hi/lo), activation, bf16 store through LDS.
//
// Operand layout.  The int8 MFMA sums over K, so A and B only have to agree
// on which channel each (lane group, byte) slot holds, and each MFMA must see
// one group only (one scale per group).  W is read 16 bytes per lane: lane
// group q = l / 16 of a column's four takes bytes 16 q .. 16 q + 15 of a pair
// of groups (64 bytes: 16 rows x 64 bytes per load, half a line each, where
// 8 bytes per lane would use a quarter).  Lanes 0-31 then hold the pair's
// first group, lanes 32-63 its second; two v_permlane32_swap per column tile
// trade half of each, so that every lane group holds 16 channels of both
// groups: lane groups 0, 1, 2, 3 hold channel blocks 1, 3, 0, 2 (block b =
// channels 16 b .. 16 b + 15).  The quantizer writes its A fragments to the
// lane group that holds its block in that order.  A packed dword of 8
// channels widens in two ALU ops to [c0 c2 c4 c6] and [c1 c3 c5 c7] (each
// code times 16), and the quantizer's codes go in the same order.  Both
// operands carry the factor 16, so the integer products are 256 times the
// code products, as in the W4A4 GEMM kernel.
#include <atomic>

#include "gemm_tail.h"
#include "quant_core.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kFW = 8;                       // waves per workgroup
constexpr int kFThreads = 64 * kFW;
constexpr int kFusedMaxK = 1280;             // 20 groups
constexpr int kFusedMaxRank = 32;            // register budget: L1 of all the wave's groups is preloaded
constexpr int kFusedMaxN = 2560;             // beyond, the re-quantization per column slice costs more
constexpr int kDepth = 2;                    // pairs of groups of W in flight per wave
constexpr int kMagicBits = 0x4B400000;       // 1.5 * 2^23
constexpr float kMagic = 12582912.0f;

// LDS: inv_s [K] f32 | afrag [G][64 lanes] 16 B | sxl [G][16] f32 | tfin [16][r] f32
// | sws [G][bn] f32 (weight scales, group-major) | bias [bn] f32
// | scratch: the waves' partial T [8][16][r] f32, later the output tile [16][bn] bf16.
struct FusedLds {
  int inv_s, afrag, sxl, tfin, sws, bias, scratch, bytes;
};
__host__ __device__ inline FusedLds fused_lds(int K, int r, int bn) {
  const int G = K / kGroup;
  FusedLds l;
  l.inv_s = 0;
  l.afrag = K * 4;
  l.sxl = l.afrag + G * 1024;
  l.tfin = l.sxl + G * 64;
  l.sws = l.tfin + 16 * r * 4;
  l.bias = l.sws + G * bn * 4;
  l.scratch = l.bias + bn * 4;
  const int tpart = kFW * 16 * r * 4, out = 16 * bn * 2;
  l.bytes = l.scratch + (tpart > out ? tpart : out);
  return l;
}

__device__ inline i32x4 widen_even_odd(uint32_t lo, uint32_t hi) {
  return i32x4{(int)((lo << 4) & 0xF0F0F0F0u), (int)(lo & 0xF0F0F0F0u),
               (int)((hi << 4) & 0xF0F0F0F0u), (int)(hi & 0xF0F0F0F0u)};
}

// Four codes (the low nibbles of the rounding adder's bit patterns) as four
// int8 bytes of value 16 q, in argument order.
__device__ inline uint32_t gather4(float a, float b, float c, float d) {
  const uint32_t ab = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0C0C0400u);
  const uint32_t cd = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x04000C0Cu);
  return ((ab | cd) << 4) & 0xF0F0F0F0u;
}

__device__ inline uint32_t cvt_bf16x2(float a, float b) {  // round-to-nearest-even pair
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ inline bf16x8 bf16x8_of(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// NT: column tiles of 16 per wave; NG: groups a wave quantizes at most
// (ceil(G / 8): 2 up to K = 1024, 3 up to K = 1280).
template <int NT, int NG>
__global__ __launch_bounds__(kFThreads, 1) void w4a4_fused_smallk_kernel(
    const uint16_t* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ L1, int r, const uint16_t* __restrict__ L2,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scales,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int N, int act,
    uint8_t* __restrict__ dbg_qx, float* __restrict__ dbg_sx) {
  constexpr int BN = 16 * NT * kFW;
  constexpr int RTMAX = kFusedMaxRank / 16;
  constexpr int SWPER = (BN * 8 * NG + kFThreads - 1) / kFThreads;   // weight scales per thread
  constexpr int BPER = (BN + kFThreads - 1) / kFThreads;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const FusedLds LL = fused_lds(K, r, BN);
  float* inv_s = reinterpret_cast<float*>(lds + LL.inv_s);
  uint4* afrag = reinterpret_cast<uint4*>(lds + LL.afrag);
  float* sxl = reinterpret_cast<float*>(lds + LL.sxl);
  float* tfin = reinterpret_cast<float*>(lds + LL.tfin);
  float* sws = reinterpret_cast<float*>(lds + LL.sws);
  float* bias_l = reinterpret_cast<float*>(lds + LL.bias);
  float* tpart = reinterpret_cast<float*>(lds + LL.scratch);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const int G = K / kGroup;
  const int KB = K / 2;
  const int RT = r / 16;
  const int m0 = blockIdx.x * 16;
  const int n0 = blockIdx.y * BN;
  const int wc = wave * 16 * NT;
  const int row = min(m0 + fr, M - 1);     // rows past M quantize a valid row, never stored

  // ---- 1. loads, in order of use
  constexpr int kSPer = kFusedMaxK / kFThreads + 1;
  float sv[kSPer];
#pragma unroll
  for (int i = 0; i < kSPer; ++i) sv[i] = smooth[min(tid + i * kFThreads, K - 1)];
  const int ng = wave < G ? (G - wave + kFW - 1) / kFW : 0;   // groups this wave quantizes (<= NG)
  uint4 xa[NG], xb[NG], la[NG][RTMAX], lb[NG][RTMAX];
  const uint16_t* xrow = X + (size_t)row * K + 16 * fk;
  const uint16_t* l1b = r > 0 ? L1 : X;                      // a valid dummy for r = 0
  const int l1k = r > 0 ? K : 0;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int g = min(wave + kFW * i, G - 1);
    xa[i] = *reinterpret_cast<const uint4*>(xrow + g * kGroup);
    xb[i] = *reinterpret_cast<const uint4*>(xrow + g * kGroup + 8);
  }
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int g = min(wave + kFW * i, G - 1);
#pragma unroll
    for (int j = 0; j < RTMAX; ++j) {
      const uint16_t* lp = l1b + (size_t)min(16 * j + fr, max(r, 1) - 1) * l1k + (r > 0 ? g * kGroup + 16 * fk : 0);
      la[i][j] = *reinterpret_cast<const uint4*>(lp);
      lb[i][j] = *reinterpret_cast<const uint4*>(lp + 8);
    }
  }
  // the workgroup's weight scales: rows n0 .. n0 + BN - 1 of [N][G] are one
  // contiguous run (rows past N: the last row); into LDS group-major
  const int nsw = BN * G;
  float swr[SWPER];
#pragma unroll
  for (int i = 0; i < SWPER; ++i) {
    const int e = min(tid + i * kFThreads, nsw - 1);
    const int nr = e / G;
    swr[i] = w_scales[(size_t)min(n0 + nr, N - 1) * G + (e - nr * G)];
  }
  const uint16_t* bb = bias ? bias : X;
  uint16_t brr[BPER];
#pragma unroll
  for (int i = 0; i < BPER; ++i) brr[i] = bb[bias ? min(n0 + min(tid + i * kFThreads, BN - 1), N - 1) : 0];
  int ncol[NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) ncol[tn] = min(n0 + wc + 16 * tn + fr, N - 1);
  const uint16_t* l2b = r > 0 ? L2 : X;
  const int jq = min(8 * fk, max(r, 8) - 8);                  // ranks 8 fk .. + 7 of the one chunk
  uint4 l2v[NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) l2v[tn] = *reinterpret_cast<const uint4*>(l2b + (r > 0 ? (size_t)ncol[tn] * r + jq : 0));

  // W, 16 bytes per lane: pair p of groups, bytes 16 fk of its 64; when G is
  // odd the last pair's second group does not exist and its lanes re-read the
  // first group (used with weight scale 0)
  const int G2 = (G + 1) / 2;
  const uint8_t* wrow[NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) wrow[tn] = Wq + (size_t)ncol[tn] * KB;
  uint4 wring[kDepth][NT];
  auto load_w = [&](int slot, int p) {
    const int off0 = min(p, G2 - 1) * 64 + 16 * fk;
    const int off = off0 + 16 > KB ? off0 - 32 : off0;
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) wring[slot][tn] = *reinterpret_cast<const uint4*>(wrow[tn] + off);
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_w(d, d);

  // ---- 2. 1/s, the weight scales and the bias into LDS; then quantize and partial T
#pragma unroll
  for (int i = 0; i < kSPer; ++i) inv_s[min(tid + i * kFThreads, K - 1)] = 1.0f / sv[i];  // duplicates equal
#pragma unroll
  for (int i = 0; i < SWPER; ++i) {
    const int e = tid + i * kFThreads;
    if (e < nsw) {
      const int nr = e / G;
      sws[(e - nr * G) * BN + nr] = swr[i];
    }
  }
#pragma unroll
  for (int i = 0; i < BPER; ++i)
    if (tid + i * kFThreads < BN) bias_l[tid + i * kFThreads] = bias ? __uint_as_float(uint32_t(brr[i]) << 16) : 0.f;
  lds_barrier();

  f32x4 at[RTMAX];
#pragma unroll
  for (int j = 0; j < RTMAX; ++j) at[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the lane group of the GEMM that holds this lane's channel block fk
  const int aslot = (fk >> 1) | ((~fk & 1) << 1);
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    if (i < ng) {
      const int g = wave + kFW * i;
      const uint32_t w[8] = {xa[i].x, xa[i].y, xa[i].z, xa[i].w, xb[i].x, xb[i].y, xb[i].z, xb[i].w};
      const float* is = inv_s + g * kGroup + 16 * fk;
      float xh[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xh[2 * e] = __uint_as_float(w[e] << 16) * is[2 * e];
        xh[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u) * is[2 * e + 1];
      }
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(xh[e]));
      amax = quant::row_group_absmax(amax);
      uint32_t scale;
      float z[16];
      quant::int4_codes<16>(xh, amax, scale, z);
      afrag[g * 64 + 16 * aslot + fr] =
          make_uint4(gather4(z[0], z[2], z[4], z[6]), gather4(z[1], z[3], z[5], z[7]),
                     gather4(z[8], z[10], z[12], z[14]), gather4(z[9], z[11], z[13], z[15]));
      if (fk == 0) sxl[g * 16 + fr] = __uint_as_float(scale);
      if (dbg_qx && blockIdx.y == 0 && m0 + fr < M) {
        *reinterpret_cast<uint2*>(dbg_qx + (size_t)(m0 + fr) * KB + g * 32 + 8 * fk) =
            make_uint2(quant::pack8(z), quant::pack8(z + 8));
        if (fk == 0) dbg_sx[(size_t)(m0 + fr) * G + g] = __uint_as_float(scale);
      }
      // lora_down: x_hat as a bf16 hi/lo pair (hi truncated, lo the exact rest rounded)
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t b0 = __float_as_uint(xh[2 * e]), b1 = __float_as_uint(xh[2 * e + 1]);
        hi[e] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
        lo[e] = cvt_bf16x2(xh[2 * e] - __uint_as_float(b0 & 0xFFFF0000u),
                           xh[2 * e + 1] - __uint_as_float(b1 & 0xFFFF0000u));
      }
      const bf16x8 ahi0 = bf16x8_of(make_uint4(hi[0], hi[1], hi[2], hi[3]));
      const bf16x8 ahi1 = bf16x8_of(make_uint4(hi[4], hi[5], hi[6], hi[7]));
      const bf16x8 alo0 = bf16x8_of(make_uint4(lo[0], lo[1], lo[2], lo[3]));
      const bf16x8 alo1 = bf16x8_of(make_uint4(lo[4], lo[5], lo[6], lo[7]));
#pragma unroll
      for (int j = 0; j < RTMAX; ++j) {
        if (j < RT) {
          const bf16x8 b0 = bf16x8_of(la[i][j]);
          const bf16x8 b1 = bf16x8_of(lb[i][j]);
          at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi0, b0, at[j], 0, 0, 0);
          at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo0, b0, at[j], 0, 0, 0);
          at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi1, b1, at[j], 0, 0, 0);
          at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo1, b1, at[j], 0, 0, 0);
        }
      }
    }
  }

  // ---- 3. T = the waves' partials summed in wave order (16x16 result layout:
  // lane l holds column l % 16, rows 4 (l / 16) + i)
#pragma unroll
  for (int j = 0; j < RTMAX; ++j)
    if (j < RT)
#pragma unroll
      for (int i = 0; i < 4; ++i) tpart[(wave * 16 + 4 * fk + i) * r + 16 * j + fr] = at[j][i];
  lds_barrier();
  for (int e = tid; e < 16 * r; e += kFThreads) {
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < kFW; ++wv) s += tpart[wv * 16 * r + e];
    tfin[e] = s;
  }
  lds_barrier();   // tfin, afrag and sxl are complete; tpart is free

  // ---- 4. the GEMM over pairs of groups, kDepth pairs of W in flight
  f32x4 acc[1][NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) acc[0][tn] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x4 cmagic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};
  const int Gp2 = (G2 + kDepth - 1) / kDepth * kDepth;
  for (int p0 = 0; p0 < Gp2; p0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      // a fence per slot: left free, the scheduler hoists every slot's work to
      // the top of the loop and waits there for all the loads in flight
      __builtin_amdgcn_sched_barrier(0);
      // trade halves between lanes 0-31 (first group) and 32-63 (second)
      uint32_t wa[NT][2], wb[NT][2];
#pragma unroll
      for (int tn = 0; tn < NT; ++tn) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(wring[d][tn].z, wring[d][tn].x, false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(wring[d][tn].w, wring[d][tn].y, false, false);
        wa[tn][0] = s0[0];
        wa[tn][1] = s1[0];
        wb[tn][0] = s0[1];
        wb[tn][1] = s1[1];
      }
      load_w(d, p0 + d + kDepth);   // past the range: clamped repeats, never used
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int g = 2 * (p0 + d) + h;
        const int ga = min(g, G - 1);
        const bool real = g < G;
        const uint4 araw = afrag[ga * 64 + lane];
        const i32x4 a = i32x4{(int)araw.x, (int)araw.y, (int)araw.z, (int)araw.w};
        const f32x4 sxv = *reinterpret_cast<const f32x4*>(sxl + ga * 16 + 4 * fk);
        i32x4 dres[NT];
        float swv[NT];
#pragma unroll
        for (int tn = 0; tn < NT; ++tn) {
          const uint32_t* wv = h ? wb[tn] : wa[tn];
          dres[tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, widen_even_odd(wv[0], wv[1]), cmagic, 0, 0, 0);
          swv[tn] = real ? sws[ga * BN + wc + 16 * tn + fr] : 0.f;
        }
#pragma unroll
        for (int tn = 0; tn < NT; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float t = __builtin_fmaf(__int_as_float(dres[tn][i]), swv[tn], -kMagic * swv[tn]);
            acc[0][tn][i] = __builtin_fmaf(t, sxv[i], acc[0][tn][i]);
          }
      }
    }
  }

  // ---- 5. 1/256, bias, T L2^T (r <= 32: one chunk of 32 ranks), activation, store
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) {
    const float bv = bias_l[wc + 16 * tn + fr];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][tn][i] = acc[0][tn][i] * (1.0f / 256.0f) + bv;
  }
  if (r > 0) {
    const bool j_ok = 8 * fk < r;
    const float* tp = tfin + fr * r + jq;
    uint32_t thi[4], tlo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = j_ok ? tp[2 * e] : 0.f, v1 = j_ok ? tp[2 * e + 1] : 0.f;
      const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
      thi[e] = uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
      tlo[e] = cvt_bf16x2(v0 - (float)h0, v1 - (float)h1);
    }
    const bf16x8 th = bf16x8_of(make_uint4(thi[0], thi[1], thi[2], thi[3]));
    const bf16x8 tl = bf16x8_of(make_uint4(tlo[0], tlo[1], tlo[2], tlo[3]));
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) {
      const bf16x8 l = bf16x8_of(j_ok ? l2v[tn] : make_uint4(0u, 0u, 0u, 0u));
      acc[0][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, l, acc[0][tn], 0, 0, 0);
      acc[0][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl, l, acc[0][tn], 0, 0, 0);
    }
  }
  uint16_t* otile = reinterpret_cast<uint16_t*>(lds + LL.scratch);
  tail::store_tile<1, NT, 16, BN, kFThreads>(acc, nullptr, Y, N, m0, n0, M, N, 0, wc, lane, tid,
                                             [&](int rr) { return otile + rr * BN; }, act);
}

// Lets every instantiation use up to the compute unit's 160 KB of LDS (once per
// instantiation; concurrent first calls set the same value).
template <int NT, int NG>
hipError_t allow_lds() {
  static std::atomic<bool> done{false};
  if (done.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(w4a4_fused_smallk_kernel<NT, NG>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}

template <int NT, int NG>
hipError_t launch_nt(const uint16_t* X, int M, int K, int N, int r, const float* smooth,
                     const uint16_t* L1, const uint16_t* L2, const uint8_t* Wq,
                     const float* w_scales, const uint16_t* bias, uint16_t* Y, int act,
                     uint8_t* dbg_qx, float* dbg_sx, hipStream_t stream) {
  constexpr int BN = 16 * NT * kFW;
  const FusedLds l = fused_lds(K, r, BN);
  const hipError_t e = allow_lds<NT, NG>();
  if (e != hipSuccess) return e;
  const dim3 grid((M + 15) / 16, (N + BN - 1) / BN);
  hipLaunchKernelGGL((w4a4_fused_smallk_kernel<NT, NG>), grid, dim3(kFThreads), l.bytes, stream, X, M, K,
                     smooth, L1, r, L2, Wq, w_scales, bias, Y, N, act, dbg_qx, dbg_sx);
  return hipGetLastError();
}

// ------------------------------------------------------------------ MXFP4
// The same forward with Q taken as MXFP4: E2M1 codes with one E8M0 scale per
// 32 channels, multiplied by v_mfma_scale_f32_16x16x128_f8f6f4, which applies
// both blocks' scales itself (lane l supplies row or column l % 16, channels
// 32 (l / 16) .. + 31 of a 128-channel step, canonical packed, and that
// block's scale byte).  So a quantizer lane owns one whole block of one row:
// the absmax is lane-local, and its 16 code bytes and scale byte are exactly
// its A operand of the step; W is read 16 bytes per lane in the same layout,
// with no exchange between lanes; and there is no per-group epilogue.  The
// quantizer is quant_core.h's (the standalone quantize kernel's), T uses the
// same bf16 hi/lo MFMAs over four 8-channel chunks of the lane's block.
constexpr int kMxStep = 128;   // channels per block-scaled MFMA
constexpr int kFmtFp4 = 4;     // cbsz / blgp code of FP4 E2M1
typedef int v8i __attribute__((ext_vector_type(8)));

// LDS: inv_s [K] f32 | afrag [S][64 lanes] 16 B | sxl [S][64] i32 (scale bytes)
// | tfin [16][r] f32 | sws [ceil(S/2)][bn][8] bytes (weight scales, k-tiled as
// in global memory) | bias [bn] f32 | scratch: the waves' partial T
// [8][16][r] f32, later the output tile [16][bn] bf16.
__host__ __device__ inline FusedLds fused_lds_mx(int K, int r, int bn) {
  const int S = K / kMxStep;
  FusedLds l;
  l.inv_s = 0;
  l.afrag = K * 4;
  l.sxl = l.afrag + S * 1024;
  l.tfin = l.sxl + S * 256;
  l.sws = l.tfin + 16 * r * 4;
  l.bias = l.sws + (S + 1) / 2 * bn * 8;
  l.scratch = l.bias + bn * 4;
  const int tpart = kFW * 16 * r * 4, out = 16 * bn * 2;
  l.bytes = l.scratch + (tpart > out ? tpart : out);
  return l;
}

// NT: column tiles of 16 per wave; NS: 128-channel steps a wave quantizes at
// most (ceil(S / 8): 1 up to K = 1024, 2 up to K = 1280).
template <int NT, int NS>
__global__ __launch_bounds__(kFThreads, 1) void mxfp4_fused_smallk_kernel(
    const uint16_t* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ L1, int r, const uint16_t* __restrict__ L2,
    const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ w_e8m0,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int N, int act,
    uint8_t* __restrict__ dbg_qx, uint8_t* __restrict__ dbg_sx) {
  constexpr int BN = 16 * NT * kFW;
  constexpr int RTMAX = kFusedMaxRank / 16;
  constexpr int T2MAX = (kFusedMaxK / kMxStep + 1) / 2;
  constexpr int SWPER = (T2MAX * BN + kFThreads - 1) / kFThreads;   // 8-byte scale rows per thread
  constexpr int BPER = (BN + kFThreads - 1) / kFThreads;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const FusedLds LL = fused_lds_mx(K, r, BN);
  float* inv_s = reinterpret_cast<float*>(lds + LL.inv_s);
  uint4* afrag = reinterpret_cast<uint4*>(lds + LL.afrag);
  int* sxl = reinterpret_cast<int*>(lds + LL.sxl);
  float* tfin = reinterpret_cast<float*>(lds + LL.tfin);
  uint8_t* sws = lds + LL.sws;
  float* bias_l = reinterpret_cast<float*>(lds + LL.bias);
  float* tpart = reinterpret_cast<float*>(lds + LL.scratch);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const int S = K / kMxStep;
  const int T2 = (S + 1) / 2;
  const int KB = K / 2;
  const int RT = r / 16;
  const int m0 = blockIdx.x * 16;
  const int n0 = blockIdx.y * BN;
  const int wc = wave * 16 * NT;
  const int row = min(m0 + fr, M - 1);     // rows past M quantize a valid row, never stored

  // ---- 1. loads, in order of use (as in the int4 kernel: unconditional,
  // clamped, so that none waits behind a branch)
  constexpr int kSPer = kFusedMaxK / kFThreads + 1;
  float sv[kSPer];
#pragma unroll
  for (int i = 0; i < kSPer; ++i) sv[i] = smooth[min(tid + i * kFThreads, K - 1)];
  const int ns = wave < S ? (S - wave + kFW - 1) / kFW : 0;   // steps this wave quantizes (<= NS)
  uint4 xv[NS][4], lv[NS][RTMAX][4];
  const uint16_t* xrow = X + (size_t)row * K + 32 * fk;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int st = min(wave + kFW * i, S - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[i][q] = *reinterpret_cast<const uint4*>(xrow + st * kMxStep + 8 * q);
  }
  const uint16_t* l1b = r > 0 ? L1 : X;                      // a valid dummy for r = 0
  const int l1k = r > 0 ? K : 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int st = min(wave + kFW * i, S - 1);
#pragma unroll
    for (int j = 0; j < RTMAX; ++j) {
      const uint16_t* lp = l1b + (size_t)min(16 * j + fr, max(r, 1) - 1) * l1k + (r > 0 ? st * kMxStep + 32 * fk : 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) lv[i][j][q] = *reinterpret_cast<const uint4*>(lp + 8 * q);
    }
  }
  // the workgroup's weight scales: k-tiled [T2][N][8], rows n0 .. n0 + BN - 1
  // of each tile one contiguous run (rows past N: the last row)
  const int nsw = T2 * BN;
  uint2 swr[SWPER];
#pragma unroll
  for (int i = 0; i < SWPER; ++i) {
    const int e = min(tid + i * kFThreads, nsw - 1);
    const int t = e / BN;
    swr[i] = *reinterpret_cast<const uint2*>(w_e8m0 + ((size_t)t * N + min(n0 + e - t * BN, N - 1)) * 8);
  }
  const uint16_t* bb = bias ? bias : X;
  uint16_t brr[BPER];
#pragma unroll
  for (int i = 0; i < BPER; ++i) brr[i] = bb[bias ? min(n0 + min(tid + i * kFThreads, BN - 1), N - 1) : 0];
  int ncol[NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) ncol[tn] = min(n0 + wc + 16 * tn + fr, N - 1);
  const uint16_t* l2b = r > 0 ? L2 : X;
  const int jq = min(8 * fk, max(r, 8) - 8);                  // ranks 8 fk .. + 7 of the one chunk
  uint4 l2v[NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) l2v[tn] = *reinterpret_cast<const uint4*>(l2b + (r > 0 ? (size_t)ncol[tn] * r + jq : 0));

  // W, 16 bytes per lane: step st, bytes 16 fk of its 64 (past the last step: clamped)
  const uint8_t* wrow[NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) wrow[tn] = Wq + (size_t)ncol[tn] * KB + 16 * fk;
  uint4 wring[kDepth][NT];
  auto load_w = [&](int slot, int st) {
    const int off = min(st, S - 1) * (kMxStep / 2);
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) wring[slot][tn] = *reinterpret_cast<const uint4*>(wrow[tn] + off);
  };
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load_w(d, d);

  // ---- 2. 1/s, the weight scales and the bias into LDS; then quantize and partial T
#pragma unroll
  for (int i = 0; i < kSPer; ++i) inv_s[min(tid + i * kFThreads, K - 1)] = 1.0f / sv[i];  // duplicates equal
#pragma unroll
  for (int i = 0; i < SWPER; ++i) {
    const int e = tid + i * kFThreads;
    if (e < nsw) *reinterpret_cast<uint2*>(sws + 8 * e) = swr[i];   // [t][column][8]
  }
#pragma unroll
  for (int i = 0; i < BPER; ++i)
    if (tid + i * kFThreads < BN) bias_l[tid + i * kFThreads] = bias ? __uint_as_float(uint32_t(brr[i]) << 16) : 0.f;
  lds_barrier();

  f32x4 at[RTMAX];
#pragma unroll
  for (int j = 0; j < RTMAX; ++j) at[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    if (i < ns) {
      const int st = wave + kFW * i;
      const uint32_t w[16] = {xv[i][0].x, xv[i][0].y, xv[i][0].z, xv[i][0].w, xv[i][1].x, xv[i][1].y,
                              xv[i][1].z, xv[i][1].w, xv[i][2].x, xv[i][2].y, xv[i][2].z, xv[i][2].w,
                              xv[i][3].x, xv[i][3].y, xv[i][3].z, xv[i][3].w};
      const float* is = inv_s + st * kMxStep + 32 * fk;
      float xh[32];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        xh[2 * e] = __uint_as_float(w[e] << 16) * is[2 * e];
        xh[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u) * is[2 * e + 1];
      }
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(xh[e]));
      const uint32_t byte = quant::mx_scale_byte(amax);
      const uint4 codes = make_uint4(quant::mx_codes8(xh, byte), quant::mx_codes8(xh + 8, byte),
                                     quant::mx_codes8(xh + 16, byte), quant::mx_codes8(xh + 24, byte));
      afrag[st * 64 + lane] = codes;
      sxl[st * 64 + lane] = (int)byte;
      if (dbg_qx && blockIdx.y == 0 && m0 + fr < M) {
        *reinterpret_cast<uint4*>(dbg_qx + (size_t)(m0 + fr) * KB + st * (kMxStep / 2) + 16 * fk) = codes;
        dbg_sx[(size_t)(m0 + fr) * (K / 32) + 4 * st + fk] = (uint8_t)byte;
      }
      // lora_down: x_hat as a bf16 hi/lo pair, four 8-channel chunks of the block
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = xh[8 * c + 2 * e], v1 = xh[8 * c + 2 * e + 1];
          const uint32_t b0 = __float_as_uint(v0), b1 = __float_as_uint(v1);
          hi[e] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
          lo[e] = cvt_bf16x2(v0 - __uint_as_float(b0 & 0xFFFF0000u), v1 - __uint_as_float(b1 & 0xFFFF0000u));
        }
        const bf16x8 ahi = bf16x8_of(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const bf16x8 alo = bf16x8_of(make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
        for (int j = 0; j < RTMAX; ++j) {
          if (j < RT) {
            const bf16x8 b = bf16x8_of(lv[i][j][c]);
            at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, at[j], 0, 0, 0);
            at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, at[j], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- 3. T = the waves' partials summed in wave order
#pragma unroll
  for (int j = 0; j < RTMAX; ++j)
    if (j < RT)
#pragma unroll
      for (int i = 0; i < 4; ++i) tpart[(wave * 16 + 4 * fk + i) * r + 16 * j + fr] = at[j][i];
  lds_barrier();
  for (int e = tid; e < 16 * r; e += kFThreads) {
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < kFW; ++wv) s += tpart[wv * 16 * r + e];
    tfin[e] = s;
  }
  lds_barrier();   // tfin, afrag and sxl are complete; tpart is free

  // ---- 4. the GEMM over 128-channel steps, kDepth steps of W in flight; a
  // step past the last (padding to whole turns) has zero A codes
  f32x4 acc[1][NT];
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) acc[0][tn] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int Sp = (S + kDepth - 1) / kDepth * kDepth;
  for (int s0 = 0; s0 < Sp; s0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      __builtin_amdgcn_sched_barrier(0);   // one slot's work at a time (see the int4 loop)
      const int s = s0 + d;
      uint4 wv[NT];
#pragma unroll
      for (int tn = 0; tn < NT; ++tn) wv[tn] = wring[d][tn];
      load_w(d, s + kDepth);
      const int sc = min(s, S - 1);
      const uint32_t am = s < S ? 0xFFFFFFFFu : 0u;
      const uint4 araw = afrag[sc * 64 + lane];
      const v8i a = v8i{(int)(araw.x & am), (int)(araw.y & am), (int)(araw.z & am), (int)(araw.w & am), 0, 0, 0, 0};
      const int sa = sxl[sc * 64 + lane];
      const uint8_t* swp = sws + ((sc >> 1) * BN + wc + fr) * 8 + 4 * (sc & 1) + fk;
#pragma unroll
      for (int tn = 0; tn < NT; ++tn) {
        const int sb = swp[16 * 8 * tn];
        const v8i b = v8i{(int)wv[tn].x, (int)wv[tn].y, (int)wv[tn].z, (int)wv[tn].w, 0, 0, 0, 0};
        acc[0][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[0][tn], kFmtFp4, kFmtFp4, 0,
                                                                     sa, 0, sb);
      }
    }
  }

  // ---- 5. bias, T L2^T (r <= 32: one chunk of 32 ranks), activation, store
#pragma unroll
  for (int tn = 0; tn < NT; ++tn) {
    const float bv = bias_l[wc + 16 * tn + fr];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][tn][i] += bv;
  }
  if (r > 0) {
    const bool j_ok = 8 * fk < r;
    const float* tp = tfin + fr * r + jq;
    uint32_t thi[4], tlo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = j_ok ? tp[2 * e] : 0.f, v1 = j_ok ? tp[2 * e + 1] : 0.f;
      const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
      thi[e] = uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
      tlo[e] = cvt_bf16x2(v0 - (float)h0, v1 - (float)h1);
    }
    const bf16x8 th = bf16x8_of(make_uint4(thi[0], thi[1], thi[2], thi[3]));
    const bf16x8 tl = bf16x8_of(make_uint4(tlo[0], tlo[1], tlo[2], tlo[3]));
#pragma unroll
    for (int tn = 0; tn < NT; ++tn) {
      const bf16x8 l = bf16x8_of(j_ok ? l2v[tn] : make_uint4(0u, 0u, 0u, 0u));
      acc[0][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(th, l, acc[0][tn], 0, 0, 0);
      acc[0][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl, l, acc[0][tn], 0, 0, 0);
    }
  }
  uint16_t* otile = reinterpret_cast<uint16_t*>(lds + LL.scratch);
  tail::store_tile<1, NT, 16, BN, kFThreads>(acc, nullptr, Y, N, m0, n0, M, N, 0, wc, lane, tid,
                                             [&](int rr) { return otile + rr * BN; }, act);
}

template <int NT, int NS>
hipError_t allow_lds_mx() {
  static std::atomic<bool> done{false};
  if (done.load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mxfp4_fused_smallk_kernel<NT, NS>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.store(true, std::memory_order_release);
  return e;
}

template <int NT, int NS>
hipError_t launch_nt_mx(const uint16_t* X, int M, int K, int N, int r, const float* smooth,
                        const uint16_t* L1, const uint16_t* L2, const uint8_t* Wq,
                        const uint8_t* w_e8m0, const uint16_t* bias, uint16_t* Y, int act,
                        uint8_t* dbg_qx, uint8_t* dbg_sx, hipStream_t stream) {
  constexpr int BN = 16 * NT * kFW;
  const FusedLds l = fused_lds_mx(K, r, BN);
  const hipError_t e = allow_lds_mx<NT, NS>();
  if (e != hipSuccess) return e;
  const dim3 grid((M + 15) / 16, (N + BN - 1) / BN);
  hipLaunchKernelGGL((mxfp4_fused_smallk_kernel<NT, NS>), grid, dim3(kFThreads), l.bytes, stream, X, M,
                     K, smooth, L1, r, L2, Wq, w_e8m0, bias, Y, N, act, dbg_qx, dbg_sx);
  return hipGetLastError();
}


}  // namespace

namespace {

// The plan of either format: used up to `per_cu` blocks of 16 x 16 outputs x
// 64 channels per compute unit (past that, the two kernels are as fast).
FusedPlan plan_for(int M, int K, int N, int r, long per_cu) {
  FusedPlan p;
  if (K > kFusedMaxK || r > kFusedMaxRank || N > kFusedMaxN || M < 1 || N < 16) return p;
  const int G = K / kGroup;
  const int cus = device_cu_count();
  const long group_tiles = (long)((M + 15) / 16) * (N / 16) * G;
  if (group_tiles > per_cu * cus) return p;
  const long row_blocks = (M + 15) / 16;
  // per-workgroup cost in group-tile units: the quantize phase (about four
  // tiles' worth per group a wave quantizes) plus the wave's GEMM over the
  // padded group range; rounds of one workgroup per compute unit
  long best = -1;
  for (int nt = 1; nt <= 5; ++nt) {
    const long blocks = row_blocks * ((N + 128 * nt - 1) / (128 * nt));
    const long rounds = (blocks + cus - 1) / cus;
    const long per_wg = 4L * ((G + kFW - 1) / kFW) + (long)nt * ((G + 2 * kDepth - 1) / (2 * kDepth) * 2 * kDepth);
    const long cost = rounds * per_wg;
    if (best < 0 || cost < best) {
      best = cost;
      p.nt = nt;
    }
  }
  p.use = true;
  return p;
}

}  // namespace

FusedPlan fused_plan(int M, int K, int N, int r) { return plan_for(M, K, N, r, 256); }

hipError_t launch_fused_smallk(const FusedPlan& plan, const uint16_t* X, int M, int K, int N, int r,
                               const float* smooth, const uint16_t* L1, const uint16_t* L2,
                               const uint8_t* Wq, const float* w_scales, const uint16_t* bias,
                               uint16_t* Y, int act, uint8_t* dbg_qx, float* dbg_sx,
                               hipStream_t stream) {
  const bool three = K > 16 * kGroup;   // more than 16 groups: some waves quantize three
#define SVDQ_FUSED_CASE(nt)                                                                          \
  case nt:                                                                                            \
    return three ? launch_nt<nt, 3>(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y, act, dbg_qx, \
                                    dbg_sx, stream)                                                    \
                 : launch_nt<nt, 2>(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y, act, dbg_qx, \
                                    dbg_sx, stream);
  switch (plan.nt) {
    SVDQ_FUSED_CASE(1)
    SVDQ_FUSED_CASE(2)
    SVDQ_FUSED_CASE(3)
    SVDQ_FUSED_CASE(4)
    SVDQ_FUSED_CASE(5)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_FUSED_CASE
}

// MXFP4 has no per-group epilogue, so its crossover lies further out where K
// is short: measured against the two MXFP4 kernels, the fused kernel was
// faster at 4096 x 640 -> 640 (400 blocks per compute unit; 14.8 against
// 16.6 us) and slower at 6144 x 640 (600); at K = 1024 and 1280 it tied or
// lost from about 256 on (1024 x 1024: 10.6 against 10.7 us; 768 x 1280,
// 300: 15.9 against 13.5 us), as the int4 kernel does.
FusedPlan fused_plan_mx(int M, int K, int N, int r) {
  if (K % kMxStep != 0) return FusedPlan{};
  return plan_for(M, K, N, r, K <= 640 ? 400 : 256);
}

hipError_t launch_fused_smallk_mx(const FusedPlan& plan, const uint16_t* X, int M, int K, int N, int r,
                                  const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                  const uint8_t* Wq, const uint8_t* w_e8m0, const uint16_t* bias,
                                  uint16_t* Y, int act, uint8_t* dbg_qx, uint8_t* dbg_sx,
                                  hipStream_t stream) {
  const bool two = K > kFW * kMxStep;   // more than 8 steps: some waves quantize two
#define SVDQ_FUSED_MX_CASE(nt)                                                                          \
  case nt:                                                                                               \
    return two ? launch_nt_mx<nt, 2>(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y, act, dbg_qx,    \
                                     dbg_sx, stream)                                                     \
               : launch_nt_mx<nt, 1>(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y, act, dbg_qx,    \
                                     dbg_sx, stream);
  switch (plan.nt) {
    SVDQ_FUSED_MX_CASE(1)
    SVDQ_FUSED_MX_CASE(2)
    SVDQ_FUSED_MX_CASE(3)
    SVDQ_FUSED_MX_CASE(4)
    SVDQ_FUSED_MX_CASE(5)
    default: return hipErrorInvalidValue;
  }
#undef SVDQ_FUSED_MX_CASE
}

}  // namespace svdq
