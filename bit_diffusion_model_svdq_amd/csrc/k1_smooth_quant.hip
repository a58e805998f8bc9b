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
// Work split.  A workgroup owns RTM row tiles of 16 rows and one slice of K
// (grid.y = slices); its 8 waves split the slice's 64-channel groups into
// contiguous runs.  A wave handles all RTM row tiles of each of its groups,
// so every lora_down fragment it loads serves RTM row tiles: L1 is read from
// L2 once per 16 * RTM rows.  Slices keep >= 256 workgroups when RTM row tiles
// per block leave too few; each slice writes its own partial T (slice-major,
// [slices][M][r]) and the GEMM kernel sums the slices in order when it loads T.
//
// Loads.  Lane l holds row (l % 16) of a tile and, of each group, channels
// 8 * (l / 16) + 0..7 and 32 + 8 * (l / 16) + 0..7: exactly the A operand of
// two 16x16x32 bf16 MFMAs, in two 16-byte loads that cover 64 contiguous bytes
// per row.  A wave keeps one group in flight: the loads of group g + 1 are
// issued as soon as group g is processed.  Deeper windows (two or more groups
// in flight) measured slower: the memory pipeline of a CU takes load
// instructions only as fast as HBM serves them, so a deeper window just
// stalls each wave at issue, and its groups still arrive at the same pace.
// Loads are branch-free: rows past M re-read valid data that is never used;
// the last window refills nothing.
//
// Stores.  Codes and scales are collected in LDS and leave at the end as whole
// row segments of the slice (16-byte stores), so no store shares the in-order
// vector-memory counter with a load still to be waited for, and HBM sees full
// lines instead of 16-byte pieces from different waves.
//
// Quantization (int4).  The arithmetic is quant_core.h's, shared with the
// fused small-K forward: the group absmax over the four lanes of a row, the
// float32 scale amax / 7 and the rounding adder that yields the codes.
//
// MXFP4 (template flag MX).  The same kernel quantizes each block of 32
// channels (a lane's 8 + the 3 other lanes of its row) to FP4 E2M1 with one
// E8M0 scale: the shared exponent floor(log2 amax) - 2 is the block absmax's
// exponent field minus 129 (clamped at -127), i.e. the E8M0 byte is
// max(exponent field - 2, 0), and v_cvt_scalef32_pk_fp4_f32 divides by the
// power-of-two scale and rounds to nearest even with saturation, two
// elements per instruction, keeping the sign of a value that rounds to zero.
// A block whose scale would be the subnormal 2^-127 (absmax < 2^-125) is
// converted as v * 2^127 with scale 1 instead.  The scale bytes leave row-major
// [M, K/32], or k-tiled for the GEMM: per 256 channels, the 8 bytes of each
// row, rows consecutive ([K/256][sx_rows][8]), so that the GEMM copies a
// tile's scales of one stage as one contiguous run.
//
// lora_down.  x_hat enters the MFMA as a bf16 hi/lo pair (hi = x_hat with the
// low 16 bits cleared, lo = bf16(x_hat - hi), an exact difference), so T keeps
// ~16 significant bits.  The waves' partial T are summed in LDS in a fixed
// order (deterministic).
#include <algorithm>

#include "quant_core.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kW = 8;                  // waves per workgroup
constexpr int kThreads = kW * 64;
constexpr size_t kLdsBudget = 152 * 1024;
constexpr int kMaxSliceGroups = 48;    // the plan below never cuts longer slices
constexpr int kMaxRT2 = 5;             // two row tiles per block up to r = 80 (register budget)

__device__ inline uint32_t cvt_bf16x2(float a, float b) {  // round-to-nearest-even pair
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// LDS layout: inv_s [gslice * 64] floats | codes [16 RTM rows][gslice * 32 + 16 B]
// | scales [16 RTM rows][gslice] floats; the T partials [waves][16 RTM][r]
// reuse the same bytes at the end.  The 16-byte row pad spreads a wave's 16
// rows over distinct banks.
__host__ __device__ inline int code_pitch(int gslice) { return gslice * 32 + 16; }
__host__ __device__ inline size_t lds_main_bytes(int rtm, int gslice) {
  return (size_t)gslice * kGroup * 4 + (size_t)16 * rtm * code_pitch(gslice) +
         (size_t)16 * rtm * gslice * 4;
}
// T partials [waves][16 rtm][r] floats: after the main part when the budget
// allows (then written before the final barrier), else over it.
__host__ __device__ inline size_t tpart_bytes(int rtm, int r) { return (size_t)kW * 16 * rtm * r * 4; }
__host__ __device__ inline size_t t_own_offset(int rtm, int gslice) {
  return (lds_main_bytes(rtm, gslice) + 15) & ~size_t(15);
}

// RT = r / 16 rank tiles; RTM row tiles per workgroup; gslice groups per K-slice.
template <int RT, int RTM, bool MX>
__global__ __launch_bounds__(kThreads) void smooth_quant_lora_down_kernel(
    const uint16_t* __restrict__ X, int M, int K, const float* __restrict__ smooth,
    const uint16_t* __restrict__ L1, int r, uint8_t* __restrict__ qx, void* __restrict__ sx_out,
    float* __restrict__ T, int gslice, int sx_rows) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  constexpr int NL = RT > 0 ? 2 * RT : 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = K / kGroup;
  const int slice = blockIdx.y;
  const int sg0 = slice * gslice;                 // first group of the slice
  const int sg1 = min(G, sg0 + gslice);
  const int per_wave = (sg1 - sg0 + kW - 1) / kW;
  const int g_begin = min(sg1, sg0 + wave * per_wave);
  const int g_end = min(sg1, g_begin + per_wave);
  const int g_last = max(g_end - 1, sg0);         // a wave without groups re-reads a valid one
  float* inv_s = lds;                             // channels of the slice
  uint8_t* lcodes = reinterpret_cast<uint8_t*>(lds + gslice * kGroup);
  // per row and group: the float32 scale's bits (int4) or the two E8M0 bytes (MX)
  uint32_t* lscales = reinterpret_cast<uint32_t*>(lcodes + 16 * RTM * code_pitch(gslice));
  const bool t_own = t_own_offset(RTM, gslice) + tpart_bytes(RTM, r) <= kLdsBudget;
  float* tpart = t_own ? lds + t_own_offset(RTM, gslice) / 4 : lds;

  const int m0 = blockIdx.x * 16 * RTM;
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const uint16_t* xrow[RTM];
#pragma unroll
  for (int t = 0; t < RTM; ++t) xrow[t] = X + (size_t)min(m0 + 16 * t + fr, M - 1) * K + 8 * fk;
  const uint16_t* l1row = L1 + (size_t)fr * K + 8 * fk;

  uint4 xa[RTM], xb[RTM], lb[NL];
  auto load_group = [&](int g) {
    const int gg = min(g, g_last);
#pragma unroll
    for (int t = 0; t < RTM; ++t) {
      xa[t] = *reinterpret_cast<const uint4*>(xrow[t] + gg * kGroup);
      xb[t] = *reinterpret_cast<const uint4*>(xrow[t] + gg * kGroup + 32);
    }
    if constexpr (RT > 0) {
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        const uint16_t* lp = l1row + (size_t)j * 16 * K + gg * kGroup;
        lb[2 * j] = *reinterpret_cast<const uint4*>(lp);
        lb[2 * j + 1] = *reinterpret_cast<const uint4*>(lp + 32);
      }
    }
  };

  // fl32(1 / s[k]) for the slice, IEEE division, once per workgroup.  The
  // values are requested before the first groups' loads, and everything up to
  // the barrier is branch-free (clamped indices, duplicates store equal
  // values): a branch there would make the compiler wait for every load in
  // flight.  The planned slices have at most kMaxSliceGroups groups; only a
  // one-slice launch on a longer row needs the loop, which runs first.
  constexpr int kPre = kMaxSliceGroups * kGroup / kThreads;
  const int c0 = sg0 * kGroup, nc = (sg1 - sg0) * kGroup;
  if (nc > kPre * kThreads)
    for (int k = tid + kPre * kThreads; k < nc; k += kThreads) inv_s[k] = 1.0f / smooth[c0 + k];
  float sv[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) sv[i] = smooth[c0 + min(tid + i * kThreads, nc - 1)];
  __builtin_amdgcn_sched_barrier(0);   // in-order counter: s must be ahead of the groups
  load_group(g_begin);
#pragma unroll
  for (int i = 0; i < kPre; ++i) inv_s[min(tid + i * kThreads, nc - 1)] = 1.0f / sv[i];

  f32x4 acc[RTM][RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < RTM; ++t)
#pragma unroll
    for (int j = 0; j < (RT > 0 ? RT : 1); ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // inv_s ready: the LDS writes are waited for, the group loads stay in flight
  // (__syncthreads would wait for them too)
  lds_barrier();

  // One group of one row tile from registers: codes, scale, and the lora_down MFMAs.
  auto process = [&](int g, uint4 va, uint4 vb, const uint4* lf, f32x4* at, uint2& codes,
                     uint32_t& scale) {
    const int k0 = (g - sg0) * kGroup + 8 * fk;
    const uint32_t w[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
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
    if constexpr (MX) {
      // blocks: channels 0..31 (xh[0..7] of the row's four lanes), 32..63 (xh[8..15])
      float am[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) am[i >> 3] = fmaxf(am[i >> 3], fabsf(xh[i]));
      uint32_t bytes[2], words[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        am[b] = fmaxf(am[b], __shfl_xor(am[b], 16));
        am[b] = fmaxf(am[b], __shfl_xor(am[b], 32));
        bytes[b] = quant::mx_scale_byte(am[b]);
        words[b] = quant::mx_codes8(xh + 8 * b, bytes[b]);
      }
      codes.x = words[0];
      codes.y = words[1];
      scale = bytes[0] | (bytes[1] << 8);
    } else {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
      amax = quant::row_group_absmax(amax);
      float z[16];
      quant::int4_codes<16>(xh, amax, scale, z);
      codes.x = quant::pack8(z);
      codes.y = quant::pack8(z + 8);
    }
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
      for (int j = 0; j < RT; ++j) {
        const bf16x8 b0 = as_bf16x8(lf[2 * j]), b1 = as_bf16x8(lf[2 * j + 1]);
        at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi0, b0, at[j], 0, 0, 0);
        at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo0, b0, at[j], 0, 0, 0);
        at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi1, b1, at[j], 0, 0, 0);
        at[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo1, b1, at[j], 0, 0, 0);
      }
    }
  };

  auto store_group = [&](int g, const uint2* codes, const uint32_t* scales) {
#pragma unroll
    for (int t = 0; t < RTM; ++t) {
      uint8_t* crow = lcodes + (16 * t + fr) * code_pitch(gslice) + (g - sg0) * 32 + 4 * fk;
      *reinterpret_cast<uint32_t*>(crow) = codes[t].x;
      *reinterpret_cast<uint32_t*>(crow + 16) = codes[t].y;
      if (fk == 0) lscales[(16 * t + fr) * gslice + (g - sg0)] = scales[t];
    }
  };
  // Process a group, load the next, then store.  The load is unconditional
  // (clamped) so that the loop body has no branch around a load: at a branch
  // join the compiler would have to assume the worst and wait for every load
  // in flight.  The last group refills nothing (a load past the run would be
  // wasted, and the final barrier would wait for it).
  int g = g_begin;
  for (; g + 1 < g_end; ++g) {
    uint2 codes[RTM];
    uint32_t scales[RTM];
#pragma unroll
    for (int t = 0; t < RTM; ++t) process(g, xa[t], xb[t], lb, acc[t], codes[t], scales[t]);
    load_group(g + 1);
    store_group(g, codes, scales);
  }
  if (g < g_end) {
    uint2 codes[RTM];
    uint32_t scales[RTM];
#pragma unroll
    for (int t = 0; t < RTM; ++t) process(g, xa[t], xb[t], lb, acc[t], codes[t], scales[t]);
    store_group(g, codes, scales);
  }

  // 16x16 MFMA result layout: lane l holds column l % 16, rows 4 * (l / 16) + i.
  // T partials [wave][row of the block][rank], summed over waves in order.
  constexpr int RB = 16 * RTM;
  auto write_tpart = [&] {
    if constexpr (RT > 0) {
#pragma unroll
      for (int t = 0; t < RTM; ++t)
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            tpart[(wave * RB + 16 * t + 4 * fk + i) * r + 16 * j + fr] = acc[t][j][i];
    }
  };
  // codes and scales of the block's rows for the slice, as whole row segments
  auto store_codes = [&] {
    const int ng = sg1 - sg0;
    const int chunks = 2 * ng;                      // 16-byte pieces per row
    for (int e = tid; e < 16 * RTM * chunks; e += kThreads) {
      const int rr = e / chunks, c = e - (e / chunks) * chunks;
      if (m0 + rr < M)
        *reinterpret_cast<uint4*>(qx + (size_t)(m0 + rr) * (K / 2) + sg0 * 32 + c * 16) =
            *reinterpret_cast<const uint4*>(lcodes + rr * code_pitch(gslice) + c * 16);
    }
    for (int e = tid; e < 16 * RTM * ng; e += kThreads) {
      const int rr = e / ng, c = e - (e / ng) * ng;
      if (m0 + rr < M) {
        const uint32_t v = lscales[rr * gslice + c];
        if constexpr (MX) {
          // the group's two E8M0 bytes: row-major [M, K/32], or k-tiled
          // [K/256][sx_rows][8] (sx_rows > 0) as the block-scaled GEMM reads them
          const int g = sg0 + c;
          const size_t at = sx_rows > 0 ? ((size_t)(g >> 2) * sx_rows + m0 + rr) * 8 + 2 * (g & 3)
                                        : (size_t)(m0 + rr) * 2 * G + 2 * g;
          *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(sx_out) + at) = (uint16_t)v;
        } else {
          static_cast<float*>(sx_out)[(size_t)(m0 + rr) * G + sg0 + c] = __uint_as_float(v);
        }
      }
    }
  };
  auto reduce_t = [&] {
    if constexpr (RT > 0) {
      float* Ts = T + (size_t)slice * M * r;
      for (int e = tid; e < RB * r; e += kThreads) {
        const int rr = e / r, c = e - (e / r) * r;
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < kW; ++wv) s += tpart[(wv * RB + rr) * r + c];
        if (m0 + rr < M) Ts[(size_t)(m0 + rr) * r + c] = s;
      }
    }
  };
  // The barriers order LDS only: the code stores need not land before the
  // partial sums are read.  With its own LDS region, T's partials go in
  // before the one barrier, and codes and T leave together.
  if (t_own) {
    write_tpart();
    lds_barrier();
    store_codes();
    reduce_t();
  } else {
    lds_barrier();
    store_codes();
    if constexpr (RT > 0) {
      lds_barrier();                                // the codes are read; LDS is reused
      write_tpart();
      lds_barrier();
      reduce_t();
    }
  }
}

size_t lds_bytes(int rtm, int gslice, int r) {
  const size_t own = t_own_offset(rtm, gslice) + tpart_bytes(rtm, r);
  return own <= kLdsBudget ? own : std::max(lds_main_bytes(rtm, gslice), tpart_bytes(rtm, r));
}

template <int RT, int RTM, bool MX>
hipError_t launch(const K1Plan& p, const uint16_t* X, int M, int K, int r, const float* smooth,
                  const uint16_t* L1, uint8_t* qx, void* sx, float* T, int sx_rows,
                  hipStream_t stream) {
  const size_t lds = lds_bytes(RTM, p.gslice, r);
  auto kern = smooth_quant_lora_down_kernel<RT, RTM, MX>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int rb = (M + 16 * RTM - 1) / (16 * RTM);
  hipLaunchKernelGGL(kern, dim3(rb, p.slices), dim3(kThreads), lds, stream, X, M, K, smooth, L1,
                     r, qx, sx, T, p.gslice, sx_rows);
  return hipGetLastError();
}

template <int RT, bool MX>
hipError_t launch_rt(const K1Plan& p, const uint16_t* X, int M, int K, int r, const float* smooth,
                     const uint16_t* L1, uint8_t* qx, void* sx, float* T, int sx_rows,
                     hipStream_t stream) {
  if constexpr (RT <= kMaxRT2)
    if (p.rtm == 2) return launch<RT, 2, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
  return launch<RT, 1, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
}

template <bool MX>
hipError_t dispatch(const uint16_t* X, int M, int K, int r, const float* smooth,
                    const uint16_t* L1, uint8_t* qx, void* sx, float* T, bool one_slice,
                    int sx_rows, hipStream_t stream) {
  const K1Plan p = k1_plan(M, K, r, one_slice);
  switch (r / 16) {
    case 0: return launch_rt<0, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 1: return launch_rt<1, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 2: return launch_rt<2, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 3: return launch_rt<3, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 4: return launch_rt<4, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 5: return launch_rt<5, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 6: return launch_rt<6, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 7: return launch_rt<7, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    case 8: return launch_rt<8, MX>(p, X, M, K, r, smooth, L1, qx, sx, T, sx_rows, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Row tiles per workgroup (RTM = 1 or 2) and K-slices, from a cost model in
// rough microseconds, fitted to measured launches on MI355X:
//   rounds * (5 + 2 * groups_per_wave * w)          waves of workgroups over 256 CUs
//   + 20 * (256 - workgroups) / 256 when under 256   idle CUs
//   + 6 per T slice beyond the first                  the GEMM re-reads every slice of
//                                                    T for each of its output tiles
//                                                    (the MXFP4 GEMM in its prologue)
// where w = 1 + 0.5 r / (16 RTM) weighs a group's X bytes with the L1
// fragments it needs (read from L2 once per 16 RTM rows).  A wave waits one
// memory round trip per group, so fewer groups per wave shorten a workgroup;
// more workgroups than CUs add a round.  Slices hold at most kMaxSliceGroups
// groups and must fit the LDS budget.  Ties keep RTM = 2 and fewer slices.
// The plan depends on the shape only (it sizes the workspace): 256 CUs.
K1Plan k1_plan(int M, int K, int r, bool one_slice) {
  K1Plan p;
  const int G = K / kGroup;
  if (one_slice) {
    p.rtm = (r > 0 && r <= 16 * kMaxRT2 && M >= 2048) ? 2 : 1;
    if (lds_bytes(p.rtm, G, r) > kLdsBudget) p.rtm = 1;
    p.gslice = G;
    p.slices = 1;
    return p;
  }
  constexpr int kCus = 256;
  double best = 1e300;
  for (int rtm = 2; rtm >= 1; --rtm) {
    if (rtm == 2 && r > 16 * kMaxRT2) continue;
    const int rb = (M + 16 * rtm - 1) / (16 * rtm);
    const double w = 1.0 + 0.5 * r / (16.0 * rtm);
    for (int want = 1; want <= G; ++want) {
      const int gslice = (G + want - 1) / want;
      const int slices = (G + gslice - 1) / gslice;
      if (slices != want || gslice > kMaxSliceGroups) continue;
      if (lds_bytes(rtm, gslice, r) > kLdsBudget) continue;
      const int per_wave = (gslice + kW - 1) / kW;
      const long n = (long)rb * slices;
      const long rounds = (n + kCus - 1) / kCus;
      const double cost = rounds * (5.0 + 2.0 * per_wave * w) +
                          (n < kCus ? 20.0 * (kCus - n) / kCus : 0.0) + 6.0 * (slices - 1);
      if (cost < best - 1e-9) {
        best = cost;
        p.rtm = rtm;
        p.gslice = gslice;
        p.slices = slices;
      }
    }
  }
  return p;
}

// The launch plans keep to kLdsBudget; a one-slice launch may use all of the
// 160 KB a workgroup can hold.
bool k1_one_slice_fits(int K, int r) {
  return lds_bytes(1, K / kGroup, r) <= 160 * 1024;
}

hipError_t launch_smooth_quant_lora_down(const uint16_t* X, int M, int K, int r,
                                         const float* smooth, const uint16_t* L1, uint8_t* qx,
                                         float* sx, float* T, bool one_slice, hipStream_t stream) {
  return dispatch<false>(X, M, K, r, smooth, L1, qx, sx, T, one_slice, 0, stream);
}

hipError_t launch_smooth_quant_lora_down_mx(const uint16_t* X, int M, int K, int r,
                                            const float* smooth, const uint16_t* L1, uint8_t* qx,
                                            uint8_t* sx_e8m0, float* T, bool one_slice,
                                            int sx_rows, hipStream_t stream) {
  return dispatch<true>(X, M, K, r, smooth, L1, qx, sx_e8m0, T, one_slice, sx_rows, stream);
}

}  // namespace svdq
