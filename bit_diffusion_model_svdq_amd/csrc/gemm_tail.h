// Shared head and tail of the two GEMM kernels (int4 and MXFP4).
//
// The bias plus the low-rank branch's up projection T L2^T (Terminology
// Entry, section 2.3, E4 second term), added to the output accumulators
// before the main loop (MXFP4, whose loop leaves registers for it) or after
// it (int4); then the optional MLP activation, bf16 rounding, and the store
// of the tile through LDS as 16-byte row segments.
#pragma once

#include <type_traits>

#include "svdq_internal.h"

namespace svdq {
namespace tail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ inline float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// acc[tm][tn] holds the 16x16 tile (wr + 16 tm, wc + 16 tn) of the block's
// BM x BN output in the MFMA result layout (lane l: column l % 16, rows
// 4 (l / 16) + i).  T holds t_slices partial sums of M x r floats, t_stride
// floats apart, added in slice order.  T (times `scale`, a power of two) is
// split into a bf16 hi/lo pair and enters bf16 MFMAs whose accumulator input
// is the tile, so the branch keeps ~16 significant bits of T.
//
// Adds scale * (b[n] + sum_j T[m,j] L2[n,j]) to acc.  `issue` is called once:
// first of all (EARLY = 0), or after the loads of the first 32 ranks (the
// first EARLY T slices, L2 and the bias) and before any of them is used.  A
// caller that runs this before its main loop puts the loop's first stage
// there; EARLY = 0 keeps the fewest registers live while it issues, the
// others let the branch's loads travel ahead of it.  Every load is unconditional:
// rows and columns past the matrix read a clamped valid address (their
// outputs are never stored), ranks past r read a valid address and are
// zeroed by a select, so no load waits behind a branch.
template <int TM, int TN, int EARLY, class Issue>
__device__ inline void lowrank_bias_add(f32x4 (&acc)[TM][TN], const float* __restrict__ T,
                                        int t_slices, long t_stride, int r,
                                        const uint16_t* __restrict__ L2,
                                        const uint16_t* __restrict__ bias, int m0, int n0,
                                        int row1, int col1, int wr, int wc, int lane,
                                        float scale, Issue&& issue) {
  static_assert(EARLY >= 0 && EARLY <= 2, "none, one or two slices ahead of the caller's loads");
  if (EARLY == 0) issue();   // the caller's loads first: fewer registers live while they issue
  const int fr = lane & 15;
  const int fk = lane >> 4;
  const float* trow[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) trow[t] = T + (size_t)min(m0 + wr + 16 * t + fr, row1 - 1) * r;
  const uint16_t* lrow[TN];
  int bcol[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    bcol[tn] = min(n0 + wc + 16 * tn + fr, col1 - 1);
    lrow[tn] = L2 + (size_t)bcol[tn] * r;
  }
  uint16_t braw[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) braw[tn] = bias ? bias[bcol[tn]] : (uint16_t)0;

  bool issued = EARLY == 0;
  for (int j0 = 0; j0 < r || !issued; j0 += 32) {
    const bool step = j0 < r;                  // r = 0: only the bias and `issue`
    const int j = j0 + 8 * fk;
    const bool j_ok = step && j < r;
    const int jc = step ? min(j, r - 8) : 0;   // r % 16 == 0, so r - 8 >= 8
    float4 ta[TM], tb[TM];
    uint4 lf[TN];
    if (step) {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        ta[t] = *reinterpret_cast<const float4*>(trow[t] + jc);
        tb[t] = *reinterpret_cast<const float4*>(trow[t] + jc + 4);
      }
      float4 ua[TM], ub[TM];
      if (EARLY != 1) {
        const long s1 = t_slices > 1 ? t_stride : 0;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          ua[t] = *reinterpret_cast<const float4*>(trow[t] + s1 + jc);
          ub[t] = *reinterpret_cast<const float4*>(trow[t] + s1 + jc + 4);
        }
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) lf[tn] = *reinterpret_cast<const uint4*>(lrow[tn] + jc);
      if (!issued) {
        issue();
        issued = true;
      }
      if (EARLY != 1 && t_slices > 1)
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          ta[t] = add4(ta[t], ua[t]);
          tb[t] = add4(tb[t], ub[t]);
        }
      for (int sl = EARLY == 1 ? 1 : 2; sl < t_slices; ++sl)
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          ta[t] = add4(ta[t], *reinterpret_cast<const float4*>(trow[t] + sl * t_stride + jc));
          tb[t] = add4(tb[t], *reinterpret_cast<const float4*>(trow[t] + sl * t_stride + jc + 4));
        }
    } else {
      issue();
      issued = true;
    }
    if (j0 == 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const float bv = __uint_as_float(uint32_t(braw[tn]) << 16) * scale;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tm][tn][i] += bv;
      }
    }
    if (!step) break;
    bf16x8 thi[TM], tlo[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const float tv[8] = {ta[t].x, ta[t].y, ta[t].z, ta[t].w, tb[t].x, tb[t].y, tb[t].z, tb[t].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = j_ok ? tv[e] * scale : 0.f;
        const __bf16 h = (__bf16)v;
        thi[t][e] = h;
        tlo[t][e] = (__bf16)(v - (float)h);
      }
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const bf16x8 l = as_bf16x8(j_ok ? lf[tn] : make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(thi[tm], l, acc[tm][tn], 0, 0, 0);
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tlo[tm], l, acc[tm][tn], 0, 0, 0);
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

// The bias (NULL: none; loads at a clamped column, without branches), the
// activation (act == kActGeluTanh: gelu_tanh of the float32 sum), bf16
// rounding and the store of the tile through LDS as 16-byte row segments.
// The stores are non-temporal: Y streams out to HBM (measured 14 % faster for
// a plain 25 MB write than stores that allocate in the caches).
// row_lds(row) is the LDS address of the tile's row `row` (BN bf16 values);
// the caller has synchronized the block so that the space is free.
template <int TM, int TN, int BM, int BN, int THREADS, class RowLds>
__device__ inline void store_tile(f32x4 (&acc)[TM][TN], const uint16_t* __restrict__ bias,
                                  uint16_t* __restrict__ Y, int ldy, int m0, int n0, int row1,
                                  int col1, int wr, int wc, int lane, int tid, RowLds&& row_lds,
                                  int act) {
  const int fr = lane & 15;
  const int fk = lane >> 4;
  float bv[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    bv[tn] = bias ? __uint_as_float(uint32_t(bias[min(n0 + wc + 16 * tn + fr, col1 - 1)]) << 16)
                  : 0.f;

  // columns swizzled by 16 elements per group of 4 rows, so that the 4 row
  // groups of a write hit distinct banks.  The activation is a compile-time
  // choice inside the loops: a run-time test there is if-converted, and the
  // GELU's exp and reciprocal would then run for every element either way.
  auto write = [&](auto gelu) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wr + 16 * tm + 4 * fk + i;
        uint16_t* orow = row_lds(row);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int col = wc + 16 * tn + fr;
          float v = acc[tm][tn][i] + bv[tn];
          if constexpr (decltype(gelu)::value) v = gelu_tanh(v);
          orow[col ^ (16 * ((row >> 2) & 3))] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
      }
  };
  if (act == kActGeluTanh)
    write(std::true_type{});
  else
    write(std::false_type{});
  __syncthreads();
  constexpr int CPR = BN / 8;   // 16-byte chunks per output row
  for (int c = tid; c < BM * CPR; c += THREADS) {
    const int row = c / CPR, ch = c - (c / CPR) * CPR;
    const int m = m0 + row, n = n0 + 8 * ch;
    if (m < row1 && n < col1) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row_lds(row) + 8 * (ch ^ (2 * ((row >> 2) & 3))));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Y + (size_t)m * ldy + n));
    }
  }
}

// Tile coordinates of tile number `id`: rastered in groups of 8 token tiles.
__device__ inline void tile_of_id(int ntm, int ntn, int id, int& tm, int& tn) {
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * ntn;
  const int grp = id / per_group;
  const int first = grp * GROUP_M;
  const int gsize = min(ntm - first, GROUP_M);
  const int in = id - grp * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

// Workgroups are dealt round-robin to the 8 XCDs; block b of `count` (a
// multiple of 8) gets tile number (b % 8) * count / 8 + b / 8, so that each
// XCD works on one compact run of tiles and keeps its operand rows in its L2.
__device__ inline int xcd_compact(int b, int count) {
  return (count & 7) == 0 ? (b & 7) * (count >> 3) + (b >> 3) : b;
}

// Remainder split of a GEMM: when the tile count leaves a last, nearly empty
// wave of workgroups, the tiles [full, full + rem) are cut along K into at
// most kMaxSplits shares, each storing its raw fp32 accumulators, thread by
// thread ([tile * splits + share][TM * TN][THREADS] float4), and a fixup
// pass sums them.
constexpr int kMaxSplits = 8;

// The fixup, for a tile of WM x WN waves of TM x TN 16x16 accumulators and
// THREADS threads.  Block (t, wm) covers the 16 TM-row band wm of remainder
// tile full + t at the tile's full width: its TM x WN waves stand in for the
// band's (16-row slice, wave column) pairs, and each sums its accumulator
// entries over the shares in split order, all of its loads issued at once.
// Then `scale`, the bias and low-rank tail, and the store, as the tile's own
// waves would run them.  rem x WM blocks spread over the chip what rem blocks
// of whole tiles would each read alone.  Launch: rem * WM blocks of
// 64 TM WN threads, 16 TM BN * 2 bytes of LDS.
template <int TM, int TN, int WM, int WN, int BM, int BN, int THREADS>
__device__ inline void split_fixup(const float* __restrict__ part, int full, int splits,
                                   float scale, const float* __restrict__ T, int t_slices,
                                   long t_stride, int r, const uint16_t* __restrict__ L2,
                                   const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                                   int ldy, int row0, int row1, int col0, int col1, int act,
                                   uint8_t* lds) {
  constexpr int NACC = TM * TN;
  constexpr int BAND = 16 * TM;                     // rows of a wave's sub-tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int slice = wave % TM;                      // the 16-row slice tm of the sub-tile
  const int wn = wave / TM;                         // the wave column it stands in for
  const int wm = blockIdx.x % WM;
  const int tr = blockIdx.x / WM;
  const int ntm = (row1 - row0 + BM - 1) / BM;
  const int ntn = (col1 - col0 + BN - 1) / BN;
  int tmi, tni;
  tile_of_id(ntm, ntn, full + tr, tmi, tni);
  const int m0 = row0 + tmi * BM + wm * BAND;       // the band
  const int n0 = col0 + tni * BN;
  const int src_tid = (wm * WN + wn) * 64 + lane;   // the share writer's thread

  f32x4 acc[1][TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) acc[0][tn] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float4* src = reinterpret_cast<const float4*>(part) + (size_t)tr * splits * NACC * THREADS +
                      (size_t)slice * TN * THREADS + src_tid;
  // every load is issued before the first add (clamped, unconditional); the
  // adds run in split order for the real shares
  float4 v[kMaxSplits][TN];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      v[sp][tn] = src[((size_t)min(sp, splits - 1) * NACC + tn) * THREADS];
#pragma unroll
  for (int sp = 0; sp < kMaxSplits; ++sp)
    if (sp < splits)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        acc[0][tn][0] += v[sp][tn].x;
        acc[0][tn][1] += v[sp][tn].y;
        acc[0][tn][2] += v[sp][tn].z;
        acc[0][tn][3] += v[sp][tn].w;
      }
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][tn][i] *= scale;
  const int wr = 16 * slice, wc = wn * TN * 16;
  lowrank_bias_add<1, TN, 2>(acc, T, t_slices, t_stride, r, L2, bias, m0, n0, row1, col1, wr, wc,
                             lane, 1.0f, [] {});
  uint16_t* otile = reinterpret_cast<uint16_t*>(lds);
  store_tile<1, TN, BAND, BN, 64 * TM * WN>(acc, nullptr, Y, ldy, m0, n0, row1, col1, wr, wc, lane,
                                             tid, [&](int row) { return otile + row * BN; }, act);
}

}  // namespace tail
}  // namespace svdq
