// k2: W4A4 GEMM with the per-group scale epilogue, lora_up and bias, gfx950.
//
// Computes the SVDQuant dual-path output (Terminology Entry, section 2.3,
// equations E4 and E7: the low-bit product is taken only for the residual R,
// the low-rank branch is added in high precision):
//
//   Y[m,n] = bf16( sum_g sx[m,g] sw[n,g] P[m,n,g]  +  sum_j T[m,j] L2[n,j]  +  b[n] )
//   P[m,n,g] = sum_{k in group g} qx[m,k] qw[n,k]
//
// Main loop.  CDNA has no 4-bit matrix instruction, so each 64-channel group
// is one v_mfma_i32_16x16x64_i8.  The 4-bit codes are widened by a shift:
// a nibble moved to the top of its byte is the int8 value 16 q, so the
// product of two widened operands is 256 P exactly, and the two nibbles of a
// byte land in different registers -- a channel permutation that both
// operands share, which leaves each group's dot product unchanged.  The
// widening happens once per workgroup, when a stage is copied into LDS.
//
// Scale epilogue.  Per output and group this is the expensive part: the
// vector ALU is 1/16 of the int8 matrix rate per output-group.  The MFMA's
// accumulator input is the constant bit pattern of 1.5 * 2^23, so the int32
// result read as float32 is exactly 1.5 * 2^23 + 256 P (|256 P| < 2^22).
// Then  t = fma(D, sw, -1.5*2^23*sw)  equals fl32(256 P sw) exactly, because
// the weight scales have their two low significand bits clear (3 sw is exact),
// and  acc = fma(t, sx, acc).  Two VALU operations per output and group, no
// integer-to-float conversion.  acc / 256 is taken once at the end.
//
// Low-rank branch and bias.  The finished tile is scaled by 1/256, the bias
// is added and then T L2^T by bf16 MFMAs with T split into a bf16 hi/lo pair
// (T keeps ~16 significant bits); all their loads are issued at once.  The
// tile is staged through LDS and leaves as 16-byte row segments.
//
// Tiling is a template: WM x WN waves, each owning TM x TN tiles of 16x16
// (tokens x features); two groups per pipeline stage, double-buffered in LDS
// with a 16-byte slot swizzle that keeps fragment reads conflict-free.
// Workgroups are remapped so that each XCD (workgroups are dealt round-robin
// to the 8 XCDs) works on one compact block of tiles, which keeps its share
// of qx and Wq in its own L2.
#include <algorithm>

#include "gemm_tail.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int GS = 2;              // groups per pipeline stage
constexpr int ROWB = 64;           // int8 bytes per row and group in LDS
constexpr int kMagicBits = 0x4B400000;  // 1.5 * 2^23
constexpr float kMagic = 12582912.0f;

template <int WM_, int WN_, int TM_, int TN_, int PF_ = 1, int NB_ = 2>
struct Tile {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int PF = PF_;            // stages staged in registers ahead of the LDS ones
  static constexpr int NB = NB_;            // LDS stage buffers (1: next stage waits in registers)
  static constexpr int BM = WM * TM * 16;   // tokens per workgroup
  static constexpr int BN = WN * TN * 16;   // features per workgroup
  static constexpr int THREADS = WM * WN * 64;
  static constexpr int A_PANEL = BM * ROWB + 16;   // +16 B: the GS panels start in different banks
  static constexpr int B_PANEL = BN * ROWB + 16;
  static constexpr int A_BYTES = GS * A_PANEL;
  static constexpr int B_BYTES = GS * B_PANEL;
  static constexpr int STAGE = A_BYTES + B_BYTES + GS * BM * 4 + 2 * GS * BN * 4;
  static constexpr int OUT = BM * BN * 2;           // bf16 output tile, staged at the end
  static constexpr int LDS = (NB * STAGE > OUT ? NB * STAGE : OUT);
  static constexpr int SU = (BM + BN + THREADS - 1) / THREADS;   // scale rows or columns per thread
  static constexpr int WPE = THREADS >= 512 ? 1 : 2;             // workgroups a CU holds
  static constexpr int MIN_WAVES = NB == 1 ? 2 : 1;   // per SIMD: two workgroups stay resident
};

using TileBig = Tile<4, 2, 4, 6>;    // 256 x 192, 8 waves
using TileBig2 = Tile<2, 2, 4, 6, 1, 1>;  // 128 x 192, 4 waves, two per CU, one LDS buffer each
using TileMed = Tile<2, 2, 4, 4>;    // 128 x 128, 4 waves
using TileSmall = Tile<2, 2, 2, 2, 2>;  //  64 x  64, 4 waves, two stages ahead

// byte offset of 16-byte slot `slot` (0..3) of row `row` within one group's panel
__device__ inline int swz(int row, int slot) {
  return row * ROWB + ((slot ^ ((row >> 1) & 3)) << 4);
}

__device__ inline uint4 widen_lo_hi(uint32_t a, uint32_t b) {  // 16 nibbles -> 16 int8 of value 16 q
  return make_uint4((a << 4) & 0xF0F0F0F0u, (b << 4) & 0xF0F0F0F0u, a & 0xF0F0F0F0u,
                    b & 0xF0F0F0F0u);
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ inline i32x4 as_i32x4(uint4 v) {
  i32x4 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// The store of one wave's share of the tile (rows wr.. wr + 16 TM, columns
// wc.. wc + 16 TN of the workgroup's tile), staged through a wave-private LDS
// region half its rows at a time, with no workgroup barrier: each wave starts
// storing as soon as its own accumulators are final.  Within a wave, LDS
// accesses complete in issue order, so the wave-scope fences only keep the
// compiler from moving the reads above the writes.  `region` holds
// 8 TM rows of 16 TN + 8 bf16 (a 16-byte pad per row spreads the writes of the
// four row groups over the banks); its address is 16-byte aligned.  The
// activation and the bf16 rounding are the same as store_tile's (the bias is
// already in the accumulators).
template <int TM, int TN>
__device__ inline void store_wave_tile(f32x4 (&acc)[TM][TN], uint16_t* __restrict__ Y, int ldy,
                                       int m0, int n0, int row1, int col1, int wr, int wc,
                                       int lane, uint16_t* region, int act) {
  static_assert(TM % 2 == 0, "two halves of the wave's rows");
  constexpr int HT = TM / 2;            // 16-row tiles per half
  constexpr int HR = 16 * HT;           // rows per half
  constexpr int PITCH = 16 * TN + 8;    // staged bf16 per row
  constexpr int CPR = 2 * TN;           // 16-byte chunks per row
  const int fr = lane & 15;
  const int fk = lane >> 4;
  auto write = [&](int h, auto gelu) {
#pragma unroll
    for (int t = 0; t < HT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t* orow = region + (16 * t + 4 * fk + i) * PITCH;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          float v = acc[h * HT + t][tn][i];
          if constexpr (decltype(gelu)::value) v = tail::gelu_tanh(v);
          orow[16 * tn + fr] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
      }
  };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (act == kActGeluTanh)
      write(h, std::true_type{});
    else
      write(h, std::false_type{});
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
    for (int c = lane; c < HR * CPR; c += 64) {
      const int row = c / CPR, ch = c - (c / CPR) * CPR;
      const int m = m0 + wr + h * HR + row, n = n0 + wc + 8 * ch;
      const tail::u32x4 v = *reinterpret_cast<const tail::u32x4*>(region + row * PITCH + 8 * ch);
      if (m < row1 && n < col1)
        __builtin_nontemporal_store(v, reinterpret_cast<tail::u32x4*>(Y + (size_t)m * ldy + n));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  }
}

using tail::tile_of_id;
using tail::xcd_compact;
using tail::kMaxSplits;

// EXPORT = false: the forward.  EXPORT = true: the forward's own launch (the
// same tiles and the same remainder shares) writes the group partials P of the
// window tokens [e_m0, e_m1) x features [e_n0, e_n1) instead of running the
// epilogue.
//
// Remainder split.  When the tile count leaves a last, nearly empty wave of
// workgroups, tile numbers [full, full + rem) are cut along K into `splits`
// shares.  MODE kWhole: block b computes whole tile number b (of `full`).
// MODE kShares: block u computes share u / rem of tile full + u % rem and
// stores its raw fp32 accumulators in `part`.  w4a4_fixup_kernel sums them.
constexpr int kWhole = 0, kShares = 1;

template <class C, bool EXPORT, int MODE>
__global__ __launch_bounds__(C::THREADS, C::MIN_WAVES) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx, const float* __restrict__ T,
    int K, int r, const uint16_t* __restrict__ L2, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scales, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ Y, int ldy, int row0, int row1, int col0, int col1,
    int32_t* __restrict__ P, int e_m0, int e_m1, int e_n0, int e_n1, int full, int rem,
    int splits, float* __restrict__ part, int t_slices, long t_stride, int act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = K / kGroup;
  const int KB = K / 2;
  const int ntm = (row1 - row0 + C::BM - 1) / C::BM;
  const int ntn = (col1 - col0 + C::BN - 1) / C::BN;
  const int stages = (G + GS - 1) / GS;
  int tmi, tni;
  int unit = 0;                       // kShares: slot of this share in `part`
  int s_begin = 0, s_end = stages;    // kShares: this share's stages
  if (MODE == kWhole) {
    tile_of_id(ntm, ntn, xcd_compact(blockIdx.x, full), tmi, tni);
  } else {
    const int tr = blockIdx.x % rem, sp = blockIdx.x / rem;
    tile_of_id(ntm, ntn, full + tr, tmi, tni);
    unit = tr * splits + sp;
    s_begin = (int)((long)stages * sp / splits);
    s_end = (int)((long)stages * (sp + 1) / splits);
  }
  const int m0 = row0 + tmi * C::BM;
  const int n0 = col0 + tni * C::BN;

  auto stage_a = [&](int buf) { return lds + buf * C::STAGE; };
  auto stage_b = [&](int buf) { return lds + buf * C::STAGE + C::A_BYTES; };
  auto stage_sx = [&](int buf) {
    return reinterpret_cast<float*>(lds + buf * C::STAGE + C::A_BYTES + C::B_BYTES);
  };
  auto stage_swn = [&](int buf) { return reinterpret_cast<float2*>(stage_sx(buf) + GS * C::BM); };

  // ---- global -> register staging.  Thread t copies 16-byte piece (t % 4) of
  // rows t/4, t/4 + RPP, ...: piece q holds half h = q % 2 of group q / 2.
  // Every load is unconditional: rows past the matrix re-read its last row,
  // and the missing second group of an odd last stage re-reads the last group.
  // None of those values reaches an output that is stored or exported, and a
  // branch around a load costs exec-mask bookkeeping in every stage.
  constexpr int RPP = C::THREADS / 4;
  constexpr int APASS = (C::BM + RPP - 1) / RPP;
  constexpr int BPASS = (C::BN + RPP - 1) / RPP;
  const int q = tid & 3;
  const int lrow = tid >> 2;
  const uint8_t* a_src[APASS];
  const uint8_t* b_src[BPASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p)
    a_src[p] = qx + (size_t)min(m0 + min(lrow + p * RPP, C::BM - 1), row1 - 1) * KB + q * 16;
#pragma unroll
  for (int p = 0; p < BPASS; ++p)
    b_src[p] = Wq + (size_t)min(n0 + min(lrow + p * RPP, C::BN - 1), col1 - 1) * KB + q * 16;
  // scale rows of this thread, slots idx = tid + u THREADS: idx < BM an
  // activation row, BM <= idx < BM + BN a weight row
  const float* s_src[C::SU];
#pragma unroll
  for (int u = 0; u < C::SU; ++u) {
    const int idx = tid + u * C::THREADS;
    s_src[u] = idx < C::BM ? sx + (size_t)min(m0 + idx, row1 - 1) * G
                           : w_scales + (size_t)min(n0 + min(idx - C::BM, C::BN - 1), col1 - 1) * G;
  }
  // register slots: stage t waits in slot (t - first stage) % PF
  uint4 sa_[C::PF][APASS], sb_[C::PF][BPASS];
  float ss_[C::PF][C::SU][GS];
  auto gload = [&](int s, int slot = 0) {
    uint4 (&sa)[APASS] = sa_[slot];
    uint4 (&sb)[BPASS] = sb_[slot];
    float (&ss)[C::SU][GS] = ss_[slot];
    const int gq = min(s * GS + (q >> 1), G - 1) - (q >> 1);   // stage's first group, clamped for this piece
#pragma unroll
    for (int p = 0; p < APASS; ++p) sa[p] = *reinterpret_cast<const uint4*>(a_src[p] + gq * 32);
#pragma unroll
    for (int p = 0; p < BPASS; ++p) sb[p] = *reinterpret_cast<const uint4*>(b_src[p] + gq * 32);
#pragma unroll
    for (int u = 0; u < C::SU; ++u)
      if (!EXPORT && tid + u * C::THREADS < C::BM + C::BN) {
#pragma unroll
        for (int j = 0; j < GS; ++j) ss[u][j] = s_src[u][min(s * GS + j, G - 1)];
      }
  };
  auto sstore = [&](int buf, int slot = 0) {
    const uint4 (&sa)[APASS] = sa_[slot];
    const uint4 (&sb)[BPASS] = sb_[slot];
    const float (&ss)[C::SU][GS] = ss_[slot];
    const int g = q >> 1, h = q & 1;
#pragma unroll
    for (int p = 0; p < APASS; ++p) {
      const int row = lrow + p * RPP;
      if ((p + 1) * RPP <= C::BM || row < C::BM) {
        uint8_t* panel = stage_a(buf) + g * C::A_PANEL;
        *reinterpret_cast<uint4*>(panel + swz(row, 2 * h)) = widen_lo_hi(sa[p].x, sa[p].y);
        *reinterpret_cast<uint4*>(panel + swz(row, 2 * h + 1)) = widen_lo_hi(sa[p].z, sa[p].w);
      }
    }
#pragma unroll
    for (int p = 0; p < BPASS; ++p) {
      const int row = lrow + p * RPP;
      if ((p + 1) * RPP <= C::BN || row < C::BN) {
        uint8_t* panel = stage_b(buf) + g * C::B_PANEL;
        *reinterpret_cast<uint4*>(panel + swz(row, 2 * h)) = widen_lo_hi(sb[p].x, sb[p].y);
        *reinterpret_cast<uint4*>(panel + swz(row, 2 * h + 1)) = widen_lo_hi(sb[p].z, sb[p].w);
      }
    }
    if (!EXPORT) {
#pragma unroll
      for (int u = 0; u < C::SU; ++u) {
        const int idx = tid + u * C::THREADS;
        if (idx < C::BM) {
#pragma unroll
          for (int j = 0; j < GS; ++j) stage_sx(buf)[j * C::BM + idx] = ss[u][j];
        } else if (idx < C::BM + C::BN) {
          const int col = idx - C::BM;
#pragma unroll
          for (int j = 0; j < GS; ++j)
            stage_swn(buf)[j * C::BN + col] = make_float2(ss[u][j], -kMagic * ss[u][j]);
        }
      }
    }
  };

  // ---- per-wave output tile: TM token tiles x TN feature tiles
  const int wm = wave / C::WN, wn = wave - (wave / C::WN) * C::WN;
  const int wr = wm * C::TM * 16;   // token offset in the workgroup tile
  const int wc = wn * C::TN * 16;   // feature offset
  const int fr = lane & 15;
  const int fk = lane >> 4;
  f32x4 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x4 cmagic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  // One group: 16x16x64 int8 MFMAs over TM x TN tiles, software-pipelined so
  // that the MFMAs of feature tile tn are in flight while the scale epilogue
  // of tile tn - 1 runs on the VALU; the next tile's fragment is read from
  // LDS one tile ahead.  MFMA result layout (16x16): lane l holds column
  // l % 16 and rows 4 * (l / 16) + i, i = 0..3.
  auto do_group = [&](int buf, int g, int gglob) {
    const uint8_t* pa = stage_a(buf) + g * C::A_PANEL;
    const uint8_t* pb = stage_b(buf) + g * C::B_PANEL;
    const float2* pswn = stage_swn(buf) + g * C::BN + wc + fr;
    i32x4 xf[C::TM];
    f32x4 sxv[C::TM];
#pragma unroll
    for (int t = 0; t < C::TM; ++t) {
      xf[t] = as_i32x4(*reinterpret_cast<const uint4*>(pa + swz(wr + 16 * t + fr, fk)));
      if (!EXPORT)
        sxv[t] = *reinterpret_cast<const f32x4*>(stage_sx(buf) + g * C::BM + wr + 16 * t + 4 * fk);
    }
    i32x4 wcur = as_i32x4(*reinterpret_cast<const uint4*>(pb + swz(wc + fr, fk)));
    float2 swc = make_float2(0.f, 0.f);
    if (!EXPORT) swc = pswn[0];
    i32x4 dprev[C::TM];
    float2 swp = swc;
    // The scale epilogue of one 16x16 tile (tn, tm): 8 FMAs (EXPORT: the
    // partials are written instead).
    auto epilogue_tile = [&](const i32x4& d, float2 sw, int tn, int tm) {
      if (EXPORT) {
        const int n = n0 + wc + 16 * tn + fr;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wr + 16 * tm + 4 * fk + i;
          if (m >= e_m0 && m < e_m1 && n >= e_n0 && n < e_n1)
            P[((size_t)(m - e_m0) * (e_n1 - e_n0) + (n - e_n0)) * G + gglob] =
                (d[i] - kMagicBits) >> 8;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float t = __builtin_fmaf(__int_as_float(d[i]), sw.x, sw.y);
          acc[tm][tn][i] = __builtin_fmaf(t, sxv[tm][i], acc[tm][tn][i]);
        }
      }
    };
    // Issue order.  Left alone, the compiler issues all TM x TN MFMAs of the
    // group before any epilogue; the two waves of a SIMD, kept in step by the
    // stage barrier, then contend for the matrix core and the VALU in turn.
    // Instead every MFMA of feature tile tn is paired with the 8 epilogue FMAs
    // of tile tn - 1 (whose MFMA left TM pairs earlier), each pair fenced off,
    // so one wave keeps the matrix core and the VALU busy together.
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      i32x4 wnext = wcur;
      float2 swn = swc;
      if (tn + 1 < C::TN) {
        wnext = as_i32x4(*reinterpret_cast<const uint4*>(pb + swz(wc + 16 * (tn + 1) + fr, fk)));
        if (!EXPORT) swn = pswn[16 * (tn + 1)];
      }
      i32x4 dcur[C::TM];
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) {
        dcur[tm] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xf[tm], wcur, cmagic, 0, 0, 0);
        if (tn > 0) epilogue_tile(dprev[tm], swp, tn - 1, tm);
        if (!EXPORT) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) dprev[tm] = dcur[tm];
      swp = swc;
      wcur = wnext;
      swc = swn;
    }
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) epilogue_tile(dprev[tm], swp, C::TN - 1, tm);
  };

  auto compute_stage = [&](int s, int buf) {
    const int gv = min(GS, G - s * GS);
#pragma nounroll
    for (int g = 0; g < gv; ++g) do_group(buf, g, s * GS + g);
  };
  // With registers to spare (PF > 1), the forward runs its last stage inside
  // the low-rank tail, after that tail's loads have been issued.
  constexpr bool kLastInTail = C::PF > 1 && MODE == kWhole && !EXPORT;
  // Two-buffer tiles store the output wave by wave, each through its own part
  // of the stage buffer that the last stage does not read, so no workgroup
  // barrier follows the last stage or precedes the stores.
  constexpr int kWaveRegion = 8 * C::TM * (16 * C::TN + 8) * 2;   // bytes per wave
  constexpr bool kWaveStore = C::PF == 1 && C::NB == 2 && MODE == kWhole && !EXPORT &&
                              (C::TM % 2) == 0 && C::WM * C::WN * kWaveRegion <= C::STAGE;

  if constexpr (C::NB == 1) {
    // One LDS buffer: stage s goes in, then the loads of stage s + 1 leave
    // while s is computed, and a second barrier frees the buffer.  The CU's
    // other workgroup computes while this one copies and waits.
    const int sb = MODE == kShares ? s_begin : 0;
    const int se = MODE == kShares ? s_end : stages;
    gload(sb);
    for (int s = sb; s < se; ++s) {
      sstore(0);
      __syncthreads();
      if (s + 1 < se) gload(s + 1);
      const int gv = min(GS, G - s * GS);
#pragma nounroll
      for (int g = 0; g < gv; ++g) do_group(0, g, s * GS + g);
      __syncthreads();
    }
  } else if constexpr (C::PF == 1) {
    if (MODE == kWhole) {
      gload(0);
      sstore(0);
      __syncthreads();

      for (int s = 0; s < stages; ++s) {
        const int buf = s & 1;
        if (s + 1 < stages) gload(s + 1);
        const int gv = min(GS, G - s * GS);
#pragma nounroll
        for (int g = 0; g < gv; ++g) do_group(buf, g, s * GS + g);
        if (s + 1 < stages) {
          sstore(buf ^ 1);
          __syncthreads();
        } else if (!kWaveStore) {
          __syncthreads();
        }
      }
    } else if (MODE == kShares) {
      gload(s_begin);
      sstore(0);
      __syncthreads();

      for (int s = s_begin; s < s_end; ++s) {
        const int buf = (s - s_begin) & 1;
        if (s + 1 < s_end) gload(s + 1);
        const int gv = min(GS, G - s * GS);
#pragma nounroll
        for (int g = 0; g < gv; ++g) do_group(buf, g, s * GS + g);
        if (s + 1 < s_end) sstore(buf ^ 1);
        __syncthreads();
      }
    }
  } else {
    // Stages sb+1 .. sb+PF wait in registers while stage sb is in LDS; after
    // each stage the next one goes to LDS and its slot takes the stage PF
    // further.  The barrier waits for the LDS stores only: the loads in
    // flight stay in flight (__syncthreads would drain them).
    const int sb = MODE == kShares ? s_begin : 0;
    const int se = MODE == kShares ? s_end : stages;
    const int last = kLastInTail ? se - 1 : se;   // stages computed here
    gload(sb, 0);
    sstore(0, 0);
#pragma unroll
    for (int j = 1; j <= C::PF; ++j)
      if (sb + j < se) gload(sb + j, j % C::PF);
    lds_barrier();
    for (int s0 = sb; s0 < last; s0 += C::PF) {
#pragma unroll
      for (int j = 0; j < C::PF; ++j) {
        const int s = s0 + j;
        if (s < last) {
          const int buf = (s - sb) & 1;
          compute_stage(s, buf);
          if (s + 1 < se) sstore(buf ^ 1, (j + 1) % C::PF);
          if (s + 1 + C::PF < se) gload(s + 1 + C::PF, (j + 1) % C::PF);
          lds_barrier();
        }
      }
    }
  }

  if (EXPORT) return;

  // ---- remainder split: store this share, or (FIXUP) sum the shares in order.
  // Thread-major float4 slots, so every store and load is one contiguous row
  // of THREADS x 16 bytes.
  constexpr int NACC = C::TM * C::TN;
  if (MODE == kShares) {
    float4* dst = reinterpret_cast<float4*>(part) + (size_t)unit * NACC * C::THREADS + tid;
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const f32x4 a = acc[tm][tn];
        dst[(size_t)(tm * C::TN + tn) * C::THREADS] = make_float4(a[0], a[1], a[2], a[3]);
      }
    return;
  }
  // ---- epilogue: 1/256, + b + T L2^T (bf16 hi/lo MFMA), bf16 store
  if constexpr (kLastInTail) {
    tail::lowrank_bias_add<C::TM, C::TN, 2>(acc, T, t_slices, t_stride, r, L2, bias, m0, n0, row1,
                                            col1, wr, wc, lane, 1.0f, [&] {
      compute_stage(stages - 1, (stages - 1) & 1);
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tm][tn][i] *= (1.0f / 256.0f);
    });
    __syncthreads();   // the last stage's buffer is read before the tile is staged over it
  } else {
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tm][tn][i] *= (1.0f / 256.0f);
    tail::lowrank_bias_add<C::TM, C::TN, 2>(acc, T, t_slices, t_stride, r, L2, bias, m0, n0, row1,
                                            col1, wr, wc, lane, 1.0f, [] {});
  }

  if constexpr (kWaveStore) {
    // the stage buffer the last stage did not read: every wave passed the
    // barrier after the stage that last read it
    const int free_buf = ((stages - 1) & 1) ^ 1;
    uint16_t* region = reinterpret_cast<uint16_t*>(lds + free_buf * C::STAGE + wave * kWaveRegion);
    store_wave_tile<C::TM, C::TN>(acc, Y, ldy, m0, n0, row1, col1, wr, wc, lane, region,
                                        act);
  } else {
    uint16_t* otile = reinterpret_cast<uint16_t*>(lds);
    tail::store_tile<C::TM, C::TN, C::BM, C::BN, C::THREADS>(
        acc, nullptr, Y, ldy, m0, n0, row1, col1, wr, wc, lane, tid,
        [&](int row) { return otile + row * C::BN; }, act);
  }
}

// Fixup of the remainder split (tail::split_fixup): the accumulators are
// 256 times the scaled sums.
template <class C>
__global__ __launch_bounds__(64 * C::TM * C::WN) void w4a4_fixup_kernel(
    const float* __restrict__ part, int full, int splits, const float* __restrict__ T,
    int t_slices, long t_stride, int r, const uint16_t* __restrict__ L2,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int ldy, int row0, int row1,
    int col0, int col1, int act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  tail::split_fixup<C::TM, C::TN, C::WM, C::WN, C::BM, C::BN, C::THREADS>(
      part, full, splits, 1.0f / 256.0f, T, t_slices, t_stride, r, L2, bias, Y, ldy, row0, row1,
      col0, col1, act, lds);
}

template <class C, bool EXPORT, int MODE>
hipError_t set_lds_attr() {
  static bool done = false;  // benign race: every caller sets the same value
  if (!done) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(w4a4_gemm_kernel<C, EXPORT, MODE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    done = true;
  }
  return hipSuccess;
}

template <class C>
int tiles_of(int rows, int cols) {
  return ((rows + C::BM - 1) / C::BM) * ((cols + C::BN - 1) / C::BN);
}

// Tile choice: the biggest tile that still gives every CU at least one
// workgroup.  Where 256 x 192 tiles leave a partly filled last wave, the
// 128 x 192 tile with two workgroups per CU takes over: it has twice the
// granularity, and each workgroup's copies and barrier waits run under the
// other's compute (measured 3-9 % faster on the 4608-token DiT layers, and
// 2 % slower where 256 x 192 tiles fill whole waves, which keep them).
int pick_tile(int rows, int cols) {
  const int cus = device_cu_count();
  const int big = tiles_of<TileBig>(rows, cols);
  if (big >= cus) return big % cus ? 3 : 2;
  if (tiles_of<TileMed>(rows, cols) >= cus) return 1;
  return 0;
}

// Remainder split of the forward (see the kernel).  Only for the big tiles,
// which fill a CU (one 256 x 192 or two 128 x 192 workgroups, so a wave of
// workgroups is `cus * WPE` tiles), and only when the last wave is at most a
// quarter full: then up to 8 K-shares per tile fit in one wave.  A fuller last
// wave gains less than the shares' partial-sum traffic and the fixup pass cost.
struct SplitPlan {
  int full = 0, rem = 0, splits = 1;
  size_t part_bytes = 0;
};

template <class C>
SplitPlan plan_split(int M, int N, int K) {
  SplitPlan p;
  const int tiles = tiles_of<C>(M, N);
  const int cus = device_cu_count() * C::WPE;
  const int stages = (K / kGroup + GS - 1) / GS;
  p.full = tiles;
  const int rem = tiles % cus;
  if (C::BM * C::BN * C::WPE < TileBig::BM * TileBig::BN || tiles < cus || rem == 0 || 4 * rem > cus)
    return p;
  const int splits = std::min(std::min(kMaxSplits, cus / rem), stages);
  if (splits < 2) return p;
  p.full = tiles - rem;
  p.rem = rem;
  p.splits = splits;
  p.part_bytes = (size_t)rem * splits * C::BM * C::BN * sizeof(float);
  return p;
}

SplitPlan plan_forward(int M, int N, int K) {
  switch (pick_tile(M, N)) {
    case 3: return plan_split<TileBig2>(M, N, K);
    case 2: return plan_split<TileBig>(M, N, K);
    case 1: return plan_split<TileMed>(M, N, K);
    default: return plan_split<TileSmall>(M, N, K);
  }
}

template <class C, bool EXPORT>
hipError_t launch_tile(const uint8_t* qx, const float* sx, const float* T, int t_slices, int K, int r,
                       const uint16_t* L2, const uint8_t* Wq, const float* w_scales,
                       const uint16_t* bias, uint16_t* Y, int ldy, int row0, int row1, int col0,
                       int col1, int32_t* P, const int* ewin, float* part, int act,
                       hipStream_t stream) {
  hipError_t e = set_lds_attr<C, EXPORT, kWhole>();
  if (e != hipSuccess) return e;
  const SplitPlan plan = plan_split<C>(row1 - row0, col1 - col0, K);
  const int em0 = EXPORT ? ewin[0] : 0, em1 = EXPORT ? ewin[1] : 0;
  const int en0 = EXPORT ? ewin[2] : 0, en1 = EXPORT ? ewin[3] : 0;
  hipLaunchKernelGGL((w4a4_gemm_kernel<C, EXPORT, kWhole>), dim3(plan.full), dim3(C::THREADS),
                     C::LDS, stream, qx, sx, T, K, r, L2, Wq, w_scales, bias, Y, ldy, row0, row1,
                     col0, col1, P, em0, em1, en0, en1, plan.full, plan.rem, plan.splits, part,
                     t_slices, (long)(row1 - row0) * r, act);
  e = hipGetLastError();
  if (e != hipSuccess || plan.rem == 0) return e;
  if ((e = set_lds_attr<C, EXPORT, kShares>()) != hipSuccess) return e;
  hipLaunchKernelGGL((w4a4_gemm_kernel<C, EXPORT, kShares>), dim3(plan.rem * plan.splits),
                     dim3(C::THREADS), C::LDS, stream, qx, sx, T, K, r, L2, Wq, w_scales, bias, Y,
                     ldy, row0, row1, col0, col1, P, em0, em1, en0, en1, plan.full, plan.rem,
                     plan.splits, part, t_slices, (long)(row1 - row0) * r, act);
  if ((e = hipGetLastError()) != hipSuccess || EXPORT) return e;
  hipLaunchKernelGGL((w4a4_fixup_kernel<C>), dim3(plan.rem * C::WM), dim3(64 * C::TM * C::WN),
                     16 * C::TM * C::BN * 2, stream, part, plan.full, plan.splits, T, t_slices,
                     (long)(row1 - row0) * r, r, L2, bias, Y, ldy, row0, row1, col0, col1, act);
  return hipGetLastError();
}

template <bool EXPORT>
hipError_t dispatch(const uint8_t* qx, const float* sx, const float* T, int t_slices, int K, int r,
                    const uint16_t* L2, const uint8_t* Wq, const float* w_scales,
                    const uint16_t* bias, uint16_t* Y, int ldy, int row0, int row1, int col0,
                    int col1, int32_t* P, const int* ewin, float* part, int act,
                    hipStream_t stream) {
  switch (pick_tile(row1 - row0, col1 - col0)) {
    case 3:
      return launch_tile<TileBig2, EXPORT>(qx, sx, T, t_slices, K, r, L2, Wq, w_scales, bias, Y, ldy,
                                           row0, row1, col0, col1, P, ewin, part, act, stream);
    case 2:
      return launch_tile<TileBig, EXPORT>(qx, sx, T, t_slices, K, r, L2, Wq, w_scales, bias, Y, ldy,
                                          row0, row1, col0, col1, P, ewin, part, act, stream);
    case 1:
      return launch_tile<TileMed, EXPORT>(qx, sx, T, t_slices, K, r, L2, Wq, w_scales, bias, Y, ldy,
                                          row0, row1, col0, col1, P, ewin, part, act, stream);
    default:
      return launch_tile<TileSmall, EXPORT>(qx, sx, T, t_slices, K, r, L2, Wq, w_scales, bias, Y,
                                            ldy, row0, row1, col0, col1, P, ewin, part, act, stream);
  }
}

}  // namespace

size_t gemm_split_bytes(int M, int K, int N) { return plan_forward(M, N, K).part_bytes; }

hipError_t launch_w4a4_gemm(const uint8_t* qx, const float* sx, const float* T, int t_slices,
                            int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                            const float* w_scales, const uint16_t* bias, uint16_t* Y,
                            float* part, int act, hipStream_t stream) {
  return dispatch<false>(qx, sx, T, t_slices, K, r, L2, Wq, w_scales, bias, Y, N, 0, M, 0, N,
                         nullptr, nullptr, part, act, stream);
}

// The forward's launch for an M x N x K problem -- its tile class, its tile
// order and its remainder shares -- with P exported for the window instead of
// the epilogue.  Every tile runs; only the window's entries are written.
hipError_t launch_group_partials(const uint8_t* qx, const uint8_t* Wq, int M, int N, int K,
                                 int m0, int m1, int n0, int n1, int32_t* P, hipStream_t stream) {
  const int win[4] = {m0, m1, n0, n1};
  return dispatch<true>(qx, nullptr, nullptr, 0, K, 0, nullptr, Wq, nullptr, nullptr, nullptr, 0, 0,
                        M, 0, N, P, win, nullptr, kActNone, stream);
}

}  // namespace svdq
