// k2, MXFP4 variant: block-scaled FP4 GEMM with the low-rank up projection and
// the bias in the epilogue, gfx950.
//
// The same dual-path output as the int4 GEMM (Terminology Entry, section 2.3,
// E4 and E7), with Q(.) taken as MXFP4: activations and the residual weights
// are FP4 E2M1 numbers with one E8M0 (power-of-two) scale per 32 input
// channels.  CDNA4 multiplies such blocks natively:
// v_mfma_scale_f32_16x16x128_f8f6f4 takes 128 channels of FP4 per row and
// column and one scale byte per lane, applies 2^(ea + eb) to each 32-channel
// block product and accumulates in fp32.  So the scales cost nothing: no
// per-group epilogue, the accumulator stays in the MFMA from the first
// channel to the last.
//
// Operand layout (measured on the hardware): lane l supplies row (or column)
// l % 16, channels 32 (l / 16) .. + 31 of the 128, as 16 bytes with channel
// 2i in the low nibble of byte i -- the canonical packed row order -- and the
// scale byte of that 32-channel block in the low byte of its scale register.
//
// Data path: two 128-channel steps per pipeline stage; the stage's A and B
// rows (128 bytes each) and scale bytes (8 per row) are copied from global
// memory straight into LDS (global_load_lds: no registers, no ALU), double
// buffered.  Both scale operands come k-tiled ([ceil(K/256)][rows][8]): a
// tile's scales of one stage are then one contiguous run, 1 KB per copy,
// where row-major [rows, K/32] scales would cost one 8-byte piece per row.  The compiler makes every LDS read wait for all copies in flight
// (it cannot tell the two buffers apart), so a wave first reads all of its
// fragments and scales of the stage, then issues its copies of the next stage,
// then runs the stage's 2 x TM x TN MFMAs while the copies travel.
//
// The 16-byte chunks of a row are XOR-swizzled (see swz_key); the direct copy
// writes lane-linear LDS addresses, so each lane fetches the global chunk that
// belongs at its LDS position.
//
// The low-rank branch's up projection T L2^T initializes the accumulators
// before the main loop (its loads are issued together, without branches, right
// after the first stage's copies), so that only the bias and the store are
// left after it.
#include "gemm_tail.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int KS = 128;           // channels per MFMA
constexpr int SK = 2;             // MFMA k-steps per pipeline stage
constexpr int ROWB = SK * KS / 2; // FP4 bytes per row and stage (128)
constexpr int SROWB = SK * KS / 32; // scale bytes per row and stage (8)
constexpr int kFmtFp4 = 4;        // cbsz / blgp code of FP4 E2M1

template <int WM_, int WN_, int TM_, int TN_>
struct MxTile {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int BM = WM * TM * 16;
  static constexpr int BN = WN * TN * 16;
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int B_BYTES = BN * ROWB;
  // scale bytes of a stage, rounded up to whole 1 KB copies (the rows past
  // the tile that fill the rest are never read)
  static constexpr int SA_BYTES = (BM * SROWB + 1023) / 1024 * 1024;
  static constexpr int SB_BYTES = (BN * SROWB + 1023) / 1024 * 1024;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int OUT = BM * BN * 2;
  static constexpr int LDS = (2 * STAGE > OUT ? 2 * STAGE : OUT);
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KB copies");
  static_assert(SA_BYTES % 1024 == 0 && SB_BYTES % 1024 == 0, "whole 1 KB copies");
};

using MxBig = MxTile<4, 2, 4, 6>;    // 256 x 192, 8 waves
using MxMed = MxTile<2, 2, 4, 4>;    // 128 x 128, 4 waves
using MxSmall = MxTile<2, 2, 2, 2>;  //  64 x  64, 4 waves

__device__ inline int xcd_compact(int b, int count) {
  return (count & 7) == 0 ? (b & 7) * (count >> 3) + (b >> 3) : b;
}

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

// The 8 chunks of a 128-byte row are XOR-swizzled by row % 8.  A fragment read
// spans 16 consecutive rows starting at a multiple of 16, so the key depends on
// the lane alone and every fragment of a wave shares one base address plus
// immediate offsets; the LDS reports no bank conflicts for this pattern.
__device__ inline int swz_key(int row) { return row & 7; }
// byte offset of logical 16-byte chunk c of LDS row `row`
__device__ inline int swz(int row, int c) { return row * ROWB + ((c ^ swz_key(row)) << 4); }

template <class C>
__global__ __launch_bounds__(C::THREADS) void mxfp4_gemm_kernel(
    const uint8_t* __restrict__ qx, const uint8_t* __restrict__ sx, int sx_rows,
    const float* __restrict__ T, int t_slices, long t_stride, int M, int K, int N, int r,
    const uint16_t* __restrict__ L2,
    const uint8_t* __restrict__ Wq, const uint8_t* __restrict__ sw,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int KB = K / 2;            // packed bytes per row
  const int ksteps = K / KS;
  const int stages = (ksteps + SK - 1) / SK;
  const int ntm = (M + C::BM - 1) / C::BM;
  const int ntn = (N + C::BN - 1) / C::BN;
  int tmi, tni;
  tile_of_id(ntm, ntn, xcd_compact(blockIdx.x, ntm * ntn), tmi, tni);
  const int m0 = tmi * C::BM;
  const int n0 = tni * C::BN;

  auto stage_a = [&](int buf) { return lds + buf * C::STAGE; };
  auto stage_b = [&](int buf) { return lds + buf * C::STAGE + C::A_BYTES; };
  auto stage_sa = [&](int buf) { return lds + buf * C::STAGE + C::A_BYTES + C::B_BYTES; };
  auto stage_sb = [&](int buf) { return stage_sa(buf) + C::SA_BYTES; };

  // ---- global -> LDS copies of stage s.  A copy instruction moves 64 lanes x
  // 16 bytes to consecutive LDS; lane j of copy q fills LDS byte q * 1024 + 16 j,
  // i.e. row (q * 1024 + 16 j) / ROWB, physical chunk j % 8, and fetches the
  // logical chunk that the swizzle puts there.  Rows past the matrix and the
  // missing second step of an odd last stage re-read valid data, never used.
  auto copy_rows = [&](const uint8_t* src, int nrows_total, int row_base, int ld, int s,
                       uint8_t* dst, int bytes) {
    const int jrow = lane >> 3, pch = lane & 7;
    for (int q = wave; q < bytes / 1024; q += C::WAVES) {
      const int row = q * (1024 / ROWB) + jrow;
      int chunk = pch ^ swz_key(row);
      if (s * SK + (chunk >> 2) >= ksteps) chunk &= 3;
      const uint8_t* g = src + (size_t)min(row_base + row, nrows_total - 1) * ld + s * ROWB + chunk * 16;
      __builtin_amdgcn_global_load_lds(g, (lds_ptr)(dst + q * 1024), 16, 0, 0);
    }
  };
  // Scales are k-tiled: stage s of rows [0, rows) is one run of 8 * rows
  // bytes (rows even), so a tile's scales of a stage are contiguous and move
  // as 1 KB copies of 16 bytes per lane.  Lanes past the run re-read its last
  // 16 bytes, into LDS rows that are never read.  An odd last stage has no
  // second step; its upper 4 bytes per row are never used.
  auto copy_scales = [&](const uint8_t* src, int rows, int row_base, int s, uint8_t* dst,
                         int bytes) {
    const uint8_t* run = src + (size_t)s * rows * SROWB;
    const int last = rows * SROWB - 16;
    for (int q = wave; q < bytes / 1024; q += C::WAVES) {
      const int off = min(row_base * SROWB + q * 1024 + lane * 16, last);
      __builtin_amdgcn_global_load_lds(run + off, (lds_ptr)(dst + q * 1024), 16, 0, 0);
    }
  };
  auto copy_stage = [&](int s, int buf) {
    copy_rows(qx, M, m0, KB, s, stage_a(buf), C::A_BYTES);
    copy_rows(Wq, N, n0, KB, s, stage_b(buf), C::B_BYTES);
    copy_scales(sx, sx_rows, m0, s, stage_sa(buf), C::SA_BYTES);
    copy_scales(sw, N, n0, s, stage_sb(buf), C::SB_BYTES);
  };

  const int wm = wave / C::WN, wn = wave - (wave / C::WN) * C::WN;
  const int wr = wm * C::TM * 16;
  const int wc = wn * C::TN * 16;
  const int fr = lane & 15;
  const int fk = lane >> 4;
  f32x4 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A stage from LDS: the fragments of both steps (16 bytes per lane each) and
  // each row's 8 scale bytes, then the copies of the next stage, then the MFMAs.
  // The scale of block fk in step ks is byte 4 ks + fk of the row's 8, moved to
  // byte 0 of the MFMA's scale operand.
  auto stage = [&](int buf, bool second, bool more, int s) {
    const uint8_t* pa = stage_a(buf);
    const uint8_t* pb = stage_b(buf);
    const uint8_t* psa = stage_sa(buf);
    const uint8_t* psb = stage_sb(buf);
    uint4 af[SK][C::TM], bf[SK][C::TN];
    uint2 sa[C::TM], sb[C::TN];
#pragma unroll
    for (int t = 0; t < C::TM; ++t) {
      const int row = wr + 16 * t + fr;
#pragma unroll
      for (int ks = 0; ks < SK; ++ks)
        af[ks][t] = *reinterpret_cast<const uint4*>(pa + swz(row, 4 * ks + fk));
      sa[t] = *reinterpret_cast<const uint2*>(psa + row * SROWB);
    }
#pragma unroll
    for (int t = 0; t < C::TN; ++t) {
      const int row = wc + 16 * t + fr;
#pragma unroll
      for (int ks = 0; ks < SK; ++ks)
        bf[ks][t] = *reinterpret_cast<const uint4*>(pb + swz(row, 4 * ks + fk));
      sb[t] = *reinterpret_cast<const uint2*>(psb + row * SROWB);
    }
    if (more) copy_stage(s + 1, buf ^ 1);
#pragma unroll
    for (int ks = 0; ks < SK; ++ks) {
      if (ks == 1 && !second) break;
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const int sbv = (int)((ks ? sb[tn].y : sb[tn].x) >> (8 * fk));
        const uint4 b = bf[ks][tn];
        const v8i bv = v8i{(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
#pragma unroll
        for (int tm = 0; tm < C::TM; ++tm) {
          const int sav = (int)((ks ? sa[tm].y : sa[tm].x) >> (8 * fk));
          const uint4 a = af[ks][tm];
          const v8i av = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              av, bv, acc[tm][tn], kFmtFp4, kFmtFp4, 0, sav, 0, sbv);
        }
      }
    }
  };

  tail::lowrank_bias_add<C::TM, C::TN, 0>(acc, T, t_slices, t_stride, r, L2, nullptr, m0, n0, M,
                                          N, wr, wc, lane, 1.0f, [&] { copy_stage(0, 0); });
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int s = 0; s < stages; ++s) {
    stage(s & 1, s * SK + 1 < ksteps, s + 1 < stages, s);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies of the next stage have landed
    __syncthreads();                 // ... and everyone's; the current buffer is free
  }

  uint16_t* otile = reinterpret_cast<uint16_t*>(lds);
  tail::store_tile<C::TM, C::TN, C::BM, C::BN, C::THREADS>(
      acc, bias, Y, N, m0, n0, M, N, wr, wc, lane, tid,
      [&](int row) { return otile + row * C::BN; }, act);
}

int cu_count_mx() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

template <class C>
int tiles_of(int rows, int cols) {
  return ((rows + C::BM - 1) / C::BM) * ((cols + C::BN - 1) / C::BN);
}

template <class C>
hipError_t launch(const uint8_t* qx, const uint8_t* sx, int sx_rows, const float* T, int t_slices,
                  int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                  const uint8_t* sw, const uint16_t* bias, uint16_t* Y, int act,
                  hipStream_t stream) {
  static bool attr = false;  // benign race: every caller sets the same value
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(mxfp4_gemm_kernel<C>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(mxfp4_gemm_kernel<C>, dim3(tiles_of<C>(M, N)), dim3(C::THREADS), C::LDS,
                     stream, qx, sx, sx_rows, T, t_slices, (long)M * r, M, K, N, r, L2, Wq, sw, bias,
                     Y, act);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp4_gemm(const uint8_t* qx, const uint8_t* sx_e8m0, int sx_rows, const float* T,
                             int t_slices, int M, int K, int N, int r, const uint16_t* L2,
                             const uint8_t* Wq, const uint8_t* w_e8m0, const uint16_t* bias,
                             uint16_t* Y, int act, hipStream_t stream) {
  const int cus = cu_count_mx();
  if (tiles_of<MxBig>(M, N) >= cus)
    return launch<MxBig>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias, Y, act, stream);
  if (tiles_of<MxMed>(M, N) >= cus)
    return launch<MxMed>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias, Y, act, stream);
  return launch<MxSmall>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias, Y, act, stream);
}

}  // namespace svdq
