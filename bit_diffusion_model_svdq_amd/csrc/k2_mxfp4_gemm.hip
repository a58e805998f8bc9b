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
// Data path: a ring of NR LDS buffers, one 128-channel step each, filled
// straight from global memory (global_load_lds: no registers, no ALU) NR - 1
// steps ahead of the MFMAs, so that the copies' latency hides behind several
// steps of work.  A buffer holds the step's A and B rows (64 bytes each,
// 16-byte chunks XOR-swizzled by row so that a fragment read spreads over the
// banks) and the tile's scale bytes of the step pair.  Both scale operands
// come k-tiled ([ceil(K/256)][rows][8]), so those are one contiguous run per
// tile and move as 1 KB copies; a step uses the low or high 4 bytes of each
// row's 8.  Every wave issues the same number of copies per step (the last is
// repeated to even them out), so s_waitcnt vmcnt waits for exactly this
// wave's copies of the step while the later steps' stay in flight; a plain
// s_barrier then makes everyone's copies visible (__syncthreads would wait
// for all copies in flight).  Each buffer is its own __shared__ array: the
// compiler then knows that reading one buffer does not depend on the copies
// into another and issues no wait for them.
//
// The low-rank branch's up projection T L2^T initializes the accumulators
// before the main loop (its loads are issued together, without branches, right
// after the first NR - 1 steps' copies), so that only the bias and the store
// are left after it.  A nearly empty last wave of tiles is cut along K into
// shares finished by tail::split_fixup, which adds the branch there instead.
#include "gemm_tail.h"
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int KS = 128;             // channels per MFMA step
constexpr int ROWB = KS / 2;        // FP4 bytes per row and step (64)
constexpr int SROWB = 8;            // k-tiled scale bytes per row and pair of steps
constexpr int kFmtFp4 = 4;          // cbsz / blgp code of FP4 E2M1

template <int WM_, int WN_, int TM_, int TN_, int NR_ = 4>
struct MxTile {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int NR = NR_;     // ring buffers: NR - 1 steps of copies ahead
  static constexpr int BM = WM * TM * 16;
  static constexpr int BN = WN * TN * 16;
  static constexpr int WAVES = WM * WN;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int ROWS_BYTES = (BM + BN) * ROWB;   // A rows, then B rows
  // scale bytes of the step pair, rounded up to whole 1 KB copies (the rows
  // past the tile that fill the rest are never read)
  static constexpr int SA_BYTES = (BM * SROWB + 1023) / 1024 * 1024;
  static constexpr int SB_BYTES = (BN * SROWB + 1023) / 1024 * 1024;
  static constexpr int BUF = ROWS_BYTES + SA_BYTES + SB_BYTES;
  static constexpr int ROW_COPIES = ROWS_BYTES / 1024;
  static constexpr int COPIES = ROW_COPIES + (SA_BYTES + SB_BYTES) / 1024;   // per step
  static constexpr int CPW = (COPIES + WAVES - 1) / WAVES;                   // per wave and step
  static constexpr int OUT_ROWS = (BM + NR - 1) / NR;   // output rows staged per buffer
  static constexpr int WPE = THREADS >= 512 ? 1 : 2;    // workgroups a CU holds
  static_assert(NR == 3 || NR == 4, "three or four ring buffers");
  static_assert(ROWS_BYTES % 1024 == 0, "whole 1 KB row copies");
  static_assert(OUT_ROWS * BN * 2 <= BUF, "the output tile fits the ring");
  static_assert(CPW * (NR - 2) < 64, "vmcnt range");
};

using MxBig = MxTile<4, 2, 4, 6>;    // 256 x 192, 8 waves
// 128 x 192, 4 waves, two workgroups per CU (a three-buffer ring of 23 KB
// each), where 256 x 192 tiles leave a partly filled last wave
using MxBig2 = MxTile<2, 2, 4, 6, 3>;
using MxMed = MxTile<2, 2, 4, 4>;    // 128 x 128, 4 waves
using MxSmall = MxTile<2, 2, 2, 2>;  //  64 x  64, 4 waves

using tail::tile_of_id;
using tail::xcd_compact;
using tail::kMaxSplits;

// XOR key of the 16-byte chunks of a 64-byte LDS row: a fragment read covers
// 16 consecutive rows (from a multiple of 16) and chunk l / 16 per lane; the
// key (row / 2) % 4 spreads them over all banks.
__device__ inline int swz_key(int row) { return (row >> 1) & 3; }

// s_waitcnt with vmcnt = n, the other counters untouched
template <int n>
__device__ inline void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// The wait before a barrier of the ring: vmcnt = n (this wave's copies of the
// step have landed; later steps' stay in flight) and lgkmcnt = 0, so that every
// LDS read this wave has issued is complete before the barrier lets another
// wave's copies into a buffer it read.  Without the lgkmcnt part the scheduler
// sinks a step's last MFMAs, and with them the wait for their operands, below
// the next barrier: a fragment read still in flight there can return bytes
// another wave's copy has just overwritten.  (A workgroup fence on LDS would
// also drain the copies in flight, since they write LDS.)
template <int n>
__device__ inline void ring_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
}

// MODE kWhole: block b computes whole tile number b of `full`.  MODE kShares
// (remainder split, see tail::split_fixup): block u computes share u / rem of
// tile full + u % rem, its steps only, and stores its raw accumulators in
// `part`; the fixup adds the low-rank branch and the bias.
constexpr int kWhole = 0, kShares = 1;

template <class C, int MODE>
__global__ __launch_bounds__(C::THREADS, 2) void mxfp4_gemm_kernel(
    const uint8_t* __restrict__ qx, const uint8_t* __restrict__ sx, int sx_rows,
    const float* __restrict__ T, int t_slices, long t_stride, int M, int K, int N, int r,
    const uint16_t* __restrict__ L2, const uint8_t* __restrict__ Wq,
    const uint8_t* __restrict__ sw, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ Y, int act, int full, int rem, int splits,
    float* __restrict__ part) {
  constexpr int NR = C::NR;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[C::BUF];
  __shared__ __attribute__((aligned(16))) uint8_t ring3[NR == 4 ? C::BUF : 16];   // NR = 3: unused
  // Four-buffer rings (one workgroup per CU) store the output wave by wave
  // through a staging area of their own beside the ring, 16 rows of a wave's
  // share at a time: no barrier after the last step, and the ring's last
  // copies (repeats past the last step, never read) may still land meanwhile.
  constexpr bool kWaveStore = MODE == kWhole && NR == 4;
  constexpr int kStagePitch = 16 * C::TN + 8;                 // bf16 per staged row (16-byte pad)
  constexpr int kStageBytes = 16 * kStagePitch * 2;           // per wave
  __shared__ __attribute__((aligned(16))) uint8_t wstage[kWaveStore ? C::WAVES * kStageBytes : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar registers
  const int KB = K / 2;            // packed bytes per row
  const int ksteps = K / KS;
  const int ntm = (M + C::BM - 1) / C::BM;
  const int ntn = (N + C::BN - 1) / C::BN;
  int tmi, tni;
  int sb = 0, se = ksteps, unit = 0;     // this block's steps; kShares: its slot in `part`
  if (MODE == kWhole) {
    tile_of_id(ntm, ntn, xcd_compact(blockIdx.x, full), tmi, tni);
  } else {
    const int tr = blockIdx.x % rem, sp = blockIdx.x / rem;
    tile_of_id(ntm, ntn, full + tr, tmi, tni);
    unit = tr * splits + sp;
    sb = (int)((long)ksteps * sp / splits);
    se = (int)((long)ksteps * (sp + 1) / splits);
  }
  const int nsteps = se - sb;
  const int m0 = tmi * C::BM;
  const int n0 = tni * C::BN;

  // ---- this wave's copies of a step: copy q = wave + i WAVES (the last one
  // repeated where the count does not divide), 1 KB each.  A row copy fills
  // LDS rows 16 q .. + 15 (A rows, then B rows), lane j the physical chunk
  // j % 4 of row 16 q + j / 4, fetched from the logical chunk the swizzle puts
  // there.  A scale copy fills 1 KB of the A or B scale run of the step pair.
  // Rows past the matrix re-read its last row, scale lanes past a run its last
  // 16 bytes: never used.
  const uint8_t* src[C::CPW];
  int dst[C::CPW];
  bool is_scale[C::CPW];
  long pair_stride[C::CPW];      // scale copies: bytes from one step pair to the next
#pragma unroll
  for (int i = 0; i < C::CPW; ++i) {
    const int q = min(wave + i * C::WAVES, C::COPIES - 1);
    is_scale[i] = q >= C::ROW_COPIES;
    if (!is_scale[i]) {
      const int row = q * 16 + (lane >> 2);
      const int chunk = (lane & 3) ^ swz_key(row);
      src[i] = (row < C::BM ? qx + (size_t)min(m0 + row, M - 1) * KB
                            : Wq + (size_t)min(n0 + row - C::BM, N - 1) * KB) + chunk * 16;
      dst[i] = q * 1024;
      pair_stride[i] = 0;
    } else {
      const int qs = q - C::ROW_COPIES;
      const bool a = qs < C::SA_BYTES / 1024;
      const int rows = a ? sx_rows : N;
      const int base = (a ? m0 : n0) * SROWB + (a ? qs : qs - C::SA_BYTES / 1024) * 1024;
      src[i] = (a ? sx : sw) + min(base + lane * 16, rows * SROWB - 16);
      dst[i] = C::ROWS_BYTES + qs * 1024;
      pair_stride[i] = (long)rows * SROWB;
    }
  }
  auto copy_step = [&](int s, uint8_t* buf) {
#pragma unroll
    for (int i = 0; i < C::CPW; ++i) {
      const uint8_t* g = src[i] + (is_scale[i] ? (s >> 1) * pair_stride[i] : (long)s * ROWB);
      __builtin_amdgcn_global_load_lds(g, (lds_ptr)(buf + dst[i]), 16, 0, 0);
    }
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

  // Fragment addresses: tile t of a wave starts 16 rows further and the
  // swizzle key of row 16 t + fr is that of fr, so every fragment of a kind is
  // one lane base plus a compile-time offset.  The scale of block fk in step
  // s is byte 4 (s % 2) + fk of the row's 8.
  const int swz_lane = (fk ^ swz_key(fr)) << 4;
  const int a_lane = (wr + fr) * ROWB + swz_lane;
  const int b_lane = (C::BM + wc + fr) * ROWB + swz_lane;
  const int sa_lane = C::ROWS_BYTES + (wr + fr) * SROWB + fk;
  const int sb_lane = C::ROWS_BYTES + C::SA_BYTES + (wc + fr) * SROWB + fk;

  // Step sb + j: wait for this wave's copies of the step (those of the next
  // two stay in flight), barrier (everyone's have landed, and everyone is done
  // with step j - 1), copy step j + NR - 1 into the buffer step j - 1 used
  // (past the last step: a repeat of the last step, never read), then the
  // step's fragments and MFMAs.
  auto step = [&](int j, const uint8_t* cur, uint8_t* freed) {
    const int s = sb + j;
    ring_wait<C::CPW * (NR - 2)>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    copy_step(sb + min(j + NR - 1, nsteps - 1), freed);
    __builtin_amdgcn_sched_barrier(0);   // the copies leave before the step's work
    const int h = 4 * (s & 1);
    uint4 af[C::TM], bf[C::TN];
    int sa[C::TM], sb[C::TN];
#pragma unroll
    for (int t = 0; t < C::TM; ++t) {
      af[t] = *reinterpret_cast<const uint4*>(cur + a_lane + t * 16 * ROWB);
      sa[t] = cur[sa_lane + h + t * 16 * SROWB];
    }
#pragma unroll
    for (int t = 0; t < C::TN; ++t) {
      bf[t] = *reinterpret_cast<const uint4*>(cur + b_lane + t * 16 * ROWB);
      sb[t] = cur[sb_lane + h + t * 16 * SROWB];
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const v8i bv = v8i{(int)bf[tn].x, (int)bf[tn].y, (int)bf[tn].z, (int)bf[tn].w, 0, 0, 0, 0};
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) {
        const v8i av = v8i{(int)af[tm].x, (int)af[tm].y, (int)af[tm].z, (int)af[tm].w, 0, 0, 0, 0};
        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            av, bv, acc[tm][tn], kFmtFp4, kFmtFp4, 0, sa[tm], 0, sb[tn]);
      }
    }
  };

  // prologue: the first NR - 1 steps' copies leave with the low-rank loads
  // (shares leave the low-rank branch to the fixup)
  auto first_copies = [&] {
    copy_step(sb, ring0);
    copy_step(sb + min(1, nsteps - 1), ring1);
    if (NR == 4) copy_step(sb + min(2, nsteps - 1), ring2);
  };
  if (MODE == kWhole && NR == 4 && r >= 16 && r <= 32 && t_slices <= 2) {
    // One chunk of ranks and at most two T slices (every rank of the usual
    // layers): the same arithmetic as tail::lowrank_bias_add, but its loads
    // leave before the first copies and the wait for them leaves the copies
    // in flight, so the branch's MFMAs run under the copies' latency.  (The
    // general routine's runtime loops over rank chunks and slices make the
    // compiler wait for every load in flight.)  Four-buffer rings only: with
    // two workgroups per CU (the three-buffer ring) the other workgroup
    // already covers the prologue, and there this head measured slower.
    const int jc = min(8 * fk, r - 8);
    const bool j_ok = 8 * fk < r;
    const long s1 = t_slices > 1 ? t_stride : 0;
    float4 ta[C::TM], tb[C::TM], ua[C::TM], ub[C::TM];
    uint4 lf[C::TN];
#pragma unroll
    for (int t = 0; t < C::TM; ++t) {
      const float* tr = T + (size_t)min(m0 + wr + 16 * t + fr, M - 1) * r + jc;
      ta[t] = *reinterpret_cast<const float4*>(tr);
      tb[t] = *reinterpret_cast<const float4*>(tr + 4);
      ua[t] = *reinterpret_cast<const float4*>(tr + s1);
      ub[t] = *reinterpret_cast<const float4*>(tr + s1 + 4);
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
      lf[tn] = *reinterpret_cast<const uint4*>(L2 + (size_t)min(n0 + wc + 16 * tn + fr, N - 1) * r + jc);
    __builtin_amdgcn_sched_barrier(0);   // the branch's loads leave first,
    first_copies();
    __builtin_amdgcn_sched_barrier(0);   // then the copies,
    wait_vmcnt<C::CPW * (NR - 1)>();     // and the wait leaves only the copies in flight
    __builtin_amdgcn_sched_barrier(0);
    // the second slice's sum, unconditional so that its loads stay ahead of
    // the copies (in a branch the compiler moves them behind the wait);
    // with one slice it adds -0, which leaves every value as it is
    const bool two = t_slices > 1;
    const float4 nz = make_float4(-0.f, -0.f, -0.f, -0.f);
#pragma unroll
    for (int t = 0; t < C::TM; ++t) {
      ta[t] = tail::add4(ta[t], two ? ua[t] : nz);
      tb[t] = tail::add4(tb[t], two ? ub[t] : nz);
    }
    // ranks past r are zeroed by a bit mask (+0, as a select would give): a
    // select on a loaded value may become a load under a lane mask, behind
    // the wait
    const uint32_t jm = j_ok ? 0xFFFFFFFFu : 0u;
    tail::bf16x8 thi[C::TM], tlo[C::TM];
#pragma unroll
    for (int t = 0; t < C::TM; ++t) {
      const float tv[8] = {ta[t].x, ta[t].y, ta[t].z, ta[t].w, tb[t].x, tb[t].y, tb[t].z, tb[t].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = __uint_as_float(__float_as_uint(tv[e]) & jm);
        const __bf16 h = (__bf16)v;
        thi[t][e] = h;
        tlo[t][e] = (__bf16)(v - (float)h);
      }
    }
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn) {
      const tail::bf16x8 l =
          tail::as_bf16x8(make_uint4(lf[tn].x & jm, lf[tn].y & jm, lf[tn].z & jm, lf[tn].w & jm));
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm) {
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(thi[tm], l, acc[tm][tn], 0, 0, 0);
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tlo[tm], l, acc[tm][tn], 0, 0, 0);
      }
    }
  } else if (MODE == kWhole) {
    tail::lowrank_bias_add<C::TM, C::TN, 0>(acc, T, t_slices, t_stride, r, L2, nullptr, m0, n0, M,
                                            N, wr, wc, lane, 1.0f, first_copies);
  } else {
    first_copies();
  }
  // whole turns of the ring without branches (so that the compiler's count of
  // the copies in flight stays exact), then the last 0..3 steps
  int j0 = 0;
  if constexpr (NR == 4) {
    for (; j0 + NR <= nsteps; j0 += NR) {
      step(j0, ring0, ring3);
      step(j0 + 1, ring1, ring0);
      step(j0 + 2, ring2, ring1);
      step(j0 + 3, ring3, ring2);
    }
    if (j0 < nsteps) step(j0, ring0, ring3);
    if (j0 + 1 < nsteps) step(j0 + 1, ring1, ring0);
    if (j0 + 2 < nsteps) step(j0 + 2, ring2, ring1);
  } else {
    for (; j0 + NR <= nsteps; j0 += NR) {
      step(j0, ring0, ring2);
      step(j0 + 1, ring1, ring0);
      step(j0 + 2, ring2, ring1);
    }
    if (j0 < nsteps) step(j0, ring0, ring2);
    if (j0 + 1 < nsteps) step(j0 + 1, ring1, ring0);
  }

  // every copy has landed (a workgroup may not leave copies into its LDS
  // behind) and every wave's reads of the ring are complete before the output
  // tile is staged over it
  ring_wait<0>();
  if constexpr (kWaveStore) {
    asm volatile("" ::: "memory");
    uint16_t* region = reinterpret_cast<uint16_t*>(wstage + wave * kStageBytes);
    float bv[C::TN];
#pragma unroll
    for (int tn = 0; tn < C::TN; ++tn)
      bv[tn] = bias ? __uint_as_float(uint32_t(bias[min(n0 + wc + 16 * tn + fr, N - 1)]) << 16) : 0.f;
    auto write = [&](int tm, auto gelu) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t* orow = region + (4 * fk + i) * kStagePitch;
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
          float v = acc[tm][tn][i] + bv[tn];
          if constexpr (decltype(gelu)::value) v = tail::gelu_tanh(v);
          orow[16 * tn + fr] = __builtin_bit_cast(uint16_t, (__bf16)v);
        }
      }
    };
    constexpr int CPR = 2 * C::TN;   // 16-byte chunks per staged row
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm) {
      if (act == kActGeluTanh)
        write(tm, std::true_type{});
      else
        write(tm, std::false_type{});
      // a wave's LDS accesses complete in issue order; the fences keep the
      // compiler's order of the writes, the reads and the next pass's writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
#pragma unroll
      for (int c = lane; c < 16 * CPR; c += 64) {
        const int row = c / CPR, ch = c - (c / CPR) * CPR;
        const int m = m0 + wr + 16 * tm + row, n = n0 + wc + 8 * ch;
        const tail::u32x4 v = *reinterpret_cast<const tail::u32x4*>(region + row * kStagePitch + 8 * ch);
        if (m < M && n < N)
          __builtin_nontemporal_store(v, reinterpret_cast<tail::u32x4*>(Y + (size_t)m * N + n));
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
    return;
  }
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  if (MODE == kShares) {
    float4* dst = reinterpret_cast<float4*>(part) + (size_t)unit * C::TM * C::TN * C::THREADS + tid;
#pragma unroll
    for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < C::TN; ++tn) {
        const f32x4 a = acc[tm][tn];
        dst[(size_t)(tm * C::TN + tn) * C::THREADS] = make_float4(a[0], a[1], a[2], a[3]);
      }
    return;
  }
  tail::store_tile<C::TM, C::TN, C::BM, C::BN, C::THREADS>(
      acc, bias, Y, N, m0, n0, M, N, wr, wc, lane, tid,
      [&](int row) {
        const int g = row / C::OUT_ROWS;
        uint8_t* b = g == 0 ? ring0 : g == 1 ? ring1 : (NR == 3 || g == 2) ? ring2 : ring3;
        return reinterpret_cast<uint16_t*>(b) + (row - g * C::OUT_ROWS) * C::BN;
      },
      act);
}

template <class C>
int tiles_of(int rows, int cols) {
  return ((rows + C::BM - 1) / C::BM) * ((cols + C::BN - 1) / C::BN);
}

// Fixup of the remainder split (tail::split_fixup); the accumulators are the sums.
template <class C>
__global__ __launch_bounds__(64 * C::TM * C::WN) void mxfp4_fixup_kernel(
    const float* __restrict__ part, int full, int splits, const float* __restrict__ T,
    int t_slices, long t_stride, int r, const uint16_t* __restrict__ L2,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int N, int act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  tail::split_fixup<C::TM, C::TN, C::WM, C::WN, C::BM, C::BN, C::THREADS>(
      part, full, splits, 1.0f, T, t_slices, t_stride, r, L2, bias, Y, N, 0, M, 0, N, act, lds);
}

// Remainder split, as for the int4 GEMM: only for tiles that fill a CU (a wave
// of workgroups is `cus * WPE` tiles), only when the last wave is at most a
// quarter full (then up to 8 K-shares per tile fit in one wave), and only for
// K of at least kMinSplitSteps steps.
struct MxSplit {
  int full = 0, rem = 0, splits = 1;
  size_t part_bytes = 0;
};

// The remainder split pays only where a share still runs enough steps to
// cover the round trip of its fp32 partials and the fixup pass.  Measured
// with a 4608 x K -> 3072 GEMM (rem = 32 of 288 tiles): at K = 4608 and 6144
// (36 and 48 steps) the 128 x 192 tile without a split was 8 and 3.5 us
// faster than 8 shares; at K = 8192 (64 steps) the split was 4 us faster; at
// K = 12288 20 us.
constexpr int kMinSplitSteps = 56;

template <class C>
MxSplit plan_split(int M, int N, int K) {
  MxSplit p;
  const int tiles = tiles_of<C>(M, N);
  const int cus = device_cu_count() * C::WPE;
  const int ksteps = K / KS;
  p.full = tiles;
  const int rem = tiles % cus;
  if (C::BM * C::BN * C::WPE < MxBig::BM * MxBig::BN || tiles < cus || rem == 0 || 4 * rem > cus ||
      ksteps < kMinSplitSteps)
    return p;
  const int splits = std::min(std::min(kMaxSplits, cus / rem), ksteps);
  if (splits < 2) return p;
  p.full = tiles - rem;
  p.rem = rem;
  p.splits = splits;
  p.part_bytes = (size_t)rem * splits * C::BM * C::BN * sizeof(float);
  return p;
}

template <class C>
hipError_t launch(const uint8_t* qx, const uint8_t* sx, int sx_rows, const float* T, int t_slices,
                  int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                  const uint8_t* sw, const uint16_t* bias, uint16_t* Y, float* part, int act,
                  hipStream_t stream) {
  const MxSplit p = plan_split<C>(M, N, K);
  hipLaunchKernelGGL((mxfp4_gemm_kernel<C, kWhole>), dim3(p.full), dim3(C::THREADS), 0, stream, qx,
                     sx, sx_rows, T, t_slices, (long)M * r, M, K, N, r, L2, Wq, sw, bias, Y, act,
                     p.full, p.rem, p.splits, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.rem == 0) return e;
  hipLaunchKernelGGL((mxfp4_gemm_kernel<C, kShares>), dim3(p.rem * p.splits), dim3(C::THREADS), 0,
                     stream, qx, sx, sx_rows, T, t_slices, (long)M * r, M, K, N, r, L2, Wq, sw,
                     bias, Y, act, p.full, p.rem, p.splits, part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((mxfp4_fixup_kernel<C>), dim3(p.rem * C::WM), dim3(64 * C::TM * C::WN),
                     16 * C::TM * C::BN * 2, stream, part, p.full, p.splits, T, t_slices,
                     (long)M * r, r, L2, bias, Y, M, N, act);
  return hipGetLastError();
}

// Tile choice: the biggest tile that still gives every CU at least one
// workgroup.  256 x 192 tiles are kept where they fill whole waves or leave a
// last wave at most a quarter full that the remainder split finishes (K of at
// least kMinSplitSteps steps); otherwise the 128 x 192 tile with two
// workgroups per CU takes over (at K = 3072 with 32 remainder tiles: 52 us
// against 66 us with the split):
// finer granularity, and one workgroup's waits run under the other's MFMAs
// (measured 9-10 % faster on the 4608-token QKV and up projections, 12 %
// slower than the split on the down projection).
int pick_tile(int M, int N, int K) {
  const int cus = device_cu_count();
  const int big = tiles_of<MxBig>(M, N);
  if (big >= cus) {
    const int rem = big % cus;
    return rem == 0 || (4 * rem <= cus && K / KS >= kMinSplitSteps) ? 2 : 3;
  }
  if (tiles_of<MxMed>(M, N) >= cus) return 1;
  return 0;
}

MxSplit plan_forward(int M, int N, int K) {
  switch (pick_tile(M, N, K)) {
    case 3: return plan_split<MxBig2>(M, N, K);
    case 2: return plan_split<MxBig>(M, N, K);
    case 1: return plan_split<MxMed>(M, N, K);
    default: return plan_split<MxSmall>(M, N, K);
  }
}

}  // namespace

size_t mxfp4_gemm_split_bytes(int M, int K, int N) { return plan_forward(M, N, K).part_bytes; }

hipError_t launch_mxfp4_gemm(const uint8_t* qx, const uint8_t* sx_e8m0, int sx_rows, const float* T,
                             int t_slices, int M, int K, int N, int r, const uint16_t* L2,
                             const uint8_t* Wq, const uint8_t* w_e8m0, const uint16_t* bias,
                             uint16_t* Y, float* part, int act, hipStream_t stream) {
  switch (pick_tile(M, N, K)) {
    case 3:
      return launch<MxBig2>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias, Y,
                            part, act, stream);
    case 2:
      return launch<MxBig>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias, Y,
                           part, act, stream);
    case 1:
      return launch<MxMed>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias, Y,
                           part, act, stream);
    default:
      return launch<MxSmall>(qx, sx_e8m0, sx_rows, T, t_slices, M, K, N, r, L2, Wq, w_e8m0, bias,
                             Y, part, act, stream);
  }
}

}  // namespace svdq
