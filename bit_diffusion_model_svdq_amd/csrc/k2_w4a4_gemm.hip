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
// byte land in different registers -- a channel permutation that A and B
// share, which leaves each group's dot product unchanged.
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
// Low-rank branch.  acc is the accumulator input of bf16 MFMAs that add
// T L2^T, with T split into a bf16 hi/lo pair (T keeps ~16 significant bits).
//
// Tiling: 128x128 outputs per workgroup, 4 waves of 64x64 (4x4 MFMA tiles),
// 4 groups (128 bytes of codes per row) per pipeline stage, double-buffered
// LDS with an XOR swizzle of 8-byte chunks so that the 16 rows a fragment
// read touches fall in distinct banks.  Workgroups are remapped so that each
// XCD (workgroups are dealt round-robin to the 8 XCDs) works on one compact
// block of tiles, which keeps its share of qx and Wq in its own L2.
#include "svdq_internal.h"

namespace svdq {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int GPS = 4;             // groups per stage
constexpr int ROWB = GPS * 32;     // code bytes per row per stage
constexpr int kThreads = 256;
constexpr int kMagicBits = 0x4B400000;  // 1.5 * 2^23
constexpr float kMagic = 12582912.0f;

struct Smem {
  uint8_t a[2][BM * ROWB];
  uint8_t b[2][BN * ROWB];
  float sx[2][GPS][BM];
  float2 sw[2][GPS][BN];
};

__device__ inline int swz(int row, int chunk) {  // byte offset of 8-byte chunk in a stage row
  return row * ROWB + ((chunk ^ (row & 15)) << 3);
}

__device__ inline i32x4 widen(uint2 v) {  // 16 nibbles -> 16 int8 of value 16 q
  i32x4 r;
  r[0] = (int)((v.x << 4) & 0xF0F0F0F0u);
  r[1] = (int)((v.y << 4) & 0xF0F0F0F0u);
  r[2] = (int)(v.x & 0xF0F0F0F0u);
  r[3] = (int)(v.y & 0xF0F0F0F0u);
  return r;
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Tile coordinates of this workgroup: XCD-compact, then grouped by 8 row tiles.
__device__ inline void tile_of_block(int ntm, int ntn, int& tm, int& tn) {
  const int total = ntm * ntn;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
  constexpr int GROUP_M = 8;
  const int per_group = GROUP_M * ntn;
  const int grp = id / per_group;
  const int first = grp * GROUP_M;
  const int gsize = min(ntm - first, GROUP_M);
  const int in = id - grp * per_group;
  tm = first + in % gsize;
  tn = in / gsize;
}

// EXPORT = false: the forward.  EXPORT = true: write the group partials P of
// rows [row0, row1) x columns [col0, col1) instead of the epilogue.
template <bool EXPORT>
__global__ __launch_bounds__(kThreads, 2) void w4a4_gemm_kernel(
    const uint8_t* __restrict__ qx, const float* __restrict__ sx, const float* __restrict__ T,
    int K, int r, const uint16_t* __restrict__ L2, const uint8_t* __restrict__ Wq,
    const float* __restrict__ w_scales, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ Y, int ldy, int row0, int row1, int col0, int col1,
    int32_t* __restrict__ P) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = K / kGroup;
  const int KB = K / 2;
  const int ntm = (row1 - row0 + BM - 1) / BM;
  const int ntn = (col1 - col0 + BN - 1) / BN;
  int tm, tn;
  tile_of_block(ntm, ntn, tm, tn);
  const int m0 = row0 + tm * BM;
  const int n0 = col0 + tn * BN;
  const int stages = (G + GPS - 1) / GPS;

  // ---- global -> register staging assignment
  const int ld_row = tid >> 3;      // + 32 i
  const int ld_q = tid & 7;         // 16-byte chunk within the stage row
  uint4 ra[4], rb[4];
  float rs[GPS];

  auto gload = [&](int s) {
    const int gv = min(GPS, G - s * GPS);
    const bool q_ok = (ld_q >> 1) < gv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = ld_row + 32 * i;
      const int m = m0 + rr, n = n0 + rr;
      ra[i] = (q_ok && m < row1)
                  ? *reinterpret_cast<const uint4*>(qx + (size_t)m * KB + s * ROWB + ld_q * 16)
                  : make_uint4(0u, 0u, 0u, 0u);
      rb[i] = (q_ok && n < col1)
                  ? *reinterpret_cast<const uint4*>(Wq + (size_t)n * KB + s * ROWB + ld_q * 16)
                  : make_uint4(0u, 0u, 0u, 0u);
    }
    if (!EXPORT) {
      const int rr = tid & 127;
      if (tid < 128) {
        const int m = m0 + rr;
#pragma unroll
        for (int j = 0; j < GPS; ++j)
          rs[j] = (j < gv && m < row1) ? sx[(size_t)m * G + s * GPS + j] : 0.f;
      } else {
        const int n = n0 + rr;
#pragma unroll
        for (int j = 0; j < GPS; ++j)
          rs[j] = (j < gv && n < col1) ? w_scales[(size_t)n * G + s * GPS + j] : 0.f;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = ld_row + 32 * i;
      *reinterpret_cast<uint2*>(&sm.a[buf][swz(rr, 2 * ld_q)]) = make_uint2(ra[i].x, ra[i].y);
      *reinterpret_cast<uint2*>(&sm.a[buf][swz(rr, 2 * ld_q + 1)]) = make_uint2(ra[i].z, ra[i].w);
      *reinterpret_cast<uint2*>(&sm.b[buf][swz(rr, 2 * ld_q)]) = make_uint2(rb[i].x, rb[i].y);
      *reinterpret_cast<uint2*>(&sm.b[buf][swz(rr, 2 * ld_q + 1)]) = make_uint2(rb[i].z, rb[i].w);
    }
    if (!EXPORT) {
      const int rr = tid & 127;
      if (tid < 128) {
#pragma unroll
        for (int j = 0; j < GPS; ++j) sm.sx[buf][j][rr] = rs[j];
      } else {
#pragma unroll
        for (int j = 0; j < GPS; ++j) sm.sw[buf][j][rr] = make_float2(rs[j], -kMagic * rs[j]);
      }
    }
  };

  // ---- per-wave output tile
  const int wr = (wave >> 1) * 64;
  const int wc = (wave & 1) * 64;
  const int fr = lane & 15;   // fragment row / column
  const int fk = lane >> 4;   // fragment k slot
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x4 cmagic = {kMagicBits, kMagicBits, kMagicBits, kMagicBits};

  gload(0);
  sstore(0);
  __syncthreads();

  for (int s = 0; s < stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < stages) gload(s + 1);
    const int gv = min(GPS, G - s * GPS);
    for (int g = 0; g < gv; ++g) {
      i32x4 af[4], bfr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ar = wr + 16 * t + fr;
        af[t] = widen(*reinterpret_cast<const uint2*>(&sm.a[buf][swz(ar, 4 * g + fk)]));
        const int br = wc + 16 * t + fr;
        bfr[t] = widen(*reinterpret_cast<const uint2*>(&sm.b[buf][swz(br, 4 * g + fk)]));
      }
      if (EXPORT) {
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int tj = 0; tj < 4; ++tj) {
            const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[ti], bfr[tj], cmagic, 0, 0, 0);
            const int n = n0 + wc + 16 * tj + fr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = m0 + wr + 16 * ti + 4 * fk + i;
              if (m < row1 && n < col1)
                P[((size_t)(m - row0) * (col1 - col0) + (n - col0)) * G + s * GPS + g] =
                    (d[i] - kMagicBits) >> 8;
            }
          }
      } else {
        f32x4 sxv[4];
        float2 swv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          sxv[t] = *reinterpret_cast<const f32x4*>(&sm.sx[buf][g][wr + 16 * t + 4 * fk]);
          swv[t] = sm.sw[buf][g][wc + 16 * t + fr];
        }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int tj = 0; tj < 4; ++tj) {
            const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[ti], bfr[tj], cmagic, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float t = __builtin_fmaf(__int_as_float(d[i]), swv[tj].x, swv[tj].y);
              acc[ti][tj][i] = __builtin_fmaf(t, sxv[ti][i], acc[ti][tj][i]);
            }
          }
      }
    }
    if (s + 1 < stages) sstore(buf ^ 1);
    __syncthreads();
  }

  if (EXPORT) return;

  // ---- epilogue: 1/256, + T L2^T (bf16 hi/lo MFMA), + bias, bf16 store
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[ti][tj][i] *= (1.0f / 256.0f);

  for (int j0 = 0; j0 < r; j0 += 32) {
    const int j = j0 + 8 * fk;
    const bool j_ok = j < r;
    bf16x8 thi[4], tlo[4], lf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = m0 + wr + 16 * t + fr;
      float tv[8];
      if (j_ok && m < row1) {
        const float4* tp = reinterpret_cast<const float4*>(T + (size_t)m * r + j);
        const float4 a = tp[0], b = tp[1];
        tv[0] = a.x; tv[1] = a.y; tv[2] = a.z; tv[3] = a.w;
        tv[4] = b.x; tv[5] = b.y; tv[6] = b.z; tv[7] = b.w;
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
      const int n = n0 + wc + 16 * t + fr;
      lf[t] = (j_ok && n < col1)
                  ? as_bf16x8(*reinterpret_cast<const uint4*>(L2 + (size_t)n * r + j))
                  : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int tj = 0; tj < 4; ++tj) {
        acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(thi[ti], lf[tj], acc[ti][tj], 0, 0, 0);
        acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tlo[ti], lf[tj], acc[ti][tj], 0, 0, 0);
      }
  }

#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    const int n = n0 + wc + 16 * tj + fr;
    if (n >= col1) continue;
    const float bv = bias ? __uint_as_float(uint32_t(bias[n]) << 16) : 0.f;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wr + 16 * ti + 4 * fk + i;
        if (m < row1) Y[(size_t)m * ldy + n] = f32_to_bf16_rne(acc[ti][tj][i] + bv);
      }
  }
}

}  // namespace

hipError_t launch_w4a4_gemm(const uint8_t* qx, const float* sx, const float* T, int M, int K,
                            int N, int r, const uint16_t* L2, const uint8_t* Wq,
                            const float* w_scales, const uint16_t* bias, uint16_t* Y,
                            hipStream_t stream) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL(w4a4_gemm_kernel<false>, dim3(tiles), dim3(kThreads), 0, stream, qx, sx, T,
                     K, r, L2, Wq, w_scales, bias, Y, N, 0, M, 0, N, nullptr);
  return hipGetLastError();
}

hipError_t launch_group_partials(const uint8_t* qx, const uint8_t* Wq, int M, int N, int K,
                                 int m0, int m1, int n0, int n1, int32_t* P, hipStream_t stream) {
  (void)M;
  (void)N;
  const int tiles = ((m1 - m0 + BM - 1) / BM) * ((n1 - n0 + BN - 1) / BN);
  hipLaunchKernelGGL(w4a4_gemm_kernel<true>, dim3(tiles), dim3(kThreads), 0, stream, qx, nullptr,
                     nullptr, K, 0, nullptr, Wq, nullptr, nullptr, nullptr, 0, m0, m1, n0, n1, P);
  return hipGetLastError();
}

}  // namespace svdq
