// Calibration statistic on the GPU: the per-channel absolute maximum of the
// activations, A_scale of the smoothing factor (Terminology Entry, section 2.3,
// equation E2 and the definition of A_scale beneath it).
//
//   amax[k] = max(amax[k], max_m |X[m,k]|)        X bf16 [M, K]
//
// A max is exact and independent of order, so the result is bit-identical to
// any sequential evaluation.  For values >= +0 the IEEE bit patterns order like
// the unsigned integers they are, so |x| is the bf16 pattern with its sign
// cleared, widened to float32 bits, and partial results meet in amax through
// an unsigned atomic max.
//
// HBM-bound: every byte of X is read once.  A wave covers 512 consecutive
// channels of a row (16 bytes per lane, whole 64-byte segments per four lanes),
// the 4 waves of a workgroup take every fourth row of the workgroup's row band,
// with four rows in flight per wave; the waves' maxima meet in LDS and each
// channel of the band leaves as one atomic.
#include "svdq_internal.h"

namespace svdq {
namespace {

constexpr int kAbsThreads = 256;
constexpr int kAbsCols = 512;          // channels per workgroup: 64 lanes x 8
constexpr int kAbsRowsInFlight = 4;

__device__ inline uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// VEC: K % 8 == 0 and X 16-byte aligned, so a lane's 8 channels are one
// aligned 16-byte load; otherwise each channel is loaded on its own.
template <bool VEC>
__global__ __launch_bounds__(kAbsThreads) void act_absmax_kernel(const uint16_t* __restrict__ X,
                                                                 int64_t M, int K,
                                                                 int64_t rows_per_block,
                                                                 uint32_t* __restrict__ amax) {
  __shared__ uint32_t red[kAbsThreads / 64][kAbsCols];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kAbsCols + 8 * lane;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < M ? r0 + rows_per_block : M;
  uint32_t mx[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};   // |x| as bf16 patterns

  if (VEC) {
    if (c0 < K) {
      const uint16_t* base = X + c0;
      int64_t m = r0 + wave;
      // four rows in flight per wave, then the ragged rest one at a time
      for (; m + (kAbsRowsInFlight - 1) * 4 < r1; m += 4 * kAbsRowsInFlight) {
        uint4 v[kAbsRowsInFlight];
#pragma unroll
        for (int j = 0; j < kAbsRowsInFlight; ++j)
          v[j] = *reinterpret_cast<const uint4*>(base + (m + 4 * j) * (int64_t)K);
#pragma unroll
        for (int j = 0; j < kAbsRowsInFlight; ++j) {
          const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            mx[2 * i] = umax(mx[2 * i], w[i] & 0x7FFFu);
            mx[2 * i + 1] = umax(mx[2 * i + 1], (w[i] >> 16) & 0x7FFFu);
          }
        }
      }
      for (; m < r1; m += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(base + m * (int64_t)K);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          mx[2 * i] = umax(mx[2 * i], w[i] & 0x7FFFu);
          mx[2 * i + 1] = umax(mx[2 * i + 1], (w[i] >> 16) & 0x7FFFu);
        }
      }
    }
  } else {
    for (int64_t m = r0 + wave; m < r1; m += 4) {
      const uint16_t* row = X + m * (int64_t)K;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c0 + i < K) mx[i] = umax(mx[i], (uint32_t)row[c0 + i] & 0x7FFFu);
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) red[wave][8 * lane + i] = mx[i];
  __syncthreads();
  for (int c = threadIdx.x; c < kAbsCols; c += kAbsThreads) {
    uint32_t v = red[0][c];
#pragma unroll
    for (int w = 1; w < kAbsThreads / 64; ++w) v = umax(v, red[w][c]);
    const int col = blockIdx.x * kAbsCols + c;
    if (col < K && v != 0u) atomicMax(amax + col, v << 16);
  }
}

}  // namespace

hipError_t launch_act_absmax(const uint16_t* X, int64_t M, int K, float* amax, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int cb = (K + kAbsCols - 1) / kAbsCols;
  // about 2048 workgroups over the chip, at least 16 rows each (4 per wave)
  int64_t rpb = (M * cb + 2047) / 2048;
  rpb = rpb < 16 ? 16 : (rpb + 15) / 16 * 16;
  int64_t rb = (M + rpb - 1) / rpb;
  if (rb > 65535) {   // grid.y limit: wider bands
    rpb = (M + 65534) / 65535;
    rpb = (rpb + 15) / 16 * 16;
    rb = (M + rpb - 1) / rpb;
  }
  const bool vec = K % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
  uint32_t* out = reinterpret_cast<uint32_t*>(amax);
  if (vec)
    hipLaunchKernelGGL(act_absmax_kernel<true>, dim3(cb, (unsigned)rb), dim3(kAbsThreads), 0, stream,
                       X, M, K, rpb, out);
  else
    hipLaunchKernelGGL(act_absmax_kernel<false>, dim3(cb, (unsigned)rb), dim3(kAbsThreads), 0, stream,
                       X, M, K, rpb, out);
  return hipGetLastError();
}

}  // namespace svdq
