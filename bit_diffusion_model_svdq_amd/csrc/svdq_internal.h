// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "svdq.h"
#include "svdq_errors.h"

namespace svdq {

constexpr int kGroup = 64;      // quantization group along K
constexpr int kMaxRank = 128;   // rank bound of the low-rank branch

svdq_status hip_check(hipError_t e, const char* what);

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count();

// Byte offsets of the workspace's parts (and its size), computed without a base
// pointer; the MXFP4 layout also fixes the row count of its k-tiled scales.
struct WorkspaceLayout {
  size_t qx = 0, sx = 0, T = 0, part = 0, bytes = 0;
  int t_slices = 1;
  int sx_rows = 0;
};
WorkspaceLayout workspace_layout(int M, int K, int N, int r);
WorkspaceLayout workspace_layout_mx(int M, int K, int N, int r);

// Workspace carving: qx [M, K/2] | sx [M, K/64] | T [slices, M, r] | split partials
// (only when k2 splits a last partial wave of tiles; N = 0 leaves them out),
// each part 256-byte aligned.
struct Workspace {
  uint8_t* qx;
  float* sx;
  float* T;         // t_slices x M x r partial sums of x_hat L1^T
  int t_slices;
  float* part;
  size_t bytes;
};
Workspace carve_workspace(void* base, int M, int K, int N, int r);

// MXFP4 workspace: qx [M, K/2] | sx k-tiled E8M0 bytes [ceil(K/256)][sx_rows][8]
// | T [slices, M, r] | split partials (only when the GEMM splits a last
// partial wave of tiles; N = 0 leaves them out).
struct MxWorkspace {
  uint8_t* qx;
  uint8_t* sx;
  int sx_rows;      // M rounded up to even: 16-byte runs of two rows stay aligned
  float* T;
  int t_slices;
  float* part;
  size_t bytes;
};
MxWorkspace carve_workspace_mx(void* base, int M, int K, int N, int r);

// Bytes of fp32 partial accumulators the MXFP4 GEMM needs for M x N x K.
size_t mxfp4_gemm_split_bytes(int M, int K, int N);

// Bytes of fp32 partial accumulators k2 needs for an M x N x K forward.
size_t gemm_split_bytes(int M, int K, int N);

// k1: x_hat = X * (1/s); per-64 absmax, scales and codes; T = x_hat L1^T.
// The launch shape: rtm row tiles of 16 per workgroup, K cut into `slices`
// slices of gslice groups; each slice writes its own partial T, so T holds
// slices x M x r floats (slice-major).  one_slice asks for a single slice,
// i.e. T itself.
struct K1Plan {
  int rtm = 1, slices = 1, gslice = 1;
};
K1Plan k1_plan(int M, int K, int r, bool one_slice);
// Whether a one-slice launch (a whole row of K channels per workgroup, as the
// canonical-layout entry points use) fits the kernel's LDS budget.
bool k1_one_slice_fits(int K, int r);
hipError_t launch_smooth_quant_lora_down(const uint16_t* X, int M, int K, int r,
                                         const float* smooth, const uint16_t* L1, uint8_t* qx,
                                         float* sx, float* T, bool one_slice, hipStream_t stream);
// The same with MXFP4 codes: qx [M, K/2] E2M1 patterns; E8M0 scale bytes
// row-major sx_e8m0 [M, K/32] (sx_rows = 0) or k-tiled [ceil(K/256)][sx_rows][8]
// (sx_rows >= M, even), the layout the block-scaled GEMM reads.
hipError_t launch_smooth_quant_lora_down_mx(const uint16_t* X, int M, int K, int r,
                                            const float* smooth, const uint16_t* L1, uint8_t* qx,
                                            uint8_t* sx_e8m0, float* T, bool one_slice,
                                            int sx_rows, hipStream_t stream);

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// (lgkmcnt) and leaves its global loads in flight.  __syncthreads also waits
// for those (vmcnt 0), which costs a pipeline that keeps stages in flight in
// registers.  The fences, limited to the local address space, stop the
// compiler from moving LDS accesses across the barrier.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Output activations of the GEMM epilogue (the values of svdq_activation).
constexpr int kActNone = 0;
constexpr int kActGeluTanh = 1;

// k2: Y = act(sum_g sx sw P_g + T L2^T + b), bf16 out.  T holds t_slices
// partial sums of M x r floats, added in order.
hipError_t launch_w4a4_gemm(const uint8_t* qx, const float* sx, const float* T, int t_slices,
                            int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                            const float* w_scales, const uint16_t* bias, uint16_t* Y,
                            float* part, int act, hipStream_t stream);

// k2, MXFP4 variant: Y = act(block-scaled FP4 product + T L2^T + b), bf16 out.
// Both scale operands are k-tiled: sx_e8m0 [ceil(K/256)][sx_rows][8] and
// w_e8m0 [ceil(K/256)][N][8].
hipError_t launch_mxfp4_gemm(const uint8_t* qx, const uint8_t* sx_e8m0, int sx_rows, const float* T,
                             int t_slices, int M, int K, int N, int r, const uint16_t* L2,
                             const uint8_t* Wq, const uint8_t* w_e8m0, const uint16_t* bias,
                             uint16_t* Y, float* part, int act, hipStream_t stream);

// Calibration statistic: amax[k] = max(amax[k], max_m |X[m,k]|) on the GPU
// (unsigned atomic max of float32 bit patterns; amax must hold values >= +0).
hipError_t launch_act_absmax(const uint16_t* X, int64_t M, int K, float* amax, hipStream_t stream);

// The fused small-K forward: quantize, lora_down, the W4A4 GEMM, lora_up, bias
// and activation in one kernel (K <= 1280, r <= 32, N <= 2560, and at most 256
// blocks of 16 x 16 outputs x 64 channels per compute unit).  nt: column
// tiles of 16 per wave (a workgroup covers 128 nt columns of 16 rows).
struct FusedPlan {
  bool use = false;
  int nt = 0;
};
FusedPlan fused_plan(int M, int K, int N, int r);
// dbg_qx / dbg_sx (both NULL, or both set): the codes ([M, K/2] packed) and
// scales ([M, K/64]) the kernel quantized, written by the first column slice.
hipError_t launch_fused_smallk(const FusedPlan& plan, const uint16_t* X, int M, int K, int N, int r,
                               const float* smooth, const uint16_t* L1, const uint16_t* L2,
                               const uint8_t* Wq, const float* w_scales, const uint16_t* bias,
                               uint16_t* Y, int act, uint8_t* dbg_qx, float* dbg_sx,
                               hipStream_t stream);

// The fused small-K forward with MXFP4 (E2M1 codes, E8M0 scales per 32
// channels; w_e8m0 k-tiled): the same range with K a multiple of 128, and up
// to 400 blocks per compute unit where K <= 640.
// dbg_qx / dbg_sx (both NULL, or both set): the codes ([M, K/2] packed) and
// the scale bytes ([M, K/32], row-major), written by the first column slice.
FusedPlan fused_plan_mx(int M, int K, int N, int r);
hipError_t launch_fused_smallk_mx(const FusedPlan& plan, const uint16_t* X, int M, int K, int N, int r,
                                  const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                  const uint8_t* Wq, const uint8_t* w_e8m0, const uint16_t* bias,
                                  uint16_t* Y, int act, uint8_t* dbg_qx, uint8_t* dbg_sx,
                                  hipStream_t stream);

// k2's main loop with the integer group partials exported instead of the epilogue.
hipError_t launch_group_partials(const uint8_t* qx, const uint8_t* Wq, int M, int N, int K,
                                 int m0, int m1, int n0, int n1, int32_t* P, hipStream_t stream);

}  // namespace svdq
