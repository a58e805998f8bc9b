// C ABI entry points for the device side: argument validation, workspace
// carving, kernel dispatch.  Host-side packing lives in pack.cpp.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "svdq_internal.h"

namespace svdq {

static thread_local char g_err[512] = "";

svdq_status fail(svdq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

svdq_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return SVDQ_OK;
  return fail(SVDQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int device_cu_count() {
  static std::atomic<int> cached[64];   // zero-initialized: 0 = not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WorkspaceLayout workspace_layout(int M, int K, int N, int r) {
  WorkspaceLayout l;
  const size_t qx_bytes = align256((size_t)M * (K / 2));
  const size_t sx_bytes = align256((size_t)M * (K / kGroup) * 4);
  l.t_slices = k1_plan(M, K, r, false).slices;
  const size_t t_bytes = align256((size_t)l.t_slices * M * r * 4);
  const size_t part_bytes = N > 0 ? align256(gemm_split_bytes(M, K, N)) : 0;
  l.qx = 0;
  l.sx = qx_bytes;
  l.T = qx_bytes + sx_bytes;
  l.part = part_bytes ? qx_bytes + sx_bytes + t_bytes : 0;
  l.bytes = qx_bytes + sx_bytes + t_bytes + part_bytes;
  return l;
}

Workspace carve_workspace(void* base, int M, int K, int N, int r) {
  const WorkspaceLayout l = workspace_layout(M, K, N, r);
  uint8_t* p = static_cast<uint8_t*>(base);
  Workspace w;
  w.qx = p + l.qx;
  w.sx = reinterpret_cast<float*>(p + l.sx);
  w.T = r > 0 ? reinterpret_cast<float*>(p + l.T) : nullptr;
  w.t_slices = l.t_slices;
  w.part = l.part ? reinterpret_cast<float*>(p + l.part) : nullptr;
  w.bytes = l.bytes;
  return w;
}

// MXFP4 workspace: qx [M, K/2] | sx k-tiled E8M0 bytes [ceil(K/256)][sx_rows][8]
// | T [slices, M, r].
WorkspaceLayout workspace_layout_mx(int M, int K, int N, int r) {
  WorkspaceLayout l;
  l.sx_rows = (M + 1) & ~1;
  const size_t qx_bytes = align256((size_t)M * (K / 2));
  const size_t sx_bytes = align256((size_t)((K + 255) / 256) * l.sx_rows * 8);
  l.t_slices = k1_plan(M, K, r, false).slices;
  const size_t t_bytes = align256((size_t)l.t_slices * M * r * 4);
  const size_t part_bytes = N > 0 ? align256(mxfp4_gemm_split_bytes(M, K, N)) : 0;
  l.qx = 0;
  l.sx = qx_bytes;
  l.T = qx_bytes + sx_bytes;
  l.part = part_bytes ? qx_bytes + sx_bytes + t_bytes : 0;
  l.bytes = qx_bytes + sx_bytes + t_bytes + part_bytes;
  return l;
}

MxWorkspace carve_workspace_mx(void* base, int M, int K, int N, int r) {
  const WorkspaceLayout l = workspace_layout_mx(M, K, N, r);
  uint8_t* p = static_cast<uint8_t*>(base);
  MxWorkspace w;
  w.sx_rows = l.sx_rows;
  w.qx = p + l.qx;
  w.sx = p + l.sx;
  w.T = r > 0 ? reinterpret_cast<float*>(p + l.T) : nullptr;
  w.t_slices = l.t_slices;
  w.part = l.part ? reinterpret_cast<float*>(p + l.part) : nullptr;
  w.bytes = l.bytes;
  return w;
}

}  // namespace svdq

using namespace svdq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The largest K a one-slice quantize launch stages in LDS (a multiple of 128,
// so it holds for MXFP4 too); include/svdq.h states the same bound.
constexpr int kMaxCanonicalK = 12544;

svdq_status check_shapes(int M, int K, int N, int r, bool need_n) {
  if (M < 1) return fail(SVDQ_ERR_INVALID_ARG, "M must be >= 1 (got %d)", M);
  if (K < kGroup || K % kGroup != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 64 (got %d)", K);
  if (need_n && (N < 16 || N % 16 != 0))
    return fail(SVDQ_ERR_INVALID_ARG, "N must be a positive multiple of 16 (got %d)", N);
  if (r < 0 || r > kMaxRank || r % 16 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "rank must be a multiple of 16 in [0, 128] (got %d)", r);
  return SVDQ_OK;
}

// MXFP4: the block-scaled MFMA takes 128 channels per step
svdq_status check_shapes_mx(int M, int K, int N, int r) {
  if (K < 128 || K % 128 != 0)
    return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 128 for MXFP4 (got %d)", K);
  return check_shapes(M, K, N, r, true);
}

svdq_status check_ptr(const void* p, const char* name, bool may_be_null) {
  if (!p) {
    if (may_be_null) return SVDQ_OK;
    return fail(SVDQ_ERR_INVALID_ARG, "%s must not be NULL", name);
  }
  if (!aligned16(p)) return fail(SVDQ_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  return SVDQ_OK;
}

#define SVDQ_TRY(expr)                   \
  do {                                   \
    const svdq_status st_ = (expr);      \
    if (st_ != SVDQ_OK) return st_;      \
  } while (0)

svdq_status stage1_checks(const uint16_t* X, int M, int K, int r, const float* smooth,
                          const uint16_t* L1) {
  SVDQ_TRY(check_ptr(X, "X", false));
  SVDQ_TRY(check_ptr(smooth, "smooth", false));
  SVDQ_TRY(check_ptr(L1, "L1", r == 0));
  (void)M;
  (void)K;
  return SVDQ_OK;
}

svdq_status stage2_checks(int r, const uint16_t* L2, const uint8_t* Wq, const float* w_scales,
                          const uint16_t* bias, const uint16_t* Y) {
  SVDQ_TRY(check_ptr(L2, "L2", r == 0));
  SVDQ_TRY(check_ptr(Wq, "Wq", false));
  SVDQ_TRY(check_ptr(w_scales, "w_scales", false));
  SVDQ_TRY(check_ptr(bias, "bias", true));
  SVDQ_TRY(check_ptr(Y, "Y", false));
  return SVDQ_OK;
}

template <class F>
svdq_status guarded(F&& f) {
  try {
    return f();
  } catch (...) {
    return fail(SVDQ_ERR_INVALID_ARG, "unexpected C++ exception");
  }
}

svdq_status check_act(int act) {
  if (act != kActNone && act != kActGeluTanh)
    return fail(SVDQ_ERR_INVALID_ARG, "activation %d is not one of svdq_activation", act);
  return SVDQ_OK;
}

svdq_status forward_gemm(int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                         const float* w_scales, const uint16_t* bias, int act, uint16_t* Y,
                         const void* workspace, size_t workspace_bytes, void* stream) {
  SVDQ_TRY(check_shapes(M, K, N, r, true));
  SVDQ_TRY(stage2_checks(r, L2, Wq, w_scales, bias, Y));
  SVDQ_TRY(check_act(act));
  SVDQ_TRY(check_ptr(workspace, "workspace", false));
  const Workspace w = carve_workspace(const_cast<void*>(workspace), M, K, N, r);
  if (workspace_bytes < w.bytes)
    return fail(SVDQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, workspace_bytes);
  return hip_check(launch_w4a4_gemm(w.qx, w.sx, w.T, w.t_slices, M, K, N, r, L2, Wq, w_scales,
                                    bias, Y, w.part, act, static_cast<hipStream_t>(stream)),
                   "w4a4_gemm launch");
}

svdq_status linear_forward(const uint16_t* X, int M, int K, int N, int r, const float* smooth,
                           const uint16_t* L1, const uint16_t* L2, const uint8_t* Wq,
                           const float* w_scales, const uint16_t* bias, int act, uint16_t* Y,
                           void* workspace, size_t workspace_bytes, void* stream) {
  // validate everything before launching anything
  SVDQ_TRY(check_shapes(M, K, N, r, true));
  SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
  SVDQ_TRY(stage2_checks(r, L2, Wq, w_scales, bias, Y));
  SVDQ_TRY(check_act(act));
  SVDQ_TRY(check_ptr(workspace, "workspace", false));
  const Workspace w = carve_workspace(workspace, M, K, N, r);
  if (workspace_bytes < w.bytes)
    return fail(SVDQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FusedPlan fp = fused_plan(M, K, N, r);
  if (fp.use)
    return hip_check(launch_fused_smallk(fp, X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y,
                                         act, nullptr, nullptr, s),
                     "fused small-K forward launch");
  SVDQ_TRY(hip_check(launch_smooth_quant_lora_down(X, M, K, r, smooth, L1, w.qx, w.sx, w.T, false, s),
                     "smooth_quant_lora_down launch"));
  return hip_check(launch_w4a4_gemm(w.qx, w.sx, w.T, w.t_slices, M, K, N, r, L2, Wq, w_scales,
                                    bias, Y, w.part, act, s),
                   "w4a4_gemm launch");
}

svdq_status forward_gemm_mx(int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                            const uint8_t* w_e8m0, const uint16_t* bias, int act, uint16_t* Y,
                            const void* workspace, size_t workspace_bytes, void* stream) {
  SVDQ_TRY(check_shapes_mx(M, K, N, r));
  SVDQ_TRY(stage2_checks(r, L2, Wq, reinterpret_cast<const float*>(w_e8m0), bias, Y));
  SVDQ_TRY(check_act(act));
  SVDQ_TRY(check_ptr(workspace, "workspace", false));
  const MxWorkspace w = carve_workspace_mx(const_cast<void*>(workspace), M, K, N, r);
  if (workspace_bytes < w.bytes)
    return fail(SVDQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, workspace_bytes);
  return hip_check(launch_mxfp4_gemm(w.qx, w.sx, w.sx_rows, w.T, w.t_slices, M, K, N, r, L2, Wq,
                                     w_e8m0, bias, Y, w.part, act, static_cast<hipStream_t>(stream)),
                   "mxfp4_gemm launch");
}

svdq_status linear_forward_mx(const uint16_t* X, int M, int K, int N, int r, const float* smooth,
                              const uint16_t* L1, const uint16_t* L2, const uint8_t* Wq,
                              const uint8_t* w_e8m0, const uint16_t* bias, int act, uint16_t* Y,
                              void* workspace, size_t workspace_bytes, void* stream) {
  SVDQ_TRY(check_shapes_mx(M, K, N, r));
  SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
  SVDQ_TRY(stage2_checks(r, L2, Wq, reinterpret_cast<const float*>(w_e8m0), bias, Y));
  SVDQ_TRY(check_act(act));
  SVDQ_TRY(check_ptr(workspace, "workspace", false));
  const MxWorkspace w = carve_workspace_mx(workspace, M, K, N, r);
  if (workspace_bytes < w.bytes)
    return fail(SVDQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const FusedPlan fp = fused_plan_mx(M, K, N, r);
  if (fp.use)
    return hip_check(launch_fused_smallk_mx(fp, X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y,
                                            act, nullptr, nullptr, s),
                     "fused small-K forward (MXFP4) launch");
  SVDQ_TRY(hip_check(launch_smooth_quant_lora_down_mx(X, M, K, r, smooth, L1, w.qx, w.sx, w.T,
                                                      false, w.sx_rows, s),
                     "smooth_quant_lora_down (MXFP4) launch"));
  return hip_check(launch_mxfp4_gemm(w.qx, w.sx, w.sx_rows, w.T, w.t_slices, M, K, N, r, L2, Wq,
                                     w_e8m0, bias, Y, w.part, act, s),
                   "mxfp4_gemm launch");
}

// ---- the allocation-free forward's workspace
// A file-scope device array serves as the forward's workspace for callers
// that cannot allocate.  Host code never uses the array's name as an address
// (on the host it only names the symbol); the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

svdq_status scratch_for_current_device(void** out) {
  int dev = 0;
  SVDQ_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SVDQ_ERR_UNSUPPORTED, "device %d is beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    SVDQ_TRY(hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!ptr) return fail(SVDQ_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SVDQ_OK;
}

}  // namespace

extern "C" {

size_t svdq_static_workspace_bytes(void) { return kScratchBytes; }

svdq_status svdq_linear_forward_noalloc(const uint16_t* X, int M, int K, int N, int r,
                                        const float* smooth, const uint16_t* L1,
                                        const uint16_t* L2, const uint8_t* Wq,
                                        const float* w_scales, const uint16_t* bias,
                                        int activation, uint16_t* Y, void* stream) {
  return guarded([&]() -> svdq_status {
    // the same checks as the workspace entry point, then the size bound
    SVDQ_TRY(check_shapes(M, K, N, r, true));
    const size_t need = workspace_layout(M, K, N, r).bytes;
    if (need > kScratchBytes)
      return fail(SVDQ_ERR_WORKSPACE,
                  "M=%d K=%d N=%d r=%d needs %zu workspace bytes; the static workspace holds %zu",
                  M, K, N, r, need, kScratchBytes);
    void* ws = nullptr;
    SVDQ_TRY(scratch_for_current_device(&ws));
    return linear_forward(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, activation, Y, ws,
                          kScratchBytes, stream);
  });
}

size_t svdq_forward_workspace_bytes(int M, int K, int N, int r) {
  if (M < 1 || K < kGroup || K % kGroup || N < 16 || N % 16 || r < 0 || r > kMaxRank || r % 16)
    return 0;
  return workspace_layout(M, K, N, r).bytes;
}

svdq_status svdq_forward_workspace_layout(int M, int K, int N, int r, size_t* qx_offset,
                                          size_t* sx_offset, size_t* t_offset, int* t_slices) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes(M, K, N, r, true));
    if (!qx_offset || !sx_offset || !t_offset || !t_slices)
      return fail(SVDQ_ERR_INVALID_ARG, "NULL output pointer");
    const WorkspaceLayout l = workspace_layout(M, K, N, r);
    *qx_offset = l.qx;
    *sx_offset = l.sx;
    *t_offset = r > 0 ? l.T : 0;
    *t_slices = r > 0 ? l.t_slices : 0;
    return SVDQ_OK;
  });
}

svdq_status svdq_forward_workspace_layout_mxfp4(int M, int K, int N, int r, size_t* qx_offset,
                                                size_t* sx_offset, size_t* t_offset, int* t_slices,
                                                int* sx_rows) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes_mx(M, K, N, r));
    if (!qx_offset || !sx_offset || !t_offset || !t_slices || !sx_rows)
      return fail(SVDQ_ERR_INVALID_ARG, "NULL output pointer");
    const WorkspaceLayout l = workspace_layout_mx(M, K, N, r);
    *qx_offset = l.qx;
    *sx_offset = l.sx;
    *t_offset = r > 0 ? l.T : 0;
    *t_slices = r > 0 ? l.t_slices : 0;
    *sx_rows = l.sx_rows;
    return SVDQ_OK;
  });
}

svdq_status svdq_forward_quantize(const uint16_t* X, int M, int K, int r, const float* smooth,
                                  const uint16_t* L1, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes(M, K, 16, r, false));
    SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
    SVDQ_TRY(check_ptr(workspace, "workspace", false));
    const Workspace w = carve_workspace(workspace, M, K, 0, r);   // stage 1 needs no partials
    if (workspace_bytes < w.bytes)
      return fail(SVDQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, workspace_bytes);
    return hip_check(launch_smooth_quant_lora_down(X, M, K, r, smooth, L1, w.qx, w.sx, w.T, false,
                                                   static_cast<hipStream_t>(stream)),
                     "smooth_quant_lora_down launch");
  });
}

svdq_status svdq_forward_gemm(int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                              const float* w_scales, const uint16_t* bias, uint16_t* Y,
                              const void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    return forward_gemm(M, K, N, r, L2, Wq, w_scales, bias, kActNone, Y, workspace,
                        workspace_bytes, stream);
  });
}

svdq_status svdq_forward_gemm_act(int M, int K, int N, int r, const uint16_t* L2,
                                  const uint8_t* Wq, const float* w_scales, const uint16_t* bias,
                                  int activation, uint16_t* Y, const void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    return forward_gemm(M, K, N, r, L2, Wq, w_scales, bias, activation, Y, workspace,
                        workspace_bytes, stream);
  });
}

svdq_status svdq_linear_forward(const uint16_t* X, int M, int K, int N, int r,
                                const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                const uint8_t* Wq, const float* w_scales, const uint16_t* bias,
                                uint16_t* Y, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return guarded([&]() -> svdq_status {
    return linear_forward(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, kActNone, Y,
                          workspace, workspace_bytes, stream);
  });
}

svdq_status svdq_linear_forward_act(const uint16_t* X, int M, int K, int N, int r,
                                    const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                    const uint8_t* Wq, const float* w_scales,
                                    const uint16_t* bias, int activation, uint16_t* Y,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    return linear_forward(X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, activation, Y,
                          workspace, workspace_bytes, stream);
  });
}

svdq_status svdq_quantize_activations(const uint16_t* X, int M, int K, const float* smooth,
                                      const uint16_t* L1, int r, uint8_t* qx, float* sx,
                                      float* T, void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes(M, K, 16, r, false));
    SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
    SVDQ_TRY(check_ptr(qx, "qx", false));
    SVDQ_TRY(check_ptr(sx, "sx", false));
    SVDQ_TRY(check_ptr(T, "T", r == 0));
    if (!k1_one_slice_fits(K, r))
      return fail(SVDQ_ERR_INVALID_ARG,
                  "K=%d: the canonical-layout quantize stages a whole row in LDS and takes K <= %d",
                  K, kMaxCanonicalK);
    return hip_check(launch_smooth_quant_lora_down(X, M, K, r, smooth, L1, qx, sx, T, true,
                                                   static_cast<hipStream_t>(stream)),
                     "smooth_quant_lora_down launch");
  });
}

svdq_status svdq_act_absmax_update_device(const uint16_t* X, int64_t M, int K, float* amax,
                                          void* stream) {
  return guarded([&]() -> svdq_status {
    if (M < 0 || K < 1)
      return fail(SVDQ_ERR_INVALID_ARG, "bad shape M=%lld K=%d", (long long)M, K);
    if (!amax || (M > 0 && !X)) return fail(SVDQ_ERR_INVALID_ARG, "NULL buffer");
    if ((reinterpret_cast<uintptr_t>(X) & 1) || (reinterpret_cast<uintptr_t>(amax) & 3))
      return fail(SVDQ_ERR_ALIGNMENT, "X must be 2-byte and amax 4-byte aligned");
    return hip_check(launch_act_absmax(X, M, K, amax, static_cast<hipStream_t>(stream)),
                     "act_absmax launch");
  });
}

svdq_status svdq_debug_group_partials(const uint8_t* qx, const uint8_t* Wq, int M, int N, int K,
                                      int m0, int m1, int n0, int n1, int32_t* P, void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes(M, K, N, 0, true));
    if (m0 < 0 || m1 > M || m0 >= m1 || n0 < 0 || n1 > N || n0 >= n1)
      return fail(SVDQ_ERR_INVALID_ARG, "block [%d,%d)x[%d,%d) outside [0,%d)x[0,%d)", m0, m1, n0,
                  n1, M, N);
    SVDQ_TRY(check_ptr(qx, "qx", false));
    SVDQ_TRY(check_ptr(Wq, "Wq", false));
    SVDQ_TRY(check_ptr(P, "P", false));
    return hip_check(
        launch_group_partials(qx, Wq, M, N, K, m0, m1, n0, n1, P, static_cast<hipStream_t>(stream)),
        "group_partials launch");
  });
}

int svdq_forward_fused(int M, int K, int N, int r) {
  if (M < 1 || K < kGroup || K % kGroup || N < 16 || N % 16 || r < 0 || r > kMaxRank || r % 16)
    return 0;
  return fused_plan(M, K, N, r).use ? 1 : 0;
}

svdq_status svdq_debug_fused_forward(const uint16_t* X, int M, int K, int N, int r,
                                     const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                     const uint8_t* Wq, const float* w_scales,
                                     const uint16_t* bias, int activation, uint16_t* Y,
                                     uint8_t* qx, float* sx, void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes(M, K, N, r, true));
    SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
    SVDQ_TRY(stage2_checks(r, L2, Wq, w_scales, bias, Y));
    SVDQ_TRY(check_act(activation));
    SVDQ_TRY(check_ptr(qx, "qx", false));
    SVDQ_TRY(check_ptr(sx, "sx", false));
    const FusedPlan fp = fused_plan(M, K, N, r);
    if (!fp.use)
      return fail(SVDQ_ERR_INVALID_ARG, "M=%d K=%d N=%d r=%d does not take the fused small-K path", M, K,
                  N, r);
    return hip_check(launch_fused_smallk(fp, X, M, K, N, r, smooth, L1, L2, Wq, w_scales, bias, Y,
                                         activation, qx, sx, static_cast<hipStream_t>(stream)),
                     "fused small-K forward launch");
  });
}

int svdq_forward_fused_mxfp4(int M, int K, int N, int r) {
  if (M < 1 || K < 128 || K % 128 || N < 16 || N % 16 || r < 0 || r > kMaxRank || r % 16) return 0;
  return fused_plan_mx(M, K, N, r).use ? 1 : 0;
}

svdq_status svdq_debug_fused_forward_mxfp4(const uint16_t* X, int M, int K, int N, int r,
                                           const float* smooth, const uint16_t* L1,
                                           const uint16_t* L2, const uint8_t* Wq,
                                           const uint8_t* w_e8m0, const uint16_t* bias,
                                           int activation, uint16_t* Y, uint8_t* qx,
                                           uint8_t* sx_e8m0, void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes_mx(M, K, N, r));
    SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
    SVDQ_TRY(stage2_checks(r, L2, Wq, reinterpret_cast<const float*>(w_e8m0), bias, Y));
    SVDQ_TRY(check_act(activation));
    SVDQ_TRY(check_ptr(qx, "qx", false));
    SVDQ_TRY(check_ptr(sx_e8m0, "sx_e8m0", false));
    const FusedPlan fp = fused_plan_mx(M, K, N, r);
    if (!fp.use)
      return fail(SVDQ_ERR_INVALID_ARG, "M=%d K=%d N=%d r=%d does not take the fused small-K path", M, K,
                  N, r);
    return hip_check(launch_fused_smallk_mx(fp, X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, Y,
                                            activation, qx, sx_e8m0, static_cast<hipStream_t>(stream)),
                     "fused small-K forward (MXFP4) launch");
  });
}

size_t svdq_forward_workspace_bytes_mxfp4(int M, int K, int N, int r) {
  if (M < 1 || K < 128 || K % 128 || N < 16 || N % 16 || r < 0 || r > kMaxRank || r % 16) return 0;
  return workspace_layout_mx(M, K, N, r).bytes;
}

svdq_status svdq_forward_quantize_mxfp4(const uint16_t* X, int M, int K, int r,
                                        const float* smooth, const uint16_t* L1, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes_mx(M, K, 16, r));
    SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
    SVDQ_TRY(check_ptr(workspace, "workspace", false));
    const MxWorkspace w = carve_workspace_mx(workspace, M, K, 0, r);   // stage 1 needs no partials
    if (workspace_bytes < w.bytes)
      return fail(SVDQ_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", w.bytes, workspace_bytes);
    return hip_check(launch_smooth_quant_lora_down_mx(X, M, K, r, smooth, L1, w.qx, w.sx, w.T,
                                                      false, w.sx_rows,
                                                      static_cast<hipStream_t>(stream)),
                     "smooth_quant_lora_down (MXFP4) launch");
  });
}

svdq_status svdq_forward_gemm_mxfp4(int M, int K, int N, int r, const uint16_t* L2,
                                    const uint8_t* Wq, const uint8_t* w_e8m0,
                                    const uint16_t* bias, uint16_t* Y, const void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    return forward_gemm_mx(M, K, N, r, L2, Wq, w_e8m0, bias, kActNone, Y, workspace,
                           workspace_bytes, stream);
  });
}

svdq_status svdq_forward_gemm_act_mxfp4(int M, int K, int N, int r, const uint16_t* L2,
                                        const uint8_t* Wq, const uint8_t* w_e8m0,
                                        const uint16_t* bias, int activation, uint16_t* Y,
                                        const void* workspace, size_t workspace_bytes,
                                        void* stream) {
  return guarded([&]() -> svdq_status {
    return forward_gemm_mx(M, K, N, r, L2, Wq, w_e8m0, bias, activation, Y, workspace,
                           workspace_bytes, stream);
  });
}

svdq_status svdq_linear_forward_mxfp4(const uint16_t* X, int M, int K, int N, int r,
                                      const float* smooth, const uint16_t* L1,
                                      const uint16_t* L2, const uint8_t* Wq,
                                      const uint8_t* w_e8m0, const uint16_t* bias, uint16_t* Y,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    return linear_forward_mx(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, kActNone, Y,
                             workspace, workspace_bytes, stream);
  });
}

svdq_status svdq_linear_forward_act_mxfp4(const uint16_t* X, int M, int K, int N, int r,
                                          const float* smooth, const uint16_t* L1,
                                          const uint16_t* L2, const uint8_t* Wq,
                                          const uint8_t* w_e8m0, const uint16_t* bias,
                                          int activation, uint16_t* Y, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return guarded([&]() -> svdq_status {
    return linear_forward_mx(X, M, K, N, r, smooth, L1, L2, Wq, w_e8m0, bias, activation, Y,
                             workspace, workspace_bytes, stream);
  });
}

svdq_status svdq_quantize_activations_mxfp4(const uint16_t* X, int M, int K, const float* smooth,
                                            const uint16_t* L1, int r, uint8_t* qx,
                                            uint8_t* sx_e8m0, float* T, void* stream) {
  return guarded([&]() -> svdq_status {
    SVDQ_TRY(check_shapes_mx(M, K, 16, r));
    SVDQ_TRY(stage1_checks(X, M, K, r, smooth, L1));
    SVDQ_TRY(check_ptr(qx, "qx", false));
    SVDQ_TRY(check_ptr(sx_e8m0, "sx_e8m0", false));
    SVDQ_TRY(check_ptr(T, "T", r == 0));
    if (!k1_one_slice_fits(K, r))
      return fail(SVDQ_ERR_INVALID_ARG,
                  "K=%d: the canonical-layout quantize stages a whole row in LDS and takes K <= %d",
                  K, kMaxCanonicalK);
    return hip_check(launch_smooth_quant_lora_down_mx(X, M, K, r, smooth, L1, qx, sx_e8m0, T, true,
                                                      0, static_cast<hipStream_t>(stream)),
                     "smooth_quant_lora_down (MXFP4) launch");
  });
}

const char* svdq_status_string(svdq_status status) {
  // callers may pass any int (the ABI carries the enum as one): read its bytes
  // as an int, since loading an out-of-range value as the enum type is undefined
  int s;
  memcpy(&s, &status, sizeof(s));
  switch (s) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_INVALID_ARG: return "invalid argument";
    case SVDQ_ERR_UNSUPPORTED: return "unsupported parameter";
    case SVDQ_ERR_ALIGNMENT: return "misaligned pointer";
    case SVDQ_ERR_WORKSPACE: return "workspace too small";
    case SVDQ_ERR_NO_CONVERGENCE: return "eigensolver did not converge";
    case SVDQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* svdq_last_error(void) { return g_err; }

}  // extern "C"
