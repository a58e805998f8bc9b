/*
 * svdq.h -- C ABI of the SVDQuant W4A4 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer computes (SVDQuant Terminology Entry, section 2.3, equation E4,
 * with the bias of its right-hand side):
 *
 *     Y = Q(X diag(s)^-1) Q(R)  +  (X diag(s)^-1 L1^T) L2^T  +  b,
 *     R = diag(s) W - (L1^T L2^T)^T   i.e.  R[n,k] = W[n,k] s[k] - sum_j L2[n,j] L1[j,k]
 *
 * where s smooths activation outliers into the weight (E1, E2), L1 and L2 are
 * the rank-r truncated SVD factors of the smoothed weight (E3, E5) kept in
 * bfloat16, and Q is symmetric 4-bit quantization with one float32 scale per
 * 64 consecutive input channels (the SVDQuant abstract fixes 4-bit weights and
 * activations; the group size and scale format are this library's reading).
 *
 * Storage conventions (all row-major, little-endian):
 *   bf16        uint16_t bit patterns of bfloat16
 *   W           float32 [N, K]      out-features x in-features
 *   X           bf16    [M, K]      M tokens
 *   s (smooth)  float32 [K]
 *   L1          bf16    [r, K]      lora_down, row j = v_j^T          (V_r^T)
 *   L2          bf16    [N, r]      lora_up,   row n = (U_r Sigma_r)[n, :]
 *   Wq          uint8   [N, K/2]    two int4 codes per byte, even k in the low nibble
 *   w_scales    float32 [N, K/64]   two lowest significand bits always zero
 *   qx          uint8   [M, K/2]    activation codes, same packing
 *   sx          float32 [M, K/64]   activation scales
 *   T           float32 [M, r]      lora_down output  x_hat L1^T
 *   bias        bf16    [N]         may be NULL (zero bias)
 *   Y           bf16    [M, N]
 * Codes are in [-7, 7]; -8 is never produced.
 *
 * Quantization of one group v[0..63] (float32):
 *   a = max|v|; a < 2^-100 (zero included) -> scale 0, codes 0; else
 *   scale = fl32(a / 7), inv = fl32(7 / a),
 *   code = clamp(round_half_even(fl32(v * inv)), -7, 7).
 *   A weight scale then has its two lowest significand bits cleared.
 * Smoothed activations: x_hat[m,k] = fl32(X[m,k] * fl32(1 / s[k])).
 *
 * Errors: every function returns an svdq_status and never throws or aborts.
 * On a validation error nothing is written.  Device functions launch work
 * asynchronously on the given stream (a hipStream_t; NULL = the null stream)
 * and do not synchronize; SVDQ_ERR_HIP reports a launch failure.  Non-finite
 * inputs are not checked: their results are undefined.  svdq_last_error()
 * returns a thread-local description of the last failure on this thread.
 *
 * Ownership: the caller owns every buffer.  Host functions take host
 * pointers; device functions take device pointers.  The library allocates no
 * device memory; scratch space comes from the caller's workspace.
 */
#ifndef SVDQ_H_
#define SVDQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = 1,    /* a size or pointer argument is out of range */
  SVDQ_ERR_UNSUPPORTED = 2,    /* a parameter the library does not implement (e.g. group != 64) */
  SVDQ_ERR_ALIGNMENT = 3,      /* a device pointer is not 16-byte aligned */
  SVDQ_ERR_WORKSPACE = 4,      /* workspace_bytes below svdq_forward_workspace_bytes() */
  SVDQ_ERR_NO_CONVERGENCE = 5, /* the packer's eigensolver did not converge */
  SVDQ_ERR_HIP = 6             /* a HIP runtime call failed */
} svdq_status;

typedef struct {
  float alpha;  /* migration strength of E2, in [0, 1] */
  int rank;     /* r: 0 <= r <= 128, r % 16 == 0 (the page recommends r <= 128) */
  int group;    /* quantization group along K; must be 64 */
  float s_min;  /* lower bound of s (E2); both statistics are floored at 1e-5 */
} svdq_pack_params;

/* ------------------------------------------------------------------ host */

/* Calibration statistic A_scale of E2 (Terminology Entry, section 2.3: the
 * per-channel absolute maximum of the activations).  Folds M rows of bf16
 * activations X [M, K] into the running maximum amax [K]:
 * amax[k] = max(amax[k], max_m |X[m,k]|).  Start from zeros.  Host memory. */
svdq_status svdq_act_absmax_update(const uint16_t* X, int64_t M, int K, float* amax);

/* Offline packing: the three stages of the Terminology Entry, section 2.1, in
 * order.  (1) s[k] = max(max(A,1e-5)^alpha / max(Wsc,1e-5)^(1-alpha), s_min) in
 * float64, stored float32 (E2), with Wsc[k] = max_n |W[n,k]|.  (2) the rank-r
 * truncated SVD of W_hat = W diag(s) (E3, E5); L1 = bf16(V_r^T),
 * L2 = bf16(U_r Sigma_r), each rounded once from float64; the sign of each
 * singular pair is chosen so that the largest-magnitude entry of v_j is
 * positive.  (3) R = fl32(W_hat - L2 L1) from the rounded factors (the sum
 * over j ascending in float64), quantized per 64-group into Wq and w_scales.
 * Host buffers, sizes as in the storage table; sigma (optional, may be NULL)
 * receives the min(N,K) singular values of W_hat in descending order.  r = 0
 * writes nothing to L1/L2 (they may be NULL).  Requires K % 64 == 0, N >= 1.
 * Returns SVDQ_ERR_NO_CONVERGENCE if the eigensolver fails. */
svdq_status svdq_pack_weights(const float* W, int N, int K, const float* act_absmax,
                              const svdq_pack_params* params, float* smooth, uint16_t* L1,
                              uint16_t* L2, uint8_t* Wq, float* w_scales, double* sigma);

/* Stage (3) alone: Wq and w_scales from given s, L1, L2 (host memory).
 * Bit-exact contract: the same inputs always give the same bytes. */
svdq_status svdq_quantize_residual(const float* W, int N, int K, const float* smooth,
                                   const uint16_t* L1, const uint16_t* L2, int r, uint8_t* Wq,
                                   float* w_scales);

/* Attach an off-the-shelf LoRA to a packed layer without re-quantizing it
 * (abstract of "SVDQuant: Absorbing Outliers by Low-Rank Components for 4-Bit
 * Diffusion Models": existing low-rank adapters are supported as they are).
 * The adapter adds X A B to the output, A [K, rl] (down) and B [rl, N] (up),
 * float32 row-major.  The low-rank branch sees X diag(s)^-1, so the adapter
 * enters as extra rank:
 *   L1_out [r + rl, K] = [L1 ; bf16((diag(s) A)^T)]  (A[k, j] s[k] rounded once)
 *   L2_out [N, r + rl] = [L2 | bf16(B^T)]
 * Wq and w_scales are unchanged.  The forward needs r + rl to be a multiple
 * of 16 and at most 128.  L1/L2 may be NULL when r == 0.  Host memory,
 * synchronous; outputs are untouched on an error. */
svdq_status svdq_append_lora(const float* smooth, int K, int N, const uint16_t* L1,
                             const uint16_t* L2, int r, const float* A, const float* B, int rl,
                             uint16_t* L1_out, uint16_t* L2_out);

/* ---------------------------------------------------------------- device */

/* Workspace the forward needs, in bytes: the activation codes qx, their
 * scales sx and T = x_hat L1^T, plus fp32 partial accumulators when the GEMM
 * cuts a last, partial wave of output tiles along K (this part depends on N
 * and on the current device's compute-unit count).  Each part is 256-byte
 * aligned.  Returns 0 for shapes the forward rejects. */
size_t svdq_forward_workspace_bytes(int M, int K, int N, int r);

/* Where the forward keeps stage 1's results inside its workspace, as byte
 * offsets from the workspace's start: qx [M, K/2] codes at *qx_offset, the
 * float32 scales sx [M, K/64] at *sx_offset, and *t_slices partial sums of
 * T = x_hat L1^T, each [M, r] float32, back to back from *t_offset (T is their
 * sum taken in slice order; *t_slices = 0 and *t_offset = 0 when r = 0).  The
 * layout depends on the shape only.  Host function; SVDQ_ERR_INVALID_ARG for
 * shapes the forward rejects or NULL outputs.  For callers that inspect or
 * reuse the quantized activations (and for tests of the forward's own launch). */
svdq_status svdq_forward_workspace_layout(int M, int K, int N, int r, size_t* qx_offset,
                                          size_t* sx_offset, size_t* t_offset, int* t_slices);

/* The SVDQuant linear forward (E4): launches the fused smooth + quantize +
 * lora_down kernel, then the W4A4 GEMM whose epilogue applies the group
 * scales, adds the lora_up product and the bias and stores bf16 Y.  Small
 * layers (svdq_forward_fused(M, K, N, r) != 0: K <= 1280, r <= 32,
 * N <= 2560 and at most 256 blocks of 16 x 16 outputs x 64 channels per
 * compute unit) run all of it as one kernel instead; the codes and scales
 * are the same, the workspace is then unused (but still required).
 * Requires M >= 1, K % 64 == 0, N % 16 == 0, 0 <= r <= 128, r % 16 == 0,
 * 16-byte aligned device pointers (bias and, for r = 0, L1/L2 may be NULL)
 * and workspace_bytes >= svdq_forward_workspace_bytes(M, K, N, r).  Asynchronous
 * on `stream`; no allocation, no synchronization. */
svdq_status svdq_linear_forward(const uint16_t* X, int M, int K, int N, int r,
                                const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                const uint8_t* Wq, const float* w_scales, const uint16_t* bias,
                                uint16_t* Y, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Output activation of the _act entry points, applied in float32 to each
 * output (after the bias) before its one rounding to bf16.
 * SVDQ_ACT_GELU_TANH is GELU in its tanh form (Hendrycks and Gimpel,
 * "Gaussian Error Linear Units", section 2),
 *   0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))),
 * the activation between the up and down projections of a DiT MLP; fusing it
 * here lets the up projection's output feed the down projection directly. */
typedef enum { SVDQ_ACT_NONE = 0, SVDQ_ACT_GELU_TANH = 1 } svdq_activation;

/* svdq_linear_forward with `activation` (an svdq_activation value; any other
 * value is SVDQ_ERR_INVALID_ARG) applied to Y. */
svdq_status svdq_linear_forward_act(const uint16_t* X, int M, int K, int N, int r,
                                    const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                    const uint8_t* Wq, const float* w_scales,
                                    const uint16_t* bias, int activation, uint16_t* Y,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * forward as svdq_linear_forward_act, with its workspace (the activation codes,
 * scales, T and the GEMM's split partials) in a static device array of
 * svdq_static_workspace_bytes() bytes (64 MiB) that each GPU the library runs
 * on holds until the process ends.  Shapes whose workspace,
 * svdq_forward_workspace_bytes(M, K, N, r), exceeds it return
 * SVDQ_ERR_WORKSPACE before anything is launched.  No allocation and no
 * synchronization; nothing in the array needs to start at zero.  Every call on
 * one GPU shares that GPU's array and it keeps the last call's contents, so
 * calls that overlap on one GPU (on different streams, or from different
 * threads) race: serialize them.  Otherwise as svdq_linear_forward_act. */
size_t svdq_static_workspace_bytes(void);
svdq_status svdq_linear_forward_noalloc(const uint16_t* X, int M, int K, int N, int r,
                                        const float* smooth, const uint16_t* L1,
                                        const uint16_t* L2, const uint8_t* Wq,
                                        const float* w_scales, const uint16_t* bias,
                                        int activation, uint16_t* Y, void* stream);

/* The two halves of svdq_linear_forward, for callers that schedule or time
 * them separately.  Stage 1 writes qx, sx, T into the workspace; stage 2
 * reads them and writes Y.  Same requirements as svdq_linear_forward. */
svdq_status svdq_forward_quantize(const uint16_t* X, int M, int K, int r, const float* smooth,
                                  const uint16_t* L1, void* workspace, size_t workspace_bytes,
                                  void* stream);
svdq_status svdq_forward_gemm(int M, int K, int N, int r, const uint16_t* L2, const uint8_t* Wq,
                              const float* w_scales, const uint16_t* bias, uint16_t* Y,
                              const void* workspace, size_t workspace_bytes, void* stream);
/* Stage 2 with an output activation, as svdq_linear_forward_act. */
svdq_status svdq_forward_gemm_act(int M, int K, int N, int r, const uint16_t* L2,
                                  const uint8_t* Wq, const float* w_scales, const uint16_t* bias,
                                  int activation, uint16_t* Y, const void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Stage 1 into caller buffers in the canonical layouts: Q(X diag(s)^-1) as
 * qx [M, K/2] and sx [M, K/64], and T = x_hat L1^T [M, r] in float32
 * (T may be NULL when r == 0).  One workgroup stages a whole row of K channels
 * in LDS, so K <= 12544 here (larger K: SVDQ_ERR_INVALID_ARG; the forward
 * itself slices K and has no such bound).  Device memory, asynchronous. */
svdq_status svdq_quantize_activations(const uint16_t* X, int M, int K, const float* smooth,
                                      const uint16_t* L1, int r, uint8_t* qx, float* sx,
                                      float* T, void* stream);

/* The calibration statistic of svdq_act_absmax_update on the GPU: A_scale of
 * E2 (Terminology Entry, section 2.3: the per-channel absolute maximum of the
 * activations).  Folds M rows of bf16 activations X [M, K] (device memory,
 * row-major) into the running maximum amax [K] (device memory, float32):
 * amax[k] = max(amax[k], max_m |X[m,k]|), bit-identical to the host function
 * (a max does not depend on the order of evaluation).  amax must hold values
 * >= +0 on entry (start from zeros): the partial maxima meet through an
 * unsigned atomic max of the float32 bit patterns, which orders those values
 * like floats.  Any K >= 1; M = 0 does nothing.  X must be 2-byte aligned and
 * amax 4-byte aligned (SVDQ_ERR_ALIGNMENT).  Asynchronous on `stream`; calls
 * that write the same amax may run concurrently (the atomics commute). */
svdq_status svdq_act_absmax_update_device(const uint16_t* X, int64_t M, int K, float* amax,
                                          void* stream);

/* The integer group partial sums of Q(x_hat) Q(R) (E4, E7) over the output
 * block rows [m0, m1) x columns [n0, n1), computed by the forward's own GEMM
 * launch for an M x N x K layer (the same tile class, tile order and, where
 * the forward cuts a last partial wave of tiles along K, the same shares):
 * every tile runs its MFMA main loop, and the tiles that cover the block write
 * P[(m-m0), (n-n0), g] = sum_{k in group g} qx[m,k] qw[n,k] instead of the
 * scale epilogue, int32 [(m1-m0), (n1-n0), K/64].  qx [M, K/2] and Wq [N, K/2]
 * are read whole.  Requires 0 <= m0 < m1 <= M, 0 <= n0 < n1 <= N,
 * N % 16 == 0, K % 64 == 0.  Device memory, asynchronous. */
svdq_status svdq_debug_group_partials(const uint8_t* qx, const uint8_t* Wq, int M, int N, int K,
                                      int m0, int m1, int n0, int n1, int32_t* P, void* stream);

/* 1 if the int4 forward (svdq_linear_forward[_act], and the no-alloc entry
 * point) runs the shape as the single fused small-K kernel, else 0 (also for
 * shapes the forward rejects).  Host only. */
int svdq_forward_fused(int M, int K, int N, int r);

/* The fused small-K forward exactly as svdq_linear_forward_act launches it,
 * also writing the activation codes it quantized, qx [M, K/2] (packed as
 * svdq_quantize_activations writes them), and their scales sx [M, K/64], so
 * that they can be checked against the quantizer's definition (E2, E3).
 * SVDQ_ERR_INVALID_ARG if svdq_forward_fused(M, K, N, r) is 0.  Device memory,
 * asynchronous; the forward's own requirements otherwise (no workspace). */
svdq_status svdq_debug_fused_forward(const uint16_t* X, int M, int K, int N, int r,
                                     const float* smooth, const uint16_t* L1, const uint16_t* L2,
                                     const uint8_t* Wq, const float* w_scales,
                                     const uint16_t* bias, int activation, uint16_t* Y,
                                     uint8_t* qx, float* sx, void* stream);

/* ------------------------------------------------------- MXFP4 variant
 * The same layer with Q(.) (Terminology Entry, section 2.3, E4) taken as the
 * OCP microscaling format MXFP4: blocks of 32 consecutive input channels
 * share one E8M0 scale byte (2^(byte - 127), exponent floor(log2 amax) - 2)
 * and every element is an FP4 E2M1 number (nearest, ties to even,
 * saturating at +-6, sign kept).  Codes are packed like the int4 ones (two per
 * byte, even channel in the low nibble).  Scales are E8M0 bytes in one of two
 * layouts:
 *   row-major  [rows, K/32]: what the packer and svdq_quantize_activations_mxfp4
 *              write, and what parity is defined on;
 *   k-tiled    [ceil(K/256)][rows][8]: byte (t * rows + n) * 8 + j is the scale
 *              of block 8 t + j of row n, blocks past K/32 are padding (127).
 *              The forward's GEMM reads its weight scales in this layout: one
 *              256-channel stage of a tile's rows is then one contiguous run.
 *              svdq_mxfp4_tile_scales converts, once per weight.
 * The GEMM runs on CDNA4's block-scaled FP4 MFMA.  Requirements as for the
 * int4 entry points, with K % 128 == 0. */

/* Bytes of the k-tiled layout of `rows` rows: ceil(K/256) * rows * 8; 0 if
 * rows < 1 or K is not a positive multiple of 128. */
size_t svdq_mxfp4_tiled_scale_bytes(int rows, int K);

/* Row-major scales [rows, K/32] -> k-tiled (svdq_mxfp4_tiled_scale_bytes bytes,
 * caller-allocated host memory; padding bytes are 127).  Host, synchronous.
 * SVDQ_ERR_INVALID_ARG for NULL pointers or the shapes rejected above. */
svdq_status svdq_mxfp4_tile_scales(const uint8_t* scales, int rows, int K, uint8_t* tiled);

/* Stage three with MXFP4 on the host: Wq [N, K/2] and row-major w_e8m0
 * [N, K/32] of R = W diag(s) - L2 L1 (R formed exactly as for
 * svdq_quantize_residual).  The forward takes the scales k-tiled. */
svdq_status svdq_quantize_residual_mxfp4(const float* W, int N, int K, const float* smooth,
                                         const uint16_t* L1, const uint16_t* L2, int r,
                                         uint8_t* Wq, uint8_t* w_e8m0);

/* Workspace of the MXFP4 forward: codes, E8M0 scales and T; 0 for rejected shapes. */
size_t svdq_forward_workspace_bytes_mxfp4(int M, int K, int N, int r);

/* The MXFP4 workspace, as svdq_forward_workspace_layout: the E8M0 activation
 * scales at *sx_offset are k-tiled, [ceil(K/256)][*sx_rows][8] bytes. */
svdq_status svdq_forward_workspace_layout_mxfp4(int M, int K, int N, int r, size_t* qx_offset,
                                                size_t* sx_offset, size_t* t_offset, int* t_slices,
                                                int* sx_rows);

/* The MXFP4 forward: quantize + lora_down, then the block-scaled GEMM whose
 * epilogue adds the lora_up product and the bias.  w_e8m0 is k-tiled
 * [ceil(K/256)][N][8] (see above); the workspace holds the activation scales
 * k-tiled too.  Small layers (svdq_forward_fused_mxfp4 != 0) run as one fused
 * kernel, as the int4 forward does, and leave the workspace untouched.
 * Device memory, asynchronous on `stream`, no allocation. */
svdq_status svdq_linear_forward_mxfp4(const uint16_t* X, int M, int K, int N, int r,
                                      const float* smooth, const uint16_t* L1,
                                      const uint16_t* L2, const uint8_t* Wq,
                                      const uint8_t* w_e8m0, const uint16_t* bias, uint16_t* Y,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* The MXFP4 forward with an output activation, as svdq_linear_forward_act. */
svdq_status svdq_linear_forward_act_mxfp4(const uint16_t* X, int M, int K, int N, int r,
                                          const float* smooth, const uint16_t* L1,
                                          const uint16_t* L2, const uint8_t* Wq,
                                          const uint8_t* w_e8m0, const uint16_t* bias,
                                          int activation, uint16_t* Y, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Its two halves, as svdq_forward_quantize / svdq_forward_gemm(_act). */
svdq_status svdq_forward_quantize_mxfp4(const uint16_t* X, int M, int K, int r,
                                        const float* smooth, const uint16_t* L1, void* workspace,
                                        size_t workspace_bytes, void* stream);
svdq_status svdq_forward_gemm_mxfp4(int M, int K, int N, int r, const uint16_t* L2,
                                    const uint8_t* Wq, const uint8_t* w_e8m0,
                                    const uint16_t* bias, uint16_t* Y, const void* workspace,
                                    size_t workspace_bytes, void* stream);
svdq_status svdq_forward_gemm_act_mxfp4(int M, int K, int N, int r, const uint16_t* L2,
                                        const uint8_t* Wq, const uint8_t* w_e8m0,
                                        const uint16_t* bias, int activation, uint16_t* Y,
                                        const void* workspace, size_t workspace_bytes,
                                        void* stream);

/* 1 if the MXFP4 forward runs the shape as the single fused small-K kernel
 * (the int4 range, with K a multiple of 128, and up to 400 blocks of
 * 16 x 16 outputs x 64 channels per compute unit where K <= 640), else 0
 * (also for shapes the forward rejects).  Host only. */
int svdq_forward_fused_mxfp4(int M, int K, int N, int r);

/* The fused MXFP4 forward exactly as svdq_linear_forward_act_mxfp4 launches
 * it, also writing the codes it quantized, qx [M, K/2] (canonical packed),
 * and their E8M0 scale bytes sx_e8m0 [M, K/32] (row-major), as
 * svdq_quantize_activations_mxfp4 writes them.  SVDQ_ERR_INVALID_ARG if
 * svdq_forward_fused_mxfp4(M, K, N, r) is 0.  Device memory, asynchronous;
 * the forward's own requirements otherwise (no workspace). */
svdq_status svdq_debug_fused_forward_mxfp4(const uint16_t* X, int M, int K, int N, int r,
                                           const float* smooth, const uint16_t* L1,
                                           const uint16_t* L2, const uint8_t* Wq,
                                           const uint8_t* w_e8m0, const uint16_t* bias,
                                           int activation, uint16_t* Y, uint8_t* qx,
                                           uint8_t* sx_e8m0, void* stream);

/* Stage 1 into canonical buffers: qx [M, K/2], sx_e8m0 [M, K/32], T [M, r];
 * K <= 12544 as for svdq_quantize_activations. */
svdq_status svdq_quantize_activations_mxfp4(const uint16_t* X, int M, int K, const float* smooth,
                                            const uint16_t* L1, int r, uint8_t* qx,
                                            uint8_t* sx_e8m0, float* T, void* stream);

const char* svdq_status_string(svdq_status status);
const char* svdq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H_ */
