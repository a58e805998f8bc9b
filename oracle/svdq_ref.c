/* Plain C oracle of the SVDQuant W4A4 linear layer with its low-rank branch.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load this code (through oracle/svdq_ref.py).
 * The product path (the HIP library and its binding) never calls it, and it
 * shares no code, header, table or helper with that path.  It is also
 * written independently of the numpy oracle in oracle/svdq_oracle.py: the two
 * are separate readings of the same pages, checked against each other and
 * against the same exact-rational pins.
 *
 * Plain, slow, single-threaded, C99: double precision everywhere except at
 * the points where the method fixes a float32 rounding (smoothing, the
 * quantization scales and codes), where C's IEEE float arithmetic is used
 * (build with -ffp-contract=off: every float operation is rounded on its own).
 *
 * Citations name the page and the equation:
 *   [Term] "SVDQuant Low-Rank Residual Quantization Algorithm Terminology
 *          Entry", section 2.3 "Mathematical Description", equations numbered
 *          in page order: E1 outlier migration, E2 smoothing factor, E3 SVD
 *          split, E4 dual-path output, E5 Eckart-Young, E6 residual energy,
 *          E7 low-bit path only for the residual.
 *   [Abs]  the SVDQuant abstract: 4-bit weights and activations, a 16-bit
 *          low-rank branch, LoRAs attached without re-quantization.
 *
 * Readings where the pages are silent (the same as the numpy oracle's):
 * W is stored [N, K] (out, in) and s indexes input channels; W_scale is the
 * per-input-channel absolute maximum; both statistics are floored at 1e-5 and
 * s at s_min; L1 = bf16(V_r^T) [r, K], L2 = bf16(U_r Sigma_r) [N, r]; R is
 * formed from the rounded factors; Q is symmetric 4-bit with one float32 scale
 * per 64 channels, scale = fl32(a / 7), codes clamp(rne(fl32(v fl32(7 / a))),
 * -7, 7), a group with a < 2^-100 is coded as zeros with scale 0; weight scales
 * have their two low significand bits cleared; x_hat = fl32(X fl32(1 / s));
 * two codes per byte, the even channel in the low nibble.  MXFP4: blocks of 32
 * share a power-of-two scale 2^e, e = floor(log2 amax) - 2 (OCP MX v1.0),
 * E2M1 elements rounded to nearest, ties to even, saturating at 6.
 *
 * The SVD is a one-sided (Hestenes) Jacobi iteration, written out here, so
 * the oracle needs no linear-algebra library.
 *
 * Every function returns 0, or -1 on an argument it does not accept.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64
#define QMAX 7
#define MX_BLOCK 32

/* ------------------------------------------------------------ bfloat16 */

static float bf16_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t float_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static float bits_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bfloat16 nearest to a double, ties to even, with one rounding from the exact
 * double value: the significand is cut to 8 bits on the grid of the value's
 * binade (at least 2^-126, where bfloat16's subnormals keep that grid). */
uint16_t oref_bf16_from_double(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return 0x7FC0;
  const uint16_t sign = v < 0 ? 0x8000 : 0;
  const double a = fabs(v);
  int e;
  frexp(a, &e);                      /* a in [2^(e-1), 2^e) */
  int lead = e - 1;
  if (lead < -126) lead = -126;
  const double ulp = ldexp(1.0, lead - 7);
  const double q = a / ulp;          /* exact: division by a power of two */
  double r = floor(q);
  const double frac = q - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) == 1.0)) r += 1.0;
  const double val = r * ulp;
  if (val >= ldexp(1.0, 128)) return sign | 0x7F80;
  return sign | (uint16_t)(float_bits((float)val) >> 16);   /* (float)val is exact */
}

/* ---------------------------------------------------- stage one: smoothing */

/* A_scale[k] = max over rows of |X[m, k]| for bf16 X [M, K] ([Term] 2.3, A_scale
 * under E2).  A max is exact. */
int oref_act_absmax(const uint16_t* X, int M, int K, float* A) {
  if (M < 0 || K <= 0) return -1;
  for (int k = 0; k < K; ++k) A[k] = 0.0f;
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) {
      const float v = fabsf(bf16_to_float(X[(size_t)m * K + k]));
      if (v > A[k]) A[k] = v;
    }
  return 0;
}

/* W_scale[k] = max over output rows n of |W[n, k]| ([Term] 2.3, W_scale under E2). */
int oref_weight_absmax(const float* W, int N, int K, float* Wsc) {
  if (N <= 0 || K <= 0) return -1;
  for (int k = 0; k < K; ++k) Wsc[k] = 0.0f;
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) {
      const float v = fabsf(W[(size_t)n * K + k]);
      if (v > Wsc[k]) Wsc[k] = v;
    }
  return 0;
}

/* s[k] = max(A^alpha / W_scale^(1 - alpha), s_min) in double, stored as float
 * ([Term] 2.3, E2); both statistics floored at 1e-5 first. */
int oref_smoothing_factors(const float* A, const float* Wsc, int K, double alpha, double s_min,
                           float* s) {
  if (K <= 0) return -1;
  for (int k = 0; k < K; ++k) {
    double a = A[k], w = Wsc[k];
    if (a < 1e-5) a = 1e-5;
    if (w < 1e-5) w = 1e-5;
    double v = pow(a, alpha) / pow(w, 1.0 - alpha);
    if (v < s_min) v = s_min;
    s[k] = (float)v;
  }
  return 0;
}

/* W_hat[n, k] = W[n, k] s[k], exact in double ([Term] 2.3, E1). */
int oref_smooth_weight(const float* W, int N, int K, const float* s, double* What) {
  if (N <= 0 || K <= 0) return -1;
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) What[(size_t)n * K + k] = (double)W[(size_t)n * K + k] * (double)s[k];
  return 0;
}

/* --------------------------------------------- stage two: low-rank branch */

/* One-sided Jacobi on the columns of B (rows x cols, column j at B + j rows,
 * rows >= cols): plane rotations of column pairs until every pair is
 * orthogonal to 1e-15 (at most 60 sweeps), applied to V (cols x cols, same
 * layout) as well.  Then B = U Sigma, and the input equals U Sigma V^T. */
static int jacobi_columns(double* B, int rows, int cols, double* V) {
  for (int j = 0; j < cols; ++j)
    for (int i = 0; i < cols; ++i) V[(size_t)j * cols + i] = i == j ? 1.0 : 0.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    double worst = 0.0;
    for (int p = 0; p < cols - 1; ++p)
      for (int q = p + 1; q < cols; ++q) {
        double* bp = B + (size_t)p * rows;
        double* bq = B + (size_t)q * rows;
        double alpha = 0.0, beta = 0.0, gamma = 0.0;
        for (int i = 0; i < rows; ++i) {
          alpha += bp[i] * bp[i];
          beta += bq[i] * bq[i];
          gamma += bp[i] * bq[i];
        }
        if (gamma == 0.0) continue;
        const double off = fabs(gamma) / sqrt(alpha * beta);
        if (off > worst) worst = off;
        if (off < 1e-15) continue;
        /* the rotation that zeroes the pair's inner product: tan of the angle
         * is the smaller root of t^2 + 2 zeta t - 1 = 0 */
        const double zeta = (beta - alpha) / (2.0 * gamma);
        const double t = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
        const double c = 1.0 / sqrt(1.0 + t * t);
        const double sn = c * t;
        for (int i = 0; i < rows; ++i) {
          const double x = bp[i], y = bq[i];
          bp[i] = c * x - sn * y;
          bq[i] = sn * x + c * y;
        }
        double* vp = V + (size_t)p * cols;
        double* vq = V + (size_t)q * cols;
        for (int i = 0; i < cols; ++i) {
          const double x = vp[i], y = vq[i];
          vp[i] = c * x - sn * y;
          vq[i] = sn * x + c * y;
        }
      }
    if (worst < 1e-15) return 0;
  }
  return 0;   /* 60 sweeps: accepted as converged (the pins check the result) */
}

/* Thin SVD W_hat = U diag(sigma) V^T of What [N, K] ([Term] 2.3, E3), p =
 * min(N, K): U [N, p], sigma [p] descending, V [K, p], all row-major.  Each
 * pair's sign puts the largest-magnitude entry of v_i positive (the first such
 * entry on a tie).  Zero singular values get zero columns of U. */
int oref_svd(const double* What, int N, int K, double* U, double* sigma, double* V) {
  if (N <= 0 || K <= 0) return -1;
  const int tall = N >= K;
  const int rows = tall ? N : K, cols = tall ? K : N;   /* Jacobi on W_hat (tall) or W_hat^T */
  double* B = (double*)malloc(sizeof(double) * (size_t)rows * cols);
  double* J = (double*)malloc(sizeof(double) * (size_t)cols * cols);
  int* order = (int*)malloc(sizeof(int) * (size_t)cols);
  double* norm = (double*)malloc(sizeof(double) * (size_t)cols);
  if (!B || !J || !order || !norm) {
    free(B); free(J); free(order); free(norm);
    return -1;
  }
  for (int j = 0; j < cols; ++j)
    for (int i = 0; i < rows; ++i)
      B[(size_t)j * rows + i] = tall ? What[(size_t)i * K + j] : What[(size_t)j * K + i];
  jacobi_columns(B, rows, cols, J);
  for (int j = 0; j < cols; ++j) {
    double s2 = 0.0;
    for (int i = 0; i < rows; ++i) s2 += B[(size_t)j * rows + i] * B[(size_t)j * rows + i];
    norm[j] = sqrt(s2);
    order[j] = j;
  }
  /* descending by norm, stable (insertion sort) */
  for (int a = 1; a < cols; ++a) {
    const int x = order[a];
    int b = a - 1;
    while (b >= 0 && norm[order[b]] < norm[x]) {
      order[b + 1] = order[b];
      --b;
    }
    order[b + 1] = x;
  }
  /* tall: W_hat = (B / sigma) sigma J^T, so U = B / sigma, V = J.
   * wide: W_hat^T = (B / sigma) sigma J^T, so U = J and V = B / sigma. */
  const int p = cols;
  for (int o = 0; o < p; ++o) {
    const int j = order[o];
    const double sg = norm[j];
    sigma[o] = sg;
    const double* bj = B + (size_t)j * rows;
    const double* jj = J + (size_t)j * cols;
    for (int n = 0; n < N; ++n) {
      const double u = tall ? (sg > 0 ? bj[n] / sg : 0.0) : jj[n];
      U[(size_t)n * p + o] = u;
    }
    for (int k = 0; k < K; ++k) {
      const double v = tall ? jj[k] : (sg > 0 ? bj[k] / sg : 0.0);
      V[(size_t)k * p + o] = v;
    }
    /* sign: largest |v_i| entry positive */
    int at = 0;
    for (int k = 1; k < K; ++k)
      if (fabs(V[(size_t)k * p + o]) > fabs(V[(size_t)at * p + o])) at = k;
    if (V[(size_t)at * p + o] < 0) {
      for (int k = 0; k < K; ++k) V[(size_t)k * p + o] = -V[(size_t)k * p + o];
      for (int n = 0; n < N; ++n) U[(size_t)n * p + o] = -U[(size_t)n * p + o];
    }
  }
  free(B); free(J); free(order); free(norm);
  return 0;
}

/* L1[j, k] = bf16(V[k, j]) [r, K] (lora_down) and L2[n, j] = bf16(U[n, j] sigma_j)
 * [N, r] (lora_up): E4 writes the branch as (X diag(s)^-1 V)(U S)^T, so sigma
 * rides with U.  U is [N, p], V is [K, p]. */
int oref_lowrank_factors(const double* U, const double* sigma, const double* V, int N, int K,
                         int p, int r, uint16_t* L1, uint16_t* L2) {
  if (r < 0 || r > p) return -1;
  for (int j = 0; j < r; ++j)
    for (int k = 0; k < K; ++k) L1[(size_t)j * K + k] = oref_bf16_from_double(V[(size_t)k * p + j]);
  for (int n = 0; n < N; ++n)
    for (int j = 0; j < r; ++j)
      L2[(size_t)n * r + j] = oref_bf16_from_double(U[(size_t)n * p + j] * sigma[j]);
  return 0;
}

/* R[n, k] = fl32(W_hat[n, k] - sum_j L2[n, j] L1[j, k]) ([Term] 2.3, E3) with
 * the stored bf16 factors; the sum runs j = 0, 1, ... in double from 0, each
 * product exact, then one subtraction and one rounding. */
int oref_residual(const double* What, int N, int K, const uint16_t* L1, const uint16_t* L2, int r,
                  float* R) {
  if (N <= 0 || K <= 0 || r < 0) return -1;
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) {
      double acc = 0.0;
      for (int j = 0; j < r; ++j)
        acc += (double)bf16_to_float(L2[(size_t)n * r + j]) * (double)bf16_to_float(L1[(size_t)j * K + k]);
      R[(size_t)n * K + k] = (float)(What[(size_t)n * K + k] - acc);
    }
  return 0;
}

/* ------------------------------------------- stage three: quantization Q */

/* Q over each 64-channel group of rows x K floats ([Term] 2.3, E4 names Q;
 * [Abs] fixes 4 bits): codes q [rows, K] in [-7, 7], scales [rows, K / 64]. */
int oref_quantize_groups(const float* v, int rows, int K, int weight_scale, int8_t* q,
                         float* scale) {
  if (rows < 0 || K <= 0 || K % GROUP) return -1;
  const int G = K / GROUP;
  const float tiny = ldexpf(1.0f, -100);
  for (int m = 0; m < rows; ++m)
    for (int g = 0; g < G; ++g) {
      const float* x = v + (size_t)m * K + (size_t)g * GROUP;
      int8_t* c = q + (size_t)m * K + (size_t)g * GROUP;
      float a = 0.0f;
      for (int i = 0; i < GROUP; ++i)
        if (fabsf(x[i]) > a) a = fabsf(x[i]);
      if (!(a >= tiny)) {
        for (int i = 0; i < GROUP; ++i) c[i] = 0;
        scale[(size_t)m * G + g] = 0.0f;
        continue;
      }
      float sc = a / (float)QMAX;
      const float inv = (float)QMAX / a;
      for (int i = 0; i < GROUP; ++i) {
        const float t = x[i] * inv;          /* one float rounding */
        float r = nearbyintf(t);             /* ties to even (default rounding mode) */
        if (r > QMAX) r = QMAX;
        if (r < -QMAX) r = -QMAX;
        c[i] = (int8_t)r;
      }
      if (weight_scale) sc = bits_float(float_bits(sc) & 0xFFFFFFFCu);
      scale[(size_t)m * G + g] = sc;
    }
  return 0;
}

/* byte i of a row = (q[2i] & 0xF) | (q[2i + 1] & 0xF) << 4 */
int oref_pack_nibbles(const int8_t* q, int rows, int K, uint8_t* out) {
  if (rows < 0 || K <= 0 || K % 2) return -1;
  for (size_t i = 0; i < (size_t)rows * K / 2; ++i)
    out[i] = (uint8_t)(((uint8_t)q[2 * i] & 0xF) | (((uint8_t)q[2 * i + 1] & 0xF) << 4));
  return 0;
}

static int nibble_value(uint8_t b, int hi) {
  const int v = hi ? (b >> 4) & 0xF : b & 0xF;
  return v >= 8 ? v - 16 : v;
}

/* Stage three of the pack: Wq [N, K / 2] and w_scales [N, K / 64] of the residual
 * of W with the given s, L1 and L2. */
int oref_quantize_residual(const float* W, int N, int K, const float* s, const uint16_t* L1,
                           const uint16_t* L2, int r, uint8_t* Wq, float* w_scales) {
  if (N <= 0 || K <= 0 || K % GROUP || r < 0) return -1;
  double* What = (double*)malloc(sizeof(double) * (size_t)N * K);
  float* R = (float*)malloc(sizeof(float) * (size_t)N * K);
  int8_t* q = (int8_t*)malloc((size_t)N * K);
  int rc = -1;
  if (What && R && q) {
    oref_smooth_weight(W, N, K, s, What);
    oref_residual(What, N, K, L1, L2, r, R);
    oref_quantize_groups(R, N, K, 1, q, w_scales);
    oref_pack_nibbles(q, N, K, Wq);
    rc = 0;
  }
  free(What); free(R); free(q);
  return rc;
}

/* The whole offline pipeline ([Term] 2.1, three stages in order; 2.3 E1-E4):
 * W_scale, s (E2), W_hat (E1), SVD (E3), L1 and L2 (E4), R and Q(R).
 * sigma [min(N, K)] may be NULL. */
int oref_pack_weights(const float* W, int N, int K, const float* A, double alpha, double s_min,
                      int r, float* s, uint16_t* L1, uint16_t* L2, uint8_t* Wq, float* w_scales,
                      double* sigma) {
  if (N <= 0 || K <= 0 || K % GROUP || r < 0) return -1;
  const int p = N < K ? N : K;
  if (r > p) return -1;
  float* Wsc = (float*)malloc(sizeof(float) * (size_t)K);
  double* What = (double*)malloc(sizeof(double) * (size_t)N * K);
  double* U = (double*)malloc(sizeof(double) * (size_t)N * p);
  double* V = (double*)malloc(sizeof(double) * (size_t)K * p);
  double* sg = (double*)malloc(sizeof(double) * (size_t)p);
  int rc = -1;
  if (Wsc && What && U && V && sg) {
    oref_weight_absmax(W, N, K, Wsc);
    oref_smoothing_factors(A, Wsc, K, alpha, s_min, s);
    oref_smooth_weight(W, N, K, s, What);
    if (oref_svd(What, N, K, U, sg, V) == 0) {
      oref_lowrank_factors(U, sg, V, N, K, p, r, L1, L2);
      rc = oref_quantize_residual(W, N, K, s, L1, L2, r, Wq, w_scales);
      if (sigma) memcpy(sigma, sg, sizeof(double) * (size_t)p);
    }
  }
  free(Wsc); free(What); free(U); free(V); free(sg);
  return rc;
}

/* ------------------------------------------------------------- forward */

/* x_hat[m, k] = fl32(X[m, k] fl32(1 / s[k])) ([Term] 2.3, E1 and E4). */
int oref_smooth_activations(const uint16_t* X, int M, int K, const float* s, float* xh) {
  if (M < 0 || K <= 0) return -1;
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) {
      const float inv = 1.0f / s[k];
      xh[(size_t)m * K + k] = bf16_to_float(X[(size_t)m * K + k]) * inv;
    }
  return 0;
}

/* The first half of E4: Q(X diag(s)^-1) as packed codes qx [M, K / 2] and
 * scales sx [M, K / 64], and lora_down T = x_hat L1^T [M, r] in double
 * (k ascending).  T may be NULL when r == 0. */
int oref_quantize_activations(const uint16_t* X, int M, int K, const float* s, const uint16_t* L1,
                              int r, uint8_t* qx, float* sx, double* T) {
  if (M < 0 || K <= 0 || K % GROUP || r < 0) return -1;
  float* xh = (float*)malloc(sizeof(float) * ((size_t)M * K + 1));
  int8_t* q = (int8_t*)malloc((size_t)M * K + 1);
  if (!xh || !q) {
    free(xh); free(q);
    return -1;
  }
  oref_smooth_activations(X, M, K, s, xh);
  oref_quantize_groups(xh, M, K, 0, q, sx);
  oref_pack_nibbles(q, M, K, qx);
  for (int m = 0; m < M; ++m)
    for (int j = 0; j < r; ++j) {
      double t = 0.0;
      for (int k = 0; k < K; ++k)
        t += (double)xh[(size_t)m * K + k] * (double)bf16_to_float(L1[(size_t)j * K + k]);
      T[(size_t)m * r + j] = t;
    }
  free(xh); free(q);
  return 0;
}

/* P[m, n, g] = sum over k in group g of qx[m, k] qw[n, k], exact in int32
 * ([Term] 2.3, E4 Q(.)Q(R) and E7: the low-bit product, taken only for R). */
int oref_group_partials(const uint8_t* qx, const uint8_t* wq, int M, int N, int K, int32_t* P) {
  if (M < 0 || N < 0 || K <= 0 || K % GROUP) return -1;
  const int G = K / GROUP, KB = K / 2;
  for (int m = 0; m < M; ++m)
    for (int n = 0; n < N; ++n)
      for (int g = 0; g < G; ++g) {
        int32_t p = 0;
        for (int i = 0; i < GROUP; ++i) {
          const int k = g * GROUP + i;
          p += nibble_value(qx[(size_t)m * KB + k / 2], k & 1) *
               nibble_value(wq[(size_t)n * KB + k / 2], k & 1);
        }
        P[((size_t)m * N + n) * G + g] = p;
      }
  return 0;
}

/* GELU, tanh form (Hendrycks and Gimpel, "Gaussian Error Linear Units",
 * section 2), in double: the activation between a DiT MLP's projections. */
double oref_gelu_tanh(double x) {
  return 0.5 * x * (1.0 + tanh(sqrt(2.0 / 3.14159265358979323846) * (x + 0.044715 * x * x * x)));
}

/* Rows [m0, m1) of the dual-path output ([Term] 2.3, E4 and E7), in double:
 *   Y[m, n] = sum_g sx[m, g] sw[n, g] P[m, n, g] + sum_j T[m, j] L2[n, j] + b[n],
 * then gelu_tanh when act == 1.  Y holds (m1 - m0) x N values.  bias may be
 * NULL (zero); L1 and L2 may be NULL when r == 0. */
int oref_forward_rows(const uint16_t* X, int M, int K, int N, int r, const float* s,
                      const uint16_t* L1, const uint16_t* L2, const uint8_t* Wq,
                      const float* w_scales, const uint16_t* bias, int act, int m0, int m1,
                      double* Y) {
  if (M < 0 || K <= 0 || K % GROUP || N <= 0 || r < 0 || m0 < 0 || m1 > M || m0 > m1) return -1;
  const int rows = m1 - m0, G = K / GROUP, KB = K / 2;
  uint8_t* qx = (uint8_t*)malloc((size_t)rows * KB + 1);
  float* sx = (float*)malloc(sizeof(float) * ((size_t)rows * G + 1));
  double* T = (double*)malloc(sizeof(double) * ((size_t)rows * r + 1));
  if (!qx || !sx || !T) {
    free(qx); free(sx); free(T);
    return -1;
  }
  oref_quantize_activations(X + (size_t)m0 * K, rows, K, s, L1, r, qx, sx, T);
  for (int m = 0; m < rows; ++m)
    for (int n = 0; n < N; ++n) {
      double main = 0.0;
      for (int g = 0; g < G; ++g) {
        int32_t p = 0;
        for (int i = 0; i < GROUP; ++i) {
          const int k = g * GROUP + i;
          p += nibble_value(qx[(size_t)m * KB + k / 2], k & 1) *
               nibble_value(Wq[(size_t)n * KB + k / 2], k & 1);
        }
        main += (double)sx[(size_t)m * G + g] * (double)w_scales[(size_t)n * G + g] * (double)p;
      }
      double low = 0.0;
      for (int j = 0; j < r; ++j)
        low += T[(size_t)m * r + j] * (double)bf16_to_float(L2[(size_t)n * r + j]);
      double y = main + low;
      if (bias) y += (double)bf16_to_float(bias[n]);
      Y[(size_t)m * N + n] = act == 1 ? oref_gelu_tanh(y) : y;
    }
  free(qx); free(sx); free(T);
  return 0;
}

/* Fold a LoRA (A [K, rl] down, B [rl, N] up; the term X A B) into the branch
 * without touching Q(R) ([Abs]): x_hat (diag(s) A) B = X A B, so
 *   L1' = [L1 ; bf16((diag(s) A)^T)]  [r + rl, K],   L2' = [L2 | bf16(B^T)]  [N, r + rl]. */
int oref_append_lora(const float* s, const uint16_t* L1, const uint16_t* L2, int K, int N, int r,
                     const float* A, const float* B, int rl, uint16_t* L1o, uint16_t* L2o) {
  if (K <= 0 || N <= 0 || r < 0 || rl < 0) return -1;
  for (int j = 0; j < r; ++j)
    for (int k = 0; k < K; ++k) L1o[(size_t)j * K + k] = L1[(size_t)j * K + k];
  for (int j = 0; j < rl; ++j)
    for (int k = 0; k < K; ++k)
      L1o[(size_t)(r + j) * K + k] = oref_bf16_from_double((double)A[(size_t)k * rl + j] * (double)s[k]);
  for (int n = 0; n < N; ++n) {
    for (int j = 0; j < r; ++j) L2o[(size_t)n * (r + rl) + j] = L2[(size_t)n * r + j];
    for (int j = 0; j < rl; ++j)
      L2o[(size_t)n * (r + rl) + r + j] = oref_bf16_from_double((double)B[(size_t)j * N + n]);
  }
  return 0;
}

/* --------------------------------------------------------- MXFP4 variant */

static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Index of the E2M1 magnitude nearest to y >= 0; a tie goes to the even index
 * (ties to even on the one significand bit); beyond 6 saturates to 6. */
int oref_e2m1_round(double y) {
  int best = 0;
  double bd = fabs(y - kE2M1[0]);
  for (int i = 1; i < 8; ++i) {
    const double d = fabs(y - kE2M1[i]);
    if (d < bd || (d == bd && i % 2 == 0)) {
      best = i;
      bd = d;
    }
  }
  return best;
}

/* The block's shared exponent: floor(log2 amax) - 2 (2 is the exponent of
 * E2M1's largest value 6 = 1.5 * 2^2), clipped to E8M0's [-127, 127]; an
 * all-zero block gets -127. */
int oref_mx_shared_exponent(double amax) {
  if (!(amax > 0)) return -127;
  int ex;
  frexp(amax, &ex);                 /* amax in [2^(ex-1), 2^ex) */
  int e = ex - 1 - 2;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* MXFP4 of float rows [rows, K]: 4-bit patterns codes [rows, K] (bit 3 the
 * sign of the input, bits 0-2 the magnitude index) and E8M0 bytes e + 127
 * [rows, K / 32], e = floor(log2 amax) - 2 clipped to [-127, 127], an all-zero
 * block -127. */
int oref_quantize_mx(const float* v, int rows, int K, uint8_t* codes, uint8_t* e8m0) {
  if (rows < 0 || K <= 0 || K % MX_BLOCK) return -1;
  const int NB = K / MX_BLOCK;
  for (int m = 0; m < rows; ++m)
    for (int b = 0; b < NB; ++b) {
      const float* x = v + (size_t)m * K + (size_t)b * MX_BLOCK;
      double amax = 0.0;
      for (int i = 0; i < MX_BLOCK; ++i)
        if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
      const int e = oref_mx_shared_exponent(amax);
      e8m0[(size_t)m * NB + b] = (uint8_t)(e + 127);
      for (int i = 0; i < MX_BLOCK; ++i) {
        const double y = ldexp(fabs((double)x[i]), -e);   /* exact */
        const int idx = oref_e2m1_round(y);
        codes[(size_t)m * K + (size_t)b * MX_BLOCK + i] = (uint8_t)(idx | (signbit(x[i]) ? 8 : 0));
      }
    }
  return 0;
}

/* Stage three with MXFP4: Wq packed [N, K / 2] (even channel in the low
 * nibble) and E8M0 bytes w_e8m0 [N, K / 32] of R = W diag(s) - L2 L1. */
int oref_quantize_residual_mx(const float* W, int N, int K, const float* s, const uint16_t* L1,
                              const uint16_t* L2, int r, uint8_t* Wq, uint8_t* w_e8m0) {
  if (N <= 0 || K <= 0 || K % GROUP || r < 0) return -1;
  double* What = (double*)malloc(sizeof(double) * (size_t)N * K);
  float* R = (float*)malloc(sizeof(float) * (size_t)N * K);
  uint8_t* c = (uint8_t*)malloc((size_t)N * K);
  int rc = -1;
  if (What && R && c) {
    oref_smooth_weight(W, N, K, s, What);
    oref_residual(What, N, K, L1, L2, r, R);
    oref_quantize_mx(R, N, K, c, w_e8m0);
    for (size_t i = 0; i < (size_t)N * K / 2; ++i) Wq[i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    rc = 0;
  }
  free(What); free(R); free(c);
  return rc;
}

/* The MXFP4 first half of E4: packed codes qx [M, K / 2] and E8M0 bytes
 * [M, K / 32] of x_hat, and T = x_hat L1^T [M, r] in double (k ascending). */
int oref_quantize_activations_mx(const uint16_t* X, int M, int K, const float* s,
                                 const uint16_t* L1, int r, uint8_t* qx, uint8_t* e8m0,
                                 double* T) {
  if (M < 0 || K <= 0 || K % GROUP || r < 0) return -1;
  float* xh = (float*)malloc(sizeof(float) * ((size_t)M * K + 1));
  uint8_t* c = (uint8_t*)malloc((size_t)M * K + 1);
  if (!xh || !c) {
    free(xh); free(c);
    return -1;
  }
  oref_smooth_activations(X, M, K, s, xh);
  oref_quantize_mx(xh, M, K, c, e8m0);
  for (size_t i = 0; i < (size_t)M * K / 2; ++i) qx[i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
  for (int m = 0; m < M; ++m)
    for (int j = 0; j < r; ++j) {
      double t = 0.0;
      for (int k = 0; k < K; ++k)
        t += (double)xh[(size_t)m * K + k] * (double)bf16_to_float(L1[(size_t)j * K + k]);
      T[(size_t)m * r + j] = t;
    }
  free(xh); free(c);
  return 0;
}

/* Value of a 4-bit E2M1 pattern: bit 3 the sign, bits 0-2 the magnitude index. */
double oref_e2m1_value(int code) {
  const double mag = kE2M1[code & 7];
  return code & 8 ? -mag : mag;
}

/* The MXFP4 forward for rows [m0, m1), in double:
 *   Y[m, n] = sum_b 2^(ea[m, b] + eb[n, b]) (a_b . w_b) + sum_j T[m, j] L2[n, j] + b[n],
 * a_b and w_b the E2M1 values of block b; Wq packed [N, K / 2], w_e8m0 [N, K / 32]
 * row-major. */
int oref_forward_mx_rows(const uint16_t* X, int M, int K, int N, int r, const float* s,
                         const uint16_t* L1, const uint16_t* L2, const uint8_t* Wq,
                         const uint8_t* w_e8m0, const uint16_t* bias, int act, int m0, int m1,
                         double* Y) {
  if (M < 0 || K <= 0 || K % GROUP || N <= 0 || r < 0 || m0 < 0 || m1 > M || m0 > m1) return -1;
  const int rows = m1 - m0, NB = K / MX_BLOCK, KB = K / 2;
  float* xh = (float*)malloc(sizeof(float) * ((size_t)rows * K + 1));
  uint8_t* ca = (uint8_t*)malloc((size_t)rows * K + 1);
  uint8_t* ea = (uint8_t*)malloc((size_t)rows * NB + 1);
  double* T = (double*)malloc(sizeof(double) * ((size_t)r + 1));
  if (!xh || !ca || !ea || !T) {
    free(xh); free(ca); free(ea); free(T);
    return -1;
  }
  oref_smooth_activations(X + (size_t)m0 * K, rows, K, s, xh);
  oref_quantize_mx(xh, rows, K, ca, ea);
  for (int m = 0; m < rows; ++m) {
    /* lora_down of this row: T = x_hat L1^T, k ascending */
    for (int j = 0; j < r; ++j) {
      double t = 0.0;
      for (int k = 0; k < K; ++k)
        t += (double)xh[(size_t)m * K + k] * (double)bf16_to_float(L1[(size_t)j * K + k]);
      T[j] = t;
    }
    for (int n = 0; n < N; ++n) {
      double main = 0.0;
      for (int b = 0; b < NB; ++b) {
        double dot = 0.0;
        for (int i = 0; i < MX_BLOCK; ++i) {
          const int k = b * MX_BLOCK + i;
          const uint8_t wb = Wq[(size_t)n * KB + k / 2];
          const uint8_t wc = (uint8_t)(k & 1 ? wb >> 4 : wb & 0xF);
          dot += oref_e2m1_value(ca[(size_t)m * K + k]) * oref_e2m1_value(wc);
        }
        const int e = (int)ea[(size_t)m * NB + b] - 127 + (int)w_e8m0[(size_t)n * NB + b] - 127;
        main += ldexp(dot, e);
      }
      double low = 0.0;
      for (int j = 0; j < r; ++j) low += T[j] * (double)bf16_to_float(L2[(size_t)n * r + j]);
      double y = main + low;
      if (bias) y += (double)bf16_to_float(bias[n]);
      Y[(size_t)m * N + n] = act == 1 ? oref_gelu_tanh(y) : y;
    }
  }
  free(xh); free(ca); free(ea); free(T);
  return 0;
}
