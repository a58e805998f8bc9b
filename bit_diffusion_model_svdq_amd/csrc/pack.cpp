// Offline packer of the SVDQuant linear layer (host, float64).
//
// The three stages of the SVDQuant Terminology Entry (section 2.1), in order:
//   1. outlier migration: s from activation and weight statistics (E2) and the
//      smoothed weight W_hat = W diag(s) (E1);
//   2. low-rank decomposition: the rank-r truncated SVD of W_hat (E3), the best
//      rank-r approximation by Eckart-Young (E5);
//   3. residual quantization: R = W_hat - L2 L1 in 4 bits, one scale per 64.
//
// The truncated SVD is computed from the Gram matrix of the smaller side:
// its eigenvalues are sigma^2 and its eigenvectors are one set of singular
// vectors; the other set follows as W_hat v / sigma (or W_hat^T u / sigma).
// The symmetric eigenproblem is solved by Householder reduction to
// tridiagonal form, Sturm-sequence bisection for the eigenvalues and inverse
// iteration for the r leading eigenvectors (Golub & Van Loan, "Matrix
// Computations", sections 8.3.1, 8.4.1 and 8.2.2).  Squaring the matrix costs
// relative accuracy only for singular values far below sigma_1, which the
// rank-r branch does not keep.
#include <math.h>
#include <cmath>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "svdq.h"
#include "svdq_errors.h"

namespace {

using svdq::fail;

constexpr int kGroup = 64;
constexpr double kStatFloor = 1e-5;

// bfloat16 nearest-even from a float64 value, with a single rounding.
uint16_t bf16_from_double(double v) {
  if (v == 0.0) return signbit(v) ? 0x8000 : 0;
  const uint16_t sign = v < 0 ? 0x8000 : 0;
  const double a = fabs(v);
  int e;
  frexp(a, &e);                      // a in [2^(e-1), 2^e)
  const int lead = std::max(e - 1, -126);
  const double ulp = ldexp(1.0, lead - 7);
  const double q = a / ulp;          // exact (power-of-two scaling)
  double rq = floor(q);
  const double frac = q - rq;
  if (frac > 0.5 || (frac == 0.5 && fmod(rq, 2.0) == 1.0)) rq += 1.0;
  const double val = rq * ulp;
  if (val >= ldexp(1.0, 128)) return sign | 0x7F80;
  const float f = (float)val;        // exact: val is a bfloat16 value
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return sign | (uint16_t)(bits >> 16);
}

double bf16_to_double(uint16_t b) {
  const uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

// ------------------------------------------------------------- eigensolver
// Householder tridiagonalization of the symmetric n x n matrix A (row-major,
// overwritten).  On return d[0..n) is the diagonal, e[0..n-1) the
// off-diagonal, and reflector k is I - beta[k] h_k h_k^T acting on rows
// k+1..n-1 with h_k stored in H[k] (h_k[0] = 1).
struct Tridiag {
  std::vector<double> d, e, beta;
  std::vector<std::vector<double>> H;
};

void tridiagonalize(std::vector<double>& A, int n, Tridiag& t) {
  t.d.assign(n, 0.0);
  t.e.assign(n > 1 ? n - 1 : 0, 0.0);
  t.beta.assign(n > 2 ? n - 2 : 0, 0.0);
  t.H.assign(n > 2 ? n - 2 : 0, std::vector<double>());
  std::vector<double> p(n), w(n);
  for (int k = 0; k + 2 < n; ++k) {
    const int m = n - k - 1;
    std::vector<double>& h = t.H[k];
    h.resize(m);
    for (int i = 0; i < m; ++i) h[i] = A[(size_t)(k + 1 + i) * n + k];
    double sigma = 0.0;
    for (int i = 1; i < m; ++i) sigma += h[i] * h[i];
    const double x0 = h[0];
    double beta = 0.0, alpha = x0;
    if (sigma != 0.0) {
      const double mu = sqrt(x0 * x0 + sigma);
      const double v0 = x0 <= 0.0 ? x0 - mu : -sigma / (x0 + mu);
      beta = 2.0 * v0 * v0 / (sigma + v0 * v0);
      for (int i = 1; i < m; ++i) h[i] /= v0;
      alpha = mu;
    } else {
      for (int i = 1; i < m; ++i) h[i] = 0.0;
    }
    h[0] = 1.0;
    t.beta[k] = beta;
    t.d[k] = A[(size_t)k * n + k];
    t.e[k] = alpha;
    if (beta == 0.0) continue;
    // p = beta * A' h over the trailing block
#pragma omp parallel for schedule(static)
    for (int i = 0; i < m; ++i) {
      const double* row = &A[(size_t)(k + 1 + i) * n + (k + 1)];
      double s = 0.0;
      for (int j = 0; j < m; ++j) s += row[j] * h[j];
      p[i] = beta * s;
    }
    double ph = 0.0;
    for (int i = 0; i < m; ++i) ph += p[i] * h[i];
    const double kk = 0.5 * beta * ph;
    for (int i = 0; i < m; ++i) w[i] = p[i] - kk * h[i];
    // A' -= h w^T + w h^T
#pragma omp parallel for schedule(static)
    for (int i = 0; i < m; ++i) {
      double* row = &A[(size_t)(k + 1 + i) * n + (k + 1)];
      const double hi = h[i], wi = w[i];
      for (int j = 0; j < m; ++j) row[j] -= hi * w[j] + wi * h[j];
    }
  }
  if (n >= 2) {
    t.d[n - 2] = A[(size_t)(n - 2) * n + (n - 2)];
    t.e[n - 2] = A[(size_t)(n - 1) * n + (n - 2)];
  }
  t.d[n - 1] = A[(size_t)(n - 1) * n + (n - 1)];
}

// Number of eigenvalues of the tridiagonal (d, e) that are < x (Sturm count).
int sturm_count(const std::vector<double>& d, const std::vector<double>& e2, double x,
                double pivmin) {
  const int n = (int)d.size();
  int cnt = 0;
  double q = d[0] - x;
  if (fabs(q) < pivmin) q = -pivmin;
  if (q < 0) ++cnt;
  for (int i = 1; i < n; ++i) {
    q = d[i] - x - e2[i - 1] / q;
    if (fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++cnt;
  }
  return cnt;
}

// All eigenvalues in descending order, by bisection.
void eigenvalues_bisect(const Tridiag& t, std::vector<double>& lam) {
  const int n = (int)t.d.size();
  std::vector<double> e2(n > 1 ? n - 1 : 0);
  double lo = t.d[0], hi = t.d[0], emax = 0.0;
  for (int i = 0; i < n; ++i) {
    const double r = (i > 0 ? fabs(t.e[i - 1]) : 0.0) + (i + 1 < n ? fabs(t.e[i]) : 0.0);
    lo = std::min(lo, t.d[i] - r);
    hi = std::max(hi, t.d[i] + r);
  }
  for (int i = 0; i + 1 < n; ++i) {
    e2[i] = t.e[i] * t.e[i];
    emax = std::max(emax, fabs(t.e[i]));
  }
  const double scale = std::max(fabs(lo), fabs(hi));
  const double pivmin = std::max(1e-300, scale * 1e-300) + emax * emax * 2.2e-308;
  lo -= 4.0 * 2.2e-16 * scale + 1e-300;
  hi += 4.0 * 2.2e-16 * scale + 1e-300;
  lam.assign(n, 0.0);
#pragma omp parallel for schedule(dynamic, 16)
  for (int j = 0; j < n; ++j) {
    // the (j+1)-th largest eigenvalue: count(< x) <= n-1-j  <=>  x <= lambda
    const int want = n - 1 - j;
    double a = lo, b = hi;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (a + b);
      if (mid == a || mid == b) break;
      if (sturm_count(t.d, e2, mid, pivmin) <= want)
        a = mid;
      else
        b = mid;
      if (b - a <= 2.2e-16 * std::max(fabs(a), fabs(b)) + 1e-300) break;
    }
    lam[j] = 0.5 * (a + b);
  }
}

// Solves (T - lambda I) x = b in place for the tridiagonal T by Gaussian
// elimination with partial pivoting; zero pivots are replaced by `tiny`.
void tridiag_solve(const Tridiag& t, double lambda, double tiny, std::vector<double>& b) {
  const int n = (int)t.d.size();
  std::vector<double> diag(n), sup(n), sub(n);
  for (int i = 0; i < n; ++i) {
    diag[i] = t.d[i] - lambda;
    sup[i] = i + 1 < n ? t.e[i] : 0.0;
    sub[i] = i > 0 ? t.e[i - 1] : 0.0;
  }
  // elimination producing an upper band with two super-diagonals
  std::vector<double> U0(n), U1(n), U2(n);
  double cd = diag[0], cs = sup[0], cs2 = 0.0;  // current row (diag, sup, sup2)
  for (int i = 0; i < n; ++i) {
    if (i + 1 < n) {
      const double nsub = sub[i + 1], ndiag = diag[i + 1], nsup = i + 2 < n ? sup[i + 1] : 0.0;
      if (fabs(nsub) > fabs(cd)) {  // swap rows i and i+1
        const double m = cd / nsub;
        U0[i] = nsub;
        U1[i] = ndiag;
        U2[i] = nsup;
        std::swap(b[i], b[i + 1]);
        b[i + 1] -= m * b[i];
        const double r_d = cs - m * ndiag, r_s = cs2 - m * nsup;
        cd = r_d;
        cs = r_s;
        cs2 = 0.0;
      } else {
        double piv = cd;
        if (fabs(piv) < tiny) piv = piv < 0 ? -tiny : tiny;
        const double m = nsub / piv;
        U0[i] = piv;
        U1[i] = cs;
        U2[i] = cs2;
        b[i + 1] -= m * b[i];
        cd = ndiag - m * cs;
        cs = nsup - m * cs2;
        cs2 = 0.0;
      }
    } else {
      double piv = cd;
      if (fabs(piv) < tiny) piv = piv < 0 ? -tiny : tiny;
      U0[i] = piv;
      U1[i] = 0.0;
      U2[i] = 0.0;
    }
  }
  for (int i = n - 1; i >= 0; --i) {
    double s = b[i];
    if (i + 1 < n) s -= U1[i] * b[i + 1];
    if (i + 2 < n) s -= U2[i] * b[i + 2];
    b[i] = s / U0[i];
  }
}

// ||T y - lambda y||_2 for the tridiagonal T.
double tridiag_residual(const Tridiag& t, double lambda, const std::vector<double>& y) {
  const int n = (int)t.d.size();
  double ss = 0.0;
  for (int i = 0; i < n; ++i) {
    double v = (t.d[i] - lambda) * y[i];
    if (i > 0) v += t.e[i - 1] * y[i - 1];
    if (i + 1 < n) v += t.e[i] * y[i + 1];
    ss += v * v;
  }
  return sqrt(ss);
}

// Inverse iteration: kMinSweeps sweeps (each one multiplies the wanted
// component by |lambda_i - shift| / |lambda_j - shift| against every other,
// which after six solves leaves the vectors of small, close eigenvalues
// accurate too), then more until the eigen-residual ||T y - lambda y|| of the
// normalized iterate is below kResidualTol * ||T||, at most kMaxSweeps.  A
// vector whose eigenvalue lies within `cluster` of an earlier one is
// re-orthogonalized against that one after every solve, so a repeated
// eigenvalue yields an orthonormal basis of its eigenspace.
constexpr int kMinSweeps = 6;
constexpr int kMaxSweeps = 40;
constexpr double kResidualTol = 1e-11;

// Leading r eigenvectors of the original matrix (columns of Z, n x r row-major)
// for eigenvalues lam[0..r) (descending).  Returns false when an iterate stops
// being finite or the residual test is not met within kMaxSweeps sweeps.
bool eigenvectors(const Tridiag& t, const std::vector<double>& lam, int r,
                  std::vector<double>& Z) {
  const int n = (int)t.d.size();
  double tnorm = 0.0;
  for (int i = 0; i < n; ++i)
    tnorm = std::max(tnorm, fabs(t.d[i]) + (i > 0 ? fabs(t.e[i - 1]) : 0.0) +
                                (i + 1 < n ? fabs(t.e[i]) : 0.0));
  if (!isfinite(tnorm)) return false;
  if (tnorm == 0.0) tnorm = 1.0;
  const double tiny = 2.2e-16 * tnorm;
  const double cluster = 1e-3 * tnorm;
  std::vector<std::vector<double>> Y(r, std::vector<double>(n));
  for (int j = 0; j < r; ++j) {
    std::vector<double>& y = Y[j];
    for (int i = 0; i < n; ++i)  // deterministic, non-degenerate start
      y[i] = 1.0 + 0.5 * sin(1.0 + 0.7 * i + 1.3 * j);
    const double shift = lam[j] + 4.0 * tiny * (1 + (j % 3));
    bool converged = false;
    for (int it = 0; it < kMaxSweeps && !converged; ++it) {
      tridiag_solve(t, shift, tiny, y);
      // orthogonalize against earlier vectors of the same cluster
      for (int q = 0; q < j; ++q) {
        if (fabs(lam[q] - lam[j]) > cluster) continue;
        double dot = 0.0;
        for (int i = 0; i < n; ++i) dot += Y[q][i] * y[i];
        for (int i = 0; i < n; ++i) y[i] -= dot * Y[q][i];
      }
      double nrm = 0.0;
      for (int i = 0; i < n; ++i) nrm += y[i] * y[i];
      nrm = sqrt(nrm);
      if (!(nrm > 0.0) || !isfinite(nrm)) return false;
      for (int i = 0; i < n; ++i) y[i] /= nrm;
      converged = it + 1 >= kMinSweeps && tridiag_residual(t, lam[j], y) <= kResidualTol * tnorm;
    }
    if (!converged) return false;
  }
  // back-transform with the reflectors, last one first
  Z.assign((size_t)n * r, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < r; ++j) {
    std::vector<double> y = Y[j];
    for (int k = (int)t.H.size() - 1; k >= 0; --k) {
      const double beta = t.beta[k];
      if (beta == 0.0) continue;
      const std::vector<double>& h = t.H[k];
      const int m = (int)h.size();
      double s = 0.0;
      for (int i = 0; i < m; ++i) s += h[i] * y[k + 1 + i];
      s *= beta;
      for (int i = 0; i < m; ++i) y[k + 1 + i] -= s * h[i];
    }
    for (int i = 0; i < n; ++i) Z[(size_t)i * r + j] = y[i];
  }
  return true;
}

// Gm = Rm Rm^T for Rm [d, o] row-major (lower triangle computed, then mirrored).
// Blocked: 64-row panels of both operands, 256-column chunks, 4x4 micro-tiles.
void gram(const std::vector<double>& Rm, int d, int o, std::vector<double>& Gm) {
  constexpr int PB = 64, OC = 256;
  const int np = (d + PB - 1) / PB;
  std::vector<std::pair<int, int>> pairs;
  for (int a = 0; a < np; ++a)
    for (int b = 0; b <= a; ++b) pairs.push_back({a, b});
#pragma omp parallel for schedule(dynamic, 1)
  for (size_t pi = 0; pi < pairs.size(); ++pi) {
    const int a0 = pairs[pi].first * PB, b0 = pairs[pi].second * PB;
    const int a1 = std::min(a0 + PB, d), b1 = std::min(b0 + PB, d);
    double acc[PB][PB];
    for (int i = 0; i < PB; ++i)
      for (int j = 0; j < PB; ++j) acc[i][j] = 0.0;
    for (int c0 = 0; c0 < o; c0 += OC) {
      const int c1 = std::min(c0 + OC, o);
      for (int a = a0; a < a1; a += 4) {
        for (int b = b0; b < b1; b += 4) {
          double t[4][4] = {};
          const double* ra[4];
          const double* rb[4];
          for (int x = 0; x < 4; ++x) {
            ra[x] = &Rm[(size_t)std::min(a + x, d - 1) * o];
            rb[x] = &Rm[(size_t)std::min(b + x, d - 1) * o];
          }
          for (int c = c0; c < c1; ++c) {
            const double va0 = ra[0][c], va1 = ra[1][c], va2 = ra[2][c], va3 = ra[3][c];
            const double vb0 = rb[0][c], vb1 = rb[1][c], vb2 = rb[2][c], vb3 = rb[3][c];
            t[0][0] += va0 * vb0; t[0][1] += va0 * vb1; t[0][2] += va0 * vb2; t[0][3] += va0 * vb3;
            t[1][0] += va1 * vb0; t[1][1] += va1 * vb1; t[1][2] += va1 * vb2; t[1][3] += va1 * vb3;
            t[2][0] += va2 * vb0; t[2][1] += va2 * vb1; t[2][2] += va2 * vb2; t[2][3] += va2 * vb3;
            t[3][0] += va3 * vb0; t[3][1] += va3 * vb1; t[3][2] += va3 * vb2; t[3][3] += va3 * vb3;
          }
          for (int x = 0; x < 4; ++x)
            for (int y = 0; y < 4; ++y)
              if (a + x < a1 && b + y < b1) acc[a + x - a0][b + y - b0] += t[x][y];
        }
      }
    }
    for (int i = a0; i < a1; ++i)
      for (int j = b0; j < b1; ++j) {
        Gm[(size_t)i * d + j] = acc[i - a0][j - b0];
        Gm[(size_t)j * d + i] = acc[i - a0][j - b0];
      }
  }
}

// ------------------------------------------------------------ quantization
// Q of one group: scale = fl32(a/7), inv = fl32(7/a), rne codes in [-7, 7];
// the weight scale has its two lowest significand bits cleared.  A group with
// a < 2^-100 is a zero group (scale 0, codes 0): 7/a would near the float32
// overflow, and such values are far below what the output resolves.
constexpr float kTinyGroup = 0x1p-100f;

void quantize_group(const float* v, uint8_t* packed, float* scale_out) {
  float a = 0.f;
  for (int i = 0; i < kGroup; ++i) a = std::max(a, fabsf(v[i]));
  float scale = 0.f, inv = 0.f;
  if (a >= kTinyGroup) {
    scale = a / 7.0f;
    inv = 7.0f / a;
  }
  for (int i = 0; i < kGroup; i += 2) {
    float q0 = nearbyintf(v[i] * inv), q1 = nearbyintf(v[i + 1] * inv);
    q0 = std::min(std::max(q0, -7.0f), 7.0f);
    q1 = std::min(std::max(q1, -7.0f), 7.0f);
    packed[i / 2] = (uint8_t)(((int)q0 & 0xF) | (((int)q1 & 0xF) << 4));
  }
  uint32_t bits;
  memcpy(&bits, &scale, 4);
  bits &= 0xFFFFFFFCu;
  memcpy(&scale, &bits, 4);
  *scale_out = scale;
}

// MXFP4 block of 32 (OCP MX v1.0): E8M0 scale 2^e with e = floor(log2 amax) - 2
// (2 = exponent of E2M1's largest value 6), clamped to [-127, 127], -127 for an
// all-zero block; each element is the nearest E2M1 value of v / 2^e, ties to
// the even significand, saturating at 6, with the sign of v.
constexpr double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

int e2m1_code(float v, int e) {
  const double y = std::ldexp(std::fabs((double)v), -e);   // exact: a power-of-two scaling
  int best = 0;
  double bd = y;
  for (int i = 1; i < 8; ++i) {
    const double d = std::fabs(y - kE2M1[i]);
    if (d < bd || (d == bd && (i & 1) == 0)) {
      best = i;
      bd = d;
    }
  }
  return best | (std::signbit(v) ? 8 : 0);
}

void quantize_block_mx(const float* v, uint8_t* packed, uint8_t* e8m0) {
  float a = 0.f;
  for (int i = 0; i < 32; ++i) a = std::max(a, fabsf(v[i]));
  int e = -127;
  if (a > 0.f) {
    int x = 0;
    std::frexp((double)a, &x);                 // a = m 2^x, m in [0.5, 1): floor(log2 a) = x - 1
    e = std::min(std::max(x - 1 - 2, -127), 127);
  }
  for (int i = 0; i < 32; i += 2)
    packed[i / 2] = (uint8_t)(e2m1_code(v[i], e) | (e2m1_code(v[i + 1], e) << 4));
  *e8m0 = (uint8_t)(e + 127);
}

// R = fl32(W diag(s) - L2 L1) row by row (sum over j ascending in double, from
// the stored bf16 factors), then quantize(R row, n).
template <class Q>
void residual_rows(const float* W, int N, int K, const float* s, const uint16_t* L1,
                   const uint16_t* L2, int r, Q quantize) {
#pragma omp parallel
  {
    std::vector<double> l2row(r);
    std::vector<float> R(K);
#pragma omp for schedule(static)
    for (int n = 0; n < N; ++n) {
      for (int j = 0; j < r; ++j) l2row[j] = bf16_to_double(L2[(size_t)n * r + j]);
      for (int k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int j = 0; j < r; ++j) acc += l2row[j] * bf16_to_double(L1[(size_t)j * K + k]);
        const double what = (double)W[(size_t)n * K + k] * (double)s[k];
        R[k] = (float)(what - acc);
      }
      quantize(R.data(), n);
    }
  }
}

void residual_quantize(const float* W, int N, int K, const float* s, const uint16_t* L1,
                       const uint16_t* L2, int r, uint8_t* Wq, float* w_scales) {
  const int G = K / kGroup;
  residual_rows(W, N, K, s, L1, L2, r, [&](const float* R, int n) {
    for (int g = 0; g < G; ++g)
      quantize_group(&R[(size_t)g * kGroup], Wq + (size_t)n * (K / 2) + g * (kGroup / 2),
                     &w_scales[(size_t)n * G + g]);
  });
}

void residual_quantize_mx(const float* W, int N, int K, const float* s, const uint16_t* L1,
                          const uint16_t* L2, int r, uint8_t* Wq, uint8_t* w_e8m0) {
  const int B = K / 32;
  residual_rows(W, N, K, s, L1, L2, r, [&](const float* R, int n) {
    for (int b = 0; b < B; ++b)
      quantize_block_mx(&R[(size_t)b * 32], Wq + (size_t)n * (K / 2) + b * 16,
                        &w_e8m0[(size_t)n * B + b]);
  });
}

svdq_status check_pack_args(const float* W, int N, int K, const float* smooth, uint8_t* Wq,
                            float* w_scales, int r) {
  if (!W || !smooth || !Wq || !w_scales) return fail(SVDQ_ERR_INVALID_ARG, "NULL buffer");
  if (N < 1) return fail(SVDQ_ERR_INVALID_ARG, "N must be >= 1 (got %d)", N);
  if (K < kGroup || K % kGroup)
    return fail(SVDQ_ERR_INVALID_ARG, "K must be a positive multiple of 64 (got %d)", K);
  if (r < 0 || r > 128 || r % 16)
    return fail(SVDQ_ERR_INVALID_ARG, "rank must be a multiple of 16 in [0, 128] (got %d)", r);
  if (r > std::min(N, K)) return fail(SVDQ_ERR_INVALID_ARG, "rank %d exceeds min(N, K)", r);
  return SVDQ_OK;
}

}  // namespace

extern "C" {

svdq_status svdq_act_absmax_update(const uint16_t* X, int64_t M, int K, float* amax) {
  try {
    if (!X || !amax) return fail(SVDQ_ERR_INVALID_ARG, "NULL buffer");
    if (M < 0 || K < 1) return fail(SVDQ_ERR_INVALID_ARG, "bad shape M=%lld K=%d", (long long)M, K);
    for (int64_t m = 0; m < M; ++m)
      for (int k = 0; k < K; ++k) {
        const uint32_t bits = (uint32_t)X[m * K + k] << 16;
        float f;
        memcpy(&f, &bits, 4);
        amax[k] = std::max(amax[k], fabsf(f));
      }
    return SVDQ_OK;
  } catch (...) {
    return fail(SVDQ_ERR_INVALID_ARG, "unexpected C++ exception");
  }
}

svdq_status svdq_quantize_residual(const float* W, int N, int K, const float* smooth,
                                   const uint16_t* L1, const uint16_t* L2, int r, uint8_t* Wq,
                                   float* w_scales) {
  try {
    const svdq_status st = check_pack_args(W, N, K, smooth, Wq, w_scales, r);
    if (st != SVDQ_OK) return st;
    if (r > 0 && (!L1 || !L2)) return fail(SVDQ_ERR_INVALID_ARG, "L1/L2 must not be NULL for r > 0");
    residual_quantize(W, N, K, smooth, L1, L2, r, Wq, w_scales);
    return SVDQ_OK;
  } catch (...) {
    return fail(SVDQ_ERR_INVALID_ARG, "unexpected C++ exception (out of memory?)");
  }
}

svdq_status svdq_quantize_residual_mxfp4(const float* W, int N, int K, const float* smooth,
                                         const uint16_t* L1, const uint16_t* L2, int r,
                                         uint8_t* Wq, uint8_t* w_e8m0) {
  try {
    const svdq_status st =
        check_pack_args(W, N, K, smooth, Wq, reinterpret_cast<float*>(w_e8m0), r);
    if (st != SVDQ_OK) return st;
    if (r > 0 && (!L1 || !L2)) return fail(SVDQ_ERR_INVALID_ARG, "L1/L2 must not be NULL for r > 0");
    residual_quantize_mx(W, N, K, smooth, L1, L2, r, Wq, w_e8m0);
    return SVDQ_OK;
  } catch (...) {
    return fail(SVDQ_ERR_INVALID_ARG, "unexpected C++ exception (out of memory?)");
  }
}

size_t svdq_mxfp4_tiled_scale_bytes(int rows, int K) {
  if (rows < 1 || K < 128 || K % 128) return 0;
  return (size_t)((K + 255) / 256) * rows * 8;
}

svdq_status svdq_mxfp4_tile_scales(const uint8_t* scales, int rows, int K, uint8_t* tiled) {
  if (!scales || !tiled) return fail(SVDQ_ERR_INVALID_ARG, "NULL scales or tiled");
  if (rows < 1 || K < 128 || K % 128)
    return fail(SVDQ_ERR_INVALID_ARG, "rows must be >= 1 and K a positive multiple of 128 (got %d, %d)",
                rows, K);
  const int nb = K / 32;                  // scale bytes per row
  const int nt = (K + 255) / 256;         // 256-channel k-tiles
  for (int t = 0; t < nt; ++t)
    for (int n = 0; n < rows; ++n)
      for (int j = 0; j < 8; ++j) {
        const int b = 8 * t + j;
        tiled[((size_t)t * rows + n) * 8 + j] = b < nb ? scales[(size_t)n * nb + b] : (uint8_t)127;
      }
  return SVDQ_OK;
}

svdq_status svdq_pack_weights(const float* W, int N, int K, const float* act_absmax,
                              const svdq_pack_params* p, float* smooth, uint16_t* L1,
                              uint16_t* L2, uint8_t* Wq, float* w_scales, double* sigma) {
  try {
    if (!p || !act_absmax) return fail(SVDQ_ERR_INVALID_ARG, "NULL params or act_absmax");
    if (p->group != kGroup) return fail(SVDQ_ERR_UNSUPPORTED, "group must be 64 (got %d)", p->group);
    if (!(p->alpha >= 0.f && p->alpha <= 1.f))
      return fail(SVDQ_ERR_INVALID_ARG, "alpha must be in [0, 1]");
    if (!(p->s_min > 0.f)) return fail(SVDQ_ERR_INVALID_ARG, "s_min must be > 0");
    const int r = p->rank;
    svdq_status st = check_pack_args(W, N, K, smooth, Wq, w_scales, r);
    if (st != SVDQ_OK) return st;
    if (r > 0 && (!L1 || !L2)) return fail(SVDQ_ERR_INVALID_ARG, "L1/L2 must not be NULL for r > 0");

    // 1. smoothing factors (E2) and the smoothed weight (E1)
    std::vector<float> s(K);
    for (int k = 0; k < K; ++k) {
      float wsc = 0.f;
      for (int n = 0; n < N; ++n) wsc = std::max(wsc, fabsf(W[(size_t)n * K + k]));
      const double a = std::max((double)act_absmax[k], kStatFloor);
      const double w = std::max((double)wsc, kStatFloor);
      const double sv = pow(a, (double)p->alpha) / pow(w, 1.0 - (double)p->alpha);
      s[k] = (float)std::max(sv, (double)p->s_min);
    }
    std::vector<double> What((size_t)N * K);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k) What[(size_t)n * K + k] = (double)W[(size_t)n * K + k] * (double)s[k];

    // 2. truncated SVD through the Gram matrix of the smaller side
    const bool right = K <= N;  // eigenvectors of W_hat^T W_hat are V
    const int d = right ? K : N;
    const int o = right ? N : K;
    std::vector<uint16_t> l1((size_t)r * K), l2((size_t)N * r);
    if (r > 0 || sigma) {
      // rows of Rm are the columns (right) or rows (left) of W_hat: Gm = Rm Rm^T
      std::vector<double> Rm;
      if (right) {
        Rm.resize((size_t)K * N);
#pragma omp parallel for schedule(static)
        for (int k = 0; k < K; ++k)
          for (int n = 0; n < N; ++n) Rm[(size_t)k * N + n] = What[(size_t)n * K + k];
      } else {
        Rm = What;
      }
      std::vector<double> Gm((size_t)d * d, 0.0);
      gram(Rm, d, o, Gm);
      Tridiag t;
      tridiagonalize(Gm, d, t);
      std::vector<double> lam;
      eigenvalues_bisect(t, lam);
      if (sigma)
        for (int i = 0; i < d; ++i) sigma[i] = sqrt(std::max(lam[i], 0.0));
      if (r > 0) {
        std::vector<double> Z;
        if (!eigenvectors(t, lam, r, Z))
          return fail(SVDQ_ERR_NO_CONVERGENCE, "inverse iteration failed");
        for (int j = 0; j < r; ++j) {
          const double sj = sqrt(std::max(lam[j], 0.0));
          std::vector<double> v(K), u(N);
          if (right) {
            for (int k = 0; k < K; ++k) v[k] = Z[(size_t)k * r + j];
#pragma omp parallel for schedule(static)
            for (int n = 0; n < N; ++n) {
              double acc = 0.0;
              const double* wr = &What[(size_t)n * K];
              for (int k = 0; k < K; ++k) acc += wr[k] * v[k];
              u[n] = sj > 0.0 ? acc / sj : 0.0;
            }
          } else {
            for (int n = 0; n < N; ++n) u[n] = Z[(size_t)n * r + j];
            std::fill(v.begin(), v.end(), 0.0);
            for (int n = 0; n < N; ++n) {
              const double* wr = &What[(size_t)n * K];
              for (int k = 0; k < K; ++k) v[k] += wr[k] * u[n];
            }
            for (int k = 0; k < K; ++k) v[k] = sj > 0.0 ? v[k] / sj : 0.0;
          }
          // sign: the largest-magnitude entry of v_j positive (first one on ties)
          int arg = 0;
          for (int k = 1; k < K; ++k)
            if (fabs(v[k]) > fabs(v[arg])) arg = k;
          const double sg = v[arg] < 0 ? -1.0 : 1.0;
          for (int k = 0; k < K; ++k) l1[(size_t)j * K + k] = bf16_from_double(sg * v[k]);
          for (int n = 0; n < N; ++n) l2[(size_t)n * r + j] = bf16_from_double(sg * sj * u[n]);
        }
      }
    }

    // 3. residual quantization from the rounded factors
    residual_quantize(W, N, K, s.data(), l1.data(), l2.data(), r, Wq, w_scales);
    memcpy(smooth, s.data(), (size_t)K * 4);
    if (r > 0) {
      memcpy(L1, l1.data(), l1.size() * 2);
      memcpy(L2, l2.data(), l2.size() * 2);
    }
    return SVDQ_OK;
  } catch (...) {
    return fail(SVDQ_ERR_INVALID_ARG, "unexpected C++ exception (out of memory?)");
  }
}

svdq_status svdq_append_lora(const float* smooth, int K, int N, const uint16_t* L1,
                             const uint16_t* L2, int r, const float* A, const float* B, int rl,
                             uint16_t* L1_out, uint16_t* L2_out) {
  try {
    if (!smooth || !A || !B || !L1_out || !L2_out) return fail(SVDQ_ERR_INVALID_ARG, "NULL buffer");
    if (K < 1 || N < 1) return fail(SVDQ_ERR_INVALID_ARG, "bad shape K=%d N=%d", K, N);
    if (r < 0 || rl < 1 || r + rl > 128)
      return fail(SVDQ_ERR_INVALID_ARG, "ranks r=%d + rl=%d must stay within 1..128", r, rl);
    if (r > 0 && (!L1 || !L2)) return fail(SVDQ_ERR_INVALID_ARG, "L1/L2 must not be NULL for r > 0");
    const int r2 = r + rl;
    // lora_down rows: the branch's r rows, then (diag(s) A)^T; A[k, j] * s[k] is
    // exact in double, so one rounding to bf16
    if (r > 0) memcpy(L1_out, L1, (size_t)r * K * sizeof(uint16_t));
    for (int j = 0; j < rl; ++j)
      for (int k = 0; k < K; ++k)
        L1_out[(size_t)(r + j) * K + k] =
            bf16_from_double((double)A[(size_t)k * rl + j] * (double)smooth[k]);
    // lora_up rows: [L2 | B^T]
    for (int n = 0; n < N; ++n) {
      if (r > 0) memcpy(L2_out + (size_t)n * r2, L2 + (size_t)n * r, (size_t)r * sizeof(uint16_t));
      for (int j = 0; j < rl; ++j)
        L2_out[(size_t)n * r2 + r + j] = bf16_from_double((double)B[(size_t)j * N + n]);
    }
    return SVDQ_OK;
  } catch (...) {
    return fail(SVDQ_ERR_INVALID_ARG, "unexpected C++ exception");
  }
}

}  // extern "C"
