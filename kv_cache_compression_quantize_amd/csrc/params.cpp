// Host-side parameter builders of libaqkv.so: the Lloyd-Max codebook for a
// rotated unit-vector coordinate and the random orthogonal rotation.
//
// TurboQuant article §二: after normalisation and a random orthogonal
// rotation (made by a QR decomposition, one seed per layer) every coordinate
// follows the same scaled-Beta law; the (b-1)-bit quantiser is the continuous
// 1-D k-means (Lloyd-Max) solution for it, computed offline.
//
// The law of one coordinate t of a uniform unit vector in R^d:
//   f_d(t) = (1 - t^2)^((d-3)/2) / B(1/2, (d-1)/2),  t in [-1, 1],
// i.e. (1 + t) / 2 ~ Beta(a, a) with a = (d - 1) / 2.  Cell probabilities use
// the regularised incomplete beta function, evaluated by its continued
// fraction (DLMF 8.17.22) with the modified Lentz method; the first moment of
// a cell has the closed form [(1-u^2)^(a'+1) - (1-v^2)^(a'+1)] / (2 (a'+1) B)
// with a' = (d-3)/2.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/aqkv.h"

namespace {

// Continued fraction of I_x(a, b) (valid, fast convergence for x < (a+1)/(a+b+2)).
double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  double c = 1.0;
  double dd = 1.0 - (a + b) * x / (a + 1.0);
  if (fabs(dd) < tiny) dd = tiny;
  dd = 1.0 / dd;
  double h = dd;
  for (int k = 1; k < 100000; ++k) {
    const double kk = static_cast<double>(k);
    // even step: d_{2k} = k (b - k) x / ((a + 2k - 1)(a + 2k))
    double num = kk * (b - kk) * x / ((a + 2 * kk - 1) * (a + 2 * kk));
    dd = 1.0 + num * dd;
    if (fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    h *= dd * c;
    // odd step: d_{2k+1} = -(a + k)(a + b + k) x / ((a + 2k)(a + 2k + 1))
    num = -(a + kk) * (a + b + kk) * x / ((a + 2 * kk) * (a + 2 * kk + 1));
    dd = 1.0 + num * dd;
    if (fabs(dd) < tiny) dd = tiny;
    c = 1.0 + num / c;
    if (fabs(c) < tiny) c = tiny;
    dd = 1.0 / dd;
    const double del = dd * c;
    h *= del;
    if (fabs(del - 1.0) < 1e-16) break;
  }
  return h;
}

// Regularised incomplete beta I_x(a, b).
double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lfront = lgamma(a + b) - lgamma(a) - lgamma(b) + a * log(x) + b * log1p(-x);
  if (x < (a + 1.0) / (a + b + 2.0)) return exp(lfront) * beta_cf(a, b, x) / a;
  return 1.0 - exp(lfront) * beta_cf(b, a, 1.0 - x) / b;
}

struct SphereCoordinate {
  int d;
  double a;       // (d - 1) / 2, Beta parameter of (1 + t) / 2
  double log_b;   // log B(1/2, (d-1)/2)
  explicit SphereCoordinate(int dim) : d(dim), a((dim - 1) / 2.0) {
    log_b = lgamma(0.5) + lgamma(a) - lgamma(a + 0.5);
  }
  double cdf(double t) const {
    if (t <= -1.0) return 0.0;
    if (t >= 1.0) return 1.0;
    return inc_beta(a, a, 0.5 * (1.0 + t));
  }
  // int_u^v t f_d(t) dt
  double first_moment(double u, double v) const {
    const double e = (d - 3) / 2.0 + 1.0;
    u = fmax(-1.0, fmin(1.0, u));
    v = fmax(-1.0, fmin(1.0, v));
    const double fu = pow(1.0 - u * u, e), fv = pow(1.0 - v * v, e);
    return (fu - fv) / (2.0 * e) * exp(-log_b);
  }
};

// Inverse of the cdf by bisection (only used for the start point).
double cdf_inverse(const SphereCoordinate &f, double p) {
  double lo = -1.0, hi = 1.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (f.cdf(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

}  // namespace

extern "C" {

aqkv_status aqkv_build_codebook(int32_t head_dim, int32_t bits, float *centroids, float *boundaries) {
  if (!centroids || !boundaries) return AQKV_ERR_NULL;
  if (bits < 1 || bits > 4 || head_dim < 3 || head_dim > 4096) return AQKV_ERR_SHAPE;
  const SphereCoordinate f(head_dim);
  const int L = 1 << bits;
  std::vector<double> c(L), cn(L), edges(L + 1);
  for (int k = 0; k < L; ++k) c[k] = cdf_inverse(f, (k + 0.5) / L);
  for (int it = 0; it < 400000; ++it) {
    edges[0] = -1.0;
    edges[L] = 1.0;
    for (int k = 1; k < L; ++k) edges[k] = 0.5 * (c[k - 1] + c[k]);
    double prev = 0.0;
    for (int k = 0; k < L; ++k) {
      const double cum = f.cdf(edges[k + 1]);
      const double mass = cum - prev;
      prev = cum;
      cn[k] = f.first_moment(edges[k], edges[k + 1]) / mass;
    }
    // the law is even: keep the iterate odd-symmetric
    double delta = 0.0;
    for (int k = 0; k < L; ++k) {
      const double s = 0.5 * (cn[k] - cn[L - 1 - k]);
      delta = fmax(delta, fabs(s - c[k]));
      c[k] = s;
    }
    if (delta < 1e-15) break;
  }
  for (int k = 0; k < L; ++k) centroids[k] = static_cast<float>(c[k]);
  for (int k = 1; k < L; ++k) boundaries[k - 1] = static_cast<float>(0.5 * (c[k - 1] + c[k]));
  return AQKV_OK;
}

aqkv_status aqkv_build_hadamard_rotation(int32_t d, const double *gaussian, float *rotation) {
  if (!gaussian || !rotation) return AQKV_ERR_NULL;
  if (d < 1 || d > 4096 || (d & (d - 1))) return AQKV_ERR_SHAPE;
  // Sylvester's H_ij = (-1)^popcount(i & j), columns flipped by the signs of the
  // first Gaussian row, scaled by 1/sqrt(d)
  const double a = 1.0 / sqrt(static_cast<double>(d));
  for (int32_t i = 0; i < d; ++i)
    for (int32_t j = 0; j < d; ++j) {
      const double h = (__builtin_popcount(static_cast<unsigned>(i & j)) & 1) ? -a : a;
      rotation[static_cast<size_t>(i) * d + j] = static_cast<float>(gaussian[j] >= 0.0 ? h : -h);
    }
  return AQKV_OK;
}

aqkv_status aqkv_build_rotation(int32_t d, const double *gaussian, float *rotation) {
  if (!gaussian || !rotation) return AQKV_ERR_NULL;
  if (d < 1 || d > 4096) return AQKV_ERR_SHAPE;
  const size_t n = static_cast<size_t>(d);
  // Householder QR of A (column operations on a column-major copy).
  std::vector<double> A(n * n);          // A[col * n + row]
  for (size_t r = 0; r < n; ++r)
    for (size_t c = 0; c < n; ++c) A[c * n + r] = gaussian[r * n + c];
  std::vector<double> V(n * n, 0.0);     // Householder vectors, column k in V[k*n ...]
  std::vector<double> rdiag(n);
  for (size_t k = 0; k < n; ++k) {
    double *x = &A[k * n];
    double norm2 = 0.0;
    for (size_t i = k; i < n; ++i) norm2 += x[i] * x[i];
    const double norm = sqrt(norm2);
    const double alpha = x[k] >= 0.0 ? -norm : norm;   // R_kk
    double *v = &V[k * n];
    for (size_t i = k; i < n; ++i) v[i] = x[i];
    v[k] -= alpha;
    double vn2 = 0.0;
    for (size_t i = k; i < n; ++i) vn2 += v[i] * v[i];
    rdiag[k] = alpha;
    if (vn2 == 0.0) continue;                          // column already reduced
    const double inv = 1.0 / sqrt(vn2);
    for (size_t i = k; i < n; ++i) v[i] *= inv;
    // apply H = I - 2 v v^T to the remaining columns
    for (size_t c = k; c < n; ++c) {
      double *col = &A[c * n];
      double dot = 0.0;
      for (size_t i = k; i < n; ++i) dot += v[i] * col[i];
      dot *= 2.0;
      for (size_t i = k; i < n; ++i) col[i] -= dot * v[i];
    }
  }
  // Q = H_0 H_1 ... H_{n-1}: apply to the identity from the last reflector down.
  std::vector<double> Q(n * n, 0.0);     // column-major
  for (size_t i = 0; i < n; ++i) Q[i * n + i] = 1.0;
  for (size_t kk = n; kk-- > 0;) {
    const double *v = &V[kk * n];
    double vn2 = 0.0;
    for (size_t i = kk; i < n; ++i) vn2 += v[i] * v[i];
    if (vn2 == 0.0) continue;
    for (size_t c = 0; c < n; ++c) {
      double *col = &Q[c * n];
      double dot = 0.0;
      for (size_t i = kk; i < n; ++i) dot += v[i] * col[i];
      dot *= 2.0;
      for (size_t i = kk; i < n; ++i) col[i] -= dot * v[i];
    }
  }
  // Pi = Q diag(sign(R_kk)): the QR factor with a positive diagonal R (Haar).
  for (size_t r = 0; r < n; ++r)
    for (size_t c = 0; c < n; ++c) {
      const double s = rdiag[c] < 0.0 ? -1.0 : 1.0;
      rotation[r * n + c] = static_cast<float>(Q[c * n + r] * s);
    }
  return AQKV_OK;
}

}  // extern "C"
