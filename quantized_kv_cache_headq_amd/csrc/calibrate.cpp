// calibrate.cpp — headq_calibrate: the per-KV-head query-PCA side basis U_h (host, fp64).
//
// HeadQ technical summary ("Technische Samenvatting"), §3 step 1: a rank-r basis U_h per layer
// and head from PCA of post-RoPE calibration queries. Reading taken here: one basis per KV head,
// pooling the g query heads that read it, from the uncentered second moment (1/n) sum q q^T,
// because the score error the side code must cancel is q.e with the raw (uncentered) query.
//
// Eigen-decomposition: Householder reduction to tridiagonal form followed by implicit
// symmetric QR steps with Wilkinson shifts (Golub & Van Loan, "Matrix Computations", §8.3).
#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

#include "headq_internal.h"

namespace headq {

namespace {

// Reduce symmetric A (n x n, row-major, overwritten) to tridiagonal T = Q^T A Q.
// diag[i] = T[i][i], off[i] = T[i+1][i]; Q (row-major) receives the accumulated reflections.
void householder_tridiagonal(int n, std::vector<double>& A, std::vector<double>& diag,
                             std::vector<double>& off, std::vector<double>& Q) {
  Q.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
  std::vector<double> v(n), p(n), w(n);
  for (int k = 0; k + 2 < n; ++k) {
    // reflect x = A[k+1..n-1][k] onto alpha * e_1
    double xnorm2 = 0.0;
    for (int i = k + 1; i < n; ++i) xnorm2 += A[(size_t)i * n + k] * A[(size_t)i * n + k];
    if (xnorm2 == 0.0) continue;
    double x0 = A[(size_t)(k + 1) * n + k];
    double alpha = (x0 > 0 ? -1.0 : 1.0) * std::sqrt(xnorm2);
    std::fill(v.begin(), v.end(), 0.0);
    for (int i = k + 1; i < n; ++i) v[i] = A[(size_t)i * n + k];
    v[k + 1] -= alpha;
    double vv = 0.0;
    for (int i = k + 1; i < n; ++i) vv += v[i] * v[i];
    if (vv == 0.0) continue;
    double beta = 2.0 / vv;
    // p = beta * A v (trailing block), w = p - (beta/2)(p.v) v ; A <- A - v w^T - w v^T
    for (int i = k + 1; i < n; ++i) {
      double s = 0.0;
      for (int j = k + 1; j < n; ++j) s += A[(size_t)i * n + j] * v[j];
      p[i] = beta * s;
    }
    double pv = 0.0;
    for (int i = k + 1; i < n; ++i) pv += p[i] * v[i];
    for (int i = k + 1; i < n; ++i) w[i] = p[i] - 0.5 * beta * pv * v[i];
    for (int i = k + 1; i < n; ++i)
      for (int j = k + 1; j < n; ++j) A[(size_t)i * n + j] -= v[i] * w[j] + w[i] * v[j];
    // column k and row k of the reflected matrix
    A[(size_t)(k + 1) * n + k] = alpha;
    A[(size_t)k * n + (k + 1)] = alpha;
    for (int i = k + 2; i < n; ++i) {
      A[(size_t)i * n + k] = 0.0;
      A[(size_t)k * n + i] = 0.0;
    }
    // Q <- Q H with H = I - beta v v^T
    for (int r = 0; r < n; ++r) {
      double s = 0.0;
      for (int j = k + 1; j < n; ++j) s += Q[(size_t)r * n + j] * v[j];
      s *= beta;
      for (int j = k + 1; j < n; ++j) Q[(size_t)r * n + j] -= s * v[j];
    }
  }
  diag.resize(n);
  off.assign(n > 1 ? n - 1 : 0, 0.0);
  for (int i = 0; i < n; ++i) diag[i] = A[(size_t)i * n + i];
  for (int i = 0; i + 1 < n; ++i) off[i] = A[(size_t)(i + 1) * n + i];
}

// Implicit symmetric tridiagonal QR with Wilkinson shifts, rotating the columns of Q along.
bool tridiagonal_qr(int n, std::vector<double>& diag, std::vector<double>& off, std::vector<double>& Q) {
  const double eps = 2.220446049250313e-16;
  int hi = n - 1;
  int iterations = 0;
  while (hi > 0) {
    // deflate converged off-diagonal entries at the bottom
    if (std::fabs(off[hi - 1]) <= eps * (std::fabs(diag[hi - 1]) + std::fabs(diag[hi]))) {
      off[hi - 1] = 0.0;
      --hi;
      continue;
    }
    int lo = hi - 1;
    while (lo > 0 && std::fabs(off[lo - 1]) > eps * (std::fabs(diag[lo - 1]) + std::fabs(diag[lo]))) --lo;
    if (++iterations > 60 * n) return false;
    // Wilkinson shift from the trailing 2x2 block
    double a = diag[hi - 1], c = diag[hi], b = off[hi - 1];
    double delta = 0.5 * (a - c);
    double sgn = delta >= 0 ? 1.0 : -1.0;
    double mu = c - b * b / (delta + sgn * std::hypot(delta, b));
    // chase the bulge from lo to hi
    double x = diag[lo] - mu, z = off[lo];
    double bulge = 0.0;
    for (int k = lo; k < hi; ++k) {
      double r = std::hypot(x, z);
      double cs = r == 0.0 ? 1.0 : x / r, sn = r == 0.0 ? 0.0 : z / r;
      if (k > lo) off[k - 1] = r;
      double dk = diag[k], dk1 = diag[k + 1], ek = off[k];
      diag[k] = cs * cs * dk + 2.0 * cs * sn * ek + sn * sn * dk1;
      diag[k + 1] = sn * sn * dk - 2.0 * cs * sn * ek + cs * cs * dk1;
      off[k] = cs * sn * (dk1 - dk) + (cs * cs - sn * sn) * ek;
      if (k + 1 < hi) {
        bulge = sn * off[k + 1];
        off[k + 1] *= cs;
      }
      for (int row = 0; row < n; ++row) {
        double qk = Q[(size_t)row * n + k], qk1 = Q[(size_t)row * n + k + 1];
        Q[(size_t)row * n + k] = cs * qk + sn * qk1;
        Q[(size_t)row * n + k + 1] = -sn * qk + cs * qk1;
      }
      if (k + 1 < hi) {
        x = off[k];
        z = bulge;
      }
    }
  }
  return true;
}

}  // namespace

bool symmetric_eigen(int n, double* A_in, double* eigenvalues, double* eigenvectors) {
  std::vector<double> A(A_in, A_in + (size_t)n * n), diag, off, Q;
  householder_tridiagonal(n, A, diag, off, Q);
  if (n > 1 && !tridiagonal_qr(n, diag, off, Q)) return false;
  for (int i = 0; i < n; ++i) eigenvalues[i] = diag[i];
  std::copy(Q.begin(), Q.end(), eigenvectors);
  return true;
}

}  // namespace headq

extern "C" headq_status headq_calibrate(const headq_config* cfg, const float* q_cal, int64_t n_cal, float* U,
                                        double* eig) {
  if (!cfg || !q_cal) return HEADQ_ERR_NULL;
  const int d = cfg->head_dim, hq = cfg->n_q_heads, hkv = cfg->n_kv_heads, r = cfg->rank;
  if (d != 64 && d != 128) return HEADQ_ERR_UNSUPPORTED;
  if (hq < 1 || hkv < 1 || hq % hkv || n_cal < 1 || r < 0 || r > d) return HEADQ_ERR_SHAPE;
  if (r != 0 && r != 4 && r != 8 && r != 16 && r != 32) return HEADQ_ERR_UNSUPPORTED;
  if (r > 0 && !U) return HEADQ_ERR_NULL;
  const int g = hq / hkv;
  for (int64_t i = 0; i < (int64_t)hq * n_cal * d; ++i)
    if (!std::isfinite(q_cal[i])) return HEADQ_ERR_NUMERIC;
  std::vector<double> M((size_t)d * d), w(d), V((size_t)d * d);
  std::vector<int> order(d);
  for (int h = 0; h < hkv; ++h) {
    std::fill(M.begin(), M.end(), 0.0);
    for (int a = h * g; a < (h + 1) * g; ++a)
      for (int64_t n = 0; n < n_cal; ++n) {
        const float* x = q_cal + ((int64_t)a * n_cal + n) * d;
        for (int i = 0; i < d; ++i) {
          const double xi = x[i];
          for (int j = i; j < d; ++j) M[(size_t)i * d + j] += xi * (double)x[j];
        }
      }
    const double inv_rows = 1.0 / ((double)g * (double)n_cal);
    for (int i = 0; i < d; ++i)
      for (int j = i; j < d; ++j) {
        M[(size_t)i * d + j] *= inv_rows;
        M[(size_t)j * d + i] = M[(size_t)i * d + j];
      }
    if (!headq::symmetric_eigen(d, M.data(), w.data(), V.data())) return HEADQ_ERR_NUMERIC;
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return w[a] > w[b]; });
    for (int col = 0; col < r; ++col) {
      const int src = order[col];
      int arg = 0;
      double best = -1.0;
      for (int i = 0; i < d; ++i) {
        const double m = std::fabs(V[(size_t)i * d + src]);
        if (m > best) {
          best = m;
          arg = i;
        }
      }
      const double sgn = V[(size_t)arg * d + src] < 0 ? -1.0 : 1.0;
      for (int i = 0; i < d; ++i) U[((int64_t)h * d + i) * r + col] = (float)(sgn * V[(size_t)i * d + src]);
      if (eig) eig[(int64_t)h * r + col] = w[src];
    }
  }
  return HEADQ_OK;
}

extern "C" headq_status headq_calibrate_mean(const headq_config* cfg, const float* q_cal, int64_t n_cal, float* a) {
  if (!cfg || !q_cal || !a) return HEADQ_ERR_NULL;
  const int d = cfg->head_dim, hq = cfg->n_q_heads, hkv = cfg->n_kv_heads;
  if (d != 64 && d != 128) return HEADQ_ERR_UNSUPPORTED;
  if (hq < 1 || hkv < 1 || hq % hkv || n_cal < 1) return HEADQ_ERR_SHAPE;
  for (int64_t i = 0; i < (int64_t)hq * n_cal * d; ++i)
    if (!std::isfinite(q_cal[i])) return HEADQ_ERR_NUMERIC;
  const int g = hq / hkv;
  for (int h = 0; h < hkv; ++h)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int hh = h * g; hh < (h + 1) * g; ++hh)
        for (int64_t n = 0; n < n_cal; ++n) acc += (double)q_cal[((int64_t)hh * n_cal + n) * d + c];
      a[(int64_t)h * d + c] = (float)(acc / ((double)g * (double)n_cal));
    }
  return HEADQ_OK;
}
