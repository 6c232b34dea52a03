// Host-side symmetric eigen-solver for the SVD split of the smoothed weight.
//
// The prep needs the top-r singular triplets of What (K x N) (chattools.cn
// overview, section "SVDQuant的技术原理": the dominant singular values go to
// the 16-bit branch, which the Eckart-Young-Mirsky item there justifies). They
// are taken from the Gram matrix of the shorter side, G = B B^T, whose
// eigenpairs are (sigma^2, u). The solver is the classical three-stage one
// (Golub & Van Loan, "Matrix Computations", ch. 8):
//   1. Householder reduction of G to symmetric tridiagonal T = Q^T G Q;
//   2. Sturm-sequence bisection for the wanted eigenvalues of T;
//   3. inverse iteration on T for their eigenvectors (re-orthogonalised
//      inside clusters), then back-transformation by the reflectors.
// Only r eigenvectors are formed, so the cost is the O(n^3) reduction plus
// O(n^2 r). Everything is fp64; the loops over rows run on OpenMP threads.
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

#include "host_internal.hpp"

namespace svdq {

// --------------------------------------------------------------------------
// G = B B^T, B: n x m row-major. Blocked dot products of row pairs; only the
// lower triangle is computed and then mirrored.
void gram_rows(const double* B, int64_t n, int64_t m, double* G) {
  const int64_t TB = 64;       // tile of rows
  const int64_t KC = 512;      // chunk of the summed dimension
  const int64_t nt = (n + TB - 1) / TB;
  std::vector<std::pair<int64_t, int64_t>> tiles;
  for (int64_t bi = 0; bi < nt; ++bi)
    for (int64_t bj = 0; bj <= bi; ++bj) tiles.emplace_back(bi, bj);
  for (int64_t i = 0; i < n * n; ++i) G[i] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < static_cast<int64_t>(tiles.size()); ++t) {
    const int64_t i0 = tiles[t].first * TB, j0 = tiles[t].second * TB;
    const int64_t i1 = std::min(n, i0 + TB), j1 = std::min(n, j0 + TB);
    double acc[TB][TB];
    for (int64_t a = 0; a < TB; ++a)
      for (int64_t b = 0; b < TB; ++b) acc[a][b] = 0.0;
    for (int64_t k0 = 0; k0 < m; k0 += KC) {
      const int64_t k1 = std::min(m, k0 + KC);
      for (int64_t i = i0; i < i1; i += 2) {
        const int64_t ia = i, ib = std::min(i + 1, i1 - 1);
        const double* ra = B + ia * m;
        const double* rb = B + ib * m;
        for (int64_t j = j0; j < j1; j += 2) {
          const int64_t ja = j, jb = std::min(j + 1, j1 - 1);
          const double* ca = B + ja * m;
          const double* cb = B + jb * m;
          double s00 = 0, s01 = 0, s10 = 0, s11 = 0;
#pragma omp simd reduction(+ : s00, s01, s10, s11)
          for (int64_t k = k0; k < k1; ++k) {
            s00 += ra[k] * ca[k];
            s01 += ra[k] * cb[k];
            s10 += rb[k] * ca[k];
            s11 += rb[k] * cb[k];
          }
          acc[ia - i0][ja - j0] += s00;
          if (jb != ja) acc[ia - i0][jb - j0] += s01;
          if (ib != ia) {
            acc[ib - i0][ja - j0] += s10;
            if (jb != ja) acc[ib - i0][jb - j0] += s11;
          }
        }
      }
    }
    for (int64_t i = i0; i < i1; ++i)
      for (int64_t j = j0; j < j1; ++j) {
        G[i * n + j] = acc[i - i0][j - j0];
        G[j * n + i] = acc[i - i0][j - j0];
      }
  }
}

namespace {

// --------------------------------------------------------------------------
// 1. Householder tridiagonalisation of a full symmetric matrix (row-major).
// On return d (n) and e (n-1) hold T; row k of A right of the diagonal holds
// the reflector vector v_k over indices k+1..n-1 (v_k[k+1] = 1) and tau its
// factor, so that G = Q T Q^T with Q = H_0 H_1 ... H_{n-3},
// H_k = I - tau_k v_k v_k^T.
void tridiagonalize(std::vector<double>& A, int64_t n, std::vector<double>& d,
                    std::vector<double>& e, std::vector<double>& tau) {
  d.assign(n, 0.0);
  e.assign(n > 1 ? n - 1 : 0, 0.0);
  tau.assign(n, 0.0);
  std::vector<double> v(n), p(n), w(n);
  for (int64_t k = 0; k + 2 < n; ++k) {
    d[k] = A[k * n + k];
    const int64_t s = n - k - 1;             // size of the trailing block
    const double* x = &A[k * n + k + 1];     // row k right of the diagonal (= column k below)
    double xn2 = 0.0;
    for (int64_t i = 1; i < s; ++i) xn2 += x[i] * x[i];
    const double x0 = x[0];
    if (xn2 == 0.0) {                        // already tridiagonal in this column
      e[k] = x0;
      tau[k] = 0.0;
      continue;
    }
    const double beta = -std::copysign(std::sqrt(x0 * x0 + xn2), x0);
    const double v0 = x0 - beta;
    v[0] = 1.0;
    for (int64_t i = 1; i < s; ++i) v[i] = x[i] / v0;
    const double t = (beta - x0) / beta;
    tau[k] = t;
    e[k] = beta;
    double* Vk = &A[k * n + k + 1];          // row k is not read again: keep v_k there
    for (int64_t i = 0; i < s; ++i) Vk[i] = v[i];
    // p = t * B v over the trailing block B = A[k+1.., k+1..]
    double* Ab = &A[(k + 1) * n + (k + 1)];
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < s; ++i) {
      const double* row = Ab + i * n;
      double acc = 0.0;
#pragma omp simd reduction(+ : acc)
      for (int64_t j = 0; j < s; ++j) acc += row[j] * v[j];
      p[i] = t * acc;
    }
    double pv = 0.0;
    for (int64_t i = 0; i < s; ++i) pv += p[i] * v[i];
    const double kk = 0.5 * t * pv;
    for (int64_t i = 0; i < s; ++i) w[i] = p[i] - kk * v[i];
    // B -= v w^T + w v^T
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < s; ++i) {
      double* row = Ab + i * n;
      const double vi = v[i], wi = w[i];
#pragma omp simd
      for (int64_t j = 0; j < s; ++j) row[j] -= vi * w[j] + wi * v[j];
    }
  }
  if (n >= 2) {
    d[n - 2] = A[(n - 2) * n + (n - 2)];
    e[n - 2] = A[(n - 2) * n + (n - 1)];
  }
  d[n - 1] = A[(n - 1) * n + (n - 1)];
}

// --------------------------------------------------------------------------
// 2. Sturm-sequence bisection.

struct Tridiag {
  const std::vector<double>& d;
  std::vector<double> e2;
  double pivmin;
  explicit Tridiag(const std::vector<double>& d_, const std::vector<double>& e_)
      : d(d_), e2(e_.size()) {
    double emax = 0.0;
    for (size_t i = 0; i < e_.size(); ++i) {
      e2[i] = e_[i] * e_[i];
      emax = std::max(emax, e2[i]);
    }
    pivmin = std::numeric_limits<double>::min() * std::max(1.0, emax);
  }
  // number of eigenvalues strictly below x
  int64_t count_below(double x) const {
    const int64_t n = static_cast<int64_t>(d.size());
    int64_t c = 0;
    double q = d[0] - x;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++c;
    for (int64_t i = 1; i < n; ++i) {
      q = d[i] - x - e2[i - 1] / q;
      if (std::fabs(q) < pivmin) q = -pivmin;
      if (q < 0) ++c;
    }
    return c;
  }
};

// eigenvalue number j (0-based, ascending) of T
double bisect(const Tridiag& T, int64_t j, double lo, double hi) {
  const double eps = std::numeric_limits<double>::epsilon();
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (hi - lo <= 2.0 * eps * std::max(std::fabs(lo), std::fabs(hi)) + T.pivmin) break;
    if (mid <= lo || mid >= hi) break;
    if (T.count_below(mid) > j)
      hi = mid;
    else
      lo = mid;
  }
  return 0.5 * (lo + hi);
}

// --------------------------------------------------------------------------
// 3. Inverse iteration: LU with partial pivoting of (T - lambda I).

struct TriLU {
  std::vector<double> u0, u1, u2, mult;
  std::vector<char> swapped;
};

void lu_factor(const std::vector<double>& d, const std::vector<double>& e, double lambda,
               double tiny, TriLU& f) {
  const int64_t n = static_cast<int64_t>(d.size());
  f.u0.assign(n, 0.0);
  f.u1.assign(n, 0.0);
  f.u2.assign(n, 0.0);
  f.mult.assign(n, 0.0);
  f.swapped.assign(n, 0);
  double p0 = d[0] - lambda, p1 = n > 1 ? e[0] : 0.0, p2 = 0.0;
  for (int64_t i = 0; i + 1 < n; ++i) {
    const double c = e[i];
    const double a = d[i + 1] - lambda;
    const double b = (i + 2 < n) ? e[i + 1] : 0.0;
    if (std::fabs(c) > std::fabs(p0)) {
      f.swapped[i] = 1;
      const double m = p0 / c;
      f.u0[i] = c;
      f.u1[i] = a;
      f.u2[i] = b;
      f.mult[i] = m;
      const double n1 = p1 - m * a, n2 = p2 - m * b;
      p0 = n1;
      p1 = n2;
      p2 = 0.0;
    } else {
      if (p0 == 0.0) p0 = tiny;
      const double m = c / p0;
      f.u0[i] = p0;
      f.u1[i] = p1;
      f.u2[i] = p2;
      f.mult[i] = m;
      const double n1 = a - m * p1, n2 = b - m * p2;
      p0 = n1;
      p1 = n2;
      p2 = 0.0;
    }
  }
  if (p0 == 0.0) p0 = tiny;
  f.u0[n - 1] = p0;
}

void lu_solve(const TriLU& f, double tiny, std::vector<double>& y) {
  const int64_t n = static_cast<int64_t>(y.size());
  for (int64_t i = 0; i + 1 < n; ++i) {
    if (f.swapped[i]) {
      const double t = y[i];
      y[i] = y[i + 1];
      y[i + 1] = t - f.mult[i] * y[i];
    } else {
      y[i + 1] -= f.mult[i] * y[i];
    }
  }
  for (int64_t i = n - 1; i >= 0; --i) {
    double s = y[i];
    if (i + 1 < n) s -= f.u1[i] * y[i + 1];
    if (i + 2 < n) s -= f.u2[i] * y[i + 2];
    double piv = f.u0[i];
    if (std::fabs(piv) < tiny) piv = std::copysign(tiny, piv == 0.0 ? 1.0 : piv);
    y[i] = s / piv;
  }
}

// deterministic start vector in [-1, 1]
double start_value(int64_t i, int64_t j) {
  uint64_t h = static_cast<uint64_t>(i) * 0x9E3779B97F4A7C15ull ^
               (static_cast<uint64_t>(j) + 0x632BE59BD9B4E019ull) * 0xC2B2AE3D27D4EB4Full;
  h ^= h >> 29;
  h *= 0xBF58476D1CE4E5B9ull;
  h ^= h >> 32;
  return static_cast<double>(h >> 11) * 0x1p-52 - 1.0;
}

}  // namespace

bool sym_top_eigen(std::vector<double>& A, int64_t n, int r, std::vector<double>& eval,
                   std::vector<double>& Z, std::vector<double>* all_evals) {
  std::vector<double> d, e, tau;
  tridiagonalize(A, n, d, e, tau);
  Tridiag T(d, e);
  double lo = d[0], hi = d[0], tnorm = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const double r0 = (i > 0 ? std::fabs(e[i - 1]) : 0.0) + (i + 1 < n ? std::fabs(e[i]) : 0.0);
    lo = std::min(lo, d[i] - r0);
    hi = std::max(hi, d[i] + r0);
    tnorm = std::max(tnorm, std::fabs(d[i]) + r0);
  }
  const double eps = std::numeric_limits<double>::epsilon();
  const double pad = 2.0 * eps * tnorm + T.pivmin;
  lo -= pad;
  hi += pad;

  if (all_evals) {
    all_evals->assign(n, 0.0);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t j = 0; j < n; ++j) (*all_evals)[n - 1 - j] = bisect(T, j, lo, hi);
  }
  eval.assign(r, 0.0);
#pragma omp parallel for schedule(dynamic, 1)
  for (int j = 0; j < r; ++j) eval[j] = bisect(T, n - 1 - j, lo, hi);

  // inverse iteration, in descending order, re-orthogonalising within clusters
  const double ortol = 1e-3 * tnorm;
  const double tiny = eps * std::max(tnorm, T.pivmin);
  std::vector<std::vector<double>> zs(r);
  bool ok = true;
  int64_t cluster_start = 0;
  double prev_shift = 0.0;
  for (int j = 0; j < r; ++j) {
    if (j > 0 && std::fabs(eval[j] - eval[j - 1]) > ortol) cluster_start = j;
    double shift = eval[j];
    // separate equal shifts inside a cluster (LAPACK dstein does the same)
    if (j > cluster_start && std::fabs(shift - prev_shift) < 10.0 * eps * tnorm)
      shift = prev_shift - 10.0 * eps * tnorm;
    prev_shift = shift;
    TriLU f;
    lu_factor(d, e, shift, tiny, f);
    std::vector<double> y(n);
    for (int64_t i = 0; i < n; ++i) y[i] = start_value(i, j);
    for (int it = 0; it < 4; ++it) {
      double ymax = 0.0;
      for (int64_t i = 0; i < n; ++i) ymax = std::max(ymax, std::fabs(y[i]));
      if (!(ymax > 0.0) || !std::isfinite(ymax)) {
        ok = false;
        break;
      }
      for (int64_t i = 0; i < n; ++i) y[i] /= ymax;
      lu_solve(f, tiny, y);
      for (int64_t c = cluster_start; c < j; ++c) {
        double dot = 0.0;
        for (int64_t i = 0; i < n; ++i) dot += zs[c][i] * y[i];
        for (int64_t i = 0; i < n; ++i) y[i] -= dot * zs[c][i];
      }
      double nrm = 0.0;
      for (int64_t i = 0; i < n; ++i) nrm += y[i] * y[i];
      nrm = std::sqrt(nrm);
      if (!(nrm > 0.0) || !std::isfinite(nrm)) {
        ok = false;
        break;
      }
      for (int64_t i = 0; i < n; ++i) y[i] /= nrm;
    }
    // residual check: |T y - lambda y| must be small against |T| (clusters
    // closer than ortol may mix, which keeps the spanned subspace)
    double res = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      double t = d[i] * y[i];
      if (i > 0) t += e[i - 1] * y[i - 1];
      if (i + 1 < n) t += e[i] * y[i + 1];
      res = std::max(res, std::fabs(t - eval[j] * y[i]));
    }
    if (!(res <= 2.0 * ortol + 1e3 * eps * tnorm)) ok = false;
    zs[j] = y;
  }
  // back-transform: z <- H_0 H_1 ... H_{n-3} z, applied to all r vectors at once
  Z.assign(static_cast<size_t>(n) * r, 0.0);
  for (int64_t i = 0; i < n; ++i)
    for (int j = 0; j < r; ++j) Z[i * r + j] = zs[j][i];
  std::vector<double> s(r);
  for (int64_t k = n - 3; k >= 0; --k) {
    if (tau[k] == 0.0) continue;
    const double* v = &A[k * n + k + 1];
    const int64_t len = n - k - 1;
    std::fill(s.begin(), s.end(), 0.0);
    for (int64_t i = 0; i < len; ++i) {
      const double vi = v[i];
      const double* zr = Z.data() + (k + 1 + i) * r;
      for (int j = 0; j < r; ++j) s[j] += vi * zr[j];
    }
    for (int j = 0; j < r; ++j) s[j] *= tau[k];
#pragma omp parallel for schedule(static) if (len * r > 65536)
    for (int64_t i = 0; i < len; ++i) {
      const double vi = v[i];
      double* zr = Z.data() + (k + 1 + i) * r;
      for (int j = 0; j < r; ++j) zr[j] -= vi * s[j];
    }
  }
  return ok;
}

}  // namespace svdq
