// Top-r singular triplets of a dense fp64 matrix, for the offline split
// W~ = U S V^T, L1 = U_r S_r, L2 = V_r^T (Zhou, SVDQuant reading notes,
// sec. 5, Eq. (10)).  The notes ask for the exact truncated SVD (Eckart-Young
// optimality); no LAPACK exists on the target hosts, so this file solves the
// symmetric eigenproblem of the Gram matrix on the smaller side directly:
//
//   1. G = A A^T (A has the smaller dimension as rows), blocked, threaded.
//   2. Householder reduction G = Q T Q^T to tridiagonal T (Golub & Van Loan,
//      Matrix Computations, Alg. 8.3.1), full symmetric storage, threaded
//      rank-2 updates.
//   3. The r largest eigenvalues of T by Sturm-sequence bisection
//      (Wilkinson; the negcount recurrence as in Demmel's "Applied Numerical
//      Linear Algebra", sec. 5.3.4).
//   4. Their eigenvectors by inverse iteration with a tridiagonal LU with
//      partial pivoting, re-orthogonalised against the eigenvectors of
//      nearby eigenvalues (the scheme of Peters & Wilkinson).
//   5. Back-transformation by the stored reflectors.
//
// A direct method is used on purpose: the truncation point falls inside the
// bulk of the spectrum for the FLUX-shaped layers, where the gap between the
// r-th and (r+1)-th singular values is tiny and subspace iteration would
// need thousands of sweeps.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <functional>
#include <thread>
#include <vector>

#include "host_internal.h"

namespace svdq {

typedef double v4d __attribute__((vector_size(32)));

static inline double dot(const double* a, const double* b, int64_t n) {
  v4d s0 = {0, 0, 0, 0}, s1 = s0, s2 = s0, s3 = s0;
  int64_t t = 0;
  for (; t + 16 <= n; t += 16) {
    v4d a0, a1, a2, a3, b0, b1, b2, b3;
    std::memcpy(&a0, a + t, 32); std::memcpy(&a1, a + t + 4, 32);
    std::memcpy(&a2, a + t + 8, 32); std::memcpy(&a3, a + t + 12, 32);
    std::memcpy(&b0, b + t, 32); std::memcpy(&b1, b + t + 4, 32);
    std::memcpy(&b2, b + t + 8, 32); std::memcpy(&b3, b + t + 12, 32);
    s0 += a0 * b0; s1 += a1 * b1; s2 += a2 * b2; s3 += a3 * b3;
  }
  v4d s = (s0 + s1) + (s2 + s3);
  double r = (s[0] + s[1]) + (s[2] + s[3]);
  for (; t < n; ++t) r += a[t] * b[t];
  return r;
}

void parallel_for(int64_t n, int threads, const std::function<void(int64_t, int64_t)>& fn) {
  if (threads <= 1 || n < 2) { fn(0, n); return; }
  int t = (int)std::min<int64_t>(threads, n);
  std::vector<std::thread> pool;
  pool.reserve(t);
  for (int i = 0; i < t; ++i) {
    int64_t a = n * i / t, b = n * (i + 1) / t;
    pool.emplace_back([&fn, a, b] { fn(a, b); });
  }
  for (auto& th : pool) th.join();
}

// G = A A^T for A [m, k] row-major (fp64); G is m x m, full storage.
static void gram_rows(const double* A, int64_t m, int64_t k, double* G, int threads) {
  const int64_t B = 64, KB = 512;
  const int64_t nb = (m + B - 1) / B;
  // enumerate lower-triangular block pairs
  std::vector<std::pair<int64_t, int64_t>> pairs;
  for (int64_t bi = 0; bi < nb; ++bi)
    for (int64_t bj = 0; bj <= bi; ++bj) pairs.emplace_back(bi, bj);
  parallel_for((int64_t)pairs.size(), threads, [&](int64_t lo, int64_t hi) {
    std::vector<double> acc(B * B);
    for (int64_t p = lo; p < hi; ++p) {
      int64_t i0 = pairs[p].first * B, j0 = pairs[p].second * B;
      int64_t i1 = std::min(m, i0 + B), j1 = std::min(m, j0 + B);
      std::fill(acc.begin(), acc.end(), 0.0);
      for (int64_t k0 = 0; k0 < k; k0 += KB) {
        int64_t k1 = std::min(k, k0 + KB);
        for (int64_t i = i0; i < i1; ++i) {
          const double* ai = A + i * k;
          double* ci = acc.data() + (i - i0) * B;
          for (int64_t j = j0; j < j1; ++j)
            ci[j - j0] += dot(ai + k0, A + j * k + k0, k1 - k0);
        }
      }
      for (int64_t i = i0; i < i1; ++i)
        for (int64_t j = j0; j < j1; ++j) {
          double v = acc[(i - i0) * B + (j - j0)];
          G[i * m + j] = v;
          G[j * m + i] = v;
        }
    }
  });
}

struct Tridiag {
  std::vector<double> d, e, tau;   // diagonal, off-diagonal, reflector scalars
};

// Householder tridiagonalisation of the symmetric matrix A (n x n, full
// storage, overwritten).  Reflector k acts on indices k+1..n-1 with
// v = (1, A[k+2..n-1][k]) and H_k = I - tau_k v v^T.
static Tridiag tridiagonalize(double* A, int64_t n, int threads) {
  Tridiag T;
  T.d.assign(n, 0.0);
  T.e.assign(n > 0 ? n - 1 : 0, 0.0);
  T.tau.assign(n > 1 ? n - 1 : 0, 0.0);
  std::vector<double> v(n), p(n), w(n);
  for (int64_t k = 0; k + 2 < n; ++k) {
    const int64_t m = n - k - 1;          // trailing size
    double x0 = A[(k + 1) * n + k];
    double xs = 0.0;
    for (int64_t i = k + 2; i < n; ++i) xs += A[i * n + k] * A[i * n + k];
    T.d[k] = A[k * n + k];
    if (xs == 0.0) {                      // already tridiagonal in this column
      T.e[k] = x0;
      T.tau[k] = 0.0;
      continue;
    }
    double beta = -std::copysign(std::sqrt(x0 * x0 + xs), x0);
    double tau = (beta - x0) / beta;
    double scal = 1.0 / (x0 - beta);
    v[0] = 1.0;
    for (int64_t i = 1; i < m; ++i) {
      double vi = A[(k + 1 + i) * n + k] * scal;
      v[i] = vi;
      A[(k + 1 + i) * n + k] = vi;        // keep the reflector below the subdiagonal
    }
    T.e[k] = beta;
    T.tau[k] = tau;
    // p = tau * S v, S = A[k+1.., k+1..]
    parallel_for(m, threads, [&](int64_t lo, int64_t hi) {
      for (int64_t i = lo; i < hi; ++i) {
        p[i] = tau * dot(A + (k + 1 + i) * n + (k + 1), v.data(), m);
      }
    });
    double pv = 0.0;
    for (int64_t i = 0; i < m; ++i) pv += p[i] * v[i];
    double half = 0.5 * tau * pv;
    for (int64_t i = 0; i < m; ++i) w[i] = p[i] - half * v[i];
    // S -= v w^T + w v^T (both triangles)
    parallel_for(m, threads, [&](int64_t lo, int64_t hi) {
      for (int64_t i = lo; i < hi; ++i) {
        double* row = A + (k + 1 + i) * n + (k + 1);
        const double vi = v[i], wi = w[i];
        for (int64_t j = 0; j < m; ++j) row[j] -= vi * w[j] + wi * v[j];
      }
    });
  }
  if (n >= 2) {
    T.d[n - 2] = A[(n - 2) * n + (n - 2)];
    T.e[n - 2] = A[(n - 1) * n + (n - 2)];
    T.tau[n - 2] = 0.0;
  }
  if (n >= 1) T.d[n - 1] = A[(n - 1) * n + (n - 1)];
  return T;
}

// Number of eigenvalues of T smaller than x (Sturm count via the LDL^T
// pivots of T - x I).
static int64_t sturm_below(const std::vector<double>& d, const std::vector<double>& e2, double x,
                           double pivmin) {
  int64_t cnt = 0;
  double q = d[0] - x;
  if (std::fabs(q) < pivmin) q = -pivmin;
  if (q < 0) ++cnt;
  for (size_t i = 1; i < d.size(); ++i) {
    q = d[i] - x - e2[i - 1] / q;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++cnt;
  }
  return cnt;
}

// Solve (T - lam I) x = b in place (b -> x) with partial pivoting.
static void tridiag_solve(const std::vector<double>& d, const std::vector<double>& e, double lam,
                          std::vector<double>& x, double tiny) {
  const int64_t n = (int64_t)d.size();
  // LU of the tridiagonal with row interchanges: U has up to 2 superdiagonals
  std::vector<double> a(n), b(n), c(n), u2(n, 0.0);
  std::vector<double> l(n, 0.0);
  std::vector<char> swp(n, 0);
  for (int64_t i = 0; i < n; ++i) { a[i] = d[i] - lam; }
  for (int64_t i = 0; i + 1 < n; ++i) { b[i] = e[i]; c[i] = e[i]; }   // super, sub
  for (int64_t i = 0; i + 1 < n; ++i) {
    if (std::fabs(a[i]) >= std::fabs(c[i])) {
      double piv = a[i] == 0.0 ? tiny : a[i];
      a[i] = piv;
      double f = c[i] / piv;
      l[i] = f;
      a[i + 1] -= f * b[i];
      u2[i] = 0.0;
    } else {
      // swap rows i and i+1
      double f = a[i] / c[i];
      l[i] = f;
      swp[i] = 1;
      a[i] = c[i];
      double tmp = a[i + 1];
      a[i + 1] = b[i] - f * tmp;
      b[i] = tmp;
      if (i + 2 < n) { u2[i] = b[i + 1]; b[i + 1] = -f * u2[i]; }
    }
  }
  if (a[n - 1] == 0.0) a[n - 1] = tiny;
  // forward: apply L (with swaps) to x
  for (int64_t i = 0; i + 1 < n; ++i) {
    if (swp[i]) { double t = x[i]; x[i] = x[i + 1]; x[i + 1] = t - l[i] * x[i]; }
    else x[i + 1] -= l[i] * x[i];
  }
  // back substitution with U (diag a, super b, super-2 u2)
  x[n - 1] /= a[n - 1];
  if (n >= 2) x[n - 2] = (x[n - 2] - b[n - 2] * x[n - 1]) / a[n - 2];
  for (int64_t i = n - 3; i >= 0; --i) x[i] = (x[i] - b[i] * x[i + 1] - u2[i] * x[i + 2]) / a[i];
}

bool top_eigenpairs(double* G, int64_t n, int64_t r, int threads, int max_iters,
                    std::vector<double>& evals, std::vector<double>& evecs) {
  evals.assign(r, 0.0);
  evecs.assign(r * n, 0.0);
  if (r == 0 || n == 0) return true;
  if (max_iters < 0) return false;
  const int iters = max_iters > 0 ? max_iters : 200;
  Tridiag T = tridiagonalize(G, n, threads);
  const std::vector<double>& d = T.d;
  std::vector<double> e2(n > 1 ? n - 1 : 0);
  double tnorm = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double s = std::fabs(d[i]) + (i > 0 ? std::fabs(T.e[i - 1]) : 0.0) + (i + 1 < n ? std::fabs(T.e[i]) : 0.0);
    tnorm = std::max(tnorm, s);
  }
  double emax2 = 0.0;
  for (int64_t i = 0; i + 1 < n; ++i) { e2[i] = T.e[i] * T.e[i]; emax2 = std::max(emax2, e2[i]); }
  const double eps = 2.220446049250313e-16;
  const double pivmin = std::max(1e-300, std::max(1.0, emax2) * 1e-300);
  // Gershgorin interval
  double lo = d[0], hi = d[0];
  for (int64_t i = 0; i < n; ++i) {
    double rad = (i > 0 ? std::fabs(T.e[i - 1]) : 0.0) + (i + 1 < n ? std::fabs(T.e[i]) : 0.0);
    lo = std::min(lo, d[i] - rad);
    hi = std::max(hi, d[i] + rad);
  }
  const double atol = 2.0 * eps * std::max(std::fabs(lo), std::fabs(hi)) + pivmin;
  lo -= atol; hi += atol;
  // eigenvalue j (0 = largest) is the (n-1-j)-th smallest
  parallel_for(r, threads, [&](int64_t a, int64_t b) {
    for (int64_t j = a; j < b; ++j) {
      const int64_t idx = n - 1 - j;   // want x with count(< x) <= idx < count(< x') ...
      double L = lo, H = hi;
      for (int it = 0; it < iters && H - L > atol + 2 * eps * std::max(std::fabs(L), std::fabs(H)); ++it) {
        double mid = 0.5 * (L + H);
        if (sturm_below(d, e2, mid, pivmin) > idx) H = mid; else L = mid;
      }
      evals[j] = 0.5 * (L + H);
    }
  });
  // eigenvectors of T by inverse iteration, re-orthogonalised within clusters
  const double ortol = 1e-3 * tnorm;
  std::vector<double> y(n);
  uint64_t seed = 0x9E3779B97F4A7C15ull;
  std::vector<std::vector<double>> ty(r);
  for (int64_t j = 0; j < r; ++j) {
    double lam = evals[j];
    // separate exactly equal eigenvalues slightly (as LAPACK's stein does)
    if (j > 0 && std::fabs(lam - evals[j - 1]) < 10 * eps * tnorm) lam = evals[j - 1] - 10 * eps * tnorm;
    for (int64_t i = 0; i < n; ++i) {
      seed ^= seed << 13; seed ^= seed >> 7; seed ^= seed << 17;
      y[i] = ((double)(seed >> 11) / 9007199254740992.0) - 0.5;
    }
    const double tiny = eps * std::max(tnorm, 1e-300);
    for (int it = 0; it < 5; ++it) {
      tridiag_solve(d, T.e, lam, y, tiny);
      for (int64_t p = 0; p < j; ++p) {
        if (std::fabs(evals[p] - evals[j]) > ortol) continue;
        double dot = 0.0;
        for (int64_t i = 0; i < n; ++i) dot += ty[p][i] * y[i];
        for (int64_t i = 0; i < n; ++i) y[i] -= dot * ty[p][i];
      }
      double nrm = 0.0;
      for (int64_t i = 0; i < n; ++i) nrm += y[i] * y[i];
      nrm = std::sqrt(nrm);
      if (!(nrm > 0.0) || !std::isfinite(nrm)) return false;
      for (int64_t i = 0; i < n; ++i) y[i] /= nrm;
    }
    ty[j] = y;
  }
  // back-transform: x = H_0 H_1 ... H_{n-3} y
  parallel_for(r, threads, [&](int64_t a, int64_t b) {
    for (int64_t j = a; j < b; ++j) {
      std::vector<double> x = ty[j];
      for (int64_t k = n - 3; k >= 0; --k) {
        const double tau = T.tau[k];
        if (tau == 0.0) continue;
        double s = x[k + 1];
        for (int64_t i = k + 2; i < n; ++i) s += G[i * n + k] * x[i];
        s *= tau;
        x[k + 1] -= s;
        for (int64_t i = k + 2; i < n; ++i) x[i] -= s * G[i * n + k];
      }
      std::memcpy(&evecs[j * n], x.data(), sizeof(double) * n);
    }
  });
  for (double ev : evals) if (!std::isfinite(ev)) return false;
  return true;
}

bool truncated_svd(const double* A, int64_t K, int64_t N, int64_t r, int threads, int max_iters,
                   std::vector<double>& L1, std::vector<double>& L2, std::vector<double>& sigma) {
  L1.assign(K * r, 0.0);
  L2.assign(r * N, 0.0);
  sigma.assign(r, 0.0);
  if (r == 0) return true;
  const bool rows_small = K <= N;
  const int64_t n = rows_small ? K : N, k = rows_small ? N : K;
  std::vector<double> At;
  const double* Am = A;
  if (!rows_small) {              // transpose so the smaller dimension indexes rows
    At.resize(N * K);
    parallel_for(N, threads, [&](int64_t lo, int64_t hi) {
      for (int64_t i = lo; i < hi; ++i)
        for (int64_t j = 0; j < K; ++j) At[i * K + j] = A[j * N + i];
    });
    Am = At.data();
  }
  std::vector<double> G(n * n);
  gram_rows(Am, n, k, G.data(), threads);
  std::vector<double> ev, vec;
  if (!top_eigenpairs(G.data(), n, r, threads, max_iters, ev, vec)) return false;
  // Am = [n, k]; vec rows are unit eigenvectors u_j of Am Am^T.
  // s_j = sqrt(ev_j); the other factor is Am^T u_j (= s_j v_j).
  std::vector<double> proj(r * k, 0.0);
  parallel_for(r, threads, [&](int64_t a, int64_t b) {
    for (int64_t j = a; j < b; ++j) {
      double* pj = &proj[j * k];
      for (int64_t i = 0; i < n; ++i) {
        const double u = vec[j * n + i];
        const double* row = Am + i * k;
        for (int64_t t = 0; t < k; ++t) pj[t] += u * row[t];
      }
    }
  });
  for (int64_t j = 0; j < r; ++j) {
    double s2 = 0.0;
    for (int64_t t = 0; t < k; ++t) s2 += proj[j * k + t] * proj[j * k + t];
    sigma[j] = std::sqrt(s2);      // |Am^T u_j| = s_j, more accurate than sqrt(ev)
  }
  for (int64_t j = 0; j < r; ++j) {
    const double s = sigma[j];
    const bool zero = !(s > 0.0);
    if (rows_small) {
      // u_j spans the K side: L1[:, j] = s_j u_j, L2[j, :] = (Am^T u_j)^T / s_j
      for (int64_t i = 0; i < K; ++i) L1[i * r + j] = zero ? 0.0 : s * vec[j * n + i];
      for (int64_t t = 0; t < N; ++t) L2[j * N + t] = zero ? 0.0 : proj[j * k + t] / s;
    } else {
      // u_j spans the N side (right singular vector): L2[j, :] = u_j^T,
      // L1[:, j] = A u_j = Am^T u_j
      for (int64_t t = 0; t < N; ++t) L2[j * N + t] = zero ? 0.0 : vec[j * n + t];
      for (int64_t i = 0; i < K; ++i) L1[i * r + j] = zero ? 0.0 : proj[j * k + i];
    }
  }
  return true;
}

}  // namespace svdq
