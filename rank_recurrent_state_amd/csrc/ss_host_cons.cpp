// ss_host_cons.cpp -- the consolidation of frozen parts on host cores (SinkState 4.3 "Asynchronous
// CPU Consolidation", Figure 7(b): the frozen region goes to the host, each state's frozen part is
// replaced by its exact SVD there, the values below eps * sigma_0 are dropped, and the result goes
// back).  This file is the host arithmetic: an exact fp64 SVD of one frozen part, and a batch over
// the states of a group spread over host threads.  The download, the upload, the staleness check
// and the install are in ss_pool.cpp and ss_consolidate.hip.
//
// For one state with frozen part F = sum_k s_k u_k v_k^T (k < f):
//   1. V = Q R, the thin QR of [v_0 .. v_{f-1}] (d_v x f) by classical Gram-Schmidt with one
//      re-orthogonalization pass, in fp64; a column whose residual is at most 1e-12 of its norm is
//      dependent, and it and its row of R are zeroed.
//   2. B = U diag(s) R^T (d_k x f), so that F = B Q^T.
//   3. B = P T, the same thin QR of B.
//   4. One-sided (Hestenes) Jacobi on the columns of T (f x f), cyclic order, to an off-diagonal
//      tolerance of 1e-15: T W = Y diag(sigma), W orthogonal.
//   5. F = (P Y) diag(sigma) (Q W)^T: component j is u = P T W_j / sigma_j, v = Q W_j, sigma_j.
//   6. Sort sigma descending (ties keep column order); keep sigma >= eps sigma_0 and sigma > 0.
// The kept components (never more than f) overwrite the state's input rows, in fp32.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <thread>
#include <vector>

#include "ss_host_cons.h"

namespace ss {

namespace {

// thin QR of the m columns of A (column-major, length d, stride d) in place: A <- Q, R (m x m,
// R[j * m + i] = R(i, j)); a dependent column becomes zero and R(j, j) = 0
void cgs2_host(double *A, int d, int m, double *R) {
  std::fill(R, R + (size_t)m * m, 0.0);
  std::vector<double> c(m);
  for (int j = 0; j < m; ++j) {
    double *aj = A + (size_t)j * d;
    double n0 = 0.0;
    for (int e = 0; e < d; ++e) n0 += aj[e] * aj[e];
    for (int pass = 0; pass < 2; ++pass) {
      for (int i = 0; i < j; ++i) {
        const double *ai = A + (size_t)i * d;
        double x = 0.0;
        for (int e = 0; e < d; ++e) x += ai[e] * aj[e];
        c[i] = x;
      }
      for (int i = 0; i < j; ++i) {
        const double *ai = A + (size_t)i * d;
        for (int e = 0; e < d; ++e) aj[e] -= c[i] * ai[e];
        R[(size_t)j * m + i] += c[i];
      }
    }
    double nu = 0.0;
    for (int e = 0; e < d; ++e) nu += aj[e] * aj[e];
    if (nu > 0.0 && nu > 1e-24 * n0) {
      const double r = std::sqrt(nu);
      for (int e = 0; e < d; ++e) aj[e] /= r;
      R[(size_t)j * m + j] = r;
    } else {  // dependent: its projections stay in R, its own direction is dropped
      std::fill(aj, aj + d, 0.0);
    }
  }
}

// one-sided Jacobi on the m columns of T (column-major m x m), rotations accumulated into W
void jacobi_host(double *T, double *W, int m) {
  std::fill(W, W + (size_t)m * m, 0.0);
  for (int i = 0; i < m; ++i) W[(size_t)i * m + i] = 1.0;
  for (int sweep = 0; sweep < 60; ++sweep) {
    bool rotated = false;
    for (int p = 0; p < m - 1; ++p) {
      for (int q = p + 1; q < m; ++q) {
        double *x = T + (size_t)p * m, *y = T + (size_t)q * m;
        double a = 0.0, b = 0.0, g = 0.0;
        for (int e = 0; e < m; ++e) {
          a += x[e] * x[e];
          b += y[e] * y[e];
          g += x[e] * y[e];
        }
        if (g == 0.0 || std::fabs(g) <= 1e-15 * std::sqrt(a * b)) continue;
        rotated = true;
        const double zeta = (b - a) / (2.0 * g);
        const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (std::fabs(zeta) + std::sqrt(1.0 + zeta * zeta));
        const double cs = 1.0 / std::sqrt(1.0 + t * t), sn = cs * t;
        for (int e = 0; e < m; ++e) {
          const double xe = x[e], ye = y[e];
          x[e] = cs * xe - sn * ye;
          y[e] = sn * xe + cs * ye;
        }
        double *wx = W + (size_t)p * m, *wy = W + (size_t)q * m;
        for (int e = 0; e < m; ++e) {
          const double xe = wx[e], ye = wy[e];
          wx[e] = cs * xe - sn * ye;
          wy[e] = sn * xe + cs * ye;
        }
      }
    }
    if (!rotated) break;
  }
}

}  // namespace

int host_consolidate_one(int dk, int dv, int f, float *u, float *v, float *s, float s0, float eps) {
  if (f <= 0) return 0;
  std::vector<double> Q((size_t)dv * f), R((size_t)f * f), B((size_t)dk * f), T((size_t)f * f), W((size_t)f * f);
  for (int k = 0; k < f; ++k)
    for (int e = 0; e < dv; ++e) Q[(size_t)k * dv + e] = v[(size_t)k * dv + e];
  cgs2_host(Q.data(), dv, f, R.data());
  // B[:, j] = sum_k R(j, k) s_k u_k  (R upper triangular: k >= j)
  std::fill(B.begin(), B.end(), 0.0);
  for (int j = 0; j < f; ++j) {
    double *bj = B.data() + (size_t)j * dk;
    for (int k = j; k < f; ++k) {
      const double c = R[(size_t)k * f + j] * (double)s[k];
      if (c == 0.0) continue;
      const float *uk = u + (size_t)k * dk;
      for (int e = 0; e < dk; ++e) bj[e] += c * (double)uk[e];
    }
  }
  cgs2_host(B.data(), dk, f, T.data());  // B <- P, T upper triangular
  jacobi_host(T.data(), W.data(), f);
  std::vector<double> sig(f);
  std::vector<int> ord(f);
  for (int j = 0; j < f; ++j) {
    double x = 0.0;
    for (int e = 0; e < f; ++e) x += T[(size_t)j * f + e] * T[(size_t)j * f + e];
    sig[j] = std::sqrt(x);
    ord[j] = j;
  }
  std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return sig[a] > sig[b]; });
  const double thr = (double)eps * (double)s0;
  int kept = 0;
  while (kept < f && sig[ord[kept]] > 0.0 && sig[ord[kept]] >= thr) ++kept;
  std::vector<double> nu((size_t)kept * dk), nv((size_t)kept * dv);
  for (int c = 0; c < kept; ++c) {
    const int j = ord[c];
    const double inv = 1.0 / sig[j];
    for (int e = 0; e < dk; ++e) {  // u = P (T W_j) / sigma_j; the rotated column of T is T[:, j]
      double x = 0.0;
      for (int i = 0; i < f; ++i) x += B[(size_t)i * dk + e] * T[(size_t)j * f + i];
      nu[(size_t)c * dk + e] = x * inv;
    }
    for (int e = 0; e < dv; ++e) {  // v = Q W_j
      double x = 0.0;
      for (int i = 0; i < f; ++i) x += Q[(size_t)i * dv + e] * W[(size_t)j * f + i];
      nv[(size_t)c * dv + e] = x;
    }
  }
  for (int c = 0; c < kept; ++c) {
    for (int e = 0; e < dk; ++e) u[(size_t)c * dk + e] = (float)nu[(size_t)c * dk + e];
    for (int e = 0; e < dv; ++e) v[(size_t)c * dv + e] = (float)nv[(size_t)c * dv + e];
    s[c] = (float)sig[ord[c]];
  }
  return kept;
}

void host_consolidate_batch(int n, int dk, int dv, int fmax, float *u, float *v, float *s, int32_t *cnt,
                            const float *s0, const float *eps, int threads) {
  std::atomic<int> next{0};
  auto work = [&]() {
    for (;;) {
      const int i = next.fetch_add(1);
      if (i >= n) return;
      const int f = cnt[i];
      if (f <= 0) continue;
      const size_t b = (size_t)i * fmax;
      cnt[i] = host_consolidate_one(dk, dv, f, u + b * dk, v + b * dv, s + b, s0[i], eps[i]);
    }
  };
  const int t = std::max(1, std::min(threads, n));
  std::vector<std::thread> pool;
  pool.reserve(t - 1);
  for (int k = 1; k < t; ++k) pool.emplace_back(work);
  work();
  for (auto &th : pool) th.join();
}

}  // namespace ss
