// Host-side key-rotation calibration in fp64.
//
// axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy barrier",
// section "어텐션 통계 기반 회전과 Triton 커널의 결합": R_K = U_Q . H_Had . P_br
// where U_Q are the eigenvectors of the query covariance
// C_Q = (1/N) sum_n q_n^T q_n.  techllm, "KV cache compression: TurboQuant,
// OSCAR, EpiCache", OSCAR section: the Hadamard + bit-reversal stage spreads
// important directions evenly over the channels.
//
// The eigenproblem is solved with the cyclic Jacobi method for symmetric
// matrices (Golub & Van Loan, "Matrix Computations", section 8.5): plane
// rotations annihilate one off-diagonal pair at a time, sweeping all pairs
// until the off-diagonal mass is negligible.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <algorithm>
#include <vector>

#include "oscar.h"

namespace oscar {
void set_error(const char* fmt, ...);
}

namespace {

bool jacobi_eigen(std::vector<double>& a, int n, std::vector<double>& v, std::vector<double>& w) {
  v.assign(static_cast<size_t>(n) * n, 0.0);
  for (int i = 0; i < n; ++i) v[static_cast<size_t>(i) * n + i] = 1.0;
  auto A = [&](int i, int j) -> double& { return a[static_cast<size_t>(i) * n + j]; };
  double total = 0.0;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) total += A(i, j) * A(i, j);
  const double tol = 1e-30 * total;
  bool converged = false;
  for (int sweep = 0; sweep < 100 && !converged; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += 2.0 * A(p, q) * A(p, q);
    if (off <= tol) {
      converged = true;
      break;
    }
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        const double apq = A(p, q);
        if (apq == 0.0) continue;
        const double app = A(p, p), aqq = A(q, q);
        // rotation angle that zeroes a_pq: tan(theta) = t, smaller root
        const double theta = (aqq - app) / (2.0 * apq);
        const double t = (theta >= 0.0 ? 1.0 : -1.0) / (std::fabs(theta) + std::sqrt(theta * theta + 1.0));
        const double c = 1.0 / std::sqrt(t * t + 1.0);
        const double s = t * c;
        // A <- J^T A J with J the rotation in the (p, q) plane
        for (int k = 0; k < n; ++k) {
          const double akp = A(k, p), akq = A(k, q);
          A(k, p) = c * akp - s * akq;
          A(k, q) = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) {
          const double apk = A(p, k), aqk = A(q, k);
          A(p, k) = c * apk - s * aqk;
          A(q, k) = s * apk + c * aqk;
        }
        A(p, q) = 0.0;
        A(q, p) = 0.0;
        for (int k = 0; k < n; ++k) {
          double& vkp = v[static_cast<size_t>(k) * n + p];
          double& vkq = v[static_cast<size_t>(k) * n + q];
          const double x = vkp, y = vkq;
          vkp = c * x - s * y;
          vkq = s * x + c * y;
        }
      }
    }
  }
  w.resize(n);
  for (int i = 0; i < n; ++i) w[i] = A(i, i);
  return converged;
}

int bit_reverse(int j, int bits) {
  int r = 0;
  for (int b = 0; b < bits; ++b)
    if (j >> b & 1) r |= 1 << (bits - 1 - b);
  return r;
}

}  // namespace

extern "C" int oscar_calibrate_host(const float* q, int64_t n, int32_t d, float* rot_out, double* eig_out) {
  if (!q || !rot_out || n < 1 || d != OSCAR_HEAD_DIM) {
    oscar::set_error("oscar_calibrate_host: need q, rot_out, n >= 1 and d == 128");
    return OSCAR_E_ARG;
  }
  const int D = d;
  // C = (1/N) sum_n q_n^T q_n, fp64 accumulation
  std::vector<double> c(static_cast<size_t>(D) * D, 0.0);
  std::vector<double> row(D);
  for (int64_t i = 0; i < n; ++i) {
    for (int k = 0; k < D; ++k) {
      const float x = q[i * D + k];
      if (!std::isfinite(x)) {
        oscar::set_error("oscar_calibrate_host: non-finite query value at row %lld", static_cast<long long>(i));
        return OSCAR_E_NUMERIC;
      }
      row[k] = x;
    }
    for (int a = 0; a < D; ++a) {
      const double ra = row[a];
      double* ca = &c[static_cast<size_t>(a) * D];
      for (int b = 0; b < D; ++b) ca[b] += ra * row[b];
    }
  }
  for (double& x : c) x /= static_cast<double>(n);

  std::vector<double> u, w;
  if (!jacobi_eigen(c, D, u, w)) {
    oscar::set_error("oscar_calibrate_host: Jacobi eigensolver did not converge");
    return OSCAR_E_NUMERIC;
  }
  // descending eigenvalues, stable
  std::vector<int> order(D);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
  std::vector<double> us(static_cast<size_t>(D) * D);
  for (int j = 0; j < D; ++j) {
    const int src = order[j];
    // sign: largest-magnitude entry positive (lowest index on ties)
    int imax = 0;
    double best = -1.0;
    for (int i = 0; i < D; ++i) {
      const double m = std::fabs(u[static_cast<size_t>(i) * D + src]);
      if (m > best) { best = m; imax = i; }
    }
    const double sgn = u[static_cast<size_t>(imax) * D + src] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < D; ++i) us[static_cast<size_t>(i) * D + j] = sgn * u[static_cast<size_t>(i) * D + src];
  }
  // R = U . H . P with H[m][k] = (-1)^popcount(m & k) / sqrt(D) and (x P)_j = x_br(j)
  const double hs = 1.0 / std::sqrt(static_cast<double>(D));
  int bits = 0;
  while ((1 << bits) < D) ++bits;
  for (int i = 0; i < D; ++i) {
    for (int j = 0; j < D; ++j) {
      const int k = bit_reverse(j, bits);
      double s = 0.0;
      for (int m = 0; m < D; ++m) {
        const double h = (__builtin_popcount(static_cast<unsigned>(m & k)) & 1) ? -hs : hs;
        s += us[static_cast<size_t>(i) * D + m] * h;
      }
      rot_out[static_cast<size_t>(i) * D + j] = static_cast<float>(s);
    }
  }
  if (eig_out)
    for (int j = 0; j < D; ++j) eig_out[j] = w[order[j]];
  return OSCAR_OK;
}
