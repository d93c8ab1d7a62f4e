// Host-side key- and value-rotation calibration in fp64, and the offline fold of R_V into the
// value and output projections.
//
// axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy barrier",
// section "어텐션 통계 기반 회전과 Triton 커널의 결합": R_K = U_Q . H_Had . P_br
// where U_Q are the eigenvectors of the query covariance
// C_Q = (1/N) sum_n q_n^T q_n.  techllm, "KV cache compression: TurboQuant,
// OSCAR, EpiCache", OSCAR section: the Hadamard + bit-reversal stage spreads
// important directions evenly over the channels.  Same axbrief section: the value rotation is
// R_V = U_S . H_Had . P_br with U_S the eigenvectors of C_S = (1/N) V^T S^T S V, and R_V is
// absorbed offline into the projection weights.
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


// R = U . H . P from a second-moment matrix c (D x D, fp64, consumed): eigenvectors by
// descending eigenvalue (stable), each column's largest-magnitude entry positive (lowest index on
// ties), H[m][k] = (-1)^popcount(m & k) / sqrt(D), (x P)_j = x_br(j).
int rotation_from_moment(std::vector<double>& c, int D, const char* who, float* rot_out, double* eig_out) {
  std::vector<double> u, w;
  if (!jacobi_eigen(c, D, u, w)) {
    oscar::set_error("%s: Jacobi eigensolver did not converge", who);
    return OSCAR_E_NUMERIC;
  }
  std::vector<int> order(D);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return w[x] > w[y]; });
  std::vector<double> us(static_cast<size_t>(D) * D);
  for (int j = 0; j < D; ++j) {
    const int src = order[j];
    int imax = 0;
    double best = -1.0;
    for (int i = 0; i < D; ++i) {
      const double m = std::fabs(u[static_cast<size_t>(i) * D + src]);
      if (m > best) { best = m; imax = i; }
    }
    const double sgn = u[static_cast<size_t>(imax) * D + src] < 0.0 ? -1.0 : 1.0;
    for (int i = 0; i < D; ++i) us[static_cast<size_t>(i) * D + j] = sgn * u[static_cast<size_t>(i) * D + src];
  }
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

// c += x^T x for one row x (fp64)
void add_outer(std::vector<double>& c, const std::vector<double>& x, int D) {
  for (int a = 0; a < D; ++a) {
    const double xa = x[a];
    double* ca = &c[static_cast<size_t>(a) * D];
    for (int b = 0; b < D; ++b) ca[b] += xa * x[b];
  }
}

}  // namespace

extern "C" int oscar_calibrate_host(const float* q, int64_t n, int32_t d, float* rot_out, double* eig_out) {
  if (!q || !rot_out || n < 1 || d != OSCAR_HEAD_DIM) {
    oscar::set_error("oscar_calibrate_host: need q, rot_out, n >= 1 and d == 128");
    return OSCAR_E_ARG;
  }
  const int D = d;
  // C_Q = (1/N) sum_n q_n^T q_n, fp64 accumulation
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
    add_outer(c, row, D);
  }
  for (double& x : c) x /= static_cast<double>(n);
  return rotation_from_moment(c, D, "oscar_calibrate_host", rot_out, eig_out);
}

extern "C" int oscar_calibrate_value_host(const float* s, const float* v, int64_t n_q, int64_t n_tok, int32_t d,
                                          float* rot_out, double* eig_out) {
  if (!s || !v || !rot_out || n_q < 1 || n_tok < 1 || d != OSCAR_HEAD_DIM) {
    oscar::set_error("oscar_calibrate_value_host: need s, v, rot_out, n_q >= 1, n_tok >= 1 and d == 128");
    return OSCAR_E_ARG;
  }
  const int D = d;
  for (int64_t i = 0; i < n_q * n_tok; ++i)
    if (!std::isfinite(s[i])) {
      oscar::set_error("oscar_calibrate_value_host: non-finite probability at %lld", static_cast<long long>(i));
      return OSCAR_E_NUMERIC;
    }
  for (int64_t i = 0; i < n_tok * D; ++i)
    if (!std::isfinite(v[i])) {
      oscar::set_error("oscar_calibrate_value_host: non-finite value at %lld", static_cast<long long>(i));
      return OSCAR_E_NUMERIC;
    }
  // C_S = (1/N) V^T S^T S V = (1/N) sum_n o_n^T o_n with o_n = sum_t s_nt v_t, fp64
  std::vector<double> c(static_cast<size_t>(D) * D, 0.0);
  std::vector<double> o(D);
  for (int64_t n = 0; n < n_q; ++n) {
    std::fill(o.begin(), o.end(), 0.0);
    const float* sr = s + n * n_tok;
    for (int64_t t = 0; t < n_tok; ++t) {
      const double p = sr[t];
      if (p == 0.0) continue;
      const float* vr = v + t * D;
      for (int k = 0; k < D; ++k) o[k] += p * vr[k];
    }
    add_outer(c, o, D);
  }
  for (double& x : c) x /= static_cast<double>(n_q);
  return rotation_from_moment(c, D, "oscar_calibrate_value_host", rot_out, eig_out);
}

extern "C" int oscar_fold_value_rotation(int32_t d_model, int32_t num_q_heads, int32_t num_kv_heads, const float* r_v,
                                         float* w_v, float* w_o) {
  const int D = OSCAR_HEAD_DIM;
  if (!r_v || !w_v || !w_o || d_model < 1 || num_kv_heads < 1 || num_q_heads < num_kv_heads ||
      num_q_heads % num_kv_heads) {
    oscar::set_error("oscar_fold_value_rotation: null pointer or bad head counts");
    return OSCAR_E_ARG;
  }
  for (int64_t i = 0; i < static_cast<int64_t>(num_kv_heads) * D * D; ++i)
    if (!std::isfinite(r_v[i])) {
      oscar::set_error("oscar_fold_value_rotation: non-finite rotation entry");
      return OSCAR_E_NUMERIC;
    }
  const int64_t wv_cols = static_cast<int64_t>(num_kv_heads) * D;
  const int g = num_q_heads / num_kv_heads;
  std::vector<double> tmp(D);
  // W_V[:, h-block] <- W_V[:, h-block] . R_V[h], row by row
  for (int h = 0; h < num_kv_heads; ++h) {
    const float* r = r_v + static_cast<size_t>(h) * D * D;
    for (int64_t row = 0; row < d_model; ++row) {
      float* x = w_v + row * wv_cols + static_cast<int64_t>(h) * D;
      for (int j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += static_cast<double>(x[i]) * r[static_cast<size_t>(i) * D + j];
        tmp[j] = acc;
      }
      for (int j = 0; j < D; ++j) x[j] = static_cast<float>(tmp[j]);
    }
  }
  // W_O[q-head block] <- R_V[h]^T . W_O[q-head block], column by column
  for (int jq = 0; jq < num_q_heads; ++jq) {
    const float* r = r_v + static_cast<size_t>(jq / g) * D * D;
    float* blk = w_o + static_cast<int64_t>(jq) * D * d_model;
    for (int64_t col = 0; col < d_model; ++col) {
      for (int a = 0; a < D; ++a) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i) acc += static_cast<double>(r[static_cast<size_t>(i) * D + a]) * blk[i * d_model + col];
        tmp[a] = acc;
      }
      for (int a = 0; a < D; ++a) blk[a * d_model + col] = static_cast<float>(tmp[a]);
    }
  }
  return OSCAR_OK;
}
