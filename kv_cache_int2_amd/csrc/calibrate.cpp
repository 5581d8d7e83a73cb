// Offline calibration on the host, fp64: query covariance and score-weighted
// value covariance -> eigenbases -> R = P_br (H / sqrt d) U^T, rounded to bf16.
// Method: P1 (gen-hub.ru, "Together AI открывает OSCAR…") «Что придумали в
// Together AI» (keys in the query-covariance eigenbasis, values in the
// eigenbasis of the attention-score-weighted value covariance, then a Hadamard
// transform and a bit-reversal permutation) and «Открытый код — это серьёзно»
// (an offline calibration pass once per model); P4 (aiforradalom.hu) «OSCAR:
// figyelem-tudatos és bevetésre kész».
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "common.h"

namespace {

constexpr int D = oscar::kD;

// Cyclic Jacobi eigen-decomposition of a symmetric n x n matrix (row-major),
// fp64.  On return a's diagonal holds the eigenvalues and v's columns the
// eigenvectors (v row-major: v[r * n + c] is entry r of eigenvector c).
void jacobi(std::vector<double>& a, int n, std::vector<double>& v) {
  v.assign((size_t)n * n, 0.0);
  for (int i = 0; i < n; ++i) v[(size_t)i * n + i] = 1.0;
  double total = 0.0;
  for (double x : a) total += x * x;
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += a[(size_t)p * n + q] * a[(size_t)p * n + q];
    if (off <= 1e-34 * total || off == 0.0) break;
    for (int p = 0; p < n - 1; ++p) {
      for (int q = p + 1; q < n; ++q) {
        double apq = a[(size_t)p * n + q];
        if (std::fabs(apq) < 1e-300) continue;
        double app = a[(size_t)p * n + p], aqq = a[(size_t)q * n + q];
        // rotation angle that zeroes a_pq: t = tan(theta) is the smaller root
        // of t^2 + 2 tau t - 1 = 0 with tau = (a_qq - a_pp) / (2 a_pq)
        double tau = (aqq - app) / (2.0 * apq);
        double t = (tau >= 0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int r = 0; r < n; ++r) {  // columns p, q
          double arp = a[(size_t)r * n + p], arq = a[(size_t)r * n + q];
          a[(size_t)r * n + p] = c * arp - s * arq;
          a[(size_t)r * n + q] = s * arp + c * arq;
        }
        for (int r = 0; r < n; ++r) {  // rows p, q
          double apr = a[(size_t)p * n + r], aqr = a[(size_t)q * n + r];
          a[(size_t)p * n + r] = c * apr - s * aqr;
          a[(size_t)q * n + r] = s * apr + c * aqr;
        }
        a[(size_t)p * n + q] = a[(size_t)q * n + p] = 0.0;
        for (int r = 0; r < n; ++r) {
          double vrp = v[(size_t)r * n + p], vrq = v[(size_t)r * n + q];
          v[(size_t)r * n + p] = c * vrp - s * vrq;
          v[(size_t)r * n + q] = s * vrp + c * vrq;
        }
      }
    }
  }
}

// Eigenpairs of a symmetric matrix, eigenvalues descending, eigenvector columns
// sign-fixed so the largest-magnitude entry is positive (first index on ties).
void eig_desc(const std::vector<double>& sym, std::vector<double>& w, std::vector<double>& u) {
  std::vector<double> a(sym), v;
  for (int i = 0; i < D; ++i)
    for (int j = i + 1; j < D; ++j) {
      double m = 0.5 * (a[(size_t)i * D + j] + a[(size_t)j * D + i]);
      a[(size_t)i * D + j] = a[(size_t)j * D + i] = m;
    }
  jacobi(a, D, v);
  std::vector<int> order(D);
  for (int i = 0; i < D; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return a[(size_t)x * D + x] > a[(size_t)y * D + y]; });
  w.resize(D);
  u.assign((size_t)D * D, 0.0);
  for (int k = 0; k < D; ++k) {
    int c = order[k];
    w[k] = a[(size_t)c * D + c];
    int best = 0;
    for (int r = 1; r < D; ++r)
      if (std::fabs(v[(size_t)r * D + c]) > std::fabs(v[(size_t)best * D + c])) best = r;
    double sg = v[(size_t)best * D + c] < 0 ? -1.0 : 1.0;
    for (int r = 0; r < D; ++r) u[(size_t)r * D + k] = sg * v[(size_t)r * D + c];
  }
}

uint16_t bf16_rne(double x) {
  if (x == 0.0) return std::signbit(x) ? 0x8000 : 0;
  int e;
  std::frexp(std::fabs(x), &e);  // |x| = m 2^e, m in [0.5, 1)
  int ex = std::max(e - 1, -126);
  double q = std::ldexp(1.0, ex - 7);
  double r = std::nearbyint(x / q) * q;  // ties to even (default rounding mode)
  float f = (float)r;                    // exact
  uint32_t bits;
  std::memcpy(&bits, &f, 4);
  return (uint16_t)(bits >> 16);
}

int bitrev7(int i) {
  int r = 0;
  for (int b = 0; b < 7; ++b) r |= ((i >> b) & 1) << (6 - b);
  return r;
}

// R[i][j] = sum_k H[br(i)][k] U[j][k] / sqrt(d), H[r][k] = (-1)^popcount(r & k)
void rotation(const std::vector<double>& u, uint16_t* out) {
  const double inv = 1.0 / std::sqrt((double)D);
  for (int i = 0; i < D; ++i) {
    int r = bitrev7(i);
    for (int j = 0; j < D; ++j) {
      double acc = 0.0;
      for (int k = 0; k < D; ++k) {
        double h = (__builtin_popcount(r & k) & 1) ? -1.0 : 1.0;
        acc += h * u[(size_t)j * D + k];
      }
      out[(size_t)i * D + j] = bf16_rne(acc * inv);
    }
  }
}

struct HeadJob {
  const float *q, *k, *v;
  int64_t nq, nkv;
  uint16_t *rk, *rv;
  double *ek, *ev;
};

void calibrate_head(const HeadJob& j) {
  // Sigma_Q = (1/n_q) sum q q^T (uncentred)
  std::vector<double> sq((size_t)D * D, 0.0);
  for (int64_t i = 0; i < j.nq; ++i) {
    const float* qi = j.q + i * D;
    for (int a = 0; a < D; ++a) {
      double qa = qi[a];
      for (int b = a; b < D; ++b) sq[(size_t)a * D + b] += qa * (double)qi[b];
    }
  }
  for (int a = 0; a < D; ++a)
    for (int b = a; b < D; ++b) sq[(size_t)b * D + a] = sq[(size_t)a * D + b] /= (double)j.nq;

  // a_t = sum_i softmax_t(q_i . k_t / sqrt d)
  std::vector<double> wt(j.nkv, 0.0), logit(j.nkv);
  std::vector<double> kd((size_t)j.nkv * D);
  for (int64_t t = 0; t < j.nkv * D; ++t) kd[t] = j.k[t];
  const double inv = 1.0 / std::sqrt((double)D);
  for (int64_t i = 0; i < j.nq; ++i) {
    double qd[D];
    for (int a = 0; a < D; ++a) qd[a] = j.q[i * D + a];
    double mx = -INFINITY;
    for (int64_t t = 0; t < j.nkv; ++t) {
      const double* kt = &kd[(size_t)t * D];
      double s = 0.0;
      for (int a = 0; a < D; ++a) s += qd[a] * kt[a];
      logit[t] = s * inv;
      mx = std::max(mx, logit[t]);
    }
    double den = 0.0;
    for (int64_t t = 0; t < j.nkv; ++t) den += (logit[t] = std::exp(logit[t] - mx));
    for (int64_t t = 0; t < j.nkv; ++t) wt[t] += logit[t] / den;
  }
  // Sigma_S = sum_t a_t v_t v_t^T / sum_t a_t
  std::vector<double> sv((size_t)D * D, 0.0);
  double wsum = 0.0;
  for (int64_t t = 0; t < j.nkv; ++t) {
    const float* vt = j.v + t * D;
    double w = wt[t];
    wsum += w;
    for (int a = 0; a < D; ++a) {
      double va = w * vt[a];
      for (int b = a; b < D; ++b) sv[(size_t)a * D + b] += va * (double)vt[b];
    }
  }
  for (int a = 0; a < D; ++a)
    for (int b = a; b < D; ++b) sv[(size_t)b * D + a] = sv[(size_t)a * D + b] /= wsum;

  std::vector<double> w, u;
  eig_desc(sq, w, u);
  rotation(u, j.rk);
  if (j.ek) std::copy(w.begin(), w.end(), j.ek);
  eig_desc(sv, w, u);
  rotation(u, j.rv);
  if (j.ev) std::copy(w.begin(), w.end(), j.ev);
}

bool finite_all(const float* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

}  // namespace

namespace {

// Calibrates n_layers x Hkv independent heads on a pool of host threads.
int calibrate_all(const oscar_shape* shape, int n_layers, const float* q_cal, int64_t n_q, const float* k_cal,
                  const float* v_cal, int64_t n_kv, uint16_t* r_k, uint16_t* r_v, double* eig_k, double* eig_v) {
  int st = oscar::check_shape(shape);
  if (st != OSCAR_OK) return st;
  if (!q_cal || !k_cal || !v_cal || !r_k || !r_v || n_q < 1 || n_kv < 1 || n_layers < 1) return OSCAR_EINVAL;
  const int64_t heads = (int64_t)n_layers * shape->n_kv_heads;
  if (!finite_all(q_cal, heads * n_q * D) || !finite_all(k_cal, heads * n_kv * D) ||
      !finite_all(v_cal, heads * n_kv * D))
    return OSCAR_EINVAL;
  std::vector<std::thread> pool;
  unsigned hw = std::max(1u, std::thread::hardware_concurrency());
  std::vector<HeadJob> jobs;
  for (int64_t h = 0; h < heads; ++h)  // layer-major: head h of the flattened [n_layers][Hkv]
    jobs.push_back(HeadJob{q_cal + (size_t)h * n_q * D, k_cal + (size_t)h * n_kv * D,
                           v_cal + (size_t)h * n_kv * D, n_q, n_kv, r_k + (size_t)h * D * D,
                           r_v + (size_t)h * D * D, eig_k ? eig_k + (size_t)h * D : nullptr,
                           eig_v ? eig_v + (size_t)h * D : nullptr});
  size_t next = 0;
  while (next < jobs.size()) {
    pool.clear();
    for (unsigned t = 0; t < hw && next < jobs.size(); ++t, ++next)
      pool.emplace_back(calibrate_head, std::cref(jobs[next]));
    for (auto& th : pool) th.join();
  }
  return OSCAR_OK;
}

}  // namespace

extern "C" int oscar_calibrate(const oscar_shape* shape, const float* q_cal, int64_t n_q,
                               const float* k_cal, const float* v_cal, int64_t n_kv, uint16_t* r_k,
                               uint16_t* r_v, double* eig_k, double* eig_v) {
  return calibrate_all(shape, 1, q_cal, n_q, k_cal, v_cal, n_kv, r_k, r_v, eig_k, eig_v);
}

extern "C" int oscar_calibrate_layers(const oscar_shape* shape, int32_t n_layers, const float* q_cal, int64_t n_q,
                                      const float* k_cal, const float* v_cal, int64_t n_kv, uint16_t* r_k,
                                      uint16_t* r_v, double* eig_k, double* eig_v) {
  return calibrate_all(shape, n_layers, q_cal, n_q, k_cal, v_cal, n_kv, r_k, r_v, eig_k, eig_v);
}
