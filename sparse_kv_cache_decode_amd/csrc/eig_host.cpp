// Top-r eigenvectors of the fp64 Gram matrices K_b^T K_b, i.e. the right singular
// vectors of the rank-r truncated SVD the pre-fill stores (K ~ A B with
// A = K Psi = U_r Sigma_r, B = Psi^T).
//
// Method: block subspace iteration with Rayleigh-Ritz (Golub & Van Loan,
// "Matrix Computations", orthogonal iteration and the Rayleigh-Ritz procedure).
// Y = G Q runs on the GPU (fp64); the orthonormalisation (modified Gram-Schmidt,
// applied twice) and the small p x p eigenproblems (cyclic Jacobi) run on the host
// in fp64, one thread per batch element.  Converged when every wanted Ritz pair
// has residual ||G u - theta u|| <= 1e-11 * theta_max.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "skv_internal.h"

namespace skv {
namespace {

// Deterministic start block: splitmix64 -> uniform(-1, 1).
void start_block(double* q, int n, int p, uint64_t seed) {
  uint64_t x = seed;
  for (int64_t i = 0; i < (int64_t)n * p; i++) {
    x += 0x9e3779b97f4a7c15ull;
    uint64_t z = x;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    q[i] = (double)(z >> 11) * (2.0 / 9007199254740992.0) - 1.0;
  }
}

// Orthonormalise the p columns of q (n x p, row-major) in place: modified
// Gram-Schmidt, twice.  Works on a column-major copy for unit-stride loops.
void orthonormalise(double* q, int n, int p) {
  std::vector<double> c((size_t)n * p);
  for (int i = 0; i < n; i++)
    for (int j = 0; j < p; j++) c[(size_t)j * n + i] = q[(size_t)i * p + j];
  for (int rep = 0; rep < 2; rep++) {
    for (int j = 0; j < p; j++) {
      double* cj = &c[(size_t)j * n];
      for (int k = 0; k < j; k++) {
        const double* ck = &c[(size_t)k * n];
        double d = 0.0;
        for (int i = 0; i < n; i++) d += ck[i] * cj[i];
        for (int i = 0; i < n; i++) cj[i] -= d * ck[i];
      }
      double nn = 0.0;
      for (int i = 0; i < n; i++) nn += cj[i] * cj[i];
      nn = std::sqrt(nn);
      const double inv = nn > 0 ? 1.0 / nn : 0.0;
      for (int i = 0; i < n; i++) cj[i] *= inv;
    }
  }
  for (int i = 0; i < n; i++)
    for (int j = 0; j < p; j++) q[(size_t)i * p + j] = c[(size_t)j * n + i];
}

// Cyclic Jacobi for a symmetric p x p matrix h (row-major, destroyed): eigenvalues
// in w, eigenvectors as columns of v.
void jacobi_eig(std::vector<double>& h, int p, std::vector<double>& w, std::vector<double>& v) {
  v.assign((size_t)p * p, 0.0);
  for (int i = 0; i < p; i++) v[(size_t)i * p + i] = 1.0;
  auto A = [&](int i, int j) -> double& { return h[(size_t)i * p + j]; };
  for (int sweep = 0; sweep < 100; sweep++) {
    double off = 0.0, tot = 0.0;
    for (int i = 0; i < p; i++)
      for (int j = 0; j < p; j++) {
        const double x = A(i, j) * A(i, j);
        tot += x;
        if (i != j) off += x;
      }
    if (off <= 1e-30 * tot) break;
    for (int a = 0; a < p - 1; a++)
      for (int b = a + 1; b < p; b++) {
        const double apq = A(a, b);
        if (std::fabs(apq) < 1e-300) continue;
        const double tau = (A(b, b) - A(a, a)) / (2.0 * apq);
        const double t = (tau >= 0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
        const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
        for (int k = 0; k < p; k++) {   // columns a, b
          const double x = A(k, a), y = A(k, b);
          A(k, a) = c * x - s * y;
          A(k, b) = s * x + c * y;
        }
        for (int k = 0; k < p; k++) {   // rows a, b
          const double x = A(a, k), y = A(b, k);
          A(a, k) = c * x - s * y;
          A(b, k) = s * x + c * y;
        }
        for (int k = 0; k < p; k++) {
          double* vr = &v[(size_t)k * p];
          const double x = vr[a], y = vr[b];
          vr[a] = c * x - s * y;
          vr[b] = s * x + c * y;
        }
      }
  }
  w.resize(p);
  for (int i = 0; i < p; i++) w[i] = A(i, i);
}

// Rayleigh-Ritz on span(q) with y = G q: fills u (n x p Ritz vectors, descending
// Ritz values theta) and returns the largest relative residual among the first r.
double rayleigh_ritz(const double* q, const double* y, int n, int p, int r, double* u,
                     std::vector<double>& theta) {
  std::vector<double> h((size_t)p * p, 0.0);
  for (int i = 0; i < n; i++) {
    const double* qi = q + (size_t)i * p;
    const double* yi = y + (size_t)i * p;
    for (int a = 0; a < p; a++) {
      const double x = qi[a];
      double* ha = &h[(size_t)a * p];
      for (int b = 0; b < p; b++) ha[b] += x * yi[b];
    }
  }
  for (int a = 0; a < p; a++)
    for (int b = a + 1; b < p; b++) {
      const double m = 0.5 * (h[(size_t)a * p + b] + h[(size_t)b * p + a]);
      h[(size_t)a * p + b] = h[(size_t)b * p + a] = m;
    }
  std::vector<double> w, v;
  jacobi_eig(h, p, w, v);
  std::vector<int> ord(p);
  for (int i = 0; i < p; i++) ord[i] = i;
  std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return w[a] > w[b]; });
  theta.resize(p);
  for (int j = 0; j < p; j++) theta[j] = w[ord[j]];
  // u = q V_sorted, yv = y V_sorted; residual of column j = ||yv_j - theta_j u_j||
  std::vector<double> res(p, 0.0);
  std::vector<double> urow(p), yrow(p);
  for (int i = 0; i < n; i++) {
    const double* qi = q + (size_t)i * p;
    const double* yi = y + (size_t)i * p;
    std::fill(urow.begin(), urow.end(), 0.0);
    std::fill(yrow.begin(), yrow.end(), 0.0);
    for (int a = 0; a < p; a++) {
      const double xq = qi[a], xy = yi[a];
      const double* va = &v[(size_t)a * p];
      for (int j = 0; j < p; j++) {
        const double vv = va[ord[j]];
        urow[j] += xq * vv;
        yrow[j] += xy * vv;
      }
    }
    for (int j = 0; j < p; j++) {
      u[(size_t)i * p + j] = urow[j];
      const double e = yrow[j] - theta[j] * urow[j];
      res[j] += e * e;
    }
  }
  const double scale = std::max(std::fabs(theta[0]), 1e-300);
  double worst = 0.0;
  for (int j = 0; j < r; j++) worst = std::max(worst, std::sqrt(res[j]) / scale);
  return worst;
}

}  // namespace

int top_eigvecs(const double* gram_dev, int b, int n, int r, hipStream_t st, double* psi,
                double* eig, hipError_t* err) {
  *err = hipSuccess;
  const int p = std::min(n, r + std::max(16, r / 4));
  const size_t blk = (size_t)n * p;
  std::vector<double> q(blk * b), y(blk * b), u(blk * b);
  for (int bi = 0; bi < b; bi++) {
    start_block(&q[blk * bi], n, p, 0x5eedull + (uint64_t)bi);
  }
  double* dq = nullptr;
  double* dy = nullptr;
  if ((*err = hipMalloc(&dq, blk * b * sizeof(double))) != hipSuccess) return 2;
  if ((*err = hipMalloc(&dy, blk * b * sizeof(double))) != hipSuccess) {
    hipFree(dq);
    return 2;
  }
  const int nthreads = std::max(1, std::min(b, (int)std::thread::hardware_concurrency()));
  auto parallel = [&](auto fn) {
    std::vector<std::thread> th;
    for (int t = 0; t < nthreads; t++)
      th.emplace_back([&, t] {
        for (int bi = t; bi < b; bi += nthreads) fn(bi);
      });
    for (auto& x : th) x.join();
  };
  auto multiply = [&]() -> bool {   // y = G q for every batch element
    if ((*err = hipMemcpyAsync(dq, q.data(), blk * b * sizeof(double), hipMemcpyHostToDevice, st)) != hipSuccess) return false;
    if ((*err = launch_gemm_f64(gram_dev, dq, dy, b, n, p, n, st)) != hipSuccess) return false;
    if ((*err = hipMemcpyAsync(y.data(), dy, blk * b * sizeof(double), hipMemcpyDeviceToHost, st)) != hipSuccess) return false;
    return (*err = hipStreamSynchronize(st)) == hipSuccess;
  };
  parallel([&](int bi) { orthonormalise(&q[blk * bi], n, p); });
  std::vector<std::vector<double>> theta(b);
  std::vector<char> done(b, 0);
  int status = 1;
  const bool square = (p == n);   // q spans everything: one Rayleigh-Ritz is exact
  for (int round = 0; round < 60; round++) {
    const int iters = square ? 0 : 3;
    bool ok = true;
    for (int it = 0; it < iters && ok; it++) {
      ok = multiply();
      if (ok) parallel([&](int bi) {
          if (done[bi]) return;
          std::memcpy(&q[blk * bi], &y[blk * bi], blk * sizeof(double));
          orthonormalise(&q[blk * bi], n, p);
        });
    }
    if (!ok || !multiply()) {
      status = 2;
      break;
    }
    std::vector<double> worst(b, 0.0);
    parallel([&](int bi) {
      if (done[bi]) return;
      worst[bi] = rayleigh_ritz(&q[blk * bi], &y[blk * bi], n, p, r, &u[blk * bi], theta[bi]);
    });
    bool all = true;
    for (int bi = 0; bi < b; bi++) {
      if (done[bi]) continue;
      if (worst[bi] <= 1e-11 || square) {
        done[bi] = 1;
      } else {
        all = false;
        // restart from the Ritz vectors (already orthonormal)
        std::memcpy(&q[blk * bi], &u[blk * bi], blk * sizeof(double));
      }
    }
    if (all) {
      status = 0;
      break;
    }
  }
  hipFree(dq);
  hipFree(dy);
  if (status != 0) return status;
  // first r Ritz vectors, sign gauge: largest-|.| entry positive (lowest index on ties)
  for (int bi = 0; bi < b; bi++) {
    const double* ub = &u[blk * bi];
    double* pb = psi + (size_t)bi * n * r;
    for (int j = 0; j < r; j++) {
      int arg = 0;
      double best = -1.0;
      for (int i = 0; i < n; i++) {
        const double a = std::fabs(ub[(size_t)i * p + j]);
        if (a > best) {
          best = a;
          arg = i;
        }
      }
      const double sg = ub[(size_t)arg * p + j] < 0 ? -1.0 : 1.0;
      for (int i = 0; i < n; i++) pb[(size_t)i * r + j] = sg * ub[(size_t)i * p + j];
      eig[(size_t)bi * r + j] = theta[bi][j];
    }
  }
  return 0;
}

}  // namespace skv
