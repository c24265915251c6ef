// Top-r eigenvectors of the fp64 Gram matrices K_b^T K_b, i.e. the right singular
// vectors of the rank-r truncated SVD the pre-fill stores (K ~ A B with
// A = K Psi = U_r Sigma_r, B = Psi^T).
//
// Method: block subspace iteration with Rayleigh-Ritz (Golub & Van Loan,
// "Matrix Computations", orthogonal iteration and the Rayleigh-Ritz procedure).
// Every n x p product runs on the GPU in fp64: Y = G Q, the Gram matrices of the
// blocks and the products with p x p factors.  The blocks are orthonormalised by
// Cholesky QR (W = X^T X = R^T R on the host, X <- X R^-1 on the GPU), once
// between power steps and twice before each Rayleigh-Ritz step (a block that
// is orthonormal only to about kappa^2 eps still spans the right subspace for
// the next power step), falling back to modified Gram-Schmidt on the host if a
// factor breaks down; the p x p Rayleigh-Ritz eigenproblem is solved on the host by Householder
// tridiagonalisation and the implicit symmetric QR algorithm with Wilkinson
// shifts (ibid., 8.3), one thread per batch element.  Converged when every wanted
// Ritz pair has residual ||G u - theta u|| <= 1e-11 * theta_max.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
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

// Eigen-decomposition of a symmetric p x p matrix (row-major `a`, destroyed):
// Householder reduction to tridiagonal form with the reflections accumulated in
// vt, then implicit QR sweeps with Wilkinson shifts on the tridiagonal (d, e),
// each sweep a chain of plane rotations in planes (k, k+1) that chases the bulge
// down the block, accumulated into vt as well.  Eigenvalues in w (unsorted),
// eigenvectors as the rows of vt (row-major, so that a rotation touches two
// contiguous rows).  False if a block does not converge within 50 p sweeps.
bool sym_eig(std::vector<double>& a, int p, std::vector<double>& w, std::vector<double>& vt) {
  auto A = [&](int i, int j) -> double& { return a[(size_t)i * p + j]; };
  vt.assign((size_t)p * p, 0.0);
  for (int i = 0; i < p; i++) vt[(size_t)i * p + i] = 1.0;
  std::vector<double> tv(p);
  std::vector<double> hv(p), u(p), wv(p);
  for (int k = 0; k + 2 < p; k++) {
    // reflection H = I - beta hv hv^T that maps column k below the diagonal onto
    // its first entry
    const int m = p - k - 1;
    double nx = 0.0;
    for (int i = 0; i < m; i++) nx += A(k + 1 + i, k) * A(k + 1 + i, k);
    nx = std::sqrt(nx);
    if (nx == 0.0) continue;
    const double alpha = A(k + 1, k) > 0 ? -nx : nx;
    for (int i = 0; i < m; i++) hv[i] = A(k + 1 + i, k);
    hv[0] -= alpha;
    double vn = 0.0;
    for (int i = 0; i < m; i++) vn += hv[i] * hv[i];
    if (vn == 0.0) continue;
    const double beta = 2.0 / vn;
    // trailing block: H A22 H = A22 - hv w^T - w hv^T with w = u - (beta/2)(u.hv) hv, u = beta A22 hv
    for (int i = 0; i < m; i++) {
      double t = 0.0;
      for (int j = 0; j < m; j++) t += A(k + 1 + i, k + 1 + j) * hv[j];
      u[i] = beta * t;
    }
    double uv = 0.0;
    for (int i = 0; i < m; i++) uv += u[i] * hv[i];
    for (int i = 0; i < m; i++) wv[i] = u[i] - 0.5 * beta * uv * hv[i];
    for (int i = 0; i < m; i++)
      for (int j = 0; j < m; j++) A(k + 1 + i, k + 1 + j) -= hv[i] * wv[j] + wv[i] * hv[j];
    A(k + 1, k) = A(k, k + 1) = alpha;
    for (int i = 1; i < m; i++) A(k + 1 + i, k) = A(k, k + 1 + i) = 0.0;
    // V <- V H, i.e. rows k+1.. of vt: vt_j -= beta hv_j (sum_i hv_i vt_i)
    std::fill(tv.begin(), tv.end(), 0.0);
    for (int j = 0; j < m; j++) {
      const double* row = &vt[(size_t)(k + 1 + j) * p];
      for (int c = 0; c < p; c++) tv[c] += hv[j] * row[c];
    }
    for (int j = 0; j < m; j++) {
      double* row = &vt[(size_t)(k + 1 + j) * p];
      const double f = beta * hv[j];
      for (int c = 0; c < p; c++) row[c] -= f * tv[c];
    }
  }
  std::vector<double> d(p), e(p, 0.0);
  for (int i = 0; i < p; i++) d[i] = A(i, i);
  for (int i = 0; i + 1 < p; i++) e[i] = A(i, i + 1);
  auto negligible = [&](int i) {
    return std::fabs(e[i]) <= DBL_EPSILON * (std::fabs(d[i]) + std::fabs(d[i + 1]));
  };
  int hi = p - 1, sweeps = 0;
  while (hi > 0) {
    if (negligible(hi - 1)) {   // d[hi] has converged
      e[hi - 1] = 0.0;
      hi--;
      continue;
    }
    if (++sweeps > 50 * p) return false;
    int lo = hi - 1;            // the unreduced block [lo, hi]
    while (lo > 0 && !negligible(lo - 1)) lo--;
    // Wilkinson shift: the eigenvalue of the trailing 2x2 block closer to d[hi]
    const double dd = 0.5 * (d[hi - 1] - d[hi]), b2 = e[hi - 1] * e[hi - 1];
    const double mu = d[hi] - b2 / (dd + std::copysign(std::sqrt(dd * dd + b2), dd));
    // rotation k acts on rows/columns (k, k+1) as [c s; -s c]; (x, z) is the pair
    // it annihilates: the shifted first column for k = lo, else (e[k-1], bulge)
    double x = d[lo] - mu, z = e[lo];
    for (int k = lo; k < hi; k++) {
      const double rr = std::hypot(x, z);
      const double c = rr == 0.0 ? 1.0 : x / rr, sn = rr == 0.0 ? 0.0 : z / rr;
      if (k > lo) e[k - 1] = rr;
      const double a0 = d[k], a1 = d[k + 1], bb = e[k];
      d[k] = c * c * a0 + 2.0 * c * sn * bb + sn * sn * a1;
      d[k + 1] = sn * sn * a0 - 2.0 * c * sn * bb + c * c * a1;
      e[k] = c * sn * (a1 - a0) + (c * c - sn * sn) * bb;
      if (k + 1 < hi) {          // the rotation pushes a bulge to (k, k+2)
        z = sn * e[k + 1];
        e[k + 1] *= c;
        x = e[k];
      }
      double* r0 = &vt[(size_t)k * p];
      double* r1 = &vt[(size_t)(k + 1) * p];
      for (int col = 0; col < p; col++) {
        const double y0 = r0[col], y1 = r1[col];
        r0[col] = c * y0 + sn * y1;
        r1[col] = -sn * y0 + c * y1;
      }
    }
  }
  w = d;
  return true;
}

// W = R^T R (R upper triangular, W symmetric p x p); rinv = R^-1 (row-major).
// False if a pivot is not clearly positive (X too close to rank deficient).
bool chol_inverse(const double* W, int p, double* rinv) {
  std::vector<double> R((size_t)p * p, 0.0);
  for (int j = 0; j < p; j++) {
    double s = W[(size_t)j * p + j];
    for (int k = 0; k < j; k++) s -= R[(size_t)k * p + j] * R[(size_t)k * p + j];
    if (!(s > 1e-14 * W[(size_t)j * p + j]) || !(s > 0.0)) return false;
    const double rjj = std::sqrt(s);
    R[(size_t)j * p + j] = rjj;
    for (int i = j + 1; i < p; i++) {
      double t = W[(size_t)j * p + i];
      for (int k = 0; k < j; k++) t -= R[(size_t)k * p + j] * R[(size_t)k * p + i];
      R[(size_t)j * p + i] = t / rjj;
    }
  }
  std::fill(rinv, rinv + (size_t)p * p, 0.0);
  for (int j = 0; j < p; j++) {   // column j of R^-1 by back substitution
    rinv[(size_t)j * p + j] = 1.0 / R[(size_t)j * p + j];
    for (int i = j - 1; i >= 0; i--) {
      double t = 0.0;
      for (int k = i + 1; k <= j; k++) t += R[(size_t)i * p + k] * rinv[(size_t)k * p + j];
      rinv[(size_t)i * p + j] = -t / R[(size_t)i * p + i];
    }
  }
  return true;
}

}  // namespace

int top_eigvecs(const double* gram_dev, int b, int n, int r, hipStream_t st, double* psi,
                double* eig, hipError_t* err) {
  *err = hipSuccess;
  const int p = std::min(n, r + std::max(16, r / 4));
  const size_t blk = (size_t)n * p, sq = (size_t)p * p;
  std::vector<double> hq(blk * b), hy(blk * b), hs(sq * b), hv(sq * b), ufinal(blk * b);
  std::vector<std::vector<double>> theta(b);
  std::vector<char> done(b, 0);
  double* dev = nullptr;   // q, y, t, u (n x p blocks), s (p x p blocks)
  if ((*err = hipMalloc(&dev, (4 * blk + sq) * b * sizeof(double))) != hipSuccess) return 2;
  double *dq = dev, *dy = dq + blk * b, *dt = dy + blk * b, *du = dt + blk * b, *ds = du + blk * b;
  const int nthreads = std::max(1, std::min(b, (int)std::thread::hardware_concurrency()));
  auto parallel = [&](auto fn) {
    std::vector<std::thread> th;
    for (int t = 0; t < nthreads; t++)
      th.emplace_back([&, t] {
        for (int bi = t; bi < b; bi += nthreads) fn(bi);
      });
    for (auto& x : th) x.join();
  };
  auto copy = [&](void* dst, const void* src, size_t doubles, hipMemcpyKind kind) {
    return (*err = hipMemcpyAsync(dst, src, doubles * sizeof(double), kind, st)) == hipSuccess;
  };
  auto sync = [&] { return (*err = hipStreamSynchronize(st)) == hipSuccess; };
  auto ok = [&](hipError_t e) { return (*err = e) == hipSuccess; };
  // orthonormalise the columns of every block of x (device) in place
  auto orth = [&](double* x, int passes) -> bool {
    for (int pass = 0; pass < passes; pass++) {
      if (!ok(launch_gemm_f64_tn(x, x, ds, b, p, p, n, st)) || !copy(hs.data(), ds, sq * b, hipMemcpyDeviceToHost) ||
          !sync())
        return false;
      std::vector<char> bad(b, 0);
      parallel([&](int bi) { bad[bi] = !chol_inverse(&hs[sq * bi], p, &hv[sq * bi]); });
      if (std::find(bad.begin(), bad.end(), 1) != bad.end()) {
        // a block too close to rank deficient for Cholesky QR: Gram-Schmidt on the host
        if (!copy(hq.data(), x, blk * b, hipMemcpyDeviceToHost) || !sync()) return false;
        parallel([&](int bi) { orthonormalise(&hq[blk * bi], n, p); });
        return copy(x, hq.data(), blk * b, hipMemcpyHostToDevice) && sync();
      }
      if (!copy(ds, hv.data(), sq * b, hipMemcpyHostToDevice) || !ok(launch_gemm_f64(x, ds, dt, b, n, p, p, st)) ||
          !copy(x, dt, blk * b, hipMemcpyDeviceToDevice))
        return false;
    }
    return true;
  };
  for (int bi = 0; bi < b; bi++) start_block(&hq[blk * bi], n, p, 0x5eedull + (uint64_t)bi);
  int status = 2;
  const bool square = (p == n);   // q spans everything: one Rayleigh-Ritz is exact
  if (copy(dq, hq.data(), blk * b, hipMemcpyHostToDevice) && orth(dq, 2)) {
    status = 1;
    for (int round = 0; round < 60; round++) {
      bool good = true;
      for (int it = 0; it < (square ? 0 : 3) && good; it++)
        good = ok(launch_gemm_f64(gram_dev, dq, dy, b, n, p, n, st)) &&
               copy(dq, dy, blk * b, hipMemcpyDeviceToDevice) && orth(dq, it == 2 ? 2 : 1);
      // Rayleigh-Ritz: H = Q^T G Q, H = V diag(theta) V^T, U = Q V, residuals G U - U diag(theta)
      good = good && ok(launch_gemm_f64(gram_dev, dq, dy, b, n, p, n, st)) &&
             ok(launch_gemm_f64_tn(dq, dy, ds, b, p, p, n, st)) &&
             copy(hs.data(), ds, sq * b, hipMemcpyDeviceToHost) && sync();
      if (!good) {
        status = 2;
        break;
      }
      std::vector<char> failed(b, 0);
      parallel([&](int bi) {
        double* h = &hs[sq * bi];
        double* vs = &hv[sq * bi];
        if (done[bi]) {   // keep the block (identity); its results are not used
          std::fill(vs, vs + sq, 0.0);
          for (int i = 0; i < p; i++) vs[(size_t)i * p + i] = 1.0;
          return;
        }
        std::vector<double> hm(h, h + sq), w, v;
        for (int i = 0; i < p; i++)
          for (int j = i + 1; j < p; j++) hm[(size_t)i * p + j] = hm[(size_t)j * p + i] =
                                              0.5 * (h[(size_t)i * p + j] + h[(size_t)j * p + i]);
        if (!sym_eig(hm, p, w, v)) {
          failed[bi] = 1;
          return;
        }
        std::vector<int> ord(p);
        for (int i = 0; i < p; i++) ord[i] = i;
        std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) { return w[x] > w[y]; });
        theta[bi].resize(p);
        for (int j = 0; j < p; j++) {
          theta[bi][j] = w[ord[j]];
          for (int i = 0; i < p; i++) vs[(size_t)i * p + j] = v[(size_t)ord[j] * p + i];
        }
      });
      if (std::find(failed.begin(), failed.end(), 1) != failed.end()) break;   // status 1
      good = copy(ds, hv.data(), sq * b, hipMemcpyHostToDevice) && ok(launch_gemm_f64(dq, ds, du, b, n, p, p, st)) &&
             ok(launch_gemm_f64(dy, ds, dt, b, n, p, p, st)) &&
             copy(hq.data(), du, blk * b, hipMemcpyDeviceToHost) &&
             copy(hy.data(), dt, blk * b, hipMemcpyDeviceToHost) && sync();
      if (!good) {
        status = 2;
        break;
      }
      parallel([&](int bi) {
        if (done[bi]) return;
        const double* u = &hq[blk * bi];
        const double* yv = &hy[blk * bi];
        std::vector<double> res(r, 0.0);
        for (int i = 0; i < n; i++)
          for (int j = 0; j < r; j++) {
            const double e = yv[(size_t)i * p + j] - theta[bi][j] * u[(size_t)i * p + j];
            res[j] += e * e;
          }
        const double scale = std::max(std::fabs(theta[bi][0]), 1e-300);
        double worst = 0.0;
        for (int j = 0; j < r; j++) worst = std::max(worst, std::sqrt(res[j]) / scale);
        if (worst <= 1e-11 || square) {
          done[bi] = 1;
          std::memcpy(&ufinal[blk * bi], u, blk * sizeof(double));
        }
      });
      if (std::find(done.begin(), done.end(), 0) == done.end()) {
        status = 0;
        break;
      }
      // restart from the Ritz vectors (orthonormal)
      if (!copy(dq, du, blk * b, hipMemcpyDeviceToDevice)) {
        status = 2;
        break;
      }
    }
  }
  (void)hipStreamSynchronize(st);
  (void)hipFree(dev);
  if (status != 0) return status;
  // first r Ritz vectors, sign gauge: largest-|.| entry positive (lowest index on ties)
  for (int bi = 0; bi < b; bi++) {
    const double* ub = &ufinal[blk * bi];
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
