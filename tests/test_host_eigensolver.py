"""Host part of the pre-fill eigensolver (csrc/eig_host.cpp), on the CPU.

The symmetric p x p eigenproblem of the Rayleigh-Ritz step (Householder
tridiagonalisation + implicit QR) and the Cholesky factor inverse of the block
orthonormalisation are compiled from the library's own source into a small
driver (the GPU products are stubbed out: these two routines never call them)
and checked against their definitions: A v = lambda v with orthonormal v,
eigenvalues equal to numpy.linalg.eigvalsh, and R^-T W R^-1 = I."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_cache_decode_amd", "csrc")

DRIVER = r'''
#include "eig_host.cpp"
#include <cstdio>
namespace skv {
hipError_t launch_gemm_f64(const double*, const double*, double*, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_gemm_f64_tn(const double*, const double*, double*, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
}
// in: mode (0 eig, 1 chol), p, p*p doubles; out: ok, then w (p) and vt (p*p), or rinv (p*p)
int main(int argc, char** argv) {
  FILE* f = fopen(argv[1], "rb");
  int mode, p;
  if (fread(&mode, 4, 1, f) != 1 || fread(&p, 4, 1, f) != 1) return 2;
  std::vector<double> a((size_t)p * p);
  if (fread(a.data(), 8, a.size(), f) != a.size()) return 2;
  fclose(f);
  FILE* o = fopen(argv[2], "wb");
  if (mode == 0) {
    std::vector<double> w, vt;
    int ok = skv::sym_eig(a, p, w, vt) ? 1 : 0;
    fwrite(&ok, 4, 1, o);
    fwrite(w.data(), 8, p, o);
    fwrite(vt.data(), 8, (size_t)p * p, o);
  } else {
    std::vector<double> ri((size_t)p * p);
    int ok = skv::chol_inverse(a.data(), p, ri.data()) ? 1 : 0;
    fwrite(&ok, 4, 1, o);
    fwrite(ri.data(), 8, ri.size(), o);
  }
  fclose(o);
  return 0;
}
'''


@pytest.fixture(scope="module")
def driver():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "drv.cpp")
    open(src, "w").write(DRIVER)
    exe = os.path.join(d, "drv")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-Wno-unused-result", "-Wno-unused-value",
                    "-I", CSRC, "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                   check=True, capture_output=True)
    yield exe, d
    shutil.rmtree(d, ignore_errors=True)


def _call(driver, mode, a):
    exe, d = driver
    p = a.shape[0]
    fin, fout = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
    with open(fin, "wb") as f:
        np.array([mode, p], np.int32).tofile(f)
        np.ascontiguousarray(a, np.float64).tofile(f)
    subprocess.run([exe, fin, fout], check=True)
    raw = open(fout, "rb").read()
    ok = int(np.frombuffer(raw[:4], np.int32)[0])
    vals = np.frombuffer(raw[4:], np.float64)
    return ok, vals


def _sym(rng, p, spectrum):
    q, _ = np.linalg.qr(rng.standard_normal((p, p)))
    return (q * spectrum) @ q.T


@pytest.mark.parametrize("p,kind", [(1, "random"), (2, "random"), (3, "random"), (57, "random"),
                                    (200, "random"), (200, "graded"), (64, "clustered"), (40, "zero"),
                                    (30, "tridiagonal")])
def test_sym_eig(driver, p, kind):
    rng = np.random.default_rng(p)
    if kind == "random":
        a = rng.standard_normal((p, p))
        a = a + a.T
    elif kind == "graded":           # Ritz values spanning 8 decades
        a = _sym(rng, p, np.logspace(4, -4, p))
    elif kind == "clustered":        # repeated eigenvalues
        a = _sym(rng, p, np.repeat([5.0, 1.0, -2.0, 0.0], p // 4))
    elif kind == "zero":
        a = np.zeros((p, p))
    else:                            # already tridiagonal (second differences)
        a = 2 * np.eye(p) - np.eye(p, k=1) - np.eye(p, k=-1)
    ok, vals = _call(driver, 0, a)
    assert ok == 1
    w, vt = vals[:p], vals[p:].reshape(p, p)
    scale = max(1.0, np.abs(a).max())
    np.testing.assert_allclose(np.sort(w), np.linalg.eigvalsh(a), atol=1e-12 * scale * p)
    np.testing.assert_allclose(vt @ vt.T, np.eye(p), atol=1e-13 * p)
    assert np.abs(a @ vt.T - vt.T * w).max() <= 1e-12 * scale * p


def test_cholesky_inverse(driver):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 40))
    w = x.T @ x
    ok, vals = _call(driver, 1, w)
    assert ok == 1
    ri = vals.reshape(40, 40)
    assert np.allclose(np.tril(ri, -1), 0.0)
    np.testing.assert_allclose(ri.T @ w @ ri, np.eye(40), atol=1e-12)
    # a rank-deficient block is refused (the caller then orthonormalises on the host)
    x[:, 7] = x[:, 3]
    ok, _ = _call(driver, 1, x.T @ x)
    assert ok == 0
