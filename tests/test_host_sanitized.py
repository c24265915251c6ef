"""The library's host code (skv_api.cpp, eig_host.cpp) under AddressSanitizer,
LeakSanitizer and UBSan, on the CPU.

tests/host_mock_hip.cpp replaces the HIP runtime by a host mock (device memory
is host memory with a registry of live allocations) and the kernel launchers by
stubs that check the extent of every buffer they are handed.  Its driver runs
every entry point in each rebuild mode, value placement, selection mode and
new-token mode, the failure injection switches (the N-th device allocation of a
build failing: SKV_ERR_OOM and nothing left allocated; the N-th HIP call of a
decode step or append failing: SKV_ERR_HIP, then SKV_ERR_STATE from every later
call) and the slot poisoning switch.  The sanitizers abort on the first report;
the driver exits non-zero on the first failed check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_kv_cache_decode_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the HIP headers are not available")
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", CSRC,
             "-I", os.path.join(ROOT, "include")] + SANITIZE
    objs = []
    for src in ("skv_api.cpp", "eig_host.cpp"):
        obj = str(tmp_path / (src + ".o"))
        subprocess.run([gxx, *flags, "-c", os.path.join(CSRC, src), "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "mock")
    subprocess.run([gxx, *flags, os.path.join(ROOT, "tests", "host_mock_hip.cpp"), *objs, "-o", exe,
                    "-lpthread"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("SKV_INJECT_FAIL", None)
    env.pop("SKV_POISON_SLOTS", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    print(r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "failures 0 live blocks 0" in r.stdout
    assert "static-split launches 0" not in r.stdout
