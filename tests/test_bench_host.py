"""Host-side logic of bench.py on the CPU: the algorithmic byte model, the
counter-summary arithmetic (scaling by the calibration kernel, read back
through the source digest), the kernel-trace summary, and the one-GPU rule."""
import csv
import json
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_kv_cache_decode_amd import synth  # noqa: E402

CALIB = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, "
         "at::native::binary_internal::MulFunctor<float> >, std::array<char*, 2ul> >(int, "
         "at::native::AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> >, "
         "std::array<char*, 2ul>)")


def test_algorithmic_bytes_llama_shape():
    s = synth.SHAPES["llama3_8b_122k"]
    # P * n_cand landmarks of d bf16 values, plus the queries
    lm = s.pairs * s.n_cand * s.head_dim * 2
    q = s.batch * s.n_q_heads * s.head_dim * 2
    by = bench.algorithmic_bytes(s, 0.0)
    assert by["score"] == lm + q == 250904576
    # FP8 landmarks halve the landmark bytes; FP8 A halves the A rows of the misses
    by8 = bench.algorithmic_bytes(s.replace(landmark_format="e5m2"), 0.0)
    assert by8["score"] == lm // 2 + q
    m = 1000.0
    r16 = bench.algorithmic_bytes(s, m)["rebuild"]
    r8 = bench.algorithmic_bytes(s.replace(a_format="e5m2"), m)["rebuild"]
    assert r16 - r8 == m * s.chunk * s.rank
    # attention: K and V of every attended token
    out = s.batch * s.n_q_heads * s.head_dim * 4
    assert by["attention"] == s.pairs * s.tokens_attended * s.head_dim * 4 + out
    # rebuilt keys go to their slots (A rows + key per token), and B once per pair
    assert bench.algorithmic_bytes(s, m)["rebuild"] == m * s.chunk * (s.rank * 2 + s.head_dim * 2) + \
        s.pairs * s.rank * s.head_dim * 2
    # a fused rebuild attends the keys it rebuilt where it made them: those keys are
    # not read back; without the temporal cache it stores none either
    f = bench.algorithmic_bytes(s, m, fused=True)
    assert by_attn_keys_saved(bench.algorithmic_bytes(s, m), f) == m * s.chunk * s.head_dim * 2
    assert f["rebuild"] == bench.algorithmic_bytes(s, m)["rebuild"]
    every = s.pairs * s.top_k
    f3 = bench.algorithmic_bytes(s, every, fused=True, temporal=False)
    assert f3["rebuild"] == every * s.chunk * s.rank * 2 + s.pairs * s.rank * s.head_dim * 2
    assert f3["attention"] == s.pairs * s.tokens_attended * s.head_dim * 4 - every * s.chunk * s.head_dim * 2 + out


def by_attn_keys_saved(plain, fused):
    return plain["attention"] - fused["attention"]


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_calibration_kernel(monkeypatch):
    # the calibration kernel reads and writes CALIB_BYTES; FETCH_SIZE reports half
    # of the read bytes on this part, so reads scale by 2 and writes by 1
    half = bench.CALIB_BYTES / 1024 / 2
    full = bench.CALIB_BYTES / 1024
    score = "void skv::score_kernel<4>(skv::DecodeArgs)"
    with tempfile.TemporaryDirectory() as d:
        f, w = os.path.join(d, "f.csv"), os.path.join(d, "w.csv")
        _counter_csv(f, "FETCH_SIZE", [(score, 1000.0), (score, 3000.0)] + [(CALIB, half)] * 3)
        _counter_csv(w, "WRITE_SIZE", [(score, 10.0), (score, 30.0)] + [(CALIB, full)] * 3)
        text = bench.summarize_counters(f, w, "python3 bench.py ...")
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        assert blob["fetch_factor"] == 2.0 and blob["write_factor"] == 1.0
        k = blob["kernels"]["skv::score_kernel<4>"]
        assert k["dispatches"] == 2
        assert k["hbm_read_bytes"] == int(2000.0 * 1024 * 2) and k["hbm_write_bytes"] == int(20.0 * 1024)
        assert k["hbm_bytes_per_launch"] == k["hbm_read_bytes"] + k["hbm_write_bytes"]
        # read back only while the sources hash to the recorded digest
        prof = os.path.join(d, "profiles")
        os.makedirs(prof)
        open(os.path.join(prof, "x_hbm_traffic.md"), "w").write(text)
        monkeypatch.setattr(bench, "PROFILES", prof)
        assert bench.measured_traffic("llama3_8b_122k", "skv::score_kernel<4>") == k["hbm_bytes_per_launch"]
        monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
        assert bench.measured_traffic("llama3_8b_122k", "skv::score_kernel<4>") is None


def test_calibration_must_close_the_run():
    with tempfile.TemporaryDirectory() as d:
        f = os.path.join(d, "f.csv")
        _counter_csv(f, "FETCH_SIZE", [(CALIB, 1.0)] * 3 + [("void skv::x(int)", 1.0)])
        with pytest.raises(AssertionError):
            bench._calibration(bench._counter_rows(f, "FETCH_SIZE"))


def test_trace_summary_reports_the_score_rate():
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "stats.csv")
        with open(p, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
            w.writeheader()
            w.writerow({"Name": "void skv::score_kernel<4>(skv::DecodeArgs)", "Calls": 10,
                        "TotalDurationNs": 500000, "AverageNs": 50000, "MinNs": 49000, "MaxNs": 51000})
            w.writerow({"Name": "some_other_kernel", "Calls": 1, "TotalDurationNs": 1, "AverageNs": 1,
                        "MinNs": 1, "MaxNs": 1})
        text = bench.summarize_trace(p, "python3 bench.py")
        assert "`skv::score_kernel<4>` | 10 | 50.00" in text and "some_other_kernel" not in text
        # 250 904 576 bytes in 50 us
        assert "5018 GB/s (0.627 of 8 TB/s)" in text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_score_kernel_follows_the_group_size():
    s = synth.SHAPES["glm4_9b_1m"]
    assert bench.score_kernel_name(s) == "skv::score_kernel<16>"
    assert bench.score_kernel_name(s.replace(landmark_format="e5m2")) == "skv::score_fp8_kernel<16>"
    assert bench.score_kernel_name(synth.SHAPES["llama3_8b_122k"]) == "skv::score_kernel<4>"
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "stats.csv")
        with open(p, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
            w.writeheader()
            w.writerow({"Name": "void skv::score_kernel<16>(skv::DecodeArgs)", "Calls": 1, "TotalDurationNs": 60000,
                        "AverageNs": 60000, "MinNs": 60000, "MaxNs": 60000})
        text = bench.summarize_trace(p, "python3 bench.py --shape glm4_9b_1m", s)
        by = bench.algorithmic_bytes(s, 0.0)["score"]
        assert "glm4_9b_1m" in text and f"{by} algorithmic bytes per launch / 60.00 us" in text
