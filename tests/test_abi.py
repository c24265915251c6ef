"""C ABI of libskv.so without a GPU: exported symbols, status codes, argument
validation (which runs before any HIP call) and struct layouts."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from sparse_kv_cache_decode_amd import skv, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skv.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:skv_status|void|const char\*|int32_t)\s+(skv_\w+)\s*\(",
                                 text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10
    lib = skv.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(skv.EXPORTED)


def test_status_strings_and_version():
    assert skv.skv_abi_version() == 8
    seen = set()
    for code in range(9):
        s = skv.skv_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert skv.skv_status_string(99) == "unknown status"


def _build_status(cfg, kp=1 << 20, vp=1 << 20):
    h = ctypes.c_void_p()
    return skv.lib().skv_build(ctypes.byref(cfg) if cfg is not None else None, kp, vp, None,
                               ctypes.byref(h)), h.value


def _cfg(**kw):
    c = skv.make_config(synth.SHAPES["tiny_8k"])
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=64), skv.SKV_ERR_UNSUPPORTED),
    (dict(n_q_heads=30), skv.SKV_ERR_SHAPE),                 # 30 % 8 != 0
    (dict(n_q_heads=24), skv.SKV_ERR_UNSUPPORTED),           # G = 3
    (dict(seq_len=8190), skv.SKV_ERR_SHAPE),                 # S % C != 0
    (dict(chunk=6), skv.SKV_ERR_UNSUPPORTED),
    (dict(window=12), skv.SKV_ERR_SHAPE),                    # W % C != 0
    (dict(top_k=0), skv.SKV_ERR_SHAPE),
    (dict(top_k=1022), skv.SKV_ERR_SHAPE),                   # > n_cand = 1017
    (dict(n_outlier=-1), skv.SKV_ERR_SHAPE),
    (dict(n_outlier=1020), skv.SKV_ERR_SHAPE),               # no candidate left
    (dict(rank=0), skv.SKV_ERR_SHAPE),
    (dict(rank=1040), skv.SKV_ERR_SHAPE),                    # > H_kv * d = 1024
    (dict(rank=100), skv.SKV_ERR_UNSUPPORTED),               # rank % 16 != 0
    (dict(rope_theta=0.0), skv.SKV_ERR_SHAPE),
    (dict(value_placement=2), skv.SKV_ERR_INVALID_ARG),
    (dict(temporal_cache=3), skv.SKV_ERR_INVALID_ARG),
    (dict(landmark_format=2), skv.SKV_ERR_INVALID_ARG),
    (dict(a_format=-1), skv.SKV_ERR_INVALID_ARG),
    (dict(b_format=7), skv.SKV_ERR_INVALID_ARG),
    (dict(batch=0), skv.SKV_ERR_SHAPE),
    (dict(max_new_tokens=-1), skv.SKV_ERR_SHAPE),
    (dict(new_token_mode=2), skv.SKV_ERR_INVALID_ARG),
    (dict(rebuild_mode=4), skv.SKV_ERR_INVALID_ARG),
    (dict(rebuild_mode=skv.SKV_REBUILD_OVERLAP, value_placement=skv.SKV_VALUES_HOST), skv.SKV_ERR_UNSUPPORTED),
    (dict(select_mode=2), skv.SKV_ERR_INVALID_ARG),
    (dict(rebuild_mode=skv.SKV_REBUILD_FUSED, value_placement=skv.SKV_VALUES_HOST), skv.SKV_ERR_UNSUPPORTED),
])
def test_build_validation(kw, expect):
    st, h = _build_status(_cfg(**kw))
    assert st == expect
    assert h is None


def test_build_null_arguments():
    assert _build_status(None)[0] == skv.SKV_ERR_INVALID_ARG
    assert _build_status(_cfg(), kp=None)[0] == skv.SKV_ERR_INVALID_ARG
    assert _build_status(_cfg(), vp=None)[0] == skv.SKV_ERR_INVALID_ARG
    lib = skv.lib()
    assert lib.skv_build(ctypes.byref(_cfg()), 1, 1, None, None) == skv.SKV_ERR_INVALID_ARG


def test_null_handle_calls():
    lib = skv.lib()
    assert lib.skv_decode_step(None, 1, 1, 1, None) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_decode_step_noalloc(None, 1, 1, 1, None) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_append_token(None, 1, 1, None) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_get_stats(None, ctypes.byref(skv.SkvStats())) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_reset_temporal_cache(None) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_export_state(None, ctypes.byref(skv.SkvStateHost())) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_set_timing(None, 4) == skv.SKV_ERR_INVALID_ARG
    lib.skv_destroy(None)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define SKV_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == skv.SKV_NOALLOC_SCRATCH_BYTES


def test_host_pointer_rejected_without_device_memory():
    # valid shape, non-null pointers that are not HIP allocations -> INVALID_ARG
    assert _build_status(_cfg())[0] == skv.SKV_ERR_INVALID_ARG


def test_struct_layouts_match_header():
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "skv.h"
#define P(T, f) printf("%s.%s %zu\n", #T, #f, offsetof(T, f));
int main(void) {
  printf("skv_config %zu\nskv_stats %zu\nskv_state_host %zu\n", sizeof(skv_config),
         sizeof(skv_stats), sizeof(skv_state_host));
  P(skv_config, seq_len) P(skv_config, rope_theta) P(skv_config, temporal_cache)
  P(skv_config, landmark_format) P(skv_config, max_new_tokens) P(skv_config, new_token_mode)
  P(skv_config, a_format) P(skv_config, b_format) P(skv_config, rebuild_mode) P(skv_config, select_mode)
  P(skv_stats, last_alpha) P(skv_stats, last_host_bytes) P(skv_stats, new_tokens)
  P(skv_state_host, eigvals)
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "layout")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = dict(line.rsplit(" ", 1) for line in subprocess.run(
            [exe], capture_output=True, text=True, check=True).stdout.splitlines())
    assert int(out["skv_config"]) == ctypes.sizeof(skv.SkvConfig)
    assert int(out["skv_stats"]) == ctypes.sizeof(skv.SkvStats)
    assert int(out["skv_state_host"]) == ctypes.sizeof(skv.SkvStateHost)
    for key, (cls, field) in {"skv_config.seq_len": (skv.SkvConfig, "seq_len"),
                              "skv_config.rope_theta": (skv.SkvConfig, "rope_theta"),
                              "skv_config.temporal_cache": (skv.SkvConfig, "temporal_cache"),
                              "skv_config.landmark_format": (skv.SkvConfig, "landmark_format"),
                              "skv_config.max_new_tokens": (skv.SkvConfig, "max_new_tokens"),
                              "skv_config.new_token_mode": (skv.SkvConfig, "new_token_mode"),
                              "skv_config.a_format": (skv.SkvConfig, "a_format"),
                              "skv_config.b_format": (skv.SkvConfig, "b_format"),
                              "skv_config.rebuild_mode": (skv.SkvConfig, "rebuild_mode"),
                              "skv_config.select_mode": (skv.SkvConfig, "select_mode"),
                              "skv_stats.new_tokens": (skv.SkvStats, "new_tokens"),
                              "skv_stats.last_alpha": (skv.SkvStats, "last_alpha"),
                              "skv_stats.last_host_bytes": (skv.SkvStats, "last_host_bytes"),
                              "skv_state_host.eigvals": (skv.SkvStateHost, "eigvals")}.items():
        assert int(out[key]) == getattr(cls, field).offset, key
