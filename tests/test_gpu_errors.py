"""Error paths of the C ABI on the GPU, forced from the host: the library's
failure injection switch makes a chosen device allocation or HIP call report
failure (only the return code: nothing faults), and the slot poisoning switch
fills the slot caches with NaN at build.

* SKV_INJECT_FAIL="alloc:N": skv_build returns SKV_ERR_OOM, sets the handle to
  NULL and leaves the device's free memory where it was; past the last
  allocation the build succeeds.
* SKV_INJECT_FAIL="hip:N": the decode step or append that reaches the N-th HIP
  call returns SKV_ERR_HIP and every later call on the handle SKV_ERR_STATE;
  the steps before it are unaffected (bitwise equal to a run without the
  switch), the device stays usable and skv_destroy frees everything.
* SKV_POISON_SLOTS=1: decode outputs are bitwise those of a run without it, so
  no step reads a slot before a step has written it."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_kv_cache_decode_amd import skv, synth

pytestmark = pytest.mark.gpu


def _free():
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def _inputs(shape, placement, steps=4, seed=0):
    k, v = synth.layer_cache_np(shape, 0, seed)
    q = synth.queries_np(shape, k, 0, steps, seed)
    kd = k.cuda()
    if placement == skv.SKV_VALUES_HOST:
        vd = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
        vd.copy_(v)
    else:
        vd = v.cuda()
    return kd, vd, [q[t].cuda() for t in range(steps)]


def _shape():
    return synth.Shape(name="errors", batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=32768, rank=64,
                       chunk=8, top_k=40, n_outlier=8, window=32, latent_rank=64)


def _bufs(shape):
    """Decode outputs allocated once, so that torch's allocator does not move the
    device's free memory between the measurements."""
    return (torch.empty((shape.batch, shape.n_q_heads, shape.head_dim), dtype=torch.float32, device="cuda"),
            torch.empty((shape.batch, shape.n_kv_heads, shape.top_k), dtype=torch.int32, device="cuda"))


def _decode_all(layer, qs, bufs=None):
    outs = []
    for q in qs:
        out, ids = layer.decode(q, *(bufs or ()))
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), ids.cpu().numpy()))
    return outs


def test_allocation_failure_returns_oom_without_leak(monkeypatch):
    shape = _shape()
    kd, vd, qs = _inputs(shape, skv.SKV_VALUES_DEVICE, steps=2)
    skv.Layer(shape, kd, vd).close()          # first build: streams and module state
    base = _free()
    n_ok = None
    for n in range(1, 9):
        monkeypatch.setenv("SKV_INJECT_FAIL", f"alloc:{n}")
        print(f"[errors] alloc:{n}", flush=True)
        cfg = skv.make_config(shape)
        h = ctypes.c_void_p(12345)
        st = skv.lib().skv_build(ctypes.byref(cfg), skv._ptr(kd), skv._ptr(vd), None, ctypes.byref(h))
        if st == skv.SKV_OK:
            n_ok = n
            assert h.value
            skv.skv_destroy(h.value)
            break
        assert st == skv.SKV_ERR_OOM
        assert h.value is None
        assert _free() == base, n
    monkeypatch.delenv("SKV_INJECT_FAIL")
    assert n_ok is not None and n_ok > 1
    assert _free() == base
    # the device still works
    layer = skv.Layer(shape, kd, vd)
    _decode_all(layer, qs)
    layer.close()


@pytest.mark.parametrize("placement,rebuild", [(skv.SKV_VALUES_DEVICE, skv.SKV_REBUILD_FUSED),
                                               (skv.SKV_VALUES_DEVICE, skv.SKV_REBUILD_OVERLAP),
                                               (skv.SKV_VALUES_HOST, skv.SKV_REBUILD_SEPARATE)])
def test_hip_failure_poisons_handle(monkeypatch, placement, rebuild):
    shape = _shape()
    steps = 4
    kd, vd, qs = _inputs(shape, placement, steps)
    bufs = _bufs(shape)
    ref_layer = skv.Layer(shape, kd, vd, placement, rebuild_mode=rebuild)
    ref = _decode_all(ref_layer, qs, bufs)
    ref_layer.close()
    base = _free()
    for n in (1, 2, 3, 5, 8, 13):
        print(f"[errors] {placement=} {rebuild=} hip:{n}", flush=True)
        monkeypatch.setenv("SKV_INJECT_FAIL", f"hip:{n}")
        layer = skv.Layer(shape, kd, vd, placement, rebuild_mode=rebuild)
        monkeypatch.delenv("SKV_INJECT_FAIL")
        failed_at = None
        for t in range(steps):
            try:
                out, ids = layer.decode(qs[t], *bufs)
            except skv.SkvError as e:
                assert e.status == skv.SKV_ERR_HIP
                failed_at = t
                break
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref[t][0]) and np.array_equal(ids.cpu().numpy(), ref[t][1])
        assert failed_at is not None, n
        torch.cuda.synchronize()                  # the work enqueued before the failure completes
        for call in (lambda: layer.decode(qs[0], *bufs), layer.stats, layer.reset, lambda: layer.append(qs[0], qs[0])):
            with pytest.raises(skv.SkvError) as e:
                call()
            assert e.value.status == skv.SKV_ERR_STATE
        layer.close()
        assert _free() == base, n


def test_append_failure_poisons_handle(monkeypatch):
    shape = _shape()
    kd, vd, qs = _inputs(shape, skv.SKV_VALUES_DEVICE, 1)
    kn = torch.zeros((shape.batch, shape.n_kv_heads * shape.head_dim), dtype=torch.bfloat16, device="cuda")
    monkeypatch.setenv("SKV_INJECT_FAIL", "hip:1")
    layer = skv.Layer(shape, kd, vd, max_new_tokens=4, new_token_mode=skv.SKV_NEW_LOWRANK)
    monkeypatch.delenv("SKV_INJECT_FAIL")
    with pytest.raises(skv.SkvError) as e:
        layer.append(kn, kn)
    assert e.value.status == skv.SKV_ERR_HIP
    with pytest.raises(skv.SkvError) as e:
        layer.decode(qs[0])
    assert e.value.status == skv.SKV_ERR_STATE
    layer.close()


@pytest.mark.parametrize("placement,rebuild,temporal", [
    (skv.SKV_VALUES_DEVICE, skv.SKV_REBUILD_FUSED, 1), (skv.SKV_VALUES_DEVICE, skv.SKV_REBUILD_SEPARATE, 1),
    (skv.SKV_VALUES_DEVICE, skv.SKV_REBUILD_OVERLAP, 1), (skv.SKV_VALUES_DEVICE, skv.SKV_REBUILD_FUSED, 0),
    (skv.SKV_VALUES_HOST, skv.SKV_REBUILD_SEPARATE, 1)])
def test_poisoned_slots_never_read_before_written(monkeypatch, placement, rebuild, temporal):
    shape = _shape()
    steps = 6
    kd, vd, qs = _inputs(shape, placement, steps)
    print(f"[errors] poison {placement=} {rebuild=} {temporal=}", flush=True)
    clean = skv.Layer(shape, kd, vd, placement, temporal, rebuild_mode=rebuild)
    ref = _decode_all(clean, qs)
    clean.close()
    monkeypatch.setenv("SKV_POISON_SLOTS", "1")
    layer = skv.Layer(shape, kd, vd, placement, temporal, rebuild_mode=rebuild)
    monkeypatch.delenv("SKV_POISON_SLOTS")
    got = _decode_all(layer, qs)
    layer.reset()
    got_after_reset = _decode_all(layer, qs[:2])
    layer.close()
    for t in range(steps):
        assert np.isfinite(got[t][0]).all(), t
        assert np.array_equal(got[t][0], ref[t][0]) and np.array_equal(got[t][1], ref[t][1]), t
    for t in range(2):
        assert np.array_equal(got_after_reset[t][0], ref[t][0]), t


def test_poisoned_slots_with_appended_tokens(monkeypatch):
    """Low-rank new-token mode: folded chunks of generated tokens are selected
    and rebuilt into the same slots."""
    shape = _shape()
    steps = 6
    kd, vd, qs = _inputs(shape, skv.SKV_VALUES_DEVICE, steps)
    g = torch.Generator().manual_seed(3)
    kn = [torch.randn((shape.batch, shape.n_kv_heads * shape.head_dim), generator=g).to(torch.bfloat16).cuda()
          for _ in range(steps * 4)]
    vn = [torch.randn((shape.batch, shape.n_kv_heads, shape.head_dim), generator=g).to(torch.bfloat16).cuda()
          for _ in range(steps * 4)]

    def run():
        layer = skv.Layer(shape, kd, vd, max_new_tokens=steps * 4, new_token_mode=skv.SKV_NEW_LOWRANK)
        res = []
        for t in range(steps):
            for i in range(4):
                layer.append(kn[t * 4 + i], vn[t * 4 + i])
            out, ids = layer.decode(qs[t])
            torch.cuda.synchronize()
            res.append((out.cpu().numpy(), ids.cpu().numpy()))
        layer.close()
        return res

    ref = run()
    monkeypatch.setenv("SKV_POISON_SLOTS", "1")
    got = run()
    monkeypatch.delenv("SKV_POISON_SLOTS")
    for t in range(steps):
        assert np.isfinite(got[t][0]).all(), t
        assert np.array_equal(got[t][0], ref[t][0]) and np.array_equal(got[t][1], ref[t][1]), t
