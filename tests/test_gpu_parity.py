"""GPU library vs CPU oracle on the same seeded inputs (end to end: both sides
build from the same bf16 keys and values, then decode the same queries)."""
import numpy as np
import pytest
import torch

from oracle import shadowkv as O
from sparse_kv_cache_decode_amd import skv, synth
from tests.parity import bits, check_build, check_ids, check_out

pytestmark = pytest.mark.gpu


def _run(shape, steps, placement=skv.SKV_VALUES_DEVICE, temporal=1, seed=0, mode="drift",
         check_state=True):
    print(f"[parity] {shape.name} b={shape.batch} S={shape.seq_len} G={shape.group} "
          f"C={shape.chunk} K={shape.top_k} O={shape.n_outlier} r={shape.rank} "
          f"placement={placement} temporal={temporal} steps={steps}", flush=True)
    k, v = synth.layer_cache_np(shape, 0, seed)
    q = synth.queries_np(shape, k, 0, steps, seed, mode=mode)
    st = O.build(O.config_from(shape), bits(k), bits(v))
    kd = k.cuda()
    if placement == skv.SKV_VALUES_HOST:
        vd = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
        vd.copy_(v)
    else:
        vd = v.cuda()
    layer = skv.Layer(shape, kd, vd, placement, temporal)
    del kd
    if check_state:
        check_build(layer.export(), st)
    prev = None
    worst = (0.0, 0.0)
    for t in range(steps):
        out, ids = layer.decode(q[t].cuda())
        torch.cuda.synchronize()
        res = O.decode_step(st, bits(q[t]), prev if temporal else None)
        differ = check_ids(ids.cpu().numpy(), st, res)
        e = check_out(out.cpu().numpy(), res.out)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        s = layer.stats()
        if differ == 0:
            if t == 0 or not temporal:
                assert s["last_hits"] == 0 and s["last_misses"] == shape.pairs * shape.top_k
            else:
                assert s["last_hits"] == int(res.hits.sum()), (s, res.hits.sum())
        prev = res.ids
    print(f"[parity] ok: max|err| {worst[0]:.2e} relL2 {worst[1]:.2e} alpha {layer.stats()['mean_alpha']:.3f}",
          flush=True)
    layer.close()
    return layer


def test_tiny_8k_end_to_end():
    _run(synth.SHAPES["tiny_8k"], steps=4)
