"""A decode step captured in a HIP graph and replayed gives, replay after
replay, exactly what eager calls give on a twin layer built from the same
inputs (same kernels, same work: bitwise equal), with eager work and
synchronisations between the replays; with values in HBM and in pinned host
memory (the gather's side stream forked from and joined back into the
capturing stream), and with FP8 landmarks, A and B."""
import pytest
import torch

from sparse_kv_cache_decode_amd import skv, synth
from tests.parity import adopt_gpu_state, bits, check_ids, check_out, reference_out
from oracle import shadowkv as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("placement,fmt,rebuild", [
    (skv.SKV_VALUES_DEVICE, "bf16", skv.SKV_REBUILD_AUTO), (skv.SKV_VALUES_HOST, "bf16", skv.SKV_REBUILD_AUTO),
    (skv.SKV_VALUES_DEVICE, "e5m2", skv.SKV_REBUILD_AUTO), (skv.SKV_VALUES_DEVICE, "bf16", skv.SKV_REBUILD_SEPARATE),
    (skv.SKV_VALUES_DEVICE, "bf16", skv.SKV_REBUILD_OVERLAP)])
def test_graph_replays_match_eager(placement, fmt, rebuild):
    shape = synth.Shape("graph", batch=8, n_q_heads=16, n_kv_heads=4, head_dim=128, seq_len=4096,
                        rank=64, chunk=8, top_k=8, n_outlier=2, window=32, latent_rank=64,
                        landmark_format=fmt, a_format=fmt, b_format=fmt)
    print(f"[graph] pairs={shape.pairs} placement={placement} storage={fmt} rebuild={rebuild}", flush=True)
    steps = 6
    k, v = synth.layer_cache_np(shape, 0, 0)
    q = synth.queries_np(shape, k, 0, steps, 0)
    if placement == skv.SKV_VALUES_HOST:
        vd = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
        vd.copy_(v)
    else:
        vd = v.cuda()
    eager = skv.Layer(shape, k.cuda(), vd, placement, rebuild_mode=rebuild)
    graphed = skv.Layer(shape, k.cuda(), vd, placement, rebuild_mode=rebuild)
    qbuf = q[0].cuda()
    out_g = torch.empty((shape.batch, shape.n_q_heads, shape.head_dim), device="cuda")
    ids_g = torch.empty((shape.batch, shape.n_kv_heads, shape.top_k), dtype=torch.int32, device="cuda")
    # step 0 eagerly on both (first calls set kernel attributes outside the capture)
    o_e, i_e = eager.decode(qbuf)
    graphed.decode(qbuf, out_g, ids_g)
    torch.cuda.synchronize()
    assert torch.equal(o_e, out_g) and torch.equal(i_e, ids_g)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.decode(qbuf, out_g, ids_g)
    st = O.build(O.config_from(shape), bits(k), bits(v))
    adopt_gpu_state(st, eager.export())
    prev = O.decode_step(st, bits(q[0])).ids
    for t in range(1, steps):
        qbuf.copy_(q[t].cuda())
        g.replay()
        o_e, i_e = eager.decode(q[t].cuda())
        torch.cuda.synchronize()
        assert torch.equal(i_e, ids_g), f"step {t}: ids differ"
        assert torch.equal(o_e, out_g), f"step {t}: outputs differ"
        assert graphed.stats()["last_hits"] == eager.stats()["last_hits"]
        res = O.decode_step(st, bits(q[t]), prev)
        gids = ids_g.cpu().numpy()
        differ = check_ids(gids, st, res)
        check_out(out_g.cpu().numpy(), reference_out(st, bits(q[t]), res, gids, differ))
        prev = res.ids
    print(f"[graph] ok: {steps - 1} replays, alpha {eager.stats()['mean_alpha']:.3f}", flush=True)
    del g
    eager.close()
    graphed.close()
