"""skv_decode_step_noalloc (the decode step whose transient scratch is the
library's static device array) against skv_decode_step on the same inputs,
through the C ABI: two handles built from the same bits decode the same
drifting queries, one through each entry point, and must agree bit for bit
(same kernels, only the scratch address differs).  A larger layer runs first,
then a smaller one, so the second call finds the array holding the first call's
contents.  A layer whose transient scratch exceeds the array is refused before
anything is enqueued."""
import pytest
import torch

from sparse_kv_cache_decode_amd import skv, synth

pytestmark = pytest.mark.gpu


def _pair_of_layers(shape):
    k, v = synth.layer_cache_np(shape, 0, 0)
    kd, vd = k.cuda(), v.cuda()
    return skv.Layer(shape, kd, vd), skv.Layer(shape, kd, vd), k


def _compare(shape, steps):
    print(f"[noalloc] {shape.name} b={shape.batch} S={shape.seq_len} G={shape.group} K={shape.top_k}", flush=True)
    ref, nol, k = _pair_of_layers(shape)
    q = synth.queries_np(shape, k, 0, steps, 0)
    for t in range(steps):
        qd = q[t].cuda()
        out_r, ids_r = ref.decode(qd)
        out_n = torch.full_like(out_r, float("nan"))
        ids_n = torch.full_like(ids_r, -1)
        skv.skv_decode_step_noalloc(nol.h, qd, out_n, ids_n)
        torch.cuda.synchronize()
        assert torch.equal(ids_n, ids_r), f"step {t}: selected chunks differ"
        assert torch.equal(out_n, out_r), f"step {t}: outputs differ"
        sr, sn = ref.stats(), nol.stats()
        assert sr["last_hits"] == sn["last_hits"] and sr["last_misses"] == sn["last_misses"]
    ref.close()
    nol.close()


def test_noalloc_matches_decode_step_then_smaller_layer():
    big = synth.SHAPES["tiny_8k"].replace(batch=2)
    small = synth.Shape(name="small", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=4096,
                        rank=64, chunk=8, top_k=8, n_outlier=2, window=32, latent_rank=64)
    _compare(big, steps=3)
    _compare(small, steps=2)


def test_noalloc_refuses_oversized_scratch():
    # 64 pairs x 16 query heads x 17 404 candidates of fp32 logits = 71 MB > 64 MiB
    shape = synth.Shape(name="big", batch=8, n_q_heads=128, n_kv_heads=8, head_dim=128, seq_len=139264,
                        rank=16, chunk=8, top_k=64, n_outlier=0, window=32, latent_rank=16)
    assert shape.pairs * shape.group * shape.n_cand * 4 > skv.SKV_NOALLOC_SCRATCH_BYTES
    print(f"[noalloc] oversized {shape.name}", flush=True)
    k, v = synth.layer_cache_torch(shape, 0, 0, "cuda")
    layer = skv.Layer(shape, k, v)
    del k
    q = torch.zeros((shape.batch, shape.n_q_heads, shape.head_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((shape.batch, shape.n_q_heads, shape.head_dim), dtype=torch.float32, device="cuda")
    ids = torch.full((shape.batch, shape.n_kv_heads, shape.top_k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(skv.SkvError) as e:
        skv.skv_decode_step_noalloc(layer.h, q, out, ids)
    assert e.value.status == skv.SKV_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((ids == -7).all()) and bool((out == 0).all())   # nothing was enqueued
    layer.decode(q)                                              # the handle is unchanged and usable
    torch.cuda.synchronize()
    layer.close()
