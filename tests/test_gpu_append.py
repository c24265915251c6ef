"""Generated tokens (skv_append_token) against the oracle, appended between
decode steps.  Exact mode: every appended token is attended after the local
window.  Low-rank mode (ShadowKV+): a token stays exact while it is in the
window region; each completed chunk pushes the oldest exact chunk into the
candidates, which are then scored, selected and rebuilt from A (first the
context's window chunks, then chunks of generated tokens).

Both sides start from the same bf16 context and receive the same bf16 new
tokens; the schedules leave the last unit of appended tokens partly filled and
make the attention split grow between steps.  Once tokens have been appended,
every other q-head aims at one of them (the rest at the context), so that the
generated tokens carry most of those heads' attention weight and folded chunks
of generated tokens are selected."""
import numpy as np
import pytest
import torch

from oracle import shadowkv as O
from sparse_kv_cache_decode_amd import skv, synth
from tests.parity import adopt_gpu_state, bits, check_build, check_ids, check_out, reference_out

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(name="small", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8168,
                rank=64, chunk=8, top_k=13, n_outlier=5, window=32, latent_rank=64)
    base.update(kw)
    return synth.Shape(**base)


def _mixed_queries(shape, k, kn, schedule, seed):
    q = synth.queries_np(shape, k, 0, len(schedule), seed)
    avail = np.cumsum(schedule)
    if avail.max() > 0:
        qn = synth.queries_new_np(shape, kn, [max(int(n), 1) for n in avail], 0, seed)
        for t, n in enumerate(avail):
            if n > 0:
                q[t, :, 1::2] = qn[t, :, 1::2]
    return q


def _run_append(shape, mode, schedule, max_new, seed=0, placement=skv.SKV_VALUES_DEVICE):
    lowrank = mode == skv.SKV_NEW_LOWRANK
    print(f"[append] {shape.name} b={shape.batch} G={shape.group} C={shape.chunk} r={shape.rank} "
          f"W={shape.window} mode={'lowrank' if lowrank else 'exact'} schedule={schedule} "
          f"max_new={max_new} placement={placement}", flush=True)
    n_tok = sum(schedule)
    k, v = synth.layer_cache_np(shape, 0, seed)
    kn, vn = synth.continuation_np(shape, 0, n_tok, seed)
    q = _mixed_queries(shape, k, kn, schedule, seed)
    st = O.build(O.config_from(shape), bits(k), bits(v))
    if placement == skv.SKV_VALUES_HOST:
        vd = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
        vd.copy_(v)
    else:
        vd = v.cuda()
    layer = skv.Layer(shape, k.cuda(), vd, placement, max_new_tokens=max_new, new_token_mode=mode)
    ex = layer.export()
    check_build(ex, st)
    adopt_gpu_state(st, ex)
    knd, vnd = kn.cuda(), vn.cuda()
    prev, prev_differ = None, False
    used = 0
    worst = (0.0, 0.0)
    for step, n in enumerate(schedule):
        for t in range(used, used + n):
            layer.append(knd[t], vnd[t])
            O.append(st, bits(kn[t]), bits(vn[t]), lowrank=lowrank)
        used += n
        out, ids = layer.decode(q[step].cuda())
        torch.cuda.synchronize()
        assert layer.stats()["new_tokens"] == used
        res = O.decode_step(st, bits(q[step]), prev)
        gids = ids.cpu().numpy()
        differ = check_ids(gids, st, res)
        e = check_out(out.cpu().numpy(), reference_out(st, bits(q[step]), res, gids, differ))
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        if not differ and not prev_differ and prev is not None:
            assert int(layer.stats()["last_hits"]) == int(res.hits.sum())
        prev, prev_differ = res.ids, bool(differ)
        folded_new = int(np.sum(gids >= shape.n_chunks))
    if lowrank:
        assert st.cand.shape[2] == shape.n_cand + used // shape.chunk
    print(f"[append] ok: {used} tokens, max|err| {worst[0]:.2e} relL2 {worst[1]:.2e}, "
          f"selected chunks of generated tokens at the last step: {folded_new}", flush=True)
    return layer, knd, vnd


@pytest.mark.parametrize("mode", [skv.SKV_NEW_EXACT, skv.SKV_NEW_LOWRANK])
def test_append_between_steps(mode):
    # 0, 3, 10, 19 tokens: the first step has none, later ones end in a partial
    # unit (C = 8), and 19 tokens add a third unit to the split count
    layer, kn, vn = _run_append(_small(), mode, [0, 3, 7, 9], max_new=21)
    layer.close()


def test_append_capacity_is_enforced():
    shape = _small(batch=1)
    layer, kn, vn = _run_append(shape, skv.SKV_NEW_EXACT, [2, 1], max_new=3)
    with pytest.raises(skv.SkvError) as e:
        layer.append(kn[0], vn[0])
    assert e.value.status == skv.SKV_ERR_SHAPE
    assert layer.stats()["new_tokens"] == 3
    layer.close()


@pytest.mark.parametrize("mode", [skv.SKV_NEW_EXACT, skv.SKV_NEW_LOWRANK])
def test_append_group_of_eight_chunk_sixteen(mode):
    shape = _small(batch=1, n_q_heads=16, seq_len=8192, chunk=16, top_k=7, n_outlier=2,
                   rank=96, latent_rank=96)
    layer, _, _ = _run_append(shape, mode, [5, 12, 20], max_new=40)
    layer.close()


def test_append_lowrank_full_rank_one_kv_head():
    # rank = H_kv * d: Psi is square (the low-rank state still goes through bf16)
    shape = _small(batch=1, n_q_heads=4, n_kv_heads=1, seq_len=2048, rank=128, latent_rank=64,
                   top_k=9, n_outlier=2)
    layer, _, _ = _run_append(shape, skv.SKV_NEW_LOWRANK, [17, 1], max_new=18, seed=3)
    layer.close()


def test_misaligned_or_host_pointers_rejected_before_any_launch():
    shape = _small(batch=1, seq_len=2048, top_k=9, n_outlier=2)
    k, v = synth.layer_cache_np(shape, 0, 1)
    kn, vn = synth.continuation_np(shape, 0, 1, 1)
    layer = skv.Layer(shape, k.cuda(), v.cuda(), max_new_tokens=2)
    lib = skv.lib()
    q = torch.zeros((1, shape.n_q_heads * shape.head_dim + 8), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, shape.n_q_heads, shape.head_dim), device="cuda")
    ids = torch.empty((1, shape.n_kv_heads, shape.top_k), dtype=torch.int32, device="cuda")
    knd = torch.zeros(kn.numel() + 8, dtype=torch.bfloat16, device="cuda")
    vnd = vn.cuda()
    assert lib.skv_decode_step(layer.h, q.data_ptr() + 2, out.data_ptr(), ids.data_ptr(), None) == \
        skv.SKV_ERR_INVALID_ARG
    assert lib.skv_decode_step(layer.h, q.data_ptr(), out.data_ptr() + 4, ids.data_ptr(), None) == \
        skv.SKV_ERR_INVALID_ARG
    assert lib.skv_append_token(layer.h, knd.data_ptr() + 2, vnd.data_ptr(), None) == skv.SKV_ERR_INVALID_ARG
    # aligned host (pageable) memory is refused too, before any launch
    qh = torch.zeros((1, shape.n_q_heads, shape.head_dim), dtype=torch.bfloat16)
    outh = torch.empty((1, shape.n_q_heads, shape.head_dim))
    idsh = torch.empty((1, shape.n_kv_heads, shape.top_k), dtype=torch.int32)
    assert qh.data_ptr() % 16 == 0 and outh.data_ptr() % 16 == 0
    assert lib.skv_decode_step(layer.h, qh.data_ptr(), out.data_ptr(), ids.data_ptr(), None) == \
        skv.SKV_ERR_INVALID_ARG
    assert lib.skv_decode_step(layer.h, q.data_ptr(), outh.data_ptr(), ids.data_ptr(), None) == \
        skv.SKV_ERR_INVALID_ARG
    assert lib.skv_decode_step(layer.h, q.data_ptr(), out.data_ptr(), idsh.data_ptr(), None) == \
        skv.SKV_ERR_INVALID_ARG
    assert lib.skv_append_token(layer.h, kn.data_ptr(), vnd.data_ptr(), None) == skv.SKV_ERR_INVALID_ARG
    assert lib.skv_append_token(layer.h, knd.data_ptr(), vn.data_ptr(), None) == skv.SKV_ERR_INVALID_ARG
    assert layer.stats()["new_tokens"] == 0 and layer.stats()["steps"] == 0
    layer.close()


def test_lowrank_folds_generated_chunks():
    # W = 16, C = 8: after 44 tokens five chunks have left the exact region, the
    # two window chunks of the context and three chunks of generated tokens,
    # whose keys are then rebuilt from their rows of A and whose values come from
    # the appended values
    shape = _small(window=16)
    layer, _, _ = _run_append(shape, skv.SKV_NEW_LOWRANK, [0, 9, 20, 15], max_new=48)
    layer.close()


def test_lowrank_no_window_host_values():
    # W = 0: the exact region is the chunk being filled; values of the context in
    # pinned host memory (gathered on the side stream), generated chunks' values
    # from the device
    shape = _small(window=0, batch=1, n_q_heads=8)
    layer, _, _ = _run_append(shape, skv.SKV_NEW_LOWRANK, [4, 8, 13, 1], max_new=26,
                              placement=skv.SKV_VALUES_HOST)
    layer.close()
