"""GPU library vs CPU oracle on the same seeded inputs (end to end: both sides
build from the same bf16 keys and values, then decode the same queries)."""
import numpy as np
import pytest
import torch

from oracle import shadowkv as O
from sparse_kv_cache_decode_amd import skv, synth
from tests.parity import (DECODE_MAX_ABS, DECODE_REL_L2, adopt_gpu_state, bits, check_build, check_ids,
                          check_out, reference_out)

pytestmark = pytest.mark.gpu


def _run(shape, steps, placement=skv.SKV_VALUES_DEVICE, temporal=1, seed=0, mode="drift",
         check_state=True, keep=False, rebuild=skv.SKV_REBUILD_AUTO, select=skv.SKV_SELECT_AUTO, q=None):
    print(f"[parity] {shape.name} b={shape.batch} S={shape.seq_len} G={shape.group} "
          f"C={shape.chunk} K={shape.top_k} O={shape.n_outlier} r={shape.rank} "
          f"landmarks={shape.landmark_format} placement={placement} temporal={temporal} "
          f"rebuild={rebuild} select={select} steps={steps}", flush=True)
    k, v = synth.layer_cache_np(shape, 0, seed)
    if q is None:
        q = synth.queries_np(shape, k, 0, steps, seed, mode=mode)
    st = O.build(O.config_from(shape), bits(k), bits(v))
    kd = k.cuda()
    if placement == skv.SKV_VALUES_HOST:
        vd = torch.empty(v.shape, dtype=v.dtype, pin_memory=True)
        vd.copy_(v)
    else:
        vd = v.cuda()
    layer = skv.Layer(shape, kd, vd, placement, temporal, rebuild_mode=rebuild, select_mode=select)
    del kd
    ex = layer.export()
    if check_state:
        check_build(ex, st)
    adopt_gpu_state(st, ex)
    prev, prev_gpu, prev_differ = None, None, True
    worst = (0.0, 0.0)
    swaps = 0
    for t in range(steps):
        out, ids = layer.decode(q[t].cuda())
        torch.cuda.synchronize()
        res = O.decode_step(st, bits(q[t]), prev if temporal else None)
        gids = ids.cpu().numpy()
        differ = check_ids(gids, st, res)
        swaps += len(differ)
        e = check_out(out.cpu().numpy(), reference_out(st, bits(q[t]), res, gids, differ), DECODE_MAX_ABS,
                      DECODE_REL_L2)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        s = layer.stats()
        if t == 0 or not temporal:
            assert s["last_hits"] == 0 and s["last_misses"] == shape.pairs * shape.top_k
        else:
            own = sum(len(set(gids[b, h]) & set(prev_gpu[b, h]))
                      for b in range(shape.batch) for h in range(shape.n_kv_heads))
            assert s["last_hits"] == own and s["last_misses"] == shape.pairs * shape.top_k - own
            if not differ and not prev_differ:
                assert s["last_hits"] == int(res.hits.sum()), (s, res.hits.sum())
        prev, prev_gpu, prev_differ = res.ids, gids, bool(differ)
    print(f"[parity] ok: max|err| {worst[0]:.2e} relL2 {worst[1]:.2e} alpha {layer.stats()['mean_alpha']:.3f}"
          f" near-tie swaps {swaps}", flush=True)
    if not keep:
        layer.close()
    return layer


def test_tiny_8k_end_to_end():
    _run(synth.SHAPES["tiny_8k"], steps=4)


# The rebuild as its own launch before the attention (SKV_REBUILD_SEPARATE), and
# beside the attention over the hits with the misses attended by a second launch
# (SKV_REBUILD_OVERLAP), on the shapes the fused default covers above: tiles,
# chunk sizes, group sizes, a budget of one, the temporal cache off, the split
# selection
@pytest.mark.parametrize("case", ["tiny", "ragged", "chunk4", "chunk16", "g16", "k1", "temporal_off", "split"])
@pytest.mark.parametrize("sep", [skv.SKV_REBUILD_SEPARATE, skv.SKV_REBUILD_OVERLAP])
def test_other_rebuild_modes(case, sep):
    if case == "tiny":
        _run(synth.SHAPES["tiny_8k"], steps=4, rebuild=sep)
    elif case == "ragged":
        _run(_small(), steps=3, rebuild=sep)
    elif case in ("chunk4", "chunk16"):
        c = 4 if case == "chunk4" else 16
        _run(_small(chunk=c, seq_len=8192, top_k=8192 // (64 * c), n_outlier=3, batch=1), steps=3, rebuild=sep)
    elif case == "g16":
        _run(_small(n_q_heads=32, n_kv_heads=2, batch=1, seq_len=4096, top_k=9, n_outlier=2, rank=48,
                    latent_rank=48), steps=2, rebuild=sep)
    elif case == "k1":
        _run(_small(top_k=1, batch=1), steps=3, rebuild=sep)
    elif case == "temporal_off":
        _run(_small(), steps=3, temporal=0, rebuild=sep)
    else:
        _run(_small(batch=1, n_q_heads=16, n_kv_heads=2, seq_len=69632, rank=32, latent_rank=32, top_k=136,
                    n_outlier=26), steps=2, rebuild=sep)


def test_fused_rebuild_explicit_and_many_tiles():
    # K = 400 at C = 4: 13 tiles of 32 missed chunks per pair on the first step
    _run(_small(chunk=4, seq_len=102400, top_k=400, n_outlier=30, batch=1, n_q_heads=8, n_kv_heads=2),
         steps=3, rebuild=skv.SKV_REBUILD_FUSED)


def _small(**kw):
    base = dict(name="small", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, seq_len=8168,
                rank=64, chunk=8, top_k=13, n_outlier=5, window=32, latent_rank=64)
    base.update(kw)
    return synth.Shape(**base)


@pytest.mark.parametrize("chunk", [4, 8, 16])
def test_static_units_over_several_selection_workgroups(chunk):
    """Fused rebuild with the two-level selection: the outlier chunks and the
    window are attended by extra workgroups of the selection launch, each 16
    waves of 32 tokens (16 * 32 / C units).  Here they need four such workgroups
    per pair, the last one partly filled, and the outputs still match the
    oracle."""
    per_wg = 16 * 32 // chunk
    shape = _small(chunk=chunk, seq_len=16384, n_outlier=3 * per_wg + 5, top_k=40, batch=2, n_q_heads=8,
                   n_kv_heads=2)
    static_units = shape.n_outlier + shape.window // chunk
    assert 3 * per_wg < static_units <= 4 * per_wg
    _run(shape, steps=3)


def test_ragged_tiles_two_batches():
    # n_cand = 1021 - 5 - 4 = 1012: not a multiple of the 16/256-landmark tiles
    _run(_small(), steps=3)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (32, 4), (32, 2)])
def test_group_sizes(hq, hkv):
    _run(_small(n_q_heads=hq, n_kv_heads=hkv, batch=1, seq_len=4096, top_k=9, n_outlier=2,
                rank=48, latent_rank=48), steps=2)


@pytest.mark.parametrize("chunk", [4, 16])
def test_chunk_sizes(chunk):
    _run(_small(chunk=chunk, seq_len=8192, top_k=8192 // (64 * chunk), n_outlier=3, batch=1), steps=3)


def test_host_values():
    _run(_small(), steps=3, placement=skv.SKV_VALUES_HOST)


def test_temporal_cache_off():
    _run(_small(), steps=3, temporal=0)


def test_full_budget_no_outliers_no_window():
    # K = n_cand: every chunk is selected; O = 0, W = 0
    s = _small(seq_len=2048, n_outlier=0, window=0, top_k=256, batch=1)
    assert s.n_cand == 256
    _run(s, steps=2)


def test_budget_of_one():
    _run(_small(top_k=1, batch=1), steps=3)


@pytest.mark.parametrize("rebuild", [skv.SKV_REBUILD_SEPARATE, skv.SKV_REBUILD_FUSED])
def test_reset_and_identical_query(rebuild):
    shape = _small(batch=1)
    print(f"[parity] reset/identical query on {shape}, rebuild {rebuild}", flush=True)
    k, v = synth.layer_cache_np(shape, 0, 0)
    q = synth.queries_np(shape, k, 0, 2, 0)
    layer = skv.Layer(shape, k.cuda(), v.cuda(), rebuild_mode=rebuild)
    q0 = q[0].cuda()
    out0, ids0 = [x.clone() for x in layer.decode(q0)]
    out1, ids1 = [x.clone() for x in layer.decode(q0)]
    torch.cuda.synchronize()
    s = layer.stats()
    assert s["last_hits"] == shape.pairs * shape.top_k and s["last_misses"] == 0
    assert torch.equal(ids0, ids1)
    if rebuild == skv.SKV_REBUILD_SEPARATE:
        assert torch.equal(out0, out1)      # the same units in the same splits: bitwise identical
    else:
        # the misses of the first step were attended by the tiles that rebuilt them,
        # the hits of the second by attention splits: the same keys and values,
        # summed in another grouping, with the softmax weights carried at 16 bits
        # relative to another running maximum (2^-16 of each weight)
        err = (out0 - out1).abs().max().item()
        assert err <= 1e-4, err
    layer.decode(q[1].cuda())
    layer.reset()
    out2, ids2 = layer.decode(q0)
    torch.cuda.synchronize()
    s = layer.stats()
    assert s["steps"] == 1 and s["last_hits"] == 0 and s["last_misses"] == shape.pairs * shape.top_k
    assert torch.equal(ids2, ids0) and torch.equal(out2, out0)
    layer.close()


def test_split_selection_many_candidates():
    # n_cand = 34816 - 3 - 4 = 34809 > 32768: the candidates are cut into parts
    # whose top-K are merged (the path of the 1M-token workload)
    s = _small(batch=1, n_q_heads=2, n_kv_heads=1, seq_len=278528, rank=16, latent_rank=16,
               top_k=64, n_outlier=3)
    assert s.n_cand > 32768
    _run(s, steps=2)


def test_split_selection_group_of_eight():
    # G * n_cand = 8 * 8674 > 65536 logits per pair: selection in parts of 592
    s = _small(batch=1, n_q_heads=16, n_kv_heads=2, seq_len=69632, rank=32, latent_rank=32,
               top_k=136, n_outlier=26)
    assert s.group * s.n_cand > 65536
    _run(s, steps=2)



def test_merge_tree_one_level():
    # K = 2048 of 49145 candidates, 16 q heads on one KV head (the 1M-token shape's
    # G and K): 12 parts; 8 part lists fit one merge workgroup, so one tree level
    # merges them into 2 lists before the final selection
    s = _small(batch=1, n_q_heads=16, n_kv_heads=1, seq_len=393216, rank=16, latent_rank=16,
               top_k=2048, n_outlier=3)
    assert s.n_cand == 49145
    _run(s, steps=2)


def test_merge_tree_two_levels():
    # K = 4096 (the largest budget) at C = 4: 18 parts, 4 lists per merge
    # workgroup: two tree levels (18 -> 5 -> 2 lists), then the final selection
    s = _small(batch=1, n_q_heads=4, n_kv_heads=1, seq_len=557104, chunk=4, rank=16, latent_rank=16,
               top_k=4096, n_outlier=3)
    assert s.n_cand == 139265
    _run(s, steps=2)


def test_eight_kv_heads_small_budget():
    # 8178 candidates, K = 60, 32 q / 8 KV heads: with the oracle's own landmarks
    # one pair's 60th and 61st chunks swap (their scores 1.3e-3 apart), because a
    # landmark value sits a bf16 rounding boundary away; on the GPU's landmarks
    # the selections agree
    _run(_small(batch=2, n_q_heads=32, n_kv_heads=8, seq_len=65536, top_k=60, n_outlier=10), steps=3)


def test_rank_deficient_prefill():
    # S = 64 tokens of 2 KV heads (n = 256) at r = 64: the Gram matrix has rank 64,
    # below the eigensolver's block of p = 80 columns, so Cholesky QR breaks down
    # after the first product and the blocks go through Gram-Schmidt on the host
    s = _small(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=64, rank=64, latent_rank=64, top_k=2,
               n_outlier=1, window=0)
    _run(s, steps=3)


# The selection as one full pass over every candidate's score (SKV_SELECT_FULL):
# one workgroup per pair, and the parts / merge-tree path beyond 32K candidates
@pytest.mark.parametrize("case", ["tiny", "ragged", "many_candidates", "group_of_eight", "tree_one", "tree_two"])
def test_full_pass_selection(case):
    full = skv.SKV_SELECT_FULL
    if case == "tiny":
        _run(synth.SHAPES["tiny_8k"], steps=3, select=full)
    elif case == "ragged":
        _run(_small(), steps=3, select=full)
    elif case == "many_candidates":
        _run(_small(batch=1, n_q_heads=2, n_kv_heads=1, seq_len=278528, rank=16, latent_rank=16, top_k=64,
                    n_outlier=3), steps=2, select=full)
    elif case == "group_of_eight":
        _run(_small(batch=1, n_q_heads=16, n_kv_heads=2, seq_len=69632, rank=32, latent_rank=32, top_k=136,
                    n_outlier=26), steps=2, select=full)
    elif case == "tree_one":
        _run(_small(batch=1, n_q_heads=16, n_kv_heads=1, seq_len=393216, rank=16, latent_rank=16, top_k=2048,
                    n_outlier=3), steps=2, select=full)
    else:
        _run(_small(batch=1, n_q_heads=4, n_kv_heads=1, seq_len=557104, chunk=4, rank=16, latent_rank=16,
                    top_k=4096, n_outlier=3), steps=2, select=full)


@pytest.mark.parametrize("select", [skv.SKV_SELECT_AUTO, skv.SKV_SELECT_FULL])
def test_equal_scores_take_lowest_chunks(select):
    # zero queries: every logit is 0 and every chunk scores the same, so the K
    # lowest chunk ids are selected; in the two-level selection every one of the
    # 512 tiles is "hot", more than the 256 its registers hold at K = 60, so the
    # second level runs from memory
    s = _small(batch=2, n_q_heads=32, n_kv_heads=8, seq_len=65536, top_k=60, n_outlier=10)
    assert (s.n_cand + 15) // 16 > 256
    q = torch.zeros((2, s.batch, s.n_q_heads, s.head_dim), dtype=torch.bfloat16)
    _run(s, steps=2, select=select, q=q)



@pytest.mark.parametrize("top_k", [512, 513])
def test_two_level_budget_limit(top_k):
    """The two-level selection serves budgets up to 512 chunks, a full pass the
    ones above: on either side of the limit both selection modes pick the same
    chunks bit for bit, and the oracle agrees."""
    shape = _small(batch=1, n_q_heads=8, n_kv_heads=2, seq_len=65536, rank=32, latent_rank=32, top_k=top_k,
                   n_outlier=20)
    k, v = synth.layer_cache_np(shape, 0, 0)
    q = synth.queries_np(shape, k, 0, 3, 0)
    ids = {}
    for sel in (skv.SKV_SELECT_AUTO, skv.SKV_SELECT_FULL):
        layer = skv.Layer(shape, k.cuda(), v.cuda(), select_mode=sel)
        got = []
        for t in range(3):
            _, i = layer.decode(q[t].cuda())
            torch.cuda.synchronize()
            got.append(i.cpu().numpy())
        layer.close()
        ids[sel] = got
    for t in range(3):
        assert np.array_equal(ids[skv.SKV_SELECT_AUTO][t], ids[skv.SKV_SELECT_FULL][t]), t
    _run(shape, steps=3)
