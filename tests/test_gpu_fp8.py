"""FP8 (E5M2) landmark storage against the oracle, which rounds its fp64 chunk
means with the same format (the precision-sensitivity study in section 5 of the
paper-graph-ui summary of ShadowKV, Tables 9 and 10, runs the method in
torch.float8_e5m2).  Build: every landmark the
oracle's rounding of the same float64 chunk mean; decode: the usual bars."""
import numpy as np
import pytest
import torch

from sparse_kv_cache_decode_amd import skv, synth
from tests.test_gpu_append import _run_append
from tests.test_gpu_parity import _run, _small

pytestmark = pytest.mark.gpu


def test_fp8_tiny_8k_end_to_end():
    _run(synth.SHAPES["tiny_8k"].replace(landmark_format="e5m2"), steps=4)


def test_fp8_ragged_blocks_two_batches():
    # n_cand = 1012 = 3 * 256 + 244: the last 256-landmark block is ragged
    _run(_small(landmark_format="e5m2"), steps=3)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (32, 4), (32, 2)])
def test_fp8_group_sizes(hq, hkv):
    _run(_small(n_q_heads=hq, n_kv_heads=hkv, batch=1, seq_len=4096, top_k=9, n_outlier=2,
                rank=48, latent_rank=48, landmark_format="e5m2"), steps=2)


def test_fp8_chunk_four_host_values():
    _run(_small(chunk=4, window=32, landmark_format="e5m2"), steps=2, placement=skv.SKV_VALUES_HOST)


def test_fp8_split_selection():
    # 34809 candidates: selection in parts and a merge, scores from 136 FP8 blocks
    s = _small(batch=1, n_q_heads=2, n_kv_heads=1, seq_len=278528, rank=16, latent_rank=16,
               top_k=64, n_outlier=3, landmark_format="e5m2")
    _run(s, steps=2)


def test_fp8_lowrank_folds_generated_chunks():
    # folded chunks get E5M2 landmarks too (the mean of their stored exact keys)
    layer, _, _ = _run_append(_small(window=16, landmark_format="e5m2"), skv.SKV_NEW_LOWRANK,
                              [0, 9, 20, 15], max_new=48)
    layer.close()


def test_fp8_a_tiny_8k_both_formats():
    # landmarks and A both FP8 (the key rebuild widens A's bytes to bf16)
    _run(synth.SHAPES["tiny_8k"].replace(landmark_format="e5m2", a_format="e5m2"), steps=4)


def test_fp8_a_only_ragged_two_batches():
    _run(_small(a_format="e5m2"), steps=3)


@pytest.mark.parametrize("chunk", [4, 16])
def test_fp8_a_chunk_sizes_host_values(chunk):
    _run(_small(chunk=chunk, seq_len=8192, top_k=8192 // (64 * chunk), n_outlier=3,
                landmark_format="e5m2", a_format="e5m2"), steps=2, placement=skv.SKV_VALUES_HOST)


def test_fp8_a_group_of_sixteen_small_rank():
    _run(_small(n_q_heads=32, n_kv_heads=2, batch=1, seq_len=4096, top_k=9, n_outlier=2,
                rank=16, latent_rank=16, landmark_format="e5m2", a_format="e5m2"), steps=2)


def test_fp8_a_lowrank_appended_rows():
    # the rows of A of generated tokens are FP8 too; folded chunks are rebuilt from them
    layer, _, _ = _run_append(_small(window=16, landmark_format="e5m2", a_format="e5m2"),
                              skv.SKV_NEW_LOWRANK, [0, 9, 20, 15], max_new=48)
    layer.close()


def test_fp8_full_budget_no_outliers_no_window():
    # K = n_cand = 256, one FP8 score block exactly; every chunk selected
    s = _small(seq_len=2048, n_outlier=0, window=0, top_k=256, batch=1, landmark_format="e5m2",
               a_format="e5m2")
    assert s.n_cand == 256
    _run(s, steps=2)


def test_fp8_budget_of_one_temporal_cache_off():
    _run(_small(top_k=1, batch=1, landmark_format="e5m2", a_format="e5m2"), steps=3, temporal=0)


def test_fp8_all_stores_tiny_8k():
    # landmarks, A and B in FP8: the key rebuild reads B^T fragments as bytes
    _run(synth.SHAPES["tiny_8k"].replace(landmark_format="e5m2", a_format="e5m2", b_format="e5m2"), steps=4)


@pytest.mark.parametrize("chunk", [4, 16])
def test_fp8_b_only_chunk_sizes_host_values(chunk):
    _run(_small(chunk=chunk, seq_len=8192, top_k=8192 // (64 * chunk), n_outlier=3, b_format="e5m2"),
         steps=2, placement=skv.SKV_VALUES_HOST)


def test_fp8_all_stores_rank_sixteen():
    # r = 16: the last (only) k-step is half empty, the upper k-groups read zeros
    _run(_small(n_q_heads=32, n_kv_heads=2, batch=1, seq_len=4096, top_k=9, n_outlier=2, rank=16,
                latent_rank=16, landmark_format="e5m2", a_format="e5m2", b_format="e5m2"), steps=2)


def test_fp8_b_lowrank_appended_rows():
    # the appended rows of A are projected with the FP8 B
    layer, _, _ = _run_append(_small(window=16, b_format="e5m2"), skv.SKV_NEW_LOWRANK, [0, 9, 20, 15],
                              max_new=48)
    layer.close()


def test_fp8_query_beyond_fp16_range_saturates():
    # FP8 landmarks are scored with q in fp16: query values past 65504 saturate
    # there instead of becoming inf (which would make the logits NaN); the step
    # stays finite and selects valid, ascending candidate chunks
    shape = synth.SHAPES["tiny_8k"].replace(landmark_format="e5m2")
    k, v = synth.layer_cache_np(shape, 0, 0)
    q = synth.queries_np(shape, k, 0, 2, 0).float()
    q[:, :, 0, :4] = 2.0e5
    q[:, :, 1, 5] = -3.0e6
    q = q.to(torch.bfloat16)
    layer = skv.Layer(shape, k.cuda(), v.cuda())
    cand = layer.export()["cand_ids"]
    for t in range(2):
        out, ids = layer.decode(q[t].cuda())
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        g = ids.cpu().numpy()
        assert np.all(np.diff(g, axis=-1) > 0)
        for h in range(shape.n_kv_heads):
            assert np.isin(g[0, h], cand[0, h]).all()
    layer.close()
