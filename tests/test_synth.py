"""The seeded input generator: determinism and the stated statistics."""
import math

import numpy as np
import torch

from sparse_kv_cache_decode_amd import synth


def _small():
    return synth.SHAPES["tiny_8k"].replace(batch=2, seq_len=4096, n_kv_heads=2, n_q_heads=8,
                                           latent_rank=16, rank=16)


def test_deterministic_and_distinct_streams():
    s = _small()
    k1, v1 = synth.layer_cache_np(s, 0, seed=0)
    k2, v2 = synth.layer_cache_np(s, 0, seed=0)
    k3, _ = synth.layer_cache_np(s, 1, seed=0)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert not torch.equal(k1, k3)
    assert k1.dtype == torch.bfloat16 and k1.shape == (2, 4096, 256)
    assert v1.shape == (2, 2, 4096, 128)


def test_ar1_statistics():
    rng = np.random.default_rng(0)
    a = synth._ar1_np(rng.standard_normal((200000, 4)), 0.95)
    assert abs(a.var() - 1.0) < 0.05
    lag1 = np.mean(a[1:] * a[:-1]) / a.var()
    assert abs(lag1 - 0.95) < 0.01
    # the doubling scan used on the GPU computes the same recurrence
    e = torch.from_numpy(rng.standard_normal((3000, 3)))
    ref = synth._ar1_np(e.numpy(), 0.9)
    np.testing.assert_allclose(synth._ar1_torch(e.clone(), 0.9).numpy(), ref, atol=1e-10)


def test_queries_are_peaked_and_drift():
    s = _small()
    k, _ = synth.layer_cache_np(s, 0)
    q = synth.queries_np(s, k, 0, steps=3)
    assert q.shape == (3, 2, 8, 128)
    qf = q.float()
    c = torch.nn.functional.cosine_similarity(qf[0], qf[1], dim=-1)
    assert c.mean() > 0.7       # AR(1) drift with rho = 0.9
    qi = synth.queries_np(s, k, 0, steps=2, mode="independent").float()
    assert torch.nn.functional.cosine_similarity(qi[0], qi[1], dim=-1).abs().mean() < 0.5
    # needle term dominates: |q| ~ 4 |k|
    assert qf[0].norm(dim=-1).mean() > 3 * k.float().view(2, 4096, 2, 128).norm(dim=-1).mean()


def test_budget_rule():
    assert synth.budget(122880, 8) == (240, 46)
    assert synth.budget(204800, 8) == (400, 77)
    assert synth.budget(1048576, 8) == (2048, 393)
    assert synth.budget(1048576, 4) == (4096, 786)
    assert synth.budget(1048576, 16) == (1024, 197)
    assert synth.budget(8192, 8) == (16, 3)


def test_continuation_shares_the_context_subspace():
    s = _small()
    k, _ = synth.layer_cache_np(s, 0)
    kn, vn = synth.continuation_np(s, 0, 6)
    assert kn.shape == (6, 2, 256) and vn.shape == (6, 2, 2, 128)
    kn2, _ = synth.continuation_np(s, 0, 6)
    assert torch.equal(kn, kn2)
    for gen in ("np", "torch"):
        if gen == "torch":
            kt, _ = synth.layer_cache_torch(s, 0, 0, "cpu")
            kn, vn = synth.continuation_torch(s, 0, 6, 0, "cpu")
            kc = kt
        else:
            kc = k
        for b in range(2):
            kb = kc[b].double().numpy()
            _, _, vt = np.linalg.svd(kb, full_matrices=False)
            top = vt[:s.latent_rank].T
            x = kn[:, b].double().numpy()
            kept = np.linalg.norm(x @ top, axis=1) / np.linalg.norm(x, axis=1)
            assert kept.min() > 0.97, (gen, kept)
            # the latent process carries on: the first new key is close to the last context key
            c0 = np.dot(x[0], kb[-1]) / (np.linalg.norm(x[0]) * np.linalg.norm(kb[-1]))
            assert c0 > 0.6, (gen, c0)
        assert abs(vn.double().std().item() - 1.0) < 0.1
