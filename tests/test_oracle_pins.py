"""Pins of the oracle against what the pages and the mathematics fix.

None of these re-type the oracle's formulas: each compares it with a closed
form, a different routine (eigh of the Gram matrix, torch's bfloat16
conversion, complex rotation), brute force in pure Python on tiny inputs, or a
value the pages print (tests/golden/).
"""
import dataclasses
import itertools
import json
import math
import os
import random

import numpy as np
import pytest
import torch

from oracle import shadowkv as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=16, seq_len=64, rank=8,
                chunk=4, top_k=3, n_outlier=2, window=8, rope_theta=10000.0)
    base.update(kw)
    return O.Config(**base)


def lowrank_keys(rng, b, S, hd, R, noise=0.05):
    a = rng.standard_normal((b, S, R))
    bm = rng.standard_normal((b, R, hd)) / math.sqrt(R)
    return a @ bm + noise * rng.standard_normal((b, S, hd))


# ---------------------------------------------------------------- bf16 helpers

def test_round_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    one = 1.0
    assert O.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0          # halfway, even down
    assert O.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6  # halfway, even up
    assert O.round_bf16(np.array([-(one + 2 ** -8 + 2 ** -30)]))[0] == -(1.0 + 2 ** -7)
    assert O.round_bf16(np.array([0.0]))[0] == 0.0


def test_bf16_bits_decode_matches_torch():
    rng = np.random.default_rng(2)
    t = torch.from_numpy(rng.standard_normal(5000).astype(np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy()
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits), t.to(torch.float64).numpy())


def test_round_e5m2_matches_torch_float8_e5m2():
    # normal and subnormal magnitudes (2^-18 .. 2^15); torch's conversion is
    # from float32, so the inputs are float32 values
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(40000) * np.exp2(rng.uniform(-18, 15, 40000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e5m2).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_e5m2(x.astype(np.float64)), ref)


def test_round_e5m2_hand_cases():
    r = lambda v: float(O.round_e5m2(np.array([v]))[0])
    assert r(1.0 + 2 ** -3) == 1.0                  # halfway between 1 and 1.25: even (1.0)
    assert r(1.0 + 3 * 2 ** -3) == 1.5              # halfway between 1.25 and 1.5: even (1.5)
    assert r(-1.3) == -1.25
    assert r(2 ** -14) == 2 ** -14                  # smallest normal
    assert r(3 * 2 ** -17) == 2 * 2 ** -16          # subnormal spacing 2^-16, tie to even
    assert r(57344.0) == 57344.0 and r(-61439.0) == -57344.0
    assert r(61440.0) == np.inf                     # halfway past the largest: rounds up, overflows
    assert r(0.0) == 0.0


# ---------------------------------------------------------------- RoPE

def test_rope_closed_forms():
    d, theta = 16, 10000.0
    e0 = np.zeros((1, d)); e0[0, 0] = 1.0
    for p in [0, 1, 7, 123456]:
        y = O.apply_rope(e0, np.array([p]), theta)[0]
        expect = np.zeros(d); expect[0] = math.cos(p); expect[d // 2] = math.sin(p)
        np.testing.assert_allclose(y, expect, atol=1e-12)
    # the slowest pair turns by p * theta^(-(d-2)/d)
    e = np.zeros((1, d)); e[0, d // 2 - 1] = 1.0
    y = O.apply_rope(e, np.array([3]), theta)[0]
    w = 3 * theta ** (-(d - 2) / d)
    assert abs(y[d // 2 - 1] - math.cos(w)) < 1e-12 and abs(y[d - 1] - math.sin(w)) < 1e-12


def test_rope_is_a_rotation_with_relative_positions():
    rng = np.random.default_rng(3)
    d, theta = 128, 500000.0
    x, y = rng.standard_normal((2, 1, d))
    for p in [0, 5, 1000, 2 ** 20 - 1]:
        rx = O.apply_rope(x, np.array([p]), theta)
        assert abs(np.linalg.norm(rx) - np.linalg.norm(x)) < 1e-10
    # <R_p x, R_p' y> depends only on p - p'
    def dot(p, pp):
        return float(O.apply_rope(x, np.array([p]), theta)[0] @ O.apply_rope(y, np.array([pp]), theta)[0])
    assert abs(dot(10, 3) - dot(1007, 1000)) < 1e-9
    assert abs(dot(900000, 899990) - dot(10, 0)) < 1e-8
    assert abs(dot(4, 4) - float(x[0] @ y[0])) < 1e-10


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(4)
    d, theta = 128, 500000.0
    x = rng.standard_normal((6, d))
    pos = np.array([0, 1, 2, 99, 65535, 1048575])
    h = d // 2
    freq = np.array([theta ** (-2.0 * i / d) for i in range(h)])
    z = (x[:, :h] + 1j * x[:, h:]) * np.exp(1j * np.outer(pos, freq))
    np.testing.assert_allclose(O.apply_rope(x, pos, theta), np.concatenate([z.real, z.imag], 1),
                               atol=1e-10)


# ---------------------------------------------------------------- SVD

def test_svd_full_rank_reconstructs_exactly():
    rng = np.random.default_rng(5)
    H, d, S = 2, 16, 80
    k = rng.standard_normal((S, H * d))
    a, b, _ = O.truncated_svd(k, H * d, H)
    for h in range(H):
        np.testing.assert_allclose(a @ b[h], k[:, h * d:(h + 1) * d], atol=1e-10)


def test_svd_eckart_young_and_subspace_vs_gram_eigh():
    rng = np.random.default_rng(6)
    H, d, S, r = 2, 16, 200, 6
    k = lowrank_keys(rng, 1, S, H * d, 6, noise=0.1)[0]
    a, b, _ = O.truncated_svd(k, r, H)
    approx = np.concatenate([a @ b[h] for h in range(H)], axis=1)
    lam, vec = np.linalg.eigh(k.T @ k)            # ascending eigenvalues
    tail = lam[: H * d - r].sum()
    assert abs(np.sum((k - approx) ** 2) - tail) < 1e-9 * np.sum(lam)
    psi = np.concatenate([b[h] for h in range(H)], axis=1).T      # [H d, r]
    np.testing.assert_allclose(psi.T @ psi, np.eye(r), atol=1e-10)
    assert O.subspace_similarity(psi, vec[:, -r:]) > 1 - 1e-10
    # A = U_r Sigma_r equals K Psi, and squared column norms are the top eigenvalues
    np.testing.assert_allclose(a, k @ psi, atol=1e-9)
    np.testing.assert_allclose(np.sort((a ** 2).sum(0)), np.sort(lam[-r:]), rtol=1e-9)


def test_svd_gauge():
    rng = np.random.default_rng(7)
    k = rng.standard_normal((50, 32))
    _, b, _ = O.truncated_svd(k, 5, 2)
    psi = np.concatenate([b[h] for h in range(2)], axis=1)   # [r, H d]
    for row in psi:
        j = int(np.argmax(np.abs(row)))
        assert row[j] > 0


def test_subspace_similarity_range():
    rng = np.random.default_rng(8)
    q1, _ = np.linalg.qr(rng.standard_normal((20, 4)))
    q2, _ = np.linalg.qr(rng.standard_normal((20, 4)))
    assert abs(O.subspace_similarity(q1, q1) - 1) < 1e-12
    e = np.eye(20)
    assert abs(O.subspace_similarity(e[:, :4], e[:, 4:8])) < 1e-12
    assert 0 <= O.subspace_similarity(q1, q2) <= 1


# ---------------------------------------------------------------- landmarks / outliers

def _py_mean(rows):
    return [sum(r[i] for r in rows) / len(rows) for i in range(len(rows[0]))]


def _py_cos(a, b):
    na = math.sqrt(sum(x * x for x in a)); nb = math.sqrt(sum(x * x for x in b))
    return sum(x * y for x, y in zip(a, b)) / max(na * nb, 1e-8)


def test_landmarks_and_min_cos_brute_force():
    rng = np.random.default_rng(9)
    kr = rng.standard_normal((2, 48, 6))
    C = 4
    lm = O.landmarks(kr, C)
    mc = O.chunk_min_cos(kr, lm, C)
    for h in range(2):
        for j in range(12):
            rows = [list(kr[h, j * C + i]) for i in range(C)]
            m = _py_mean(rows)
            assert np.allclose(lm[h, j], m, atol=1e-12)
            assert abs(mc[h, j] - min(_py_cos(r, m) for r in rows)) < 1e-12


def test_constant_chunk_and_planted_outlier():
    rng = np.random.default_rng(10)
    base = rng.standard_normal(8)
    kr = np.tile(base, (1, 32, 1)) + 0.01 * rng.standard_normal((1, 32, 8))
    kr[0, 8:12] = base                    # chunk 2: identical keys
    kr[0, 21] = -base                     # chunk 5: one key points the other way
    lm = O.landmarks(kr, 4)
    mc = O.chunk_min_cos(kr, lm, 4)
    np.testing.assert_allclose(lm[0, 2], base, atol=1e-12)
    assert abs(mc[0, 2] - 1.0) < 1e-12 and mc[0, 5] < 0
    assert list(O.pick_outliers(mc[0], 1, 8)) == [5]
    z = np.zeros((1, 8, 3))                # zero vectors give cosine 0
    assert np.all(O.chunk_min_cos(z, O.landmarks(z, 4), 4) == 0)


@pytest.mark.parametrize("seed", range(5))
def test_topk_and_outliers_exhaustive_sort(seed):
    rnd = random.Random(seed)
    n = rnd.randint(20, 256)
    # many exact ties on purpose
    vals = [rnd.choice([0.1, 0.2, 0.25, 0.5]) if rnd.random() < 0.5 else rnd.random() for _ in range(n)]
    ids = list(range(100, 100 + n))
    for k in [1, 2, n // 3, n - 1, n]:
        ref = sorted(sorted(zip(vals, ids), key=lambda t: (-t[0], t[1]))[:k], key=lambda t: t[1])
        got = O.top_k(np.array(vals), np.array(ids), k)
        assert list(got) == [i for _, i in ref]
        ref_o = sorted(sorted(range(n), key=lambda j: (vals[j], j))[:k])
        assert list(O.pick_outliers(np.array(vals), k, n)) == ref_o


# ---------------------------------------------------------------- scoring

def test_scores_brute_force_and_group_max():
    rng = np.random.default_rng(11)
    cfg = small_cfg(top_k=4)
    k = lowrank_keys(rng, 1, cfg.seq_len, cfg.n_kv_heads * cfg.head_dim, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v, storage_rounding=False)
    q = rng.standard_normal((cfg.n_q_heads, cfg.head_dim)) * 2
    G, d = cfg.group, cfg.head_dim
    for h in range(cfg.n_kv_heads):
        s2 = O.chunk_scores(st, q, 0, h)
        lms = [list(x) for x in st.L[0, h]]
        probs = []
        for g in range(G):
            lg = [sum(a * b for a, b in zip(q[h * G + g], l)) / math.sqrt(d) for l in lms]
            mx = max(lg)
            e = [math.exp(x - mx) for x in lg]
            z = sum(e)
            probs.append([x / z for x in e])
            assert abs(sum(probs[-1]) - 1.0) < 1e-12
        ref = [max(probs[g][c] for g in range(G)) for c in range(len(lms))]
        np.testing.assert_allclose(s2, ref, rtol=1e-12)


def test_group_of_one_selects_by_raw_logits():
    rng = np.random.default_rng(12)
    cfg = small_cfg(n_q_heads=2, n_kv_heads=2, top_k=5)
    k = lowrank_keys(rng, 1, cfg.seq_len, 2 * cfg.head_dim, 8)
    v = rng.standard_normal((1, 2, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v)
    q = rng.standard_normal((1, 2, cfg.head_dim))
    res = O.decode_step(st, q)
    for h in range(2):
        raw = st.L[0, h] @ q[0, h]
        assert list(res.ids[0, h]) == list(np.sort(st.cand[0, h][np.argsort(-raw, kind="stable")[:5]]))


def test_group_max_two_heads_hand_example():
    # two candidates, head 0 prefers chunk a (logit gap g0), head 1 prefers b
    cfg = small_cfg(n_q_heads=2, n_kv_heads=1, head_dim=4, seq_len=16, chunk=4, top_k=1,
                    n_outlier=0, window=8)
    st = O.State(cfg, None, None, None, np.array([[[[1.0, 0, 0, 0], [0, 1.0, 0, 0]]]]),
                 np.array([[[0, 1]]]), None, None, None, None, None, None, None, False)
    q = np.array([[4.0, 0, 0, 0], [0, 6.0, 0, 0]])      # logits / sqrt(4): (2, 0) and (0, 3)
    s2 = O.chunk_scores(st, q, 0, 0)
    p0 = 1 / (1 + math.exp(-2)); p1 = 1 / (1 + math.exp(-3))
    np.testing.assert_allclose(s2, [p0, p1], rtol=1e-12)


# ---------------------------------------------------------------- attention

def test_full_budget_equals_dense_attention():
    rng = np.random.default_rng(13)
    cfg = small_cfg()
    n_c = cfg.seq_len // cfg.chunk
    cfg = small_cfg(top_k=n_c - 2 - 2, rank=cfg.n_kv_heads * cfg.head_dim)
    hd = cfg.n_kv_heads * cfg.head_dim
    k = rng.standard_normal((1, cfg.seq_len, hd))
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v, storage_rounding=False)
    q = rng.standard_normal((1, cfg.n_q_heads, cfg.head_dim)) * 3
    res = O.decode_step(st, q)
    d, G = cfg.head_dim, cfg.group
    pos = np.arange(cfg.seq_len)
    for hq in range(cfg.n_q_heads):
        h = hq // G
        kr = O.apply_rope(k[0, :, h * d:(h + 1) * d], pos, cfg.rope_theta)
        s = kr @ q[0, hq] / math.sqrt(d)
        p = np.exp(s - s.max()); p /= p.sum()
        np.testing.assert_allclose(res.out[0, hq], p @ v[0, h], atol=1e-9)


def test_sparse_attention_brute_force():
    rng = np.random.default_rng(14)
    cfg = small_cfg(top_k=3)
    hd = cfg.n_kv_heads * cfg.head_dim
    k = lowrank_keys(rng, 1, cfg.seq_len, hd, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v, storage_rounding=False)
    q = rng.standard_normal((1, cfg.n_q_heads, cfg.head_dim)) * 3
    res = O.decode_step(st, q)
    d, G, C = cfg.head_dim, cfg.group, cfg.chunk
    S = cfg.seq_len
    for hq in range(cfg.n_q_heads):
        h = hq // G
        toks = sorted(set(t for j in list(st.outliers[0, h]) + list(res.ids[0, h])
                          for t in range(j * C, j * C + C)) | set(range(S - cfg.window, S)))
        keys = []
        for t in toks:
            exact = t >= S - cfg.window or (t // C) in set(st.outliers[0, h])
            if exact:
                row = k[0, t, h * d:(h + 1) * d]
            else:   # rebuilt from the factors
                row = [sum(st.A[0, t, i] * st.B[0, h, i, c] for i in range(cfg.rank)) for c in range(d)]
            keys.append(O.apply_rope(np.array([row]), np.array([t]), cfg.rope_theta)[0])
        logits = [sum(a * b for a, b in zip(q[0, hq], kk)) / math.sqrt(d) for kk in keys]
        mx = max(logits)
        w = [math.exp(x - mx) for x in logits]
        z = sum(w)
        ref = [sum(w[i] * v[0, h, t, c] for i, t in enumerate(toks)) / z for c in range(d)]
        np.testing.assert_allclose(res.out[0, hq], ref, atol=1e-10)


# ---------------------------------------------------------------- temporal cache

def test_hit_counts_against_set_algebra():
    rng = np.random.default_rng(15)
    cfg = small_cfg(seq_len=256, top_k=10, n_outlier=3)
    hd = cfg.n_kv_heads * cfg.head_dim
    k = lowrank_keys(rng, 1, cfg.seq_len, hd, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v)
    q = rng.standard_normal((1, cfg.n_q_heads, cfg.head_dim))
    r0 = O.decode_step(st, q)
    r1 = O.decode_step(st, q, r0.ids)
    assert np.all(r1.hits == cfg.top_k)                     # identical query => alpha = 1
    np.testing.assert_array_equal(r1.out, r0.out)
    prev = r0.ids
    for _ in range(5):
        q = 0.9 * q + math.sqrt(0.19) * rng.standard_normal(q.shape)
        r = O.decode_step(st, q, prev)
        for h in range(cfg.n_kv_heads):
            assert r.hits[0, h] == len(set(r.ids[0, h]) & set(prev[0, h]))
            assert len(set(r.ids[0, h])) == cfg.top_k
            assert not (set(r.ids[0, h]) & set(st.outliers[0, h]))
            assert max(r.ids[0, h]) < cfg.n_chunks - cfg.n_win_chunks
        prev = r.ids


def test_build_partitions_chunks():
    rng = np.random.default_rng(16)
    cfg = small_cfg(batch=2, seq_len=128, n_outlier=4)
    hd = cfg.n_kv_heads * cfg.head_dim
    k = lowrank_keys(rng, 2, cfg.seq_len, hd, 8)
    v = rng.standard_normal((2, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v)
    n_elig = cfg.n_chunks - cfg.n_win_chunks
    for b in range(2):
        for h in range(cfg.n_kv_heads):
            both = np.sort(np.concatenate([st.cand[b, h], st.outliers[b, h]]))
            np.testing.assert_array_equal(both, np.arange(n_elig))
            # outliers have the lowest min-cos among the eligible chunks
            assert st.min_cos[b, h, st.outliers[b, h]].max() <= st.min_cos[b, h, st.cand[b, h]].min()


# ---------------------------------------------------------------- printed formulas

def test_equivalent_bandwidth_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "equivalent_bandwidth.json")))
    i = g["inputs"]
    bt = O.equivalent_bandwidth(i["S"], i["C"], i["K"], i["O"], g["alpha"],
                                i["B_gpu_TBps"], i["B_pcie_GBps"] / 1000.0)
    assert abs(bt - g["expected_TBps"]) <= g["abs_tol_TBps"]
    assert abs(bt / i["B_gpu_TBps"] - g["expected_ratio_to_gpu"]) <= g["abs_tol_ratio"]
    # no PCIe penalty at alpha = 1: 2 S / (S/C + 2 (K+O) C) times B_gpu
    full = O.equivalent_bandwidth(i["S"], i["C"], i["K"], i["O"], 1.0, 2.0, 0.0315)
    assert abs(full - 2 * 131072 * 2.0 / (16384 + 4864)) < 1e-9


def test_memory_savings_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "memory_savings.json")))
    i = g["inputs"]
    ms = O.memory_savings(i["S"], i["M"], i["C"], i["K"], i["O"], i["r"])
    assert abs(ms - g["expected"]) <= g["abs_tol"]


# ---------------------------------------------------------------- storage rounding

def test_storage_rounding_is_applied_to_stored_state():
    rng = np.random.default_rng(17)
    cfg = small_cfg()
    hd = cfg.n_kv_heads * cfg.head_dim
    k = lowrank_keys(rng, 1, cfg.seq_len, hd, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    st = O.build(cfg, k, v, storage_rounding=True)
    for x in [st.A, st.B, st.L, st.K_out, st.K_win]:
        np.testing.assert_array_equal(O.round_bf16(x), x)
    st0 = O.build(cfg, k, v, storage_rounding=False)
    assert not np.array_equal(st0.A, st.A)
    np.testing.assert_allclose(st0.A, st.A, rtol=2 ** -8)


def test_fp8_formats_round_landmarks_a_and_b():
    # FP8 landmarks and A: exactly the E5M2 rounding of the unrounded build's
    # values; B (unless asked for) and the exact keys stay bf16; a decode step
    # rebuilds its keys from the rounded A (its outputs differ from the bf16
    # build's)
    rng = np.random.default_rng(19)
    cfg = small_cfg()
    hd = cfg.n_kv_heads * cfg.head_dim
    k = lowrank_keys(rng, 1, cfg.seq_len, hd, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, cfg.head_dim))
    q = rng.standard_normal((1, cfg.n_q_heads, cfg.head_dim))
    st0 = O.build(cfg, k, v, storage_rounding=False)
    st = O.build(dataclasses.replace(cfg, landmark_format="e5m2", a_format="e5m2"), k, v)
    np.testing.assert_array_equal(st.L, O.round_e5m2(st0.L))
    np.testing.assert_array_equal(st.A, O.round_e5m2(st0.A))
    np.testing.assert_array_equal(st.B, O.round_bf16(st0.B))
    np.testing.assert_array_equal(st.K_out, O.round_bf16(st0.K_out))
    assert np.abs(st.A - st0.A).max() > 2 ** -6 * np.abs(st0.A).max()   # a coarse grid indeed
    bf = O.build(cfg, k, v)
    r8, rb = O.decode_step(st, q), O.decode_step(bf, q)
    assert not np.array_equal(r8.out, rb.out)
    # FP8 B as well: B is the E5M2 rounding, and the appended rows of A are
    # projected with that B
    st_b = O.build(dataclasses.replace(cfg, b_format="e5m2"), k, v)
    np.testing.assert_array_equal(st_b.B, O.round_e5m2(st0.B))
    np.testing.assert_array_equal(st_b.A, O.round_bf16(st0.A))
    kb = rng.standard_normal((1, hd))
    O.append(st_b, kb, rng.standard_normal((1, cfg.n_kv_heads, cfg.head_dim)), lowrank=True)
    np.testing.assert_array_equal(st_b.A[:, -1], O.round_bf16(kb[0] @ O.psi_t(st_b, 0).T)[None])
    assert np.array_equal(O.psi_t(st_b, 0), O.round_e5m2(O.psi_t(st_b, 0)))
    # the appended rows of A take the same format
    kn = rng.standard_normal((1, hd))
    O.append(st, kn, rng.standard_normal((1, cfg.n_kv_heads, cfg.head_dim)), lowrank=True)
    np.testing.assert_array_equal(st.A[:, -1], O.round_e5m2(kn[0] @ O.psi_t(st, 0).T)[None])


# ---------------------------------------------------------------- generated tokens

@pytest.mark.parametrize("lowrank", [False, True])
def test_appended_tokens_full_budget_equals_dense_attention(lowrank):
    # full rank and every candidate selected: attention over the context and the
    # generated tokens is plain dense attention over the grown sequence, the
    # t-th generated token rotated at position seq_len + t (with a square
    # orthogonal Psi the low-rank state loses nothing)
    rng = np.random.default_rng(31)
    cfg = small_cfg()
    n_c = cfg.seq_len // cfg.chunk
    cfg = small_cfg(top_k=n_c - 2 - 2, rank=cfg.n_kv_heads * cfg.head_dim)
    hd, d, G, S = cfg.n_kv_heads * cfg.head_dim, cfg.head_dim, cfg.group, cfg.seq_len
    T = 3
    k = rng.standard_normal((1, S + T, hd))
    v = rng.standard_normal((1, cfg.n_kv_heads, S + T, d))
    st = O.build(cfg, k[:, :S], v[:, :, :S], storage_rounding=False)
    for t in range(T):
        O.append(st, k[:, S + t], v[:, :, S + t], lowrank=lowrank)
    q = rng.standard_normal((1, cfg.n_q_heads, d)) * 3
    res = O.decode_step(st, q)
    pos = np.arange(S + T)
    for hq in range(cfg.n_q_heads):
        h = hq // G
        kr = O.apply_rope(k[0, :, h * d:(h + 1) * d], pos, cfg.rope_theta)
        s = kr @ q[0, hq] / math.sqrt(d)
        p = np.exp(s - s.max()); p /= p.sum()
        np.testing.assert_allclose(res.out[0, hq], p @ v[0, h], atol=1e-9)


def test_lowrank_state_is_the_projection_on_the_context_subspace():
    # a generated token's row of A, mapped back through Psi^T, is k' projected on
    # the top-r right singular subspace of the context keys (computed here from
    # eigh of the Gram matrix), and a context key appended again gets exactly
    # its own row of A (A = K Psi)
    rng = np.random.default_rng(32)
    cfg = small_cfg(seq_len=128, rank=6)
    hd, d, S = cfg.n_kv_heads * cfg.head_dim, cfg.head_dim, cfg.seq_len
    k = lowrank_keys(rng, 1, S, hd, 10)
    v = rng.standard_normal((1, cfg.n_kv_heads, S, d))
    st = O.build(cfg, k, v, storage_rounding=False)
    w, U = np.linalg.eigh(k[0].T @ k[0])
    top = U[:, np.argsort(w)[::-1][:cfg.rank]]
    proj = top @ top.T
    knew = [rng.standard_normal(hd), k[0, 17]]
    for kn in knew:
        O.append(st, kn[None], rng.standard_normal((1, cfg.n_kv_heads, d)), lowrank=True)
    psi_t = np.concatenate([st.B[0, h] for h in range(cfg.n_kv_heads)], axis=1)   # [r, H d]
    for t, kn in enumerate(knew):
        back = st.A[0, S + t] @ psi_t
        np.testing.assert_allclose(back, kn @ proj, atol=1e-9)
        assert np.abs((kn - back) @ top).max() < 1e-9          # residual orthogonal to Psi
    np.testing.assert_allclose(st.A[0, S + 1], st.A[0, 17], atol=1e-9)


def test_appended_tokens_leave_selection_alone_and_are_rounded():
    # fewer tokens than a chunk: nothing joins the candidates yet
    rng = np.random.default_rng(33)
    cfg = small_cfg(seq_len=128, top_k=4)
    hd, d, S = cfg.n_kv_heads * cfg.head_dim, cfg.head_dim, cfg.seq_len
    k = lowrank_keys(rng, 1, cfg.seq_len, hd, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, cfg.seq_len, d))
    q = rng.standard_normal((1, cfg.n_q_heads, d)) * 3
    st = O.build(cfg, k, v)
    before = O.decode_step(st, q)
    for lowrank in (False, True):
        st2 = O.build(cfg, k, v)
        for _ in range(cfg.chunk - 1):
            O.append(st2, rng.standard_normal((1, hd)), rng.standard_normal((1, cfg.n_kv_heads, d)),
                     lowrank=lowrank)
        after = O.decode_step(st2, q)
        np.testing.assert_array_equal(after.ids, before.ids)
        assert not np.allclose(after.out, before.out)
        stored = [st2.A[:, S:], st2.K_win] if lowrank else [st2.K_new]
        for arr in stored:
            as32 = torch.tensor(arr, dtype=torch.float32)
            np.testing.assert_array_equal(as32.to(torch.bfloat16).to(torch.float64).numpy(), arr)


@pytest.mark.parametrize("window,n_new", [(8, 14), (8, 12), (0, 9)])
def test_lowrank_folding_equals_a_build_on_the_grown_context(window, n_new):
    # no outliers, full rank, no storage rounding: after n = m C + p appended
    # tokens the ShadowKV+ state decodes exactly like a build on the first
    # S + m C tokens of the grown sequence with the last p tokens appended in
    # exact mode (folded landmarks, chunk ids, rolled window, A rows and values
    # all have to line up)
    rng = np.random.default_rng(34)
    cfg = small_cfg(n_outlier=0, window=window, top_k=3)
    cfg = small_cfg(n_outlier=0, window=window, top_k=3, rank=cfg.n_kv_heads * cfg.head_dim)
    hd, d, S, C = cfg.n_kv_heads * cfg.head_dim, cfg.head_dim, cfg.seq_len, cfg.chunk
    m, p = divmod(n_new, C)
    k = lowrank_keys(rng, 1, S + n_new, hd, 8)
    v = rng.standard_normal((1, cfg.n_kv_heads, S + n_new, d))
    st = O.build(cfg, k[:, :S], v[:, :, :S], storage_rounding=False)
    for t in range(n_new):
        O.append(st, k[:, S + t], v[:, :, S + t], lowrank=True)
    grown = dataclasses.replace(cfg, seq_len=S + m * C)
    ref = O.build(grown, k[:, :S + m * C], v[:, :, :S + m * C], storage_rounding=False)
    for t in range(p):
        O.append(ref, k[:, S + m * C + t], v[:, :, S + m * C + t], lowrank=False)
    np.testing.assert_array_equal(st.cand, ref.cand)
    np.testing.assert_allclose(st.L, ref.L, atol=1e-12)
    assert st.cand.shape[2] == cfg.n_cand + m
    for _ in range(3):
        q = rng.standard_normal((1, cfg.n_q_heads, d)) * 3
        a, b = O.decode_step(st, q), O.decode_step(ref, q)
        np.testing.assert_array_equal(a.ids, b.ids)
        np.testing.assert_allclose(a.out, b.out, atol=1e-9)
