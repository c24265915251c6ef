"""Comparison rules between the GPU library and the CPU oracle.

Bars (floating point from bf16 storage with fp32 accumulation):
* selected chunk ids bit-exact, except chunks whose oracle score S2 lies within
  1e-3 relative of the oracle's K-th score (near ties may swap);
* attention outputs: max |err| <= 2e-2 and relative L2 <= 5e-3, against the
  oracle's output for its own selection; for a pair whose selection swapped a
  near tie (several selections are then correct), against the oracle's exact
  attention over the selection the GPU made, once that selection has passed the
  tie rule;
* hit counts exact against the oracle whenever the selections agree, and always
  equal to |I_t & I_{t-1}| of the GPU's own consecutive selections;
* build state (check_build): outlier and candidate ids exact; every landmark
  value and every exact outlier / window key equal to the oracle's rounding (the
  GPU rotates and averages in float64 and rounds once, as the oracle does); B
  and the rows of A equal to the oracle's rounding except where the GPU's
  eigenvector basis (subspace iteration on a Gram matrix with fp32 sums of 8
  exact products) and LAPACK's SVD differ near a rounding boundary: those
  values are one spacing of the storage format away and at most 1 in 1000 of
  them differ (seen: a few in a million at the benchmarked shapes); columns of nearly equal singular
  values are fixed only as a subspace and are covered by A B per head within
  1e-2 relative Frobenius.

Two protocols use these bars.  End to end (test_gpu_end_to_end.py and the
64-step full-size case), the oracle decodes on its own build.  On the GPU's
state (adopt_gpu_state: the oracle decodes on the exported landmarks, A and B),
the comparison measures the decode arithmetic alone and is held to the tighter
DECODE_* bars.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import shadowkv as O

TIE_REL = 1e-3
MAX_ABS = 2e-2
REL_L2 = 5e-3
# Decode steps on the adopted state (landmarks, A, B as the GPU built them), no
# appended tokens: what remains is the decode path's own arithmetic -- fp32
# logits, softmax weights carried at 16 bits, and rebuilt keys rounded to bf16
# from an fp32 sum (the oracle's from fp64; one that straddles a rounding
# boundary moves one key element by a bf16 spacing).  Seen at most 2.8e-4 max
# and 2.7e-5 relative L2 over the parity cases; the bars leave 7x room.
DECODE_MAX_ABS = 2e-3
DECODE_REL_L2 = 2e-4
LANDMARK_DIFF_FRACTION = 1e-3
FACTOR_DIFF_FRACTION = 1e-3


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 numpy bit patterns (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_ids(gpu_ids: np.ndarray, st: O.State, res: O.StepResult) -> list:
    """Assert the tie rule per pair; returns the pairs (b, h) whose ids differ."""
    cfg = st.cfg
    K = cfg.top_k
    differ = []
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            g = gpu_ids[b, h]
            assert np.all(np.diff(g) > 0), f"pair ({b},{h}) ids not strictly ascending"
            o = res.ids[b, h]
            if np.array_equal(g, o):
                continue
            differ.append((b, h))
            cand = st.cand[b, h]
            pos = np.searchsorted(cand, g)
            assert np.all(pos < len(cand)) and np.array_equal(cand[np.minimum(pos, len(cand) - 1)], g), \
                f"pair ({b},{h}) selected a non-candidate chunk"
            s2 = res.scores[b, h]
            kth = np.sort(s2)[::-1][K - 1]
            for c in set(g.tolist()) ^ set(o.tolist()):
                sc = s2[np.searchsorted(cand, c)]
                assert abs(sc - kth) <= TIE_REL * kth, \
                    f"pair ({b},{h}) chunk {c}: score {sc} vs K-th {kth} is not a near tie"
    return differ


def reference_out(st: O.State, q_bits, res: O.StepResult, gpu_ids: np.ndarray, differ: list):
    """Oracle outputs, with tie-swapped pairs recomputed over the GPU's selection."""
    ref = res.out.copy()
    q = O.bf16_bits_to_f64(q_bits)
    G = st.cfg.group
    for b, h in differ:
        ref[b, h * G:(h + 1) * G] = O.pair_output(st, q[b], b, h, gpu_ids[b, h].astype(np.int64))
    return ref


def check_out(gpu_out: np.ndarray, ref: np.ndarray, max_abs=MAX_ABS, rel_l2=REL_L2):
    err = np.abs(gpu_out.astype(np.float64) - ref)
    rl2 = np.linalg.norm(gpu_out.astype(np.float64) - ref) / np.linalg.norm(ref)
    assert err.max() <= max_abs, f"max |err| {err.max():.3e} > {max_abs}"
    assert rl2 <= rel_l2, f"rel L2 {rl2:.3e} > {rel_l2}"
    return float(err.max()), float(rl2)


def bf16_close(gpu_bits: np.ndarray, ref: np.ndarray, slack: float) -> float:
    """Worst excess of |gpu - ref| over one bf16 spacing at ref plus an absolute
    slack (fp32 arithmetic on O(1) values can land on either side of a rounding
    boundary, and cancellation makes tiny results inexact in absolute terms).
    Returns max(|gpu - ref| - spacing(ref) - slack); <= 0 passes."""
    if ref.size == 0:
        return -np.inf
    g = O.bf16_bits_to_f64(gpu_bits)
    _, e = np.frexp(ref)
    spacing = np.where(ref == 0, 0.0, np.ldexp(1.0, e - 8))
    return float(np.max(np.abs(g - ref) - spacing - slack))


def e5m2_close(gpu_bits: np.ndarray, ref: np.ndarray, slack: float = 0.0) -> tuple[float, float]:
    """FP8 values exported as bf16 bits vs the oracle's E5M2-rounded values.
    Returns (worst excess of |gpu - ref| over one E5M2 spacing at ref plus an
    absolute slack, fraction of values that differ)."""
    if ref.size == 0:
        return -np.inf, 0.0
    g = O.bf16_bits_to_f64(gpu_bits)
    assert np.array_equal(O.round_e5m2(g), g), "exported values are not E5M2 values"
    _, e = np.frexp(ref)
    spacing = np.where(np.abs(ref) < 2.0 ** -14, 2.0 ** -16, np.ldexp(1.0, e - 3))
    diff = np.abs(g - ref)
    return float(np.max(diff - spacing - slack)), float(np.mean(diff > 0))


def adopt_gpu_state(st: O.State, gpu: dict) -> None:
    """Run the oracle's decode on the landmarks and the factors A, B the GPU
    built, once they have passed check_build (module docstring)."""
    st.L = O.bf16_bits_to_f64(gpu["landmarks"]).reshape(st.L.shape)
    st.A = O.bf16_bits_to_f64(gpu["A"]).reshape(st.A.shape)
    st.B = O.bf16_bits_to_f64(gpu["B"]).reshape(st.B.shape)


def check_build(gpu: dict, st: O.State, exact_landmarks: bool = True):
    """Build-state parity: outliers, candidates, landmarks, exact caches, factors.

    The GPU rotates, averages and takes cosines in float64 and rounds each stored
    value once, so with ``exact_landmarks`` every landmark value and every exact
    outlier / window key must equal the oracle's rounding (a float64 mean within
    ~1e-15 of a rounding boundary could still go either way; none is expected at
    these sizes)."""
    cfg = st.cfg
    np.testing.assert_array_equal(gpu["outlier_ids"], st.outliers)
    np.testing.assert_array_equal(gpu["cand_ids"], st.cand)
    # min-cos is computed in float64 and exported as float32
    np.testing.assert_allclose(gpu["min_cos"], st.min_cos, rtol=0, atol=1e-6)
    if exact_landmarks:
        lm = O.bf16_bits_to_f64(gpu["landmarks"]).reshape(st.L.shape)
        nd = int(np.sum(lm != st.L))
        assert nd == 0, f"{nd} landmark values differ from the oracle's rounding"
        np.testing.assert_array_equal(O.bf16_bits_to_f64(gpu["k_outlier"]).reshape(st.K_out.shape), st.K_out)
        np.testing.assert_array_equal(O.bf16_bits_to_f64(gpu["k_window"]).reshape(st.K_win.shape), st.K_win)
    if cfg.landmark_format == "e5m2":
        excess, frac = e5m2_close(gpu["landmarks"], st.L)
        assert excess <= 0, f"FP8 landmark off by more than one spacing ({excess})"
        assert frac <= LANDMARK_DIFF_FRACTION, f"{frac:.2e} of the FP8 landmarks differ"
    else:
        assert bf16_close(gpu["landmarks"], st.L, 1e-5) <= 0
        if st.L.size:
            frac = float(np.mean(O.bf16_bits_to_f64(gpu["landmarks"]) != st.L))
            assert frac <= LANDMARK_DIFF_FRACTION, f"{frac:.2e} of the bf16 landmarks differ"
    assert bf16_close(gpu["k_outlier"], st.K_out, 1e-5) <= 0
    assert bf16_close(gpu["k_window"], st.K_win, 1e-5) <= 0
    np.testing.assert_array_equal(O.bf16_bits_to_f64(gpu["v_outlier"]), st.V_out)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(gpu["v_window"]), st.V_win)
    r = cfg.rank
    # the GPU's Gram adds fp32 sums of 8 exact bf16 products in fp64: its error is
    # about 1e-9 of the largest entries, and by Weyl's theorem no eigenvalue moves
    # by more than the error's spectral norm, so the bar is relative to lambda_max
    lam = st.sigma[:, :r] ** 2
    np.testing.assert_allclose(gpu["eigvals"], lam, rtol=1e-8, atol=1e-8 * float(lam.max()))
    A = O.bf16_bits_to_f64(gpu["A"])
    B = O.bf16_bits_to_f64(gpu["B"])
    # Same gauge: the factors agree column by column up to rounding where the
    # singular vector is well determined.  Davis-Kahan bounds the perturbation of
    # eigenvector j by ||dG|| / gap_j (gap to the neighbouring eigenvalues of the
    # full spectrum); with ||dG|| <= 1e-8 lambda_max (the bar above) a column is
    # compared element by element where that bound is below 1e-4, with the bound
    # as extra absolute slack.  Columns inside a cluster of nearly equal
    # eigenvalues are determined only as a subspace: the A B products below cover
    # them.
    for bi in range(cfg.batch):
        lam_all = st.sigma[bi] ** 2
        gap = np.full(r, np.inf)
        gap[1:] = np.minimum(gap[1:], lam_all[:r - 1] - lam_all[1:r])
        nxt = min(r, len(lam_all) - 1)
        gap[:nxt] = np.minimum(gap[:nxt], lam_all[:nxt] - lam_all[1:nxt + 1])
        dk = 1e-8 * lam_all[0] / np.maximum(gap, 1e-300)
        well = dk < 1e-4
        gb, ob = B[bi][:, well], st.B[bi][:, well]                    # [H, n_well, d]
        _, e = np.frexp(ob)
        if cfg.b_format == "e5m2":
            spacing = np.where(np.abs(ob) < 2.0 ** -14, 2.0 ** -16, np.ldexp(1.0, e - 3))
        else:
            spacing = np.where(ob == 0, 0.0, np.ldexp(1.0, e - 8))
        excess = np.abs(gb - ob) - spacing - 1e-9 - dk[well][None, :, None]
        assert excess.size == 0 or excess.max() <= 0, f"B differs beyond rounding ({excess.max()})"
        # A = K Psi in float64 on both sides, rounded once: equal but for values
        # within the two bases' difference of a rounding boundary.  Column j of
        # the basis moves by at most dk_j, so an element of A moves by at most
        # sigma_max * dk_j (a row of K has norm <= sigma_max).
        slack = st.sigma[bi][0] * dk[well][None, :] + 1e-9 * np.abs(st.A[bi]).max()
        if cfg.a_format == "e5m2":
            excess, frac = e5m2_close(gpu["A"][bi][:, well], st.A[bi][:, well], slack)
            assert excess <= 0, f"FP8 A off by more than one spacing ({excess})"
        else:
            ga, oa = A[bi][:, well], st.A[bi][:, well]
            _, e = np.frexp(oa)
            excess = np.abs(ga - oa) - np.where(oa == 0, 0.0, np.ldexp(1.0, e - 8)) - slack
            assert excess.size == 0 or excess.max() <= 0, f"A differs beyond one spacing ({excess.max()})"
            frac = float(np.mean(ga != oa)) if ga.size else 0.0
        assert frac <= FACTOR_DIFF_FRACTION, f"{frac:.2e} of the values of A differ"
        if gb.size:
            fb = float(np.mean(gb != ob))
            assert fb <= FACTOR_DIFF_FRACTION, f"{fb:.2e} of the values of B differ"
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            pg = A[b] @ B[b, h]
            po = st.A[b] @ st.B[b, h]
            assert np.linalg.norm(pg - po) <= 1e-2 * np.linalg.norm(po)
