"""CPU oracle of ShadowKV's pre-fill (Algorithm 1) and decode step (Algorithm 2).

TEST INFRASTRUCTURE ONLY.  Plain, slow, float64 NumPy, written from the pages'
definitions.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the GPU library never does,
and this module shares no code with it.

Sources (page titles as given on each page):
* "ShadowKV: KV Cache in Shadows for High-Throughput Long-Context LLM
  Inference" (paper-graph-ui summary), section 3.4: low-rank pre-RoPE key
  compression (K ~ A x3 B), landmark construction (chunk means), outlier
  detection (minimum in-chunk cosine), decoding-time selection (softmax of
  Q L^T / sqrt(d), sum over query tokens, max over the KV group, ArgTopK),
  temporal KV cache (hit/miss index scan), key reconstruction
  MatMul(Gather(A, I), B) followed by RoPE, assembly
  [outliers; sparse; local], theoretical equivalent bandwidth (section 3.4
  "Theoretical Equivalent Bandwidth Model") and the memory-savings formula.
* papercache deep notes of the same paper, section A2: Algorithm 1 (pre-fill)
  and Algorithm 2 (decode) pseudocode, the equivalent-bandwidth definition and
  its worked example; appendix A7 for the memory-savings example.
* The paper-graph-ui summary, section 3.4 "Sparse KV Reconstruction and
  Overlapping Strategy": the assembled cache ends with the generated tokens'
  K_new, V_new; its ShadowKV+ paragraph keeps a generated pre-RoPE key k' as
  k' Psi and reconstructs it as (k' Psi) Psi^T with the pre-fill's Psi.

Readings taken where the pages are silent (each also listed in the design
notes): rotate-half RoPE with inv_freq_i = theta^(-2i/d), angles in float64;
the SVD is per batch element over the heads concatenated, A = U_r Sigma_r is
shared by the KV heads and B = V_r^T is split per head; a sign gauge makes the
largest-magnitude entry of every right singular vector positive (lowest index
on ties); the last ``window`` context tokens are kept exact and take part in
neither outlier detection nor selection; the selection softmax runs over the
candidate chunks only (neither outliers nor window chunks) with scale
1/sqrt(head_dim); the group aggregation takes the maximum of per-head
probabilities; ties in top-K prefer the lower chunk id, ties in the outlier
test prefer the lower chunk id; selected ids are returned ascending; cosine
with a zero vector is 0; stored state (A, B, landmarks, outlier and window
keys, rebuilt keys) is rounded once to bfloat16 with round-to-nearest-even
when ``storage_rounding`` is on; with ``landmark_format = "e5m2"`` the
landmarks are rounded instead to FP8 E5M2 (the torch.float8_e5m2 precision of
the summary's precision-sensitivity paragraph, section 5), and with
``a_format = "e5m2"`` the rows of A likewise (context rows and the rows of
generated tokens), and with ``b_format = "e5m2"`` B (bfloat16 by default: the
summary's section 7 expects A, whose rows are each used once per selection, to
tolerate lower precision than B, which enters every rebuilt key).  Generated tokens: the t-th appended token
(t = 0, 1, ...) sits at position seq_len + t and its value is kept as given.
Exact mode (ShadowKV's assembly): every decode step attends to all of them
with the exact key RoPE(k'), and they take no part in scoring or selection.
Low-rank mode (ShadowKV+): a' = k' Psi, with Psi^T the stored B of the batch
element (heads concatenated), is kept as the token's row of A; the last
``window`` tokens of the completed chunks and the tokens of the chunk being
filled stay exact (RoPE(k')); when a chunk completes, the oldest exact chunk
leaves that region and joins the candidates (never the outliers) with the
mean of its stored exact keys as landmark, and from then on is scored,
selected and rebuilt from A like any context chunk.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ----------------------------------------------------------------------------
# bfloat16 helpers (inputs arrive as raw 16-bit patterns)


def bf16_bits_to_f64(u16) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16 / int16 array) to float64."""
    u = np.asarray(u16).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), as float64.

    bfloat16 keeps 8 significant bits.  Values are assumed finite and inside
    the normal range of bfloat16 (zero is kept exactly).
    """
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x))
    m, e = np.frexp(x)              # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0) / 256.0  # 8 significant bits, ties to even
    return np.ldexp(r, e)


def round_e5m2(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest FP8 E5M2 value (ties to even), as
    float64: 1 sign, 5 exponent bits with bias 15, 2 mantissa bits, so normal
    values keep 3 significant bits from 2^-14 up to 57344, and below 2^-14 the
    values are multiples of 2^-16.  Magnitudes that round past 57344 become inf."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x))
    m, e = np.frexp(x)                                  # x = m * 2^e, 0.5 <= |m| < 1
    normal = np.ldexp(np.rint(m * 8.0) / 8.0, e)        # 3 significant bits
    sub = np.rint(x * 2.0 ** 16) / 2.0 ** 16            # fixed spacing 2^-16
    r = np.where(np.abs(x) >= 2.0 ** -14, normal, sub)
    return np.where(np.abs(r) > 57344.0, np.copysign(np.inf, x), r)


# ----------------------------------------------------------------------------
# RoPE (rotate-half), the positional rotation applied to keys after rebuild


def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    i = np.arange(d // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d)


def apply_rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate the last axis of ``x`` (length d) by position ``pos`` (broadcast over
    the second-to-last axis): pairs (i, i + d/2) turn by pos * theta^(-2i/d)."""
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ----------------------------------------------------------------------------
# Pre-fill pieces (Algorithm 1)


def truncated_svd(kb: np.ndarray, r: int, n_heads: int):
    """Rank-r SVD of one batch element's pre-RoPE keys ``kb`` [S, H*d].

    Returns (A [S, r] = U_r Sigma_r, B [H, r, d] = V_r^T split per head,
    sigma [min(S, H*d)]).  Gauge: every right singular vector has its
    largest-|.| entry positive (first index on ties); U flips with it.
    """
    u, sig, vt = np.linalg.svd(kb, full_matrices=False)
    u, vt = u[:, :r].copy(), vt[:r].copy()
    j = np.argmax(np.abs(vt), axis=1)
    sign = np.where(vt[np.arange(r), j] < 0, -1.0, 1.0)
    vt *= sign[:, None]
    u *= sign[None, :]
    a = u * sig[:r][None, :]
    d = kb.shape[1] // n_heads
    b = vt.reshape(r, n_heads, d).transpose(1, 0, 2).copy()
    return a, b, sig


def landmarks(kr: np.ndarray, c: int) -> np.ndarray:
    """Chunk means of post-RoPE keys: kr [..., S, d] -> [..., S/c, d]."""
    sh = kr.shape
    return kr.reshape(sh[:-2] + (sh[-2] // c, c, sh[-1])).mean(axis=-2)


def chunk_min_cos(kr: np.ndarray, lm: np.ndarray, c: int) -> np.ndarray:
    """For every chunk, the minimum over its keys of cos(key, chunk mean)."""
    sh = kr.shape
    k = kr.reshape(sh[:-2] + (sh[-2] // c, c, sh[-1]))
    dots = np.einsum("...jid,...jd->...ji", k, lm)
    nk = np.linalg.norm(k, axis=-1)
    nl = np.linalg.norm(lm, axis=-1)[..., None]
    cos = dots / np.maximum(nk * nl, 1e-8)
    return cos.min(axis=-1)


def pick_outliers(min_cos: np.ndarray, o: int, n_eligible: int) -> np.ndarray:
    """The o eligible chunks (ids < n_eligible) with the lowest min-cosine;
    ties go to the lower id.  Returned ascending."""
    ids = np.arange(n_eligible)
    order = np.lexsort((ids, min_cos[:n_eligible]))
    return np.sort(order[:o])


def top_k(scores: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest scores; larger score first, then lower id on ties.
    Returned ascending."""
    order = np.lexsort((ids, -scores))
    return np.sort(ids[order[:k]])


# ----------------------------------------------------------------------------
# State and configuration


@dataclasses.dataclass
class Config:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    rank: int
    chunk: int
    top_k: int
    n_outlier: int
    window: int
    rope_theta: float = 500000.0
    landmark_format: str = "bf16"    # storage of the landmarks: "bf16" or "e5m2" (FP8)
    a_format: str = "bf16"           # storage of the rows of A: "bf16" or "e5m2" (FP8)
    b_format: str = "bf16"           # storage of B: "bf16" or "e5m2" (FP8)

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_chunks(self):
        return self.seq_len // self.chunk

    @property
    def n_win_chunks(self):
        return self.window // self.chunk

    @property
    def n_cand(self):
        return self.n_chunks - self.n_outlier - self.n_win_chunks


def config_from(shape) -> Config:
    """Take the ShadowKV fields from any object carrying them."""
    return Config(shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                  shape.seq_len, shape.rank, shape.chunk, shape.top_k, shape.n_outlier,
                  shape.window, shape.rope_theta, getattr(shape, "landmark_format", "bf16"),
                  getattr(shape, "a_format", "bf16"), getattr(shape, "b_format", "bf16"))


@dataclasses.dataclass
class State:
    cfg: Config
    A: np.ndarray            # [b, S, r]
    B: np.ndarray            # [b, H, r, d]
    sigma: np.ndarray        # [b, min(S, H d)] singular values
    L: np.ndarray            # [b, H, n_cand, d] landmarks of candidate chunks
    cand: np.ndarray         # [b, H, n_cand] chunk ids of candidates (ascending)
    outliers: np.ndarray     # [b, H, O] outlier chunk ids (ascending)
    min_cos: np.ndarray      # [b, H, n_c]
    K_out: np.ndarray        # [b, H, O*C, d] post-RoPE keys of outlier chunks
    V_out: np.ndarray        # [b, H, O*C, d]
    K_win: np.ndarray        # [b, H, W, d] post-RoPE keys of the local window
    V_win: np.ndarray        # [b, H, W, d]
    V: np.ndarray            # [b, H, S, d] value store (V_CPU plus the rest)
    storage_rounding: bool = True
    K_new: np.ndarray | None = None   # exact mode: [b, H, T, d] post-RoPE keys of generated tokens
    V_new: np.ndarray | None = None   # exact mode: [b, H, T, d] their values
    n_new: int = 0                    # generated tokens appended so far
    new_mode: str | None = None       # "exact" or "lowrank" once a token is appended

    def keep(self, x):
        return round_bf16(x) if self.storage_rounding else x

    def keep_a(self, x):
        if not self.storage_rounding:
            return x
        return round_e5m2(x) if self.cfg.a_format == "e5m2" else round_bf16(x)

    def keep_landmark(self, x):
        if not self.storage_rounding:
            return x
        return round_e5m2(x) if self.cfg.landmark_format == "e5m2" else round_bf16(x)


def build(cfg: Config, k_pre, v, storage_rounding: bool = True) -> State:
    """Algorithm 1 for every batch element.

    ``k_pre``: [b, S, H*d] pre-RoPE keys, ``v``: [b, H, S, d] values; either raw
    bfloat16 bit patterns (uint16/int16) or float arrays.
    """
    k_pre = _as_f64(k_pre)
    v = _as_f64(v)
    b, S, H, d, C = cfg.batch, cfg.seq_len, cfg.n_kv_heads, cfg.head_dim, cfg.chunk
    assert k_pre.shape == (b, S, H * d) and v.shape == (b, H, S, d)
    assert S % C == 0 and cfg.window % C == 0 and 1 <= cfg.top_k <= cfg.n_cand
    n_c, n_elig = cfg.n_chunks, cfg.n_chunks - cfg.n_win_chunks
    rnd = round_bf16 if storage_rounding else (lambda x: x)
    rnd_l = (round_e5m2 if cfg.landmark_format == "e5m2" else round_bf16) if storage_rounding else (lambda x: x)
    rnd_a = (round_e5m2 if cfg.a_format == "e5m2" else round_bf16) if storage_rounding else (lambda x: x)
    rnd_b = (round_e5m2 if cfg.b_format == "e5m2" else round_bf16) if storage_rounding else (lambda x: x)
    pos = np.arange(S)

    As, Bs, sigs, Ls, cands, outs, mcs, kos, vos, kws, vws = ([] for _ in range(11))
    for bi in range(b):
        a, bm, sig = truncated_svd(k_pre[bi], cfg.rank, H)
        As.append(rnd_a(a)); Bs.append(rnd_b(bm)); sigs.append(sig)
        kr = apply_rope(k_pre[bi].reshape(S, H, d).transpose(1, 0, 2), pos, cfg.rope_theta)
        lm = landmarks(kr, C)                      # [H, n_c, d]
        mc = chunk_min_cos(kr, lm, C)              # [H, n_c]
        o_ids = np.stack([pick_outliers(mc[h], cfg.n_outlier, n_elig) for h in range(H)])
        cand = np.stack([np.setdiff1d(np.arange(n_elig), o_ids[h]) for h in range(H)])
        Ls.append(rnd_l(np.stack([lm[h, cand[h]] for h in range(H)])))
        tok = (o_ids[:, :, None] * C + np.arange(C)).reshape(H, -1)
        kos.append(rnd(np.stack([kr[h, tok[h]] for h in range(H)])))
        vos.append(np.stack([v[bi, h, tok[h]] for h in range(H)]))
        kws.append(rnd(kr[:, S - cfg.window:]))
        vws.append(v[bi, :, S - cfg.window:])
        cands.append(cand); outs.append(o_ids); mcs.append(mc)
    return State(cfg, np.stack(As), np.stack(Bs), np.stack(sigs), np.stack(Ls),
                 np.stack(cands), np.stack(outs), np.stack(mcs), np.stack(kos),
                 np.stack(vos), np.stack(kws), np.stack(vws), v, storage_rounding)


def psi_t(st: State, bi: int) -> np.ndarray:
    """Psi^T of batch element bi as stored: [r, H*d], the heads' B side by side."""
    B = st.B[bi]                                   # [H, r, d]
    return B.transpose(1, 0, 2).reshape(B.shape[1], -1)


def append(st: State, k_new, v_new, lowrank: bool = False) -> None:
    """Add one generated token per batch element (ShadowKV+ when ``lowrank``).

    ``k_new``: [b, H*d] pre-RoPE key (heads concatenated), ``v_new``: [b, H, d];
    bf16 bit patterns or floats.  The token's position is seq_len plus the
    number of tokens appended before it.  A state takes one mode for all its
    appended tokens.
    """
    cfg = st.cfg
    k_new, v_new = _as_f64(k_new), _as_f64(v_new)
    b, H, d, C = cfg.batch, cfg.n_kv_heads, cfg.head_dim, cfg.chunk
    assert k_new.shape == (b, H * d) and v_new.shape == (b, H, d)
    mode = "lowrank" if lowrank else "exact"
    assert st.new_mode in (None, mode), "one mode per state"
    st.new_mode = mode
    t = st.n_new
    pos = np.array([cfg.seq_len + t])
    keys = np.zeros((b, H, 1, d))
    for bi in range(b):
        for h in range(H):
            keys[bi, h] = st.keep(apply_rope(k_new[bi, h * d:(h + 1) * d][None], pos, cfg.rope_theta))
    vals = v_new[:, :, None, :]
    st.n_new += 1
    if not lowrank:
        st.K_new = keys if st.K_new is None else np.concatenate([st.K_new, keys], axis=2)
        st.V_new = vals if st.V_new is None else np.concatenate([st.V_new, vals], axis=2)
        return
    # the low-rank state joins A, the value joins the value store
    a_rows = np.stack([st.keep_a(k_new[bi] @ psi_t(st, bi).T) for bi in range(b)])[:, None]
    st.A = np.concatenate([st.A, a_rows], axis=1)
    st.V = np.concatenate([st.V, vals], axis=2)
    # the exact region grows by the new token; a completed chunk pushes the
    # oldest exact chunk out to the candidates
    st.K_win = np.concatenate([st.K_win, keys], axis=2)
    st.V_win = np.concatenate([st.V_win, vals], axis=2)
    if st.n_new % C == 0:
        lm = st.keep_landmark(st.K_win[:, :, :C].mean(axis=2))    # [b, H, d]
        chunk = (cfg.seq_len - cfg.window) // C + st.n_new // C - 1
        st.L = np.concatenate([st.L, lm[:, :, None]], axis=2)
        st.cand = np.concatenate([st.cand, np.full((b, H, 1), chunk, dtype=st.cand.dtype)], axis=2)
        st.K_win, st.V_win = st.K_win[:, :, C:], st.V_win[:, :, C:]


def _as_f64(x):
    x = np.asarray(x)
    if x.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(x)
    return x.astype(np.float64)


# ----------------------------------------------------------------------------
# Decode step (Algorithm 2)


def chunk_scores(st: State, q: np.ndarray, bi: int, h: int) -> np.ndarray:
    """S2 over the candidate chunks of pair (bi, h): max over the G q-heads of
    softmax_c(q_g . L_c / sqrt(d)).  ``q``: [H_q, d] (one query token, so the
    sum over query tokens is the identity)."""
    cfg = st.cfg
    G = cfg.group
    qg = q[h * G:(h + 1) * G]                       # [G, d]
    logits = qg @ st.L[bi, h].T / math.sqrt(cfg.head_dim)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p.max(axis=0)


def rebuild_keys(st: State, bi: int, h: int, chunk_ids: np.ndarray) -> np.ndarray:
    """RoPE(Gather(A, I) @ B) for the tokens of the given chunks: [n*C, d]."""
    C = st.cfg.chunk
    tok = (chunk_ids[:, None] * C + np.arange(C)).reshape(-1)
    k = st.A[bi, tok] @ st.B[bi, h]
    return st.keep(apply_rope(k, tok, st.cfg.rope_theta))


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Exact softmax(q k^T / sqrt(d)) v; q [G, d], k/v [T, d]."""
    s = q @ k.T / math.sqrt(q.shape[-1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


@dataclasses.dataclass
class StepResult:
    out: np.ndarray          # [b, H_q, d]
    ids: np.ndarray          # [b, H, K] selected chunk ids, ascending
    scores: np.ndarray       # [b, H, n_cand] S2 over candidates
    hits: np.ndarray         # [b, H] |I_t & I_{t-1}| (0 without a previous step)


def pair_output(st: State, q: np.ndarray, bi: int, h: int, sel: np.ndarray) -> np.ndarray:
    """Exact attention of the G query heads of pair (bi, h) over
    [outlier chunks; rebuilt keys of the chunks `sel`; local window; generated
    tokens]; q [H_q, d]."""
    cfg = st.cfg
    G, C = cfg.group, cfg.chunk
    ks = rebuild_keys(st, bi, h, sel)
    tok = (sel[:, None] * C + np.arange(C)).reshape(-1)
    keys = [st.K_out[bi, h], ks, st.K_win[bi, h]]
    vals = [st.V_out[bi, h], st.V[bi, h, tok], st.V_win[bi, h]]
    if st.K_new is not None:
        keys.append(st.K_new[bi, h])
        vals.append(st.V_new[bi, h])
    keys, vals = np.concatenate(keys), np.concatenate(vals)
    return attend(q[h * G:(h + 1) * G], keys, vals)


def decode_step(st: State, q, prev_ids: np.ndarray | None = None) -> StepResult:
    """One decode step for every (batch, KV head) pair.

    ``q``: [b, H_q, d] post-RoPE queries (bf16 bit patterns or floats);
    ``prev_ids``: the previous step's selection [b, H, K] or None.
    """
    cfg = st.cfg
    q = _as_f64(q)
    b, H, G, C, K = cfg.batch, cfg.n_kv_heads, cfg.group, cfg.chunk, cfg.top_k
    out = np.zeros((b, cfg.n_q_heads, cfg.head_dim))
    ids = np.zeros((b, H, K), dtype=np.int64)
    scores = np.zeros((b, H, st.cand.shape[2]))
    hits = np.zeros((b, H), dtype=np.int64)
    for bi in range(b):
        for h in range(H):
            s2 = chunk_scores(st, q[bi], bi, h)
            sel = top_k(s2, st.cand[bi, h], K)
            scores[bi, h], ids[bi, h] = s2, sel
            if prev_ids is not None:
                hits[bi, h] = len(np.intersect1d(sel, prev_ids[bi, h]))
            out[bi, h * G:(h + 1) * G] = pair_output(st, q[bi], bi, h, sel)
    return StepResult(out, ids, scores, hits)


# ----------------------------------------------------------------------------
# The pages' closed-form performance models


def equivalent_bandwidth(S, C, K, O, alpha, b_gpu, b_pcie):
    """Theoretical equivalent bandwidth 2 S B_gpu / (S/C + 2(K+O)C +
    (1-alpha) K C B_gpu / B_pcie), in the unit of b_gpu."""
    return 2.0 * S * b_gpu / (S / C + 2.0 * (K + O) * C + (1.0 - alpha) * K * C * b_gpu / b_pcie)


def memory_savings(S, M, C, K, O, r):
    """GPU memory savings 2 S M / (S M / C + 2 (K+O) C + S r + r M), as printed."""
    return 2.0 * S * M / (S * M / C + 2.0 * (K + O) * C + S * r + r * M)


def subspace_similarity(psi1: np.ndarray, psi2: np.ndarray) -> float:
    """D(H1, H2) = <H1, H2>_F / r for H_i = Psi_i Psi_i^T (orthonormal columns)."""
    r = psi1.shape[1]
    return float(np.sum((psi1 @ psi1.T) * (psi2 @ psi2.T)) / r)
