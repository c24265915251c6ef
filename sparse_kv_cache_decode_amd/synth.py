"""Seeded synthetic inputs for the ShadowKV decode step.

This module only *draws* inputs: it holds no step of ShadowKV (no SVD, no
landmarks, no outlier test, no scoring, no selection, no attention).  The same
bits it produces feed both the GPU library and the CPU oracle.

Recipe (per layer l and batch element b, each with its own counter-free
``numpy.random.SeedSequence(seed, spawn_key=(l, b, 0))`` stream on the CPU, or
a ``torch.Generator`` seeded from the same triple on the GPU):

* ``A_gen[S, R]``: every column an AR(1) process across tokens,
  ``a_0 ~ N(0,1)``, ``a_t = rho*a_{t-1} + sqrt(1-rho^2)*eps_t`` (unit variance).
* ``B_gen[R, H_kv*d] ~ N(0, 1/R)``.
* pre-RoPE keys ``k_pre[b] = A_gen @ B_gen + noise*N(0,1)``, rows = token
  positions 0..S-1, heads concatenated along columns.
* values ``v[b, h, t, :] ~ N(0,1)``.
* queries (stream ``(l, b, 1)``): for each q-head a fresh draw
  ``z + 4*k_post[j]``, with ``z ~ N(0,1)^d`` and ``j ~ U{0..S-1}`` an
  independent needle position, ``k_post[j]`` the key of the matching KV head
  rotated to position ``j``.  Successive decode steps drift as AR(1):
  ``q_t = 0.9*q_{t-1} + sqrt(0.19)*fresh_t``; the "independent" mode draws
  every step afresh.
* generated tokens (stream ``(l, b, 2)``, ``continuation_*``): the context's
  latent process carried on, ``a_{S+t} = rho*a_{S+t-1} + sqrt(1-rho^2)*eps``,
  the key ``a_{S+t} @ B_gen + noise*N(0,1)`` with the context's ``B_gen`` (so
  new keys share the context's low-rank subspace), the value ``N(0,1)``.
  ``queries_new_np`` (stream ``(l, b, 3)``) aims every q-head of a step at one
  of the tokens generated so far instead (``j ~ U{0..n-1}`` at position S+j),
  each step drawn afresh.

Every tensor is rounded once to bfloat16 (round-to-nearest-even) and returned
as ``torch.bfloat16``.  The rotation used to aim the queries is the synthetic
model's own positional encoding (rotate-half, angles in float64); it shapes the
query distribution only and is written here independently of the library and
of the oracle.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Shape:
    """One workload: model shape plus ShadowKV budget."""

    name: str
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
    latent_rank: int
    layers: int = 1
    steps: int = 1
    rope_theta: float = 500000.0
    rho: float = 0.95
    noise: float = 0.05
    landmark_format: str = "bf16"   # landmark storage: "bf16" or "e5m2" (FP8)
    a_format: str = "bf16"          # storage of the rows of A: "bf16" or "e5m2" (FP8)
    b_format: str = "bf16"          # storage of B: "bf16" or "e5m2" (FP8)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_chunks(self) -> int:
        return self.seq_len // self.chunk

    @property
    def n_cand(self) -> int:
        return self.n_chunks - self.n_outlier - self.window // self.chunk

    @property
    def pairs(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def tokens_attended(self) -> int:
        return (self.top_k + self.n_outlier) * self.chunk + self.window

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


def budget(seq_len: int, chunk: int) -> tuple[int, int]:
    """Sparse budget of 1/64 of the tokens (1.56 %) and 0.3 % outlier chunks."""
    n_c = seq_len // chunk
    return seq_len // (64 * chunk), int(math.floor(0.003 * n_c + 0.5))


def _shape(name, batch, hq, hkv, seq, rank, chunk, latent, layers, steps):
    k, o = budget(seq, chunk)
    return Shape(name, batch, hq, hkv, 128, seq, rank, chunk, k, o, 32, latent,
                 layers=layers, steps=steps)


SHAPES = {
    # single layer, batch 1, 8K tokens: the small case the oracle finishes in seconds
    "tiny_8k": _shape("tiny_8k", 1, 32, 8, 8192, 160, 8, 160, 1, 1),
    # Llama-3.1-8B shape at 122 880 tokens, batch 8, 32 layers, 64 drifting steps
    "llama3_8b_122k": _shape("llama3_8b_122k", 8, 32, 8, 122880, 160, 8, 160, 32, 64),
    # Yi-9B-200K shape
    "yi_9b_200k": _shape("yi_9b_200k", 8, 32, 4, 204800, 96, 8, 96, 48, 64),
    # GLM-4-9B-1M shape
    "glm4_9b_1m": _shape("glm4_9b_1m", 4, 32, 2, 1048576, 48, 8, 48, 40, 64),
}
assert SHAPES["tiny_8k"].top_k == 16 and SHAPES["tiny_8k"].n_outlier == 3
assert SHAPES["llama3_8b_122k"].top_k == 240 and SHAPES["llama3_8b_122k"].n_outlier == 46


def glm_chunk_variant(chunk: int) -> Shape:
    s = SHAPES["glm4_9b_1m"]
    k, o = budget(s.seq_len, chunk)
    return s.replace(name=f"glm4_9b_1m_c{chunk}", chunk=chunk, top_k=k, n_outlier=o)


# ----------------------------------------------------------------------------
# CPU (numpy) generator


def _rng(seed: int, layer: int, b: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(seed, spawn_key=(layer, b, stream))))


def _ar1_np(eps: np.ndarray, rho: float) -> np.ndarray:
    """AR(1) along axis 0 with a_0 = eps_0 (unit-variance stationary start)."""
    from scipy.signal import lfilter
    c = math.sqrt(1.0 - rho * rho)
    x = eps.copy()
    x[0] /= c
    return lfilter([c], [1.0, -rho], x, axis=0)


def _to_bf16(x) -> torch.Tensor:
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(torch.float32).to(torch.bfloat16)


def _rotate_np(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Synthetic model's rotate-half positional rotation, float64 complex form."""
    d = x.shape[-1]
    h = d // 2
    freq = np.exp(-(2.0 * np.arange(h) / d) * math.log(theta))
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * (pos[..., None] * freq))
    return np.concatenate([z.real, z.imag], axis=-1)


def layer_cache_np(s: Shape, layer: int, seed: int = 0):
    """Return (k_pre bf16 [b][S][H_kv*d], v bf16 [b][H_kv][S][d]) on the CPU."""
    hd = s.n_kv_heads * s.head_dim
    ks, vs = [], []
    for b in range(s.batch):
        g = _rng(seed, layer, b, 0)
        a = _ar1_np(g.standard_normal((s.seq_len, s.latent_rank)), s.rho)
        bm = g.standard_normal((s.latent_rank, hd)) / math.sqrt(s.latent_rank)
        k = a @ bm + s.noise * g.standard_normal((s.seq_len, hd))
        v = g.standard_normal((s.n_kv_heads, s.seq_len, s.head_dim))
        ks.append(_to_bf16(k))
        vs.append(_to_bf16(v))
    return torch.stack(ks), torch.stack(vs)


def continuation_np(s: Shape, layer: int, n_tokens: int, seed: int = 0):
    """Generated tokens after the context of ``layer_cache_np(s, layer, seed)``:
    (k_new bf16 [n][b][H_kv*d], v_new bf16 [n][b][H_kv][d])."""
    hd = s.n_kv_heads * s.head_dim
    k_new = np.zeros((n_tokens, s.batch, hd))
    v_new = np.zeros((n_tokens, s.batch, s.n_kv_heads, s.head_dim))
    c = math.sqrt(1.0 - s.rho * s.rho)
    for b in range(s.batch):
        g = _rng(seed, layer, b, 0)                   # the context's draws, in order
        a = _ar1_np(g.standard_normal((s.seq_len, s.latent_rank)), s.rho)[-1]
        bm = g.standard_normal((s.latent_rank, hd)) / math.sqrt(s.latent_rank)
        g2 = _rng(seed, layer, b, 2)
        for t in range(n_tokens):
            a = s.rho * a + c * g2.standard_normal(s.latent_rank)
            k_new[t, b] = a @ bm + s.noise * g2.standard_normal(hd)
            v_new[t, b] = g2.standard_normal((s.n_kv_heads, s.head_dim))
    return _to_bf16(k_new), _to_bf16(v_new)


def queries_np(s: Shape, k_pre: torch.Tensor, layer: int, steps: int, seed: int = 0,
               mode: str = "drift") -> torch.Tensor:
    """Queries bf16 [steps][b][H_q][d] aimed at random keys (see module doc)."""
    d, G = s.head_dim, s.group
    out = np.zeros((steps, s.batch, s.n_q_heads, d))
    for b in range(s.batch):
        g = _rng(seed, layer, b, 1)
        kb = k_pre[b].to(torch.float64).numpy().reshape(s.seq_len, s.n_kv_heads, d)
        prev = None
        for t in range(steps):
            pos = g.integers(0, s.seq_len, size=s.n_q_heads)
            z = g.standard_normal((s.n_q_heads, d))
            heads = np.arange(s.n_q_heads) // G
            needle = _rotate_np(kb[pos, heads], pos.astype(np.float64), s.rope_theta)
            fresh = z + 4.0 * needle
            if prev is None or mode == "independent":
                q = fresh
            else:
                q = 0.9 * prev + math.sqrt(0.19) * fresh
            out[t, b] = q
            prev = q
    return _to_bf16(out)


def queries_new_np(s: Shape, k_new: torch.Tensor, n_avail: list, layer: int = 0,
                   seed: int = 0) -> torch.Tensor:
    """Queries bf16 [len(n_avail)][b][H_q][d] aimed at generated tokens: step t
    picks its needles among the first n_avail[t] > 0 rows of k_new [n][b][H_kv*d]."""
    d, G = s.head_dim, s.group
    out = np.zeros((len(n_avail), s.batch, s.n_q_heads, d))
    heads = np.arange(s.n_q_heads) // G
    for b in range(s.batch):
        g = _rng(seed, layer, b, 3)
        kb = k_new[:, b].to(torch.float64).numpy().reshape(-1, s.n_kv_heads, d)
        for t, n in enumerate(n_avail):
            j = g.integers(0, n, size=s.n_q_heads)
            z = g.standard_normal((s.n_q_heads, d))
            pos = (s.seq_len + j).astype(np.float64)
            out[t, b] = z + 4.0 * _rotate_np(kb[j, heads], pos, s.rope_theta)
    return _to_bf16(out)


# ----------------------------------------------------------------------------
# GPU (torch) generator: same recipe, torch's Philox streams, for full sizes


def _tgen(seed: int, layer: int, b: int, stream: int, device) -> torch.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(layer, b, stream))
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return g


def _ar1_torch(eps: torch.Tensor, rho: float) -> torch.Tensor:
    """AR(1) along dim 0 by a doubling scan (float64): y_t = sum_s rho^s e_{t-s}."""
    c = math.sqrt(1.0 - rho * rho)
    y = eps * c
    y[0] = eps[0]
    n = y.shape[0]
    off, coef = 1, rho
    while off < n:
        nxt = y.clone()
        nxt[off:] += coef * y[:-off]
        y = nxt
        off *= 2
        coef = coef * coef
    return y


def layer_cache_torch(s: Shape, layer: int, seed: int = 0, device="cuda",
                      value_out: torch.Tensor | None = None):
    """Same recipe drawn on ``device``; returns (k_pre, v) bf16 tensors there.

    ``value_out`` (bf16 [b][H_kv][S][d], any device, e.g. pinned host) receives
    the values instead of a new device tensor when given.
    """
    hd = s.n_kv_heads * s.head_dim
    k_pre = torch.empty((s.batch, s.seq_len, hd), dtype=torch.bfloat16, device=device)
    v = value_out if value_out is not None else torch.empty(
        (s.batch, s.n_kv_heads, s.seq_len, s.head_dim), dtype=torch.bfloat16, device=device)
    for b in range(s.batch):
        g = _tgen(seed, layer, b, 0, device)
        eps = torch.randn((s.seq_len, s.latent_rank), generator=g, device=device,
                          dtype=torch.float64)
        a = _ar1_torch(eps, s.rho).to(torch.float32)
        del eps
        bm = torch.randn((s.latent_rank, hd), generator=g, device=device) / math.sqrt(s.latent_rank)
        k = torch.randn((s.seq_len, hd), generator=g, device=device)
        k.mul_(s.noise).add_(a @ bm)
        k_pre[b].copy_(k.to(torch.bfloat16))
        del a, k
        for h in range(s.n_kv_heads):
            vh = torch.randn((s.seq_len, s.head_dim), generator=g, device=device)
            v[b, h].copy_(vh.to(torch.bfloat16))
    return k_pre, v


def continuation_torch(s: Shape, layer: int, n_tokens: int, seed: int = 0, device="cuda"):
    """Generated tokens after the context of ``layer_cache_torch(s, layer, seed)``,
    drawn on ``device``: (k_new bf16 [n][b][H_kv*d], v_new bf16 [n][b][H_kv][d])."""
    hd = s.n_kv_heads * s.head_dim
    k_new = torch.empty((n_tokens, s.batch, hd), dtype=torch.bfloat16, device=device)
    v_new = torch.empty((n_tokens, s.batch, s.n_kv_heads, s.head_dim), dtype=torch.bfloat16,
                        device=device)
    c = math.sqrt(1.0 - s.rho * s.rho)
    for b in range(s.batch):
        g = _tgen(seed, layer, b, 0, device)          # the context's draws, in order
        eps = torch.randn((s.seq_len, s.latent_rank), generator=g, device=device,
                          dtype=torch.float64)
        a = _ar1_torch(eps, s.rho)[-1]
        del eps
        bm = torch.randn((s.latent_rank, hd), generator=g, device=device) / math.sqrt(s.latent_rank)
        g2 = _tgen(seed, layer, b, 2, device)
        for t in range(n_tokens):
            a = s.rho * a + c * torch.randn(s.latent_rank, generator=g2, device=device,
                                            dtype=torch.float64)
            k = a.to(torch.float32) @ bm + s.noise * torch.randn(hd, generator=g2, device=device)
            k_new[t, b] = k.to(torch.bfloat16)
            v_new[t, b] = torch.randn((s.n_kv_heads, s.head_dim), generator=g2,
                                      device=device).to(torch.bfloat16)
    return k_new, v_new


def _rotate_torch(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    d = x.shape[-1]
    h = d // 2
    freq = torch.exp(-(2.0 * torch.arange(h, device=x.device, dtype=torch.float64) / d)
                     * math.log(theta))
    ang = pos.to(torch.float64)[..., None] * freq
    re, im = x[..., :h], x[..., h:]
    c, sn = torch.cos(ang), torch.sin(ang)
    return torch.cat([re * c - im * sn, re * sn + im * c], dim=-1)


def queries_torch(s: Shape, k_pre: torch.Tensor, layer: int, steps: int, seed: int = 0,
                  mode: str = "drift") -> torch.Tensor:
    """Queries bf16 [steps][b][H_q][d] on k_pre's device (see module doc)."""
    dev = k_pre.device
    d, G = s.head_dim, s.group
    out = torch.empty((steps, s.batch, s.n_q_heads, d), dtype=torch.bfloat16, device=dev)
    heads = torch.arange(s.n_q_heads, device=dev) // G
    for b in range(s.batch):
        g = _tgen(seed, layer, b, 1, dev)
        kb = k_pre[b].view(s.seq_len, s.n_kv_heads, d)
        prev = None
        for t in range(steps):
            pos = torch.randint(0, s.seq_len, (s.n_q_heads,), generator=g, device=dev)
            z = torch.randn((s.n_q_heads, d), generator=g, device=dev, dtype=torch.float64)
            needle = _rotate_torch(kb[pos, heads].to(torch.float64), pos, s.rope_theta)
            fresh = z + 4.0 * needle
            q = fresh if (prev is None or mode == "independent") else \
                0.9 * prev + math.sqrt(0.19) * fresh
            out[t, b] = q.to(torch.float32).to(torch.bfloat16)
            prev = q
    return out
