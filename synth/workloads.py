"""Synthetic shared-context KV caches, planted low-rank deltas and online anchors.

The workloads stand in for the caches that the KVCMAS pages measure on (Llama-3.1-8B-,
Qwen2.5-Coder-7B- and LLaVA-OneVision-7B-shaped models, shared contexts of 2K-32K tokens;
"KVCMAS", thelatestinai listing, Table 4 and the Fig. 5 / Table 9 captions).  No dataset
item and no trained weight is used: every tensor is drawn here from a seeded torch
generator, on the device the caller names.

Recipe (one shared-context segment = one (layer, kv-head) pair, K and V drawn separately):

* base cache R ~ N(0, 1) per entry, ``outliers`` channels per segment multiplied by
  ``outlier_gain``; tokens in ``visual`` get variance ``visual_var``; stored in the
  cache dtype (bf16 round-to-nearest-even, or fp32);
* planted delta D = U_o diag(sigma) V_o^T + N(0, noise^2), with U_o (T x r) and V_o
  (d x r) orthonormal (QR of Gaussians, signs fixed by diag(R) > 0) and
  sigma_i = scale0 * decay^i * ||R||_F, so sigma_i / sqrt(T d) is the per-entry scale;
* exact cache of the next agent E' = dtype(E + D), so for the first edge E = R;
* anchor 0 carries the planted factors (U_o diag(sigma), V_o^T); further anchors keep
  V_o^T and perturb U_o by a Gaussian of relative size 1/3 ("cosine" mode), or carry an
  independent planted delta ("query_noise" mode, the tiny case);
* descriptor targets: per segment a cosine c_a for every anchor and a random direction;
  ``build_descriptors`` turns a pooled query vector q (computed by whoever consumes the
  case) into anchor descriptors with exactly those cosines.  With probability
  ``fallback_prob`` every c_a < tau - guard, otherwise c_0 > tau + guard, which keeps
  a +-guard band around the reliability threshold.

This module holds no step of the correction or of the anchor fit.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = [
    "Config",
    "CONFIGS",
    "Edge",
    "Case",
    "generate",
    "generate_fanout",
    "generate_pool",
    "pool_descriptors",
    "build_descriptors",
    "fit_input",
    "planted_spectrum",
    "to_f64",
]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    L: int
    H: int
    T: int
    d: int
    dtype: str  # "bf16" | "f32"
    A: int
    r: int
    tau: float
    scale0: float = 0.3
    decay: float = 0.9
    noise: float = 1e-3
    outliers: int = 0
    outlier_gain: float = 8.0
    visual: Optional[tuple] = None  # (first, stop) token range
    visual_var: float = 2.0
    desc_mode: str = "cosine"  # "cosine" | "query_noise"
    desc_noise: float = 0.05
    fallback_prob: float = 0.2
    guard: float = 0.02
    n_edges: int = 1
    fit: bool = False
    seed: int = 0

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    @property
    def S(self) -> int:
        return self.L * self.H


CONFIGS = {
    # 1 layer x 1 kv-head, head_dim 64, 256 shared tokens, fp32, two anchors of rank 8,
    # per-entry delta scale 0.3 * 0.8^i, noise 1e-4, query = anchor-0 descriptor + N(0, 0.05).
    "tiny": Config("tiny", 1, 1, 256, 64, "f32", A=2, r=8, tau=0.3, decay=0.8, noise=1e-4,
                   desc_mode="query_noise", fit=True, seed=0),
    # Llama-3.1-8B KV shape (32 layers x 8 kv-heads x 128), 2048 shared tokens.
    "llama8b_t2048": Config("llama8b_t2048", 32, 8, 2048, 128, "bf16", A=4, r=32, tau=0.32,
                            outliers=4, seed=1),
    # Same shape at 8192 tokens, with the anchor fit of exact - reused.
    "llama8b_t8192_fit": Config("llama8b_t8192_fit", 32, 8, 8192, 128, "bf16", A=4, r=32,
                                tau=0.32, outliers=4, fit=True, seed=2),
    # Chained workflow A0 -> A1 -> A2 -> A3 at 32768 tokens; A0's cache is exact.
    "chain_t32768": Config("chain_t32768", 32, 8, 32768, 128, "bf16", A=4, r=32, tau=0.32,
                           outliers=4, n_edges=3, seed=3),
    # Vision-language shape (28 layers x 4 kv-heads x 128), 9216 tokens of which 7000
    # "visual" tokens have twice the variance of the text tokens.
    "vl_t9216": Config("vl_t9216", 28, 4, 9216, 128, "bf16", A=6, r=32, tau=0.6,
                       visual=(1024, 8024), fit=True, seed=4),
}


@dataclasses.dataclass
class Edge:
    """One workflow edge i -> i+1: the anchors of its segments and agent i+1's exact cache."""

    U: torch.Tensor  # [2, L, H, A, T, r] cache dtype (index 0 = K, 1 = V)
    W: torch.Tensor  # [2, L, H, A, r, d] cache dtype
    exact_K: torch.Tensor  # [L, H, T, d] cache dtype
    exact_V: torch.Tensor
    sigma: torch.Tensor  # [2, L, H, r] float64, planted singular values
    cos_target: Optional[torch.Tensor] = None  # [L, H, A] float64 ("cosine" mode)
    direction: Optional[torch.Tensor] = None  # [L, H, A, 2d] float64 ("cosine" mode)
    query_noise: Optional[torch.Tensor] = None  # [L, H, 2d] float64 ("query_noise" mode)
    other_desc: Optional[torch.Tensor] = None  # [L, H, A-1, 2d] float64 ("query_noise" mode)


@dataclasses.dataclass
class Case:
    cfg: Config
    K0: torch.Tensor  # [L, H, T, d] source cache of edge 0 (agent A0's exact cache)
    V0: torch.Tensor
    edges: list

    @property
    def device(self) -> torch.device:
        return self.K0.device


def _seed(*parts: int) -> int:
    return int(np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts]).generate_state(1)[0])


def _gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


# stream ids (kept stable so that a case can be regenerated stream by stream)
_S_BASE, _S_OUTLIER, _S_UO, _S_VO, _S_NOISE, _S_ANCHOR, _S_COS, _S_DIR, _S_QNOISE, _S_OTHER, \
    _S_MASKED = range(11)


def _orthonormal(shape_batch, n, k, g, device) -> torch.Tensor:
    """[..., n, k] float64 with orthonormal columns: the Q factor (diag(R) > 0) of a Gaussian,
    formed by Gram-Schmidt with one re-orthogonalisation pass (plain tensor arithmetic, so the
    generator needs no dense solver library on the device).

    When n < k only n columns can be orthonormal; the remaining k - n columns are zero.
    """
    x = torch.randn(*shape_batch, n, k, generator=g, device=device, dtype=torch.float64)
    m = min(n, k)
    q = torch.zeros(*shape_batch, n, k, dtype=torch.float64, device=device)
    for j in range(m):
        v = x[..., :, j]
        if j > 0:
            prev = q[..., :, :j]
            for _ in range(2):
                c = (prev * v.unsqueeze(-1)).sum(-2)
                v = v - (prev * c.unsqueeze(-2)).sum(-1)
        q[..., :, j] = v / torch.linalg.vector_norm(v, dim=-1, keepdim=True)
    return q


def planted_spectrum(cfg: Config, base_norm) -> torch.Tensor:
    """sigma_i = scale0 * decay^i * ||base||_F for i < r (last axis)."""
    base_norm = torch.as_tensor(base_norm, dtype=torch.float64)
    i = torch.arange(cfg.r, dtype=torch.float64, device=base_norm.device)
    return cfg.scale0 * (cfg.decay ** i) * base_norm.unsqueeze(-1)


def _base_cache(cfg: Config, which: int, device) -> torch.Tensor:
    L, H, T, d = cfg.L, cfg.H, cfg.T, cfg.d
    g = _gen(device, cfg.seed, _S_BASE, which)
    x = torch.randn(L, H, T, d, generator=g, device=device, dtype=torch.float32)
    if cfg.outliers > 0:
        go = _gen(device, cfg.seed, _S_OUTLIER, which)
        keys = torch.rand(L, H, d, generator=go, device=device)
        idx = torch.argsort(keys, dim=-1)[..., : cfg.outliers]  # [L, H, n_out]
        gain = torch.ones(L, H, d, device=device, dtype=torch.float32)
        gain.scatter_(-1, idx, cfg.outlier_gain)
        x = x * gain.unsqueeze(2)
    if cfg.visual is not None:
        a, b = cfg.visual
        x[:, :, a:b, :] *= math.sqrt(cfg.visual_var)
    return x.to(cfg.torch_dtype)


def _frob(x: torch.Tensor) -> torch.Tensor:
    """Frobenius norm of every [T, d] segment, float64, shape [L, H]."""
    return torch.linalg.vector_norm(x.to(torch.float64), dim=(-2, -1))


def _edge(cfg: Config, e: int, srcK: torch.Tensor, srcV: torch.Tensor, device) -> Edge:
    L, H, T, d, A, r = cfg.L, cfg.H, cfg.T, cfg.d, cfg.A, cfg.r
    dt = cfg.torch_dtype
    U = torch.empty(2, L, H, A, T, r, dtype=dt, device=device)
    W = torch.empty(2, L, H, A, r, d, dtype=dt, device=device)
    sig_all = torch.empty(2, L, H, r, dtype=torch.float64, device=device)
    exact = []
    for which, src in enumerate((srcK, srcV)):
        uo = _orthonormal((L, H), T, r, _gen(device, cfg.seed, _S_UO, e, which), device)
        vo = _orthonormal((L, H), d, r, _gen(device, cfg.seed, _S_VO, e, which), device)
        sig = planted_spectrum(cfg, _frob(src))  # [L, H, r]
        sig_all[which] = sig
        us = uo * sig.unsqueeze(-2)  # U_o diag(sigma)
        D = torch.matmul(us, vo.transpose(-1, -2))  # [L, H, T, d] float64
        gn = _gen(device, cfg.seed, _S_NOISE, e, which)
        D += cfg.noise * torch.randn(L, H, T, d, generator=gn, device=device, dtype=torch.float64)
        exact.append((src.to(torch.float64) + D).to(dt))
        del D
        U[which, :, :, 0] = us.to(dt)
        W[which, :, :, 0] = vo.transpose(-1, -2).to(dt)
        ga = _gen(device, cfg.seed, _S_ANCHOR, e, which)
        for a in range(1, A):
            if cfg.desc_mode == "query_noise":
                uo2 = _orthonormal((L, H), T, r, ga, device)
                vo2 = _orthonormal((L, H), d, r, ga, device)
                U[which, :, :, a] = (uo2 * sig.unsqueeze(-2)).to(dt)
                W[which, :, :, a] = vo2.transpose(-1, -2).to(dt)
            else:
                pert = torch.randn(L, H, T, r, generator=ga, device=device, dtype=torch.float64)
                ua = (uo + pert / (3.0 * math.sqrt(T))) * sig.unsqueeze(-2)
                U[which, :, :, a] = ua.to(dt)
                W[which, :, :, a] = vo.transpose(-1, -2).to(dt)
    edge = Edge(U=U, W=W, exact_K=exact[0], exact_V=exact[1], sigma=sig_all)
    if cfg.desc_mode == "query_noise":
        gq = _gen(device, cfg.seed, _S_QNOISE, e)
        edge.query_noise = cfg.desc_noise * torch.randn(L, H, 2 * d, generator=gq, device=device,
                                                        dtype=torch.float64)
        go = _gen(device, cfg.seed, _S_OTHER, e)
        edge.other_desc = torch.randn(L, H, A - 1, 2 * d, generator=go, device=device,
                                      dtype=torch.float64) / math.sqrt(T)
    else:
        gc = _gen(device, cfg.seed, _S_COS, e)
        lo, tau, gd = -0.2, cfg.tau, cfg.guard
        u = torch.rand(L, H, A, generator=gc, device=device, dtype=torch.float64)
        masked = torch.rand(L, H, generator=_gen(device, cfg.seed, _S_MASKED, e), device=device,
                            dtype=torch.float64) < cfg.fallback_prob
        c_masked = lo + u * ((tau - gd) - lo)
        c_other = lo + u * (1.0 - lo)
        c_first = (tau + gd) + u[..., :1] * (1.0 - (tau + gd))
        c_keep = torch.cat([c_first, c_other[..., 1:]], dim=-1)
        edge.cos_target = torch.where(masked.unsqueeze(-1), c_masked, c_keep).clamp(-1.0, 1.0)
        edge.direction = torch.randn(L, H, A, 2 * d, generator=_gen(device, cfg.seed, _S_DIR, e),
                                     device=device, dtype=torch.float64)
    return edge


def generate(cfg: Config | str, device="cpu") -> Case:
    """Draw a whole case (all edges) on ``device``; deterministic for a given config."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    device = torch.device(device)
    K0 = _base_cache(cfg, 0, device)
    V0 = _base_cache(cfg, 1, device)
    edges = []
    srcK, srcV = K0, V0
    for e in range(cfg.n_edges):
        ed = _edge(cfg, e, srcK, srcV, device)
        edges.append(ed)
        srcK, srcV = ed.exact_K, ed.exact_V
    return Case(cfg=cfg, K0=K0, V0=V0, edges=edges)


def generate_fanout(cfg: Config | str, device="cpu") -> Case:
    """Non-chained workload: (K0, V0) is a context-free reference cache of the shared context
    and edge j belongs to agent j, whose exact cache is reference + agent j's own planted
    delta; every edge's source is the reference.  Deterministic for a given config (agent 0's
    delta is the one ``generate`` plants on its first edge)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    device = torch.device(device)
    K0 = _base_cache(cfg, 0, device)
    V0 = _base_cache(cfg, 1, device)
    edges = [_edge(cfg, e, K0, V0, device) for e in range(cfg.n_edges)]
    return Case(cfg=cfg, K0=K0, V0=V0, edges=edges)


_S_POOL_U, _S_POOL_W, _S_POOL_COUNT, _S_POOL_COS, _S_POOL_DIR, _S_POOL_ALLLOW = range(20, 26)


def generate_pool(cfg: Config, Vc: int, device="cpu", full: bool = False) -> dict:
    """Contents of an online anchor pool with ``Vc`` slots per segment (listing Table 13):
    factors U [2, L, H, Vc, T, r] (Gaussian, standard deviation ``scale0``) and W [2, L, H, Vc, r, d] (orthonormal rows), both in the cache dtype;
    count [L, H] int32 valid slots (uniform in 0..Vc, or Vc when ``full``); per-slot target
    cosines [L, H, Vc] drawn without repetition from a grid of step 0.04 (0.02 for pools of more
    than 26 slots) on [-0.2, 1) that skips +-0.02 around tau (with probability ``fallback_prob`` a segment's valid slots all
    lie below tau), so selections and decisions stay away from rounding ties; random
    directions [L, H, Vc, 2d] for ``pool_descriptors``."""
    L, H, T, d, r = cfg.L, cfg.H, cfg.T, cfg.d, cfg.r
    dt = cfg.torch_dtype
    g = _gen(device, cfg.seed, _S_POOL_U)
    U = (cfg.scale0 * torch.randn(2, L, H, Vc, T, r, generator=g, device=device)).to(dt)
    vo = _orthonormal((2, L, H, Vc), d, r, _gen(device, cfg.seed, _S_POOL_W), device)
    W = vo.transpose(-1, -2).to(dt).contiguous()
    if full:
        count = torch.full((L, H), Vc, dtype=torch.int32, device=device)
    else:
        count = torch.randint(0, Vc + 1, (L, H), generator=_gen(device, cfg.seed, _S_POOL_COUNT),
                              device=device, dtype=torch.int32)
    step = 0.04 if Vc <= 26 else 0.02  # enough distinct cosines for every slot
    grid = torch.arange(-0.2, 1.0, step, dtype=torch.float64)
    grid = grid[(grid - cfg.tau).abs() > 0.02]
    low = grid[grid < cfg.tau]
    gc = _gen("cpu", cfg.seed, _S_POOL_COS)
    all_low = torch.rand(L, H, generator=_gen("cpu", cfg.seed, _S_POOL_ALLLOW),
                         dtype=torch.float64) < cfg.fallback_prob
    cos = torch.empty(L, H, Vc, dtype=torch.float64)
    for l in range(L):
        for h in range(H):
            src = low if (all_low[l, h] and Vc <= low.numel()) else grid
            cos[l, h] = src[torch.randperm(src.numel(), generator=gc)[:Vc]]
    direction = torch.randn(L, H, Vc, 2 * d, generator=_gen(device, cfg.seed, _S_POOL_DIR),
                            device=device, dtype=torch.float64)
    return {"U": U, "W": W, "count": count, "cos": cos.to(device), "direction": direction}


def pool_descriptors(pool: dict, q) -> torch.Tensor:
    """Descriptors [L, H, Vc, 2d] float32 with cos(q, desc_v) = the pool's target cosines, built
    as in ``build_descriptors`` for a pooled query ``q`` [L, H, 2d] supplied by the consumer."""
    e = pool["direction"]
    dev = e.device
    q = torch.as_tensor(np.asarray(q) if not isinstance(q, torch.Tensor) else q)
    q = q.to(device=dev, dtype=torch.float64)
    qn = torch.linalg.vector_norm(q, dim=-1, keepdim=True)
    safe = torch.where(qn > 0, qn, torch.ones_like(qn))
    qh = (q / safe).unsqueeze(2)
    e = e - (e * qh).sum(-1, keepdim=True) * qh
    e = e / torch.linalg.vector_norm(e, dim=-1, keepdim=True)
    c = pool["cos"].unsqueeze(-1)
    desc = qn.unsqueeze(2) * (c * qh + torch.sqrt(torch.clamp(1.0 - c * c, min=0.0)) * e)
    desc = torch.where(qn.unsqueeze(2) > 0, desc, pool["direction"])
    return desc.to(torch.float32)


def build_descriptors(case: Case, edge: int, q) -> torch.Tensor:
    """Anchor descriptors [L, H, A, 2d] float32 for a pooled query ``q`` [L, H, 2d].

    ``q`` is supplied by the consumer of the case (the oracle in tests).  In "cosine"
    mode descriptor a is ||q|| (c_a q^ + sqrt(1 - c_a^2) e_a), with e_a the unit part of
    a random direction orthogonal to q^, so cos(q, desc_a) = c_a.  In "query_noise" mode
    anchor 0's descriptor is q minus N(0, desc_noise^2) noise (the query is that
    descriptor plus noise) and the other anchors get independent random vectors.
    """
    cfg = case.cfg
    ed = case.edges[edge]
    dev = case.device
    q = torch.as_tensor(np.asarray(q) if not isinstance(q, torch.Tensor) else q)
    q = q.to(device=dev, dtype=torch.float64).reshape(cfg.L, cfg.H, 2 * cfg.d)
    if cfg.desc_mode == "query_noise":
        d0 = (q - ed.query_noise).unsqueeze(2)
        return torch.cat([d0, ed.other_desc], dim=2).to(torch.float32)
    qn = torch.linalg.vector_norm(q, dim=-1, keepdim=True)
    safe = torch.where(qn > 0, qn, torch.ones_like(qn))
    qh = (q / safe).unsqueeze(2)  # [L, H, 1, 2d]
    e = ed.direction
    e = e - (e * qh).sum(-1, keepdim=True) * qh
    e = e / torch.linalg.vector_norm(e, dim=-1, keepdim=True)
    c = ed.cos_target.unsqueeze(-1)
    desc = qn.unsqueeze(2) * (c * qh + torch.sqrt(torch.clamp(1.0 - c * c, min=0.0)) * e)
    desc = torch.where(qn.unsqueeze(2) > 0, desc, ed.direction)
    return desc.to(torch.float32)


def fit_input(case: Case, edge: int = 0) -> torch.Tensor:
    """Delta = exact - reused for every (K|V, layer, head): [2*L*H, T, d] in the cache dtype.

    The difference is taken in float64 and stored once in the cache dtype
    (round-to-nearest-even), as a caller would store it before handing it to the fit.
    """
    cfg = case.cfg
    if edge == 0:
        srcK, srcV = case.K0, case.V0
    else:
        srcK, srcV = case.edges[edge - 1].exact_K, case.edges[edge - 1].exact_V
    ed = case.edges[edge]
    out = torch.empty(2, cfg.L, cfg.H, cfg.T, cfg.d, dtype=cfg.torch_dtype, device=case.device)
    out[0] = (ed.exact_K.to(torch.float64) - srcK.to(torch.float64)).to(cfg.torch_dtype)
    out[1] = (ed.exact_V.to(torch.float64) - srcV.to(torch.float64)).to(cfg.torch_dtype)
    return out.reshape(2 * cfg.L * cfg.H, cfg.T, cfg.d)


def to_f64(x: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 / fp32 tensor to a float64 numpy array on the host."""
    return x.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)
