"""Seeded synthetic workloads for retrieval-based sparse-attention decode.

This module only draws random inputs of the shapes and distributions the
workloads call for. It holds none of the method's arithmetic: no scoring, no
selection, no attention and no cache policy. Both the HIP path (through the
Python binding) and the CPU oracle consume what it produces.

Every tensor is drawn by torch from its own generator, seeded from
(workload seed, tensor tag), so the same seed gives the same bytes on the
same device type. CPU and GPU generators differ, so a test draws on one device
and hands copies to the other side.

The five workloads:

  0  tiny inverted-index case: 1 head, d=128, fp32, N=4096 keys from a
     mixture of C=64 Gaussians (centres N(0,1), within-cluster sd 0.3),
     values N(0,1), query = one centre + N(0, 0.3^2) noise, top-4 lists.
  1  the KARAT worked-example shape (paper-daily digest "Heterogeneous LLM
     Serving with General-Purpose Processing-Near-Memory for Retrieval-Based
     Sparse Attention", worked example): 1 request, 100,000 tokens, 8 KV heads
     and 32 query heads, d=128, bf16, C=1000 centres per KV head, top-10.
  2  batched inverted-index decode: 64 requests x 32,768 tokens, 8/32 heads,
     bf16, one codebook of C=256 centres per KV head shared by all requests,
     top-16 lists.
  3  token-level indexer top-k (DSA style, as in the HiSparse notes): 16
     requests x 200,000 tokens, indexer keys d_idx=64, top-2048 tokens,
     attention over 32/8 heads, 256 planted high-score tokens per request.
  4  HiSparse-style hierarchical KV ("KV卸载上主机:HiSparse、PDD与DDR4回收",
     HiSparse analysis): 32 requests x 131,072 tokens, 8 KV heads, bf16,
     4096 hot slots per request, top-2048 selections whose consecutive steps
     overlap in exactly round(0.85 * 2048) = 1741 tokens.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = [
    "WorkloadConfig",
    "CONFIGS",
    "config",
    "ivf_problem",
    "ivf_queries",
    "token_problem",
    "token_queries",
    "cache_problem",
    "selection_trace",
    "DTYPES",
]

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# Generator tags: one independent stream per tensor role.
_TAG = {
    "centroids": 1,
    "components": 2,
    "key_noise": 3,
    "values": 4,
    "q_components": 5,
    "q_noise": 6,
    "idx_keys": 7,
    "planted": 8,
    "idx_dir": 9,
    "kv_dir": 10,
    "q_idx_noise": 11,
    "trace": 12,
    "keys": 13,
}


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    """Shape and distribution of one synthetic workload."""

    index: int
    name: str
    kind: str  # "ivf" | "token" | "cache"
    batch: int
    n_tokens: int
    n_kv_heads: int
    n_q_heads: int
    head_dim: int
    top_k: int
    dtype: str
    steps: int
    seed: int
    # inverted-index workloads
    n_centroids: int = 0
    shared_codebook: bool = True
    cluster_sd: float = 0.3
    # token-indexer workload
    idx_dim: int = 0
    n_planted: int = 0
    planted_idx_scale: float = 12.0
    planted_kv_scale: float = 8.0
    # hierarchical cache workload
    n_slots: int = 0
    overlap: int = 0
    # selection-trace locality (0 = uniform draws): token popularity
    # (standard deviation of the log-normal weights) and recency (the share
    # of each step's new tokens drawn from tokens dropped within the last
    # recency_window steps)
    popularity_sd: float = 0.0
    recency: float = 0.0
    recency_window: int = 8

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def replace(self, **kw) -> "WorkloadConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    0: WorkloadConfig(
        index=0, name="tiny-ivf-f32", kind="ivf", batch=1, n_tokens=4096,
        n_kv_heads=1, n_q_heads=1, head_dim=128, top_k=4, dtype="f32",
        steps=1, seed=0, n_centroids=64, shared_codebook=True),
    1: WorkloadConfig(
        index=1, name="karat-ivf-100k", kind="ivf", batch=1, n_tokens=100_000,
        n_kv_heads=8, n_q_heads=32, head_dim=128, top_k=10, dtype="bf16",
        steps=64, seed=1, n_centroids=1000, shared_codebook=False),
    2: WorkloadConfig(
        index=2, name="batched-ivf-64x32k", kind="ivf", batch=64,
        n_tokens=32_768, n_kv_heads=8, n_q_heads=32, head_dim=128, top_k=16,
        dtype="bf16", steps=64, seed=2, n_centroids=256, shared_codebook=True),
    3: WorkloadConfig(
        index=3, name="token-topk-16x200k", kind="token", batch=16,
        n_tokens=200_000, n_kv_heads=8, n_q_heads=32, head_dim=128,
        top_k=2048, dtype="bf16", steps=64, seed=3, idx_dim=64,
        n_planted=256),
    4: WorkloadConfig(
        index=4, name="hier-cache-32x128k", kind="cache", batch=32,
        n_tokens=131_072, n_kv_heads=8, n_q_heads=32, head_dim=128,
        top_k=2048, dtype="bf16", steps=64, seed=4, n_slots=4096,
        overlap=1741),
}


def config(i: int, **overrides) -> WorkloadConfig:
    """Workload ``i`` with optional field overrides (smaller test shapes)."""
    return CONFIGS[i].replace(**overrides) if overrides else CONFIGS[i]


def _gen(seed: int, tag: str, device, salt: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + _TAG[tag] * 7919 + salt * 104_729) & 0x7FFF_FFFF_FFFF)
    return g


def _randn(shape, gen, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


# ----------------------------------------------------------------------------
# Inverted-index workloads (0, 1, 2)
# ----------------------------------------------------------------------------

def ivf_problem(cfg: WorkloadConfig, device="cpu") -> dict:
    """Codebook, clustered keys and Gaussian values for an inverted-index workload.

    Returns a dict with
      centroids  [Bc][Hkv][C][d]  (Bc = 1 when the codebook is shared)
      keys       [B][N][Hkv][d]   the K cache: centre of a uniformly drawn
                                  component plus cluster_sd * N(0, I)
      values     [B][N][Hkv][d]   N(0, I)
    all in the workload dtype. The drawn component of each key is not
    returned: posting lists come from the index build, not from the draw.
    """
    assert cfg.kind == "ivf"
    B, N, Hkv, d, C = cfg.batch, cfg.n_tokens, cfg.n_kv_heads, cfg.head_dim, cfg.n_centroids
    Bc = 1 if cfg.shared_codebook else B
    dt = cfg.torch_dtype
    cent32 = _randn((Bc, Hkv, C, d), _gen(cfg.seed, "centroids", device), device)
    g_comp = _gen(cfg.seed, "components", device)
    g_noise = _gen(cfg.seed, "key_noise", device)
    g_val = _gen(cfg.seed, "values", device)
    keys = torch.empty((B, N, Hkv, d), dtype=dt, device=device)
    values = torch.empty((B, N, Hkv, d), dtype=dt, device=device)
    head = torch.arange(Hkv, device=device)
    for b in range(B):  # one request at a time bounds the fp32 temporaries
        cb = cent32[0 if cfg.shared_codebook else b]  # [Hkv][C][d]
        comp = torch.randint(0, C, (N, Hkv), generator=g_comp, device=device)
        centre = cb[head[None, :].expand(N, Hkv), comp]  # [N][Hkv][d]
        noise = _randn((N, Hkv, d), g_noise, device)
        keys[b] = (centre + cfg.cluster_sd * noise).to(dt)
        values[b] = _randn((N, Hkv, d), g_val, device).to(dt)
    return {"centroids": cent32.to(dt), "keys": keys, "values": values}


def ivf_queries(cfg: WorkloadConfig, centroids: torch.Tensor, steps: Optional[int] = None,
                salt: int = 0) -> torch.Tensor:
    """Decode queries [steps][B][Hq][d]: the centre of a freshly drawn component
    of the query head's KV group plus cluster_sd * N(0, I), in the workload dtype.

    ``salt`` selects an independent redraw of the same distribution.
    """
    steps = cfg.steps if steps is None else steps
    device = centroids.device
    B, Hq, d, C, G = cfg.batch, cfg.n_q_heads, cfg.head_dim, cfg.n_centroids, cfg.group
    cent32 = centroids.to(torch.float32)
    comp = torch.randint(0, C, (steps, B, Hq), generator=_gen(cfg.seed, "q_components", device, salt),
                         device=device)
    noise = _randn((steps, B, Hq, d), _gen(cfg.seed, "q_noise", device, salt), device)
    bidx = torch.arange(B, device=device)[None, :, None].expand(steps, B, Hq)
    if cent32.shape[0] == 1:
        bidx = torch.zeros_like(bidx)
    gidx = (torch.arange(Hq, device=device) // G)[None, None, :].expand(steps, B, Hq)
    centre = cent32[bidx, gidx, comp]
    return (centre + cfg.cluster_sd * noise).to(cfg.torch_dtype)


# ----------------------------------------------------------------------------
# Token-indexer workload (3)
# ----------------------------------------------------------------------------

def _unit_rows(shape, gen, device) -> torch.Tensor:
    v = _randn(shape, gen, device)
    return v / v.norm(dim=-1, keepdim=True)


def token_problem(cfg: WorkloadConfig, device="cpu") -> dict:
    """Indexer keys and K/V with planted high-score tokens.

    Returns
      k_idx    [B][N][d_idx]  N(0, I); at the planted positions
                               planted_idx_scale * u_b + N(0, I)
      keys     [B][N][Hkv][d] N(0, I); planted: planted_kv_scale * w_{b,g} + N(0, I)
      values   [B][N][Hkv][d] N(0, I)
      planted  [B][n_planted] int64 planted positions (ascending)
      u        [B][d_idx] fp32 unit directions, w [B][Hkv][d] fp32 unit directions
    """
    assert cfg.kind == "token"
    B, N, Hkv, d, di, P = (cfg.batch, cfg.n_tokens, cfg.n_kv_heads, cfg.head_dim,
                           cfg.idx_dim, cfg.n_planted)
    dt = cfg.torch_dtype
    u = _unit_rows((B, di), _gen(cfg.seed, "idx_dir", device), device)
    w = _unit_rows((B, Hkv, d), _gen(cfg.seed, "kv_dir", device), device)
    g_pl = _gen(cfg.seed, "planted", device)
    g_idx = _gen(cfg.seed, "idx_keys", device)
    g_key = _gen(cfg.seed, "keys", device)
    g_val = _gen(cfg.seed, "values", device)
    k_idx = torch.empty((B, N, di), dtype=dt, device=device)
    keys = torch.empty((B, N, Hkv, d), dtype=dt, device=device)
    values = torch.empty((B, N, Hkv, d), dtype=dt, device=device)
    planted = torch.empty((B, P), dtype=torch.int64, device=device)
    for b in range(B):
        pos = torch.randperm(N, generator=g_pl, device=device)[:P].sort().values
        planted[b] = pos
        ki = _randn((N, di), g_idx, device)
        ki[pos] += cfg.planted_idx_scale * u[b]
        k_idx[b] = ki.to(dt)
        kk = _randn((N, Hkv, d), g_key, device)
        kk[pos] += cfg.planted_kv_scale * w[b]
        keys[b] = kk.to(dt)
        values[b] = _randn((N, Hkv, d), g_val, device).to(dt)
    return {"k_idx": k_idx, "keys": keys, "values": values, "planted": planted, "u": u, "w": w}


def token_queries(cfg: WorkloadConfig, prob: dict, steps: Optional[int] = None, salt: int = 0):
    """Per-step indexer queries q_idx [steps][B][d_idx] = planted_idx_scale * u_b + N(0, I)
    and attention queries q [steps][B][Hq][d] = planted_kv_scale * w_{b, h div G} + N(0, I)."""
    steps = cfg.steps if steps is None else steps
    u, w = prob["u"], prob["w"]
    device = u.device
    B, Hq, d, di, G = cfg.batch, cfg.n_q_heads, cfg.head_dim, cfg.idx_dim, cfg.group
    g = _gen(cfg.seed, "q_idx_noise", device, salt)
    q_idx = cfg.planted_idx_scale * u[None] + _randn((steps, B, di), g, device)
    gq = _gen(cfg.seed, "q_noise", device, salt)
    wq = w.repeat_interleave(G, dim=1)  # [B][Hq][d]
    q = cfg.planted_kv_scale * wq[None] + _randn((steps, B, Hq, d), gq, device)
    return q_idx.to(cfg.torch_dtype), q.to(cfg.torch_dtype)


# ----------------------------------------------------------------------------
# Hierarchical-cache workload (4)
# ----------------------------------------------------------------------------

def selection_trace(cfg: WorkloadConfig, steps: Optional[int] = None) -> torch.Tensor:
    """Per-step token selections [steps][B][k] int32, ascending within each row.

    Step 0: k distinct tokens drawn uniformly from [0, N). Step t+1 keeps
    ``overlap`` tokens drawn uniformly from step t's set and adds k - overlap
    tokens drawn uniformly from the tokens step t did not select.
    Drawn on the CPU so the trace is the same whatever device consumes it.
    """
    steps = cfg.steps if steps is None else steps
    if cfg.popularity_sd > 0 or cfg.recency > 0:
        return _selection_trace_local(cfg, steps)
    B, N, k, keep = cfg.batch, cfg.n_tokens, cfg.top_k, cfg.overlap
    assert 0 <= keep <= k <= N
    g = _gen(cfg.seed, "trace", "cpu")
    out = torch.empty((steps, B, k), dtype=torch.int32)
    for b in range(B):
        cur = torch.randperm(N, generator=g)[:k].sort().values
        out[0, b] = cur.to(torch.int32)
        for t in range(1, steps):
            kept = cur[torch.randperm(k, generator=g)[:keep]]
            taken = torch.zeros(N, dtype=torch.bool)
            taken[cur] = True
            pool = torch.randperm(N, generator=g)
            fresh = pool[~taken[pool]][: k - keep]
            cur = torch.cat([kept, fresh]).sort().values
            out[t, b] = cur.to(torch.int32)
    return out


def _selection_trace_local(cfg: WorkloadConfig, steps: int) -> torch.Tensor:
    """A selection trace with the locality of real ones: popular tokens stay
    selected longer and come back more often, and recently dropped tokens
    return. Every token of a request has a fixed log-normal weight
    exp(popularity_sd * z). Step 0 draws k tokens without replacement with
    probability proportional to the weights; step t+1 keeps ``overlap`` of
    step t's tokens the same way, then draws round(recency * (k - overlap))
    new tokens, by weight, from the tokens dropped within the last
    ``recency_window`` steps (as many as there are), and the rest by weight
    from every token step t did not select. Consecutive steps share exactly
    ``overlap`` tokens. Weighted draws use Gumbel top-m (log-weight plus
    standard Gumbel noise, the m largest). Drawn on the CPU in fp64.
    """
    B, N, k, keep = cfg.batch, cfg.n_tokens, cfg.top_k, cfg.overlap
    assert 0 <= keep <= k <= N and 0.0 <= cfg.recency <= 1.0 and cfg.recency_window >= 1
    g = _gen(cfg.seed, "trace", "cpu")
    out = torch.empty((steps, B, k), dtype=torch.int32)
    never = -(1 << 62)
    for b in range(B):
        lw = cfg.popularity_sd * torch.randn(N, generator=g, dtype=torch.float64)

        def draw(idx, m):
            if m <= 0:
                return idx[:0]
            u = torch.rand(idx.numel(), generator=g, dtype=torch.float64).clamp_min(1e-300)
            return idx[torch.topk(lw[idx] - torch.log(-torch.log(u)), m).indices]

        cur = draw(torch.arange(N), k).sort().values
        out[0, b] = cur.to(torch.int32)
        last_drop = torch.full((N,), never, dtype=torch.int64)
        for t in range(1, steps):
            kept = draw(cur, keep)
            in_cur = torch.zeros(N, dtype=torch.bool)
            in_cur[cur] = True
            n_new = k - keep
            pool = torch.nonzero((last_drop >= t - cfg.recency_window) & ~in_cur).flatten()
            back = draw(pool, min(int(round(cfg.recency * n_new)), pool.numel()))
            excl = in_cur.clone()
            excl[back] = True
            fresh = draw(torch.nonzero(~excl).flatten(), n_new - back.numel())
            nxt = torch.cat([kept, back, fresh]).sort().values
            in_nxt = torch.zeros(N, dtype=torch.bool)
            in_nxt[nxt] = True
            last_drop[cur[~in_nxt[cur]]] = t
            cur = nxt
            out[t, b] = cur.to(torch.int32)
    return out


def cache_problem(cfg: WorkloadConfig, device="cpu", kv_device=None) -> dict:
    """Full K/V [B][N][Hkv][d] (N(0, I), workload dtype), queries
    [steps][B][Hq][d] and the selection trace. ``kv_device`` is where the
    full K/V is drawn (default: ``device``)."""
    assert cfg.kind == "cache"
    kv_device = device if kv_device is None else kv_device
    B, N, Hkv, d, Hq = cfg.batch, cfg.n_tokens, cfg.n_kv_heads, cfg.head_dim, cfg.n_q_heads
    dt = cfg.torch_dtype
    g_key = _gen(cfg.seed, "keys", kv_device)
    g_val = _gen(cfg.seed, "values", kv_device)
    keys = torch.empty((B, N, Hkv, d), dtype=dt, device=kv_device)
    values = torch.empty((B, N, Hkv, d), dtype=dt, device=kv_device)
    for b in range(B):
        keys[b] = _randn((N, Hkv, d), g_key, kv_device).to(dt)
        values[b] = _randn((N, Hkv, d), g_val, kv_device).to(dt)
    q = _randn((cfg.steps, B, Hq, d), _gen(cfg.seed, "q_noise", device), device).to(dt)
    return {"keys": keys, "values": values, "q": q, "trace": selection_trace(cfg).to(device)}
