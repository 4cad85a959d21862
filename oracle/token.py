"""Oracle for token-level indexer top-k sparse attention (DSA-style selector).

TEST INFRASTRUCTURE ONLY (see the package docstring): plain fp64 numpy.

Sources:
  [HISPARSE-NOTES] "10月14日学习笔记", HiSparse, motivation: an indexer picks
    the top-k tokens for each attention, so the work per step falls from
    O(context) to O(k).
  [HISPARSE-NEWS] "KV卸载上主机:HiSparse、PDD与DDR4回收", paper analysis 1:
    the sparse selector (DSA / NSA / Quest) states every step which KV
    positions it needs; attention reads only those.
  [KARAT] paper-daily digest, Eq. 2 (masked softmax over the selected set).

Readings: the indexer score of token i is the raw dot product of the
request's indexer query with the token's indexer key; the top-k (ties ->
lower token id) is shared by every head of the request; the selection is
reported in ascending token order; attention is Eq. 2 over that set with
1/sqrt(d_k) scaling.
"""

from __future__ import annotations

import numpy as np

from .ivf import attend, top_k, selection_gap

__all__ = ["indexer_scores", "token_topk", "token_decode"]


def indexer_scores(q_idx, k_idx):
    """s_i = sum_t q_idx_t * k_idx_{i,t}. q_idx [d_idx], k_idx [N][d_idx] -> [N]."""
    return np.asarray(k_idx, dtype=np.float64) @ np.asarray(q_idx, dtype=np.float64)


def token_topk(q_idx, k_idx, k: int):
    """The k highest-scoring tokens (ties -> lower id), ascending, and the
    relative score gap at the boundary."""
    s = indexer_scores(q_idx, k_idx)
    return top_k(s, k), selection_gap(s, k)


def token_decode(q_idx, k_idx, q, K, V, k: int, requests=None, heads=None):
    """One decode step for a batch.

    q_idx [B][d_idx], k_idx [B][N][d_idx], q [B][Hq][d], K, V [B][N][Hkv][d].
    ``requests`` restricts the work to some requests; ``heads`` to some
    query heads of each. Returns dict with sel [B][k] (-1 if skipped),
    gap [B], out [B][Hq][d] (NaN where skipped).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = np.asarray(K).shape[2]
    G = Hq // Hkv
    requests = range(B) if requests is None else requests
    heads = range(Hq) if heads is None else heads
    sel = np.full((B, k), -1, dtype=np.int64)
    gap = np.full(B, np.nan)
    out = np.full((B, Hq, np.asarray(V).shape[3]), np.nan)
    for b in requests:
        rows, gap[b] = token_topk(q_idx[b], k_idx[b], k)
        sel[b] = rows
        for h in heads:
            g = h // G
            out[b, h], _ = attend(q[b, h], K[b][rows, g, :], V[b][rows, g, :])
    return {"sel": sel, "gap": gap, "out": out}
