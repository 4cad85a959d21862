"""Oracle for the HiSparse-style hierarchical KV cache (RESOLVE) and the
attention over the hot slots.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain numpy, exact
integer state, fp64 attention.

Sources:
  [HISPARSE-NEWS] "KV卸载上主机:HiSparse、PDD与DDR4回收", paper analysis 1
    (HiSparse): the authoritative full KV of each request lives in pinned host
    memory; HBM holds a fixed hot cache of B slots per request per layer,
    driven by a page table plus LRU metadata; one RESOLVE step does hit
    detection, LRU replacement, metadata update and the host fetch; only the
    placement of KV changes, never the selected positions or the attention,
    so the result is exact. Its measurements name LRU, FIFO, random and the
    offline Belady policy.
  [HISPARSE-NOTES] "10月14日学习笔记", HiSparse, method 1: consecutive decode
    steps select overlapping positions and LRU fits that pattern best.

Readings (batch-step LRU, where the page does not spell out the order of
events inside one step):
  * Hits are the selected tokens whose page-table entry is a slot; each hit
    slot's last-use stamp becomes the step index t, so hits are protected.
  * Misses are the selected tokens not resident, taken in ascending token
    order.
  * Victims are the slots whose last use is before t, ordered by
    (last use ascending, slot ascending); free slots carry last use -1 and so
    go first. The r-th miss takes the r-th victim: the victim's previous
    token (if any) leaves the page table, the miss enters it, the slot's
    stamp becomes t, and the token's K/V rows are copied from the host copy
    into the slot.
  * A slot holds one token's K and V rows for every KV head of the layer.
"""

from __future__ import annotations

import numpy as np

from .ivf import attend

__all__ = ["CacheState", "lru_step", "fetch_rows", "attend_slots"]


class CacheState:
    """Per-request cache metadata: page_table [N] (slot or -1),
    slot_token [S] (token or -1), last_use [S] (step or -1)."""

    def __init__(self, n_tokens: int, n_slots: int):
        self.page_table = np.full(n_tokens, -1, dtype=np.int64)
        self.slot_token = np.full(n_slots, -1, dtype=np.int64)
        self.last_use = np.full(n_slots, -1, dtype=np.int64)

    def copy(self) -> "CacheState":
        c = CacheState.__new__(CacheState)
        c.page_table = self.page_table.copy()
        c.slot_token = self.slot_token.copy()
        c.last_use = self.last_use.copy()
        return c


def lru_step(state: CacheState, selected, t: int):
    """One RESOLVE step for one request (mutates ``state``).

    selected: the step's distinct token ids. Returns (slots, n_hits,
    n_misses, fetches) where slots[i] is the slot that holds selected[i] after
    the step and fetches is the list of (token, slot) copies from host memory,
    in miss order.
    """
    sel = np.asarray(selected, dtype=np.int64)
    pt, st, lu = state.page_table, state.slot_token, state.last_use
    resident = pt[sel] >= 0
    lu[pt[sel[resident]]] = t                                   # (1) hits, protected
    misses = np.sort(sel[~resident])                            # (2) ascending token order
    cand = np.nonzero(lu < t)[0]                                # (3) not used this step
    victims = cand[np.lexsort((cand, lu[cand]))][: len(misses)]
    if len(victims) < len(misses):
        raise ValueError("more misses than evictable slots (k > n_slots?)")
    fetches = []
    for tok, v in zip(misses, victims):                        # (4) replace + fetch
        old = st[v]
        if old >= 0:
            pt[old] = -1
        pt[tok] = v
        st[v] = tok
        lu[v] = t
        fetches.append((int(tok), int(v)))
    return pt[sel].copy(), int(resident.sum()), len(misses), fetches


def fetch_rows(pool_k, pool_v, host_k, host_v, fetches):
    """Copy each fetched token's K/V rows (all KV heads) from the host copy
    into its slot. pool_* [S][Hkv][d], host_* [N][Hkv][d]."""
    for tok, v in fetches:
        pool_k[v] = host_k[tok]
        pool_v[v] = host_v[tok]


def attend_slots(q, pool_k, pool_v, slots):
    """Attention of every query head of one request over the rows held in
    ``slots``. q [Hq][d], pool_* [S][Hkv][d] -> [Hq][d]."""
    q = np.asarray(q)
    Hq = q.shape[0]
    Hkv = pool_k.shape[1]
    G = Hq // Hkv
    slots = np.asarray(slots, dtype=np.int64)
    out = np.empty((Hq, pool_v.shape[2]))
    for h in range(Hq):
        g = h // G
        out[h], _ = attend(q[h], pool_k[slots, g, :], pool_v[slots, g, :])
    return out
