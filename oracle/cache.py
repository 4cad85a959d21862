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

A layer group that shares one selection (a model reusing the indexer's
choice across layers) keeps one set of tables; every layer's pool receives
the same missed tokens' rows of its own host copy.

Other replacement policies (the page compares LRU with FIFO, random and the
offline Belady policy by miss rate; it does not define them further):
  * FIFO: a hit leaves the slot's stamp alone, so the stamp is the step of
    the slot's last fetch; victims by (fetch step, slot).
  * Random: victims by a per-(request, step, slot) key from the SplitMix64
    generator (Steele, Lea and Flood, "Fast Splittable Pseudorandom Number
    Generators", OOPSLA 2014), then slot.
  * Belady (priority): the caller gives, per token, the next step at which
    it will be selected (a large value for never); victims are the resident
    tokens needed furthest in the future, ties to the lower slot.
  Under every policy the step's hits are protected, free slots go first, and
  the r-th miss (ascending token order) takes the r-th victim.
"""

from __future__ import annotations

import numpy as np

from .ivf import attend

__all__ = ["CacheState", "lru_step", "policy_step", "group_step", "splitmix64", "random_key", "next_use_table",
           "fetch_rows", "attend_slots", "POLICIES", "NEVER"]

POLICIES = ("lru", "fifo", "random", "belady")
NEVER = 2**31 - 1          # "not selected again" in a next-use table
_M64 = (1 << 64) - 1


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


def splitmix64(x: int) -> int:
    """One output of SplitMix64 for state x (the state is advanced by the
    golden-ratio increment, then mixed): Steele, Lea and Flood, OOPSLA 2014."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def random_key(seed: int, request: int, step: int, slot: int) -> int:
    """31-bit eviction key of one slot at one step: SplitMix64 chained over
    (seed, request, step, slot), top 31 bits."""
    x = splitmix64(seed & _M64)
    x = splitmix64((x + request) & _M64)
    x = splitmix64((x + step) & _M64)
    x = splitmix64((x + slot) & _M64)
    return x >> 33


def next_use_table(trace):
    """For a selection trace [T][k] of one request: nu[t] maps token -> the
    first step u > t that selects it (NEVER if none), as a dict per step."""
    T = len(trace)
    out = [None] * T
    nxt = {}
    for t in range(T - 1, -1, -1):
        out[t] = dict(nxt)
        for tok in np.asarray(trace[t]).tolist():
            nxt[int(tok)] = t
    return out


def policy_step(state: CacheState, selected, t: int, policy: str = "lru", *, seed: int = 0,
                request: int = 0, next_use=None):
    """One RESOLVE step under a replacement policy (mutates ``state``).

    policy: "lru" (== lru_step), "fifo", "random" (needs seed, request) or
    "belady" (needs next_use: token -> next selecting step, NEVER if none;
    tokens missing from it count as NEVER). Returns what lru_step returns.
    """
    if policy == "lru":
        return lru_step(state, selected, t)
    if policy not in POLICIES:
        raise ValueError(f"unknown policy {policy}")
    sel = np.asarray(selected, dtype=np.int64)
    pt, st, lu = state.page_table, state.slot_token, state.last_use
    resident = pt[sel] >= 0
    hit_slots = set(pt[sel[resident]].tolist())
    if policy != "fifo":
        lu[pt[sel[resident]]] = t                               # bookkeeping only
    misses = np.sort(sel[~resident])
    cand = [s for s in range(len(st)) if s not in hit_slots]

    def key(s):
        if st[s] < 0:
            return (0, 0, s)                                    # free slots first
        if policy == "fifo":
            return (1, int(lu[s]), s)
        if policy == "random":
            return (1, random_key(seed, request, t, s), s)
        nu = NEVER if next_use is None else int(next_use.get(int(st[s]), NEVER))
        return (1, -nu, s)                                      # furthest next use first

    victims = sorted(cand, key=key)[: len(misses)]
    if len(victims) < len(misses):
        raise ValueError("more misses than evictable slots (k > n_slots?)")
    fetches = []
    for tok, v in zip(misses, victims):
        old = st[v]
        if old >= 0:
            pt[old] = -1
        pt[tok] = v
        st[v] = tok
        lu[v] = t
        fetches.append((int(tok), int(v)))
    return pt[sel].copy(), int(resident.sum()), len(misses), fetches


def group_step(state: CacheState, selected, t: int, hosts, pools, policy: str = "lru", **kw):
    """One RESOLVE step for a group of layers that share the selection
    ([HISPARSE-NOTES] method 3: a layer group reuses the indexer's choice).

    The slot tables are shared: a shared selection drives every layer's
    cache through the same decisions. The missed tokens' rows are copied for
    every layer. hosts: [(host_k, host_v)] per layer ([N][Hkv][d]);
    pools: [(pool_k, pool_v)] per layer ([S][Hkv][d], written in place).
    Returns what policy_step returns."""
    slots, h, m, fetches = policy_step(state, selected, t, policy, **kw)
    for (hk, hv), (pk, pv) in zip(hosts, pools):
        fetch_rows(pk, pv, hk, hv, fetches)
    return slots, h, m, fetches


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
