"""Oracle for the inverted-index decode variants: cosine similarity, a
fixed sink/window set attended beside the retrieved lists, and lists built
with several assignments per key.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain fp64 numpy.

Sources, by page and section:
  [KARAT] paper-daily digest "Heterogeneous LLM Serving with General-Purpose
  Processing-Near-Memory for Retrieval-Based Sparse Attention".
    - Worked example, step 3: the query is compared with every centroid by
      cosine similarity.
    - Method details, last item: the general-purpose cores also run
      window-based sparse attention (StreamingLLM) beside cluster- and
      retrieval-based schemes.
    - How, index structure: a KV entry is placed into several posting lists
      according to its key.

Readings (each also listed in the design notes):
  * Cosine: s_c = q.c / |c|. The factor 1/|q| is the same for every centroid
    of one query and is left out (it changes no ranking). A zero centroid
    scores 0.
  * Multi-assignment: each key joins its m nearest lists (squared L2, ties
    to the lower index; m = 1 is the plain index). A token in several chosen
    lists is attended once: the retrieved set is the union of the lists.
  * Sink/window (StreamingLLM's pattern of the first tokens plus the most
    recent ones): the first n_sink tokens and the last n_window tokens before
    the request's current length L are attended in every step, in addition
    to the retrieved lists. The attended set is the union (no token counted
    twice); both ranges are clipped to [0, L).
"""

from __future__ import annotations

import numpy as np

from .ivf import attend, retrieved_rows, selection_gap, squared_distances_near, top_k

__all__ = ["cosine_scores", "fixed_rows", "decode_head_ex", "sparse_decode_ex", "nearest_centroids",
           "posting_lists_multi", "index_build_multi"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def cosine_scores(q, centroids):
    """s_c = q.c / |c| for every centroid (0 for a zero centroid). q [d], centroids [C][d]."""
    Cn = _f64(centroids)
    dots = Cn @ _f64(q)
    norms = np.sqrt(np.sum(Cn * Cn, axis=1))
    return np.where(norms > 0, dots / np.where(norms > 0, norms, 1.0), 0.0)


def fixed_rows(n_sink: int, n_window: int, length: int):
    """Token ids always attended: [0, n_sink) and [length - n_window, length),
    clipped to [0, length), ascending, without repeats."""
    sink = np.arange(0, max(0, min(n_sink, length)))
    win = np.arange(max(0, length - n_window), max(0, length)) if n_window > 0 else np.arange(0)
    return np.union1d(sink, win).astype(np.int64)


def decode_head_ex(q, centroids, offsets, ids, K, V, k: int, *, similarity: str = "dot", n_sink: int = 0,
                   n_window: int = 0, length: int | None = None):
    """One query head: score the centroids (dot or cosine), keep the top-k
    lists, attend over the union of their rows with the sink and window rows.
    Returns (out [d], lists [k], rows (ascending), gap)."""
    if similarity == "dot":
        s = _f64(centroids) @ _f64(q)
    elif similarity == "cosine":
        s = cosine_scores(q, centroids)
    else:
        raise ValueError(f"unknown similarity {similarity}")
    lists = top_k(s, k)
    L = np.asarray(K).shape[0] if length is None else length
    rows = np.union1d(retrieved_rows(lists, offsets, ids), fixed_rows(n_sink, n_window, L)).astype(np.int64)
    o, _ = attend(q, np.asarray(K)[rows], np.asarray(V)[rows])
    return o, lists, rows, selection_gap(s, k)


def sparse_decode_ex(q, centroids, offsets, ids, K, V, k: int, *, similarity: str = "dot", n_sink: int = 0,
                     n_window: int = 0, lengths=None, heads=None):
    """A batch of decode queries under the variants. q [B][Hq][d];
    centroids [Bc][Hkv][C][d]; offsets/ids CSR per (request, KV head);
    K, V [B][N][Hkv][d]; lengths [B] (default N). Returns dict with out,
    sel, gap, n_rows (NaN / -1 where not computed)."""
    q = np.asarray(q)
    B, Hq, d = q.shape
    Cn = np.asarray(centroids)
    Hkv = Cn.shape[1]
    G = Hq // Hkv
    N = np.asarray(K).shape[1]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    out = np.full((B, Hq, np.asarray(V).shape[3]), np.nan)
    sel = np.full((B, Hq, k), -1, dtype=np.int64)
    gap = np.full((B, Hq), np.nan)
    n_rows = np.full((B, Hq), -1, dtype=np.int64)
    for b, h in heads:
        g = h // G
        L = N if lengths is None else int(lengths[b])
        o, lists, rows, gp = decode_head_ex(q[b, h], Cn[0 if Cn.shape[0] == 1 else b, g], offsets[b, g], ids[b, g],
                                            np.asarray(K)[b, :, g, :], np.asarray(V)[b, :, g, :], k,
                                            similarity=similarity, n_sink=n_sink, n_window=n_window, length=L)
        out[b, h], sel[b, h], gap[b, h], n_rows[b, h] = o, lists, gp, len(rows)
    return {"out": out, "sel": sel, "gap": gap, "n_rows": n_rows}


def nearest_centroids(keys, centroids, m: int):
    """The m nearest centroids of every key by squared Euclidean distance,
    nearest first, ties to the lower index. keys [n][d], centroids [C][d].
    Returns (assign [n][m], gap [n]) where gap = (d2_(m+1) - d2_(m)) / d2_(m)
    is the relative margin that decides the m-th choice (inf if m == C)."""
    K = _f64(keys)
    Cn = _f64(centroids)
    d2 = squared_distances_near(K, Cn, m)    # direct sums for every centroid that can rank <= m + 1
    C = Cn.shape[0]
    order = np.lexsort((np.broadcast_to(np.arange(C), d2.shape), d2), axis=1)  # distance, then index
    assign = order[:, :m]
    if m >= C:
        return assign, np.full(K.shape[0], np.inf)
    dm = np.take_along_axis(d2, order[:, m - 1:m], axis=1)[:, 0]
    dn = np.take_along_axis(d2, order[:, m:m + 1], axis=1)[:, 0]
    with np.errstate(divide="ignore", invalid="ignore"):
        gap = np.where(dm > 0, (dn - dm) / dm, np.inf)
    return assign, gap


def posting_lists_multi(assign, n_lists: int):
    """CSR lists from an m-way assignment [n][m]: list c holds every token
    that chose it, ascending. Returns offsets [C+1], ids [n*m], and alt
    [n*m]: for each entry, the token's other chosen lists (m - 1 of them,
    in the token's order of preference; shape [n*m][m-1])."""
    a = np.asarray(assign, dtype=np.int64)
    n, m = a.shape
    offsets = np.zeros(n_lists + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.bincount(a.ravel(), minlength=n_lists))
    ids = np.empty(n * m, dtype=np.int64)
    alt = np.empty((n * m, max(m - 1, 0)), dtype=np.int64)
    fill = offsets[:-1].copy()
    for i in range(n):               # ascending token ids inside every list
        for r in range(m):
            c = a[i, r]
            ids[fill[c]] = i
            alt[fill[c]] = np.delete(a[i], r)
            fill[c] += 1
    return offsets, ids, alt


def index_build_multi(keys, centroids, m: int):
    """m-way posting lists for every (request, KV head): keys [B][N][Hkv][d],
    centroids [Bc][Hkv][C][d]. Returns offsets [B][Hkv][C+1],
    ids [B][Hkv][N*m], alt [B][Hkv][N*m][m-1] and the smallest m-th-choice
    margin seen."""
    K = np.asarray(keys)
    Cn = np.asarray(centroids)
    B, N, Hkv, _ = K.shape
    C = Cn.shape[2]
    offsets = np.empty((B, Hkv, C + 1), dtype=np.int64)
    ids = np.empty((B, Hkv, N * m), dtype=np.int64)
    alt = np.empty((B, Hkv, N * m, max(m - 1, 0)), dtype=np.int64)
    margin = np.inf
    for b in range(B):
        for g in range(Hkv):
            a, gap = nearest_centroids(K[b, :, g], Cn[0 if Cn.shape[0] == 1 else b, g], m)
            offsets[b, g], ids[b, g], alt[b, g] = posting_lists_multi(a, C)
            margin = min(margin, float(gap.min()))
    return offsets, ids, alt, margin
