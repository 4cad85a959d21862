"""Oracle for inverted-index (centroid) sparse-attention decode.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain fp64 numpy.

Sources, by page and section:
  [KARAT] paper-daily digest "Heterogeneous LLM Serving with General-Purpose
  Processing-Near-Memory for Retrieval-Based Sparse Attention".
    - How, index structure: every KV entry is placed in posting lists
      according to its key; a query is compared with the list centroids and
      the top-k most similar lists are scanned.
    - Core formulas, Eq. 2: Attention = softmax(Q K^T / sqrt(d_k) (.) M) V
      with M a sparse mask fixed by the retrieval; only retrieved entries are
      touched.
    - Worked example, step 3: similarity of q to C=1000 centroids of 128 dims
      costs 1000 x 128 = 128K multiply-adds; top-10 lists are chosen.
    - Worked example, step 4: scanning 10 x 1000 entries costs 10K x 128 =
      1.28M multiply-adds for the scores and the same again for the output.
    - Worked example, GPU-only comparison: full attention is 100K x 128 =
      12.8M multiply-adds.

Readings where the page is silent or garbled (each also listed in the design
notes):
  * Eq. 2's (.) M: masked logits are -inf, i.e. the softmax runs over the
    retrieved set only; an elementwise 0/1 product would leave weight e^0 on
    entries the page says are never accessed.
  * Similarity: raw dot product q . c (the worked example says cosine; the
    tiny workload says dot product; for one query, cosine ranking equals the
    dot ranking against unit-norm centroids, and scaling does not change a
    ranking).
  * Assignment: each key goes to exactly one list, its nearest centroid by
    squared Euclidean distance, ties to the lower centroid index.
  * Selection granularity: per query head; query head h reads KV head
    h div (Hq/Hkv).
  * Top-k ties: lower index wins; the selection is reported in ascending
    index order.
  * Softmax scale 1/sqrt(d_k), natural exp, no causal mask (every cached
    token precedes the decode query).
  * An empty retrieved set gives a zero output and is flagged.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "squared_distances_near",
    "nearest_centroid",
    "posting_lists",
    "index_build",
    "centroid_scores",
    "top_k",
    "selection_gap",
    "retrieved_rows",
    "attend",
    "OpCounts",
    "decode_head",
    "sparse_decode",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# Index build
# ----------------------------------------------------------------------------

def squared_distances_near(keys, centroids, m: int, chunk: int = 4096):
    """Squared Euclidean distances sum_t (k_t - c_t)^2, evaluated term by term
    in fp64, for every centroid that can be one of the m + 1 nearest of each
    key; +inf for the others.

    [KARAT] How, index structure (an entry goes to a list by its key); the
    tiny workload names the rule: nearest centroid.

    Which centroids need the direct sum is decided from the cheap expansion
    e_c = |k|^2 - 2 k.c + |c|^2 (one fp64 matrix product), with a rounding
    bound instead of trust: both e_c and the direct sum are within
    b_c = gamma (|k| + |c|)^2 of the exact distance, gamma = (d+3) u /
    (1 - (d+3) u) and u = 2^-53 (the textbook bound for a length-d fp64 dot
    product; every term is at most (|k| + |c|)^2 in total). Let U be the
    (m+1)-th smallest e_c + 2 b_c over the centroids: at least m + 1 direct
    sums are <= U, so a centroid with e_c - 2 b_c > U has a direct sum larger
    than the (m+1)-th smallest and cannot be among the m + 1 nearest. Every
    other centroid gets its direct sum. Near-ties, and large keys whose
    expansion cancels, therefore fall back to the direct sum for as many
    centroids as the bound requires (all of them, if need be).

    keys [n][d], centroids [C][d]. Returns d2 [n][C] fp64.
    """
    K = _f64(keys)
    Cn = _f64(centroids)
    n, d = K.shape
    C = Cn.shape[0]
    u = 2.0 ** -53
    gamma = (d + 3) * u / (1.0 - (d + 3) * u)
    out = np.full((n, C), np.inf)
    c2 = np.sum(Cn * Cn, axis=1)
    cn = np.sqrt(c2)
    M = min(m + 1, C)
    for s in range(0, n, chunk):
        Kc = K[s:s + chunk]
        k2 = np.sum(Kc * Kc, axis=1)
        e = k2[:, None] - 2.0 * (Kc @ Cn.T) + c2[None, :]
        b = gamma * (np.sqrt(k2)[:, None] + cn[None, :]) ** 2
        U = np.partition(e + 2.0 * b, M - 1, axis=1)[:, M - 1]
        rows, cols = np.nonzero(e - 2.0 * b <= U[:, None])
        step = max(1, (1 << 22) // max(d, 1))          # bound the temporary to ~32 MB
        for t in range(0, rows.shape[0], step):
            r, c = rows[t:t + step], cols[t:t + step]
            diff = Kc[r] - Cn[c]
            out[s + r, c] = np.sum(diff * diff, axis=1)
    return out


def nearest_centroid(keys, centroids, chunk: int = 4096):
    """Nearest centroid of every key by squared Euclidean distance.

    [KARAT] How, index structure (entries go to lists by their key); reading:
    single assignment to the nearest centroid, ties -> lower centroid index.
    The deciding distances are the direct sums of (k_t - c_t)^2
    (``squared_distances_near``).

    keys [n][d], centroids [C][d]. Returns (assign [n] int64, margin [n]) where
    margin = (d2_second - d2_best) / d2_best, the relative distance gap that
    decides the assignment (inf when the key sits on its centroid).
    """
    d2 = squared_distances_near(keys, centroids, 1, chunk)
    n, C = d2.shape
    assign = np.argmin(d2, axis=1)                                  # first minimum: lower index
    if C == 1:
        return assign, np.full(n, np.inf)
    part = np.partition(d2, 1, axis=1)
    d_best, d_second = part[:, 0], part[:, 1]
    with np.errstate(divide="ignore", invalid="ignore"):
        margin = np.where(d_best > 0, (d_second - d_best) / d_best, np.inf)
    return assign, margin


def posting_lists(assign, n_lists: int):
    """Posting lists in CSR form from an assignment.

    offsets [C+1] int32 (list c holds ids[offsets[c]:offsets[c+1]]) and
    ids [n] int32 with token ids ascending inside every list.
    """
    a = np.asarray(assign, dtype=np.int64)
    counts = np.bincount(a, minlength=n_lists)
    offsets = np.zeros(n_lists + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    ids = np.argsort(a, kind="stable")  # stable: ascending token id within a list
    return offsets.astype(np.int32), ids.astype(np.int32)


def index_build(keys, centroids):
    """Posting lists for every (request, KV head).

    keys [B][N][Hkv][d]; centroids [Bc][Hkv][C][d] with Bc = 1 (one codebook
    shared by all requests) or Bc = B.
    Returns offsets [B][Hkv][C+1], ids [B][Hkv][N] (int32) and the assignment
    margins [B][Hkv][N].
    """
    K = np.asarray(keys)
    Cn = np.asarray(centroids)
    B, N, Hkv, _ = K.shape
    C = Cn.shape[2]
    offsets = np.empty((B, Hkv, C + 1), dtype=np.int32)
    ids = np.empty((B, Hkv, N), dtype=np.int32)
    margins = np.empty((B, Hkv, N), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            cb = Cn[0 if Cn.shape[0] == 1 else b, g]
            a, m = nearest_centroid(K[b, :, g, :], cb)
            offsets[b, g], ids[b, g] = posting_lists(a, C)
            margins[b, g] = m
    return offsets, ids, margins


# ----------------------------------------------------------------------------
# Retrieval
# ----------------------------------------------------------------------------

def centroid_scores(q, centroids):
    """Similarity of one query to every centroid: s_c = sum_t q_t * c_{c,t}.

    [KARAT] worked example, step 3 (C x d multiply-adds); reading: raw dot
    product. q [d], centroids [C][d] -> [C].
    """
    return _f64(centroids) @ _f64(q)


def top_k(scores, k: int):
    """Indices of the k largest scores, ties -> lower index, ascending order.

    [KARAT] How (choose the top-k most similar lists); worked example step 3
    (top-10). k must satisfy 1 <= k <= len(scores).
    """
    s = _f64(scores)
    n = s.shape[0]
    if not 1 <= k <= n:
        raise ValueError(f"k={k} outside [1, {n}]")
    order = np.lexsort((np.arange(n), -s))  # by score descending, then index ascending
    return np.sort(order[:k])


def selection_gap(scores, k: int) -> float:
    """Relative gap at the selection boundary:
    (s_(k) - s_(k+1)) / max(|s_(k)|, |s_(k+1)|), inf when k == len(scores).

    A selection made in lower precision equals this one whenever its score
    error stays well below this gap.
    """
    s = np.sort(_f64(scores))[::-1]
    if k >= s.shape[0]:
        return math.inf
    a, b = s[k - 1], s[k]
    den = max(abs(a), abs(b))
    return 0.0 if den == 0 else (a - b) / den


def retrieved_rows(lists, offsets, ids):
    """Token ids covered by the chosen posting lists, ascending.

    [KARAT] worked example, step 4 (scan the entries of the chosen lists).
    Lists are disjoint under single assignment; duplicates are removed anyway.
    """
    off = np.asarray(offsets)
    rows = [np.asarray(ids[off[c]:off[c + 1]]) for c in lists]
    if not rows:
        return np.empty(0, dtype=np.int64)
    return np.unique(np.concatenate(rows).astype(np.int64))


def attend(q, K_rows, V_rows, d_k: int | None = None):
    """Softmax attention of one query over the retrieved rows only.

    [KARAT] Eq. 2 with the reading that masked logits are -inf:
      z_i = q . K_i / sqrt(d_k);  p_i = exp(z_i - max z) / sum_j exp(z_j - max z);
      o = sum_i p_i V_i.
    Returns (o [d_v], p [n]); an empty row set returns (zeros, empty).
    """
    q = _f64(q)
    K = _f64(K_rows)
    V = _f64(V_rows)
    d_k = q.shape[0] if d_k is None else d_k
    if K.shape[0] == 0:
        return np.zeros(V.shape[1] if V.ndim == 2 else q.shape[0]), np.empty(0)
    z = (K @ q) / math.sqrt(d_k)
    m = np.max(z)
    w = np.exp(z - m)
    p = w / np.sum(w)
    return p @ V, p


# ----------------------------------------------------------------------------
# One decode query and a whole batch
# ----------------------------------------------------------------------------

@dataclass
class OpCounts:
    """Multiply-adds of one decode query, as the KARAT worked example counts them.

    retrieve = C x d (step 3), score = |R| x d_k and output = |R| x d_v
    (step 4), full_score = N x d_k (the GPU-only comparison counts only the
    scores; full_score_output adds the output pass).
    """

    retrieve: int = 0
    score: int = 0
    output: int = 0
    full_score: int = 0
    full_score_output: int = 0

    def add(self, other: "OpCounts") -> "OpCounts":
        for f in ("retrieve", "score", "output", "full_score", "full_score_output"):
            setattr(self, f, getattr(self, f) + getattr(other, f))
        return self


@dataclass
class HeadResult:
    out: np.ndarray
    lists: np.ndarray
    rows: np.ndarray
    gap: float
    empty: bool
    counts: OpCounts = field(default_factory=OpCounts)


def decode_head(q, centroids, offsets, ids, K, V, k: int, n_tokens: int | None = None) -> HeadResult:
    """Retrieval-based sparse attention for one query head.

    q [d]; centroids [C][d] of the head's KV group; offsets/ids its posting
    lists; K, V [N][d] the group's key and value rows. Steps in the page's
    order: score the centroids, keep the top-k lists, gather their rows,
    attend over them.
    """
    s = centroid_scores(q, centroids)
    lists = top_k(s, k)
    rows = retrieved_rows(lists, offsets, ids)
    o, _ = attend(q, np.asarray(K)[rows], np.asarray(V)[rows])
    C, d = np.asarray(centroids).shape
    N = np.asarray(K).shape[0] if n_tokens is None else n_tokens
    dv = np.asarray(V).shape[1]
    counts = OpCounts(retrieve=C * d, score=len(rows) * d, output=len(rows) * dv,
                      full_score=N * d, full_score_output=N * d + N * dv)
    return HeadResult(out=o, lists=lists, rows=rows, gap=selection_gap(s, k),
                      empty=len(rows) == 0, counts=counts)


def sparse_decode(q, centroids, offsets, ids, K, V, k: int, heads=None):
    """Decode one step for a batch.

    q [B][Hq][d]; centroids [Bc][Hkv][C][d]; offsets [B][Hkv][C+1];
    ids [B][Hkv][N]; K, V [B][N][Hkv][d]. Query head h uses KV head
    h div (Hq / Hkv). ``heads`` optionally restricts the work to a list of
    (b, h) pairs (sampled checks at full size).

    Returns dict with out [B][Hq][d] (NaN where not computed), sel [B][Hq][k]
    (-1 where not computed), gap [B][Hq], n_rows [B][Hq], empty [B][Hq] and the
    summed OpCounts.
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Cn = np.asarray(centroids)
    Hkv = Cn.shape[1]
    G = Hq // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    out = np.full((B, Hq, np.asarray(V).shape[3]), np.nan)
    sel = np.full((B, Hq, k), -1, dtype=np.int64)
    gap = np.full((B, Hq), np.nan)
    n_rows = np.full((B, Hq), -1, dtype=np.int64)
    empty = np.zeros((B, Hq), dtype=bool)
    total = OpCounts()
    for b, h in heads:
        g = h // G
        cb = Cn[0 if Cn.shape[0] == 1 else b, g]
        r = decode_head(q[b, h], cb, offsets[b, g], ids[b, g], K[b, :, g, :], V[b, :, g, :], k)
        out[b, h], sel[b, h], gap[b, h] = r.out, r.lists, r.gap
        n_rows[b, h], empty[b, h] = len(r.rows), r.empty
        total.add(r.counts)
    return {"out": out, "sel": sel, "gap": gap, "n_rows": n_rows, "empty": empty, "counts": total}
