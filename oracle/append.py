"""Oracle for the per-step KV and index append of the inverted index.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain fp64 numpy.

Sources, by page and section:
  [KARAT] paper-daily digest "Heterogeneous LLM Serving with General-Purpose
  Processing-Near-Memory for Retrieval-Based Sparse Attention".
    - Worked example, step 6: after attention the GPU updates the KV cache
      and the index; each new KV entry is added to its posting list.
    - Limitations, item 3: as the KV cache grows, keeping the index up to
      date costs extra compute and storage.

Readings (each also listed in the design notes):
  * The new entry goes to the list of its nearest centroid by squared
    Euclidean distance, ties to the lower index: the same rule that built the
    lists.
  * Storage for growth: every list is followed by `slack` free entries (-1).
    A list keeps its valid ids in ascending order at the front of its range
    and holds its valid count in `lens`. An append to a full list leaves the
    index unchanged and is reported; the caller rebuilds the index. The
    pages do not say how a full list is handled.
  * Appended token ids grow step by step, so every list stays in ascending
    id order.
  * Several lists per key ([KARAT] How, index structure: an entry can be
    placed in more than one posting list): a key joins its m nearest lists.
    List storage then holds N * m entries, and every entry carries the
    token's other m - 1 lists (`alt`, in the token's order of preference),
    which a decode needs to attend a token chosen through two lists once.
    An append is all or nothing: when one of the key's m lists is full, the
    key joins none of them and the append is reported, so every indexed
    token sits in exactly its m lists.
  * A full list is recovered by re-laying the lists out with fresh free
    entries after each (`regrow`, keeping every list's valid entries in
    order) and appending the reported keys again; no key is reassigned. The
    pages say nothing about this; it is the plainest repair that keeps the
    lists' contents.
"""

from __future__ import annotations

import numpy as np

from .ivf import nearest_centroid
from .variants import nearest_centroids

__all__ = ["index_build_dynamic", "append_key", "compact", "append_step", "index_build_dynamic_multi",
           "append_key_multi", "regrow", "regrow_slack"]


def index_build_dynamic(keys, centroids, n_prefix: int, slack: int):
    """Posting lists over the first n_prefix keys of one (request, KV head),
    with `slack` free entries after each list.

    keys [N][d] (N = capacity), centroids [C][d]. Requires
    n_prefix + C * slack <= N. Returns offsets [C+1] (list c owns
    ids[offsets[c]:offsets[c+1]]), lens [C] (valid entries at the front of
    each range) and ids [N] (-1 where free).
    """
    K = np.asarray(keys)
    N = K.shape[0]
    C = np.asarray(centroids).shape[0]
    if not (1 <= n_prefix <= N and slack >= 0 and n_prefix + C * slack <= N):
        raise ValueError("need 1 <= n_prefix <= N and n_prefix + C * slack <= N")
    a, _ = nearest_centroid(K[:n_prefix], centroids)
    counts = np.bincount(a, minlength=C)
    offsets = np.zeros(C + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts + slack)
    ids = np.full(N, -1, dtype=np.int64)
    for c in range(C):
        members = np.flatnonzero(a == c)  # ascending token ids
        ids[offsets[c]:offsets[c] + members.size] = members
    return offsets, counts.astype(np.int64), ids


def append_key(offsets, lens, ids, centroids, key, pos: int):
    """Add token `pos` with key `key` to the list of its nearest centroid.

    Updates lens and ids in place when the list has a free entry. Returns
    (list, inserted).
    """
    a, _ = nearest_centroid(np.asarray(key)[None, :], centroids)
    c = int(a[0])
    if lens[c] < offsets[c + 1] - offsets[c]:
        ids[offsets[c] + lens[c]] = pos
        lens[c] += 1
        return c, True
    return c, False


def compact(offsets, lens, ids):
    """The valid lists of a dynamic index as an ordinary CSR (offsets [C+1],
    ids [sum lens]): the same lists, without the free entries."""
    C = len(lens)
    out_off = np.zeros(C + 1, dtype=np.int64)
    out_off[1:] = np.cumsum(lens)
    out_ids = np.concatenate([ids[offsets[c]:offsets[c] + lens[c]] for c in range(C)]) if C else np.zeros(0)
    return out_off.astype(np.int32), np.asarray(out_ids, dtype=np.int32)


def index_build_dynamic_multi(keys, centroids, n_prefix: int, slack: int, m: int):
    """m-way posting lists over the first n_prefix keys of one (request, KV
    head), with `slack` free entries after each list.

    keys [N][d] (N = capacity in tokens; the lists hold N * m entries),
    centroids [C][d]. Requires n_prefix * m + C * slack <= N * m. Returns
    offsets [C+1], lens [C], ids [N*m] (-1 where free) and alt [N*m][m-1]
    (each valid entry's other lists, in the token's order of preference; -1
    where free).
    """
    K = np.asarray(keys)
    N = K.shape[0]
    C = np.asarray(centroids).shape[0]
    if not (1 <= m <= C and 1 <= n_prefix <= N and slack >= 0 and n_prefix * m + C * slack <= N * m):
        raise ValueError("need 1 <= m <= C, 1 <= n_prefix <= N and n_prefix * m + C * slack <= N * m")
    a, _ = nearest_centroids(K[:n_prefix], centroids, m)
    counts = np.bincount(a.ravel(), minlength=C)
    offsets = np.zeros(C + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts + slack)
    ids = np.full(N * m, -1, dtype=np.int64)
    alt = np.full((N * m, m - 1), -1, dtype=np.int64)
    for c in range(C):
        members = np.flatnonzero((a == c).any(axis=1))  # ascending token ids
        for j, t in enumerate(members):
            ids[offsets[c] + j] = t
            alt[offsets[c] + j] = [x for x in a[t] if x != c]
    return offsets, counts.astype(np.int64), ids, alt


def append_key_multi(offsets, lens, ids, alt, centroids, key, pos: int, m: int):
    """Add token `pos` to the lists of its m nearest centroids, all or
    nothing: when every one of them has a free entry the token is written at
    the end of each (with its other lists in `alt`); otherwise nothing
    changes. Returns (lists, inserted)."""
    a, _ = nearest_centroids(np.asarray(key)[None, :], centroids, m)
    lists = [int(c) for c in a[0]]
    if any(lens[c] >= offsets[c + 1] - offsets[c] for c in lists):
        return lists, False
    for c in lists:
        e = offsets[c] + lens[c]
        ids[e] = pos
        alt[e] = [x for x in lists if x != c]
        lens[c] += 1
    return lists, True


def regrow_slack(lens, capacity: int) -> int:
    """The largest number of free entries every list can get after its valid
    ones in `capacity` entries (negative when the valid entries alone do not
    fit)."""
    C = len(lens)
    return (capacity - int(np.sum(lens))) // C


def regrow(offsets, lens, ids, alt, slack: int):
    """The same lists laid out again with `slack` free entries after each:
    list c keeps its lens[c] valid entries, in order (and their alt rows),
    at offsets'[c] = sum over c' < c of (lens[c'] + slack). Returns
    (offsets', lens', ids', alt'); entries past the valid ones are -1.
    Requires sum(lens) + C * slack <= len(ids)."""
    lens = np.asarray(lens, dtype=np.int64)
    C = len(lens)
    cap = len(ids)
    if slack < 0 or int(lens.sum()) + C * slack > cap:
        raise ValueError("the valid entries plus the free entries do not fit")
    alt = np.asarray(alt)
    new_off = np.zeros(C + 1, dtype=np.int64)
    new_off[1:] = np.cumsum(lens + slack)
    new_ids = np.full(cap, -1, dtype=np.int64)
    new_alt = np.full(alt.shape, -1, dtype=np.int64)
    for c in range(C):
        n = int(lens[c])
        new_ids[new_off[c]:new_off[c] + n] = ids[offsets[c]:offsets[c] + n]
        new_alt[new_off[c]:new_off[c] + n] = alt[offsets[c]:offsets[c] + n]
    return new_off, lens.copy(), new_ids, new_alt


def append_step(state, new_k, new_v, pos, centroids, K, V):
    """One decode step's append for a batch.

    state: dict (b, g) -> (offsets, lens, ids) of the dynamic index, or
    (offsets, lens, ids, alt) of an m-way one (m = alt.shape[1] + 1);
    new_k, new_v [B][Hkv][d]; pos [B] (row of the new token per request);
    centroids [Bc][Hkv][C][d]; K, V [B][N][Hkv][d] (written in place).
    Returns status [B][Hkv]: 0 inserted, 1 a list full (row stored, not
    indexed), 2 position outside [0, N) (nothing stored).
    """
    new_k = np.asarray(new_k)
    B, Hkv, _ = new_k.shape
    N = K.shape[1]
    Cn = np.asarray(centroids)
    status = np.zeros((B, Hkv), dtype=np.int64)
    for b in range(B):
        p = int(pos[b])
        if not 0 <= p < N:
            status[b, :] = 2
            continue
        for g in range(Hkv):
            K[b, p, g] = new_k[b, g]
            V[b, p, g] = new_v[b, g]
            st = state[(b, g)]
            cb = Cn[0 if Cn.shape[0] == 1 else b, g]
            if len(st) == 4:
                offsets, lens, ids, alt = st
                _, ok = append_key_multi(offsets, lens, ids, alt, cb, new_k[b, g], p, alt.shape[1] + 1)
            else:
                offsets, lens, ids = st
                _, ok = append_key(offsets, lens, ids, cb, new_k[b, g], p)
            status[b, g] = 0 if ok else 1
    return status
