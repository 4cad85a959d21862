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
"""

from __future__ import annotations

import numpy as np

from .ivf import nearest_centroid

__all__ = ["index_build_dynamic", "append_key", "compact", "append_step"]


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


def append_step(state, new_k, new_v, pos, centroids, K, V):
    """One decode step's append for a batch.

    state: dict (b, g) -> (offsets, lens, ids) of the dynamic index;
    new_k, new_v [B][Hkv][d]; pos [B] (row of the new token per request);
    centroids [Bc][Hkv][C][d]; K, V [B][N][Hkv][d] (written in place).
    Returns status [B][Hkv]: 0 inserted, 1 list full (row stored, not indexed),
    2 position outside [0, N) (nothing stored).
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
            offsets, lens, ids = state[(b, g)]
            _, ok = append_key(offsets, lens, ids, Cn[0 if Cn.shape[0] == 1 else b, g], new_k[b, g], p)
            status[b, g] = 0 if ok else 1
    return status
