"""Pins of the decode variants: cosine similarity ([KARAT] worked example,
step 3) and sink/window rows beside the lists ([KARAT] method details:
window-based sparse attention such as StreamingLLM)."""

import math

import numpy as np
import pytest
import torch

from oracle import ivf, variants


def _clustered(rng, N, C, d, sd=0.3):
    cent = rng.standard_normal((C, d))
    lab = rng.integers(0, C, N)
    return cent, cent[lab] + sd * rng.standard_normal((N, d))


def test_cosine_equals_dot_on_unit_centroids():
    rng = np.random.default_rng(1)
    C, d = 50, 16
    cent = rng.standard_normal((C, d))
    unit = cent / np.linalg.norm(cent, axis=1, keepdims=True)
    q = rng.standard_normal(d)
    assert np.allclose(variants.cosine_scores(q, unit), unit @ q, rtol=0, atol=1e-14)
    # and cosine of the raw codebook is the dot score of the normalised one
    assert np.allclose(variants.cosine_scores(q, cent), unit @ q, rtol=0, atol=1e-14)


def test_cosine_ignores_centroid_scale_but_dot_does_not():
    rng = np.random.default_rng(2)
    C, d, k = 40, 8, 5
    cent = rng.standard_normal((C, d))
    q = rng.standard_normal(d)
    top = set(ivf.top_k(cent @ q, k).tolist())
    low = next(int(c) for c in np.argsort(-(cent @ q)) if c not in top and cent[c] @ q > 0)
    scaled = cent.copy()
    scaled[low] *= 50.0                      # a positive-score centroid outside the top-k
    assert np.array_equal(ivf.top_k(variants.cosine_scores(q, scaled), k), ivf.top_k(variants.cosine_scores(q, cent), k))
    assert low in ivf.top_k(scaled @ q, k)


def test_cosine_closed_forms():
    c = np.array([[3.0, 4.0], [0.0, 0.0], [-1.0, 0.0]])
    q = np.array([1.0, 0.0])
    assert np.allclose(variants.cosine_scores(q, c), [0.6, 0.0, -1.0], atol=1e-15)


def test_fixed_rows_ranges_and_union():
    assert variants.fixed_rows(4, 3, 20).tolist() == [0, 1, 2, 3, 17, 18, 19]
    assert variants.fixed_rows(4, 0, 20).tolist() == [0, 1, 2, 3]
    assert variants.fixed_rows(0, 3, 20).tolist() == [17, 18, 19]
    assert variants.fixed_rows(5, 5, 8).tolist() == list(range(8))      # overlap: each token once
    assert variants.fixed_rows(30, 0, 8).tolist() == list(range(8))     # clipped to the length
    assert variants.fixed_rows(0, 0, 8).tolist() == []


def _masked_dense(q, K, V, keep):
    z = torch.from_numpy(K) @ torch.from_numpy(q) / math.sqrt(K.shape[1])
    z = torch.where(torch.from_numpy(keep), z, torch.tensor(-math.inf, dtype=torch.float64))
    p = torch.softmax(z, dim=0)
    return (p @ torch.from_numpy(V)).numpy()


@pytest.mark.parametrize("sim", ["dot", "cosine"])
def test_decode_with_sink_and_window_is_masked_attention_over_the_union(sim):
    rng = np.random.default_rng(3)
    N, C, d, k = 400, 12, 16, 3
    cent, K = _clustered(rng, N, C, d)
    V = rng.standard_normal((N, d))
    off, ids = ivf.posting_lists(ivf.nearest_centroid(K, cent)[0], C)
    q = cent[5] + 0.2 * rng.standard_normal(d)
    L = 350
    o, lists, rows, _ = variants.decode_head_ex(q, cent, off, ids, K, V, k, similarity=sim, n_sink=10,
                                                n_window=25, length=L)
    keep = np.zeros(N, dtype=bool)
    for c in lists:
        keep[ids[off[c]:off[c + 1]]] = True
    keep[:10] = True
    keep[L - 25:L] = True
    assert np.array_equal(rows, np.flatnonzero(keep))
    assert np.allclose(o, _masked_dense(q, K, V, keep), rtol=0, atol=1e-12)


def test_sink_covering_the_context_is_dense_attention():
    rng = np.random.default_rng(4)
    N, C, d = 120, 6, 8
    cent, K = _clustered(rng, N, C, d)
    V = rng.standard_normal((N, d))
    off, ids = ivf.posting_lists(ivf.nearest_centroid(K, cent)[0], C)
    q = rng.standard_normal(d)
    o, _, rows, _ = variants.decode_head_ex(q, cent, off, ids, K, V, 1, n_sink=N)
    assert np.array_equal(rows, np.arange(N))
    assert np.allclose(o, _masked_dense(q, K, V, np.ones(N, dtype=bool)), rtol=0, atol=1e-12)


def test_no_variant_is_the_plain_decode():
    rng = np.random.default_rng(5)
    N, C, d, k = 300, 10, 8, 2
    cent, K = _clustered(rng, N, C, d)
    V = rng.standard_normal((N, d))
    off, ids = ivf.posting_lists(ivf.nearest_centroid(K, cent)[0], C)
    q = rng.standard_normal(d)
    o, lists, rows, _ = variants.decode_head_ex(q, cent, off, ids, K, V, k)
    r = ivf.decode_head(q, cent, off, ids, K, V, k)
    assert np.array_equal(lists, r.lists) and np.array_equal(rows, r.rows)
    assert np.array_equal(o, r.out)


def test_nearest_centroids_brute_force_and_m1():
    rng = np.random.default_rng(8)
    C, d = 9, 6
    cent = rng.standard_normal((C, d))
    keys = rng.standard_normal((40, d))
    a, gap = variants.nearest_centroids(keys, cent, 3)
    for i in range(40):
        d2 = [float(np.sum((keys[i] - cent[c]) ** 2)) for c in range(C)]
        order = sorted(range(C), key=lambda c: (d2[c], c))
        assert a[i].tolist() == order[:3]
    # m = 1 is the plain assignment
    a1, _ = variants.nearest_centroids(keys, cent, 1)
    assert np.array_equal(a1[:, 0], ivf.nearest_centroid(keys, cent)[0])
    # ties go to the lower index: a key midway between centroids 0 and 1
    c2 = np.array([[1.0, 0.0], [-1.0, 0.0], [0.0, 5.0]])
    a2, _ = variants.nearest_centroids(np.array([[0.0, 0.0]]), c2, 2)
    assert a2[0].tolist() == [0, 1]


@pytest.mark.parametrize("m", [2, 3, 4])
def test_multi_assignment_lists_and_dedup_in_the_union(m):
    rng = np.random.default_rng(9)
    N, C, d = 300, 10, 8
    cent, K = _clustered(rng, N, C, d)
    V = rng.standard_normal((N, d))
    a, _ = variants.nearest_centroids(K, cent, m)
    off, ids, alt = variants.posting_lists_multi(a, C)
    assert off[-1] == N * m
    for c in range(C):
        lst = ids[off[c]:off[c + 1]]
        assert np.all(np.diff(lst) > 0)                          # ascending, each token once per list
        assert np.array_equal(np.sort(lst), np.flatnonzero((a == c).any(axis=1)))
        for e in range(off[c], off[c + 1]):                       # alt names the token's other list
            assert set(alt[e].tolist()) | {c} == set(a[ids[e]].tolist())
    # every token appears in exactly m lists
    assert np.array_equal(np.bincount(ids, minlength=N), np.full(N, m))
    # the decode attends the union once: masked attention over it
    q = cent[3] + 0.1 * rng.standard_normal(d)
    o, lists, rows, _ = variants.decode_head_ex(q, cent, off, ids, K, V, 3)
    keep = np.zeros(N, dtype=bool)
    for c in lists:
        keep[ids[off[c]:off[c + 1]]] = True
    assert np.array_equal(rows, np.flatnonzero(keep))
    assert np.allclose(o, _masked_dense(q, K, V, keep), rtol=0, atol=1e-12)


@pytest.mark.parametrize("sim", ["dot", "cosine"])
def test_variant_decode_gqa_groups_are_contiguous_query_heads(sim):
    # Query head h reads KV head h div (Hq/Hkv): KV head g's codebook puts
    # list g first (its selection names g), and with zero keys over N = 16
    # rows whose values equal the KV head's index, the output does too. The
    # interleaved reading h mod Hkv gives 0,1,0,1,... and fails.
    B, N, Hkv, G, d = 1, 16, 2, 4, 8
    Hq = Hkv * G
    want = np.arange(Hq) // G
    q = np.zeros((B, Hq, d))
    q[..., 0] = 1.0
    cent = np.zeros((1, Hkv, Hkv, d))
    for g in range(Hkv):
        cent[0, g, :, 0] = -10.0
        cent[0, g, g, 0] = 10.0
    K = np.zeros((B, N, Hkv, d))
    V = np.broadcast_to(np.arange(Hkv, dtype=float)[None, None, :, None], (B, N, Hkv, d)).copy()
    off, ids, _ = ivf.index_build(K, cent)
    res = variants.sparse_decode_ex(q, cent, off, ids, K, V, 1, similarity=sim)
    assert np.array_equal(res["sel"][0, :, 0], want)
    res = variants.sparse_decode_ex(q, cent, off, ids, K, V, Hkv, similarity=sim)
    assert np.array_equal(res["out"][0], np.broadcast_to(want[:, None].astype(float), (Hq, d)))
