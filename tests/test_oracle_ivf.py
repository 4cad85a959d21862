"""Pins for the inverted-index oracle against what the pages and the
mathematics fix (closed forms, constructions with known answers, a library
routine for the dense special case, the KARAT worked example's counts)."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ivf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# index build
# ----------------------------------------------------------------------------

def _separated_centroids(rng, C, d, scale=10.0):
    return scale * rng.standard_normal((C, d))


def test_keys_on_centroids_land_in_their_own_list():
    rng = np.random.default_rng(0)
    C, d = 17, 8
    cent = _separated_centroids(rng, C, d)
    perm = rng.integers(0, C, size=200)
    a, margin = ivf.nearest_centroid(cent[perm], cent)
    assert np.array_equal(a, perm)
    assert np.all(np.isinf(margin))  # the key sits on its centroid: distance exactly 0


def test_perturbed_keys_keep_their_centroid():
    # A perturbation shorter than half the smallest centroid separation cannot
    # change the nearest centroid (triangle inequality).
    rng = np.random.default_rng(1)
    C, d = 23, 16
    cent = _separated_centroids(rng, C, d)
    sep = min(np.linalg.norm(cent[i] - cent[j]) for i in range(C) for j in range(i + 1, C))
    comp = rng.integers(0, C, size=500)
    noise = rng.standard_normal((500, d))
    noise *= (0.49 * sep * rng.random((500, 1))) / np.linalg.norm(noise, axis=1, keepdims=True)
    a, margin = ivf.nearest_centroid(cent[comp] + noise, cent)
    assert np.array_equal(a, comp)
    assert np.all(margin > 0)


def test_equidistant_key_goes_to_lower_centroid():
    cent = np.zeros((6, 3))
    cent[2] = [1.0, 0, 0]
    cent[5] = [-1.0, 0, 0]
    for i in (0, 1, 3, 4):
        cent[i] = [0, 100.0 + i, 0]
    a, margin = ivf.nearest_centroid(np.zeros((1, 3)), cent)
    assert a[0] == 2 and margin[0] == 0.0


def _exact_d2(x, c):
    """Squared distance of two fp64 vectors in exact rational arithmetic."""
    return sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(x, c))


@pytest.mark.parametrize("offset", [0.0, 1.0e6])
def test_near_ties_match_exact_rational_distances(offset):
    # Keys on the far side of the bisector of two centroids at relative
    # margins 1e-4 ... 1e-8, checked against brute-force distances in exact
    # rational arithmetic. With a common offset of 1e6 every |k|^2 and |c|^2
    # is ~1e14, so an expansion |k|^2 - 2k.c + |c|^2 alone would lose the
    # decision (its rounding is ~1e-2 against gaps of ~1e-7).
    rng = np.random.default_rng(21)
    C, d = 10, 48
    cent = offset + 10.0 * rng.standard_normal((C, d))
    keys, want_margin = [], []
    for r in (1e-4, 1e-5, 1e-6, 1e-7, 1e-8):
        for side in (1.0, -1.0):
            a, b = rng.choice(C, 2, replace=False)
            D = np.linalg.norm(cent[a] - cent[b])
            u = (cent[a] - cent[b]) / D
            w = rng.standard_normal(d)
            w -= (w @ u) * u
            w *= 3.0 / np.linalg.norm(w)
            t = r * (D * D / 4 + 9.0) / (2 * D)
            keys.append((cent[a] + cent[b]) / 2 + side * t * u + w)
            want_margin.append(r)
    keys = np.array(keys)
    a, margin = ivf.nearest_centroid(keys, cent)
    for i, x in enumerate(keys):
        d2 = [_exact_d2(x, c) for c in cent]
        best = min(range(C), key=lambda j: (d2[j], j))
        second = min((d2[j] for j in range(C) if j != best))
        exact_margin = float((second - d2[best]) / d2[best])
        assert a[i] == best
        assert 0.3 * want_margin[i] < exact_margin < 3 * want_margin[i]
        assert abs(margin[i] - exact_margin) <= 1e-4 * exact_margin


def test_nearest_candidates_cover_every_centroid_when_all_tie():
    # A key equidistant from every centroid: the direct sums all tie and the
    # lowest index wins, with a zero margin.
    C, d = 7, 5
    cent = np.zeros((C, d))
    for c in range(C):
        cent[c, c % d] = 2.0 if c < d else -2.0
    a, margin = ivf.nearest_centroid(np.zeros((3, d)), cent)
    assert np.array_equal(a, [0, 0, 0]) and np.all(margin == 0.0)


def test_squared_distance_not_dot_product():
    # The nearest centroid by distance differs from the one with the largest
    # dot product when norms differ: catches a distance replaced by a score.
    cent = np.array([[1.0, 0.0], [10.0, 0.0]])
    a, _ = ivf.nearest_centroid(np.array([[1.2, 0.0]]), cent)
    assert a[0] == 0


def test_posting_lists_invariants():
    rng = np.random.default_rng(2)
    C, n = 37, 1000
    assign = rng.integers(0, C - 3, size=n)  # some lists stay empty
    off, ids = ivf.posting_lists(assign, C)
    assert off[0] == 0 and off[-1] == n and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(ids), np.arange(n))           # every token exactly once
    for c in range(C):
        members = ids[off[c]:off[c + 1]]
        assert np.all(np.diff(members) > 0)                      # ascending ids
        assert np.all(assign[members] == c)
        assert len(members) == np.count_nonzero(assign == c)


def test_index_build_shared_and_per_request_codebooks():
    rng = np.random.default_rng(3)
    B, N, Hkv, C, d = 2, 64, 2, 5, 4
    cent = _separated_centroids(rng, C * B * Hkv, d).reshape(B, Hkv, C, d)
    comp = rng.integers(0, C, size=(B, N, Hkv))
    keys = np.empty((B, N, Hkv, d))
    for b in range(B):
        for g in range(Hkv):
            keys[b, :, g] = cent[b, g, comp[b, :, g]] + 0.01 * rng.standard_normal((N, d))
    off, ids, margins = ivf.index_build(keys, cent)
    for b in range(B):
        for g in range(Hkv):
            for c in range(C):
                assert set(ids[b, g, off[b, g, c]:off[b, g, c + 1]]) == set(np.nonzero(comp[b, :, g] == c)[0])
    # shared codebook: request 1 uses codebook 0
    off_s, ids_s, _ = ivf.index_build(keys[:1], cent[:1])
    assert np.array_equal(off_s[0], off[0]) and np.array_equal(ids_s[0], ids[0])


# ----------------------------------------------------------------------------
# scores and top-k
# ----------------------------------------------------------------------------

def test_scores_against_basis_queries():
    rng = np.random.default_rng(4)
    cent = rng.standard_normal((9, 6))
    for t in range(6):
        e = np.zeros(6)
        e[t] = 1.0
        assert np.array_equal(ivf.centroid_scores(e, cent), cent[:, t])


def test_scores_are_linear_in_the_query():
    rng = np.random.default_rng(5)
    cent = rng.integers(-8, 9, size=(11, 7)).astype(float)
    q1 = rng.integers(-8, 9, size=7).astype(float)
    q2 = rng.integers(-8, 9, size=7).astype(float)
    # integer lattice: every sum is exact in fp64
    assert np.array_equal(ivf.centroid_scores(3 * q1 - 2 * q2, cent),
                          3 * ivf.centroid_scores(q1, cent) - 2 * ivf.centroid_scores(q2, cent))


def _rank_count_selection(s, k):
    """Selected iff fewer than k scores beat it (greater, or equal with a lower index)."""
    n = len(s)
    return [i for i in range(n)
            if sum(1 for j in range(n) if s[j] > s[i] or (s[j] == s[i] and j < i)) < k]


@pytest.mark.parametrize("seed", range(20))
def test_top_k_matches_rank_counting(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    k = int(rng.integers(1, n + 1))
    s = rng.integers(-4, 5, size=n).astype(float)  # many ties
    assert list(ivf.top_k(s, k)) == _rank_count_selection(list(s), k)


def test_top_k_special_cases():
    s = np.array([3.0, 5.0, 5.0, 1.0, 5.0])
    assert list(ivf.top_k(s, 2)) == [1, 2]          # ties -> lower index
    assert list(ivf.top_k(s, 5)) == [0, 1, 2, 3, 4]  # k = n selects all
    rng = np.random.default_rng(6)
    x = rng.standard_normal(100)
    assert list(ivf.top_k(x, 1)) == [int(np.argmax(x))]
    with pytest.raises(ValueError):
        ivf.top_k(s, 0)
    with pytest.raises(ValueError):
        ivf.top_k(s, 6)


def test_selection_gap():
    assert ivf.selection_gap([10.0, 8.0, 4.0], 2) == pytest.approx((8 - 4) / 8)
    assert ivf.selection_gap([1.0, 1.0], 1) == 0.0
    assert ivf.selection_gap([1.0, 2.0], 2) == math.inf
    assert ivf.selection_gap([-1.0, -3.0], 1) == pytest.approx(2 / 3)


# ----------------------------------------------------------------------------
# attention (Eq. 2 with the -inf mask reading)
# ----------------------------------------------------------------------------

def _sdpa_masked(q, K, V, keep):
    """torch's fp64 CPU scaled-dot-product attention with a boolean mask."""
    qt = torch.from_numpy(q)[None, None, None, :]
    Kt = torch.from_numpy(K)[None, None]
    Vt = torch.from_numpy(V)[None, None]
    mask = torch.from_numpy(keep)[None, None, None, :]
    return torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mask)[0, 0, 0].numpy()


def test_attend_equals_masked_library_attention():
    rng = np.random.default_rng(7)
    N, d = 300, 128
    q = rng.standard_normal(d)
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    keep = rng.random(N) < 0.2
    o, p = ivf.attend(q, K[keep], V[keep])
    np.testing.assert_allclose(o, _sdpa_masked(q, K, V, keep), rtol=1e-12, atol=1e-13)


def test_attend_probability_properties():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(128)
    K = 3 * rng.standard_normal((50, 128))
    V = rng.standard_normal((50, 128))
    o, p = ivf.attend(q, K, V)
    assert np.all(p >= 0) and abs(p.sum() - 1) < 1e-14
    perm = rng.permutation(50)
    o2, _ = ivf.attend(q, K[perm], V[perm])
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)


def test_attend_degenerate_cases():
    rng = np.random.default_rng(9)
    q = rng.standard_normal(128)
    V = rng.standard_normal((7, 128))
    o, p = ivf.attend(q, rng.standard_normal((1, 128)), V[:1])
    assert np.array_equal(o, V[0]) and p[0] == 1.0                 # one row -> that row
    Ksame = np.repeat(rng.standard_normal((1, 128)), 7, axis=0)
    o, _ = ivf.attend(q, Ksame, V)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-13, atol=1e-14)  # equal logits -> mean
    o, p = ivf.attend(q, np.empty((0, 128)), np.empty((0, 128)))
    assert np.array_equal(o, np.zeros(128)) and p.size == 0        # empty set -> zeros
    Kbig = 1e4 * rng.standard_normal((7, 128))                        # no overflow
    o, p = ivf.attend(q, Kbig, V)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, V[np.argmax(Kbig @ q)], rtol=1e-9)


def test_attend_scale_is_inverse_sqrt_dk():
    # Two rows whose logits differ by exactly sqrt(d) * ln 3 give weights 3:1.
    d = 64
    q = np.zeros(d)
    q[0] = 1.0
    K = np.zeros((2, d))
    K[0, 0] = math.sqrt(d) * math.log(3.0)
    V = np.array([[1.0] * d, [0.0] * d])
    o, p = ivf.attend(q, K, V)
    np.testing.assert_allclose(p, [0.75, 0.25], rtol=1e-14)


# ----------------------------------------------------------------------------
# whole decode query
# ----------------------------------------------------------------------------

def _clustered(rng, N, C, d, sd=0.3):
    cent = rng.standard_normal((C, d))
    comp = rng.integers(0, C, size=N)
    return cent, cent[comp] + sd * rng.standard_normal((N, d))


def test_selecting_every_list_is_dense_attention():
    rng = np.random.default_rng(10)
    N, C, d = 512, 8, 128
    cent, K = _clustered(rng, N, C, d)
    V = rng.standard_normal((N, d))
    a, _ = ivf.nearest_centroid(K, cent)
    off, ids = ivf.posting_lists(a, C)
    q = cent[3] + 0.3 * rng.standard_normal(d)
    r = ivf.decode_head(q, cent, off, ids, K, V, k=C)
    assert len(r.rows) == N
    np.testing.assert_allclose(r.out, _sdpa_masked(q, K, V, np.ones(N, bool)), rtol=1e-12, atol=1e-13)


def test_decode_head_is_masked_attention_over_chosen_lists():
    rng = np.random.default_rng(11)
    N, C, d, k = 1024, 16, 128, 3
    cent, K = _clustered(rng, N, C, d)
    V = rng.standard_normal((N, d))
    a, _ = ivf.nearest_centroid(K, cent)
    off, ids = ivf.posting_lists(a, C)
    q = cent[5] + 0.3 * rng.standard_normal(d)
    r = ivf.decode_head(q, cent, off, ids, K, V, k=k)
    keep = np.isin(a, r.lists)
    assert np.array_equal(r.rows, np.nonzero(keep)[0])
    np.testing.assert_allclose(r.out, _sdpa_masked(q, K, V, keep), rtol=1e-12, atol=1e-13)
    assert 5 in r.lists  # the query sits on centroid 5


def test_karat_worked_example_counts():
    """The oracle's counters reproduce the worked example's multiply-add counts
    on an index of its shape: C=1000 centroids, d=128, the query's top-10 lists
    holding 1000 entries each, 100K tokens in total."""
    g = json.load(open(os.path.join(GOLDEN, "karat_worked_example.json")))
    N, d, C, k, per = (g["context_tokens"], g["d_k"], g["n_centroids"], g["top_lists"],
                       g["entries_per_list"])
    rng = np.random.default_rng(12)
    cent = rng.standard_normal((C, d))
    q = rng.standard_normal(d)
    top = ivf.top_k(ivf.centroid_scores(q, cent), k)
    others = np.setdiff1d(np.arange(C), top)
    assign = np.empty(N, dtype=np.int64)
    assign[: k * per] = np.repeat(top, per)
    assign[k * per:] = rng.choice(others, size=N - k * per)
    rng.shuffle(assign)
    off, ids = ivf.posting_lists(assign, C)
    K = rng.standard_normal((N, d)).astype(np.float32)
    V = rng.standard_normal((N, d)).astype(np.float32)
    r = ivf.decode_head(q, cent, off, ids, K, V, k=k)
    c = r.counts
    assert list(r.lists) == list(top)
    assert len(r.rows) == g["scanned_entries"]
    assert c.retrieve == g["retrieve_macs"]
    assert c.score == g["score_macs"]
    assert c.output == g["output_macs"]
    assert c.full_score == g["full_attention_macs"]
    # the page's illustrative timings follow from the counts at 1 MAC per ns
    ns = g["ns_per_mac"]
    assert c.retrieve * ns / 1e3 == pytest.approx(g["t_retrieve_us"])
    assert c.score * ns / 1e6 == pytest.approx(g["t_score_ms"])
    assert c.output * ns / 1e6 == pytest.approx(g["t_output_ms"])
    assert (c.score + c.output) * ns / 1e6 == pytest.approx(g["t_attn_ms"])
    t_send_ns = g["q_bytes"] / g["link_bytes_per_s"] * 1e9
    assert t_send_ns == pytest.approx(g["t_send_ns"])
    total_ms = (g["t_proj_us"] * 1e3 + t_send_ns + c.retrieve * ns + (c.score + c.output) * ns
                + g["t_moe_us"] * 1e3) / 1e6
    assert round(total_ms, 2) == g["t_total_ms_printed"]
    assert c.full_score * ns / 1e6 == pytest.approx(g["t_full_ms"])
    assert 9.5 < c.full_score / c.score < 10.5   # "about 10x"


def test_work_scales_with_selection_not_context():
    # O(k) per step: doubling the context at fixed selection leaves score and
    # output work unchanged while the full-attention count doubles.
    rng = np.random.default_rng(13)
    d, C = 32, 10
    cent = rng.standard_normal((C, d))
    q = rng.standard_normal(d)
    top = ivf.top_k(ivf.centroid_scores(q, cent), 2)
    counts = []
    for N in (400, 800):
        assign = np.where(np.arange(N) < 100, top[np.arange(N) % 2],
                          np.setdiff1d(np.arange(C), top)[np.arange(N) % (C - 2)])
        off, ids = ivf.posting_lists(assign, C)
        K = rng.standard_normal((N, d))
        r = ivf.decode_head(q, cent, off, ids, K, K, k=2)
        counts.append(r.counts)
    assert counts[0].score == counts[1].score == 100 * d
    assert counts[1].full_score == 2 * counts[0].full_score


def test_sparse_decode_batch_layout_and_gqa():
    rng = np.random.default_rng(14)
    B, N, Hkv, G, C, d, k = 2, 256, 2, 2, 8, 16, 2
    cent = rng.standard_normal((1, Hkv, C, d))
    K = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    off, ids, _ = ivf.index_build(K, cent)
    q = rng.standard_normal((B, Hkv * G, d))
    res = ivf.sparse_decode(q, cent, off, ids, K, V, k)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            r = ivf.decode_head(q[b, h], cent[0, g], off[b, g], ids[b, g], K[b, :, g], V[b, :, g], k)
            assert np.array_equal(res["out"][b, h], r.out)
            assert np.array_equal(res["sel"][b, h], r.lists)
    part = ivf.sparse_decode(q, cent, off, ids, K, V, k, heads=[(1, 3)])
    assert np.array_equal(part["out"][1, 3], res["out"][1, 3])
    assert np.isnan(part["out"][0, 0]).all()


def test_gqa_groups_are_contiguous_query_heads():
    # Query head h must read KV head h div (Hq/Hkv): contiguous groups. Each
    # of the three reads is pinned by a construction whose output names the
    # KV head it came from (Hq = 8, Hkv = 2; the interleaved reading h mod Hkv
    # gives 0,1,0,1,... and fails).
    B, N, Hkv, G, d = 1, 16, 2, 4, 8
    Hq = Hkv * G
    want = np.arange(Hq) // G
    e0 = np.zeros(d)
    e0[0] = 1.0
    q = np.broadcast_to(e0, (B, Hq, d)).copy()
    # (1) centroids: KV head g's codebook puts list g far ahead of the others.
    cent = np.full((1, Hkv, Hkv, d), 0.0)
    for g in range(Hkv):
        cent[0, g, :, 0] = -10.0
        cent[0, g, g, 0] = 10.0
    K = np.zeros((B, N, Hkv, d))
    V = np.zeros((B, N, Hkv, d))
    off, ids, _ = ivf.index_build(K, cent)
    res = ivf.sparse_decode(q, cent, off, ids, K, V, 1)
    assert np.array_equal(res["sel"][0, :, 0], want)
    # (2) keys: every list chosen (dense); KV head g's only large logit is
    # token g, and V row i holds the value i in every KV head.
    K = np.zeros((B, N, Hkv, d))
    for g in range(Hkv):
        K[0, g, g, 0] = 1000.0 * math.sqrt(d)
    V = np.broadcast_to(np.arange(N, dtype=float)[None, :, None, None], (B, N, Hkv, d)).copy()
    off, ids, _ = ivf.index_build(K, cent)
    res = ivf.sparse_decode(q, cent, off, ids, K, V, Hkv)
    assert np.array_equal(res["out"][0], np.broadcast_to(want[:, None].astype(float), (Hq, d)))
    # (3) values: uniform weights (all keys zero) over N = 16 rows, KV head g's
    # values all equal g; the mean is exact in binary.
    K = np.zeros((B, N, Hkv, d))
    V = np.broadcast_to(np.arange(Hkv, dtype=float)[None, None, :, None], (B, N, Hkv, d)).copy()
    off, ids, _ = ivf.index_build(K, cent)
    res = ivf.sparse_decode(q, cent, off, ids, K, V, Hkv)
    assert np.array_equal(res["out"][0], np.broadcast_to(want[:, None].astype(float), (Hq, d)))
