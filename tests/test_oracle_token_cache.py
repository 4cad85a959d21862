"""Pins for the token-indexer oracle and the hierarchical-cache (LRU) oracle."""

from collections import OrderedDict

import numpy as np
import pytest
import torch

from oracle import cache, ivf, token
from top_sparse_attention_centroid_amd import workloads as W


# ----------------------------------------------------------------------------
# token indexer
# ----------------------------------------------------------------------------

def test_indexer_scores_basis_and_lattice():
    rng = np.random.default_rng(0)
    kidx = rng.integers(-16, 17, size=(50, 64)).astype(float)
    e = np.zeros(64)
    e[9] = 1.0
    assert np.array_equal(token.indexer_scores(e, kidx), kidx[:, 9])
    q = rng.integers(-16, 17, size=64).astype(float)
    brute = [sum(int(q[t]) * int(kidx[i, t]) for t in range(64)) for i in range(50)]
    assert np.array_equal(token.indexer_scores(q, kidx), np.array(brute, dtype=float))


def test_token_topk_lattice_ties_prefer_lower_ids():
    # integer scores with many exact ties: rank counting decides
    rng = np.random.default_rng(1)
    kidx = rng.integers(-2, 3, size=(300, 4)).astype(float)
    q = np.array([1.0, 1.0, 0.0, 0.0])
    s = kidx @ q
    sel, _ = token.token_topk(q, kidx, 40)
    expect = [i for i in range(300) if sum(1 for j in range(300) if s[j] > s[i] or (s[j] == s[i] and j < i)) < 40]
    assert list(sel) == expect


def test_planted_tokens_are_all_selected():
    cfg = W.config(3, batch=2, n_tokens=20_000, top_k=512, n_planted=64, steps=2)
    prob = W.token_problem(cfg)
    q_idx, q = W.token_queries(cfg, prob)
    k_idx = prob["k_idx"].double().numpy()
    for t in range(cfg.steps):
        for b in range(cfg.batch):
            sel, gap = token.token_topk(q_idx[t, b].double().numpy(), k_idx[b], cfg.top_k)
            assert set(prob["planted"][b].tolist()) <= set(sel.tolist())
            assert np.all(np.diff(sel) > 0)


def test_token_decode_full_selection_is_dense_attention():
    rng = np.random.default_rng(2)
    B, N, Hkv, G, d, di = 1, 200, 2, 2, 32, 8
    K = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    kidx = rng.standard_normal((B, N, di))
    qidx = rng.standard_normal((B, di))
    q = rng.standard_normal((B, Hkv * G, d))
    res = token.token_decode(qidx, kidx, q, K, V, k=N)
    for h in range(Hkv * G):
        g = h // G
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, h])[None, None, None], torch.from_numpy(K[0, :, g])[None, None],
            torch.from_numpy(V[0, :, g])[None, None])[0, 0, 0].numpy()
        np.testing.assert_allclose(res["out"][0, h], ref, rtol=1e-12, atol=1e-13)


def test_token_decode_uses_one_selection_for_all_heads():
    rng = np.random.default_rng(3)
    B, N, Hkv, G, d, di, k = 2, 300, 2, 4, 16, 8, 20
    K = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    kidx = rng.standard_normal((B, N, di))
    qidx = rng.standard_normal((B, di))
    q = rng.standard_normal((B, Hkv * G, d))
    res = token.token_decode(qidx, kidx, q, K, V, k)
    for b in range(B):
        rows = res["sel"][b]
        assert list(rows) == list(ivf.top_k(kidx[b] @ qidx[b], k))
        for h in range(Hkv * G):
            o, _ = ivf.attend(q[b, h], K[b, rows, h // G], V[b, rows, h // G])
            assert np.array_equal(res["out"][b, h], o)


# ----------------------------------------------------------------------------
# LRU / RESOLVE
# ----------------------------------------------------------------------------

def _check_state(st: cache.CacheState, sel, t):
    pt, tok, lu = st.page_table, st.slot_token, st.last_use
    res_tokens = np.nonzero(pt >= 0)[0]
    assert np.array_equal(tok[pt[res_tokens]], res_tokens)          # inverse maps
    used = np.nonzero(tok >= 0)[0]
    assert np.array_equal(pt[tok[used]], used)
    assert np.all(pt[np.asarray(sel)] >= 0)                           # all selected resident
    assert np.all(lu[pt[np.asarray(sel)]] == t)
    assert np.all(lu <= t) and np.all((lu >= 0) == (tok >= 0))


def test_token_decode_gqa_groups_are_contiguous_query_heads():
    # Query head h reads KV head h div (Hq/Hkv). Keys: KV head g's only large
    # logit is token g, and V row i holds i, so head h's output names the KV
    # head its keys came from. Values: zero keys give uniform weights over
    # N = 16 rows and KV head g's values all equal g. The interleaved reading
    # h mod Hkv gives 0,1,0,1,... and fails both.
    B, N, Hkv, G, d, di = 1, 16, 2, 4, 8, 4
    Hq = Hkv * G
    want = (np.arange(Hq) // G).astype(float)
    q_idx = np.ones((B, di))
    k_idx = np.zeros((B, N, di))
    q = np.zeros((B, Hq, d))
    q[..., 0] = 1.0
    K = np.zeros((B, N, Hkv, d))
    for g in range(Hkv):
        K[0, g, g, 0] = 1000.0 * np.sqrt(d)
    V = np.broadcast_to(np.arange(N, dtype=float)[None, :, None, None], (B, N, Hkv, d)).copy()
    res = token.token_decode(q_idx, k_idx, q, K, V, N)
    assert np.array_equal(res["out"][0], np.broadcast_to(want[:, None], (Hq, d)))
    K = np.zeros((B, N, Hkv, d))
    V = np.broadcast_to(np.arange(Hkv, dtype=float)[None, None, :, None], (B, N, Hkv, d)).copy()
    res = token.token_decode(q_idx, k_idx, q, K, V, N)
    assert np.array_equal(res["out"][0], np.broadcast_to(want[:, None], (Hq, d)))


def test_attend_slots_gqa_groups_are_contiguous_query_heads():
    # The same two constructions through the hot pool (slot s holds token s).
    S, Hkv, G, d = 16, 2, 4, 8
    Hq = Hkv * G
    want = np.broadcast_to((np.arange(Hq) // G).astype(float)[:, None], (Hq, d))
    q = np.zeros((Hq, d))
    q[:, 0] = 1.0
    slots = np.arange(S)
    pk = np.zeros((S, Hkv, d))
    for g in range(Hkv):
        pk[g, g, 0] = 1000.0 * np.sqrt(d)
    pv = np.broadcast_to(np.arange(S, dtype=float)[:, None, None], (S, Hkv, d)).copy()
    assert np.array_equal(cache.attend_slots(q, pk, pv, slots), want)
    pk = np.zeros((S, Hkv, d))
    pv = np.broadcast_to(np.arange(Hkv, dtype=float)[None, :, None], (S, Hkv, d)).copy()
    assert np.array_equal(cache.attend_slots(q, pk, pv, slots), want)


def test_first_step_misses_everything_and_fills_free_slots_in_order():
    st = cache.CacheState(100, 8)
    slots, hits, misses, fetches = cache.lru_step(st, [40, 3, 77, 12], 0)
    assert hits == 0 and misses == 4
    assert fetches == [(3, 0), (12, 1), (40, 2), (77, 3)]             # ascending tokens -> free slots
    assert list(slots) == [2, 0, 3, 1]                                # reported in selection order
    _check_state(st, [40, 3, 77, 12], 0)


def test_victim_order_is_last_use_then_slot():
    st = cache.CacheState(100, 4)
    cache.lru_step(st, [10, 20], 0)          # slots 0, 1
    cache.lru_step(st, [30, 40], 1)          # free slots 2, 3
    _, h, m, f = cache.lru_step(st, [50], 2)  # oldest stamp 0 at slots 0,1 -> slot 0
    assert (h, m, f) == (0, 1, [(50, 0)])
    assert st.page_table[10] == -1 and st.page_table[20] == 1
    _, h, m, f = cache.lru_step(st, [20, 60, 70], 3)  # 20 hits (protected); victims: slot 2, then 3
    assert (h, m) == (1, 2) and f == [(60, 2), (70, 3)]
    _check_state(st, [20, 60, 70], 3)


def test_pool_equal_to_selection_misses_exactly_the_new_tokens():
    # With as many slots as selected tokens the resident set after a step is
    # that step's selection, so misses_t = |S_t \ S_{t-1}| (= k - overlap).
    cfg = W.config(4, batch=2, n_tokens=5000, top_k=200, overlap=170, n_slots=200, steps=12)
    trace = W.selection_trace(cfg).numpy()
    for b in range(cfg.batch):
        st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
        for t in range(cfg.steps):
            _, h, m, _ = cache.lru_step(st, trace[t, b], t)
            assert m == (cfg.top_k if t == 0 else cfg.top_k - cfg.overlap)
            assert h + m == cfg.top_k
            _check_state(st, trace[t, b], t)


def test_pool_covering_context_never_evicts():
    cfg = W.config(4, batch=1, n_tokens=600, top_k=64, overlap=40, n_slots=600, steps=15)
    trace = W.selection_trace(cfg).numpy()
    st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
    seen = set()
    for t in range(cfg.steps):
        _, h, m, _ = cache.lru_step(st, trace[t, 0], t)
        assert m == len(set(trace[t, 0].tolist()) - seen)
        seen |= set(trace[t, 0].tolist())


def test_single_token_steps_match_textbook_lru():
    # With one token per step there are no ties inside a step: the batch-step
    # policy must be the classic LRU cache.
    rng = np.random.default_rng(5)
    N, S = 40, 7
    st = cache.CacheState(N, S)
    ref = OrderedDict()
    for t in range(400):
        tok = int(rng.integers(0, N))
        _, h, m, _ = cache.lru_step(st, [tok], t)
        if tok in ref:
            ref.move_to_end(tok)
            ref_hit = True
        else:
            if len(ref) == S:
                ref.popitem(last=False)
            ref[tok] = True
            ref_hit = False
        assert (h == 1) == ref_hit
        assert set(np.nonzero(st.page_table >= 0)[0].tolist()) == set(ref.keys())


def test_evictions_respect_recency():
    cfg = W.config(4, batch=1, n_tokens=3000, top_k=128, overlap=100, n_slots=300, steps=30)
    trace = W.selection_trace(cfg).numpy()
    st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
    for t in range(cfg.steps):
        before = st.copy()
        sel = trace[t, 0]
        _, _, _, fetches = cache.lru_step(st, sel, t)
        evicted_slots = [v for _, v in fetches if before.slot_token[v] >= 0]
        kept = [s for s in range(cfg.n_slots) if before.slot_token[s] >= 0 and s not in evicted_slots
                and before.slot_token[s] not in set(sel.tolist())]
        for v in evicted_slots:
            for s in kept:
                assert (before.last_use[v], v) < (before.last_use[s], s)


def test_checkpoint_resume_reproduces_the_rest():
    cfg = W.config(4, batch=1, n_tokens=4000, top_k=128, overlap=109, n_slots=256, steps=20)
    trace = W.selection_trace(cfg).numpy()
    st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
    for t in range(8):
        cache.lru_step(st, trace[t, 0], t)
    snap = st.copy()
    a = [cache.lru_step(st, trace[t, 0], t)[:3] for t in range(8, 20)]
    b = [cache.lru_step(snap, trace[t, 0], t)[:3] for t in range(8, 20)]
    for x, y in zip(a, b):
        assert np.array_equal(x[0], y[0]) and x[1:] == y[1:]
    assert np.array_equal(st.page_table, snap.page_table)


def test_flush_makes_next_step_miss_everything():
    cfg = W.config(4, batch=1, n_tokens=4000, top_k=128, overlap=109, n_slots=256, steps=6)
    trace = W.selection_trace(cfg).numpy()
    st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
    for t in range(5):
        cache.lru_step(st, trace[t, 0], t)
    st = cache.CacheState(cfg.n_tokens, cfg.n_slots)  # disposable: host copy is authoritative
    _, h, m, _ = cache.lru_step(st, trace[5, 0], 5)
    assert (h, m) == (0, cfg.top_k)


def test_cache_mediated_attention_is_exact():
    """Attention over the hot slots equals attention over the host rows of the
    same selection: only placement changes (HiSparse exactness)."""
    cfg = W.config(4, batch=1, n_tokens=3000, top_k=256, overlap=218, n_slots=512, steps=6,
                   n_kv_heads=2, n_q_heads=8, head_dim=32)
    prob = W.cache_problem(cfg)
    K = prob["keys"][0].double().numpy()
    V = prob["values"][0].double().numpy()
    pool_k = np.zeros((cfg.n_slots, cfg.n_kv_heads, cfg.head_dim))
    pool_v = np.zeros_like(pool_k)
    st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
    for t in range(cfg.steps):
        sel = prob["trace"][t, 0].numpy()
        slots, _, _, fetches = cache.lru_step(st, sel, t)
        cache.fetch_rows(pool_k, pool_v, K, V, fetches)
        assert np.array_equal(pool_k[slots], K[sel]) and np.array_equal(pool_v[slots], V[sel])
        q = prob["q"][t, 0].double().numpy()
        o_cache = cache.attend_slots(q, pool_k, pool_v, slots)
        o_direct = cache.attend_slots(q, K, V, sel)
        np.testing.assert_allclose(o_cache, o_direct, rtol=1e-15, atol=1e-15)


def test_more_misses_than_slots_is_an_error():
    st = cache.CacheState(10, 2)
    with pytest.raises(ValueError):
        cache.lru_step(st, [1, 2, 3], 0)


def test_capacity_ratio_matches_the_hisparse_figures():
    """HiSparse analysis: at 128K context with B = 4096 slots the per-request KV
    falls from 13.09 GB to about 0.4 GB (~30x). The slot pool is B/N of the
    full KV whatever the model's per-token size."""
    cfg = W.config(4)
    frac = cfg.n_slots / cfg.n_tokens
    assert frac == 1 / 32
    assert 13.09 * frac == pytest.approx(0.409, abs=0.001)
