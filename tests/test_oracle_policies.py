"""Pins of the replacement policies of the hot cache ([HISPARSE-NEWS] compares
LRU, FIFO, random and offline Belady by miss rate)."""

import collections
import json
import os

import numpy as np
import pytest

from oracle import cache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_state0.json")


def test_splitmix64_reference_outputs():
    ref = [int(h, 16) for h in json.load(open(GOLDEN))["state0_outputs_hex"]]
    state, got = 0, []
    for _ in range(3):
        got.append(cache.splitmix64(state))
        state = (state + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
    assert got == ref


def _run(policy, trace, N, S, **kw):
    st = cache.CacheState(N, S)
    misses = []
    nu = cache.next_use_table(trace) if policy == "belady" else None
    for t, sel in enumerate(trace):
        slots, h, m, _ = cache.policy_step(st, sel, t, policy, next_use=None if nu is None else nu[t], **kw)
        assert h + m == len(sel)
        # invariants: tables are inverse maps, the selection is resident
        res = np.flatnonzero(st.page_table >= 0)
        assert np.array_equal(np.sort(st.slot_token[st.page_table[res]]), np.sort(res))
        assert np.array_equal(st.slot_token[slots], np.asarray(sel))
        misses.append(m)
    return misses


def _one_token_trace(rng, N, T):
    return [[int(x)] for x in rng.integers(0, N, T)]


@pytest.mark.parametrize("seed", range(5))
def test_fifo_one_token_per_step_is_a_textbook_queue(seed):
    rng = np.random.default_rng(seed)
    N, S, T = 9, 4, 60
    trace = _one_token_trace(rng, N, T)
    q, resident, ref = collections.deque(), set(), []
    for (tok,) in trace:
        if tok in resident:
            ref.append(0)
            continue
        ref.append(1)
        if len(q) == S:
            resident.discard(q.popleft())
        q.append(tok)
        resident.add(tok)
    assert _run("fifo", trace, N, S) == ref


def _min_misses(trace, S):
    """Fewest misses any eviction choice reaches (exhaustive search)."""
    best = {frozenset(): 0}
    for (tok,) in trace:
        nxt = {}
        for res, m in best.items():
            if tok in res:
                outs = [(res, m)]
            elif len(res) < S:
                outs = [(res | {tok}, m + 1)]
            else:
                outs = [((res - {v}) | {tok}, m + 1) for v in res]
            for r, mm in outs:
                if nxt.get(r, 1 << 30) > mm:
                    nxt[r] = mm
        best = nxt
    return min(best.values())


@pytest.mark.parametrize("seed", range(6))
def test_belady_one_token_per_step_is_optimal(seed):
    rng = np.random.default_rng(100 + seed)
    N, S, T = 7, 3, 16
    trace = _one_token_trace(rng, N, T)
    got = sum(_run("belady", trace, N, S))
    assert got == _min_misses(trace, S)
    assert got <= sum(_run("lru", trace, N, S)) and got <= sum(_run("fifo", trace, N, S))


def test_fifo_differs_from_lru_on_a_hit_to_the_oldest():
    # S = 2: tokens 0, 1 fetched; 0 hit; 2 misses. LRU evicts 1 (least recent),
    # FIFO evicts 0 (first in).
    trace = [[0], [1], [0], [2], [0]]
    assert _run("lru", trace, 3, 2) == [1, 1, 0, 1, 0]
    assert _run("fifo", trace, 3, 2) == [1, 1, 0, 1, 1]


def test_random_policy_is_seeded_protects_hits_and_spreads_evictions():
    rng = np.random.default_rng(7)
    N, S, T = 40, 8, 3000
    trace = [list(rng.choice(N, size=3, replace=False)) for _ in range(T)]
    a = _run("random", trace, N, S, seed=11, request=2)
    assert a == _run("random", trace, N, S, seed=11, request=2)
    assert a != _run("random", trace, N, S, seed=12, request=2)
    # victim slots of single misses over many steps are close to uniform
    st = cache.CacheState(N, S)
    counts = np.zeros(S)
    for t, sel in enumerate(trace):
        before = st.slot_token.copy()
        cache.policy_step(st, sel, t, "random", seed=11, request=2)
        changed = np.flatnonzero(st.slot_token != before)
        counts[changed] += 1
        for s in changed:  # an evicted slot never held a token of this step's selection before
            assert before[s] not in sel
    exp = counts.sum() / S
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 30.0, chi2     # 7 degrees of freedom; p ~ 1e-4 at 30


def test_random_key_is_31_bits_and_depends_on_every_coordinate():
    base = cache.random_key(1, 2, 3, 4)
    assert 0 <= base < 2**31
    assert len({base, cache.random_key(2, 2, 3, 4), cache.random_key(1, 3, 3, 4), cache.random_key(1, 2, 4, 4),
                cache.random_key(1, 2, 3, 5)}) == 5


@pytest.mark.parametrize("policy", cache.POLICIES)
def test_no_eviction_when_the_pool_holds_everything(policy):
    rng = np.random.default_rng(9)
    N, T = 30, 12
    trace = [list(rng.choice(N, size=6, replace=False)) for _ in range(T)]
    seen, ref = set(), []
    for sel in trace:
        ref.append(len(set(sel) - seen))
        seen |= set(sel)
    assert _run(policy, trace, N, N, seed=3) == ref


def test_next_use_table():
    trace = [[1, 2], [2, 3], [1], [4]]
    nu = cache.next_use_table(trace)
    assert nu[0] == {2: 1, 3: 1, 1: 2, 4: 3}
    assert nu[1] == {1: 2, 4: 3}
    assert nu[3] == {}
    assert cache.next_use_table([[5]])[0].get(5, cache.NEVER) == cache.NEVER


def test_layer_group_shares_tables_and_keeps_every_pool_exact():
    """A group of layers sharing the selection: the tables evolve as for one
    layer, and every layer's pool holds its own rows of each resident token,
    so attention through the cache equals direct attention in every layer."""
    rng = np.random.default_rng(21)
    N, S, Hkv, d, Hq, L, T = 200, 48, 2, 8, 4, 3, 12
    hosts = [(rng.standard_normal((N, Hkv, d)), rng.standard_normal((N, Hkv, d))) for _ in range(L)]
    pools = [(np.zeros((S, Hkv, d)), np.zeros((S, Hkv, d))) for _ in range(L)]
    grp, single = cache.CacheState(N, S), cache.CacheState(N, S)
    sel = rng.choice(N, size=32, replace=False)
    for t in range(T):
        keep = rng.choice(sel, size=24, replace=False)
        fresh = rng.choice(np.setdiff1d(np.arange(N), sel), size=8, replace=False)
        sel = np.concatenate([keep, fresh])
        slots, h, m, _ = cache.group_step(grp, sel, t, hosts, pools)
        s1, h1, m1, _ = cache.lru_step(single, sel, t)
        assert np.array_equal(slots, s1) and (h, m) == (h1, m1)
        assert np.array_equal(grp.page_table, single.page_table)
        res = np.flatnonzero(grp.slot_token >= 0)
        for (hk, hv), (pk, pv) in zip(hosts, pools):
            assert np.array_equal(pk[res], hk[grp.slot_token[res]]) and np.array_equal(pv[res], hv[grp.slot_token[res]])
            q = rng.standard_normal((Hq, d))
            direct = cache.attend_slots(q, hk, hv, sel)
            assert np.array_equal(cache.attend_slots(q, pk, pv, slots), direct)


def test_a_trace_with_locality_orders_the_policies_as_real_selections_do():
    """[HISPARSE-NEWS] ranks the policies by miss rate on real selection
    traces: Belady (offline) lowest, then LRU, random, FIFO. A uniform
    synthetic trace makes the online policies coincide (a dropped token is no
    likelier to return than any other). With popular tokens that persist and
    recently dropped tokens that return, the oracle gives the same order."""
    from top_sparse_attention_centroid_amd import workloads as W

    cfg = W.config(4, batch=1, n_tokens=16384, n_slots=512, top_k=256, overlap=218, steps=50,
                   popularity_sd=2.0, recency=0.3)
    tr = W.selection_trace(cfg).numpy()[:, 0]
    nu = cache.next_use_table(tr)
    rate = {}
    for pol in ("lru", "fifo", "random", "belady"):
        st = cache.CacheState(cfg.n_tokens, cfg.n_slots)
        m = [cache.policy_step(st, sel, t, pol, seed=0x5EED, request=0, next_use=nu[t])[2] for t, sel in enumerate(tr)]
        rate[pol] = np.mean(m[1:]) / cfg.top_k
    assert rate["belady"] < rate["lru"] < rate["random"] < rate["fifo"], rate

