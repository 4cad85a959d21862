"""Pins of the per-step append oracle ([KARAT] worked example, step 6).

The dynamic index is tied to the static index build, which is pinned on its
own: building over a prefix and appending the rest one token at a time must
give exactly the lists that the static build gives over all keys."""

import numpy as np
import pytest

from oracle import append, ivf, variants


def _clustered(rng, N, C, d, sd=0.3):
    cent = rng.standard_normal((C, d))
    lab = rng.integers(0, C, N)
    return cent, cent[lab] + sd * rng.standard_normal((N, d))


@pytest.mark.parametrize("n_prefix", [1, 37, 400])
def test_prefix_build_plus_appends_equals_static_build(n_prefix):
    rng = np.random.default_rng(n_prefix)
    N, C, d = 600, 12, 16
    cent, keys = _clustered(rng, N, C, d)
    # room for every remaining token in any list: capacity n_prefix + C * (N - n_prefix)
    spare = N - n_prefix
    padded = np.concatenate([keys, np.zeros(((C - 1) * spare, d))])
    big_off, big_lens, big_ids = append.index_build_dynamic(padded, cent, n_prefix, spare)
    for i in range(n_prefix, N):
        c, ok = append.append_key(big_off, big_lens, big_ids, cent, keys[i], i)
        assert ok
    s_off, s_ids = ivf.posting_lists(ivf.nearest_centroid(keys, cent)[0], C)
    c_off, c_ids = append.compact(big_off, big_lens, big_ids)
    assert np.array_equal(c_off, s_off) and np.array_equal(c_ids, s_ids)
    # the zero-slack prefix build is the static build of the prefix
    offsets, lens, ids = append.index_build_dynamic(keys, cent, n_prefix, 0)
    p_off, p_ids = ivf.posting_lists(ivf.nearest_centroid(keys[:n_prefix], cent)[0], C)
    z_off, z_ids = append.compact(offsets, lens, ids)
    assert np.array_equal(z_off, p_off) and np.array_equal(z_ids, p_ids)


def test_slack_bookkeeping():
    rng = np.random.default_rng(3)
    N, C, d, n_prefix, slack = 500, 8, 8, 300, 20
    cent, keys = _clustered(rng, N, C, d)
    off, lens, ids = append.index_build_dynamic(keys, cent, n_prefix, slack)
    assert off[0] == 0 and off[-1] == n_prefix + C * slack
    assert np.array_equal(np.diff(off), lens + slack)
    assert lens.sum() == n_prefix
    for c in range(C):
        valid = ids[off[c]:off[c] + lens[c]]
        assert np.all(np.diff(valid) > 0) and np.all(valid < n_prefix)
        assert np.all(ids[off[c] + lens[c]:off[c + 1]] == -1)
    assert np.all(ids[off[-1]:] == -1)
    # every prefix token appears exactly once
    assert np.array_equal(np.sort(ids[ids >= 0]), np.arange(n_prefix))


def test_key_on_centroid_lands_in_that_list_at_its_end():
    rng = np.random.default_rng(4)
    N, C, d = 200, 6, 8
    cent, keys = _clustered(rng, N, C, d)
    off, lens, ids = append.index_build_dynamic(keys, cent, 100, 10)
    for j in range(C):
        before = lens[j]
        c, ok = append.append_key(off, lens, ids, cent, cent[j], 150 + j)
        assert (c, ok) == (j, True)
        assert lens[j] == before + 1 and ids[off[j] + before] == 150 + j


def test_full_list_reports_and_leaves_index_unchanged():
    rng = np.random.default_rng(5)
    N, C, d = 100, 4, 8
    cent, keys = _clustered(rng, N, C, d)
    off, lens, ids = append.index_build_dynamic(keys, cent, 60, 0)
    snap = (off.copy(), lens.copy(), ids.copy())
    c, ok = append.append_key(off, lens, ids, cent, cent[2], 70)
    assert (c, ok) == (2, False)
    for a, b in zip((off, lens, ids), snap):
        assert np.array_equal(a, b)


def test_append_step_writes_rows_and_reports_status():
    rng = np.random.default_rng(6)
    B, N, Hkv, C, d = 2, 50, 2, 3, 8
    cent = rng.standard_normal((1, Hkv, C, d))
    K = rng.standard_normal((B, N, Hkv, d))
    V = rng.standard_normal((B, N, Hkv, d))
    state = {(b, g): append.index_build_dynamic(K[b, :, g], cent[0, g], 30, 3) for b in range(B) for g in range(Hkv)}
    nk = cent[0][None].repeat(B, 0)[:, :, 1]    # every new key sits on centroid 1
    nv = rng.standard_normal((B, Hkv, d))
    st = append.append_step(state, nk, nv, [30, N], cent, K, V)
    assert np.array_equal(st, [[0, 0], [2, 2]])
    assert np.array_equal(K[0, 30], nk[0]) and np.array_equal(V[0, 30], nv[0])
    for g in range(Hkv):
        off, lens, ids = state[(0, g)]
        assert ids[off[1] + lens[1] - 1] == 30


def _brute_nearest(key, cent, m):
    d2 = [(float(sum((float(a) - float(b)) ** 2 for a, b in zip(key, cent[c]))), c) for c in range(len(cent))]
    return [c for _, c in sorted(d2)[:m]]


@pytest.mark.parametrize("m", [2, 3, 4])
def test_multi_prefix_build_plus_appends_equals_static_multi_build(m):
    # several lists per key ([KARAT] How, index structure): a prefix build
    # plus one append per remaining token gives the static m-way lists, and
    # every entry's alt row is the token's other lists in preference order
    rng = np.random.default_rng(100 + m)
    N, C, d = 160, 7, 5
    cent, keys = _clustered(rng, N, C, d, sd=0.8)
    n_prefix = 40
    spare = N - n_prefix                      # room for every remaining token in any list
    cap = n_prefix + C * spare                # capacity in tokens: n_prefix * m + C * slack <= cap * m
    padded = np.concatenate([keys, np.zeros((cap - N, d))])
    off, lens, ids, alt = append.index_build_dynamic_multi(padded, cent, n_prefix, spare, m)
    assert ids.shape == (cap * m,) and alt.shape == (cap * m, m - 1)
    for i in range(n_prefix, N):
        lists, ok = append.append_key_multi(off, lens, ids, alt, cent, keys[i], i, m)
        assert ok and lists == _brute_nearest(keys[i], cent, m)
    s_off, s_ids, s_alt = variants.posting_lists_multi(variants.nearest_centroids(keys, cent, m)[0], C)
    c_off, c_ids = append.compact(off, lens, ids)
    assert np.array_equal(c_off, s_off) and np.array_equal(c_ids, s_ids)
    c_alt = np.concatenate([alt[off[c]:off[c] + lens[c]] for c in range(C)])
    assert np.array_equal(c_alt, s_alt)
    for c in range(C):                        # brute force on every entry
        for e in range(off[c], off[c] + lens[c]):
            pref = _brute_nearest(keys[ids[e]], cent, m)
            assert alt[e].tolist() == [x for x in pref if x != c]
        assert np.all(ids[off[c] + lens[c]:off[c + 1]] == -1)


def test_multi_append_is_all_or_nothing():
    rng = np.random.default_rng(7)
    N, C, d, m = 60, 5, 4, 2
    cent, keys = _clustered(rng, N, C, d)
    off, lens, ids, alt = append.index_build_dynamic_multi(keys, cent, 30, 1, m)
    key = cent[2] + 1e-3                      # nearest list 2; fill list 2 first
    first = _brute_nearest(key, cent, m)
    assert first[0] == 2
    lists, ok = append.append_key_multi(off, lens, ids, alt, cent, key, 30, m)
    assert ok and lists == first
    before = (lens.copy(), ids.copy(), alt.copy())
    lists, ok = append.append_key_multi(off, lens, ids, alt, cent, key, 31, m)
    assert not ok and lists == first          # list 2 has no free entry left
    assert np.array_equal(lens, before[0]) and np.array_equal(ids, before[1]) and np.array_equal(alt, before[2])


@pytest.mark.parametrize("m", [1, 2])
def test_regrow_keeps_every_list_and_makes_room(m):
    rng = np.random.default_rng(40 + m)
    N, C, d = 200, 6, 8
    cent, keys = _clustered(rng, N, C, d)
    off, lens, ids, alt = append.index_build_dynamic_multi(keys, cent, 120, 0, m)
    # zero slack: the next token's lists are full
    lists, ok = append.append_key_multi(off, lens, ids, alt, cent, keys[120], 120, m)
    assert not ok
    slack = append.regrow_slack(lens, len(ids))
    assert slack == (N * m - 120 * m) // C and slack > 0
    n_off, n_lens, n_ids, n_alt = append.regrow(off, lens, ids, alt, slack)
    assert np.array_equal(n_lens, lens)
    assert np.array_equal(n_off[1:] - n_off[:-1], lens + slack)
    assert np.array_equal(append.compact(n_off, n_lens, n_ids)[1], append.compact(off, lens, ids)[1])
    for c in range(C):
        assert np.array_equal(n_alt[n_off[c]:n_off[c] + lens[c]], alt[off[c]:off[c] + lens[c]])
        assert np.all(n_ids[n_off[c] + lens[c]:n_off[c + 1]] == -1)
    assert np.all(n_ids[n_off[C]:] == -1)
    # the append that failed now goes in, and so do the rest while room lasts
    lists2, ok = append.append_key_multi(n_off, n_lens, n_ids, n_alt, cent, keys[120], 120, m)
    assert ok and lists2 == lists
    # the result is the m-way build of the first 121 keys
    s_off, s_ids, _ = variants.posting_lists_multi(variants.nearest_centroids(keys[:121], cent, m)[0], C)
    assert np.array_equal(append.compact(n_off, n_lens, n_ids)[1], s_ids)
    with pytest.raises(ValueError):
        append.regrow(off, lens, ids, alt, slack + 1 + (N * m) // C)


def test_one_way_dynamic_multi_build_is_the_one_way_build():
    rng = np.random.default_rng(3)
    N, C, d = 90, 5, 6
    cent, keys = _clustered(rng, N, C, d)
    off1, lens1, ids1 = append.index_build_dynamic(keys, cent, 50, 4)
    off, lens, ids, alt = append.index_build_dynamic_multi(keys, cent, 50, 4, 1)
    assert np.array_equal(off, off1) and np.array_equal(lens, lens1) and np.array_equal(ids, ids1)
    assert alt.shape == (N, 0)


def test_append_step_with_multi_state():
    rng = np.random.default_rng(5)
    B, Hkv, N, C, d, m = 2, 2, 40, 4, 8, 2
    cent = rng.standard_normal((1, Hkv, C, d))
    K = np.zeros((B, N, Hkv, d))
    V = np.zeros((B, N, Hkv, d))
    K[:, :20] = rng.standard_normal((B, 20, Hkv, d))
    state = {(b, g): append.index_build_dynamic_multi(K[b, :, g], cent[0, g], 20, 2, m)
             for b in range(B) for g in range(Hkv)}
    new_k = rng.standard_normal((B, Hkv, d))
    new_v = rng.standard_normal((B, Hkv, d))
    st = append.append_step(state, new_k, new_v, np.array([20, 21]), cent, K, V)
    assert np.array_equal(st, np.zeros((B, Hkv)))
    for b, p in ((0, 20), (1, 21)):
        for g in range(Hkv):
            off, lens, ids, alt = state[(b, g)]
            where = [c for c in range(C) if p in ids[off[c]:off[c] + lens[c]]]
            assert sorted(where) == sorted(_brute_nearest(new_k[b, g], cent[0, g], m))
    assert np.array_equal(K[0, 20], new_k[0]) and np.array_equal(V[1, 21], new_v[1])
