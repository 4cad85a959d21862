"""Pins of the per-step append oracle ([KARAT] worked example, step 6).

The dynamic index is tied to the static index build, which is pinned on its
own: building over a prefix and appending the rest one token at a time must
give exactly the lists that the static build gives over all keys."""

import numpy as np
import pytest

from oracle import append, ivf


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
