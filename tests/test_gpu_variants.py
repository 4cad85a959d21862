"""GPU parity of the decode variants (cosine similarity, sink/window rows
beside the lists, their mix with a growing index) against the variants
oracle, and the token selector feeding the hot cache end to end."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import append, cache, ivf, token, variants
from top_sparse_attention_centroid_amd import workloads as W

from helpers import GAP_MIN, MARGIN_MIN, OUT_TOL, announce, condition_token_keys, f64, out_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _problem(seed_scale=0, **kw):
    base = dict(batch=3, n_tokens=6000, n_centroids=64, top_k=6, n_kv_heads=2, n_q_heads=8, steps=1)
    base.update(kw)
    cfg = W.config(2, **base)
    p = W.ivf_problem(cfg, device=DEV)
    if seed_scale:
        # unequal centroid norms, so that cosine and dot rankings differ; every
        # key moves with its own centre (its nearest unscaled centroid, found
        # by the oracle), so it keeps a wide assignment margin
        g = torch.Generator(device=DEV).manual_seed(seed_scale)
        f = torch.rand(p["centroids"].shape[:-1] + (1,), generator=g, device=DEV) * 1.5 + 0.5
        c32 = p["centroids"].float()
        keys = p["keys"].float()
        c64 = f64(p["centroids"])
        for b in range(cfg.batch):
            for h in range(cfg.n_kv_heads):
                comp, _ = ivf.nearest_centroid(f64(p["keys"][b, :, h]), c64[0, h])
                comp = torch.from_numpy(comp).to(DEV)
                keys[b, :, h] += (f[0, h, comp] - 1.0) * c32[0, h, comp]
        p["keys"] = keys.to(cfg.torch_dtype)
        p["centroids"] = (c32 * f).to(cfg.torch_dtype)
    return cfg, p


def _queries(cfg, p, similarity, max_rounds=40):
    """Queries whose oracle top-k gap (under `similarity`) is >= GAP_MIN."""
    c64 = f64(p["centroids"])
    G = cfg.group

    def gap(qv, b, h):
        cb = c64[0 if c64.shape[0] == 1 else b, h // G]
        s = variants.cosine_scores(qv, cb) if similarity == "cosine" else cb @ qv
        return ivf.selection_gap(s, cfg.top_k)

    q = W.ivf_queries(cfg, p["centroids"], steps=1)[0]
    for salt in range(1, max_rounds + 1):
        q64 = f64(q)
        bad = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads) if gap(q64[b, h], b, h) < GAP_MIN]
        if not bad:
            return q
        fresh = W.ivf_queries(cfg, p["centroids"], steps=1, salt=salt)[0]
        for b, h in bad:
            q[b, h] = fresh[b, h]
    raise RuntimeError("could not draw well-separated queries")


def _check(cfg, p, q, off, ids, out, sel, **kw):
    """The oracle builds its own posting lists (every assignment margin must
    be wide enough for an exact comparison), which must equal the GPU's, then
    decodes over them; the selection must match exactly and the output within
    OUT_TOL."""
    k64, v64, c64 = f64(p["keys"]), f64(p["values"]), f64(p["centroids"])
    r_off, r_ids, margins = ivf.index_build(k64, c64)
    assert margins.min() >= MARGIN_MIN, f"assignment margin {margins.min()} too small for an exact comparison"
    assert np.array_equal(off.cpu().numpy(), r_off) and np.array_equal(ids.cpu().numpy(), r_ids)
    r = variants.sparse_decode_ex(f64(q), c64, r_off, r_ids, k64, v64, cfg.top_k, **kw)
    assert np.all(r["gap"] >= GAP_MIN)
    assert np.array_equal(sel.cpu().numpy(), r["sel"]), "selection differs from the oracle"
    err = out_error(out.cpu().numpy(), r["out"])
    assert err <= OUT_TOL, f"output error {err}"
    return r


def test_cosine_selection_and_output():
    cfg, p = _problem(seed_scale=7)
    announce("variants: cosine")
    off, ids = tsa.index_build(p["keys"], p["centroids"])
    q = _queries(cfg, p, "cosine")
    sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k,
                               similarity="cosine", sel_out=sel)
    torch.cuda.synchronize()
    _check(cfg, p, q, off, ids, out, sel, similarity="cosine")
    sel_dot = torch.empty_like(sel)
    tsa.sparse_decode(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k, sel_out=sel_dot)
    torch.cuda.synchronize()
    assert not torch.equal(sel, sel_dot), "scaled codebook should make cosine and dot choose differently"


def test_sink_and_window_with_lengths():
    cfg, p = _problem()
    announce("variants: sink 64 + window 300, per-request lengths")
    off, ids = tsa.index_build(p["keys"], p["centroids"])
    q = _queries(cfg, p, "dot")
    lengths = torch.tensor([6000, 4321, 777], dtype=torch.int32, device=DEV)
    sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k, n_sink=64,
                               n_window=300, lengths=lengths, sel_out=sel)
    torch.cuda.synchronize()
    _check(cfg, p, q, off, ids, out, sel, n_sink=64, n_window=300, lengths=lengths.cpu().numpy())


def test_overlapping_sink_and_window_cover_a_short_request():
    # L = 1000 with a 600-token sink and a 700-token window: the ranges overlap
    # and cover the whole request; list rows below L are all inside them
    cfg, p = _problem(n_tokens=3000)
    announce("variants: overlapping sink/window")
    off, ids = tsa.index_build(p["keys"], p["centroids"])
    q = _queries(cfg, p, "dot")
    lengths = torch.tensor([1000, 1000, 2999], dtype=torch.int32, device=DEV)
    sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k, n_sink=600,
                               n_window=700, lengths=lengths, sel_out=sel)
    torch.cuda.synchronize()
    _check(cfg, p, q, off, ids, out, sel, n_sink=600, n_window=700, lengths=lengths.cpu().numpy())


def test_no_variant_is_bitwise_the_plain_decode():
    cfg, p = _problem()
    announce("variants: defaults == sparse_decode")
    off, ids = tsa.index_build(p["keys"], p["centroids"])
    q = _queries(cfg, p, "dot")
    a = tsa.sparse_decode_ex(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k)
    b = tsa.sparse_decode(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# C = 2: every key in both lists; C = 7: one 16-centroid tile, mostly
# padding; C = 300: two codebook stages, the second ending inside a tile.
# N = 3001 and 2500 leave a last workgroup with a partial 16-key tile and
# idle key tiles in its last pass.
@pytest.mark.parametrize("batch,n_kv_heads", [(3, 2), (16, 8)])
def test_variants_over_a_growing_index(batch, n_kv_heads):
    """Cosine + sink/window over a dynamic index (list lengths) equals the
    same variants over the compacted static lists."""
    cfg, p = _problem(seed_scale=3, n_tokens=5000, batch=batch, n_kv_heads=n_kv_heads, n_q_heads=4 * n_kv_heads)
    announce(f"variants over a growing index, {batch} x {n_kv_heads} KV heads")
    n_prefix = 4000
    off, lens, ids = tsa.index_build_dyn(p["keys"], p["centroids"], n_prefix)
    status = torch.empty((cfg.batch, cfg.n_kv_heads), dtype=torch.int32, device=DEV)
    k_cache, v_cache = p["keys"].clone(), p["values"].clone()
    for row in range(n_prefix, n_prefix + 200):
        pos = torch.full((cfg.batch,), row, dtype=torch.int32, device=DEV)
        tsa.kv_append(p["keys"][:, row].contiguous(), p["values"][:, row].contiguous(), pos, p["centroids"],
                      k_cache, v_cache, off, lens, ids, status=status)
    lengths = torch.full((cfg.batch,), n_prefix + 200, dtype=torch.int32, device=DEV)
    q = _queries(cfg, p, "cosine")
    sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, k_cache, v_cache, cfg.top_k, similarity="cosine",
                               n_sink=32, n_window=128, lengths=lengths, lens=lens, sel_out=sel)
    torch.cuda.synchronize()
    # the oracle grows its own index over the same keys: a prefix build with
    # the same slack, then one append per row, in row order
    k64, c64 = f64(p["keys"]), f64(p["centroids"])
    B, Hkv, C = cfg.batch, cfg.n_kv_heads, cfg.n_centroids
    slack = (cfg.n_tokens - n_prefix) // C
    for b in range(B):
        for g in range(Hkv):
            _, margin = ivf.nearest_centroid(k64[b, :n_prefix + 200, g], c64[0, g])
            assert margin.min() >= MARGIN_MIN, f"assignment margin {margin.min()} too small for an exact comparison"
    state = {(b, g): append.index_build_dynamic(k64[b, :, g], c64[0, g], n_prefix, slack)
             for b in range(B) for g in range(Hkv)}
    K_ref, V_ref = k64.copy(), f64(p["values"])
    for row in range(n_prefix, n_prefix + 200):
        append.append_step(state, k64[:, row], V_ref[:, row].copy(), np.full(B, row), c64, K_ref, V_ref)
    og, lg, ig = off.cpu().numpy(), lens.cpu().numpy(), ids.cpu().numpy()
    s_off = np.zeros((B, Hkv, C + 1), dtype=np.int64)
    s_ids = np.full((B, Hkv, cfg.n_tokens), -1, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            r_off, r_lens, r_ids = state[(b, g)]
            assert np.array_equal(og[b, g], r_off) and np.array_equal(lg[b, g], r_lens)
            assert np.array_equal(ig[b, g], r_ids), f"growing lists differ (request {b}, KV head {g})"
            co, ci = append.compact(r_off, r_lens, r_ids)
            s_off[b, g] = co
            s_ids[b, g, :len(ci)] = ci
    assert int(status.max()) <= 1
    r = variants.sparse_decode_ex(f64(q), c64, s_off, s_ids, K_ref, V_ref,
                                  cfg.top_k, similarity="cosine", n_sink=32, n_window=128,
                                  lengths=lengths.cpu().numpy())
    assert np.all(r["gap"] >= GAP_MIN)
    assert np.array_equal(sel.cpu().numpy(), r["sel"])
    err = out_error(out.cpu().numpy(), r["out"])
    assert err <= OUT_TOL, f"output error {err}"


def test_token_selection_feeds_the_hot_cache():
    """The indexer's selection drives RESOLVE, then attention over the slots,
    checked against the oracle's chain: its top-k over the indexer scores, its
    LRU step on that selection (tables, hits, misses, fetched rows into its
    own pool) and its attention over its own pool's slots. The GPU's cache
    path is also bitwise the token decode's direct attention."""
    cfg = W.config(3, batch=2, n_tokens=30_000, top_k=512, n_planted=16, steps=4)
    announce("token selection -> RESOLVE -> attention over slots")
    B, N, Hkv, d, k = cfg.batch, cfg.n_tokens, cfg.n_kv_heads, cfg.head_dim, cfg.top_k
    S, steps = 1024, 4
    prob = W.token_problem(cfg, device=DEV)
    q_idx, q = W.token_queries(cfg, prob, steps=steps)
    k_idx = condition_token_keys(q_idx, prob["k_idx"], k, steps)
    hk = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
    hv = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
    hk.tensor.copy_(prob["keys"])
    hv.tensor.copy_(prob["values"])
    pt = torch.empty((B, N), dtype=torch.int32, device=DEV)
    st = torch.empty((B, S), dtype=torch.int32, device=DEV)
    lu = torch.empty((B, S), dtype=torch.int32, device=DEV)
    tsa.cache_reset(pt, st, lu)
    pool_k = torch.zeros((B, S, Hkv, d), dtype=cfg.torch_dtype, device=DEV)
    pool_v = torch.zeros_like(pool_k)
    sel = torch.empty((B, k), dtype=torch.int32, device=DEV)
    ref = [cache.CacheState(N, S) for _ in range(B)]
    host_k, host_v = f64(prob["keys"]), f64(prob["values"])
    ref_pk, ref_pv = np.zeros((B, S, Hkv, d)), np.zeros((B, S, Hkv, d))
    qi64, q64, kidx64 = f64(q_idx), f64(q), f64(k_idx)
    misses = []
    for t in range(steps):
        out_tok = tsa.token_decode(q_idx[t], k_idx, q[t], prob["keys"], prob["values"], k, sel_out=sel)
        slots, hits, miss = tsa.resolve(pt, st, lu, sel, t, hk.tensor, hv.tensor, pool_k, pool_v)
        out_cache = tsa.attend_rows(q[t], pool_k, pool_v, slots)
        torch.cuda.synchronize()
        assert torch.equal(out_cache, out_tok), f"step {t}: cache path differs from the direct path"
        sel_g, slots_g, hits_g, miss_g = sel.cpu().numpy(), slots.cpu().numpy(), hits.cpu().numpy(), miss.cpu().numpy()
        pt_g, st_g, lu_g, out_g = pt.cpu().numpy(), st.cpu().numpy(), lu.cpu().numpy(), out_cache.cpu().numpy()
        for b in range(B):
            r_sel, gap = token.token_topk(qi64[t, b], kidx64[b], k)
            assert gap >= GAP_MIN
            assert np.array_equal(sel_g[b], r_sel), f"selection differs (step {t}, request {b})"
            r_slots, r_h, r_m, fetches = cache.lru_step(ref[b], r_sel, t)
            cache.fetch_rows(ref_pk[b], ref_pv[b], host_k[b], host_v[b], fetches)
            assert np.array_equal(slots_g[b], r_slots) and (hits_g[b], miss_g[b]) == (r_h, r_m)
            assert np.array_equal(pt_g[b], ref[b].page_table) and np.array_equal(st_g[b], ref[b].slot_token)
            assert np.array_equal(lu_g[b], ref[b].last_use)
            o = cache.attend_slots(q64[t, b], ref_pk[b], ref_pv[b], r_slots)
            err = out_error(out_g[b], o)
            assert err <= OUT_TOL, f"output error {err} (step {t}, request {b})"
        misses.append(int(miss.sum()))
    assert misses[0] == B * k and min(misses[1:]) < B * k   # planted tokens stay selected and hit


def _two_way_keys(cfg, centroids, seed, min_gap=None):
    """Keys between two centroids (0.6 c_a + 0.4 c_b + 0.1 noise, a != b): a
    clear first and second nearest list and a wide margin to the third.
    With min_gap, keys whose second-vs-third choice margin (as the oracle
    measures it on the stored values) is below it get fresh noise until
    none is left (many keys reach deeper into the margin's tail)."""
    g = torch.Generator().manual_seed(seed)
    B, N, Hkv, d = cfg.batch, cfg.n_tokens, cfg.n_kv_heads, cfg.head_dim
    C = centroids.shape[2]
    cent = centroids.float().cpu()
    a = torch.randint(0, C, (B, N, Hkv), generator=g)
    b = (a + torch.randint(1, C, (B, N, Hkv), generator=g)) % C
    head = torch.arange(Hkv)[None, None, :].expand(B, N, Hkv)
    keys = (0.6 * cent[0][head, a] + 0.4 * cent[0][head, b] + 0.1 * torch.randn((B, N, Hkv, d), generator=g))
    keys = keys.to(cfg.torch_dtype)
    if min_gap is not None:
        c64 = centroids.double().cpu().numpy()
        for _ in range(20):
            redrawn = 0
            for bi in range(B):
                for gi in range(Hkv):
                    _, gap = variants.nearest_centroids(keys[bi, :, gi].double().numpy(), c64[0, gi], 2)
                    bad = torch.from_numpy(np.nonzero(gap < min_gap)[0])
                    if len(bad):
                        redrawn += len(bad)
                        fresh = (0.6 * cent[0, gi][a[bi, bad, gi]] + 0.4 * cent[0, gi][b[bi, bad, gi]]
                                 + 0.1 * torch.randn((len(bad), d), generator=g))
                        keys[bi, bad, gi] = fresh.to(cfg.torch_dtype)
            if redrawn == 0:
                break
        else:
            raise RuntimeError("could not draw keys with the required second-choice margin")
    return keys.to(DEV)


# C = 2: every key in both lists; C = 7: one 16-centroid tile, mostly
# padding; C = 300: two codebook stages, the second ending inside a tile.
# N = 3001 and 2500 leave a last workgroup with a partial 16-key tile and
# idle key tiles in its last pass.
@pytest.mark.parametrize("n_tokens,C", [(3001, 2), (3001, 7), (2500, 300)])
def test_two_way_index_build_ragged_shapes(n_tokens, C):
    cfg, p = _problem(n_tokens=n_tokens, n_centroids=C, top_k=2, batch=2, n_kv_heads=2, n_q_heads=8)
    announce(f"variants: two lists per key, index build N={n_tokens} C={C}")
    p["keys"] = _two_way_keys(cfg, p["centroids"], 23 + C, min_gap=1e-3 if C > 2 else None)
    off, ids, alt = tsa.index_build_multi(p["keys"], p["centroids"], 2)
    s_off, s_ids = tsa.index_build(p["keys"], p["centroids"])
    torch.cuda.synchronize()
    k64, c64 = f64(p["keys"]), f64(p["centroids"])
    r_off, r_ids, r_alt, margin = variants.index_build_multi(k64, c64, 2)
    assert margin >= 1e-3, f"assignment margin {margin} too small for an exact comparison"
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert np.array_equal(alt.cpu().numpy(), r_alt)
    # the nearest list of each key, from the one-list build, is its first choice
    r1_off, r1_ids, _, margin1 = variants.index_build_multi(k64, c64, 1)
    assert margin1 >= 1e-3, f"first-choice margin {margin1} too small for an exact comparison"
    assert np.array_equal(s_off.cpu().numpy(), r1_off)
    assert np.array_equal(s_ids.cpu().numpy(), r1_ids)
    if C == 2:
        # both lists hold every token
        assert np.all(r_off[..., -1] == 2 * n_tokens)


# 3 x 2 KV heads: a wave per plan segment; 16 x 8: merged gather sets
@pytest.mark.parametrize("batch,n_kv_heads", [(3, 2), (16, 8)])
def test_two_way_lists_build_and_decode(batch, n_kv_heads):
    """Every key in its two nearest lists: lists and alt exact against the
    oracle; decode attends each token once per head (union of the lists),
    alone and with cosine + sink/window."""
    cfg, p = _problem(n_tokens=4000, n_centroids=32, top_k=5, batch=batch, n_kv_heads=n_kv_heads,
                      n_q_heads=4 * n_kv_heads)
    announce(f"variants: two lists per key, {batch} x {n_kv_heads} KV heads")
    p["keys"] = _two_way_keys(cfg, p["centroids"], 17, min_gap=2e-3 if batch * n_kv_heads >= 128 else None)
    off, ids, alt = tsa.index_build_multi(p["keys"], p["centroids"], 2)
    torch.cuda.synchronize()
    k64, c64 = f64(p["keys"]), f64(p["centroids"])
    r_off, r_ids, r_alt, margin = variants.index_build_multi(k64, c64, 2)
    assert margin >= 1e-3, f"second-choice margin {margin} too small for an exact comparison"
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert np.array_equal(alt.cpu().numpy(), r_alt)
    # one list per key through the same entry point equals the plain build
    o1, i1, a1 = tsa.index_build_multi(p["keys"], p["centroids"], 1)
    s_off, s_ids = tsa.index_build(p["keys"], p["centroids"])
    torch.cuda.synchronize()
    assert a1 is None and torch.equal(o1, s_off) and torch.equal(i1, s_ids)

    for kw in ({}, {"similarity": "cosine", "n_sink": 16, "n_window": 200}):
        q = _queries(cfg, p, kw.get("similarity", "dot"))
        sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
        out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k, alt=alt,
                                   sel_out=sel, **kw)
        torch.cuda.synchronize()
        r = variants.sparse_decode_ex(f64(q), c64, r_off, r_ids, k64, f64(p["values"]), cfg.top_k, **kw)
        assert np.all(r["gap"] >= GAP_MIN)
        assert np.array_equal(sel.cpu().numpy(), r["sel"])
        err = out_error(out.cpu().numpy(), r["out"])
        assert err <= OUT_TOL, f"output error {err} ({kw})"
        if not kw:
            # the case does hold tokens in two chosen lists of one head: counting
            # them twice would move the output well past the bar
            G = cfg.group
            worst = 0.0
            for b in range(cfg.batch):
                for h in range(cfg.n_q_heads):
                    g = h // G
                    lists = r["sel"][b, h]
                    rows = np.concatenate([r_ids[b, g][r_off[b, g][c]:r_off[b, g][c + 1]] for c in lists])
                    o2, _ = ivf.attend(f64(q)[b, h], k64[b, rows, g], f64(p["values"])[b, rows, g])
                    worst = max(worst, out_error(out.cpu().numpy()[b, h], o2))
            assert worst > 10 * OUT_TOL, "no token was in two chosen lists; the case tests nothing"
