"""GPU parity of indexes in which every key joins several posting lists
([KARAT] How, index structure: an entry may sit in more than one list):
static m-way builds and decodes for m = 3 and 4, a growing m-way index
(prefix build, all-or-nothing appends, decode over list lengths), and the
repair of a growing index whose lists ran full (regrow, then the refused
appends again), each against the oracle's own index and decode."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import append, ivf, variants
from top_sparse_attention_centroid_amd import workloads as W

from helpers import GAP_MIN, OUT_TOL, announce, f64, out_error

pytestmark = pytest.mark.gpu
DEV = "cuda"
WEIGHTS = (0.4, 0.3, 0.2, 0.1)


def _problem(**kw):
    base = dict(batch=3, n_tokens=3000, n_centroids=32, top_k=5, n_kv_heads=2, n_q_heads=8, steps=1)
    base.update(kw)
    cfg = W.config(2, **base)
    return cfg, W.ivf_problem(cfg, device=DEV)


def _m_way_keys(cfg, centroids, m, seed, min_gap=1e-3):
    """Keys near a weighted mix of m distinct centroids (weights 0.4, 0.3,
    ...), so the m nearest lists are clear; keys whose m-th vs (m+1)-th
    choice margin (the oracle's, on the stored values) is below min_gap are
    drawn again (new centroids and noise) until none is left."""
    g = torch.Generator().manual_seed(seed)
    B, N, Hkv, d = cfg.batch, cfg.n_tokens, cfg.n_kv_heads, cfg.head_dim
    C = centroids.shape[2]
    cent = centroids.float().cpu()
    w = (torch.tensor(WEIGHTS[:m]) / sum(WEIGHTS[:m]))[:, None]

    def draw(n, h):
        pick = torch.argsort(torch.rand((n, C), generator=g), dim=-1)[:, :m]    # m distinct lists per key
        return (w * cent[0, h][pick]).sum(dim=-2) + 0.05 * torch.randn((n, d), generator=g)

    keys = torch.empty((B, N, Hkv, d))
    for b in range(B):
        for h in range(Hkv):
            keys[b, :, h] = draw(N, h)
    keys = keys.to(cfg.torch_dtype)
    c64 = centroids.double().cpu().numpy()
    for _ in range(30):
        redrawn = 0
        for b in range(B):
            for h in range(Hkv):
                _, gap = variants.nearest_centroids(keys[b, :, h].double().numpy(), c64[0, h], m)
                bad = np.nonzero(gap < min_gap)[0]
                if len(bad):
                    redrawn += len(bad)
                    keys[b, torch.from_numpy(bad), h] = draw(len(bad), h).to(cfg.torch_dtype)
        if redrawn == 0:
            return keys.to(DEV)
    raise RuntimeError("could not draw keys with the required m-th choice margin")


def _queries(cfg, p):
    c64 = f64(p["centroids"])
    q = W.ivf_queries(cfg, p["centroids"], steps=1)[0]
    for salt in range(1, 40):
        q64 = f64(q)
        bad = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_q_heads)
               if ivf.selection_gap(c64[0, h // cfg.group] @ q64[b, h], cfg.top_k) < GAP_MIN]
        if not bad:
            return q
        fresh = W.ivf_queries(cfg, p["centroids"], steps=1, salt=salt)[0]
        for b, h in bad:
            q[b, h] = fresh[b, h]
    raise RuntimeError("could not draw queries with the required top-k gap")


def _same_alt_rows(alt_gpu, alt_ref, valid):
    """alt rows of the valid entries, as sets: the order of a key's choices
    below its m-th does not decide any list membership."""
    a = np.sort(alt_gpu[valid], axis=-1)
    r = np.sort(alt_ref[valid], axis=-1)
    return np.array_equal(a, r)


# 3 x 2 KV heads: a wave per plan segment; 16 x 8: merged gather sets
@pytest.mark.parametrize("m", [3, 4])
@pytest.mark.parametrize("batch,n_kv_heads", [(3, 2), (16, 8)])
def test_m_way_lists_build_and_decode(m, batch, n_kv_heads):
    cfg, p = _problem(batch=batch, n_kv_heads=n_kv_heads, n_q_heads=4 * n_kv_heads)
    announce(f"multi: {m} lists per key, static build + decode, {batch} x {n_kv_heads}")
    p["keys"] = _m_way_keys(cfg, p["centroids"], m, 50 + m + batch)
    off, ids, alt = tsa.index_build_multi(p["keys"], p["centroids"], m)
    torch.cuda.synchronize()
    k64, c64, v64 = f64(p["keys"]), f64(p["centroids"]), f64(p["values"])
    r_off, r_ids, r_alt, margin = variants.index_build_multi(k64, c64, m)
    assert margin >= 1e-3, f"m-th choice margin {margin} too small for an exact comparison"
    assert tuple(alt.shape) == r_alt.shape
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert _same_alt_rows(alt.cpu().numpy(), r_alt, np.ones(r_ids.shape, dtype=bool))

    q = _queries(cfg, p)
    for kw in ({}, {"n_sink": 8, "n_window": 100}):
        sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
        out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, p["keys"], p["values"], cfg.top_k, alt=alt,
                                   sel_out=sel, **kw)
        torch.cuda.synchronize()
        r = variants.sparse_decode_ex(f64(q), c64, r_off, r_ids, k64, v64, cfg.top_k, **kw)
        assert np.all(r["gap"] >= GAP_MIN)
        assert np.array_equal(sel.cpu().numpy(), r["sel"])
        err = out_error(out.cpu().numpy(), r["out"])
        assert err <= OUT_TOL, f"output error {err} ({kw})"
    # tokens do sit in several chosen lists of one head: attending them once
    # per list instead of once would move the output well past the bar
    G, worst = cfg.group, 0.0
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            g = h // G
            rows = np.concatenate([r_ids[b, g][r_off[b, g][c]:r_off[b, g][c + 1]] for c in r["sel"][b, h]])
            o2, _ = ivf.attend(f64(q)[b, h], k64[b, rows, g], v64[b, rows, g])
            worst = max(worst, out_error(out.cpu().numpy()[b, h], o2))
    assert worst > 10 * OUT_TOL, "no token was in two chosen lists of a head; the case tests nothing"


@pytest.mark.parametrize("m", [2, 3])
@pytest.mark.parametrize("batch,n_kv_heads", [(3, 2), (16, 8)])
def test_growing_m_way_index_appends_and_decodes(m, batch, n_kv_heads):
    """Prefix build with free entries, then one all-or-nothing append per row
    (some lists run full, so some appends are refused), then a decode over the
    list lengths: lists, lengths, alt rows and statuses equal the oracle's own
    growing index; selection and output equal its decode over the compacted
    lists."""
    cfg, p = _problem(batch=batch, n_kv_heads=n_kv_heads, n_q_heads=4 * n_kv_heads, n_tokens=2400, n_centroids=24)
    announce(f"multi: growing index with {m} lists per key, {batch} x {n_kv_heads}")
    p["keys"] = _m_way_keys(cfg, p["centroids"], m, 70 + m + batch)
    n_prefix, n_add = 1800, 300
    slack = 12                                   # a list takes about n_add * m / C = 25-37 appends: some run full
    off, lens, ids, alt = tsa.index_build_dyn_multi(p["keys"], p["centroids"], n_prefix, m, slack)
    k_cache, v_cache = p["keys"].clone(), p["values"].clone()
    status = torch.empty((n_add, cfg.batch, cfg.n_kv_heads), dtype=torch.int32, device=DEV)
    for i in range(n_add):
        row = n_prefix + i
        pos = torch.full((cfg.batch,), row, dtype=torch.int32, device=DEV)
        tsa.kv_append(p["keys"][:, row].contiguous(), p["values"][:, row].contiguous(), pos, p["centroids"],
                      k_cache, v_cache, off, lens, ids, alt=alt, status=status[i])
    torch.cuda.synchronize()
    k64, c64, v64 = f64(p["keys"]), f64(p["centroids"]), f64(p["values"])
    B, Hkv, C, N = cfg.batch, cfg.n_kv_heads, cfg.n_centroids, cfg.n_tokens
    state = {(b, g): append.index_build_dynamic_multi(k64[b, :, g], c64[0, g], n_prefix, slack, m)
             for b in range(B) for g in range(Hkv)}
    K_ref, V_ref = k64.copy(), v64.copy()
    r_status = np.stack([append.append_step(state, k64[:, n_prefix + i], v64[:, n_prefix + i].copy(),
                                            np.full(B, n_prefix + i), c64, K_ref, V_ref) for i in range(n_add)])
    assert np.array_equal(status.cpu().numpy(), r_status)
    assert (r_status == 1).any() and (r_status == 0).any(), "the case needs both accepted and refused appends"
    og, lg, ig, ag = off.cpu().numpy(), lens.cpu().numpy(), ids.cpu().numpy(), alt.cpu().numpy()
    s_off = np.zeros((B, Hkv, C + 1), dtype=np.int64)
    s_ids = np.full((B, Hkv, N * m), -1, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            r_off, r_lens, r_ids, r_alt = state[(b, g)]
            assert np.array_equal(og[b, g], r_off) and np.array_equal(lg[b, g], r_lens)
            assert np.array_equal(ig[b, g], r_ids), f"growing lists differ (request {b}, KV head {g})"
            assert _same_alt_rows(ag[b, g], r_alt, r_ids >= 0)
            co, ci = append.compact(r_off, r_lens, r_ids)
            s_off[b, g], s_ids[b, g, :len(ci)] = co, ci
    assert np.array_equal(K_ref, f64(k_cache)) and np.array_equal(V_ref, f64(v_cache))
    q = _queries(cfg, p)
    sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
    lengths = torch.full((cfg.batch,), n_prefix + n_add, dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode_ex(q, p["centroids"], off, ids, k_cache, v_cache, cfg.top_k, lens=lens, alt=alt,
                               n_window=64, lengths=lengths, sel_out=sel)
    torch.cuda.synchronize()
    r = variants.sparse_decode_ex(f64(q), c64, s_off, s_ids, K_ref, V_ref, cfg.top_k, n_window=64,
                                  lengths=lengths.cpu().numpy())
    assert np.all(r["gap"] >= GAP_MIN)
    assert np.array_equal(sel.cpu().numpy(), r["sel"])
    err = out_error(out.cpu().numpy(), r["out"])
    assert err <= OUT_TOL, f"output error {err}"


@pytest.mark.parametrize("m", [1, 2])
def test_regrow_repairs_full_lists(m):
    """A growing index with no free entries refuses appends; regrow lays the
    same lists out again with the largest slack that fits (as the oracle's
    regrow does), the refused appends then go in, and the index decodes like
    the oracle's m-way lists over all those tokens."""
    cfg, p = _problem(batch=4, n_kv_heads=2, n_q_heads=8, n_tokens=2000, n_centroids=16)
    announce(f"multi: regrow of a full index, {m} lists per key")
    p["keys"] = _m_way_keys(cfg, p["centroids"], m, 90 + m)
    n_prefix, n_add = 1500, 40
    off, lens, ids, alt = tsa.index_build_dyn_multi(p["keys"], p["centroids"], n_prefix, m, 0)
    rows = torch.arange(n_prefix, n_prefix + n_add, device=DEV)

    def append_rows(off, lens, ids, alt):
        st = torch.empty((n_add, cfg.batch, cfg.n_kv_heads), dtype=torch.int32, device=DEV)
        for i in range(n_add):
            pos = torch.full((cfg.batch,), int(rows[i]), dtype=torch.int32, device=DEV)
            tsa.kv_append(p["keys"][:, rows[i]].contiguous(), p["values"][:, rows[i]].contiguous(), pos,
                          p["centroids"], p["keys"], p["values"], off, lens, ids, alt=alt, status=st[i])
        return st

    st0 = append_rows(off, lens, ids, alt)
    torch.cuda.synchronize()
    assert int(st0.min()) == 1, "with no free entries every append is refused"
    (n_off, n_lens, n_ids, n_alt), status = tsa.index_regrow(off, lens, ids, alt)
    torch.cuda.synchronize()
    assert int(status.max()) == 0
    k64, c64, v64 = f64(p["keys"]), f64(p["centroids"]), f64(p["values"])
    B, Hkv, N = cfg.batch, cfg.n_kv_heads, cfg.n_tokens
    for b in range(B):
        for g in range(Hkv):
            o0, l0, i0, a0 = append.index_build_dynamic_multi(k64[b, :, g], c64[0, g], n_prefix, 0, m)
            slack = append.regrow_slack(l0, N * m)
            r_off, r_lens, r_ids, r_alt = append.regrow(o0, l0, i0, a0, slack)
            assert np.array_equal(n_off[b, g].cpu().numpy(), r_off)
            assert np.array_equal(n_lens[b, g].cpu().numpy(), r_lens)
            assert np.array_equal(n_ids[b, g].cpu().numpy(), r_ids)
            if m > 1:
                assert _same_alt_rows(n_alt[b, g].cpu().numpy(), r_alt, r_ids >= 0)
    st1 = append_rows(n_off, n_lens, n_ids, n_alt)
    torch.cuda.synchronize()
    assert int(st1.max()) == 0, "after the regrow every refused append goes in"
    # the repaired index holds the m-way lists of the first n_prefix + n_add keys
    for b in range(B):
        for g in range(Hkv):
            s_off, s_ids, _, _ = variants.index_build_multi(k64[b:b + 1, :n_prefix + n_add, g:g + 1],
                                                            c64[:, g:g + 1], m)
            co, ci = append.compact(n_off[b, g].cpu().numpy(), n_lens[b, g].cpu().numpy(),
                                    n_ids[b, g].cpu().numpy())
            assert np.array_equal(co, s_off[0, 0]) and np.array_equal(ci, s_ids[0, 0])
    q = _queries(cfg, p)
    sel = torch.empty((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode_ex(q, p["centroids"], n_off, n_ids, p["keys"], p["values"], cfg.top_k, lens=n_lens,
                               alt=n_alt, sel_out=sel)
    torch.cuda.synchronize()
    full_off = np.zeros((B, Hkv, cfg.n_centroids + 1), dtype=np.int64)
    full_ids = np.full((B, Hkv, N * m), -1, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            co, ci = append.compact(n_off[b, g].cpu().numpy(), n_lens[b, g].cpu().numpy(), n_ids[b, g].cpu().numpy())
            full_off[b, g], full_ids[b, g, :len(ci)] = co, ci
    r = variants.sparse_decode_ex(f64(q), c64, full_off, full_ids, k64, v64, cfg.top_k)
    assert np.array_equal(sel.cpu().numpy(), r["sel"])
    assert out_error(out.cpu().numpy(), r["out"]) <= OUT_TOL


def test_regrow_reports_lists_that_do_not_fit():
    cfg, p = _problem(batch=2, n_kv_heads=2, n_q_heads=8, n_tokens=1000, n_centroids=16)
    announce("multi: regrow with too much slack")
    off, lens, ids, alt = tsa.index_build_dyn_multi(p["keys"], p["centroids"], 900, 1, 0)
    out0 = (torch.full_like(off, -7), torch.full_like(lens, -7), torch.full_like(ids, -7), None)
    out, status = tsa.index_regrow(off, lens, ids, None, slack=100, out=out0)
    torch.cuda.synchronize()
    assert torch.equal(status, torch.ones_like(status))
    assert all(int(t.min()) == -7 and int(t.max()) == -7 for t in out[:3])


@pytest.mark.parametrize("m", [2, 3])
def test_m_way_build_with_a_large_codebook(m):
    """C above the per-wave counter limit (1024 lists): the posting lists and
    alt rows come from the one-workgroup CSR kernel."""
    cfg, p = _problem(batch=1, n_kv_heads=2, n_q_heads=8, n_tokens=2500, n_centroids=1100, top_k=8)
    announce(f"multi: {m} lists per key, C = 1100")
    p["keys"] = _m_way_keys(cfg, p["centroids"], m, 110 + m)
    off, ids, alt = tsa.index_build_multi(p["keys"], p["centroids"], m)
    torch.cuda.synchronize()
    r_off, r_ids, r_alt, margin = variants.index_build_multi(f64(p["keys"]), f64(p["centroids"]), m)
    assert margin >= 1e-3, f"m-th choice margin {margin} too small for an exact comparison"
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(ids.cpu().numpy(), r_ids)
    assert _same_alt_rows(alt.cpu().numpy(), r_alt, np.ones(r_ids.shape, dtype=bool))
