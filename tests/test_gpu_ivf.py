"""GPU parity of the inverted-index path (index build, centroid scoring, top-k
lists, gathered attention) against the fp64 oracle, through the C ABI.

Bars: posting lists and selected lists bit-exact; per-head row counts exact;
outputs within OUT_TOL = 2e-3 (max over heads of the inf-norm error relative to
the inf-norm of the oracle output)."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import ivf
from top_sparse_attention_centroid_amd import workloads as W

from helpers import (GAP_MIN, MARGIN_MIN, OUT_TOL, announce, conditioned_ivf_queries, f64,
                      oracle_index, out_error)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _problem(cfg):
    p = W.ivf_problem(cfg, device=DEV)
    torch.cuda.synchronize()
    return p


def _check_index(p, requests, offsets, ids):
    ref, margin = oracle_index(p["keys"], p["centroids"], requests)
    assert margin >= MARGIN_MIN, f"assignment margin {margin} too small for an exact comparison"
    off_g, ids_g = offsets.cpu().numpy(), ids.cpu().numpy()
    for b in requests:
        assert np.array_equal(off_g[b], ref[b][0]), f"offsets differ (request {b})"
        assert np.array_equal(ids_g[b], ref[b][1]), f"ids differ (request {b})"
    return ref


def _f32(t: torch.Tensor) -> np.ndarray:
    """Host copy widened to fp32 (exact for bf16 and fp32 storage); the oracle
    widens it to fp64 itself."""
    return t.detach().to("cpu", torch.float32).numpy()


def _decode(schedule, q, p, offsets, ids, k, **kw):
    """One decode step under `schedule`: "auto" through tsa_sparse_decode (the
    library's choice), "staged" or "fused" through tsa_sparse_decode_ex."""
    if schedule == "auto":
        return tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, **kw)
    return tsa.sparse_decode_ex(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, schedule=schedule, **kw)


def _decode_and_check(cfg, p, ref_lists, requests, steps, q=None, sel_requests=(), schedule="auto"):
    """Decodes `steps` steps of the whole batch and checks `requests` in full
    (selection, row counts, unique rows, outputs) against the oracle's own
    index; `sel_requests` get their selections checked too (scores alone)."""
    B, Hq, Hkv, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    if q is None:
        q = conditioned_ivf_queries(cfg, p["centroids"], steps)
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    rows = torch.empty((B, Hq), dtype=torch.int32, device=DEV)
    uniq = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    K64 = {b: _f32(p["keys"][b:b + 1]) for b in requests}
    V64 = {b: _f32(p["values"][b:b + 1]) for b in requests}
    cent64 = f64(p["centroids"])
    for t in range(steps):
        out = _decode(schedule, q[t], p, offsets, ids, k, sel_out=sel, rows_out=rows, uniq_out=uniq)
        torch.cuda.synchronize()
        q64 = f64(q[t])
        out_g, sel_g, rows_g, uniq_g = out.cpu().numpy(), sel.cpu().numpy(), rows.cpu().numpy(), uniq.cpu().numpy()
        for b in sel_requests:
            cb = cent64[0 if cent64.shape[0] == 1 else b]
            for h in range(Hq):
                s_bh = ivf.centroid_scores(q64[b, h], cb[h // (Hq // Hkv)])
                assert ivf.selection_gap(s_bh, k) >= GAP_MIN
                assert np.array_equal(sel_g[b, h], ivf.top_k(s_bh, k)), f"selection differs (step {t}, {b}, {h})"
        for b in requests:
            off_b = ref_lists[b][0][None]
            ids_b = ref_lists[b][1][None]
            cb = cent64[0:1] if cent64.shape[0] == 1 else cent64[b:b + 1]
            r = ivf.sparse_decode(q64[b:b + 1], cb, off_b, ids_b, K64[b], V64[b], k)
            assert np.all(r["gap"] >= GAP_MIN)
            assert np.array_equal(sel_g[b], r["sel"][0]), f"selection differs (step {t}, request {b})"
            assert np.array_equal(rows_g[b], r["n_rows"][0])
            for g in range(Hkv):
                G = Hq // Hkv
                union = set()
                for h in range(g * G, (g + 1) * G):
                    union |= set(ivf.retrieved_rows(r["sel"][0, h], ref_lists[b][0][g], ref_lists[b][1][g]).tolist())
                assert uniq_g[b, g] == len(union)
            err = out_error(out_g[b], r["out"][0])
            assert err <= OUT_TOL, f"output error {err} (step {t}, request {b})"
    return q


@pytest.mark.parametrize("schedule", ["auto", "staged"])
def test_tiny_fp32_workload(schedule):
    cfg = W.config(0)
    announce(f"ivf {cfg.name} schedule={schedule}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, [0], offsets, ids)
    _decode_and_check(cfg, p, ref, [0], steps=4, schedule=schedule)


# the split schedule scores bf16 codebooks only
@pytest.mark.parametrize("dtype,schedule", [("f32", "fused"), ("f32", "staged"), ("bf16", "fused"),
                                            ("bf16", "split"), ("bf16", "staged")])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_ragged_shapes(dtype, G, schedule):
    # N not a multiple of any tile, odd C, lists longer than one segment (and,
    # fused, than one round of a head's rows over the workgroup's waves)
    cfg = W.config(1, batch=3, n_tokens=3001, n_kv_heads=2, n_q_heads=2 * G, n_centroids=7,
                   top_k=3, dtype=dtype, steps=2, shared_codebook=(G % 2 == 0), seed=11 + G)
    announce(f"ivf ragged dtype={dtype} G={G} schedule={schedule}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, range(cfg.batch), offsets, ids)
    _decode_and_check(cfg, p, ref, range(cfg.batch), steps=2, schedule=schedule)


# bf16 nearest-centroid search on matrix cores: fewer keys than one 16-key
# tile, and codebooks whose last 256-centroid stage holds 1 or 16 centroids
@pytest.mark.parametrize("n_tokens,C", [(1, 3), (5, 257), (17, 16), (600, 272)])
def test_index_build_tile_and_stage_edges(n_tokens, C):
    cfg = W.config(1, batch=2, n_tokens=n_tokens, n_kv_heads=2, n_q_heads=8, n_centroids=C, top_k=1,
                   steps=1, seed=5 + C)
    announce(f"ivf index build edges N={n_tokens} C={C}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    torch.cuda.synchronize()
    _check_index(p, range(cfg.batch), offsets, ids)


def test_selecting_every_list_is_dense_attention():
    cfg = W.config(1, batch=2, n_tokens=777, n_kv_heads=2, n_q_heads=8, n_centroids=5, top_k=5,
                   steps=1, shared_codebook=True, seed=21)
    announce("ivf k == C")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    q = W.ivf_queries(cfg, p["centroids"], steps=1)
    out = tsa.sparse_decode(q[0], p["centroids"], offsets, ids, p["keys"], p["values"], cfg.top_k)
    K, V, q64 = f64(p["keys"]), f64(p["values"]), f64(q[0])
    ref = np.empty_like(out.cpu().numpy(), dtype=np.float64)
    for b in range(cfg.batch):
        for h in range(cfg.n_q_heads):
            g = h // cfg.group
            ref[b, h], _ = ivf.attend(q64[b, h], K[b, :, g], V[b, :, g])
    assert out_error(out.cpu().numpy(), ref) <= OUT_TOL


@pytest.mark.parametrize("dtype,schedule", [("f32", "auto"), ("f32", "staged"), ("bf16", "fused"),
                                            ("bf16", "split"), ("bf16", "staged")])
def test_empty_selection_gives_zero_and_flag(dtype, schedule):
    # Small centroids live in dims 0..63, three far centroids in dims 64..127 and
    # own no keys. Head 0's query is a far centroid, so its top-1 list is empty
    # (under the split schedule every share of head 0 attends no row); head 1's
    # query is small centroid 1 itself (orthogonal to every far one).
    g = torch.Generator().manual_seed(0)
    B, N, Hkv, G, C, d = 1, 600, 1, 2, 8, 128
    cent = torch.zeros(1, Hkv, C, d)
    cent[0, 0, :5, :64] = torch.randn(5, 64, generator=g)
    cent[0, 0, 5:, 64:] = 40.0 * torch.randn(3, 64, generator=g)
    comp = torch.randint(0, 5, (N,), generator=g)
    keys = (cent[0, 0, comp] + 0.3 * torch.randn(N, d, generator=g)).view(B, N, Hkv, d)
    vals = torch.randn(B, N, Hkv, d, generator=g)
    q = torch.stack([cent[0, 0, 6], cent[0, 0, 1]]).view(B, G, d)
    announce(f"ivf empty selection dtype={dtype} schedule={schedule}")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    keys, vals, cent, q = (x.to(DEV, dt) for x in (keys, vals, cent, q))
    offsets, ids = tsa.index_build(keys, cent)
    rows = torch.empty((B, G), dtype=torch.int32, device=DEV)
    sel = torch.empty((B, G, 1), dtype=torch.int32, device=DEV)
    p = {"centroids": cent, "keys": keys, "values": vals}
    out = _decode(schedule, q, p, offsets, ids, 1, rows_out=rows, sel_out=sel)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert sel[0, 0, 0].item() == 6 and sel[0, 1, 0].item() == 1
    assert rows[0, 0].item() == 0 and np.all(o[0, 0] == 0.0)
    assert rows[0, 1].item() > 0
    off_o, ids_o, _ = ivf.index_build(f64(keys), f64(cent))
    r = ivf.decode_head(f64(q[0, 1]), f64(cent[0, 0]), off_o[0, 0], ids_o[0, 0],
                        f64(keys[0, :, 0]), f64(vals[0, :, 0]), 1)
    assert r.empty is False and len(r.rows) == rows[0, 1].item()
    assert out_error(o[0, 1], r.out) <= OUT_TOL


def test_batched_workload_full_size():
    """64 requests x 32K tokens, shared codebook C=256, top-16: the selections
    of all 64 requests are checked; eight requests spread over the batch
    (including the last) are checked in full by the oracle (its own index,
    its own selection, row counts and outputs)."""
    cfg = W.config(2)
    announce(f"ivf {cfg.name} full size")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    sample = [0, 9, 18, 27, 36, 45, 54, 63]
    ref = _check_index(p, sample, offsets, ids)
    q = _decode_and_check(cfg, p, ref, sample, steps=2, sel_requests=range(cfg.batch))
    # determinism: a second identical call is bitwise identical
    o1 = tsa.sparse_decode(q[0], p["centroids"], offsets, ids, p["keys"], p["values"], cfg.top_k)
    o2 = tsa.sparse_decode(q[0], p["centroids"], offsets, ids, p["keys"], p["values"], cfg.top_k)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("schedule", ["auto", "fused", "staged"])
def test_karat_shape_full_size(schedule):
    """1 request x 100,000 tokens, 8 KV / 32 query heads, C=1000 per KV head,
    top-10: the split launches (the library's choice here), the fused single
    launch and the staged launches."""
    cfg = W.config(1)
    announce(f"ivf {cfg.name} full size schedule={schedule}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, [0], offsets, ids)
    _decode_and_check(cfg, p, ref, [0], steps=2, schedule=schedule)


# the per-head schedules hold k <= 64 lists
@pytest.mark.parametrize("C,k,schedule", [(C, k, s) for C, k in ((300, 10), (300, 64), (300, 100), (1000, 10))
                                          for s in ("auto", "staged", "fused", "split") if k <= 64 or s in ("auto", "staged")])
def test_top_k_paths_and_ties(C, k, schedule):
    """Selections through every search of the k-th largest score: the short
    candidate search (k <= 64, several keys per lane), its fallback when more
    than 64 keys reach the candidate bound (an all-zero query ties every
    list), and the full search (k > 64). Bit-exact against the oracle's top-k,
    ties to the lower list id; outputs against the oracle."""
    cfg = W.config(1, batch=2, n_tokens=8000, n_kv_heads=2, n_q_heads=8, n_centroids=C, top_k=k, steps=1,
                   shared_codebook=True, seed=31)
    announce(f"ivf top-k paths C={C} k={k} schedule={schedule}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, range(cfg.batch), offsets, ids)
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0].clone()
    zero = {(0, 1), (1, 6)}
    for b, h in zero:
        q[b, h] = 0
    B, Hq, G = cfg.batch, cfg.n_q_heads, cfg.group
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    out = _decode(schedule, q, p, offsets, ids, k, sel_out=sel)
    torch.cuda.synchronize()
    q64, c64, K, V = f64(q), f64(p["centroids"]), f64(p["keys"]), f64(p["values"])
    sel_g, out_g = sel.cpu().numpy(), out.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            g = h // G
            r = ivf.decode_head(q64[b, h], c64[0, g], ref[b][0][g], ref[b][1][g], K[b, :, g], V[b, :, g], k)
            if (b, h) in zero:
                assert np.array_equal(sel_g[b, h], np.arange(k)), "all-equal scores must take the lowest list ids"
            assert np.array_equal(sel_g[b, h], r.lists), f"selection differs (request {b}, head {h})"
            assert out_error(out_g[b, h], r.out) <= OUT_TOL


@pytest.mark.parametrize("k", [3, 5, 7])
def test_exact_ties_among_the_top_lists(k):
    """Five identical centroid rows (lists 7, 100, 101, 102, 103) hold the
    largest score of a query that equals them: their scores tie exactly, in
    the candidate ranking of the selection. k = 3 takes three of the five
    (the lowest ids), k = 5 all of them, k = 7 all plus the next two. The
    lists of every schedule equal the oracle's top-k (ties to the lower id);
    outputs agree across schedules. (Keys assigned to identical centroids
    tie too, so the index is not compared with the oracle's here.)"""
    cfg = W.config(1, batch=2, n_tokens=8000, n_kv_heads=2, n_q_heads=8, n_centroids=300, top_k=k, steps=1,
                   shared_codebook=True, seed=33)
    announce(f"ivf exact ties k={k}")
    p = _problem(cfg)
    cent = p["centroids"].clone()
    for c in (100, 101, 102, 103):
        cent[:, :, c] = cent[:, :, 7]
    p = dict(p, centroids=cent)
    offsets, ids = tsa.index_build(p["keys"], cent)
    q = W.ivf_queries(cfg, cent, steps=1)[0].clone()
    q[0, 1] = cent[0, 0, 7]      # request 0, head 1 (KV head 0)
    q[1, 6] = cent[0, 1, 7]      # request 1, head 6 (KV head 1)
    B, Hq, G = cfg.batch, cfg.n_q_heads, cfg.group
    q64, c64 = f64(q), f64(cent)
    # the tied heads against the oracle (the other heads' random queries are
    # not conditioned on a score gap: they are compared across schedules only)
    want = {(b, h): ivf.top_k(ivf.centroid_scores(q64[b, h], c64[0, h // G]), k) for b, h in ((0, 1), (1, 6))}
    tied = [7, 100, 101, 102, 103]
    for w in want.values():  # the oracle's own reading of the ties
        assert set(tied[:min(k, 5)]) <= set(w.tolist()) and (k > 5 or not set(tied[k:]) & set(w.tolist()))
    outs, sels = {}, {}
    for schedule in ("staged", "fused", "split"):
        sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
        outs[schedule] = _decode(schedule, q, p, offsets, ids, k, sel_out=sel)
        torch.cuda.synchronize()
        sels[schedule] = sel
        sel_g = sel.cpu().numpy()
        for (b, h), w in want.items():
            assert np.array_equal(sel_g[b, h], w), f"{schedule}: selection differs (request {b}, head {h})"
    for schedule in ("fused", "split"):
        assert torch.equal(sels[schedule], sels["staged"])
        assert out_error(outs[schedule].cpu().numpy(), outs["staged"].cpu().numpy()) <= 1e-4


def test_split_and_fused_scoring_choose_the_same_lists():
    """Staged small batches score the centroids in a launch of their own,
    large ones inside the selection kernel, and the fused decode inside its
    one workgroup per head; all run the same per-tile contraction, so a
    request selects the same lists every way (and the outputs match the
    oracle)."""
    cfg = W.config(2, batch=16, n_tokens=2048, n_centroids=200, top_k=12, steps=1)  # 128 groups: in-select
    announce("ivf split vs fused scoring")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0].clone()
    q[1, 3] = 0  # every list ties: the candidate search falls back to the full one
    B, Hq, k = cfg.batch, cfg.n_q_heads, cfg.top_k
    sel_big = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    out_big = tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, sel_out=sel_big)
    n = 2  # 16 groups: split (staged) or fused
    part = {"centroids": p["centroids"], "keys": p["keys"][:n].contiguous(), "values": p["values"][:n].contiguous()}
    sel_small = torch.empty((n, Hq, k), dtype=torch.int32, device=DEV)
    out_small = _decode("staged", q[:n].contiguous(), part, offsets[:n].contiguous(), ids[:n].contiguous(), k,
                        sel_out=sel_small)
    sel_fused = torch.empty((n, Hq, k), dtype=torch.int32, device=DEV)
    out_fused = _decode("fused", q[:n].contiguous(), part, offsets[:n].contiguous(), ids[:n].contiguous(), k,
                        sel_out=sel_fused)
    sel_split = torch.empty((n, Hq, k), dtype=torch.int32, device=DEV)
    out_split = _decode("split", q[:n].contiguous(), part, offsets[:n].contiguous(), ids[:n].contiguous(), k,
                        sel_out=sel_split)
    torch.cuda.synchronize()
    assert torch.equal(sel_small, sel_big[:n])
    assert torch.equal(sel_fused, sel_big[:n])
    assert torch.equal(sel_split, sel_big[:n])
    assert np.array_equal(sel_big[1, 3].cpu().numpy(), np.arange(k))
    ref = _check_index(p, [0], offsets, ids)
    r = ivf.sparse_decode(f64(q[0:1]), f64(p["centroids"]), ref[0][0][None], ref[0][1][None],
                          f64(p["keys"][0:1]), f64(p["values"][0:1]), k)
    assert np.array_equal(sel_small[0].cpu().numpy(), r["sel"][0])
    assert out_error(out_small[0].cpu().numpy(), r["out"][0]) <= OUT_TOL
    assert out_error(out_fused[0].cpu().numpy(), r["out"][0]) <= OUT_TOL
    assert out_error(out_split[0].cpu().numpy(), r["out"][0]) <= OUT_TOL
    assert out_error(out_big[0].cpu().numpy(), r["out"][0]) <= OUT_TOL


@pytest.mark.parametrize("k", [8, 12, 16])
def test_plan_segment_lengths(k):
    """2 requests x 8 KV heads with ~200-row lists: k = 8, 12, 16 cut the lists
    into 64-, 128- and 256-row plan segments (several per list, ragged tails).
    Selections, row counts and outputs against the oracle."""
    cfg = W.config(2, batch=2, n_tokens=6400, n_centroids=32, top_k=k, steps=1, seed=41 + k)
    announce(f"ivf plan segments k={k}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, range(cfg.batch), offsets, ids)
    _decode_and_check(cfg, p, ref, range(cfg.batch), steps=1, schedule="staged")


@pytest.mark.parametrize("dtype,G,C,k", [("bf16", 4, 2048, 10), ("bf16", 4, 2048, 100), ("bf16", 8, 1500, 12),
                                         ("f32", 2, 1200, 8)])
def test_large_codebooks(dtype, G, C, k):
    """Codebooks above 1024 centroids (64 keys per lane in the selection),
    with k on both sides of the 64-key candidate bound; bf16 scores on
    matrix cores, fp32 on the vector units. Index, selections, row counts and
    outputs against the oracle."""
    cfg = W.config(1, batch=2, n_tokens=20_000, n_kv_heads=2, n_q_heads=2 * G, n_centroids=C, top_k=k,
                   dtype=dtype, steps=1, shared_codebook=False, seed=51 + k)
    announce(f"ivf large codebook dtype={dtype} G={G} C={C} k={k}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, range(cfg.batch), offsets, ids)
    _decode_and_check(cfg, p, ref, range(cfg.batch), steps=1)


def test_split_and_fused_cosine_scores_choose_the_same_lists():
    """Cosine scoring (q.c / |c|) inside the selection kernel (128 groups) and in
    its own launch (16 groups) chooses the same lists for the same requests."""
    cfg = W.config(2, batch=16, n_tokens=2048, n_centroids=200, top_k=12, steps=1, seed=7)
    announce("ivf split vs fused cosine scoring")
    p = _problem(cfg)
    # centroids of very different norms, so cosine and dot rankings differ
    scale = torch.exp(torch.linspace(-1.5, 1.5, cfg.n_centroids, device=DEV)).view(1, 1, -1, 1)
    cent = (p["centroids"].float() * scale).to(p["centroids"].dtype)
    offsets, ids = tsa.index_build(p["keys"], cent)
    q = conditioned_ivf_queries(cfg, cent, 1)[0]
    B, Hq, k = cfg.batch, cfg.n_q_heads, cfg.top_k
    sel_big = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    out_big = tsa.sparse_decode_ex(q, cent, offsets, ids, p["keys"], p["values"], k, similarity="cosine",
                                   sel_out=sel_big)
    n = 2
    small = {}
    for schedule in ("staged", "fused", "split"):
        sel_small = torch.empty((n, Hq, k), dtype=torch.int32, device=DEV)
        out_small = tsa.sparse_decode_ex(q[:n].contiguous(), cent, offsets[:n].contiguous(), ids[:n].contiguous(),
                                         p["keys"][:n].contiguous(), p["values"][:n].contiguous(), k,
                                         similarity="cosine", sel_out=sel_small, schedule=schedule)
        small[schedule] = (sel_small, out_small)
    sel_dot = torch.empty_like(sel_big)
    tsa.sparse_decode(q, cent, offsets, ids, p["keys"], p["values"], k, sel_out=sel_dot)
    torch.cuda.synchronize()
    sel_small, out_small = small["staged"]
    assert torch.equal(sel_small, sel_big[:n])
    for schedule in ("fused", "split"):
        assert torch.equal(small[schedule][0], sel_big[:n])
        assert out_error(small[schedule][1].cpu().numpy(), out_big[:n].cpu().numpy()) <= 1e-4
    assert not torch.equal(sel_big, sel_dot), "the scaled codebook should make cosine and dot choose differently"
    assert out_error(out_small.cpu().numpy(), out_big[:n].cpu().numpy()) <= 1e-4
