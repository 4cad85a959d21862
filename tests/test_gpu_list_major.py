"""List-major K/V copies (tsa_kv_list_major): each posting list's rows laid
out contiguously, as an inverted file keeps its entries ([KARAT] How, index
structure). The copy must be exactly the cache rows in list order, and a
decode that reads the chosen lists from it must reproduce the decode that
reads the caches by row id: the same rows, in the same order, so the same
selections, counts and outputs bit for bit, under every schedule; one request
is also checked against the oracle."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import ivf
from top_sparse_attention_centroid_amd import workloads as W

from helpers import OUT_TOL, announce, conditioned_ivf_queries, f64, out_error
from test_gpu_ivf import _check_index, _problem

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _copy_ref(ids, cache):
    """cache[b][ids[b][g][e]][g] for every (b, g, e); zero rows where the id
    lies outside [0, N)."""
    B, N, Hkv, d = cache.shape
    safe = ids.clamp(0, N - 1).long()
    ref = torch.stack([cache[b][safe[b].T, torch.arange(Hkv, device=cache.device)].permute(1, 0, 2)
                       for b in range(B)])
    return torch.where((ids >= 0)[..., None] & (ids < N)[..., None], ref, torch.zeros_like(ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_is_the_cache_rows_in_list_order(dtype):
    """Static index (every entry a token) and a growing index's layout
    (free entries, id -1, become zero rows); N not a multiple of the copy
    kernel's 256 entries."""
    cfg = W.config(2, batch=3, n_tokens=5000, n_centroids=40, top_k=4, n_kv_heads=2, n_q_heads=8, steps=1,
                   dtype=dtype, seed=71)
    announce(f"kv_list_major copy dtype={dtype}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    kl, vl = tsa.kv_list_major(ids, p["keys"], p["values"])
    torch.cuda.synchronize()
    assert torch.equal(kl, _copy_ref(ids, p["keys"])) and torch.equal(vl, _copy_ref(ids, p["values"]))
    off_d, lens_d, ids_d = tsa.index_build_dyn(p["keys"], p["centroids"], 3000, 7)
    assert int((ids_d < 0).sum()) > 0
    kl, vl = tsa.kv_list_major(ids_d, p["keys"], p["values"])
    torch.cuda.synchronize()
    assert torch.equal(kl, _copy_ref(ids_d, p["keys"])) and torch.equal(vl, _copy_ref(ids_d, p["values"]))


def _decode(q, p, offsets, ids, k, schedule, lists=None, **kw):
    B, Hq, _ = q.shape
    Hkv = ids.shape[1]
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    rows = torch.empty((B, Hq), dtype=torch.int32, device=DEV)
    uniq = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    kl, vl = lists if lists is not None else (None, None)
    out = tsa.sparse_decode_ex(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, schedule=schedule,
                               k_lists=kl, v_lists=vl, sel_out=sel, rows_out=rows, uniq_out=uniq, **kw)
    torch.cuda.synchronize()
    return sel, rows, uniq, out


CASES = [
    # (name, config overrides, schedules): one request of 30K tokens (split and
    # fused per head, staged with a wave per segment), a batch large enough for
    # the merged gather sets, fp32
    ("one-request", dict(batch=1, n_tokens=30_000, n_kv_heads=4, n_q_heads=16, n_centroids=300, top_k=10,
                         shared_codebook=False), ("auto", "staged", "split", "fused")),
    ("batched", dict(batch=40, n_tokens=4096, n_kv_heads=4, n_q_heads=16, n_centroids=64, top_k=6),
     ("auto", "staged")),
    ("f32", dict(batch=2, n_tokens=6000, n_kv_heads=2, n_q_heads=8, n_centroids=50, top_k=5, dtype="f32",
                 shared_codebook=False), ("auto", "staged", "fused")),
]


@pytest.mark.parametrize("name,over,schedules", CASES, ids=[c[0] for c in CASES])
def test_decode_from_the_copies_matches_the_cache_decode(name, over, schedules):
    cfg = W.config(1 if over.get("shared_codebook") is False else 2, steps=1, seed=72, **over)
    announce(f"list-major decode {name}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    lists = tsa.kv_list_major(ids, p["keys"], p["values"])
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    for schedule in schedules:
        for sim in ("dot", "cosine"):
            a = _decode(q, p, offsets, ids, cfg.top_k, schedule, similarity=sim)
            b = _decode(q, p, offsets, ids, cfg.top_k, schedule, lists=lists, similarity=sim)
            for x, y, what in zip(a, b, ("selection", "row counts", "union counts", "outputs")):
                assert torch.equal(x, y), f"{name}, {schedule}, {sim}: {what} differ with the list-major copies"
    # one request against the oracle, through the copies
    ref = _check_index(p, [0], offsets, ids)
    _, _, _, out = _decode(q, p, offsets, ids, cfg.top_k, "auto", lists=lists)
    r = ivf.sparse_decode(f64(q[0:1]), f64(p["centroids"][0:1]), ref[0][0][None], ref[0][1][None],
                          f64(p["keys"][0:1]), f64(p["values"][0:1]), cfg.top_k)
    assert out_error(out[0].cpu().numpy(), r["out"][0]) <= OUT_TOL


def test_copies_of_another_index_change_only_the_rows_read():
    """The copies are read by list entry: copies built for this index but
    with the value rows of another cache give the decode over that cache
    (same lists and counts, the other values' outputs)."""
    cfg = W.config(2, batch=2, n_tokens=4000, n_centroids=32, top_k=4, n_kv_heads=2, n_q_heads=8, steps=1, seed=73)
    announce("list-major copies read by entry")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    v2 = torch.randn_like(p["values"])
    kl, _ = tsa.kv_list_major(ids, p["keys"], p["values"])
    _, vl2 = tsa.kv_list_major(ids, p["keys"], v2)
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    a = _decode(q, p, offsets, ids, cfg.top_k, "staged", lists=(kl, vl2))
    p2 = dict(p, values=v2)
    b = _decode(q, p2, offsets, ids, cfg.top_k, "staged")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
