"""Bound calls (bind=True): a decode whose arguments were checked and
marshalled once, issued again per step. The kernels and their inputs are the
same as the direct call's, so the outputs are bit-identical to it, and a
bound call reads whatever its tensors hold when it runs."""

import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from top_sparse_attention_centroid_amd import workloads as W

from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("cfg_id", [0, 1])
def test_bound_sparse_decode_matches_the_direct_call(cfg_id):
    cfg = W.config(cfg_id, n_tokens=20_000, steps=3) if cfg_id == 1 else W.config(0, steps=3)
    announce(f"bound sparse_decode, config {cfg_id}")
    p = W.ivf_problem(cfg, device=DEV)
    qs = W.ivf_queries(cfg, p["centroids"], steps=3)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    B, Hq, Hkv, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k
    q = qs[0].clone()
    out = torch.empty((B, Hq, cfg.head_dim), dtype=torch.float32, device=DEV)
    uniq = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
    call = tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, out=out, uniq_out=uniq,
                             bind=True)
    assert isinstance(call, tsa.BoundCall)
    for j in range(3):
        q.copy_(qs[j])
        assert call() is out
        got, got_u = out.clone(), uniq.clone()
        want_u = torch.empty_like(uniq)
        want = tsa.sparse_decode(qs[j], p["centroids"], offsets, ids, p["keys"], p["values"], k, uniq_out=want_u)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {j}: outputs differ"
        assert torch.equal(got_u, want_u), f"step {j}: union counts differ"


def test_bound_token_decode_matches_the_direct_call():
    cfg = W.config(3, batch=3, n_tokens=30_001, top_k=700, n_planted=32, steps=2)
    announce("bound token_decode")
    prob = W.token_problem(cfg, device=DEV)
    q_idx, q = W.token_queries(cfg, prob, steps=2)
    qi, qa = q_idx[0].clone(), q[0].clone()
    sel = torch.empty((cfg.batch, cfg.top_k), dtype=torch.int32, device=DEV)
    call = tsa.token_decode(qi, prob["k_idx"], qa, prob["keys"], prob["values"], cfg.top_k, sel_out=sel, bind=True)
    for j in range(2):
        qi.copy_(q_idx[j])
        qa.copy_(q[j])
        got = call().clone()
        got_sel = sel.clone()
        want_sel = torch.empty_like(sel)
        want = tsa.token_decode(q_idx[j], prob["k_idx"], q[j], prob["keys"], prob["values"], cfg.top_k,
                                sel_out=want_sel)
        torch.cuda.synchronize()
        assert torch.equal(got_sel, want_sel), f"step {j}: selections differ"
        assert torch.equal(got, want), f"step {j}: outputs differ"



def test_bound_growing_index_steps_match_the_direct_calls():
    """Decode over a growing index and append the step's token, three steps,
    once through bound calls (bound before the first step) and once through
    direct calls on copies of the same cache and lists: the same outputs,
    statuses, lengths and list entries."""
    cfg = W.config(1, batch=2, n_tokens=6000, n_kv_heads=2, n_q_heads=8, n_centroids=50, top_k=5, steps=3,
                   shared_codebook=False, seed=66)
    announce("bound growing-index steps")
    p = W.ivf_problem(cfg, device=DEV)
    qs = W.ivf_queries(cfg, p["centroids"], steps=3)
    prefix, steps = 5000, 3
    B, Hq, Hkv, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k
    off, lens, ids = tsa.index_build_dyn(p["keys"], p["centroids"], prefix, 20)
    new_k = p["keys"][:, prefix:prefix + steps].transpose(0, 1).contiguous()
    new_v = p["values"][:, prefix:prefix + steps].transpose(0, 1).contiguous()
    pos = (prefix + torch.arange(steps, device=DEV, dtype=torch.int32))[:, None].expand(steps, B).contiguous()
    runs = []
    for bound in (True, False):
        kc, vc, ln, ix = p["keys"].clone(), p["values"].clone(), lens.clone(), ids.clone()
        out = torch.empty((steps, B, Hq, cfg.head_dim), dtype=torch.float32, device=DEV)
        st = torch.empty((steps, B, Hkv), dtype=torch.int32, device=DEV)
        calls = []
        for i in range(steps):
            kw = dict(out=out[i], bind=True) if bound else dict(out=out[i])
            dec = lambda i=i, kw=kw: tsa.sparse_decode_dyn(qs[i], p["centroids"], off, ln, ix, kc, vc, k, **kw)
            app = lambda i=i, b=bound: tsa.kv_append(new_k[i], new_v[i], pos[i], p["centroids"], kc, vc, off, ln, ix,
                                                     status=st[i], bind=b)
            calls.append((dec(), app()) if bound else (dec, app))
        for d, a in calls:
            d()
            a()
        torch.cuda.synchronize()
        runs.append((out, st, ln, ix))
    for a, b, what in zip(runs[0], runs[1], ("outputs", "statuses", "lengths", "list entries")):
        assert torch.equal(a, b), f"bound and direct {what} differ"
