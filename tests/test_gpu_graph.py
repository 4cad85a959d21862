"""The decode steps captured into HIP graphs: every entry point issues only
kernel launches (and, when asked, event records) on the caller's stream, so a
step can be captured once and replayed. Each replay is checked bitwise
against the same step launched eagerly, with eager work and host
synchronisations between replays."""

import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from top_sparse_attention_centroid_amd import workloads as W

from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"
REPLAYS = 4


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# 6 requests: a wave per plan segment; 16 x 8 KV heads: merged gather sets
@pytest.mark.parametrize("batch,n_tokens", [(6, 9000), (16, 4096)])
def test_graph_sparse_decode_replays(batch, n_tokens):
    cfg = W.config(2, batch=batch, n_tokens=n_tokens, n_centroids=96, top_k=7, steps=3)
    announce(f"graph sparse_decode, {batch} requests")
    p = W.ivf_problem(cfg, device=DEV)
    q = W.ivf_queries(cfg, p["centroids"], steps=3)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    B, Hq, k = cfg.batch, cfg.n_q_heads, cfg.top_k
    out = torch.empty((B, Hq, cfg.head_dim), dtype=torch.float32, device=DEV)
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    uniq = torch.empty((B, cfg.n_kv_heads), dtype=torch.int32, device=DEV)
    desc = tsa.binding.ivf_desc(p["keys"], p["centroids"], Hq)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE, desc, k), dtype=torch.uint8, device=DEV)
    qin = q[0].clone()

    def step():
        tsa.sparse_decode(qin, p["centroids"], offsets, ids, p["keys"], p["values"], k, out=out,
                          sel_out=sel, uniq_out=uniq, ws=ws)

    eager = []
    for t in range(3):
        qin.copy_(q[t])
        step()
        eager.append((out.clone(), sel.clone(), uniq.clone()))
    g = _capture(step)
    for r in range(REPLAYS):
        t = r % 3
        qin.copy_(q[t])
        out.fill_(float("nan"))
        sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[t][0]), f"replay {r}: output differs"
        assert torch.equal(sel, eager[t][1]), f"replay {r}: selection differs"
        assert torch.equal(uniq, eager[t][2])
        # eager work on the same buffers between replays
        tsa.sparse_decode(q[(t + 1) % 3], p["centroids"], offsets, ids, p["keys"], p["values"], k, out=out, ws=ws)
        torch.cuda.synchronize()


def test_graph_token_decode_replays():
    cfg = W.config(3, batch=3, n_tokens=30_001, top_k=700, n_planted=32, steps=2)
    announce("graph token_decode")
    prob = W.token_problem(cfg, device=DEV)
    q_idx, q = W.token_queries(cfg, prob, steps=2)
    B, k = cfg.batch, cfg.top_k
    out = torch.empty((B, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=DEV)
    sel = torch.empty((B, k), dtype=torch.int32, device=DEV)
    desc = tsa.binding.token_desc(prob["k_idx"], prob["keys"], cfg.n_q_heads)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_TOKEN_DECODE, desc, k), dtype=torch.uint8, device=DEV)
    qi, qa = q_idx[0].clone(), q[0].clone()

    def step():
        tsa.token_decode(qi, prob["k_idx"], qa, prob["keys"], prob["values"], k, out=out, sel_out=sel, ws=ws)

    eager = []
    for t in range(2):
        qi.copy_(q_idx[t])
        qa.copy_(q[t])
        step()
        eager.append((out.clone(), sel.clone()))
    g = _capture(step)
    for r in range(REPLAYS):
        t = r % 2
        qi.copy_(q_idx[t])
        qa.copy_(q[t])
        out.fill_(float("nan"))
        sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[t][0]), f"replay {r}: output differs"
        assert torch.equal(sel, eager[t][1]), f"replay {r}: selection differs"
        tsa.token_decode(q_idx[1 - t], prob["k_idx"], q[1 - t], prob["keys"], prob["values"], k, out=out, ws=ws)
        torch.cuda.synchronize()


def _cache_state(cfg, prob):
    B, N, S, Hkv, d = cfg.batch, cfg.n_tokens, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim
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
    return hk, hv, pt, st, lu, pool_k, pool_v


def test_graph_resolve_attend_replays():
    """One graph per decode step (each step has its own selection and stamp);
    replaying them in order walks the cache through the same states as eager
    calls on a twin cache."""
    steps = 5
    cfg = W.config(4, batch=3, n_tokens=6000, n_slots=512, top_k=256, overlap=180, steps=steps,
                   n_kv_heads=2, n_q_heads=8)
    announce("graph resolve + attend_rows")
    prob = W.cache_problem(cfg, device=DEV)
    trace = prob["trace"].to(DEV)
    B, k = cfg.batch, cfg.top_k
    eg = _cache_state(cfg, prob)
    gr = _cache_state(cfg, prob)
    slots = torch.empty((B, k), dtype=torch.int32, device=DEV)
    hits = torch.empty((B,), dtype=torch.int32, device=DEV)
    misses = torch.empty((B,), dtype=torch.int32, device=DEV)
    out = torch.empty((B, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=DEV)
    desc = tsa.binding.attn_desc(gr[5], cfg.n_q_heads, k)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_ATTEND_ROWS, desc), dtype=torch.uint8, device=DEV)

    def make(t):
        hk, hv, pt, st, lu, pk, pv = gr

        def step():
            tsa.resolve(pt, st, lu, trace[t], t, hk.tensor, hv.tensor, pk, pv, slots_out=slots, hits=hits,
                        misses=misses)
            tsa.attend_rows(prob["q"][t], pk, pv, slots, out=out, ws=ws)
        return step

    graphs = [_capture(make(t)) for t in range(steps)]
    hk, hv, pt, st, lu, pk, pv = eg
    for t in range(steps):
        e_slots, e_hits, e_miss = tsa.resolve(pt, st, lu, trace[t], t, hk.tensor, hv.tensor, pk, pv)
        e_out = tsa.attend_rows(prob["q"][t], pk, pv, e_slots)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        graphs[t].replay()
        torch.cuda.synchronize()
        assert torch.equal(slots, e_slots), f"step {t}: slots differ"
        assert torch.equal(hits, e_hits) and torch.equal(misses, e_miss)
        assert torch.equal(out, e_out), f"step {t}: output differs"
        for a, b in zip(gr[2:], eg[2:]):
            assert torch.equal(a, b), f"step {t}: cache state differs"
