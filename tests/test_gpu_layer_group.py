"""GPU parity of a layer group sharing one selection ([HISPARSE-NOTES]
method 3: selection reuse makes cross-layer prefetch exact): one RESOLVE
for the group, the other layers' rows fetched on a second stream while the
first layers attend. Tables against the oracle, every layer's output
bitwise equal to direct attention on that layer's full KV, and the
overlapped schedule equal to the in-order one."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import cache
from top_sparse_attention_centroid_amd import workloads as W

from helpers import OUT_TOL, announce, f64, out_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _layers(cfg, n_layers):
    B, N, S, Hkv, Hq, d = cfg.batch, cfg.n_tokens, cfg.n_slots, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    out = []
    for j in range(n_layers):
        g = torch.Generator(device=DEV).manual_seed(1000 + j)
        kf = torch.randn((B, N, Hkv, d), generator=g, device=DEV).to(cfg.torch_dtype)
        vf = torch.randn((B, N, Hkv, d), generator=g, device=DEV).to(cfg.torch_dtype)
        hk = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
        hv = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
        hk.tensor.copy_(kf)
        hv.tensor.copy_(vf)
        q = torch.randn((cfg.steps, B, Hq, d), generator=g, device=DEV).to(cfg.torch_dtype)
        out.append({"kf": kf, "vf": vf, "hk": hk, "hv": hv, "q": q})
    return out


def _state(cfg, n_layers):
    B, N, S, Hkv, Hq, d = cfg.batch, cfg.n_tokens, cfg.n_slots, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    pt = torch.empty((B, N), dtype=torch.int32, device=DEV)
    st = torch.empty((B, S), dtype=torch.int32, device=DEV)
    lu = torch.empty((B, S), dtype=torch.int32, device=DEV)
    tsa.cache_reset(pt, st, lu)
    pools = [(torch.zeros((B, S, Hkv, d), dtype=cfg.torch_dtype, device=DEV),
              torch.zeros((B, S, Hkv, d), dtype=cfg.torch_dtype, device=DEV)) for _ in range(n_layers)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=DEV) for _ in range(n_layers)]
    return pt, st, lu, pools, outs


@pytest.mark.parametrize("policy", ["lru", "fifo"])
def test_layer_group_prefetch(policy):
    n_layers, steps = 3, 6
    cfg = W.config(4, batch=3, n_tokens=4000, n_slots=400, top_k=256, overlap=170, steps=steps,
                   n_kv_heads=2, n_q_heads=8)
    announce(f"layer group x{n_layers}, prefetch on a second stream, {policy}")
    B, N, S = cfg.batch, cfg.n_tokens, cfg.n_slots
    trace = W.selection_trace(cfg).to(DEV)
    tr_np = trace.cpu().numpy()
    lay = _layers(cfg, n_layers)
    over = _state(cfg, n_layers)
    inorder = _state(cfg, n_layers)
    fetch_stream = torch.cuda.Stream()
    events = [torch.cuda.Event(), torch.cuda.Event()]
    ref = {b: cache.CacheState(N, S) for b in range(B)}
    hosts = [[(f64(L["kf"][b]), f64(L["vf"][b])) for L in lay] for b in range(B)]
    Hkv, d = cfg.n_kv_heads, cfg.head_dim
    ref_pools = [[(np.zeros((S, Hkv, d)), np.zeros((S, Hkv, d))) for _ in lay] for b in range(B)]
    for t in range(steps):
        results = []
        for (pt, st, lu, pools, outs), fs in ((over, fetch_stream), (inorder, None)):
            io = [{"host_k": L["hk"].tensor, "host_v": L["hv"].tensor, "pool_k": pools[j][0], "pool_v": pools[j][1],
                   "q": L["q"][t], "out": outs[j]} for j, L in enumerate(lay)]
            slots, hits, misses = tsa.hier_group_step(io, pt, st, lu, trace[t], t, policy=policy,
                                                      fetch_stream=fs, events=events if fs else None)
            results.append((slots.clone(), hits.clone(), misses.clone(), [o.clone() for o in outs]))
        torch.cuda.synchronize()
        (s_o, h_o, m_o, out_o), (s_i, h_i, m_i, out_i) = results
        assert torch.equal(s_o, s_i) and torch.equal(h_o, h_i) and torch.equal(m_o, m_i)
        for j, L in enumerate(lay):
            direct = tsa.attend_rows(L["q"][t], L["kf"], L["vf"], trace[t])
            torch.cuda.synchronize()
            assert torch.equal(out_o[j], direct), f"step {t}, layer {j}: prefetched cache differs from direct"
            assert torch.equal(out_i[j], direct)
        sg, pt_g = s_o.cpu().numpy(), over[0].cpu().numpy()
        for b in range(B):
            # the oracle's group step: one shared set of tables, every layer's
            # own rows fetched into its own pool; then attention per layer
            r_slots, r_h, r_m, _ = cache.group_step(ref[b], tr_np[t, b], t, hosts[b], ref_pools[b], policy)
            assert np.array_equal(sg[b], r_slots), f"slots differ (step {t}, request {b})"
            assert (int(h_o[b]), int(m_o[b])) == (r_h, r_m)
            assert np.array_equal(pt_g[b], ref[b].page_table)
            for j, L in enumerate(lay):
                o = cache.attend_slots(f64(L["q"][t, b]), ref_pools[b][j][0], ref_pools[b][j][1], r_slots)
                err = out_error(out_o[j][b].cpu().numpy(), o)
                assert err <= OUT_TOL, f"output error {err} (step {t}, layer {j}, request {b})"
    # every layer's pool holds its own rows of every resident token
    st_g = over[1].cpu()
    for j, L in enumerate(lay):
        pk = over[3][j][0].cpu()
        for b in range(B):
            res = torch.nonzero(st_g[b] >= 0).flatten()
            assert torch.equal(pk[b, res], L["kf"][b, st_g[b, res].long()].cpu())


def test_single_layer_group_is_resolve_then_attend():
    cfg = W.config(4, batch=2, n_tokens=3000, n_slots=300, top_k=128, overlap=100, steps=3,
                   n_kv_heads=2, n_q_heads=8)
    announce("layer group of one")
    trace = W.selection_trace(cfg).to(DEV)
    lay = _layers(cfg, 1)
    pt, st, lu, pools, outs = _state(cfg, 1)
    pt2, st2, lu2, pools2, _ = _state(cfg, 1)
    for t in range(3):
        io = [{"host_k": lay[0]["hk"].tensor, "host_v": lay[0]["hv"].tensor, "pool_k": pools[0][0],
               "pool_v": pools[0][1], "q": lay[0]["q"][t], "out": outs[0]}]
        slots, _, _ = tsa.hier_group_step(io, pt, st, lu, trace[t], t)
        s2, _, _ = tsa.resolve(pt2, st2, lu2, trace[t], t, lay[0]["hk"].tensor, lay[0]["hv"].tensor, pools2[0][0],
                               pools2[0][1])
        o2 = tsa.attend_rows(lay[0]["q"][t], pools2[0][0], pools2[0][1], s2)
        torch.cuda.synchronize()
        assert torch.equal(slots, s2) and torch.equal(outs[0], o2)
