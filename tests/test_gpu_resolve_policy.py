"""GPU parity of RESOLVE under FIFO, random and offline-Belady replacement
([HISPARSE-NEWS] compares them with LRU by miss rate) against the policy
oracle: slots, hit/miss counts and all three tables exact at every step, and
attention through the cache equal to attention on the full KV."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import cache
from top_sparse_attention_centroid_amd import workloads as W

from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _next_use_dense(trace_np, N):
    """[T][B][N] int32: the next step after t that selects each token (INT32_MAX if none)."""
    T, B, _ = trace_np.shape
    out = np.full((T, B, N), cache.NEVER, dtype=np.int32)
    nxt = np.full((B, N), cache.NEVER, dtype=np.int64)
    for t in range(T - 1, -1, -1):
        out[t] = nxt
        for b in range(B):
            nxt[b, trace_np[t, b]] = t
    return out


@pytest.mark.parametrize("locality", [False, True])
@pytest.mark.parametrize("policy", ["fifo", "random", "belady"])
def test_policy_matches_oracle(policy, locality):
    """Uniform trace, and a trace with popularity and recency (returning
    tokens, where the policies evict differently)."""
    steps = 10
    cfg = W.config(4, batch=3, n_tokens=4000, n_slots=400, top_k=256, overlap=170, steps=steps,
                   n_kv_heads=2, n_q_heads=8)
    if locality:
        cfg = cfg.replace(popularity_sd=2.0, recency=0.3)
    announce(f"resolve policy {policy} locality={locality}")
    B, N, S, Hkv, d = cfg.batch, cfg.n_tokens, cfg.n_slots, cfg.n_kv_heads, cfg.head_dim
    prob = W.cache_problem(cfg, device=DEV)
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
    trace = prob["trace"].to(DEV)
    tr_np = prob["trace"].cpu().numpy()
    seed = 0x1234_5678_9ABC
    gpu_policy = "priority" if policy == "belady" else policy
    nu = _next_use_dense(tr_np, N) if policy == "belady" else None
    nu_dev = torch.from_numpy(nu).to(DEV) if nu is not None else None
    ref = {b: cache.CacheState(N, S) for b in range(B)}
    total_misses = 0
    for t in range(steps):
        slots, hits, misses = tsa.resolve(pt, st, lu, trace[t], t, hk.tensor, hv.tensor, pool_k, pool_v,
                                          policy=gpu_policy, seed=seed,
                                          priority=None if nu_dev is None else nu_dev[t])
        out_c = tsa.attend_rows(prob["q"][t], pool_k, pool_v, slots)
        out_d = tsa.attend_rows(prob["q"][t], prob["keys"], prob["values"], trace[t])
        torch.cuda.synchronize()
        assert torch.equal(out_c, out_d), f"cache-mediated attention differs at step {t}"
        sg, hg, mg = slots.cpu().numpy(), hits.cpu().numpy(), misses.cpu().numpy()
        ptg, stg, lug = pt.cpu().numpy(), st.cpu().numpy(), lu.cpu().numpy()
        for b in range(B):
            nub = None
            if nu is not None:
                nub = {int(x): int(nu[t, b, x]) for x in np.flatnonzero(nu[t, b] != cache.NEVER)}
            r_slots, r_h, r_m, _ = cache.policy_step(ref[b], tr_np[t, b], t, policy, seed=seed, request=b,
                                                     next_use=nub)
            assert np.array_equal(sg[b], r_slots), f"slots differ (step {t}, request {b})"
            assert (hg[b], mg[b]) == (r_h, r_m)
            assert np.array_equal(ptg[b], ref[b].page_table)
            assert np.array_equal(stg[b], ref[b].slot_token)
            assert np.array_equal(lug[b], ref[b].last_use)
        total_misses += int(mg.sum())
    assert total_misses > B * 256   # evictions happened after the first step
