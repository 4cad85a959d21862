"""GPU parity of the fused RESOLVE step (hit detection, batch-step LRU, table
update, zero-copy host fetch) and of attention over the hot slots, against
the oracle's exact LRU and fp64 attention."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import cache
from top_sparse_attention_centroid_amd import workloads as W

from helpers import OUT_TOL, announce, f64, out_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(cfg):
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
    torch.cuda.synchronize()
    return prob, hk, hv, pt, st, lu, pool_k, pool_v, trace


def _f32(t: torch.Tensor) -> np.ndarray:
    """Host copy widened to fp32 (exact for bf16 and fp32 storage); the oracle
    widens it to fp64 itself."""
    return t.detach().to("cpu", torch.float32).numpy()


def _run(cfg, steps, attn_requests, state_requests=None):
    """Runs `steps` RESOLVE + attention steps and checks them against the
    oracle. Returns (misses [steps][B], evictions [steps][B]): evictions are
    the oracle's fetches that landed on a slot holding another token."""
    B = cfg.batch
    state_requests = range(B) if state_requests is None else state_requests
    prob, hk, hv, pt, st, lu, pool_k, pool_v, trace = _setup(cfg)
    ref = {b: cache.CacheState(cfg.n_tokens, cfg.n_slots) for b in state_requests}
    K32 = {b: _f32(prob["keys"][b]) for b in attn_requests}
    V32 = {b: _f32(prob["values"][b]) for b in attn_requests}
    miss_log, evict_log = [], []
    for t in range(steps):
        slots, hits, misses = tsa.resolve(pt, st, lu, trace[t], t, hk.tensor, hv.tensor, pool_k, pool_v)
        out_c = tsa.attend_rows(prob["q"][t], pool_k, pool_v, slots)
        out_d = tsa.attend_rows(prob["q"][t], prob["keys"], prob["values"], trace[t])
        torch.cuda.synchronize()
        # exactness: attention through the hot cache equals attention on the full KV, bitwise
        assert torch.equal(out_c, out_d)
        slots_g, hits_g, miss_g = slots.cpu().numpy(), hits.cpu().numpy(), misses.cpu().numpy()
        pt_g, st_g, lu_g = pt.cpu().numpy(), st.cpu().numpy(), lu.cpu().numpy()
        miss_log.append(miss_g.copy())
        evicted = np.zeros(B, dtype=np.int64)
        q64 = f64(prob["q"][t])
        tr = trace[t].cpu().numpy()
        for b in state_requests:
            before = ref[b].slot_token.copy()
            r_slots, r_h, r_m, fetches = cache.lru_step(ref[b], tr[b], t)
            evicted[b] = sum(1 for _, v in fetches if before[v] >= 0)
            assert np.array_equal(slots_g[b], r_slots), f"slots differ (step {t}, request {b})"
            assert (hits_g[b], miss_g[b]) == (r_h, r_m)
            assert np.array_equal(pt_g[b], ref[b].page_table), f"page table differs (step {t}, request {b})"
            assert np.array_equal(st_g[b], ref[b].slot_token), f"slot owners differ (step {t}, request {b})"
            assert np.array_equal(lu_g[b], ref[b].last_use), f"last use differs (step {t}, request {b})"
            if b in attn_requests:
                pk = pool_k[b].cpu()
                assert torch.equal(pk[torch.from_numpy(r_slots).long()], prob["keys"][b, torch.from_numpy(tr[b]).long()].cpu())
                o = cache.attend_slots(q64[b], K32[b], V32[b], tr[b])
                err = out_error(out_c[b].cpu().numpy(), o)
                assert err <= OUT_TOL, f"output error {err} (step {t}, request {b})"
        evict_log.append(evicted)
    return np.array(miss_log), np.array(evict_log)


def test_resolve_small_pool_equals_selection():
    # S == k: after step t the resident set is exactly S_t, so misses = k - overlap
    cfg = W.config(4, batch=3, n_tokens=5000, n_slots=256, top_k=256, overlap=200, steps=6,
                   n_kv_heads=2, n_q_heads=8)
    announce("resolve S == k")
    m, ev = _run(cfg, 6, range(3))
    assert np.all(m[0] == 256) and np.all(m[1:] == 56)
    assert np.all(ev[1:] == 56)   # every miss after the first step replaces a resident token


def test_resolve_eviction_and_fetch():
    # 2600 slots for k = 2048: step 0 leaves 552 free, step 1's ~307 misses
    # leave ~245, so from step 2 on every step evicts residents whose
    # last-use stamps differ (dropped at different steps)
    cfg = W.config(4, batch=4, n_tokens=16_384, n_slots=2600, top_k=2048, steps=10)
    announce("resolve B=4 N=16384 S=2600 k=2048, evicting")
    _, ev = _run(cfg, 10, [0, 3])
    assert np.all(ev[:2] == 0)
    assert np.all(ev[2:] > 0), f"steps without evictions: {ev}"


def test_resolve_fp32_ragged():
    cfg = W.config(4, batch=2, n_tokens=3001, n_slots=1000, top_k=333, overlap=250, steps=14,
                   n_kv_heads=1, n_q_heads=4, dtype="f32")
    announce("resolve fp32 ragged")
    _, ev = _run(cfg, 14, range(2))
    assert np.all(ev[12:] > 0)


def test_reset_flushes_the_cache():
    cfg = W.config(4, batch=2, n_tokens=4000, n_slots=512, top_k=128, overlap=100, steps=3,
                   n_kv_heads=2, n_q_heads=8)
    announce("resolve reset")
    prob, hk, hv, pt, st, lu, pool_k, pool_v, trace = _setup(cfg)
    for t in range(2):
        tsa.resolve(pt, st, lu, trace[t], t, hk.tensor, hv.tensor, pool_k, pool_v)
    tsa.cache_reset(pt, st, lu)
    _, hits, misses = tsa.resolve(pt, st, lu, trace[2], 2, hk.tensor, hv.tensor, pool_k, pool_v)
    torch.cuda.synchronize()
    assert hits.tolist() == [0, 0] and misses.tolist() == [128, 128]


def test_hier_cache_workload_full_size():
    """32 requests x 131,072 tokens, 4096 slots, top-2048 with 1741 carried
    over: every request's tables are checked exactly for 14 steps (the pool
    fills at step 7, after 2048 + 6 x ~302 fetches, and evicts from then on);
    attention of three requests."""
    cfg = W.config(4)
    announce(f"resolve {cfg.name} full size, 14 steps")
    m, ev = _run(cfg, 14, [0, 17, 31])
    assert np.all(m[0] == 2048) and np.all(m[1] == 307)
    assert np.all(ev[:6] == 0)
    assert np.all(ev[8:] > 0), f"requests without evictions after the pool filled: {ev[8:]}"
