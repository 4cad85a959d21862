"""GPU parity of the token-indexer path (indexer scan, exact top-k over all
tokens, attention over the selection) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import token
from top_sparse_attention_centroid_amd import workloads as W

from helpers import GAP_MIN, OUT_TOL, announce, condition_token_keys, f64, out_error

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(cfg, steps, check_requests, attn_requests):
    """Decodes `steps` steps of the whole batch, then checks the selections of
    `check_requests` and the outputs of `attn_requests` against the oracle.
    The K/V of one request at a time is copied to the host (fp32, exact for
    bf16), so every request of the full-size workload can be checked."""
    prob = W.token_problem(cfg, device=DEV)
    q_idx, q = W.token_queries(cfg, prob, steps=steps)
    k_idx = condition_token_keys(q_idx, prob["k_idx"], cfg.top_k, steps, requests=check_requests)
    torch.cuda.synchronize()
    B, k = cfg.batch, cfg.top_k
    sel = torch.empty((B, k), dtype=torch.int32, device=DEV)
    sels, outs = [], []
    for t in range(steps):
        out = tsa.token_decode(q_idx[t], k_idx, q[t], prob["keys"], prob["values"], k, sel_out=sel)
        torch.cuda.synchronize()
        sels.append(sel.cpu().numpy().copy())
        outs.append(out.cpu().numpy())
    qi64, q64 = f64(q_idx), f64(q)
    for b in check_requests:
        kidx64 = f64(k_idx[b])
        K32 = V32 = None
        if b in attn_requests:
            K32 = prob["keys"][b].to("cpu", torch.float32).numpy()[None]
            V32 = prob["values"][b].to("cpu", torch.float32).numpy()[None]
        for t in range(steps):
            ref_sel, gap = token.token_topk(qi64[t, b], kidx64, k)
            assert gap >= GAP_MIN
            assert np.array_equal(sels[t][b], ref_sel), f"selection differs (step {t}, request {b})"
            assert set(prob["planted"][b].tolist()) <= set(sels[t][b].tolist())
            if K32 is not None:
                r = token.token_decode(qi64[t, b:b + 1], kidx64[None], q64[t, b:b + 1], K32, V32, k)
                err = out_error(outs[t][b], r["out"][0])
                assert err <= OUT_TOL, f"output error {err} (step {t}, request {b})"
        del K32, V32


def test_token_topk_small():
    cfg = W.config(3, batch=3, n_tokens=20_001, top_k=1000, n_planted=64, steps=2)
    announce("token small N=20001 k=1000")
    _run(cfg, 2, range(3), range(3))


def test_token_topk_single_chunk_and_k_equals_n():
    # one chunk shorter than k, and a selection of every token (dense attention)
    cfg = W.config(3, batch=2, n_tokens=1500, top_k=1500, n_planted=8, steps=1)
    announce("token k == N")
    _run(cfg, 1, range(2), range(2))


def test_token_topk_ragged_tiles():
    # ragged last score tile (2048 tokens) and filter tile (4096 keys)
    cfg = W.config(3, batch=2, n_tokens=5 * 4096 + 100, top_k=1000, n_planted=32, steps=2)
    announce("token ragged tiles")
    _run(cfg, 2, range(2), [1])


def _run_exact(cfg, q_idx, k_idx, attn=True):
    """Integer-lattice indexer inputs: every score is an exact small integer in
    fp32 and fp64 alike, so ties are real and the lower token id must win."""
    prob = W.token_problem(cfg, device=DEV)
    _, q = W.token_queries(cfg, prob, steps=1)
    B, k = cfg.batch, cfg.top_k
    sel = torch.empty((B, k), dtype=torch.int32, device=DEV)
    out = tsa.token_decode(q_idx, k_idx, q[0], prob["keys"], prob["values"], k, sel_out=sel)
    torch.cuda.synchronize()
    sel_g, out_g = sel.cpu().numpy(), out.cpu().numpy()
    qi64, ki64 = f64(q_idx), f64(k_idx)
    for b in range(B):
        ref_sel, _ = token.token_topk(qi64[b], ki64[b], k)
        assert np.array_equal(sel_g[b], ref_sel), f"selection differs (request {b})"
        if attn:
            r = token.token_decode(qi64[b:b + 1], ki64[b][None], f64(q[0][b:b + 1]), f64(prob["keys"][b])[None],
                                   f64(prob["values"][b])[None], k)
            err = out_error(out_g[b], r["out"][0])
            assert err <= OUT_TOL, f"output error {err} (request {b})"


def test_token_topk_integer_ties():
    cfg = W.config(3, batch=2, n_tokens=9000, top_k=1500, n_planted=8, steps=1)
    announce("token integer ties")
    g = torch.Generator().manual_seed(11)
    q_idx = torch.randint(-2, 3, (2, 64), generator=g).to(torch.bfloat16).to(DEV)
    k_idx = torch.randint(-1, 2, (2, 9000, 64), generator=g).to(torch.bfloat16).to(DEV)
    _run_exact(cfg, q_idx, k_idx)


# The scan's workgroups cover the first N - N // 10 tokens in fixed shares and
# take the rest in 512-token chunks: no shared tail (N < 10), one short
# chunk, several chunks with a ragged last one, and one request alone (every
# workgroup on its chunks, 64 of them sharing the tail).
@pytest.mark.parametrize("batch,n,k", [(3, 7, 3), (3, 3000, 200), (2, 15_377, 700), (1, 120_001, 900)])
def test_token_topk_shared_tail(batch, n, k):
    cfg = W.config(3, batch=batch, n_tokens=n, top_k=k, n_planted=min(8, k), steps=1)
    announce(f"token shared scan tail B={batch} N={n} k={k}")
    g = torch.Generator().manual_seed(n)
    q_idx = torch.randint(-2, 3, (batch, 64), generator=g).to(torch.bfloat16).to(DEV)
    k_idx = torch.randint(-1, 2, (batch, n, 64), generator=g).to(torch.bfloat16).to(DEV)
    _run_exact(cfg, q_idx, k_idx, attn=n <= 3000)


def test_token_topk_all_scores_equal():
    # q_idx = 0: every score is 0, so the selection is the k lowest token ids
    cfg = W.config(3, batch=2, n_tokens=10_000, top_k=777, n_planted=8, steps=1)
    announce("token all-equal scores")
    q_idx = torch.zeros((2, 64), dtype=torch.bfloat16, device=DEV)
    k_idx = torch.randn((2, 10_000, 64), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(DEV)
    _run_exact(cfg, q_idx, k_idx, attn=False)


def test_token_topk_ragged_gqa():
    cfg = W.config(3, batch=2, n_tokens=8193 * 2 + 7, top_k=333, n_planted=16, steps=2,
                   n_kv_heads=2, n_q_heads=16)
    announce("token ragged G=8")
    _run(cfg, 2, range(2), range(2))


def test_token_workload_full_size():
    """16 requests x 200,000 tokens, top-2048: selections and attention
    outputs of every request are checked, for two steps."""
    cfg = W.config(3)
    announce(f"token {cfg.name} full size")
    _run(cfg, 2, range(cfg.batch), range(cfg.batch))


# a small and a large batch (3 and 16 requests x 8 KV heads)
@pytest.mark.parametrize("batch", [3, 16])
def test_token_workspace_contents_never_reach_the_output(batch):
    # The row-list attention merges partial states like the inverted-index
    # path: a workspace holding NaN bit patterns, then zeros, before the call
    # gives bitwise equal, finite outputs and the same selection.
    cfg = W.config(3, batch=batch, n_tokens=20_001, top_k=1000, n_planted=64, steps=1)
    announce(f"token workspace contents, {batch} requests")
    prob = W.token_problem(cfg, device=DEV)
    q_idx, q = W.token_queries(cfg, prob, steps=1)
    B, k = cfg.batch, cfg.top_k
    desc = tsa.binding.token_desc(prob["k_idx"], prob["keys"], cfg.n_q_heads)
    nbytes = tsa.workspace_bytes(tsa.binding.OP_TOKEN_DECODE, desc, k)
    outs, sels = [], []
    for fill in (0xFF, 0x00):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        sel = torch.empty((B, k), dtype=torch.int32, device=DEV)
        outs.append(tsa.token_decode(q_idx[0], prob["k_idx"], q[0], prob["keys"], prob["values"], k, sel_out=sel,
                                     ws=ws))
        sels.append(sel)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(o).all()) for o in outs)
    assert torch.equal(outs[0], outs[1]) and torch.equal(sels[0], sels[1])


def test_token_consecutive_calls_on_one_workspace():
    """Twelve decodes in a row on one workspace, each selection against the
    oracle. Every call clears the histogram and the chunk counters that the
    previous call left and marks them cleared with a tag of its own; the
    scan's other workgroups wait for that tag. A tag equal to the previous
    call's would let them add their counts before the clear (a tag built from
    epoch ^ nonce did so for about a third of consecutive calls, since both
    advance by one a call)."""
    cfg = W.config(3, batch=4, n_tokens=30_011, top_k=700, n_planted=16, steps=12)
    announce("token: 12 consecutive calls on one workspace")
    prob = W.token_problem(cfg, device=DEV)
    q_idx, q = W.token_queries(cfg, prob, steps=12)
    k_idx = condition_token_keys(q_idx, prob["k_idx"], cfg.top_k, 12, requests=range(cfg.batch))
    B, k = cfg.batch, cfg.top_k
    desc = tsa.binding.token_desc(k_idx, prob["keys"], cfg.n_q_heads)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_TOKEN_DECODE, desc, k), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, cfg.n_q_heads, cfg.head_dim), dtype=torch.float32, device=DEV)
    sels = torch.empty((12, B, k), dtype=torch.int32, device=DEV)
    for t in range(12):  # back to back on one stream, no host sync between calls
        tsa.token_decode(q_idx[t], k_idx, q[t], prob["keys"], prob["values"], k, out=out, sel_out=sels[t], ws=ws)
    torch.cuda.synchronize()
    got = sels.cpu().numpy()
    qi64 = f64(q_idx)
    for b in range(B):
        kidx64 = f64(k_idx[b])
        for t in range(12):
            ref_sel, gap = token.token_topk(qi64[t, b], kidx64, k)
            assert gap >= GAP_MIN
            assert np.array_equal(got[t][b], ref_sel), f"selection differs (call {t}, request {b})"
