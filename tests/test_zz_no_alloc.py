"""The allocation-free decode entry point (static device scratch) against the
ordinary entry point with a caller workspace: bitwise equal outputs,
selections and row counts on two calls in a row, the second with a smaller
batch, and a decode too large for the scratch rejected before any launch."""

import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from top_sparse_attention_centroid_amd import workloads as W

from helpers import announce, conditioned_ivf_queries

DEV = "cuda"


def _case(cfg):
    p = W.ivf_problem(cfg, device=DEV)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    return p, offsets, ids, q


def _compare(cfg, p, offsets, ids, q):
    B, Hq, Hkv, k, d = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k, cfg.head_dim
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        sel = torch.full((B, Hq, k), -7, dtype=torch.int32, device=DEV)
        rows = torch.full((B, Hq), -7, dtype=torch.int32, device=DEV)
        uniq = torch.full((B, Hkv), -7, dtype=torch.int32, device=DEV)
        if noalloc:
            tsa.sparse_decode_noalloc(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, out=out,
                                      sel_out=sel, rows_out=rows, uniq_out=uniq)
        else:
            tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, out=out, sel_out=sel,
                              rows_out=rows, uniq_out=uniq)
        outs.append((out, sel, rows, uniq))
    torch.cuda.synchronize()
    (o0, s0, r0, u0), (o1, s1, r1, u1) = outs
    assert bool(torch.isfinite(o1).all())
    assert torch.equal(s0, s1) and torch.equal(r0, r1) and torch.equal(u0, u1)
    assert torch.equal(o0, o1), f"max difference {float((o0 - o1).abs().max())}"


@pytest.mark.gpu
def test_noalloc_decode_equals_workspace_decode_twice_then_smaller():
    # a 16 x 32K batch (60.9 MiB of workspace, near the 64 MiB limit), then
    # 3 x 20K on the same scratch: the second call must not see the first
    big = W.config(2, batch=16, steps=1)
    small = W.config(2, batch=3, n_tokens=20_000, n_centroids=200, top_k=12, steps=1)
    for cfg in (big, small):
        announce(f"no-alloc decode {cfg.batch} x {cfg.n_tokens}, C={cfg.n_centroids}, k={cfg.top_k}")
        p, offsets, ids, q = _case(cfg)
        _compare(cfg, p, offsets, ids, q)
        del p, offsets, ids, q
        torch.cuda.empty_cache()


@pytest.mark.gpu
def test_noalloc_decode_rejects_a_workspace_beyond_the_scratch():
    cfg = W.config(2, batch=20, n_tokens=32_768, steps=1)   # needs ~76 MiB
    announce("no-alloc decode beyond the scratch")
    p = W.ivf_problem(cfg, device=DEV)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    q = W.ivf_queries(cfg, p["centroids"], steps=1)[0]
    out = torch.full((cfg.batch, cfg.n_q_heads, cfg.head_dim), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(tsa.binding.TsaError, match="TSA_ERR_WORKSPACE"):
        tsa.sparse_decode_noalloc(q, p["centroids"], offsets, ids, p["keys"], p["values"], cfg.top_k, out=out)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())   # nothing was enqueued


@pytest.mark.parametrize("batch,expect", [(20, "WORKSPACE"), (16, None)])
def test_noalloc_scratch_limit_is_checked_on_the_host(batch, expect):
    # Runs without a GPU: sizes beyond the static scratch are rejected before
    # the scratch address is looked up or anything is enqueued; a null q is
    # rejected first in every case.
    import ctypes
    from top_sparse_attention_centroid_amd import binding as B
    lib = B.load()
    d = B.IvfDesc(batch, 32768, 8, 32, 128, 256, 1, B.TSA_BF16)
    fake = ctypes.c_void_p(0x10000)
    st = lib.tsa_sparse_decode_noalloc(ctypes.byref(d), None, fake, fake, fake, fake, fake, 16, fake, None, None,
                                       None, None)
    assert st == B.TSA_ERR_INVALID_ARG
    st = lib.tsa_sparse_decode_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 300, fake,
                                       None, None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG        # k > C
    if expect:
        st = lib.tsa_sparse_decode_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, 16, fake, None,
                                           None, None, None)
        assert st == B.TSA_ERR_WORKSPACE and b"static scratch" in lib.tsa_last_error()
