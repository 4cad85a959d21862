"""GPU parity of the per-head inverted-index decodes against the fp64 oracle
and against the staged launches, through the C ABI: fused (one workgroup per
query head scores the codebook, selects the lists and attends their rows in
one launch) and split (a scoring launch, then workgroups per share of each
head's rows select the head's lists and attend their share; the head's last
share to finish merges the shares' states).

Bars as for the staged path: selected lists, per-head row counts and union
counts bit-exact; outputs within OUT_TOL of the oracle; per-head and staged
outputs within 1e-4 of each other (fp32 sums in another order)."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import ivf
from top_sparse_attention_centroid_amd import workloads as W

from helpers import OUT_TOL, announce, conditioned_ivf_queries, f64, out_error
from test_gpu_ivf import _check_index, _decode, _decode_and_check, _problem

pytestmark = pytest.mark.gpu
DEV = "cuda"
PATH_TOL = 1e-4


def _all(q, p, offsets, ids, k, schedules=("fused", "split", "staged"), **kw):
    """sel, rows, uniq and out of one step under each schedule."""
    B, Hq, _ = q.shape
    Hkv = ids.shape[1]
    res = {}
    for schedule in schedules:
        sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
        rows = torch.empty((B, Hq), dtype=torch.int32, device=DEV)
        uniq = torch.empty((B, Hkv), dtype=torch.int32, device=DEV)
        out = _decode(schedule, q, p, offsets, ids, k, sel_out=sel, rows_out=rows, uniq_out=uniq, **kw)
        res[schedule] = (sel, rows, uniq, out)
    torch.cuda.synchronize()
    return res


def _agree(res):
    s = res["staged"]
    for name, f in res.items():
        for a, b, what in zip(f[:3], s[:3], ("selection", "row counts", "union counts")):
            assert torch.equal(a, b), f"{name} and staged {what} differ"
        assert out_error(f[3].cpu().numpy(), s[3].cpu().numpy()) <= PATH_TOL, name


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_lists_take_many_rounds(dtype):
    """~3,750-row lists, top-4: ~15,000 rows per head, about 15 rounds of 64
    rows for each of the workgroup's 16 waves."""
    cfg = W.config(1, batch=1, n_tokens=60_000, n_kv_heads=2, n_q_heads=8, n_centroids=16, top_k=4,
                   dtype=dtype, steps=1, shared_codebook=False, seed=61)
    announce(f"fused long lists dtype={dtype}")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, [0], offsets, ids)
    q = _decode_and_check(cfg, p, ref, [0], steps=1, schedule="fused")
    if dtype == "bf16":
        _decode_and_check(cfg, p, ref, [0], steps=1, q=q, schedule="split")
    _agree(_all(q[0], p, offsets, ids, cfg.top_k,
                schedules=("fused", "split", "staged") if dtype == "bf16" else ("fused", "staged")))


def test_widest_group_largest_codebook_and_k():
    """8 query heads per KV head, C = 1024 lists and k = 64 (the fused
    decode's limits: the group's scores fill its LDS, the head's lists one per
    lane)."""
    cfg = W.config(1, batch=1, n_tokens=40_000, n_kv_heads=2, n_q_heads=16, n_centroids=1024, top_k=64,
                   steps=1, shared_codebook=False, seed=62)
    announce("fused G=8 C=1024 k=64")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, [0], offsets, ids)
    q = _decode_and_check(cfg, p, ref, [0], steps=1, schedule="fused")
    _decode_and_check(cfg, p, ref, [0], steps=1, q=q, schedule="split")
    _agree(_all(q[0], p, offsets, ids, cfg.top_k))


@pytest.mark.parametrize("schedule", ["fused", "split"])
def test_per_head_schedules_on_a_larger_batch(schedule):
    """16 requests x 32 query heads (512 heads, 128 groups: beyond both
    automatic choices) under the per-head schedules: the same lists, counts
    and (to rounding) outputs as the staged launches; two requests in full
    against the oracle."""
    cfg = W.config(2, batch=16, n_tokens=4096, n_centroids=256, top_k=16, steps=1, seed=63)
    announce(f"{schedule} 16 x 32 heads")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, [0, 15], offsets, ids)
    q = _decode_and_check(cfg, p, ref, [0, 15], steps=1, sel_requests=range(cfg.batch), schedule=schedule)
    _agree(_all(q[0], p, offsets, ids, cfg.top_k, schedules=(schedule, "staged")))


def test_growing_index_per_head_and_staged_agree():
    """A growing index (lists with free entries, lengths in lens) decoded by
    the fused, split and staged launches; one request against the oracle
    over the indexed prefix."""
    cfg = W.config(1, batch=2, n_tokens=12_000, n_kv_heads=2, n_q_heads=8, n_centroids=100, top_k=10, steps=1,
                   shared_codebook=False, seed=64)
    announce("per-head decodes, growing index")
    p = _problem(cfg)
    prefix = 9000
    offsets, lens, ids = tsa.index_build_dyn(p["keys"], p["centroids"], prefix)
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    res = _all(q, p, offsets, ids, cfg.top_k, lens=lens)
    _agree(res)
    # the oracle on the prefix: its own index of the first `prefix` keys
    keys = p["keys"][0:1, :prefix]
    vals = p["values"][0:1, :prefix]
    off_o, ids_o, margin = ivf.index_build(f64(keys), f64(p["centroids"][0:1]))
    assert margin.min() >= 1e-3
    r = ivf.sparse_decode(f64(q[0:1]), f64(p["centroids"][0:1]), off_o, ids_o, f64(keys), f64(vals), cfg.top_k)
    for schedule in ("fused", "split"):
        sel, rows, _, out = res[schedule]
        assert np.array_equal(sel[0].cpu().numpy(), r["sel"][0])
        assert np.array_equal(rows[0].cpu().numpy(), r["n_rows"][0])
        assert out_error(out[0].cpu().numpy(), r["out"][0]) <= OUT_TOL


def test_split_merge_by_the_last_share_is_repeatable():
    """The split decode's last share to finish merges the head's records in
    share order, whatever order the shares finish in, and each call's
    scoring launch clears the arrival counters: forty calls in a row (two
    inputs alternating, the second with fewer rows per head) give
    bit-identical outputs per input, within PATH_TOL of the staged launches
    and, for one request at the conditioned k, within OUT_TOL of the
    oracle."""
    cfg = W.config(1, batch=2, n_tokens=30_000, n_kv_heads=4, n_q_heads=16, n_centroids=300, top_k=10, steps=2,
                   shared_codebook=False, seed=65)
    announce("split merge, 40 calls")
    p = _problem(cfg)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref = _check_index(p, [1], offsets, ids)
    qs = conditioned_ivf_queries(cfg, p["centroids"], 2)
    k_small = 3
    first = {}
    for i in range(40):
        j = i % 2
        k = cfg.top_k if j == 0 else k_small
        out = _decode("split", qs[j], p, offsets, ids, k).clone()
        if j not in first:
            first[j] = out
        else:
            assert torch.equal(out, first[j]), f"call {i} differs from the first call on the same input"
    for j, k in ((0, cfg.top_k), (1, k_small)):
        staged = _decode("staged", qs[j], p, offsets, ids, k)
        assert out_error(first[j].cpu().numpy(), staged.cpu().numpy()) <= PATH_TOL
    # the oracle at the k the queries were conditioned for
    r = ivf.sparse_decode(f64(qs[0][1:2]), f64(p["centroids"][1:2]), ref[1][0][None], ref[1][1][None],
                          f64(p["keys"][1:2]), f64(p["values"][1:2]), cfg.top_k)
    assert out_error(first[0][1].cpu().numpy(), r["out"][0]) <= OUT_TOL
