"""GPU parity of the merged gather sets against the fp64 oracle, through the C ABI.

Large bf16 batches (at least 128 (request, KV head) groups, up to 4 query heads
per KV head) gather in workgroups of a few waves that take as many consecutive
plan segments, a segment per wave, and merge the heads' states through LDS
before writing them. These tests check every request and head of such batches:
sets of one head, sets that cross a head-class boundary or hold lists several
heads chose (the all-heads pass), sink/window ranges beside the lists, and a
list long enough that a workgroup loops over several sets.

Bars: selected lists bit-exact; outputs within OUT_TOL (max over heads of the
inf-norm error relative to the inf-norm of the oracle output)."""

import numpy as np
import pytest
import torch

import top_sparse_attention_centroid_amd as tsa
from oracle import ivf, variants
from top_sparse_attention_centroid_amd import workloads as W

from helpers import (GAP_MIN, MARGIN_MIN, OUT_TOL, announce, conditioned_ivf_queries, f64,
                      oracle_index, out_error)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _index_checked(p):
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    ref, margin = oracle_index(p["keys"], p["centroids"])
    assert margin >= MARGIN_MIN
    off_g, ids_g = offsets.cpu().numpy(), ids.cpu().numpy()
    for b, (o, i) in ref.items():
        assert np.array_equal(off_g[b], o) and np.array_equal(ids_g[b], i), f"index differs (request {b})"
    return offsets, ids


def test_merged_sets_whole_batch():
    # 16 x 8 = 128 groups (merged sets); 24 lists of ~170 rows, top-6 per head:
    # lists chosen by one head, by several, and class boundaries inside sets
    cfg = W.config(2, batch=16, n_tokens=4096, n_centroids=24, top_k=6, steps=1, seed=51)
    announce("merged sets: 16 x 4096, C = 24, top-6, every request")
    p = W.ivf_problem(cfg, device=DEV)
    offsets, ids = _index_checked(p)
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    B, Hq, k = cfg.batch, cfg.n_q_heads, cfg.top_k
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, sel_out=sel)
    torch.cuda.synchronize()
    k64, v64, c64 = f64(p["keys"]), f64(p["values"]), f64(p["centroids"])
    o64, i64 = offsets.cpu().numpy(), ids.cpu().numpy()
    r = ivf.sparse_decode(f64(q), c64, o64, i64, k64, v64, k)
    assert np.all(r["gap"] >= GAP_MIN)
    sel_g = sel.cpu().numpy()
    assert np.array_equal(sel_g, r["sel"]), "selection differs from the oracle"
    # the batch has both kinds of sets: lists one head chose and lists several chose
    per_list = np.zeros((B, cfg.n_kv_heads, cfg.n_centroids), dtype=int)
    for b in range(B):
        for h in range(Hq):
            per_list[b, h // cfg.group, sel_g[b, h]] += 1
    assert (per_list == 1).any() and (per_list >= 2).any()
    err = out_error(out.cpu().numpy(), r["out"])
    assert err <= OUT_TOL, f"output error {err}"

    # the same batch with a 64-token sink and a 300-token window before ragged
    # request lengths: direct segments ride in the mixed sets
    announce("merged sets: sink 64 + window 300, ragged lengths")
    lengths = torch.tensor([4096 - 97 * b for b in range(B)], dtype=torch.int32, device=DEV)
    sel2 = torch.empty_like(sel)
    out2 = tsa.sparse_decode_ex(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, n_sink=64,
                                n_window=300, lengths=lengths, sel_out=sel2)
    torch.cuda.synchronize()
    r2 = variants.sparse_decode_ex(f64(q), c64, o64, i64, k64, v64, k, n_sink=64, n_window=300,
                                   lengths=lengths.cpu().numpy())
    assert np.array_equal(sel2.cpu().numpy(), r2["sel"])
    err2 = out_error(out2.cpu().numpy(), r2["out"])
    assert err2 <= OUT_TOL, f"output error {err2}"


def test_merged_sets_loop_over_a_long_list():
    # 16 x 8 groups; most tokens of every request sit in list 0, so the chosen
    # list 0 is cut into far more segments than the average list length plans
    # for, and each workgroup walks several sets. Heads 0-1 of a group look for
    # list 0 and heads 2-3 for list 1: both lists are chosen by two heads.
    B, N, Hkv, Hq, C, k = 16, 4096, 8, 32, 8, 1
    cfg = W.config(2, batch=B, n_tokens=N, n_kv_heads=Hkv, n_q_heads=Hq, n_centroids=C, top_k=k, steps=1,
                   seed=52)
    announce("merged sets: one list of ~3000 rows, workgroups loop over sets")
    base = W.ivf_problem(cfg, device="cpu")
    cent = base["centroids"].float()  # [1][Hkv][C][d]
    gen = torch.Generator().manual_seed(520)
    comp = torch.randint(0, C, (B, N, Hkv), generator=gen)
    comp[:, : N * 3 // 4] = 0  # three quarters of the tokens in list 0
    noise = torch.randn((B, N, Hkv, cfg.head_dim), generator=gen)
    centre = cent[0][torch.arange(Hkv)[None, None, :], comp]  # [B][N][Hkv][d]
    keys = (centre + cfg.cluster_sd * noise).to(torch.bfloat16)
    p = {"centroids": base["centroids"].to(DEV), "keys": keys.to(DEV), "values": base["values"].to(DEV)}
    offsets, ids = _index_checked(p)
    want = torch.tensor([0, 0, 1, 1] * Hkv)  # target list per query head
    q = (cent[0][torch.arange(Hq) // cfg.group, want][None]
         + cfg.cluster_sd * torch.randn((B, Hq, cfg.head_dim), generator=gen)).to(torch.bfloat16).to(DEV)
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    rows = torch.empty((B, Hq), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, sel_out=sel,
                            rows_out=rows)
    torch.cuda.synchronize()
    r = ivf.sparse_decode(f64(q), f64(p["centroids"]), offsets.cpu().numpy(), ids.cpu().numpy(),
                          f64(p["keys"]), f64(p["values"]), k)
    assert np.all(r["gap"] >= GAP_MIN)
    assert np.array_equal(sel.cpu().numpy(), r["sel"])
    assert np.array_equal(sel.cpu().numpy()[..., 0], want[None].expand(B, Hq).numpy())
    assert np.array_equal(rows.cpu().numpy(), r["n_rows"])
    assert rows[:, 0].min().item() >= N * 3 // 4
    err = out_error(out.cpu().numpy(), r["out"])
    assert err <= OUT_TOL, f"output error {err}"


def test_merged_sets_empty_groups():
    # 32 requests x 4 KV heads = 128 groups, bf16, 2 query heads per KV head.
    # Small centroids live in dims 0..63; three far centroids in dims 64..127
    # own no keys. Requests b % 3 == 0: both heads of every group query a far
    # centroid, so the group has no plan segment at all; b % 3 == 1: head 0
    # far, head 1 small; b % 3 == 2: both small. Empty heads must come out
    # exactly zero with 0 rows; the rest match the oracle.
    g = torch.Generator().manual_seed(3)
    B, N, Hkv, G, C, d = 32, 600, 4, 2, 8, 128
    cent = torch.zeros(1, Hkv, C, d)
    cent[0, :, :5, :64] = torch.randn(Hkv, 5, 64, generator=g)
    cent[0, :, 5:, 64:] = 40.0 * torch.randn(Hkv, 3, 64, generator=g)
    comp = torch.randint(0, 5, (B, N, Hkv), generator=g)
    keys = cent[0][torch.arange(Hkv)[None, None, :], comp] + 0.3 * torch.randn(B, N, Hkv, d, generator=g)
    vals = torch.randn(B, N, Hkv, d, generator=g)
    target = torch.empty(B, Hkv * G, dtype=torch.long)
    for b in range(B):
        for h in range(Hkv * G):
            far = (b % 3 == 0) or (b % 3 == 1 and h % G == 0)
            target[b, h] = 5 + (b + h) % 3 if far else (b + h) % 5
    q = cent[0][torch.arange(Hkv * G)[None, :] // G, target]
    announce("merged sets: groups and heads with empty selections")
    keys, vals, cent, q = (x.to(torch.bfloat16).to(DEV) for x in (keys, vals, cent, q))
    offsets, ids = _index_checked({"keys": keys, "centroids": cent})
    rows = torch.empty((B, Hkv * G), dtype=torch.int32, device=DEV)
    sel = torch.empty((B, Hkv * G, 1), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode(q, cent, offsets, ids, keys, vals, 1, rows_out=rows, sel_out=sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy()[..., 0], target.numpy())
    r = ivf.sparse_decode(f64(q), f64(cent), offsets.cpu().numpy(), ids.cpu().numpy(), f64(keys), f64(vals), 1)
    assert np.array_equal(sel.cpu().numpy(), r["sel"])
    assert np.array_equal(rows.cpu().numpy(), r["n_rows"])
    o = out.cpu().numpy()
    empty = target.numpy() >= 5
    assert empty.any() and (~empty).any()
    assert np.all(rows.cpu().numpy()[empty] == 0) and np.all(o[empty] == 0.0)
    assert out_error(o[~empty], r["out"][~empty]) <= OUT_TOL


@pytest.mark.parametrize("batch", [2, 16])
def test_workspace_contents_never_reach_the_output(batch):
    # Records a head does not own stay unwritten; whatever the caller's
    # workspace held before (here NaN bit patterns, then zeros) must not
    # change the output. 2 x 8 groups: a wave per segment; 16 x 8: merged sets.
    cfg = W.config(2, batch=batch, n_tokens=4096, n_centroids=24, top_k=6, steps=1, seed=53)
    announce(f"workspace contents, {batch} requests")
    p = W.ivf_problem(cfg, device=DEV)
    offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    desc = tsa.binding.ivf_desc(p["keys"], p["centroids"], cfg.n_q_heads)
    nbytes = tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE_EX, desc, cfg.top_k)
    lengths = torch.tensor([4096 - 97 * b for b in range(batch)], dtype=torch.int32, device=DEV)
    outs = []
    for fill in (0xFF, 0x00):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        for kw in ({}, {"n_sink": 64, "n_window": 300, "lengths": lengths}):
            outs.append(tsa.sparse_decode_ex(q, p["centroids"], offsets, ids, p["keys"], p["values"], cfg.top_k,
                                             ws=ws, **kw))
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(o).all()) for o in outs)
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])


@pytest.mark.parametrize("G", [1, 2])
def test_merged_sets_fewer_query_heads_than_waves(G):
    # 16 x 8 groups with 1 or 2 query heads per KV head: some waves of a set
    # merge no head; every request and head against the oracle.
    cfg = W.config(2, batch=16, n_tokens=4096, n_kv_heads=8, n_q_heads=8 * G, n_centroids=24, top_k=6, steps=1,
                   seed=54 + G)
    announce(f"merged sets, {G} query heads per KV head")
    p = W.ivf_problem(cfg, device=DEV)
    offsets, ids = _index_checked(p)
    q = conditioned_ivf_queries(cfg, p["centroids"], 1)[0]
    B, Hq, k = cfg.batch, cfg.n_q_heads, cfg.top_k
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=DEV)
    out = tsa.sparse_decode(q, p["centroids"], offsets, ids, p["keys"], p["values"], k, sel_out=sel)
    torch.cuda.synchronize()
    r = ivf.sparse_decode(f64(q), f64(p["centroids"]), offsets.cpu().numpy(), ids.cpu().numpy(), f64(p["keys"]),
                          f64(p["values"]), k)
    assert np.all(r["gap"] >= GAP_MIN)
    assert np.array_equal(sel.cpu().numpy(), r["sel"])
    err = out_error(out.cpu().numpy(), r["out"])
    assert err <= OUT_TOL, f"output error {err}"
