"""The seeded input generators: determinism, shapes and the trace's overlap."""

import numpy as np
import torch

from top_sparse_attention_centroid_amd import workloads as W


def test_same_seed_same_bytes():
    cfg = W.config(0, n_tokens=512)
    a = W.ivf_problem(cfg)
    b = W.ivf_problem(cfg)
    for k in a:
        assert torch.equal(a[k], b[k])
    qa = W.ivf_queries(cfg, a["centroids"])
    qb = W.ivf_queries(cfg, b["centroids"])
    assert torch.equal(qa, qb)
    assert not torch.equal(qa, W.ivf_queries(cfg, a["centroids"], salt=1))
    c = W.ivf_problem(cfg.replace(seed=99))
    assert not torch.equal(a["keys"], c["keys"])


def test_ivf_shapes_and_dtypes():
    cfg = W.config(1, n_tokens=300, n_centroids=10, steps=3, batch=2)
    p = W.ivf_problem(cfg)
    assert p["centroids"].shape == (2, 8, 10, 128) and p["centroids"].dtype == torch.bfloat16
    assert p["keys"].shape == (2, 300, 8, 128) and p["values"].shape == (2, 300, 8, 128)
    q = W.ivf_queries(cfg, p["centroids"])
    assert q.shape == (3, 2, 32, 128) and q.dtype == torch.bfloat16
    cfg2 = W.config(2, n_tokens=300, batch=3, steps=2)
    p2 = W.ivf_problem(cfg2)
    assert p2["centroids"].shape == (1, 8, 256, 128)


def test_keys_cluster_around_the_codebook():
    cfg = W.config(0, n_tokens=2048)
    p = W.ivf_problem(cfg)
    k = p["keys"][0, :, 0].double()
    c = p["centroids"][0, 0].double()
    dist = torch.cdist(k, c).min(dim=1).values
    # within-cluster sd 0.3 in 128 dims: distance to the own centre ~ 0.3 * sqrt(128)
    assert abs(dist.mean().item() - 0.3 * 128 ** 0.5) < 0.1


def test_selection_trace_overlap_is_exact():
    cfg = W.config(4, batch=3, n_tokens=10_000, steps=6)
    tr = W.selection_trace(cfg)
    assert tr.shape == (6, 3, 2048) and tr.dtype == torch.int32
    for b in range(3):
        for t in range(6):
            row = tr[t, b]
            assert torch.all(row[1:] > row[:-1]) and row.min() >= 0 and row.max() < cfg.n_tokens
            if t:
                prev = set(tr[t - 1, b].tolist())
                assert len(prev & set(row.tolist())) == cfg.overlap == 1741
    assert torch.equal(tr, W.selection_trace(cfg))


def test_token_problem_plants_tokens():
    cfg = W.config(3, batch=2, n_tokens=5000, n_planted=32, steps=2)
    p = W.token_problem(cfg)
    assert p["k_idx"].shape == (2, 5000, 64) and p["planted"].shape == (2, 32)
    q_idx, q = W.token_queries(cfg, p)
    assert q_idx.shape == (2, 2, 64) and q.shape == (2, 2, 32, 128)
    s = (p["k_idx"][0].float() @ q_idx[0, 0].float())
    assert s[p["planted"][0]].min() > s.median() + 50


def test_locality_trace_keeps_the_overlap_and_returns_dropped_tokens():
    cfg = W.config(4, batch=2, n_tokens=6000, top_k=300, overlap=255, steps=30, popularity_sd=2.0, recency=0.3)
    tr = W.selection_trace(cfg).numpy()
    assert np.array_equal(tr, W.selection_trace(cfg).numpy())  # seeded
    returned = 0
    for b in range(cfg.batch):
        seen_dropped = set()
        for t in range(tr.shape[0]):
            row = tr[t, b]
            assert np.all(np.diff(row) > 0) and row.min() >= 0 and row.max() < cfg.n_tokens
            if t:
                prev = tr[t - 1, b]
                assert len(np.intersect1d(row, prev)) == cfg.overlap
                new = np.setdiff1d(row, prev)
                returned += len(np.intersect1d(new, np.fromiter(seen_dropped, dtype=np.int64)))
                seen_dropped |= set(np.setdiff1d(prev, row).tolist())
    # about 30 % of the 45 new tokens per step come back from recent drops
    assert returned >= 0.25 * 45 * (tr.shape[0] - 2) * cfg.batch
    # the uniform generator is untouched by the new fields' defaults
    base = W.config(4, batch=1, n_tokens=3000, top_k=200, overlap=170, steps=4)
    assert base.popularity_sd == 0 and base.recency == 0

