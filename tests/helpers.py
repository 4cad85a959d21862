"""Test-side helpers: input conditioning that uses only the oracle, tensor
conversions, the output error metric, and GPU-case announcements.

Conditioning makes every discrete decision of a parity case robust to the
difference between the oracle's fp64 arithmetic and the kernels' fp32
arithmetic: queries whose top-k boundary gap is below 1e-3 (relative) are
redrawn; indexer keys inside the boundary band are pushed below it.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import ivf, token
from top_sparse_attention_centroid_amd import workloads as W

GAP_MIN = 1e-3        # relative score gap at the top-k boundary
MARGIN_MIN = 1e-3     # relative squared-distance gap of every key assignment
OUT_TOL = 2e-3        # max over heads of |o - o_ref|_inf / |o_ref|_inf


def announce(msg: str):
    """Name the case before GPU work starts (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def out_error(out: np.ndarray, ref: np.ndarray) -> float:
    """max over (b, h) of |o - ref|_inf / |ref|_inf (refs with norm 0 compare absolutely)."""
    out = out.reshape(-1, out.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    num = np.max(np.abs(out - ref), axis=1)
    den = np.max(np.abs(ref), axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))


# ----------------------------------------------------------------------------
# inverted-index workloads
# ----------------------------------------------------------------------------

def ivf_query_gaps(q64: np.ndarray, cent64: np.ndarray, G: int, k: int) -> np.ndarray:
    """Oracle top-k boundary gap of every query. q64 [T][B][Hq][d], cent64 [Bc][Hkv][C][d]."""
    T, B, Hq, _ = q64.shape
    gaps = np.empty((T, B, Hq))
    for t in range(T):
        for b in range(B):
            cb = cent64[0 if cent64.shape[0] == 1 else b]
            for h in range(Hq):
                gaps[t, b, h] = ivf.selection_gap(ivf.centroid_scores(q64[t, b, h], cb[h // G]), k)
    return gaps


def conditioned_ivf_queries(cfg: W.WorkloadConfig, centroids: torch.Tensor, steps: int,
                            max_rounds: int = 40) -> torch.Tensor:
    """Queries [steps][B][Hq][d] (workload distribution) whose oracle top-k gap
    is >= GAP_MIN everywhere: failing queries are replaced by fresh draws."""
    q = W.ivf_queries(cfg, centroids, steps=steps)
    cent64 = f64(centroids)
    bad = ivf_query_gaps(f64(q), cent64, cfg.group, cfg.top_k) < GAP_MIN
    for salt in range(1, max_rounds + 1):
        if not bad.any():
            return q
        fresh = W.ivf_queries(cfg, centroids, steps=steps, salt=salt)
        mask = torch.from_numpy(bad).to(q.device)
        q = torch.where(mask[..., None], fresh, q)
        idx = np.argwhere(bad)
        q64 = f64(q)
        for t, b, h in idx:
            cb = cent64[0 if cent64.shape[0] == 1 else b]
            bad[t, b, h] = ivf.selection_gap(ivf.centroid_scores(q64[t, b, h], cb[h // cfg.group]),
                                             cfg.top_k) < GAP_MIN
    raise RuntimeError("could not draw queries with the required top-k gap")


def oracle_index(keys: torch.Tensor, centroids: torch.Tensor, requests=None):
    """Oracle posting lists for some requests (all by default): dict b -> (offsets, ids),
    plus the smallest assignment margin seen."""
    B = keys.shape[0]
    requests = range(B) if requests is None else requests
    cent64 = f64(centroids)
    lists, min_margin = {}, np.inf
    for b in requests:
        kb = f64(keys[b:b + 1])
        cb = cent64[0:1] if cent64.shape[0] == 1 else cent64[b:b + 1]
        off, ids, margins = ivf.index_build(kb, cb)
        lists[b] = (off[0], ids[0])
        min_margin = min(min_margin, float(margins.min()))
    return lists, min_margin


# ----------------------------------------------------------------------------
# token-indexer workload
# ----------------------------------------------------------------------------

def condition_token_keys(q_idx: torch.Tensor, k_idx: torch.Tensor, k: int, steps: int,
                         requests=None, push: float = 4e-3, max_passes: int = 16) -> torch.Tensor:
    """Return a copy of k_idx (same device/dtype) in which, for every step and
    request, no unselected token scores within GAP_MIN of the k-th score:
    such tokens are moved along -q by just enough to sit `push` (relative)
    below the k-th score, then re-rounded to the stored dtype; repeated until
    every (step, request) passes."""
    B = k_idx.shape[0]
    requests = range(B) if requests is None else requests
    kc = k_idx.detach().to("cpu").clone()
    q64 = f64(q_idx)
    for _ in range(max_passes):
        moved = False
        for b in requests:
            kb = kc[b].to(torch.float64).numpy()
            for t in range(steps):
                qv = q64[t, b]
                s = token.indexer_scores(qv, kb)
                order = np.lexsort((np.arange(len(s)), -s))
                sk = s[order[k - 1]]
                floor = sk - push * abs(sk)
                rest = order[k:]
                band = rest[s[rest] > sk - GAP_MIN * abs(sk)]
                if band.size == 0:
                    continue
                delta = (s[band] - floor)[:, None] * qv[None, :] / float(qv @ qv)
                new = torch.from_numpy(kb[band] - delta).to(kc.dtype)
                kc[b, torch.from_numpy(band)] = new
                kb[band] = new.to(torch.float64).numpy()
                moved = True
        if not moved:
            return kc.to(k_idx.device)
    raise RuntimeError("indexer keys could not be conditioned")
