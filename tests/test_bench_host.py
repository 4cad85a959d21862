"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the label of the
kernel whose roofline is reported, and the rule that stored HBM-traffic
counters are reported only for the kernel source they were taken on."""

import importlib
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    # imported under its own name from the repository root, so that the CPU
    # baseline's spawned workers can import it too
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    return importlib.import_module("bench")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _library_small_batch_groups():
    with open(os.path.join(ROOT, "top_sparse_attention_centroid_amd", "csrc", "capi.cpp")) as f:
        m = re.search(r"constexpr long long kSmallBatchGroups = (\d+);", f.read())
    assert m, "capi.cpp no longer defines the small-batch threshold"
    return int(m.group(1))


def _library_constant(fname, name):
    with open(os.path.join(ROOT, "top_sparse_attention_centroid_amd", "csrc", fname)) as f:
        m = re.search(rf"constexpr (?:long long|int) {name} = (\d+);", f.read())
    assert m, f"{fname} no longer defines {name}"
    return int(m.group(1))


def test_roofline_kernel_label_follows_the_library_dispatch(bench):
    from top_sparse_attention_centroid_amd import workloads as W

    threshold = _library_small_batch_groups()
    assert bench.SMALL_BATCH_GROUPS == threshold
    assert bench.FUSED_MAX_HEADS == _library_constant("capi.cpp", "kFusedMaxHeads")
    assert bench.FUSED_MAX_ROWS == _library_constant("capi.cpp", "kFusedMaxRows")
    assert bench.FUSED_MAX_CODEBOOK == _library_constant("capi.cpp", "kFusedMaxCodebook")
    assert bench.HEAD_MAX_C == _library_constant("kernels.hpp", "kHeadMaxC")
    assert bench.HEAD_MAX_K == _library_constant("kernels.hpp", "kHeadMaxK")

    class Auto:
        schedule, assign, sink, window = "auto", 1, 0, 0

    class Staged(Auto):
        schedule = "staged"

    names, staged, sched = {}, {}, {}
    for i in range(5):
        cfg = W.config(i)
        names[cfg.name] = bench.gather_kernel_name(cfg, Auto)
        staged[cfg.name] = bench.gather_kernel_name(cfg, Staged)
        sched[cfg.name] = bench.ivf_schedule(cfg, Auto)
        merged = (cfg.kind == "ivf" and cfg.batch * cfg.n_kv_heads >= threshold and cfg.dtype == "bf16"
                  and cfg.group <= 4)
        assert (staged[cfg.name] == "gather_merge_kernel") == merged, cfg.name
    assert sched == {"tiny-ivf-f32": "fused", "karat-ivf-100k": "split", "batched-ivf-64x32k": "staged",
                     "token-topk-16x200k": None, "hier-cache-32x128k": None}
    assert names["batched-ivf-64x32k"] == "gather_merge_kernel"
    assert names["karat-ivf-100k"] == names["tiny-ivf-f32"] == "ivf_head_kernel"
    assert staged["karat-ivf-100k"] == "gather_attn_kernel"
    assert names["token-topk-16x200k"] == "gather_attn_kernel"

    class TwoLists(Auto):
        assign = 2
    assert bench.gather_kernel_name(W.config(1), TwoLists) == "gather_attn_kernel"
    assert bench.ivf_schedule(W.config(0), None) == "fused"


def test_stored_traffic_is_used_only_for_the_source_it_was_taken_on(bench, tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    assert re.fullmatch(r"[0-9a-f]{16}", sha)
    good = tmp_path / "traffic.json"
    good.write_text(json.dumps({"batched-ivf-64x32k/gather_merge_kernel": {"kernel_source_sha": sha,
                                                                            "hbm_bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic("batched-ivf-64x32k", "gather_merge_kernel") == 123
    assert bench.measured_traffic("batched-ivf-64x32k", "gather_attn_kernel") is None
    assert bench.measured_traffic("karat-ivf-100k", "gather_merge_kernel") is None

    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"batched-ivf-64x32k/gather_merge_kernel": {"kernel_source_sha": "0" * 16,
                                                                             "hbm_bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic("batched-ivf-64x32k", "gather_merge_kernel") is None

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("batched-ivf-64x32k", "gather_merge_kernel") is None


def test_source_hash_covers_launch_code_and_header(bench, tmp_path, monkeypatch):
    """A change to any library source (not only the gather kernel's file)
    invalidates stored counter bytes."""
    import shutil
    src = tmp_path / "csrc"
    shutil.copytree(bench.SRC_DIR, src)
    hdr = tmp_path / "tsa.h"
    shutil.copy(bench.HEADER, hdr)
    monkeypatch.setattr(bench, "SRC_DIR", str(src))
    monkeypatch.setattr(bench, "HEADER", str(hdr))
    base = bench.kernel_source_sha()
    for path in (src / "kernels.hpp", src / "capi.cpp", src / "ivf.hip", hdr):
        orig = path.read_bytes()
        path.write_bytes(orig + b"\n// x\n")
        assert bench.kernel_source_sha() != base, path.name
        path.write_bytes(orig)
    assert bench.kernel_source_sha() == base


def test_committed_traffic_record_is_well_formed(bench):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    for key, entry in rec.items():
        workload, kernel = key.split("/")
        assert workload and kernel.endswith("_kernel"), key
        assert re.fullmatch(r"[0-9a-f]{16}", entry["kernel_source_sha"])
        assert entry["hbm_bytes_per_launch"] > 0
        assert entry["traffic_over_algorithmic"] == pytest.approx(
            entry["hbm_bytes_per_launch"] / entry["algorithmic_bytes_per_launch"], rel=1e-3)
        assert all(c.startswith("rocprofv3 --pmc ") and " -- python -u bench.py " in c for c in entry["commands"])


def _counter_csv(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    head = ('"Correlation_Id","Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
    body = "".join(f'{i},{i},"{name}","X",{val}\n' for i, (name, val) in enumerate(rows))
    path.write_text(head + body)


def test_traffic_record_scales_counters_by_the_copy_calibration(bench, tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE per dispatch of each kernel, scaled by what the
    counters read for a 1 GiB copy, against the bench line's algorithmic bytes."""
    d = tmp_path / "pmc"
    line = {"warmup": 0, "steps": 4, "config": {"workload": "token-topk-16x200k"}, "kernel_source_sha": "ab" * 8,
            "counter_kernels": {"gather_attn_kernel": 1000.0, "token_score_kernel": 4096.0}}
    d.mkdir()
    (d / "c3_FETCH_SIZE.log").write_text("[bench] noise\n" + json.dumps(line) + "\n")
    gk = "void tsa::gather_attn_kernel<__hip_bfloat16, 4>(tsa::AttnParams)"
    sk = "void tsa::token_score_kernel<__hip_bfloat16>(tsa::TokenSelectParams)"
    _counter_csv(d / "c3_FETCH_SIZE" / "run_counter_collection.csv",
                 [(gk, 1.0), (sk, 2.0), (gk, 3.0), (sk, 2.0), ("void tsa::gather_attn_kernel_x()", 99.0)])
    _counter_csv(d / "c3_WRITE_SIZE" / "run_counter_collection.csv", [(gk, 0.5), (sk, 1.0), (gk, 0.5), (sk, 1.0)])
    # the calibration copy reads half a GiB of FETCH_SIZE units for 1 GiB read: scale 2
    _counter_csv(d / "copy_FETCH_SIZE" / "run_counter_collection.csv", [("__amd_rocclr_copyBuffer", 524288.0)])
    _counter_csv(d / "copy_WRITE_SIZE" / "run_counter_collection.csv", [("__amd_rocclr_copyBuffer", 1048576.0)])
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))

    class A:
        record_traffic, config = str(d), 3
    bench.record_traffic(A)
    out = json.loads(rec.read_text())
    g = out["token-topk-16x200k/gather_attn_kernel"]
    assert g["dispatches"] == [2, 2]
    assert g["hbm_bytes_per_launch"] == round(2.0 * 1024 * 2 + 0.5 * 1024)
    assert g["traffic_over_algorithmic"] == pytest.approx(g["hbm_bytes_per_launch"] / 1000.0, rel=1e-3)
    s = out["token-topk-16x200k/token_score_kernel"]
    assert s["hbm_bytes_per_launch"] == 2.0 * 1024 * 2 + 1.0 * 1024
    assert s["kernel_source_sha"] == "ab" * 8


def test_oracle_baseline_runs_on_a_small_sample_on_one_and_several_cores(bench):
    """The CPU baseline leg: the oracle over a sample written for its worker
    processes, single-core in-process and on a spawned pool."""
    import torch

    from top_sparse_attention_centroid_amd import workloads as W
    cfg = W.config(0, n_tokens=512, n_centroids=16)
    p = W.ivf_problem(cfg)
    q = W.ivf_queries(cfg, p["centroids"], steps=3)
    data_dir, what = bench.cpu_sample_ivf(cfg, p, q, torch)

    class A:
        cpu_seconds = 0.4
    pool = bench.start_cpu_pool(2)
    try:
        res = bench.cpu_baseline(A, "ivf", data_dir, what, pool)
    finally:
        pool.terminate()
    assert res["kind"] == "oracle" and res["cores"] == 2 and res["unit"] == "queries/s"
    assert res["value"] > 0 and res["single_core_value"] > 0
    assert res["cpu_model"]
    assert not os.path.exists(data_dir)


def test_oracle_baseline_runner_covers_token_and_cache_samples(bench):
    import torch

    from top_sparse_attention_centroid_amd import workloads as W
    cfg = W.config(3, batch=1, n_tokens=3000, top_k=64, n_planted=16)
    prob = W.token_problem(cfg)
    q_idx, q = W.token_queries(cfg, prob, steps=2)
    data_dir, _ = bench.cpu_sample_token(cfg, prob, q_idx, q, torch)
    run = bench._OracleRunner("token", data_dir)
    for _ in range(3):
        run()
    import shutil
    shutil.rmtree(data_dir)

    cfg = W.config(4, batch=1, n_tokens=2000, n_slots=300, top_k=100, overlap=85, steps=4)
    prob = W.cache_problem(cfg)
    data_dir, _ = bench.cpu_sample_cache(cfg, prob["keys"], prob["values"], prob["q"], prob["trace"], 4, torch)
    run = bench._OracleRunner("cache", data_dir)
    for _ in range(9):                      # wraps past the trace's end: a fresh cold cache
        run()
    shutil.rmtree(data_dir)
