"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the label of the
kernel whose roofline is reported, and the rule that stored HBM-traffic
counters are reported only for the kernel source they were taken on."""

import importlib.util
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


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


def test_roofline_kernel_label_follows_the_library_dispatch(bench):
    from top_sparse_attention_centroid_amd import workloads as W

    threshold = _library_small_batch_groups()
    names = {}
    for i in range(5):
        cfg = W.config(i)
        names[cfg.name] = bench.gather_kernel_name(cfg, None)
        merged = (cfg.kind == "ivf" and cfg.batch * cfg.n_kv_heads >= threshold and cfg.dtype == "bf16"
                  and cfg.group <= 4)
        assert (names[cfg.name] == "gather_merge_kernel") == merged, cfg.name
    assert names["batched-ivf-64x32k"] == "gather_merge_kernel"
    assert names["karat-ivf-100k"] == "gather_attn_kernel"
    assert names["token-topk-16x200k"] == "gather_attn_kernel"


def test_stored_traffic_is_used_only_for_the_source_it_was_taken_on(bench, tmp_path, monkeypatch):
    sha = bench.gather_source_sha()
    assert re.fullmatch(r"[0-9a-f]{16}", sha)
    good = tmp_path / "traffic.json"
    good.write_text(json.dumps({"batched-ivf-64x32k": {"kernel_source_sha": sha, "hbm_bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.measured_traffic("batched-ivf-64x32k") == 123
    assert bench.measured_traffic("karat-ivf-100k") is None

    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"batched-ivf-64x32k": {"kernel_source_sha": "0" * 16,
                                                         "hbm_bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.measured_traffic("batched-ivf-64x32k") is None

    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("batched-ivf-64x32k") is None


def test_committed_traffic_record_is_well_formed(bench):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    entry = rec["batched-ivf-64x32k"]
    assert re.fullmatch(r"[0-9a-f]{16}", entry["kernel_source_sha"])
    assert entry["hbm_bytes_per_launch"] > 0
