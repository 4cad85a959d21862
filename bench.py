"""Benchmark of retrieval-based sparse-attention decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one decode step of every request of the workload through the whole
hot path (centroid scoring, top-k lists, gather plan, gathered attention for
the inverted-index workloads; indexer scan, top-k and attention for the token
workload; RESOLVE and attention over the hot slots for the cache workload),
with inputs resident in HBM (the cache workload's authoritative KV in pinned
host memory). Prints one JSON line.

value  = decode queries per second (one query = one request's decode step,
         all of its heads) over the K timed steps;
roofline = the gather-attention kernel: algorithmic bytes (512 B per unique
         (request, KV head, token) K+V row it reads) / its mean launch time,
         timed with HIP events recorded by the library around each launch.
cpu_baseline = the fp64 oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-decode queries/s + gathered-KV GB/s as % of MI355X HBM peak"
HBM_PEAK_GBPS = 8000.0
ROW_BYTES_BF16 = 2 * 128 * 2  # one K row + one V row, 128 bf16 each
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
SRC_DIR = os.path.join(ROOT, "top_sparse_attention_centroid_amd", "csrc")
HEADER = os.path.join(ROOT, "include", "tsa.h")
KERNEL_NAMES = {"token_scan": "token_score_kernel", "resolve": "resolve_kernel"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", type=int, default=2, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--event-stride", type=int, default=7,
                    help="time the gather kernel with HIP events on every n-th timed step "
                         "(event records between kernels slow the stream a little)")
    ap.add_argument("--grow", type=int, default=0, metavar="PREFIX",
                    help="inverted-index workloads: build the index over the first PREFIX tokens with the "
                         "spare rows as per-list slack, then every step decodes over the growing index and "
                         "appends one new token per request (KV rows + posting list)")
    ap.add_argument("--slack", type=int, default=-1,
                    help="with --grow: free entries after every list (-1: the spare entries shared evenly); "
                         "a small slack makes lists run full, and the regrow that repairs them is timed")
    ap.add_argument("--schedule", default="auto", choices=["auto", "staged", "fused", "split"],
                    help="inverted-index decode: the library's choice, the staged launches, the fused single "
                         "launch or the split per-head launches (the last two: small plain decodes)")
    ap.add_argument("--kv-layout", default="token", choices=["token", "lists"],
                    help="inverted-index workloads: read the chosen lists' rows from the caches by token id "
                         "(token), or from list-major copies of the caches built once after the index "
                         "(lists: each list one contiguous run of rows)")
    ap.add_argument("--policy", default="lru", choices=["lru", "fifo", "random", "belady"],
                    help="hot-cache workload: replacement policy of RESOLVE (belady = offline, from the "
                         "trace's next-use steps)")
    ap.add_argument("--similarity", default="dot", choices=["dot", "cosine"],
                    help="inverted-index workloads: centroid similarity")
    ap.add_argument("--sink", type=int, default=0, help="inverted-index workloads: leading tokens always attended")
    ap.add_argument("--assign", type=int, default=1, choices=[1, 2, 3, 4],
                    help="inverted-index workloads: lists per key (m > 1: every key joins its m nearest lists; "
                         "with --grow, appends go into all m lists or none)")
    ap.add_argument("--window", type=int, default=0,
                    help="inverted-index workloads: trailing tokens always attended")
    ap.add_argument("--popularity", type=float, default=0.0,
                    help="hot-cache workload: selection trace with token popularity (standard deviation of "
                         "the log-normal token weights; 0 = uniform draws)")
    ap.add_argument("--recency", type=float, default=0.0,
                    help="hot-cache workload: share of each step's new tokens drawn from tokens dropped within "
                         "the last 8 steps (0 = none)")
    ap.add_argument("--layers", type=int, default=1,
                    help="hot-cache workload: a group of this many layers sharing each step's selection "
                         "(batch divided by the layer count, so host memory stays the same); the later "
                         "layers' rows are prefetched on a second stream while earlier layers attend")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (the gather kernel is then timed "
                         "in an eager pass over the same steps after the timed region)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline sample (0 disables it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--gpu-phase", metavar="FILE", help=argparse.SUPPRESS)
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write the HBM-traffic record of this workload's kernels from rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE passes under DIR (see record_traffic) and exit; no GPU work")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """sha256 prefix over every library source (kernels, launch and plan code,
    the C-ABI header): counter bytes are reported only while it matches."""
    h = hashlib.sha256()
    files = sorted(n for n in os.listdir(SRC_DIR) if n.endswith((".hip", ".hpp", ".cpp", ".h")))
    for path in [os.path.join(SRC_DIR, n) for n in files] + [HEADER]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# the library's automatic choice of an inverted-index decode's launches
FUSED_MAX_HEADS, FUSED_MAX_ROWS, FUSED_MAX_CODEBOOK = 256, 512, 65536
HEAD_MAX_C, HEAD_MAX_K = 1024, 64
SMALL_BATCH_GROUPS = 128


def ivf_schedule(cfg, args):
    """The launches libtsa runs this inverted-index decode with: "fused" (one
    workgroup per query head, one launch) when every head's work fits one CU,
    "split" (scoring, shares of every head's rows, combine) for other small
    bf16 batches, "staged" (scoring and plan, gather, combine) otherwise;
    only plain decodes (one list per key, no sink or window rows, C <= 1024,
    k <= 64) take the per-head ones. None for other workloads."""
    if cfg.kind != "ivf":
        return None
    schedule = getattr(args, "schedule", "auto")
    if schedule != "auto":
        return schedule
    plain = (getattr(args, "assign", 1) <= 1 and getattr(args, "sink", 0) == 0 and getattr(args, "window", 0) == 0
             and cfg.n_centroids <= HEAD_MAX_C and cfg.top_k <= HEAD_MAX_K)
    if not plain:
        return "staged"
    rows = cfg.top_k * cfg.n_tokens // cfg.n_centroids
    codebook = cfg.n_centroids * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
    if cfg.batch * cfg.n_q_heads <= FUSED_MAX_HEADS and rows <= FUSED_MAX_ROWS and codebook <= FUSED_MAX_CODEBOOK:
        return "fused"
    if cfg.dtype == "bf16" and cfg.batch * cfg.n_kv_heads < SMALL_BATCH_GROUPS:
        return "split"
    return "staged"


def gather_kernel_name(cfg, args) -> str:
    """The kernel libtsa runs the gather in for this workload: the per-head
    decode kernel under the fused and split schedules; under the staged one,
    merged sets of plan segments for inverted-index batches of at least 128
    bf16 (request, KV head) groups with up to 4 query heads per KV head, one
    wave per segment (or per row-list segment) otherwise."""
    if ivf_schedule(cfg, args) in ("fused", "split"):
        return "ivf_head_kernel"
    groups = cfg.batch * cfg.n_kv_heads
    if cfg.kind == "ivf" and groups >= SMALL_BATCH_GROUPS and cfg.dtype == "bf16" and cfg.group <= 4:
        return "gather_merge_kernel"
    return "gather_attn_kernel"


def codebook_bytes(cfg) -> int:
    """Bytes of the centroids one decode step scores (every KV head's codebook
    of every request; a shared codebook counts once per request here, as
    each request's scoring reads it)."""
    return cfg.batch * cfg.n_kv_heads * cfg.n_centroids * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    record, if it was taken on the current library source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(f"{workload}/{kernel}")
    if not entry or entry.get("kernel_source_sha") != kernel_source_sha():
        return None
    return entry.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------
# inverted-index workloads
# ----------------------------------------------------------------------------

def bench_ivf_grow(args, cfg, torch, tsa, W):
    """Decode over a growing index, then append the next token of every
    request; the append kernel is timed with its own events."""
    dev = "cuda"
    B, Hq, Hkv, k, N, C = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k, cfg.n_tokens, cfg.n_centroids
    prefix = args.grow
    total = args.warmup + args.steps
    if not (1 <= prefix and prefix + total <= N):
        sys.exit(f"bench: --grow needs 1 <= PREFIX and PREFIX + warmup + steps <= {N}")
    if args.graph:
        sys.exit("bench: --grow changes the index every step; it runs eagerly")
    if args.kv_layout != "token":
        sys.exit("bench: --grow reads the caches by token id (the list-major copies describe a static index)")
    log(f"generating {cfg.name} on the GPU (growing from {prefix} tokens)")
    p = W.ivf_problem(cfg, device=dev)
    nq = min(cfg.steps, 64)
    q_all = W.ivf_queries(cfg, p["centroids"], steps=nq)
    m = args.assign
    slack = (N - prefix) * m // C if args.slack < 0 else args.slack
    k_cache, v_cache = p["keys"], p["values"]       # rows >= prefix are rewritten by the appends
    offsets, lens, ids, alt = tsa.index_build_dyn_multi(k_cache, p["centroids"], prefix, m, slack)
    new_k = p["keys"][:, prefix:prefix + total].transpose(0, 1).contiguous()    # [steps][B][Hkv][d]
    new_v = p["values"][:, prefix:prefix + total].transpose(0, 1).contiguous()
    pos = (prefix + torch.arange(total, device=dev, dtype=torch.int32))[:, None].expand(total, B).contiguous()
    status = torch.empty((total, B, Hkv), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, cfg.head_dim), dtype=torch.float32, device=dev)
    uniq = torch.empty((total, B, Hkv), dtype=torch.int32, device=dev)
    desc = tsa.binding.ivf_desc(k_cache, p["centroids"], Hq)
    if m == 1:  # the options' workspace covers the plain decode too
        ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE_EX, desc, k), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE_EX_MULTI, desc, k, m), dtype=torch.uint8,
                         device=dev)
    torch.cuda.synchronize()

    def bind_step(i):
        """Step i's decode and append, bound once (see bound_steps)."""
        if m == 1 and args.schedule == "auto":
            dec = tsa.sparse_decode_dyn(q_all[i % nq], p["centroids"], offsets, lens, ids, k_cache, v_cache, k,
                                        out=out, uniq_out=uniq[i], ws=ws, bind=True)
        else:
            dec = tsa.sparse_decode_ex(q_all[i % nq], p["centroids"], offsets, ids, k_cache, v_cache, k, lens=lens,
                                       alt=alt, out=out, uniq_out=uniq[i], ws=ws, schedule=args.schedule, bind=True)
        app = tsa.kv_append(new_k[i], new_v[i], pos[i], p["centroids"], k_cache, v_cache, offsets, lens, ids,
                            alt=alt, status=status[i], bind=True)
        return dec, app

    steps = [bind_step(i) for i in range(total)]

    def call(i):
        dec, app = steps[i]
        dec()
        app()

    res = _timed(args, call, torch, tsa, n_distinct=total, offset=args.warmup)
    row_bytes = 2 * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
    per_step = uniq.sum(dim=(1, 2)).cpu().double()[args.warmup:]
    res["step_bytes"] = [float(x) * row_bytes for x in per_step]
    res.update({"gathered_bytes": float(per_step.sum()) * row_bytes, "queries": B * args.steps,
                "unique_rows_per_step": float(per_step.mean())})
    if ivf_schedule(cfg, args) == "fused":
        res["gather_launch_bytes"] = [x + codebook_bytes(cfg) for x in res["step_bytes"]]
    st = status[args.warmup:].cpu()
    # the append kernel, timed after the timed region (event records inside
    # it slow the whole eager step): the timed steps' appends again, on
    # copies of the lists (the K/V rows are rewritten with the same values)
    lens_c, ids_c = lens.clone(), ids.clone()
    alt_c = None if alt is None else alt.clone()
    st_c = torch.empty_like(status[0])
    aev = {}
    for j in res["timed_steps"]:
        i = j + args.warmup
        aev[i] = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        tsa.time_next_launch(tsa.binding.TIMED_APPEND, *aev[i])
        tsa.kv_append(new_k[i], new_v[i], pos[i], p["centroids"], k_cache, v_cache, offsets, lens_c, ids_c,
                      alt=alt_c, status=st_c)
    torch.cuda.synchronize()
    a_ms = [a.elapsed_time(b) for a, b in aev.values()]
    del lens_c, ids_c, alt_c
    # repair of the grown index: the same lists laid out again with the
    # largest slack that fits, its kernel timed with events over five runs
    # (after the timed region; the arrays are written to a second set)
    out_arrays = (torch.empty_like(offsets), torch.empty_like(lens), torch.empty_like(ids),
                  None if alt is None else torch.empty_like(alt))
    rstat = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    r_ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tsa.time_next_launch(tsa.binding.TIMED_REGROW, e0, e1)
        tsa.index_regrow(offsets, lens, ids, alt, -1, out=out_arrays, status=rstat)
        torch.cuda.synchronize()
        r_ms.append(e0.elapsed_time(e1))
    # every output entry is written once and every valid entry read once
    # (m ints per entry: the id and its m - 1 other lists)
    cap = ids.shape[-1]
    valid = int(lens.clamp(min=0).sum())
    r_bytes = (B * Hkv * cap + valid) * m * 4
    r_mean = sum(r_ms) / len(r_ms)
    res["regrow"] = {"mean_us": round(r_mean * 1e3, 2), "min_us": round(min(r_ms) * 1e3, 2),
                     "capacity_per_group": cap, "valid_entries": valid, "bytes_per_launch": r_bytes,
                     "gbps": round(r_bytes / (r_mean * 1e-3) / 1e9, 1), "groups_that_fit": int((rstat == 0).sum()),
                     "timing": "HIP events recorded by the library around the regrow kernel "
                               "(tsa_time_next_launch), 5 runs after the timed region"}
    res["append"] = {"prefix_tokens": prefix, "slack_per_list": slack, "lists_per_key": m,
                     "mean_us": round(sum(a_ms) / len(a_ms) * 1e3, 2),
                     "indexed": int((st == 0).sum()), "list_full": int((st == 1).sum()),
                     "bytes_per_launch": B * Hkv * 2 * row_bytes,
                     "refused_appends": "a key whose m lists are not all free joins none (status 1); "
                                        "index_regrow lays the lists out again with fresh free entries",
                     "timing": "HIP events recorded by the library around the kv_append kernel "
                               "(tsa_time_next_launch), the timed steps' appends repeated on copies of the lists "
                               "after the timed region"}
    return res


def bench_ivf(args, cfg, torch, tsa, W):
    if args.grow:
        return bench_ivf_grow(args, cfg, torch, tsa, W)
    dev = "cuda"
    B, Hq, Hkv, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k
    log(f"generating {cfg.name} on the GPU")
    p = W.ivf_problem(cfg, device=dev)
    nq = min(cfg.steps, 64)
    q_all = W.ivf_queries(cfg, p["centroids"], steps=nq)
    t0 = time.perf_counter()
    alt = None
    if args.assign > 1:
        offsets, ids, alt = tsa.index_build_multi(p["keys"], p["centroids"], args.assign)
    else:
        offsets, ids = tsa.index_build(p["keys"], p["centroids"])
    torch.cuda.synchronize()
    index_ms = (time.perf_counter() - t0) * 1e3
    k_lists = v_lists = None
    lists_ms = None
    if args.kv_layout == "lists":
        t0 = time.perf_counter()
        k_lists, v_lists = tsa.kv_list_major(ids, p["keys"], p["values"])
        torch.cuda.synchronize()
        lists_ms = (time.perf_counter() - t0) * 1e3
    out = torch.empty((B, Hq, cfg.head_dim), dtype=torch.float32, device=dev)
    uniq = torch.empty((nq, B, Hkv), dtype=torch.int32, device=dev)
    desc = tsa.binding.ivf_desc(p["keys"], p["centroids"], Hq)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE, desc, k), dtype=torch.uint8, device=dev)

    variant = (args.similarity != "dot" or args.sink > 0 or args.window > 0 or alt is not None
               or args.schedule != "auto" or k_lists is not None)
    # the schedule and the K/V layout change how, not what, the step computes
    same_math = args.similarity == "dot" and args.sink == 0 and args.window == 0 and alt is None
    if variant:
        if alt is not None:
            need = tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE_EX_MULTI, desc, k, args.assign)
        else:
            need = tsa.workspace_bytes(tsa.binding.OP_SPARSE_DECODE_EX, desc, k)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def decode(i, bind=False):
        if variant:
            return tsa.sparse_decode_ex(q_all[i % nq], p["centroids"], offsets, ids, p["keys"], p["values"], k,
                                        similarity=args.similarity, n_sink=args.sink, n_window=args.window,
                                        alt=alt, out=out, uniq_out=uniq[i % nq], ws=ws, schedule=args.schedule,
                                        k_lists=k_lists, v_lists=v_lists, bind=bind)
        return tsa.sparse_decode(q_all[i % nq], p["centroids"], offsets, ids, p["keys"], p["values"], k,
                                 out=out, uniq_out=uniq[i % nq], ws=ws, bind=bind)

    res = _timed(args, bound_steps(args, decode, nq), torch, tsa, n_distinct=nq)
    # rows read per step: unique list rows, plus the sink / window rows (an
    # upper bound: a list row inside those ranges is read once, counted twice;
    # with m lists per key, list entries: a token in several chosen lists of
    # the group counts once per list)
    fixed = min(args.sink + args.window, cfg.n_tokens) * B * Hkv
    rows_per_set = uniq.sum(dim=(1, 2)).cpu().double() + fixed
    rows = sum(float(rows_per_set[i % nq]) for i in range(args.steps))
    res["step_bytes"] = [float(rows_per_set[i % nq]) * (2 * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4))
                         for i in range(args.steps)]
    row_bytes = 2 * cfg.head_dim * (2 if cfg.dtype == "bf16" else 4)
    res.update({"gathered_bytes": rows * row_bytes, "queries": B * args.steps, "index_build_ms": index_ms,
                "unique_rows_per_step": rows / args.steps})
    if lists_ms is not None:
        res["kv_lists_build_ms"] = lists_ms
    if ivf_schedule(cfg, args) == "fused":
        # the fused kernel also scores the codebook: its bytes once per group
        res["gather_launch_bytes"] = [x + codebook_bytes(cfg) for x in res["step_bytes"]]
    if args.cpu_seconds > 0 and same_math:
        res["cpu_sample"] = ("ivf",) + cpu_sample_ivf(cfg, p, q_all, torch)
    return res


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload, on one
# core and on all the host cores this process may use (one process per core,
# one BLAS thread each). It runs in the parent process after the GPU run (a
# child process) has ended: worker processes alive during the timed GPU
# region were measured to slow the host's launches several times over.
# ----------------------------------------------------------------------------

CPU_SAMPLE_REQUESTS = 2      # requests of the sample (queries cycle over them and the steps)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    """Cores this process may run on, capped at the 16 a one-GPU share of the
    host provides."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _worker_ready(_):
    time.sleep(0.2)
    return os.getpid()


def start_cpu_pool(n):
    """Worker processes for the all-cores leg, waited for until every one has
    started (the process that starts them never touches the GPU)."""
    import multiprocessing as mp
    pool = mp.get_context("spawn").Pool(n)
    for _ in range(20):
        if len(set(pool.map(_worker_ready, range(2 * n), chunksize=1))) == n:
            break
    return pool


def cpu_quota():
    """The cgroup CPU limit of this process, in cores (None if unlimited or
    unknown)."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()[:2]
        return None if quota == "max" else round(int(quota) / int(period), 2)
    except (OSError, ValueError):
        return None


class _OracleRunner:
    """One oracle decode query of the sample per call: the data is the
    sample's arrays, saved as fp32 (exact for bf16) .npy files and mapped
    read-only, so every worker shares one copy in the page cache."""

    def __init__(self, kind, data_dir, offset=0):
        import numpy as np

        def ld(name):
            return np.load(os.path.join(data_dir, name + ".npy"), mmap_mode="r")

        with open(os.path.join(data_dir, "meta.json")) as f:
            self.meta = json.load(f)
        self.kind, self.i = kind, offset
        self.R, self.T = self.meta["requests"], self.meta["steps"]
        self.K = [ld(f"K{r}") for r in range(self.R)]
        self.V = [ld(f"V{r}") for r in range(self.R)]
        self.q = ld("q")
        if kind == "ivf":
            self.cent = [ld(f"cent{r}") for r in range(self.R)]
            self.off = [ld(f"off{r}") for r in range(self.R)]
            self.ids = [ld(f"ids{r}") for r in range(self.R)]
        elif kind == "token":
            self.kidx = [ld(f"kidx{r}") for r in range(self.R)]
            self.qidx = ld("qidx")
        else:
            self.trace = ld("trace")
            self._fresh_caches()

    def _fresh_caches(self):
        import numpy as np
        from oracle import cache
        m = self.meta
        self.state = [cache.CacheState(m["n_tokens"], m["n_slots"]) for _ in range(self.R)]
        shape = (m["n_slots"], m["n_kv_heads"], m["head_dim"])
        self.pool = [(np.zeros(shape), np.zeros(shape)) for _ in range(self.R)]

    def __call__(self):
        from oracle import cache, ivf, token
        i, R, k = self.i, self.R, self.meta["top_k"]
        self.i += 1
        r = i % R
        t = (i // R) % self.T
        if self.kind == "ivf":
            ivf.sparse_decode(self.q[t, r:r + 1], self.cent[r], self.off[r], self.ids[r], self.K[r], self.V[r], k)
        elif self.kind == "token":
            token.token_decode(self.qidx[t, r:r + 1], self.kidx[r][None], self.q[t, r:r + 1], self.K[r][None],
                               self.V[r][None], k)
        else:
            if t == 0 and r == 0 and i > 0:
                self._fresh_caches()             # the trace starts over from a cold cache
            slots, _, _, fetches = cache.lru_step(self.state[r], self.trace[t, r], t)
            cache.fetch_rows(self.pool[r][0], self.pool[r][1], self.K[r], self.V[r], fetches)
            cache.attend_slots(self.q[t, r], self.pool[r][0], self.pool[r][1], slots)


def cpu_oracle_loop(task):
    """Runs oracle queries for `seconds`; returns (queries done, seconds)."""
    kind, data_dir, seconds, offset = task
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        run = _OracleRunner(kind, data_dir, offset)
        run()                                     # page the sample in, untimed
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            run()
            done += 1
        return done, time.perf_counter() - t0


def cpu_baseline(args, kind, data_dir, what, pool):
    """Single-core leg in this process, then the all-cores leg on the pool."""
    import shutil
    try:
        one, el1 = cpu_oracle_loop((kind, data_dir, args.cpu_seconds / 2, 0))
        res = {"value": one / el1, "unit": "queries/s", "cores": 1, "kind": "oracle",
               "sample": f"{one} {what} over {el1:.1f} s on one core (fp64 numpy, one BLAS thread)",
               "cpu_model": cpu_model(), "cpu_quota_cores": cpu_quota(), "os_cpu_count": os.cpu_count()}
        if pool is not None:
            n = pool._processes
            outs = pool.map(cpu_oracle_loop, [(kind, data_dir, args.cpu_seconds / 2, 7919 * w) for w in range(n)])
            total = sum(c for c, _ in outs)
            el = max(e for _, e in outs)
            res.update({"value": sum(c / e for c, e in outs), "cores": n,
                        "sample": f"{total} {what} over {el:.1f} s on {n} cores (one process per core, fp64 "
                                  f"numpy, one BLAS thread each); one core: {one} in {el1:.1f} s",
                        "single_core_value": one / el1})
        return res
    finally:
        shutil.rmtree(data_dir, ignore_errors=True)


def _sample_dir(meta, arrays):
    """Writes the sample's arrays (fp32 / int) for the oracle workers."""
    import tempfile

    import numpy as np
    d = tempfile.mkdtemp(prefix="tsa_oracle_", dir="/tmp")
    for name, a in arrays.items():
        np.save(os.path.join(d, name + ".npy"), a)
    with open(os.path.join(d, "meta.json"), "w") as f:
        json.dump(meta, f)
    return d


def _f32np(t, torch):
    return t.detach().to("cpu", torch.float32).numpy()


def cpu_sample_ivf(cfg, p, q_all, torch):
    from oracle import ivf
    R = min(CPU_SAMPLE_REQUESTS, cfg.batch)
    log(f"oracle baseline: building its index for requests 0..{R - 1}")
    arrays = {"q": _f32np(q_all[:, :R], torch)}
    cent = _f32np(p["centroids"], torch)
    for r in range(R):
        cb = cent[0:1] if cent.shape[0] == 1 else cent[r:r + 1]
        K = _f32np(p["keys"][r:r + 1], torch)
        off, ids, _ = ivf.index_build(K, cb)
        arrays.update({f"K{r}": K, f"V{r}": _f32np(p["values"][r:r + 1], torch), f"cent{r}": cb,
                       f"off{r}": off, f"ids{r}": ids})
    meta = {"requests": R, "steps": int(q_all.shape[0]), "top_k": cfg.top_k}
    return _sample_dir(meta, arrays), f"whole decode queries (all {cfg.n_q_heads} heads; index built untimed)"


def cpu_sample_token(cfg, prob, q_idx, q, torch):
    R = 1                        # one request's 200K-token K/V (fp32) is already 1.6 GB of sample
    arrays = {"q": _f32np(q[:, :R], torch), "qidx": _f32np(q_idx[:, :R], torch)}
    for r in range(R):
        arrays.update({f"K{r}": _f32np(prob["keys"][r], torch), f"V{r}": _f32np(prob["values"][r], torch),
                       f"kidx{r}": _f32np(prob["k_idx"][r], torch)})
    meta = {"requests": R, "steps": int(q.shape[0]), "top_k": cfg.top_k}
    return _sample_dir(meta, arrays), (f"whole decode queries (indexer top-{cfg.top_k} over {cfg.n_tokens} "
                                       f"tokens, attention of all {cfg.n_q_heads} heads)")


def cpu_sample_cache(cfg, hk, hv, q, trace, steps, torch):
    R = 1                        # one request's 128K-token K/V (fp32) is already 1 GB of sample
    arrays = {"q": _f32np(q[:steps, :R], torch), "trace": trace[:steps, :R].cpu().numpy()}
    for r in range(R):
        arrays.update({f"K{r}": _f32np(hk[r], torch), f"V{r}": _f32np(hv[r], torch)})
    meta = {"requests": R, "steps": steps, "top_k": cfg.top_k, "n_tokens": cfg.n_tokens, "n_slots": cfg.n_slots,
            "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim}
    return _sample_dir(meta, arrays), (f"decode queries from a cold cache (LRU step, host fetch into the "
                                       f"oracle's pool, attention of all {cfg.n_q_heads} heads over the slots)")


# ----------------------------------------------------------------------------
# token-indexer workload
# ----------------------------------------------------------------------------

def bench_token(args, cfg, torch, tsa, W):
    dev = "cuda"
    B, Hq, k = cfg.batch, cfg.n_q_heads, cfg.top_k
    log(f"generating {cfg.name} on the GPU")
    prob = W.token_problem(cfg, device=dev)
    nq = min(cfg.steps, 64)
    q_idx, q = W.token_queries(cfg, prob, steps=nq)
    out = torch.empty((B, Hq, cfg.head_dim), dtype=torch.float32, device=dev)
    desc = tsa.binding.token_desc(prob["k_idx"], prob["keys"], Hq)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_TOKEN_DECODE, desc, k), dtype=torch.uint8, device=dev)

    def decode(i, bind=False):
        return tsa.token_decode(q_idx[i % nq], prob["k_idx"], q[i % nq], prob["keys"], prob["values"], k,
                                out=out, ws=ws, bind=bind)

    res = _timed(args, bound_steps(args, decode, nq), torch, tsa, n_distinct=nq, kernels=("gather", "token_scan"))
    res["gathered_bytes"] = args.steps * B * cfg.n_kv_heads * k * ROW_BYTES_BF16
    res["step_bytes"] = [B * cfg.n_kv_heads * k * ROW_BYTES_BF16] * args.steps
    # the scan reads every indexer key (d_idx bf16) and writes one 4-byte score key per token
    res["kernel_step_bytes"] = {"token_scan": [B * cfg.n_tokens * (cfg.idx_dim * 2 + 4)] * args.steps}
    res["queries"] = B * args.steps
    res["indexer_bytes_per_step"] = B * cfg.n_tokens * cfg.idx_dim * 2
    if args.cpu_seconds > 0:
        res["cpu_sample"] = ("token",) + cpu_sample_token(cfg, prob, q_idx, q, torch)
    return res


# ----------------------------------------------------------------------------
# hierarchical-cache workload
# ----------------------------------------------------------------------------

def bench_cache_layers(args, cfg, torch, tsa, W):
    """A layer group sharing the selection: RESOLVE once per step, the other
    layers' rows fetched on a second stream while earlier layers attend.
    Runs the overlapped schedule (timed as the result) and then the in-order
    schedule on a fresh cache over the same trace, for comparison."""
    dev = "cuda"
    L = args.layers
    if args.graph:
        sys.exit("bench: --layers runs eagerly (the cache walks its state once per step)")
    cfg = cfg.replace(batch=max(1, cfg.batch // L))
    B, N, S, Hkv, Hq, d, k = (cfg.batch, cfg.n_tokens, cfg.n_slots, cfg.n_kv_heads, cfg.n_q_heads,
                              cfg.head_dim, cfg.top_k)
    steps = args.warmup + args.steps
    log(f"generating {cfg.name} x {L} layers ({B} requests): full KV of every layer in pinned host memory")
    cfg_t = cfg.replace(steps=steps)
    trace = W.selection_trace(cfg_t).to(dev)
    layers = []
    for j in range(L):
        prob = W.cache_problem(cfg_t.replace(seed=cfg.seed + 100 * j), device=dev)
        hk = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
        hv = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
        hk.tensor.copy_(prob["keys"])
        hv.tensor.copy_(prob["values"])
        layers.append({"hk": hk, "hv": hv, "q": prob["q"]})
        del prob
    torch.cuda.empty_cache()

    def fresh_state():
        pt = torch.empty((B, N), dtype=torch.int32, device=dev)
        st = torch.empty((B, S), dtype=torch.int32, device=dev)
        lu = torch.empty((B, S), dtype=torch.int32, device=dev)
        tsa.cache_reset(pt, st, lu)
        pools = [(torch.zeros((B, S, Hkv, d), dtype=cfg.torch_dtype, device=dev),
                  torch.zeros((B, S, Hkv, d), dtype=cfg.torch_dtype, device=dev)) for _ in range(L)]
        outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(L)]
        return pt, st, lu, pools, outs

    misses = torch.empty((steps, B), dtype=torch.int32, device=dev)
    slots = torch.empty((B, k), dtype=torch.int32, device=dev)
    miss_tok = torch.empty((B, k), dtype=torch.int32, device=dev)
    miss_slot = torch.empty((B, k), dtype=torch.int32, device=dev)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_ATTEND_ROWS, tsa.binding.AttnDesc(B, S, Hkv, Hq, d, k, 1)),
                     dtype=torch.uint8, device=dev)
    fetch_stream = torch.cuda.Stream()
    events = [torch.cuda.Event(), torch.cuda.Event()]

    def make_call(state, fs):
        pt, st, lu, pools, outs = state

        def call(i):
            io = [{"host_k": Lj["hk"].tensor, "host_v": Lj["hv"].tensor, "pool_k": pools[j][0],
                   "pool_v": pools[j][1], "q": Lj["q"][i], "out": outs[j]} for j, Lj in enumerate(layers)]
            tsa.hier_group_step(io, pt, st, lu, trace[i], i, slots_out=slots, misses=misses[i], miss_tok=miss_tok,
                                miss_slot=miss_slot, ws=ws, fetch_stream=fs, events=events if fs else None)
        return call

    # alternate the schedules (in order, overlapped, twice each, each from a
    # fresh cache over the same trace) so that neither gains from the other
    # having warmed the host mappings; the second round is reported
    for _ in range(2):
        serial = _timed(args, make_call(fresh_state(), None), torch, tsa, n_distinct=steps, offset=args.warmup)
        res = _timed(args, make_call(fresh_state(), fetch_stream), torch, tsa, n_distinct=steps, offset=args.warmup)
    m = misses.cpu()
    res["gathered_bytes"] = args.steps * L * B * Hkv * k * ROW_BYTES_BF16
    res["step_bytes"] = [B * Hkv * k * ROW_BYTES_BF16] * args.steps     # one timed gather = one layer
    res["queries"] = B * args.steps
    res["misses_per_step"] = m.sum(dim=1).tolist()
    res["miss_rate_steady"] = float(m[args.warmup:].double().mean() / k)
    res["fetched_bytes"] = float(m[args.warmup:].double().sum()) * Hkv * d * 2 * 2 * L
    res["batch"] = B
    res["layer_group"] = {"layers": L, "requests": B, "prefetch_stream": True, "rounds": 2,
                          "ms_per_step_overlapped": round(res["ms_total"] / args.steps, 4),
                          "ms_per_step_in_order": round(serial["ms_total"] / args.steps, 4)}
    return res


def bench_cache(args, cfg, torch, tsa, W):
    if args.layers > 1:
        return bench_cache_layers(args, cfg, torch, tsa, W)
    dev = "cuda"
    B, N, S, Hkv, Hq, d, k = (cfg.batch, cfg.n_tokens, cfg.n_slots, cfg.n_kv_heads, cfg.n_q_heads,
                              cfg.head_dim, cfg.top_k)
    if args.graph:
        sys.exit("bench: --graph is for the stateless decode workloads; the cache walks its state "
                 "once per step, so its steps cannot be re-run for the kernel timing pass")
    steps = args.warmup + args.steps
    log(f"generating {cfg.name}: full KV into pinned host memory")
    cfg_t = cfg.replace(steps=steps)
    prob = W.cache_problem(cfg_t, device=dev)
    hk = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
    hv = tsa.HostArray((B, N, Hkv, d), cfg.torch_dtype)
    hk.tensor.copy_(prob["keys"])
    hv.tensor.copy_(prob["values"])
    del prob["keys"], prob["values"]
    pt = torch.empty((B, N), dtype=torch.int32, device=dev)
    st = torch.empty((B, S), dtype=torch.int32, device=dev)
    lu = torch.empty((B, S), dtype=torch.int32, device=dev)
    tsa.cache_reset(pt, st, lu)
    pool_k = torch.zeros((B, S, Hkv, d), dtype=cfg.torch_dtype, device=dev)
    pool_v = torch.zeros_like(pool_k)
    trace = prob["trace"].to(dev)
    q = prob["q"]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    slots = torch.empty((B, k), dtype=torch.int32, device=dev)
    hits = torch.empty((steps, B), dtype=torch.int32, device=dev)
    misses = torch.empty((steps, B), dtype=torch.int32, device=dev)
    desc = tsa.binding.attn_desc(pool_k, Hq, k)
    ws = torch.empty(tsa.workspace_bytes(tsa.binding.OP_ATTEND_ROWS, desc), dtype=torch.uint8, device=dev)

    # events around each RESOLVE launch (same stream as the library call)
    rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    prio = None
    if args.policy == "belady":
        # next step that selects each token, per step (offline knowledge of the trace)
        never = 2**31 - 1
        prio = torch.empty((steps, B, N), dtype=torch.int32, device=dev)
        nxt = torch.full((B, N), never, dtype=torch.int32, device=dev)
        for t in range(steps - 1, -1, -1):
            prio[t] = nxt
            nxt.scatter_(1, trace[t].long(), t)
    gpu_policy = "priority" if args.policy == "belady" else args.policy

    def call(i):
        rev[i][0].record()
        tsa.resolve(pt, st, lu, trace[i], i, hk.tensor, hv.tensor, pool_k, pool_v, slots_out=slots,
                    hits=hits[i], misses=misses[i], policy=gpu_policy, seed=0x5EED,
                    priority=None if prio is None else prio[i])
        rev[i][1].record()
        tsa.attend_rows(q[i], pool_k, pool_v, slots, out=out, ws=ws)

    res = _timed(args, call, torch, tsa, n_distinct=steps, offset=args.warmup)
    res["gathered_bytes"] = args.steps * B * Hkv * k * ROW_BYTES_BF16
    res["step_bytes"] = [B * Hkv * k * ROW_BYTES_BF16] * args.steps
    res["queries"] = B * args.steps
    m = misses.cpu()
    res["misses_per_step"] = m.sum(dim=1).tolist()
    res["miss_rate_steady"] = float(m[args.warmup:].double().mean() / k)
    fetched = m[args.warmup:].double().sum(dim=1) * Hkv * d * 2 * 2  # K and V rows per miss
    res["fetched_bytes"] = float(fetched.sum())
    res["counter_bytes"] = {"resolve": [float(x) for x in fetched]}
    r_ms = [rev[i][0].elapsed_time(rev[i][1]) for i in range(args.warmup, steps)]
    # steady state: steps after the first (step 0 misses every slot)
    first = 1 if args.warmup == 0 else 0
    steady_bytes = float(fetched[first:].sum())
    steady_ms = sum(r_ms[first:])
    h2d = measure_h2d_gbps(torch)
    fetch_gbps = steady_bytes / (steady_ms / 1e3) / 1e9 if steady_ms > 0 else None
    res["resolve"] = {
        "policy": args.policy,
        "mean_us": round(sum(r_ms) / len(r_ms) * 1e3, 2),
        "steady_mean_us": round(steady_ms / max(len(r_ms) - first, 1) * 1e3, 2),
        "fetch_gbps": round(fetch_gbps, 2) if fetch_gbps else None,
        "bound": "host link",
        "h2d_copy_gbps_measured": round(h2d, 2),
        "frac_of_h2d": round(fetch_gbps / h2d, 4) if fetch_gbps else None,
        "timing": "torch events around each resolve launch on the call's stream",
    }
    if args.cpu_seconds > 0:
        res["cpu_sample"] = ("cache",) + cpu_sample_cache(cfg, hk.tensor, hv.tensor, q, trace, min(steps, 64), torch)
    return res


def bound_steps(args, decode, n_distinct):
    """The step function of a decode workload: decode(i) runs step i, whose
    inputs repeat with period n_distinct. Eager runs bind each distinct
    step's call once (the binding checks and marshals its arguments then) and
    issue it per step as one foreign call, as a serving loop calling the C
    ABI would; every kernel still runs each step. Graph capture records the
    plain call on the capturing stream."""
    if args.graph:
        return decode
    bound = [decode(j, bind=True) for j in range(n_distinct)]
    return lambda i: bound[i % n_distinct]()


def _timed(args, call, torch, tsa, n_distinct, offset=0, kernels=("gather",)):
    """Warm up, then time args.steps steps (step i runs call(i + offset)).

    Eager (default): every step launches directly; on every event-stride-th
    step the library records HIP events around the gather-attention kernel's
    launch on the call's stream, so that kernel is timed inside the timed
    region. Other kernels in `kernels` (the token indexer scan) are timed the
    same way in an eager pass over the same steps after the timed region:
    event records placed inside the indexer's launch sequence were measured
    to slow the whole timed region of the token workload (0.20-0.35 ms per
    step against 0.128 ms without them). With --graph each distinct step
    (i mod n_distinct) is captured once into a HIP graph and the timed loop
    replays the graphs; event records captured in a graph do not bracket the
    kernels, so every kernel is then timed in the eager pass.
    """
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    which = {"gather": tsa.binding.TIMED_GATHER, "token_scan": tsa.binding.TIMED_TOKEN_SCAN}

    def new_events(names):
        return {kn: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for kn in names}

    def eager(i, ev):
        for kn, (a, b) in ev.items():
            tsa.time_next_launch(which[kn], a, b)
        call(i + offset)

    graphs = []
    if args.graph:
        n = min(n_distinct, args.steps)
        for j in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                call(j + offset)
            graphs.append(g)
        torch.cuda.synchronize()
    inner = [] if graphs else [kn for kn in kernels if kn == "gather"]
    post = [kn for kn in kernels if kn not in inner]
    evs = [new_events(inner) for _ in range(args.steps)]
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    stride = max(1, args.event_stride)
    timed = []
    for i in range(args.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        elif i % stride == 0:
            eager(i, evs[i])
            timed.append(i)
        else:
            call(i + offset)
    t_stop.record()
    torch.cuda.synchronize()
    res = {"ms_total": t_start.elapsed_time(t_stop), "wall_s": time.perf_counter() - wall0}
    if graphs:
        timed = list(range(min(args.steps, n_distinct)))
    kernel_ms = {kn: [evs[i][kn][0].elapsed_time(evs[i][kn][1]) for i in timed] for kn in inner}
    timing = {kn: f"HIP events recorded by the library around the kernel's launch on every {stride}-th step "
                  "inside the timed region" for kn in inner}
    if post:
        pev = {i: new_events(post) for i in timed}
        for i in timed:
            eager(i, pev[i])
        torch.cuda.synchronize()
        for kn in post:
            kernel_ms[kn] = [pev[i][kn][0].elapsed_time(pev[i][kn][1]) for i in timed]
            timing[kn] = ("HIP events recorded by the library around each launch in an eager pass over the same "
                          "steps after the timed region")
    res["kernel_ms"] = kernel_ms
    res["kernel_timing"] = timing
    res["gather_ms"] = kernel_ms["gather"]
    res["timed_steps"] = timed
    return res


def measure_stream_read_gbps(torch, tsa, nbytes=8 << 30):
    """Measured HBM read ceiling: the library's streaming-read probe (16-byte
    non-temporal loads over every CU) over an 8 GiB buffer, best of 5."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = tsa.stream_read(buf)
    torch.cuda.synchronize()
    best = None
    for _ in range(5):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        tsa.stream_read(buf, sink)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e)
        best = ms if best is None else min(best, ms)
    del buf
    torch.cuda.empty_cache()
    return nbytes / (best / 1e3) / 1e9


# ----------------------------------------------------------------------------

def measure_h2d_gbps(torch, nbytes=512 << 20):
    """Pinned host -> HBM copy rate (DMA), the host-link reference for RESOLVE."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dv = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dv.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(4):
        dv.copy_(h, non_blocking=True)
    e.record()
    torch.cuda.synchronize()
    return 4 * nbytes / (s.elapsed_time(e) / 1e3) / 1e9


def measure_copy_gbps(torch, nbytes=1 << 30):
    """Device-to-device copy rate (bytes read + written per second): a
    measured streaming ceiling to set beside the nominal HBM peak."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(4):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    rate = 4 * 2 * nbytes / (s.elapsed_time(e) / 1e3) / 1e9
    del a, b
    return rate


def calibrate_copy(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "gbps_read_plus_write": 2 * n / ms / 1e6}))


def _mean(xs):
    xs = list(xs)
    return sum(xs) / len(xs)


def kernel_rooflines(res, cfg, args, workload):
    """Per timed kernel: algorithmic bytes per launch (of exactly the launches
    that were timed) over the mean event-timed launch duration."""
    out = {}
    for kn, ms in res["kernel_ms"].items():
        step_bytes = res.get("gather_launch_bytes", res["step_bytes"]) if kn == "gather" else \
            res["kernel_step_bytes"][kn]
        name = gather_kernel_name(cfg, args) if kn == "gather" else KERNEL_NAMES[kn]
        bpl = _mean(step_bytes[i] for i in res["timed_steps"])
        mean_ms = _mean(ms)
        achieved = bpl / (mean_ms / 1e3) / 1e9
        traffic = measured_traffic(workload, name)
        out[name] = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "traffic_over_algorithmic": round(traffic / bpl, 4) if traffic else None,
                     "algorithmic_bytes_per_launch": round(bpl), "mean_launch_us": round(mean_ms * 1e3, 2),
                     "launches_timed": len(ms), "timing": res["kernel_timing"][kn]}
    return out


def counter_kernels(res, cfg, args):
    """Mean algorithmic bytes per launch over every timed step, for each kernel
    a counter pass attributes bytes to (with --warmup 0 these are all of the
    run's launches of that kernel)."""
    out = {gather_kernel_name(cfg, args): _mean(res.get("gather_launch_bytes", res["step_bytes"]))}
    for kn, sb in res.get("kernel_step_bytes", {}).items():
        out[KERNEL_NAMES[kn]] = _mean(sb)
    for kn, sb in res.get("counter_bytes", {}).items():
        out[KERNEL_NAMES[kn]] = _mean(sb)
    return out


def _counter_kib(csv_path, kernel):
    """Mean Counter_Value (KiB) per dispatch of `kernel` in a rocprofv3 counter
    collection CSV, and the number of dispatches."""
    import csv
    import re
    pat = re.compile(rf"(^|[^A-Za-z0-9_]){re.escape(kernel)}([^A-Za-z0-9_]|$)")
    vals = []
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if pat.search(row["Kernel_Name"]):
                vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"bench: no dispatch of {kernel} in {csv_path}")
    return sum(vals) / len(vals), len(vals)


def record_traffic(args):
    """Builds HBM bytes per launch of this workload's kernels from four
    rocprofv3 counter passes under DIR and merges them into the committed
    traffic record:

        DIR/c<N>_FETCH_SIZE/, DIR/c<N>_WRITE_SIZE/   bench.py --config N --steps K --warmup 0 --cpu-seconds 0
                                                      under rocprofv3 --pmc FETCH_SIZE (WRITE_SIZE)
        DIR/copy_FETCH_SIZE/, DIR/copy_WRITE_SIZE/   bench.py --calibrate-copy under the same passes
        DIR/c<N>_FETCH_SIZE.log                      the bench run's stdout (its JSON line)

    each pass written with `--output-format csv -o run`. The counters of a
    plain 1 GiB copy (1 GiB read, 1 GiB written) give the scale from counter
    units to bytes."""
    d, n = args.record_traffic, args.config
    with open(os.path.join(d, f"c{n}_FETCH_SIZE.log")) as f:
        line = json.loads([ln for ln in f if ln.startswith("{")][-1])
    if line["warmup"] != 0:
        raise SystemExit("bench: counter passes must run with --warmup 0 (every dispatch a timed step)")
    csv_of = {c: os.path.join(d, f"c{n}_{c}", "run_counter_collection.csv") for c in ("FETCH_SIZE", "WRITE_SIZE")}
    copy_kib = {c: _counter_kib(os.path.join(d, f"copy_{c}", "run_counter_collection.csv"),
                                "__amd_rocclr_copyBuffer")[0] for c in ("FETCH_SIZE", "WRITE_SIZE")}
    scale = {c: (1 << 30) / (copy_kib[c] * 1024) for c in copy_kib}
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    workload = line["config"]["workload"]
    # the workload's entries taken on another source no longer describe it
    rec = {key: v for key, v in rec.items()
           if key.split("/")[0] != workload or v.get("kernel_source_sha") == line["kernel_source_sha"]}
    bench_cmd = f"python -u bench.py --config {n} --steps {line['steps']} --warmup 0 --cpu-seconds 0"
    for kernel, alg in line["counter_kernels"].items():
        fetch, nf = _counter_kib(csv_of["FETCH_SIZE"], kernel)
        write, nw = _counter_kib(csv_of["WRITE_SIZE"], kernel)
        hbm = fetch * 1024 * scale["FETCH_SIZE"] + write * 1024 * scale["WRITE_SIZE"]
        rec[f"{workload}/{kernel}"] = {
            "kernel_source_sha": line["kernel_source_sha"],
            "dispatches": [nf, nw],
            "fetch_size_kib_per_dispatch": round(fetch, 1), "write_size_kib_per_dispatch": round(write, 1),
            "fetch_scale_from_copy": round(scale["FETCH_SIZE"], 5),
            "write_scale_from_copy": round(scale["WRITE_SIZE"], 5),
            "hbm_bytes_per_launch": round(hbm), "algorithmic_bytes_per_launch": round(alg),
            "traffic_over_algorithmic": round(hbm / alg, 4) if alg else None,
            "commands": [f"rocprofv3 --pmc {c} --output-format csv -d {d}/c{n}_{c} -o run -- {bench_cmd}"
                         for c in ("FETCH_SIZE", "WRITE_SIZE")] +
                        [f"rocprofv3 --pmc {c} --output-format csv -d {d}/copy_{c} -o run -- "
                         "python -u bench.py --calibrate-copy" for c in ("FETCH_SIZE", "WRITE_SIZE")],
        }
        log(f"{workload}/{kernel}: {hbm / 1e6:.1f} MB per launch, {hbm / alg:.3f}x algorithmic")
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")


def workload_name(cfg, args):
    workload = cfg.name + (f"+grow-from-{args.grow}" if args.grow else "")
    if cfg.kind == "ivf":
        if args.grow and args.slack >= 0:
            workload += f"+slack{args.slack}"
        if args.similarity != "dot":
            workload += f"+{args.similarity}"
        if args.sink or args.window:
            workload += f"+sink{args.sink}+window{args.window}"
        if args.assign > 1:
            workload += f"+{args.assign}-lists-per-key"
        if args.schedule != "auto":
            workload += f"+{args.schedule}"
        if args.kv_layout != "token":
            workload += "+list-major-kv"
    if cfg.kind == "cache" and (cfg.popularity_sd or cfg.recency):
        workload += f"+popularity{cfg.popularity_sd:g}+recency{cfg.recency:g}"
    if cfg.kind == "cache" and args.policy != "lru":
        workload += f"+{args.policy}"
    if cfg.kind == "cache" and args.layers > 1:
        workload = f"hier-cache-{max(1, cfg.batch // args.layers)}x128k-{args.layers}layers"
    return workload


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported by this build "
              "(across GPUs the decode path would shard by request, one batch slice per GPU)", file=sys.stderr)
        sys.exit(2)
    if args.record_traffic:
        record_traffic(args)
        return
    if args.cpu_seconds > 0 and not args.calibrate_copy and not args.gpu_phase:
        # the GPU run in a child process; this process, which never touches
        # the GPU, then times the oracle on the sample the child wrote
        import subprocess
        import tempfile
        fd, path = tempfile.mkstemp(prefix="tsa_bench_", suffix=".json", dir="/tmp")
        os.close(fd)
        try:
            rc = subprocess.run([sys.executable, os.path.abspath(__file__), *sys.argv[1:], "--gpu-phase", path]).returncode
            if rc != 0:
                sys.exit(rc)
            with open(path) as f:
                line = json.load(f)
        finally:
            os.unlink(path)
        sample = line.pop("cpu_sample", None)
        if sample:
            kind_s, data_dir, what = sample
            log(f"oracle baseline: {what}")
            pool = start_cpu_pool(host_cores())
            try:
                line["cpu_baseline"] = cpu_baseline(args, kind_s, data_dir, what, pool)
            finally:
                pool.terminate()
        print(json.dumps(line), flush=True)
        return
    import torch

    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    line = gpu_run(args, torch)
    if args.gpu_phase:
        with open(args.gpu_phase, "w") as f:
            json.dump(line, f)
    else:
        line.pop("cpu_sample", None)
        print(json.dumps(line), flush=True)


def gpu_run(args, torch):
    import top_sparse_attention_centroid_amd as tsa
    from top_sparse_attention_centroid_amd import workloads as W

    tsa.load()
    cfg = W.config(args.config)
    if args.popularity or args.recency:
        if cfg.kind != "cache":
            sys.exit("bench: --popularity / --recency shape the hot-cache workload's selection trace")
        cfg = cfg.replace(popularity_sd=args.popularity, recency=args.recency)
    kind = {"ivf": bench_ivf, "token": bench_token, "cache": bench_cache}[cfg.kind]
    res = kind(args, cfg, torch, tsa, W)

    K = args.steps
    ms_step = res["ms_total"] / K
    value = res["queries"] / (res["ms_total"] / 1e3)
    gb_s = res["gathered_bytes"] / (res["ms_total"] / 1e3) / 1e9
    workload = workload_name(cfg, args)
    kernels = kernel_rooflines(res, cfg, args, workload)
    dominant = max(kernels.values(), key=lambda r: r["mean_launch_us"])
    read_gbps = measure_stream_read_gbps(torch, tsa)
    copy_gbps = measure_copy_gbps(torch)
    for r in kernels.values():
        r["measured_read_ceiling_gbps"] = round(read_gbps, 1)
        r["frac_of_measured_read_ceiling"] = round(r["achieved"] / read_gbps, 4)
    roofline = dict(dominant)
    roofline["torch_d2d_copy_gbps"] = round(copy_gbps, 1)
    roofline["read_ceiling"] = ("the library's streaming-read probe: 16-byte non-temporal loads over every CU, "
                                "one pass over an 8 GiB buffer, best of 5")
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload, "batch": res.get("batch", cfg.batch), "context": cfg.n_tokens,
                   "kv_heads": cfg.n_kv_heads, "q_heads": cfg.n_q_heads, "head_dim": cfg.head_dim,
                   "top_k": cfg.top_k, "centroids": cfg.n_centroids or None,
                   "slots": cfg.n_slots or None, "parallelism": "none (1 GPU)",
                   "kv_layout": ("list-major copies" if args.kv_layout == "lists" else "token-major caches")
                   if cfg.kind == "ivf" else None},
        "gathered_kv_gbps": round(gb_s, 1),
        "gathered_kv_frac_of_peak": round(gb_s / HBM_PEAK_GBPS, 4),
        "graph": bool(args.graph),
        "roofline": roofline,
        "other_kernels": [r for r in kernels.values() if r is not dominant],
        "cpu_baseline": None,
        "kernel_source_sha": kernel_source_sha(),
        "counter_kernels": counter_kernels(res, cfg, args),
    }
    for key in ("index_build_ms", "kv_lists_build_ms", "unique_rows_per_step", "misses_per_step", "miss_rate_steady",
                "fetched_bytes", "resolve", "append", "regrow", "layer_group", "indexer_bytes_per_step"):
        if key in res:
            line[key] = res[key]
    if "cpu_sample" in res:
        line["cpu_sample"] = list(res["cpu_sample"])
    return line


if __name__ == "__main__":
    main()
