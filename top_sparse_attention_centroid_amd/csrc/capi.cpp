// C-ABI layer of libtsa: argument validation, workspace layout, launch
// sequencing and error reporting. Every check runs on the host before the
// first launch, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <random>
#include <mutex>
#include <string>

#include "kernels.hpp"
#include "tsa.h"

using namespace tsa;

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_gather_evs[2] = {nullptr, nullptr};   // gather (tsa_time_next_launch)
thread_local hipEvent_t g_scan_ev0 = nullptr;   // token indexer scan (tsa_time_next_launch)
thread_local hipEvent_t g_scan_ev1 = nullptr;
thread_local hipEvent_t g_append_evs[2] = {nullptr, nullptr};   // kv_append (tsa_time_next_launch)
thread_local hipEvent_t g_regrow_evs[2] = {nullptr, nullptr};   // regrow (tsa_time_next_launch)

// Records the one-shot event pair `ev` (if set) around one launch on s.
template <typename Launch>
hipError_t launch_between(hipEvent_t (&ev)[2], hipStream_t s, Launch&& launch) {
  hipEvent_t e0 = ev[0], e1 = ev[1];
  ev[0] = ev[1] = nullptr;
  hipError_t e;
  if (e0 && (e = hipEventRecord(e0, s)) != hipSuccess) return e;
  if ((e = launch()) != hipSuccess) return e;
  if (e1 && (e = hipEventRecord(e1, s)) != hipSuccess) return e;
  return hipSuccess;
}

tsa_status fail(tsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

tsa_status ok() {
  g_last_error.clear();
  return TSA_OK;
}

tsa_status hip_fail(hipError_t e, const char* where) {
  return fail(TSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

bool valid_group(int Hq, int Hkv) {
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

float qscale(int d) { return static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d))); }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Workgroups per (request, KV head) for gather_attn: one wave per expected
// segment; short-lived workgroups let the dispatcher balance uneven segments.
int gather_blocks_per_head(int expected_segments, bool explicit_plan) {
  const int waves = explicit_plan ? kGatherWavesExplicit : kGatherWavesRows;
  return std::max(1, ceil_div(expected_segments, waves * kGatherSegsPerWave));
}

// Rows per attention segment for per-request row lists: the longest of
// 256 / 128 / 64 rows that still gives at least 2048 segments (8 waves per
// CU). Longer segments write fewer partial softmax states; shorter ones keep
// every CU busy when the batch is small.
constexpr long long kMinRowSegments = 2048;
int row_seg_rows(long long pairs, int max_rows) {
  for (int r = kSegRows; r > kRowSegRows; r >>= 1)
    if (pairs * ceil_div(max_rows, r) >= kMinRowSegments) return r;
  return kRowSegRows;
}

// Fetch of a miss list for `layers` layers. Host reads have long latency and
// clog the memory pipeline of the CUs that issue them, so the fetch is kept
// on a few CUs: about kFetchWorkgroups large workgroups in all, which still
// keep the host link busy, and leave the other CUs to attention running
// beside it.
constexpr long long kFetchWorkgroups = 64;
FetchParams fetch_params(const tsa_cache_desc& d, const int32_t* miss_tok, const int32_t* miss_slot,
                         const int32_t* misses, int k, int layers) {
  FetchParams fp{};
  fp.miss_tok = miss_tok; fp.miss_slot = miss_slot; fp.misses = misses;
  fp.n_layers = layers;
  const long long units = static_cast<long long>(d.batch) * std::max(layers, 1);
  fp.split = static_cast<int>(std::min<long long>(32, std::max<long long>(1, kFetchWorkgroups / units)));
  fp.row_bytes = static_cast<long long>(d.n_kv_heads) * d.head_dim * esize(d.dtype);
  fp.B = d.batch; fp.N = d.n_tokens; fp.S = d.n_slots; fp.k = k;
  return fp;
}

// ----------------------------------------------------------------- layouts
struct IvfLayout {
  int G = 0, smax = 0, seg_rows = 0;
  bool small_batch = false, split_score = false, merge = false;
  size_t seg = 0, nseg = 0, partial = 0, lmask = 0, keys = 0, arrive = 0, total = 0;
};

// A batch with fewer (request, KV head) groups than this is small: its decode
// is bound by the latency of a few workgroups rather than by bandwidth. Then
// centroid scoring runs as its own launch (one wave per 16 centroids; bf16
// data), since one select workgroup per group would read the whole codebook
// through a few CUs; and list segments that several heads chose get one
// cacheable pass per head instead of one all-heads pass.
constexpr long long kSmallBatchGroups = 128;

// Plan segments expected for one chosen list with `rows`-row segments: its
// average length N * m / C in segments, rounded, plus room for a ragged tail.
int ivf_list_segs(const tsa_ivf_desc& d, int m, int rows) {
  const long long avg_list = static_cast<long long>(d.n_tokens) * m / d.n_centroids;
  return std::max(1, static_cast<int>((2LL * avg_list + rows) / (2 * rows)) + (avg_list > rows / 2 ? 1 : 0));
}

// Rows per plan segment of an inverted-index decode: the longest of 256,
// 128, 64, 32 rows for which the batch still expects kMinIvfSegments
// segments (one wave each, 8 per CU). Large batches keep 256-row segments
// and write the fewest partial states; a single request cuts its lists finer
// so that enough waves stream rows at once. A segment count bound per
// (request, KV head) keeps the worst-case workspace of long contexts in check.
constexpr long long kMinIvfSegments = 2048;
constexpr int kIvfMinSegRows = 32;
constexpr long long kIvfMaxPlanSegs = 16384;
int ivf_seg_rows(const tsa_ivf_desc& d, int k, int m) {
  const long long bh = static_cast<long long>(d.batch) * d.n_kv_heads;
  const long long gk = static_cast<long long>(d.n_q_heads / d.n_kv_heads) * k;
  const long long entries = static_cast<long long>(d.n_tokens) * m;
  int r = kSegRows;
  while (r > kIvfMinSegRows && bh * gk * ivf_list_segs(d, m, r) < kMinIvfSegments &&
         (entries + r / 2 - 1) / (r / 2) <= kIvfMaxPlanSegs)
    r >>= 1;
  return r;
}

// with_fixed: room for the sink / window segments of tsa_sparse_decode_ex;
// m: lists per token (2: twice the list entries and the chosen-list masks)
IvfLayout ivf_layout(const tsa_ivf_desc& d, int k, bool with_fixed = false, int m = 1) {
  IvfLayout L;
  L.G = d.n_q_heads / d.n_kv_heads;
  L.seg_rows = ivf_seg_rows(d, k, m);
  const size_t bh = static_cast<size_t>(d.batch) * d.n_kv_heads;
  L.small_batch = static_cast<long long>(bh) < kSmallBatchGroups;
  // Large bf16 batches (bound by HBM) with up to 4 query heads per KV head
  // gather in merged sets of kMergeWaves segments; small ones, bound by the
  // latency of their waves, keep a wave per segment, and so do fp32 and
  // wider groups.
  L.merge = !L.small_batch && d.dtype == TSA_BF16 && L.G <= 4;
  L.smax = L.G * k + ceil_div(static_cast<long long>(d.n_tokens) * m, L.seg_rows) +
           (with_fixed ? kMaxFixedRows / L.seg_rows + 2 : 0);
  size_t off = 0;
  L.seg = off;    off += align_up(bh * L.smax * sizeof(int4));
  L.nseg = off;   off += align_up(bh * sizeof(int32_t));
  L.partial = off; off += align_up(bh * L.smax * L.G * kPartStride * sizeof(float));
  L.lmask = off;   off += m > 1 ? align_up(bh * d.n_centroids * sizeof(uint32_t)) : 0;
  // the scores of a separate scoring launch: the staged path's small bf16
  // batches and every split decode (any bf16 batch may ask for one)
  L.split_score = d.dtype == TSA_BF16 && L.small_batch;
  L.keys = off;    off += d.dtype == TSA_BF16 ? align_up(bh * L.G * d.n_centroids * sizeof(uint32_t)) : 0;
  // arrival counters of the split decode (bf16), one per query head
  L.arrive = off;  off += d.dtype == TSA_BF16 ? align_up(bh * L.G * sizeof(uint32_t)) : 0;
  L.total = off;
  return L;
}

struct TokLayout {
  int G = 0, smax = 0, seg_rows = 0, nfchunk = 0;
  size_t keys = 0, hist = 0, cand_key = 0, cand_id = 0, cand_cnt = 0, sel = 0, partial = 0, epoch = 0,
         ready = 0, grab = 0, total = 0;
};

TokLayout tok_layout(const tsa_token_desc& d, int k) {
  TokLayout L;
  L.G = d.n_q_heads / d.n_kv_heads;
  L.seg_rows = row_seg_rows(static_cast<long long>(d.batch) * d.n_kv_heads, k);
  L.smax = ceil_div(k, L.seg_rows);
  L.nfchunk = ceil_div(d.n_tokens, kTokFilterTile);
  const size_t bn = static_cast<size_t>(d.batch) * d.n_tokens;
  size_t off = 0;
  L.keys = off;     off += align_up(bn * sizeof(uint32_t));
  L.hist = off;     off += align_up(static_cast<size_t>(d.batch) * kTokHistBins * sizeof(int32_t));
  L.cand_key = off; off += align_up(bn * sizeof(uint32_t));
  L.cand_id = off;  off += align_up(bn * sizeof(int32_t));
  L.cand_cnt = off; off += align_up(static_cast<size_t>(d.batch) * L.nfchunk * sizeof(int32_t));
  L.sel = off;      off += align_up(static_cast<size_t>(d.batch) * k * sizeof(int32_t));
  L.partial = off;
  off += align_up(static_cast<size_t>(d.batch) * d.n_kv_heads * L.smax * L.G * kPartStride * sizeof(float));
  // the scan's histogram-clear handshake: the workspace's epoch and one
  // ready tag per request; the scan's per-request chunk counters
  L.epoch = off;    off += align_up(sizeof(uint64_t));
  L.ready = off;    off += align_up(static_cast<size_t>(d.batch) * sizeof(uint64_t));
  L.grab = off;     off += align_up(static_cast<size_t>(d.batch) * sizeof(int32_t));
  L.total = off;
  return L;
}

// Per-call nonces of the token decode's histogram-clear tag: a process-wide
// counter from a seed drawn once, so that calls of different processes on
// one workspace, and a call after a failed one, get different tags too.
uint64_t next_token_nonce() {
  static std::atomic<uint64_t> counter{[] {
    std::random_device rd;
    const uint64_t t = static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count());
    return (static_cast<uint64_t>(rd()) << 32) ^ rd() ^ (t * 0x9E3779B97F4A7C15ull);
  }()};
  return counter.fetch_add(1, std::memory_order_relaxed);
}

struct RowsLayout {
  int G = 0, smax = 0, seg_rows = 0;
  size_t partial = 0, total = 0;
};

RowsLayout rows_layout(const tsa_attn_desc& d) {
  RowsLayout L;
  L.G = d.n_q_heads / d.n_kv_heads;
  L.seg_rows = row_seg_rows(static_cast<long long>(d.batch) * d.n_kv_heads, std::max(1, d.max_rows));
  L.smax = std::max(1, ceil_div(d.max_rows, L.seg_rows));
  L.total = align_up(static_cast<size_t>(d.batch) * d.n_kv_heads * L.smax * L.G * kPartStride * sizeof(float));
  return L;
}

size_t index_assign_bytes(const tsa_ivf_desc& d, int m = 1) {
  return align_up(static_cast<size_t>(d.batch) * d.n_kv_heads * d.n_tokens * m * sizeof(int32_t));
}
size_t index_ws(const tsa_ivf_desc& d, int m = 1) {
  const size_t bc = d.shared_codebook ? 1 : static_cast<size_t>(d.batch);
  return index_assign_bytes(d, m) + align_up(bc * d.n_kv_heads * d.n_centroids * sizeof(float));
}

// ------------------------------------------------------------- validation
tsa_status check_dtype(int dtype) {
  if (dtype != TSA_F32 && dtype != TSA_BF16) return fail(TSA_ERR_UNSUPPORTED, "dtype %d is not TSA_F32 or TSA_BF16", dtype);
  return TSA_OK;
}

tsa_status check_ivf(const tsa_ivf_desc* d) {
  if (!d) return fail(TSA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch <= 0 || d->n_tokens <= 0 || d->n_kv_heads <= 0 || d->n_q_heads <= 0 ||
      d->head_dim <= 0 || d->n_centroids <= 0)
    return fail(TSA_ERR_INVALID_ARG, "non-positive size in tsa_ivf_desc");
  if (d->head_dim != kHeadDimRows) return fail(TSA_ERR_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (!valid_group(d->n_q_heads, d->n_kv_heads))
    return fail(TSA_ERR_UNSUPPORTED, "n_q_heads/n_kv_heads = %d/%d is not 1, 2, 4 or 8", d->n_q_heads, d->n_kv_heads);
  const int G = d->n_q_heads / d->n_kv_heads;
  if (d->n_centroids > kMaxCentroids || static_cast<long long>(d->n_centroids) * (G + 2) + 1 > 16384)
    return fail(TSA_ERR_UNSUPPORTED, "n_centroids %d too large for group %d", d->n_centroids, G);
  if (d->shared_codebook != 0 && d->shared_codebook != 1)
    return fail(TSA_ERR_INVALID_ARG, "shared_codebook must be 0 or 1");
  return check_dtype(d->dtype);
}

// lists per key of a multi-way index
tsa_status check_m(const tsa_ivf_desc* d, int m) {
  if (m < 1 || m > kMaxAssign) return fail(TSA_ERR_UNSUPPORTED, "m=%d: 1 to %d lists per key", m, kMaxAssign);
  if (m > d->n_centroids) return fail(TSA_ERR_INVALID_ARG, "m=%d > C=%d", m, d->n_centroids);
  if (static_cast<long long>(d->n_tokens) * m > INT32_MAX) return fail(TSA_ERR_UNSUPPORTED, "N * m exceeds int32");
  return TSA_OK;
}

tsa_status check_token(const tsa_token_desc* d, int k) {
  if (!d) return fail(TSA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch <= 0 || d->n_tokens <= 0 || d->n_kv_heads <= 0 || d->n_q_heads <= 0 ||
      d->head_dim <= 0 || d->idx_dim <= 0)
    return fail(TSA_ERR_INVALID_ARG, "non-positive size in tsa_token_desc");
  if (d->head_dim != kHeadDimRows) return fail(TSA_ERR_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (d->idx_dim != 64) return fail(TSA_ERR_UNSUPPORTED, "idx_dim %d != 64", d->idx_dim);
  if (!valid_group(d->n_q_heads, d->n_kv_heads))
    return fail(TSA_ERR_UNSUPPORTED, "n_q_heads/n_kv_heads = %d/%d is not 1, 2, 4 or 8", d->n_q_heads, d->n_kv_heads);
  if (k < 1 || k > d->n_tokens) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, N=%d]", k, d->n_tokens);
  if (k > kMaxTokenK) return fail(TSA_ERR_UNSUPPORTED, "k=%d > %d", k, kMaxTokenK);
  if (ceil_div(d->n_tokens, kTokFilterTile) > kMaxTokFilterChunks)
    return fail(TSA_ERR_UNSUPPORTED, "N=%d > %d tokens", d->n_tokens, kTokFilterTile * kMaxTokFilterChunks);
  return check_dtype(d->dtype);
}

tsa_status check_attn(const tsa_attn_desc* d) {
  if (!d) return fail(TSA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch <= 0 || d->n_rows <= 0 || d->n_kv_heads <= 0 || d->n_q_heads <= 0 ||
      d->head_dim <= 0 || d->max_rows < 0)
    return fail(TSA_ERR_INVALID_ARG, "bad size in tsa_attn_desc");
  if (d->head_dim != kHeadDimRows) return fail(TSA_ERR_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (!valid_group(d->n_q_heads, d->n_kv_heads))
    return fail(TSA_ERR_UNSUPPORTED, "n_q_heads/n_kv_heads = %d/%d is not 1, 2, 4 or 8", d->n_q_heads, d->n_kv_heads);
  return check_dtype(d->dtype);
}

tsa_status check_cache(const tsa_cache_desc* d) {
  if (!d) return fail(TSA_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch <= 0 || d->n_tokens <= 0 || d->n_slots <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0)
    return fail(TSA_ERR_INVALID_ARG, "non-positive size in tsa_cache_desc");
  if (d->head_dim != kHeadDimRows) return fail(TSA_ERR_UNSUPPORTED, "head_dim %d != 128", d->head_dim);
  if (d->n_slots > kMaxSlots) return fail(TSA_ERR_UNSUPPORTED, "n_slots %d > %d", d->n_slots, kMaxSlots);
  return check_dtype(d->dtype);
}

#define REQUIRE_PTR(p)                                                     \
  do {                                                                     \
    if (!(p)) return fail(TSA_ERR_INVALID_ARG, "%s is NULL", #p);           \
  } while (0)

#define REQUIRE_ALIGN(p, a)                                                \
  do {                                                                     \
    if ((p) && !aligned((p), (a)))                                         \
      return fail(TSA_ERR_INVALID_ARG, "%s is not %d-byte aligned", #p, (int)(a)); \
  } while (0)

tsa_status launch_gather_timed(const GatherParams& gp, int dtype, int G, bool explicit_plan,
                               hipStream_t s) {
  hipError_t e = launch_between(g_gather_evs, s, [&] { return launch_gather(gp, dtype, G, explicit_plan, s); });
  if (e != hipSuccess) return hip_fail(e, "gather_attn launch");
  e = launch_combine(gp, G, explicit_plan, s);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return TSA_OK;
}

}  // namespace

namespace {

long long codebook_stride(const tsa_ivf_desc& d) {
  return d.shared_codebook ? 0LL : static_cast<long long>(d.n_kv_heads) * d.n_centroids * kHeadDimRows;
}

tsa_status index_build_impl(const tsa_ivf_desc* desc, const void* keys, const void* centroids, int n_prefix,
                            int slack, int32_t* offsets, int32_t* lens, int32_t* ids, void* ws, size_t ws_bytes,
                            void* stream, int m = 1, int32_t* alt = nullptr) {
  REQUIRE_PTR(keys); REQUIRE_PTR(centroids); REQUIRE_PTR(offsets); REQUIRE_PTR(ids); REQUIRE_PTR(ws);
  REQUIRE_ALIGN(keys, 16); REQUIRE_ALIGN(centroids, 16); REQUIRE_ALIGN(ws, 16);
  const size_t need = index_ws(*desc, m);
  if (ws_bytes < need) return fail(TSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  const tsa_ivf_desc& d = *desc;
  hipStream_t s = as_stream(stream);
  AssignParams ap{keys, centroids, codebook_stride(d), static_cast<int32_t*>(ws),
                  d.batch, d.n_tokens, d.n_kv_heads, d.n_centroids, n_prefix, m};
  hipError_t e =
      launch_assign(ap, d.dtype, reinterpret_cast<float*>(static_cast<char*>(ws) + index_assign_bytes(d, m)), s);
  if (e != hipSuccess) return hip_fail(e, "assign launch");
  CsrParams cp{static_cast<const int32_t*>(ws), offsets, ids, lens, alt, d.batch, d.n_tokens, d.n_kv_heads,
               d.n_centroids, n_prefix, slack, m};
  e = launch_csr(cp, s);
  if (e != hipSuccess) return hip_fail(e, "csr launch");
  return ok();
}

// The per-head schedules (fused, split) take plain list decodes whose
// codebook and k fit one workgroup: one list per token, no sink or window
// rows, C <= kHeadMaxC, k <= kHeadMaxK.
bool head_qualifies(const tsa_ivf_desc& d, int k, const tsa_decode_opts* opts) {
  if (opts && (opts->assign_per_key > 1 || opts->n_sink > 0 || opts->n_window > 0)) return false;
  return d.n_centroids <= kHeadMaxC && k <= kHeadMaxK;
}

// AUTO takes the fused decode when every head's work fits one CU (a CU reads
// some 40 GB/s, so a head's rows and its group's codebook must be small):
// at most kFusedMaxHeads heads, about kFusedMaxRows rows a head and
// kFusedMaxCodebook bytes of codebook per KV head. Otherwise bf16 batches of
// fewer than kSmallBatchGroups groups take the split decode, which spreads
// the scoring and every head's rows over many CUs; the rest the staged path.
constexpr long long kFusedMaxHeads = 256;
constexpr long long kFusedMaxRows = 512;
constexpr long long kFusedMaxCodebook = 65536;  // 64 KiB

int resolve_schedule(const tsa_ivf_desc& d, int k, const tsa_decode_opts* opts) {
  const int sched = opts ? opts->schedule : TSA_SCHED_AUTO;
  if (sched != TSA_SCHED_AUTO) return sched;  // FUSED / SPLIT checked to qualify by the caller
  if (!head_qualifies(d, k, opts)) return TSA_SCHED_STAGED;
  const long long rows = static_cast<long long>(k) * d.n_tokens / d.n_centroids;
  const long long codebook = static_cast<long long>(d.n_centroids) * d.head_dim * esize(d.dtype);
  if (static_cast<long long>(d.batch) * d.n_q_heads <= kFusedMaxHeads && rows <= kFusedMaxRows &&
      codebook <= kFusedMaxCodebook)
    return TSA_SCHED_FUSED;
  if (d.dtype == TSA_BF16 && static_cast<long long>(d.batch) * d.n_kv_heads < kSmallBatchGroups)
    return TSA_SCHED_SPLIT;
  return TSA_SCHED_STAGED;
}

// Split decode: shares per query head so that each of a share's kSplitWaves
// waves attends about half a batch (16 rows) of an average head (k * N / C
// rows), at most kSplitMaxWorkgroups workgroups in all, and G * S partial
// records within the plan's smax per group. At one 100K-token request
// (1,000 rows a head, 8 shares) 8 waves of 16 rows beat 4 waves of 32
// (16.0 against 17.0 us for the kernel); 4 or 16 shares, and 4 or 16 waves,
// were slower.
constexpr long long kSplitRowsPerShare = kSplitWaves * 16;
constexpr long long kSplitMaxWorkgroups = 2048;
int split_shares(const tsa_ivf_desc& d, int k, const IvfLayout& L) {
  const long long rows = static_cast<long long>(k) * d.n_tokens / d.n_centroids;
  long long S = std::max(1LL, (rows + kSplitRowsPerShare - 1) / kSplitRowsPerShare);
  S = std::min(S, std::max(1LL, kSplitMaxWorkgroups / (static_cast<long long>(d.batch) * d.n_q_heads)));
  S = std::min(S, static_cast<long long>(L.smax / L.G));
  return static_cast<int>(std::max(1LL, S));
}

tsa_status sparse_decode_impl(const tsa_ivf_desc* desc, const tsa_decode_opts* opts, const void* q,
                              const void* centroids, const int32_t* offsets, const int32_t* lens,
                              const int32_t* ids, const void* k_cache, const void* v_cache, int32_t k, float* out,
                              int32_t* sel_out, int32_t* rows_out, int32_t* uniq_out, void* ws, size_t ws_bytes,
                              void* stream) {
  REQUIRE_PTR(q); REQUIRE_PTR(centroids); REQUIRE_PTR(offsets); REQUIRE_PTR(ids);
  REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache); REQUIRE_PTR(out); REQUIRE_PTR(ws);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(centroids, 16); REQUIRE_ALIGN(k_cache, 16);
  REQUIRE_ALIGN(v_cache, 16); REQUIRE_ALIGN(out, 8); REQUIRE_ALIGN(ws, 16);
  const tsa_ivf_desc& d = *desc;
  if (k < 1 || k > d.n_centroids) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, C=%d]", k, d.n_centroids);
  const int m = opts && opts->assign_per_key > 1 ? opts->assign_per_key : 1;
  const IvfLayout L = ivf_layout(d, k, opts != nullptr, m);
  if (ws_bytes < L.total) return fail(TSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  hipStream_t s = as_stream(stream);

  SelectParams selp{q, centroids, codebook_stride(d), offsets, lens, sel_out, rows_out, uniq_out,
                    reinterpret_cast<int4*>(w + L.seg), reinterpret_cast<int32_t*>(w + L.nseg),
                    d.batch, d.n_kv_heads, d.n_centroids, k, L.smax, d.n_tokens};
  selp.n_entries = d.n_tokens * m;
  if (opts) {
    selp.cosine = opts->similarity == TSA_SIM_COSINE;
    selp.n_sink = opts->n_sink;
    selp.n_window = opts->n_window;
    selp.lengths = opts->lengths;
  }
  const int sched = resolve_schedule(d, k, opts);
  if (sched == TSA_SCHED_FUSED || sched == TSA_SCHED_SPLIT) {
    HeadDecodeParams hp{};
    hp.s = selp;
    hp.ids = ids; hp.k = k_cache; hp.v = v_cache; hp.out = out;
    if (opts) {
      hp.kl = opts->k_lists;
      hp.vl = opts->v_lists;
    }
    hp.qscale = qscale(d.head_dim);
    hp.Hq = d.n_q_heads;
    if (sched == TSA_SCHED_FUSED) {
      // the one kernel of the step answers the gather timing hook
      hipError_t e = launch_between(g_gather_evs, s, [&] { return launch_fused_decode(hp, d.dtype, L.G, s); });
      if (e != hipSuccess) return hip_fail(e, "fused decode launch");
      return ok();
    }
    hp.s.keys = reinterpret_cast<uint32_t*>(w + L.keys);
    hp.s.arrive_heads = reinterpret_cast<uint32_t*>(w + L.arrive);
    hp.partial = reinterpret_cast<float*>(w + L.partial);
    hp.S = split_shares(d, k, L);
    hipError_t e = launch_centroid_score(hp.s, L.G, s);
    if (e != hipSuccess) return hip_fail(e, "centroid_score launch");
    e = launch_between(g_gather_evs, s, [&] { return launch_split_decode(hp, L.G, s); });
    if (e != hipSuccess) return hip_fail(e, "split decode launch");
    return ok();
  }
  if (m > 1) selp.lmask_out = reinterpret_cast<uint32_t*>(w + L.lmask);
  selp.seg_rows = L.seg_rows;
  selp.class_order = L.merge ? 1 : 0;
  if (L.split_score) selp.keys = reinterpret_cast<uint32_t*>(w + L.keys);
  hipError_t e = launch_ivf_select(selp, d.dtype, L.G, s);
  if (e != hipSuccess) return hip_fail(e, "ivf_select launch");

  GatherParams gp{};
  gp.q = q; gp.k = k_cache; gp.v = v_cache; gp.n_rows = d.n_tokens;
  gp.rowids = ids; gp.rid_bstride = static_cast<long long>(d.n_kv_heads) * d.n_tokens * m;
  gp.rid_gstride = static_cast<long long>(d.n_tokens) * m;
  gp.seg = reinterpret_cast<const int4*>(w + L.seg); gp.nseg = reinterpret_cast<const int32_t*>(w + L.nseg);
  gp.counts = nullptr; gp.count_const = 0;
  gp.partial = reinterpret_cast<float*>(w + L.partial); gp.out = out;
  gp.B = d.batch; gp.Hkv = d.n_kv_heads; gp.smax = L.smax;
  // expected segments: those of every chosen list of the group, plus the
  // sink / window segments
  int fixed_segs = 0;
  if (opts) {
    fixed_segs = ceil_div(std::min(opts->n_sink, d.n_tokens), L.seg_rows) +
                 ceil_div(std::min(opts->n_window, d.n_tokens), L.seg_rows) + (opts->n_window > 0 ? 1 : 0);
  }
  const int expected_segs = std::min(L.smax, L.G * k * ivf_list_segs(d, m, L.seg_rows) + fixed_segs);
  gp.seg_rows = L.seg_rows;
  gp.multi_all = L.small_batch ? 0 : 1;
  gp.merge = L.merge ? 1 : 0;
  gp.W = L.merge ? std::max(1, ceil_div(expected_segs, kMergeWaves)) : gather_blocks_per_head(expected_segs, true);
  gp.qscale = qscale(d.head_dim);
  if (opts) {
    gp.n_sink = opts->n_sink;
    gp.n_window = opts->n_window;
    gp.lengths = opts->lengths;
    gp.kl = opts->k_lists;
    gp.vl = opts->v_lists;
  }
  if (m > 1) {
    gp.alt = opts->alt;
    gp.alt_w = m - 1;
    gp.lmask = reinterpret_cast<const uint32_t*>(w + L.lmask);
    gp.C = d.n_centroids;
  }
  if (tsa_status st = launch_gather_timed(gp, d.dtype, L.G, true, s)) return st;
  return ok();
}

}  // namespace

extern "C" {

int32_t tsa_abi_version(void) { return TSA_ABI_VERSION; }

const char* tsa_status_str(tsa_status s) {
  switch (s) {
    case TSA_OK: return "TSA_OK";
    case TSA_ERR_INVALID_ARG: return "TSA_ERR_INVALID_ARG";
    case TSA_ERR_UNSUPPORTED: return "TSA_ERR_UNSUPPORTED";
    case TSA_ERR_WORKSPACE: return "TSA_ERR_WORKSPACE";
    case TSA_ERR_HIP: return "TSA_ERR_HIP";
  }
  return "TSA_ERR_UNKNOWN";
}

const char* tsa_last_error(void) { return g_last_error.c_str(); }

tsa_status tsa_workspace_bytes_multi(int32_t op, const void* desc, int32_t k, int32_t m, size_t* bytes) {
  REQUIRE_PTR(bytes);
  REQUIRE_PTR(desc);
  if (op != TSA_OP_INDEX_BUILD_MULTI && op != TSA_OP_SPARSE_DECODE_EX_MULTI) return tsa_workspace_bytes(op, desc, k, bytes);
  const auto* d = static_cast<const tsa_ivf_desc*>(desc);
  if (tsa_status s = check_ivf(d)) return s;
  if (tsa_status s = check_m(d, m)) return s;
  if (op == TSA_OP_INDEX_BUILD_MULTI) {
    *bytes = index_ws(*d, m);
    return ok();
  }
  if (k < 1 || k > d->n_centroids) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, C=%d]", k, d->n_centroids);
  *bytes = ivf_layout(*d, k, true, m).total;
  return ok();
}

tsa_status tsa_workspace_bytes(int32_t op, const void* desc, int32_t k, size_t* bytes) {
  REQUIRE_PTR(bytes);
  REQUIRE_PTR(desc);
  switch (op) {
    case TSA_OP_INDEX_BUILD: {
      const auto* d = static_cast<const tsa_ivf_desc*>(desc);
      if (tsa_status s = check_ivf(d)) return s;
      *bytes = index_ws(*d);
      return ok();
    }
    case TSA_OP_SPARSE_DECODE: {
      const auto* d = static_cast<const tsa_ivf_desc*>(desc);
      if (tsa_status s = check_ivf(d)) return s;
      if (k < 1 || k > d->n_centroids) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, C=%d]", k, d->n_centroids);
      *bytes = ivf_layout(*d, k).total;
      return ok();
    }
    case TSA_OP_SPARSE_DECODE_EX: {
      const auto* d = static_cast<const tsa_ivf_desc*>(desc);
      if (tsa_status s = check_ivf(d)) return s;
      if (k < 1 || k > d->n_centroids) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, C=%d]", k, d->n_centroids);
      *bytes = ivf_layout(*d, k, true).total;
      return ok();
    }
    case TSA_OP_INDEX_BUILD_MULTI: {
      const auto* d = static_cast<const tsa_ivf_desc*>(desc);
      if (tsa_status s = check_ivf(d)) return s;
      *bytes = index_ws(*d, 2);
      return ok();
    }
    case TSA_OP_SPARSE_DECODE_EX_MULTI: {
      const auto* d = static_cast<const tsa_ivf_desc*>(desc);
      if (tsa_status s = check_ivf(d)) return s;
      if (k < 1 || k > d->n_centroids) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, C=%d]", k, d->n_centroids);
      *bytes = ivf_layout(*d, k, true, 2).total;
      return ok();
    }
    case TSA_OP_TOKEN_DECODE: {
      const auto* d = static_cast<const tsa_token_desc*>(desc);
      if (tsa_status s = check_token(d, k)) return s;
      *bytes = tok_layout(*d, k).total;
      return ok();
    }
    case TSA_OP_ATTEND_ROWS: {
      const auto* d = static_cast<const tsa_attn_desc*>(desc);
      if (tsa_status s = check_attn(d)) return s;
      *bytes = rows_layout(*d).total;
      return ok();
    }
    default:
      return fail(TSA_ERR_INVALID_ARG, "unknown op %d", op);
  }
}

tsa_status tsa_index_build(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                           int32_t* offsets, int32_t* ids, void* ws, size_t ws_bytes,
                           void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  return index_build_impl(desc, keys, centroids, desc->n_tokens, 0, offsets, nullptr, ids, ws, ws_bytes, stream);
}

tsa_status tsa_index_build_dyn(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                               int32_t n_prefix, int32_t slack, int32_t* offsets, int32_t* lens, int32_t* ids,
                               void* ws, size_t ws_bytes, void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  REQUIRE_PTR(lens);
  if (n_prefix < 1 || n_prefix > desc->n_tokens)
    return fail(TSA_ERR_INVALID_ARG, "n_prefix=%d outside [1, N=%d]", n_prefix, desc->n_tokens);
  if (slack < 0 || n_prefix + static_cast<long long>(desc->n_centroids) * slack > desc->n_tokens)
    return fail(TSA_ERR_INVALID_ARG, "n_prefix + C * slack = %lld exceeds N=%d",
                n_prefix + static_cast<long long>(desc->n_centroids) * slack, desc->n_tokens);
  return index_build_impl(desc, keys, centroids, n_prefix, slack, offsets, lens, ids, ws, ws_bytes, stream);
}

tsa_status tsa_index_build_multi(const tsa_ivf_desc* desc, const void* keys, const void* centroids, int32_t m,
                                 int32_t* offsets, int32_t* ids, int32_t* alt, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  if (tsa_status s = check_m(desc, m)) return s;
  if (m > 1) REQUIRE_PTR(alt);
  return index_build_impl(desc, keys, centroids, desc->n_tokens, 0, offsets, nullptr, ids, ws, ws_bytes, stream, m,
                          m > 1 ? alt : nullptr);
}

tsa_status tsa_index_build_dyn_multi(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                                     int32_t n_prefix, int32_t slack, int32_t m, int32_t* offsets, int32_t* lens,
                                     int32_t* ids, int32_t* alt, void* ws, size_t ws_bytes, void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  if (tsa_status s = check_m(desc, m)) return s;
  REQUIRE_PTR(lens);
  if (m > 1) REQUIRE_PTR(alt);
  if (n_prefix < 1 || n_prefix > desc->n_tokens)
    return fail(TSA_ERR_INVALID_ARG, "n_prefix=%d outside [1, N=%d]", n_prefix, desc->n_tokens);
  const long long need = static_cast<long long>(n_prefix) * m + static_cast<long long>(desc->n_centroids) * slack;
  if (slack < 0 || need > static_cast<long long>(desc->n_tokens) * m)
    return fail(TSA_ERR_INVALID_ARG, "n_prefix * m + C * slack = %lld exceeds N * m = %lld", need,
                static_cast<long long>(desc->n_tokens) * m);
  return index_build_impl(desc, keys, centroids, n_prefix, slack, offsets, lens, ids, ws, ws_bytes, stream, m,
                          m > 1 ? alt : nullptr);
}

tsa_status tsa_kv_append_multi(const tsa_ivf_desc* desc, int32_t m, const void* new_k, const void* new_v,
                               const int32_t* pos, const void* centroids, void* k_cache, void* v_cache,
                               const int32_t* offsets, int32_t* lens, int32_t* ids, int32_t* alt, int32_t* status,
                               void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  if (tsa_status s = check_m(desc, m)) return s;
  REQUIRE_PTR(new_k); REQUIRE_PTR(new_v); REQUIRE_PTR(pos); REQUIRE_PTR(centroids); REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache); REQUIRE_PTR(offsets); REQUIRE_PTR(lens); REQUIRE_PTR(ids);
  if (m > 1) REQUIRE_PTR(alt);
  REQUIRE_ALIGN(new_k, 16); REQUIRE_ALIGN(new_v, 16); REQUIRE_ALIGN(centroids, 16); REQUIRE_ALIGN(k_cache, 16);
  REQUIRE_ALIGN(v_cache, 16);
  const tsa_ivf_desc& d = *desc;
  AppendParams ap{new_k, new_v, pos, centroids, codebook_stride(d), k_cache, v_cache, offsets, lens, ids, status,
                  d.batch, d.n_tokens, d.n_kv_heads, d.n_centroids};
  ap.m = m;
  ap.alt = m > 1 ? alt : nullptr;
  const hipStream_t s = as_stream(stream);
  hipError_t e = launch_between(g_append_evs, s, [&] { return launch_kv_append(ap, d.dtype, s); });
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return ok();
}

tsa_status tsa_kv_append(const tsa_ivf_desc* desc, const void* new_k, const void* new_v, const int32_t* pos,
                         const void* centroids, void* k_cache, void* v_cache, const int32_t* offsets,
                         int32_t* lens, int32_t* ids, int32_t* status, void* stream) {
  return tsa_kv_append_multi(desc, 1, new_k, new_v, pos, centroids, k_cache, v_cache, offsets, lens, ids, nullptr,
                             status, stream);
}

tsa_status tsa_index_regrow(const tsa_ivf_desc* desc, int32_t m, const int32_t* offsets, const int32_t* lens,
                            const int32_t* ids, const int32_t* alt, int32_t slack, int32_t* offsets_out,
                            int32_t* lens_out, int32_t* ids_out, int32_t* alt_out, int32_t* status, void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  if (tsa_status s = check_m(desc, m)) return s;
  REQUIRE_PTR(offsets); REQUIRE_PTR(lens); REQUIRE_PTR(ids);
  REQUIRE_PTR(offsets_out); REQUIRE_PTR(lens_out); REQUIRE_PTR(ids_out);
  if (m > 1) {
    REQUIRE_PTR(alt);
    REQUIRE_PTR(alt_out);
  }
  if (ids_out == ids || offsets_out == offsets || lens_out == lens || (m > 1 && alt_out == alt))
    return fail(TSA_ERR_INVALID_ARG, "regrow writes separate output arrays (an output aliases its input)");
  RegrowParams rp{offsets, lens, ids, m > 1 ? alt : nullptr, offsets_out, lens_out, ids_out,
                  m > 1 ? alt_out : nullptr, status, desc->batch, desc->n_kv_heads, desc->n_centroids,
                  desc->n_tokens * m, m, slack};
  const hipStream_t s = as_stream(stream);
  hipError_t e = launch_between(g_regrow_evs, s, [&] { return launch_regrow(rp, s); });
  if (e != hipSuccess) return hip_fail(e, "regrow launch");
  return ok();
}

tsa_status tsa_sparse_decode(const tsa_ivf_desc* desc, const void* q, const void* centroids,
                             const int32_t* offsets, const int32_t* ids, const void* k_cache,
                             const void* v_cache, int32_t k, float* out, int32_t* sel_out,
                             int32_t* rows_out, int32_t* uniq_out, void* ws, size_t ws_bytes,
                             void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  return sparse_decode_impl(desc, nullptr, q, centroids, offsets, nullptr, ids, k_cache, v_cache, k, out, sel_out,
                            rows_out, uniq_out, ws, ws_bytes, stream);
}

tsa_status tsa_sparse_decode_dyn(const tsa_ivf_desc* desc, const void* q, const void* centroids,
                                 const int32_t* offsets, const int32_t* lens, const int32_t* ids,
                                 const void* k_cache, const void* v_cache, int32_t k, float* out,
                                 int32_t* sel_out, int32_t* rows_out, int32_t* uniq_out, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  REQUIRE_PTR(lens);
  return sparse_decode_impl(desc, nullptr, q, centroids, offsets, lens, ids, k_cache, v_cache, k, out, sel_out,
                            rows_out, uniq_out, ws, ws_bytes, stream);
}

tsa_status tsa_kv_list_major(const tsa_ivf_desc* desc, const int32_t* ids, const void* k_cache,
                             const void* v_cache, void* k_lists, void* v_lists, void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  REQUIRE_PTR(ids); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache); REQUIRE_PTR(k_lists); REQUIRE_PTR(v_lists);
  REQUIRE_ALIGN(k_cache, 16); REQUIRE_ALIGN(v_cache, 16); REQUIRE_ALIGN(k_lists, 16); REQUIRE_ALIGN(v_lists, 16);
  if (k_lists == v_lists || k_lists == k_cache || k_lists == v_cache || v_lists == k_cache || v_lists == v_cache)
    return fail(TSA_ERR_INVALID_ARG, "the list-major copies must be separate arrays from each other and the caches");
  const tsa_ivf_desc& d = *desc;
  if (static_cast<long long>(d.batch) * d.n_kv_heads > 65535)
    return fail(TSA_ERR_UNSUPPORTED, "batch * n_kv_heads = %lld > 65535",
                static_cast<long long>(d.batch) * d.n_kv_heads);
  KvListsParams kp{ids, k_cache, v_cache, k_lists, v_lists, d.batch, d.n_tokens, d.n_kv_heads};
  const hipError_t e = launch_kv_list_major(kp, d.dtype, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "kv_list_major launch");
  return ok();
}

tsa_status tsa_sparse_decode_ex(const tsa_ivf_desc* desc, const tsa_decode_opts* opts, const void* q,
                                const void* centroids, const int32_t* offsets, const int32_t* ids,
                                const void* k_cache, const void* v_cache, int32_t k, float* out,
                                int32_t* sel_out, int32_t* rows_out, int32_t* uniq_out, void* ws, size_t ws_bytes,
                                void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  REQUIRE_PTR(opts);
  if (opts->similarity != TSA_SIM_DOT && opts->similarity != TSA_SIM_COSINE)
    return fail(TSA_ERR_INVALID_ARG, "unknown similarity %d", opts->similarity);
  if (opts->n_sink < 0 || opts->n_window < 0 ||
      static_cast<long long>(opts->n_sink) + opts->n_window > kMaxFixedRows)
    return fail(TSA_ERR_INVALID_ARG, "n_sink=%d, n_window=%d: each >= 0 and together <= %d", opts->n_sink,
                opts->n_window, kMaxFixedRows);
  if (opts->assign_per_key < 0 || opts->assign_per_key > kMaxAssign)
    return fail(TSA_ERR_INVALID_ARG, "assign_per_key=%d outside [0, %d]", opts->assign_per_key, kMaxAssign);
  if (opts->assign_per_key > 1) {
    if (tsa_status s = check_m(desc, opts->assign_per_key)) return s;
    if (!opts->alt) return fail(TSA_ERR_INVALID_ARG, "opts->alt is NULL for %d lists per token", opts->assign_per_key);
  }
  if (opts->schedule < TSA_SCHED_AUTO || opts->schedule > TSA_SCHED_SPLIT)
    return fail(TSA_ERR_INVALID_ARG, "unknown schedule %d", opts->schedule);
  if ((opts->schedule == TSA_SCHED_FUSED || opts->schedule == TSA_SCHED_SPLIT) && !head_qualifies(*desc, k, opts))
    return fail(TSA_ERR_UNSUPPORTED, "the fused and split decodes need one list per token, no sink or window, "
                "C <= %d and k <= %d", kHeadMaxC, kHeadMaxK);
  if (opts->schedule == TSA_SCHED_SPLIT && desc->dtype != TSA_BF16)
    return fail(TSA_ERR_UNSUPPORTED, "the split decode scores bf16 codebooks only");
  if ((opts->k_lists == nullptr) != (opts->v_lists == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "opts->k_lists and opts->v_lists: give both or neither");
  if (opts->k_lists) {
    REQUIRE_ALIGN(opts->k_lists, 16);
    REQUIRE_ALIGN(opts->v_lists, 16);
    if (opts->assign_per_key > 1 || opts->n_sink > 0 || opts->n_window > 0 || opts->lens)
      return fail(TSA_ERR_UNSUPPORTED, "the list-major copies take plain lists: one list per token, no sink, "
                  "window or growing index");
  }
  return sparse_decode_impl(desc, opts, q, centroids, offsets, opts->lens, ids, k_cache, v_cache, k, out, sel_out,
                            rows_out, uniq_out, ws, ws_bytes, stream);
}

tsa_status tsa_token_decode(const tsa_token_desc* desc, const void* q_idx, const void* k_idx,
                            const void* q, const void* k_cache, const void* v_cache, int32_t k,
                            float* out, int32_t* sel_out, void* ws, size_t ws_bytes, void* stream) {
  if (tsa_status s = check_token(desc, k)) return s;
  REQUIRE_PTR(q_idx); REQUIRE_PTR(k_idx); REQUIRE_PTR(q); REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache);
  REQUIRE_PTR(out); REQUIRE_PTR(ws);
  REQUIRE_ALIGN(q_idx, 16); REQUIRE_ALIGN(k_idx, 16); REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k_cache, 16);
  REQUIRE_ALIGN(v_cache, 16); REQUIRE_ALIGN(out, 8); REQUIRE_ALIGN(ws, 16);
  const tsa_token_desc& d = *desc;
  const TokLayout L = tok_layout(d, k);
  if (ws_bytes < L.total) return fail(TSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  char* w = static_cast<char*>(ws);
  hipStream_t s = as_stream(stream);
  int32_t* sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(w + L.sel);
  TokenSelectParams tp{q_idx, k_idx, reinterpret_cast<uint32_t*>(w + L.keys),
                       reinterpret_cast<int32_t*>(w + L.hist), reinterpret_cast<uint32_t*>(w + L.cand_key),
                       reinterpret_cast<int32_t*>(w + L.cand_id), reinterpret_cast<int32_t*>(w + L.cand_cnt),
                       sel, d.batch, d.n_tokens, k, L.nfchunk};
  tp.score_ev0 = g_scan_ev0;
  tp.score_ev1 = g_scan_ev1;
  tp.epoch = reinterpret_cast<uint64_t*>(w + L.epoch);
  tp.ready = reinterpret_cast<uint64_t*>(w + L.ready);
  tp.grab = reinterpret_cast<int32_t*>(w + L.grab);
  tp.nonce = next_token_nonce();
  g_scan_ev0 = g_scan_ev1 = nullptr;
  hipError_t e = launch_token_select(tp, d.dtype, s);
  if (e != hipSuccess) return hip_fail(e, "token_select launch");

  GatherParams gp{};
  gp.q = q; gp.k = k_cache; gp.v = v_cache; gp.n_rows = d.n_tokens;
  gp.rowids = sel; gp.rid_bstride = k; gp.rid_gstride = 0;
  gp.seg = nullptr; gp.nseg = nullptr; gp.counts = nullptr; gp.count_const = k; gp.count_max = k;
  gp.partial = reinterpret_cast<float*>(w + L.partial); gp.out = out;
  gp.B = d.batch; gp.Hkv = d.n_kv_heads; gp.smax = L.smax;
  gp.W = gather_blocks_per_head(L.smax, false); gp.seg_rows = L.seg_rows;
  gp.qscale = qscale(d.head_dim);
  if (tsa_status st = launch_gather_timed(gp, d.dtype, L.G, false, s)) return st;
  return ok();
}

tsa_status tsa_attend_rows(const tsa_attn_desc* desc, const void* q, const void* k_rows,
                           const void* v_rows, const int32_t* row_ids, const int32_t* row_counts,
                           float* out, void* ws, size_t ws_bytes, void* stream) {
  if (tsa_status s = check_attn(desc)) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(k_rows); REQUIRE_PTR(v_rows); REQUIRE_PTR(out); REQUIRE_PTR(ws);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(k_rows, 16); REQUIRE_ALIGN(v_rows, 16); REQUIRE_ALIGN(out, 8);
  REQUIRE_ALIGN(ws, 16);
  const tsa_attn_desc& d = *desc;
  if (d.max_rows > 0) REQUIRE_PTR(row_ids);
  const RowsLayout L = rows_layout(d);
  if (ws_bytes < L.total) return fail(TSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, L.total);
  hipStream_t s = as_stream(stream);
  GatherParams gp{};
  gp.q = q; gp.k = k_rows; gp.v = v_rows; gp.n_rows = d.n_rows;
  gp.rowids = row_ids; gp.rid_bstride = d.max_rows; gp.rid_gstride = 0;
  gp.seg = nullptr; gp.nseg = nullptr; gp.counts = row_counts; gp.count_const = d.max_rows;
  gp.count_max = d.max_rows;
  gp.partial = static_cast<float*>(ws); gp.out = out;
  gp.B = d.batch; gp.Hkv = d.n_kv_heads; gp.smax = L.smax;
  gp.W = gather_blocks_per_head(L.smax, false); gp.seg_rows = L.seg_rows;
  gp.qscale = qscale(d.head_dim);
  if (tsa_status st = launch_gather_timed(gp, d.dtype, L.G, false, s)) return st;
  return ok();
}

tsa_status tsa_resolve_policy(const tsa_cache_desc* desc, int32_t* page_table, int32_t* slot_token,
                              int32_t* last_use, const int32_t* sel, int32_t k, int32_t step, int32_t policy,
                              uint64_t seed, const int32_t* priority, const void* host_k, const void* host_v,
                              void* pool_k, void* pool_v, int32_t* slots_out, int32_t* hits, int32_t* misses,
                              int32_t* miss_tok, int32_t* miss_slot, void* stream) {
  if (tsa_status s = check_cache(desc)) return s;
  REQUIRE_PTR(page_table); REQUIRE_PTR(slot_token); REQUIRE_PTR(last_use); REQUIRE_PTR(sel);
  REQUIRE_PTR(host_k); REQUIRE_PTR(host_v); REQUIRE_PTR(pool_k); REQUIRE_PTR(pool_v); REQUIRE_PTR(slots_out);
  REQUIRE_ALIGN(host_k, 16); REQUIRE_ALIGN(host_v, 16); REQUIRE_ALIGN(pool_k, 16); REQUIRE_ALIGN(pool_v, 16);
  const tsa_cache_desc& d = *desc;
  if (k < 1 || k > d.n_slots || k > kMaxTokenK)
    return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, min(S=%d, %d)]", k, d.n_slots, kMaxTokenK);
  if (step < 0 || step == INT32_MAX) return fail(TSA_ERR_INVALID_ARG, "step %d out of range", step);
  if (policy < TSA_EVICT_LRU || policy > TSA_EVICT_PRIORITY)
    return fail(TSA_ERR_INVALID_ARG, "unknown replacement policy %d", policy);
  if (policy == TSA_EVICT_PRIORITY) REQUIRE_PTR(priority);
  if ((miss_tok == nullptr) != (miss_slot == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "miss_tok and miss_slot must both be given or both be NULL");
  ResolveParams rp{page_table, slot_token, last_use, sel, host_k, host_v, pool_k, pool_v, slots_out, hits,
                   misses, static_cast<long long>(d.n_kv_heads) * d.head_dim * esize(d.dtype),
                   d.batch, d.n_tokens, d.n_slots, k, step, policy, static_cast<unsigned long long>(seed),
                   priority, miss_tok, miss_slot};
  hipError_t e = launch_resolve(rp, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "resolve launch");
  return ok();
}

tsa_status tsa_resolve(const tsa_cache_desc* desc, int32_t* page_table, int32_t* slot_token,
                       int32_t* last_use, const int32_t* sel, int32_t k, int32_t step,
                       const void* host_k, const void* host_v, void* pool_k, void* pool_v,
                       int32_t* slots_out, int32_t* hits, int32_t* misses, void* stream) {
  return tsa_resolve_policy(desc, page_table, slot_token, last_use, sel, k, step, TSA_EVICT_LRU, 0, nullptr,
                            host_k, host_v, pool_k, pool_v, slots_out, hits, misses, nullptr, nullptr, stream);
}

tsa_status tsa_fetch_rows(const tsa_cache_desc* desc, const int32_t* miss_tok, const int32_t* miss_slot,
                          const int32_t* misses, int32_t k, const void* host_k, const void* host_v, void* pool_k,
                          void* pool_v, void* stream) {
  if (tsa_status s = check_cache(desc)) return s;
  REQUIRE_PTR(miss_tok); REQUIRE_PTR(miss_slot); REQUIRE_PTR(misses);
  REQUIRE_PTR(host_k); REQUIRE_PTR(host_v); REQUIRE_PTR(pool_k); REQUIRE_PTR(pool_v);
  REQUIRE_ALIGN(host_k, 16); REQUIRE_ALIGN(host_v, 16); REQUIRE_ALIGN(pool_k, 16); REQUIRE_ALIGN(pool_v, 16);
  const tsa_cache_desc& d = *desc;
  if (k < 1 || k > d.n_slots || k > kMaxTokenK)
    return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, min(S=%d, %d)]", k, d.n_slots, kMaxTokenK);
  FetchParams fp = fetch_params(d, miss_tok, miss_slot, misses, k, 1);
  fp.host_k[0] = host_k; fp.host_v[0] = host_v; fp.pool_k[0] = pool_k; fp.pool_v[0] = pool_v;
  hipError_t e = launch_fetch_rows(fp, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "fetch_rows launch");
  return ok();
}

tsa_status tsa_hier_group_step(const tsa_cache_desc* desc, int32_t n_q_heads, int32_t n_layers,
                               const tsa_layer_io* layers, int32_t* page_table, int32_t* slot_token,
                               int32_t* last_use, const int32_t* sel, int32_t k, int32_t step, int32_t policy,
                               uint64_t seed, const int32_t* priority, int32_t* slots_out, int32_t* hits,
                               int32_t* misses, int32_t* miss_tok, int32_t* miss_slot, void* ws, size_t ws_bytes,
                               void* stream, void* fetch_stream, void* const* events) {
  if (tsa_status s = check_cache(desc)) return s;
  REQUIRE_PTR(layers); REQUIRE_PTR(slots_out);
  if (n_layers < 1 || n_layers > kMaxFetchLayers + 1)
    return fail(TSA_ERR_INVALID_ARG, "n_layers=%d outside [1, %d]", n_layers, kMaxFetchLayers + 1);
  const tsa_cache_desc& d = *desc;
  const tsa_attn_desc ad{d.batch, d.n_slots, d.n_kv_heads, n_q_heads, d.head_dim, k, d.dtype};
  if (tsa_status s = check_attn(&ad)) return s;
  if (n_layers > 1) {
    REQUIRE_PTR(misses); REQUIRE_PTR(miss_tok); REQUIRE_PTR(miss_slot);
    if (fetch_stream) {
      REQUIRE_PTR(events);
      if (!events[0] || !events[1]) return fail(TSA_ERR_INVALID_ARG, "events[0] and events[1] must be given");
    }
  }
  for (int j = 0; j < n_layers; ++j) {
    const tsa_layer_io& L = layers[j];
    if (!L.host_k || !L.host_v || !L.pool_k || !L.pool_v || !L.q || !L.out)
      return fail(TSA_ERR_INVALID_ARG, "layers[%d] has a NULL pointer", j);
    if (!aligned(L.host_k, 16) || !aligned(L.host_v, 16) || !aligned(L.pool_k, 16) || !aligned(L.pool_v, 16) ||
        !aligned(L.q, 16) || !aligned(L.out, 8))
      return fail(TSA_ERR_INVALID_ARG, "layers[%d] has a misaligned pointer", j);
  }
  const size_t need = rows_layout(ad).total;
  if (ws_bytes < need) return fail(TSA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  hipStream_t s = as_stream(stream);
  hipStream_t fs = fetch_stream ? as_stream(fetch_stream) : nullptr;

  // RESOLVE once for the group: tables, miss list and the first layer's rows
  if (tsa_status st = tsa_resolve_policy(desc, page_table, slot_token, last_use, sel, k, step, policy, seed,
                                         priority, layers[0].host_k, layers[0].host_v, layers[0].pool_k,
                                         layers[0].pool_v, slots_out, hits, misses,
                                         n_layers > 1 ? miss_tok : nullptr, n_layers > 1 ? miss_slot : nullptr,
                                         stream))
    return st;
  // the other layers' rows: one launch for the whole group
  FetchParams fp = fetch_params(d, miss_tok, miss_slot, misses, k, n_layers - 1);
  for (int j = 1; j < n_layers; ++j) {
    fp.host_k[j - 1] = layers[j].host_k; fp.host_v[j - 1] = layers[j].host_v;
    fp.pool_k[j - 1] = layers[j].pool_k; fp.pool_v[j - 1] = layers[j].pool_v;
  }
  hipError_t e = hipSuccess;
  if (n_layers > 1 && fs) {
    // prefetch: the rows stream in on the second stream while layer 0 attends
    e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s);
    if (e == hipSuccess) e = hipStreamWaitEvent(fs, static_cast<hipEvent_t>(events[0]), 0);
    if (e == hipSuccess) e = launch_fetch_rows(fp, fs);
    if (e == hipSuccess) e = hipEventRecord(static_cast<hipEvent_t>(events[1]), fs);
    if (e != hipSuccess) return hip_fail(e, "layer prefetch");
  }
  for (int j = 0; j < n_layers; ++j) {
    if (j == 1) {
      e = fs ? hipStreamWaitEvent(s, static_cast<hipEvent_t>(events[1]), 0) : launch_fetch_rows(fp, s);
      if (e != hipSuccess) return hip_fail(e, "layer fetch");
    }
    if (tsa_status st = tsa_attend_rows(&ad, layers[j].q, layers[j].pool_k, layers[j].pool_v, slots_out, nullptr,
                                        layers[j].out, ws, ws_bytes, stream))
      return st;
  }
  return ok();
}

tsa_status tsa_cache_reset(const tsa_cache_desc* desc, int32_t* page_table, int32_t* slot_token,
                           int32_t* last_use, void* stream) {
  if (tsa_status s = check_cache(desc)) return s;
  REQUIRE_PTR(page_table); REQUIRE_PTR(slot_token); REQUIRE_PTR(last_use);
  const tsa_cache_desc& d = *desc;
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_fill_i32(page_table, static_cast<long long>(d.batch) * d.n_tokens, -1, s);
  if (e == hipSuccess) e = launch_fill_i32(slot_token, static_cast<long long>(d.batch) * d.n_slots, -1, s);
  if (e == hipSuccess) e = launch_fill_i32(last_use, static_cast<long long>(d.batch) * d.n_slots, -1, s);
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  return ok();
}

tsa_status tsa_host_alloc(size_t bytes, void** host_ptr) {
  REQUIRE_PTR(host_ptr);
  if (bytes == 0) return fail(TSA_ERR_INVALID_ARG, "bytes == 0");
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc");
  *host_ptr = p;
  return ok();
}

tsa_status tsa_host_free(void* host_ptr) {
  REQUIRE_PTR(host_ptr);
  hipError_t e = hipHostFree(host_ptr);
  if (e != hipSuccess) return hip_fail(e, "hipHostFree");
  return ok();
}

// Allocation-free decode. The workspace of tsa_sparse_decode_noalloc is a
// fixed array in the library's device code object instead of caller memory:
// each GPU the library runs on holds its own copy until the process ends.
// In host code the array's name stands for a host-side shadow, so kernels get
// the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[TSA_NOALLOC_SCRATCH_BYTES];

}  // extern "C"

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device, with the device current).
tsa_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(TSA_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(TSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSA_OK;
}

}  // namespace

extern "C" {

tsa_status tsa_sparse_decode_noalloc(const tsa_ivf_desc* desc, const void* q, const void* centroids,
                                     const int32_t* offsets, const int32_t* ids, const void* k_cache,
                                     const void* v_cache, int32_t k, float* out, int32_t* sel_out,
                                     int32_t* rows_out, int32_t* uniq_out, void* stream) {
  if (tsa_status s = check_ivf(desc)) return s;
  // every check runs before the scratch address is looked up
  REQUIRE_PTR(q); REQUIRE_PTR(centroids); REQUIRE_PTR(offsets); REQUIRE_PTR(ids);
  REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache); REQUIRE_PTR(out);
  REQUIRE_ALIGN(q, 16); REQUIRE_ALIGN(centroids, 16); REQUIRE_ALIGN(k_cache, 16);
  REQUIRE_ALIGN(v_cache, 16); REQUIRE_ALIGN(out, 8);
  if (k < 1 || k > desc->n_centroids) return fail(TSA_ERR_INVALID_ARG, "k=%d outside [1, C=%d]", k, desc->n_centroids);
  const size_t need = ivf_layout(*desc, k, false, 1).total;
  if (need > static_cast<size_t>(TSA_NOALLOC_SCRATCH_BYTES))
    return fail(TSA_ERR_WORKSPACE, "this decode needs %zu bytes of workspace; the static scratch holds %zu",
                need, static_cast<size_t>(TSA_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (tsa_status s = scratch_ptr(&ws)) return s;
  return sparse_decode_impl(desc, nullptr, q, centroids, offsets, nullptr, ids, k_cache, v_cache, k, out, sel_out,
                            rows_out, uniq_out, ws, static_cast<size_t>(TSA_NOALLOC_SCRATCH_BYTES), stream);
}

tsa_status tsa_time_next_gather(void* ev_start, void* ev_stop) {
  return tsa_time_next_launch(TSA_TIMED_GATHER, ev_start, ev_stop);
}

tsa_status tsa_time_next_launch(int32_t kernel, void* ev_start, void* ev_stop) {
  if ((ev_start == nullptr) != (ev_stop == nullptr))
    return fail(TSA_ERR_INVALID_ARG, "give both events or neither");
  switch (kernel) {
    case TSA_TIMED_GATHER:
      g_gather_evs[0] = static_cast<hipEvent_t>(ev_start);
      g_gather_evs[1] = static_cast<hipEvent_t>(ev_stop);
      return ok();
    case TSA_TIMED_TOKEN_SCAN:
      g_scan_ev0 = static_cast<hipEvent_t>(ev_start);
      g_scan_ev1 = static_cast<hipEvent_t>(ev_stop);
      return ok();
    case TSA_TIMED_APPEND:
      g_append_evs[0] = static_cast<hipEvent_t>(ev_start);
      g_append_evs[1] = static_cast<hipEvent_t>(ev_stop);
      return ok();
    case TSA_TIMED_REGROW:
      g_regrow_evs[0] = static_cast<hipEvent_t>(ev_start);
      g_regrow_evs[1] = static_cast<hipEvent_t>(ev_stop);
      return ok();
  }
  return fail(TSA_ERR_INVALID_ARG, "unknown timed kernel %d", kernel);
}

tsa_status tsa_stream_read(const void* p, size_t bytes, uint32_t* sink, size_t sink_bytes, void* stream) {
  REQUIRE_PTR(p); REQUIRE_PTR(sink);
  REQUIRE_ALIGN(p, 16); REQUIRE_ALIGN(sink, 4);
  if (bytes == 0 || bytes % 16) return fail(TSA_ERR_INVALID_ARG, "bytes %zu is not a positive multiple of 16", bytes);
  const size_t need = tsa_stream_read_sink_bytes();
  if (sink_bytes < need) return fail(TSA_ERR_WORKSPACE, "sink %zu < %zu bytes", sink_bytes, need);
  hipError_t e = launch_stream_read(p, static_cast<long long>(bytes / 16), sink, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  return ok();
}

size_t tsa_stream_read_sink_bytes(void) {
  return static_cast<size_t>(stream_read_blocks()) * stream_read_waves_per_block() * sizeof(uint32_t);
}

}  // extern "C"
