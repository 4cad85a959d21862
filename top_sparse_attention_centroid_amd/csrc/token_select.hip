// Token-level indexer top-k for gfx950 (DSA-style selector: "10月14日学习笔记",
// HiSparse motivation -- the indexer keeps the top-k tokens so attention work
// is O(k); "KV卸载上主机:HiSparse、PDD与DDR4回收", HiSparse analysis -- the
// selector names the positions each step needs).
//
// The selection is the k largest scores under the total order (score desc,
// token id asc), emitted in ascending id order. Three kernels:
//   score  -- streams the indexer keys (d_idx = 64 bf16 = 128 B per token,
//             8 lanes x 16 B), each workgroup an equal share of a request's
//             first nine tenths, then chunks of the rest as it gets to them,
//             writes one order-preserving 32-bit key per token and adds
//             every key's top 12 bits to a per-request histogram (one LDS
//             histogram per workgroup, flushed once with global atomics
//             into the request's histogram, which the request's first
//             workgroup clears in the same launch).
//   filter -- every workgroup reads the histogram, finds the threshold bin
//             (the highest bin at which the count from the top reaches k)
//             and compacts the keys at or above it, in id order, into its
//             own region of the candidate buffer.
//   final  -- one workgroup per request: an exact radix select over the
//             low 20 bits of the threshold-bin candidates gives the k-th key
//             T and how many keys equal to T are taken; the candidates are
//             then emitted in id order from running block scans.
// Every key above T lies above or in the threshold bin, so the candidates
// hold the whole selection and the result is exact for any score
// distribution (ties included); only the work of the final kernel grows
// with the number of keys that share the threshold bin.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kIdxDim = 64;
constexpr int kScoreThreads = 512;
constexpr int kScoreUnroll = 4;  // 16-B loads in flight per lane (8 waves x 4 beat 4 waves x 8)
constexpr int kTokScoreTile = 2048;  // tokens per LDS-staged sub-tile of a scan workgroup
constexpr int kTokFirstTile = 256;   // the clearing workgroup's first sub-tile, after which it publishes
constexpr int kTokDynDiv = 10;       // the last N / kTokDynDiv tokens of a request are shared out in chunks
constexpr int kTokGrab = 512;        // tokens per shared chunk
constexpr long long kScoreWorkgroups = 1024;  // scan workgroups per launch: 4 per CU
constexpr long long kScoreMinShare = 1024;    // fewest tokens a scan workgroup takes
constexpr int kFilterThreads = 512;
constexpr int kFinalThreads = 1024;
constexpr int kHistShift = 32 - kTokHistBits;
constexpr int kFinalLdsCands = 8192;  // candidates the final kernel stages in LDS
constexpr int kRadixBits = 10;        // digit of the final kernel's radix select
constexpr int kRadixBins = 1 << kRadixBits;

// The threshold bin of a request: the highest bin t with
// count(bins >= t) >= k, and the count of keys in bins above t. NT threads,
// each owning kTokHistBins / NT consecutive bins. scratch: NT / 64 ints;
// misc: 2 ints.
template <int NT>
__device__ __forceinline__ void threshold_bin(const int32_t* hist, int k, int* scratch, int* misc, int* tbin,
                                              int* above) {
  constexpr int PB = kTokHistBins / NT;
  const int tid = threadIdx.x;
  int c[PB], v = 0;
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    c[q] = hist[tid * PB + q];
    v += c[q];
  }
  if (tid == 0) {
    misc[0] = 0;  // unreachable when the histogram holds all N >= k keys
    misc[1] = 0;
  }
  int total;
  const int excl = block_exclusive_scan<NT / kWave>(v, scratch, &total);
  int a = total - excl - v;  // keys in the bins of higher threads
  if (a < k && a + v >= k) {
    int t = -1, at = 0;
#pragma unroll
    for (int q = PB - 1; q >= 0; --q) {
      if (t < 0 && a + c[q] >= k) {
        t = tid * PB + q;
        at = a;
      }
      a += c[q];
    }
    misc[0] = t;
    misc[1] = at;
  }
  __syncthreads();
  *tbin = misc[0];
  *above = misc[1];
  __syncthreads();
}

// The tag a call publishes once its histogram is clear: the SplitMix64
// output function (Steele, Lea and Flood, OOPSLA 2014), a bijection on 64-bit
// words, of epoch * phi + nonce (phi = 0x9E3779B97F4A7C15, odd). Between a
// call and the one before it on the same workspace the epoch has advanced by
// one and the nonce has changed, so that input differs (by phi plus the nonce
// step), and so does the tag: the tag left by the previous call never passes
// for this call's. (Mixing epoch ^ nonce instead is not enough: when both go
// up by one and end in the same run of one bits, the XOR does not change.)
// Graph replays keep the nonce and advance the epoch, and a workspace of any
// other contents matches only by a 2^-64 coincidence.
__device__ __forceinline__ uint64_t ready_tag(uint64_t epoch, uint64_t nonce) {
  uint64_t z = epoch * 0x9E3779B97F4A7C15ull + nonce;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
constexpr uint32_t kReadySpinLimit = 1u << 20;  // about 0.2 s of s_sleep; workgroup 0 runs first

// Scores tokens [start, start + n) of request b, n <= kTokScoreTile: the
// keys go to LDS first, so that each wave round's keys leave as whole lines,
// then out to keys[b], and their top bits into the workgroup's LDS histogram.
// Ends with every thread past the LDS reads of sk except its own: the caller
// puts a barrier between two calls.
template <typename T>
__device__ __forceinline__ void score_tile(const TokenSelectParams& p, const QFrag<T>& qv, int b, int start, int n,
                                           uint32_t* sk, int* h) {
  constexpr int NW = kScoreThreads / kWave;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int e = lane & 7, tq = lane >> 3;
  const T* kb = static_cast<const T*>(p.k_idx) + (static_cast<long long>(b) * p.N + start) * kIdxDim + e * 8;
  for (int iw = wave * 8; iw < n; iw += NW * 8 * kScoreUnroll) {
    Raw8<T> raw[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int i = min(iw + u * NW * 8 + tq, n - 1);  // clamped: straight-line loads
      raw[u].load_stream(kb + static_cast<long long>(i) * kIdxDim);
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int i = iw + u * NW * 8 + tq;
      const float sc = group8_sum(qv.dot(raw[u]));
      if (e == 0 && i < n) sk[i] = order_key(sc);
    }
  }
  __syncthreads();
  uint32_t* kout = p.keys + static_cast<long long>(b) * p.N + start;
  for (int i = tid; i < n; i += kScoreThreads) {
    const uint32_t kv = sk[i];
    kout[i] = kv;
    atomicAdd(&h[kv >> kHistShift], 1);
  }
}

// Workgroup x of request b first scans its fixed share of the request's
// leading tokens, [x * S / X, (x + 1) * S / X) with S = N - N / kTokDynDiv and
// X = gridDim.x, in sub-tiles of kTokScoreTile. The rest, [S, N), is taken in
// kTokGrab-token chunks from a per-request counter by whichever workgroups of
// the request get there first: CUs do not stream at the same rate (they
// differ by about a sixth at 16 x 200K tokens, whole XCDs included), and the
// launch ends with its slowest CU. Shorter chunks and larger shared parts
// were slower: each chunk costs a barrier round and a drained load pipeline. X is chosen so that the B * X workgroups
// fill every CU the same number of times. Scores: bf16 dot2 products, 8 lanes
// a token. The workgroup's LDS histogram covers all the tokens it scanned and
// is flushed once, at its end.
//
// The request's global histogram and chunk counter are cleared here, not by a
// launch of their own: workgroup 0 of the request, the first of the request's
// workgroups to be dispatched, zeroes them with agent-scope (write-through)
// stores as it starts, scans a short first sub-tile and then, once those
// stores have completed, publishes the call's tag. Every other workgroup
// waits for the tag after its fixed share (a bounded wait: the workgroup it
// waits on is already running) before it takes chunks or adds its counts.
template <typename T>
__global__ __launch_bounds__(kScoreThreads) void token_score_kernel(TokenSelectParams p) {
  __shared__ uint32_t sk[kTokScoreTile];
  __shared__ int h[kTokHistBins];
  __shared__ int next_chunk;
  const int b = blockIdx.y;
  const int S = p.N - p.N / kTokDynDiv;
  const int share_lo = static_cast<int>(static_cast<long long>(S) * blockIdx.x / gridDim.x);
  const int share_hi = static_cast<int>(static_cast<long long>(S) * (blockIdx.x + 1) / gridDim.x);
  const int tid = threadIdx.x, lane = lane_id();
  const int e = lane & 7;
  for (int i = tid; i < kTokHistBins; i += kScoreThreads) h[i] = 0;
  int32_t* gh = p.hist + static_cast<long long>(b) * kTokHistBins;
  const uint64_t tag = ready_tag(*p.epoch, p.nonce);
  const bool clears = blockIdx.x == 0;
  if (clears) {
    uint64_t* gh64 = reinterpret_cast<uint64_t*>(gh);
    for (int i = tid; i < kTokHistBins / 2; i += kScoreThreads)
      __hip_atomic_store(gh64 + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) __hip_atomic_store(p.grab + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  bool published = !clears;

  QFrag<T> qv;
  qv.load(static_cast<const T*>(p.q_idx) + static_cast<long long>(b) * kIdxDim + e * 8);
  for (int start = share_lo; start < share_hi;) {
    const int n = min(published ? kTokScoreTile : kTokFirstTile, share_hi - start);
    score_tile<T>(p, qv, b, start, n, sk, h);
    start += n;
    if (!published) {  // the clearing stores of every wave have completed
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    __syncthreads();  // the next sub-tile overwrites sk
    if (!published) {
      if (tid == 0) __hip_atomic_store(p.ready + b, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      published = true;
    }
  }
  if (!published) {  // an empty share: publish after the clearing stores alone
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(p.ready + b, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!clears && tid == 0) {
    uint32_t spins = 0;
    while (__hip_atomic_load(p.ready + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag &&
           ++spins < kReadySpinLimit)
      __builtin_amdgcn_s_sleep(8);
  }
  // the shared tail, a chunk at a time; the next chunk is asked for before
  // the current one is scanned
  const int nchunks = (p.N - S + kTokGrab - 1) / kTokGrab;
  if (tid == 0) next_chunk = atomicAdd(p.grab + b, 1);
  __syncthreads();
  for (int c = next_chunk; c < nchunks; c = next_chunk) {
    int ahead = 0;
    if (tid == 0) ahead = atomicAdd(p.grab + b, 1);
    const int start = S + c * kTokGrab;
    score_tile<T>(p, qv, b, start, min(kTokGrab, p.N - start), sk, h);
    if (tid == 0) next_chunk = ahead;  // every thread read next_chunk before score_tile's barrier
    __syncthreads();
  }
  for (int i = tid; i < kTokHistBins; i += kScoreThreads) {
    const int c = h[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

__global__ __launch_bounds__(kFilterThreads) void token_filter_kernel(TokenSelectParams p) {
  constexpr int NW = kFilterThreads / kWave;
  constexpr int PER = kTokFilterTile / kFilterThreads;
  static_assert(PER * NW == kWave, "one count per lane of the scanning wave");
  __shared__ int scratch[NW];
  __shared__ int misc[2];
  __shared__ int cnt[PER * NW];
  const int b = blockIdx.y, c = blockIdx.x;
  const int start = c * kTokFilterTile;
  const int n = min(kTokFilterTile, p.N - start);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  // the chunk's keys are requested before the histogram is read, so the two
  // round trips overlap
  const long long base = static_cast<long long>(b) * p.N + start;
  uint32_t kk[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kFilterThreads + tid;
    kk[j] = p.keys[base + min(i, n - 1)];
  }
  int tbin, above;
  threshold_bin<kFilterThreads>(p.hist + static_cast<long long>(b) * kTokHistBins, p.k, scratch, misc, &tbin,
                                &above);
  uint64_t bal[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kFilterThreads + tid;
    bal[j] = __ballot(i < n && static_cast<int>(kk[j] >> kHistShift) >= tbin);
    if (lane == 0) cnt[j * NW + wave] = __popcll(bal[j]);
  }
  __syncthreads();
  if (wave == 0) {
    const int v = cnt[lane];
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    cnt[lane] = x - v;
    if (lane == kWave - 1) p.cand_cnt[static_cast<long long>(b) * p.nfchunk + c] = x;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if ((bal[j] >> lane) & 1u) {
      const int pos = cnt[j * NW + wave] + prefix_count(bal[j]);
      p.cand_key[base + pos] = kk[j];
      p.cand_id[base + pos] = start + j * kFilterThreads + tid;
    }
  }
}

// Candidate m of a request (m in [0, M)) sits in filter chunk c with
// coff[c] <= m < coff[c + 1], at position m - coff[c] of that chunk's region.
__device__ __forceinline__ long long cand_index(const int* coff, int nf, int m) {
  int lo = 0, hi = nf;  // invariant: coff[lo] <= m < coff[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (coff[mid] <= m) lo = mid;
    else hi = mid;
  }
  return static_cast<long long>(lo) * kTokFilterTile + (m - coff[lo]);
}

__global__ __launch_bounds__(kFinalThreads) void token_final_kernel(TokenSelectParams p) {
  constexpr int NW = kFinalThreads / kWave;
  __shared__ int coff[kMaxTokFilterChunks + 1];
  __shared__ uint32_t lkey[kFinalLdsCands];
  __shared__ int32_t lid[kFinalLdsCands];
  __shared__ int hist[kRadixBins];
  __shared__ int scratch[NW];
  __shared__ int misc[2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int nf = p.nfchunk;
  // the last kernel of the call to use the histogram advances the epoch
  if (b == 0 && tid == 0) *p.epoch = *p.epoch + 1;
  // the first chunk counts are requested before the histogram is scanned, so
  // the two round trips overlap
  const int cnt0 = tid < nf ? p.cand_cnt[static_cast<long long>(b) * nf + tid] : 0;
  int tbin, above;
  threshold_bin<kFinalThreads>(p.hist + static_cast<long long>(b) * kTokHistBins, p.k, scratch, misc, &tbin,
                               &above);
  // chunk offsets of the compacted candidates
  int run = 0;
  for (int c0 = 0; c0 < nf; c0 += kFinalThreads) {
    const int c = c0 + tid;
    const int v = c0 == 0 ? cnt0 : (c < nf ? p.cand_cnt[static_cast<long long>(b) * nf + c] : 0);
    int total;
    const int excl = block_exclusive_scan<NW>(v, scratch, &total);
    if (c < nf) coff[c] = run + excl;
    run += total;
  }
  if (tid == 0) coff[nf] = run;
  __syncthreads();
  const int M = run;
  const long long base = static_cast<long long>(b) * p.N;
  const uint32_t* ck = p.cand_key + base;
  const int32_t* cid = p.cand_id + base;
  // Candidates are read many times below: stage them in LDS when they fit
  // (the usual case: the selection plus one histogram bin), else read them
  // through the chunk offsets each time.
  const bool staged = M <= kFinalLdsCands;
  if (staged) {
    // every thread's candidates located first, then all their loads in
    // flight together (a slot past M reloads candidate 0 and is dropped)
    constexpr int kStagePer = kFinalLdsCands / kFinalThreads;
    static_assert(kStagePer * kFinalThreads == kFinalLdsCands, "whole rounds of candidates per thread");
    long long ci[kStagePer];
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const int m = tid + u * kFinalThreads;
      ci[u] = m < M ? cand_index(coff, nf, m) : 0;
    }
    uint32_t kv[kStagePer];
    int32_t iv[kStagePer];
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      kv[u] = ck[ci[u]];
      iv[u] = cid[ci[u]];
    }
#pragma unroll
    for (int u = 0; u < kStagePer; ++u) {
      const int m = tid + u * kFinalThreads;
      if (m < M) {
        lkey[m] = kv[u];
        lid[m] = iv[u];
      }
    }
    __syncthreads();
  }
  auto key_at = [&](int m) { return staged ? lkey[m] : ck[cand_index(coff, nf, m)]; };
  auto id_at = [&](int m) { return staged ? lid[m] : cid[cand_index(coff, nf, m)]; };

  // radix select of the (k - above)-th largest key inside the threshold bin:
  // two passes over 10-bit digits of the low 20 bits, one shared histogram
  // bin per thread (the bin's keys spread over many digits, so its atomics
  // rarely collide), the digit found by a block scan from the top
  static_assert(kHistShift == 2 * kRadixBits && kRadixBins == kFinalThreads, "two digits, one bin per thread");
  uint32_t prefix = static_cast<uint32_t>(tbin) << kHistShift;
  uint32_t pmask = ~0u << kHistShift;
  int krem = p.k - above;
  for (int sh = kRadixBits; sh >= 0; sh -= kRadixBits) {
    hist[tid] = 0;
    if (tid == 0) {
      misc[0] = 0;  // unreachable: the keys under the prefix number at least krem
      misc[1] = krem;
    }
    __syncthreads();
    for (int m = tid; m < M; m += kFinalThreads) {
      const uint32_t key = key_at(m);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & (kRadixBins - 1)], 1);
    }
    __syncthreads();
    const int v = hist[tid];
    int total;
    const int excl = block_exclusive_scan<NW>(v, scratch, &total);
    const int a = total - excl - v;  // keys under the prefix with a higher digit
    if (a < krem && a + v >= krem) {
      misc[0] = tid;
      misc[1] = krem - a;
    }
    __syncthreads();
    prefix |= static_cast<uint32_t>(misc[0]) << sh;
    pmask |= static_cast<uint32_t>(kRadixBins - 1) << sh;
    krem = misc[1];
    __syncthreads();
  }
  const uint32_t Tk = prefix;
  const int need_eq = krem;

  // ordered emission: keys above Tk, then the first need_eq keys equal to Tk.
  // Each thread takes kEmitPer consecutive candidates, so one block scan
  // places kEmitPer * kFinalThreads of them (counts below 2^16 per round).
  constexpr int kEmitPer = 4;
  int32_t* sel = p.sel + static_cast<long long>(b) * p.k;
  int run_gt = 0, run_eq = 0;
  for (int m0 = 0; m0 < M; m0 += kEmitPer * kFinalThreads) {
    const int mb = m0 + tid * kEmitPer;
    bool gt[kEmitPer], eq[kEmitPer];
    int v = 0;
#pragma unroll
    for (int u = 0; u < kEmitPer; ++u) {
      gt[u] = eq[u] = false;
      if (mb + u < M) {
        const uint32_t key = key_at(mb + u);
        gt[u] = key > Tk;
        eq[u] = key == Tk;
      }
      v += (gt[u] ? 1 : 0) | (eq[u] ? 1 << 16 : 0);
    }
    int total;
    const int excl = block_exclusive_scan<NW>(v, scratch, &total);
    int gt_before = run_gt + (excl & 0xffff), eq_before = run_eq + (excl >> 16);
#pragma unroll
    for (int u = 0; u < kEmitPer; ++u) {
      if (gt[u] || (eq[u] && eq_before < need_eq)) sel[gt_before + min(eq_before, need_eq)] = id_at(mb + u);
      gt_before += gt[u] ? 1 : 0;
      eq_before += eq[u] ? 1 : 0;
    }
    run_gt += total & 0xffff;
    run_eq += total >> 16;
  }
}

template <typename T>
static hipError_t token_select_typed(const TokenSelectParams& p, hipStream_t s) {
  hipError_t e;
  // shares per request: kScoreWorkgroups in all (every CU the same number of
  // workgroups), at least kScoreMinShare tokens each, at least one
  const long long want = (kScoreWorkgroups + p.B - 1) / p.B;
  const long long most = (static_cast<long long>(p.N) + kScoreMinShare - 1) / kScoreMinShare;
  const int nscore = static_cast<int>(std::max(1LL, std::min(want, most)));
  if (p.score_ev0 && (e = hipEventRecord(p.score_ev0, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(token_score_kernel<T>, dim3(nscore, p.B), dim3(kScoreThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.score_ev1 && (e = hipEventRecord(p.score_ev1, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(token_filter_kernel, dim3(p.nfchunk, p.B), dim3(kFilterThreads), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(token_final_kernel, dim3(p.B), dim3(kFinalThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_token_select(const TokenSelectParams& p, int dtype, hipStream_t s) {
  return dtype == kBF16 ? token_select_typed<bf16_t>(p, s) : token_select_typed<float>(p, s);
}

}  // namespace tsa
