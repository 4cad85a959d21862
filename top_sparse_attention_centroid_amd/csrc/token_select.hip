// Token-level indexer top-k for gfx950 (DSA-style selector: "10月14日学习笔记",
// HiSparse motivation -- the indexer keeps the top-k tokens so attention work
// is O(k); "KV卸载上主机:HiSparse、PDD与DDR4回收", HiSparse analysis -- the
// selector names the positions each step needs).
//
// Stage 1 (token_local_kernel): a workgroup streams kTokChunk indexer keys of
// one request (d_idx = 64 bf16 = 128 B per token, 8 lanes x 16 B), keeps their
// order-preserving score keys in LDS and selects the chunk's own top-k under
// the total order (score desc, token id asc). The global top-k lies inside the
// union of the chunks' top-k under that order, so stage 2 is exact.
// Stage 2 (token_merge_kernel): one workgroup per request holds every
// candidate in registers, finds the k-th largest key bit by bit with block
// counts, and writes the selection in ascending token order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kIdxDim = 64;
constexpr int kLocalThreads = 256;
constexpr int kLocalUnroll = 8;

template <int NW, int PER>
__device__ __forceinline__ uint32_t block_kth_key(const uint32_t (&kk)[PER], int k, int* scratch,
                                                  int* n_gt) {
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) c += kk[j] >= cand ? 1 : 0;
    if (block_sum<NW>(c, scratch) >= k) T = cand;
  }
  int c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) c += kk[j] > T ? 1 : 0;
  *n_gt = block_sum<NW>(c, scratch);
  return T;
}

// Emits, in the order (tile j, thread) = ascending candidate index, every key
// above T and the first (k - n_gt) keys equal to T. Calls put(pos, j) for
// each taken candidate.
template <int NW, int PER, typename Put>
__device__ __forceinline__ void block_emit(const uint32_t (&kk)[PER], uint32_t T, int k, int n_gt,
                                           int* scratch, Put put) {
  const int need_eq = k - n_gt;
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool gt = kk[j] > T;
    const bool eq = kk[j] == T;
    int tot;
    const int ex = block_exclusive_scan<NW>((gt ? 1 : 0) | (eq ? 0x10000 : 0), scratch, &tot);
    const int gt_before = ex & 0xffff, eq_before = ex >> 16;
    const int eq_room = max(0, need_eq - eq_seen);
    const bool take = gt || (eq && eq_before < eq_room);
    if (take) put(base + gt_before + min(eq_before, eq_room), j);
    base += (tot & 0xffff) + min(tot >> 16, eq_room);
    eq_seen += tot >> 16;
  }
}

template <typename T>
__global__ __launch_bounds__(kLocalThreads) void token_local_kernel(TokenSelectParams p) {
  constexpr int NW = kLocalThreads / kWave;
  constexpr int PER = kTokChunk / kLocalThreads;
  __shared__ uint32_t keys[kTokChunk];
  __shared__ int scratch[NW];
  const int b = blockIdx.y, ch = blockIdx.x;
  const int start = ch * kTokChunk;
  const int n = min(kTokChunk, p.N - start);
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int e = lane & 7, tq = lane >> 3;

  float qf[8];
  load8(static_cast<const T*>(p.q_idx) + static_cast<long long>(b) * kIdxDim + e * 8, qf);
  const T* kb = static_cast<const T*>(p.k_idx) + (static_cast<long long>(b) * p.N + start) * kIdxDim + e * 8;
  for (int iw = wave * 8; iw < n; iw += NW * 8 * kLocalUnroll) {
    Raw8<T> raw[kLocalUnroll];
#pragma unroll
    for (int u = 0; u < kLocalUnroll; ++u) {
      const int i = min(iw + u * NW * 8 + tq, n - 1);  // clamped: straight-line loads
      raw[u].load_stream(kb + static_cast<long long>(i) * kIdxDim);
    }
#pragma unroll
    for (int u = 0; u < kLocalUnroll; ++u) {
      const int i = iw + u * NW * 8 + tq;
      float x[8];
      raw[u].widen(x);
      const float sc = group8_sum(dot8(qf, x));
      if (e == 0 && i < n) keys[i] = order_key(sc);
    }
  }
  __syncthreads();

  const long long cbase = (static_cast<long long>(b) * p.nchunk + ch) * p.k;
  if (n <= p.k) {
    for (int i = tid; i < n; i += kLocalThreads) {
      p.cand_key[cbase + i] = keys[i];
      p.cand_id[cbase + i] = start + i;
    }
    return;
  }
  uint32_t kk[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kLocalThreads + tid;
    kk[j] = i < n ? keys[i] : 0u;
  }
  int n_gt;
  const uint32_t Tk = block_kth_key<NW, PER>(kk, p.k, scratch, &n_gt);
  block_emit<NW, PER>(kk, Tk, p.k, n_gt, scratch, [&](int pos, int j) {
    p.cand_key[cbase + pos] = kk[j];
    p.cand_id[cbase + pos] = start + j * kLocalThreads + tid;
  });
}

template <int PER>
__global__ __launch_bounds__(kMergeThreads) void token_merge_kernel(TokenSelectParams p) {
  constexpr int NW = kMergeThreads / kWave;
  __shared__ int scratch[NW];
  const int b = blockIdx.x, tid = threadIdx.x;
  const long long P = static_cast<long long>(p.nchunk) * p.k;
  const uint32_t* ck = p.cand_key + b * P;
  const int32_t* ci = p.cand_id + b * P;
  uint32_t kk[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const long long L = static_cast<long long>(j) * kMergeThreads + tid;
    bool valid = L < P;
    if (valid) {
      const int chunk = static_cast<int>(L / p.k), i = static_cast<int>(L % p.k);
      valid = i < min(p.k, p.N - chunk * kTokChunk);
    }
    kk[j] = valid ? ck[L] : 0u;
  }
  int n_gt;
  const uint32_t Tk = block_kth_key<NW, PER>(kk, p.k, scratch, &n_gt);
  int32_t* sel = p.sel + static_cast<long long>(b) * p.k;
  block_emit<NW, PER>(kk, Tk, p.k, n_gt, scratch, [&](int pos, int j) {
    sel[pos] = ci[static_cast<long long>(j) * kMergeThreads + tid];
  });
}

template <typename T>
static hipError_t token_select_typed(const TokenSelectParams& p, hipStream_t s) {
  hipLaunchKernelGGL(token_local_kernel<T>, dim3(p.nchunk, p.B), dim3(kLocalThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long P = static_cast<long long>(p.nchunk) * p.k;
  const int per = static_cast<int>((P + kMergeThreads - 1) / kMergeThreads);
  const dim3 grid(p.B), block(kMergeThreads);
  if (per <= 8) hipLaunchKernelGGL(token_merge_kernel<8>, grid, block, 0, s, p);
  else if (per <= 16) hipLaunchKernelGGL(token_merge_kernel<16>, grid, block, 0, s, p);
  else if (per <= 32) hipLaunchKernelGGL(token_merge_kernel<32>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(token_merge_kernel<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_token_select(const TokenSelectParams& p, int dtype, hipStream_t s) {
  return dtype == kBF16 ? token_select_typed<bf16_t>(p, s) : token_select_typed<float>(p, s);
}

}  // namespace tsa
