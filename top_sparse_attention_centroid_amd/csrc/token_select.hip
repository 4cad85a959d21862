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
// candidate in registers and selects the top-k among them.
// Both stages find the k-th largest key with an exact 8-bit radix select
// (four passes over per-wave LDS histograms) and emit in ascending index
// order from per-(tile, wave) ballot counts.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kIdxDim = 64;
constexpr int kLocalThreads = 256;
constexpr int kLocalUnroll = 8;

// In-place exclusive prefix sum of n ints in LDS by the calling wave
// (each lane scans a contiguous run, then the lane totals are scanned).
__device__ __forceinline__ void wave_exclusive_scan_lds(int* a, int n) {
  const int lane = lane_id();
  const int per = (n + kWave - 1) / kWave;
  const int lo = min(lane * per, n), hi = min(lo + per, n);
  int run = 0;
  for (int i = lo; i < hi; ++i) run += a[i];
  int x = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  int acc = x - run;
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = acc;
    acc += v;
  }
}

// The k-th largest of the valid keys held by a block (thread t holds the
// keys of indices j * (NW * 64) + t; bit j of vmask marks key j valid): an exact
// MSB-first radix select, 8 bits per pass, over per-wave LDS histograms
// (hist: NW * 256 ints; misc: 2 ints). Returns the key T and sets *need_eq
// to how many keys equal to T belong to the top k.
template <int NW, int PER>
__device__ __forceinline__ uint32_t block_radix_kth(const uint32_t (&kk)[PER], uint64_t vmask, int k, int* hist,
                                                    int* misc, int* need_eq) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < NW * 256; i += NW * kWave) hist[i] = 0;
    __syncthreads();
    int* wh = hist + wave * 256;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (((vmask >> j) & 1u) && (kk[j] & pmask) == prefix) atomicAdd(&wh[(kk[j] >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      int c[4], t = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = 0;
        for (int w = 0; w < NW; ++w) c[q] += hist[w * 256 + lane * 4 + q];
        t += c[q];
      }
      // suffix sum over lanes above this one
      int x = t;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_down(x, o);
        if (lane + o < kWave) x += y;
      }
      int above = x - t;  // keys in bins of higher lanes
      int best = -1, best_above = 0;
#pragma unroll
      for (int q = 3; q >= 0; --q) {  // bins lane*4+q, descending
        if (best < 0 && above + c[q] >= krem) {
          best = lane * 4 + q;
          best_above = above;
        }
        above += c[q];
      }
      // the digit is the largest bin whose suffix count reaches krem
      int d = best, da = best_above;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int od = __shfl_xor(d, o), oa = __shfl_xor(da, o);
        if (od > d) {
          d = od;
          da = oa;
        }
      }
      if (lane == 0) {
        misc[0] = d;
        misc[1] = krem - da;
      }
    }
    __syncthreads();
    const int d = misc[0];
    krem = misc[1];
    prefix |= static_cast<uint32_t>(d) << shift;
    pmask |= 255u << shift;
  }
  *need_eq = krem;
  return prefix;
}

// Emits, in ascending index order, every valid key above T and the first
// need_eq keys equal to T: put(position, j) for each. Positions come from
// per-(tile, wave) ballot counts and one wave-level scan. cnt: 2 * PER * NW ints.
template <int NW, int PER, typename Put>
__device__ __forceinline__ void block_emit_ordered(const uint32_t (&kk)[PER], uint64_t vmask, uint32_t T, int need_eq,
                                                   int* cnt, Put put) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  int* cgt = cnt;
  int* ceq = cnt + PER * NW;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool v = (vmask >> j) & 1u;
    const uint64_t bgt = __ballot(v && kk[j] > T), beq = __ballot(v && kk[j] == T);
    if (lane == 0) {
      cgt[j * NW + wave] = __popcll(bgt);
      ceq[j * NW + wave] = __popcll(beq);
    }
  }
  __syncthreads();
  if (wave == 0) wave_exclusive_scan_lds(cgt, PER * NW);
  if (wave == (NW > 1 ? 1 : 0)) {
    if (NW == 1) __builtin_amdgcn_wave_barrier();
    wave_exclusive_scan_lds(ceq, PER * NW);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool v = (vmask >> j) & 1u;
    const bool gt = v && kk[j] > T, eq = v && kk[j] == T;
    const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
    const int gt_before = cgt[j * NW + wave] + prefix_count(bgt);
    const int eq_before = ceq[j * NW + wave] + prefix_count(beq);
    if (gt || (eq && eq_before < need_eq)) put(gt_before + min(eq_before, need_eq), j);
  }
}

template <typename T>
__global__ __launch_bounds__(kLocalThreads) void token_local_kernel(TokenSelectParams p) {
  constexpr int NW = kLocalThreads / kWave;
  constexpr int PER = kTokChunk / kLocalThreads;
  __shared__ uint32_t keys[kTokChunk];
  __shared__ int hist[NW * 256];
  __shared__ int cnt[2 * PER * NW];
  __shared__ int misc[2];
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
  uint64_t vmask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = j * kLocalThreads + tid;
    kk[j] = i < n ? keys[i] : 0u;
    vmask |= static_cast<uint64_t>(i < n) << j;
  }
  int need_eq;
  const uint32_t Tk = block_radix_kth<NW, PER>(kk, vmask, p.k, hist, misc, &need_eq);
  block_emit_ordered<NW, PER>(kk, vmask, Tk, need_eq, cnt, [&](int pos, int j) {
    p.cand_key[cbase + pos] = kk[j];
    p.cand_id[cbase + pos] = start + j * kLocalThreads + tid;
  });
}

template <int PER>
__global__ __launch_bounds__(kMergeThreads) void token_merge_kernel(TokenSelectParams p) {
  constexpr int NW = kMergeThreads / kWave;
  __shared__ int hist[NW * 256];
  __shared__ int cnt[2 * PER * NW];
  __shared__ int misc[2];
  const int b = blockIdx.x, tid = threadIdx.x;
  const long long P = static_cast<long long>(p.nchunk) * p.k;
  const uint32_t* ck = p.cand_key + b * P;
  const int32_t* ci = p.cand_id + b * P;
  // candidate L = chunk * k + i is real when i < min(k, tokens in the chunk)
  uint32_t kk[PER];
  uint64_t vmask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const long long L = static_cast<long long>(j) * kMergeThreads + tid;
    bool valid = L < P;
    if (valid) {
      const int chunk = static_cast<int>(L / p.k), i = static_cast<int>(L % p.k);
      valid = i < min(p.k, p.N - chunk * kTokChunk);
    }
    kk[j] = valid ? ck[L] : 0u;
    vmask |= static_cast<uint64_t>(valid) << j;
  }
  int need_eq;
  const uint32_t Tk = block_radix_kth<NW, PER>(kk, vmask, p.k, hist, misc, &need_eq);
  int32_t* sel = p.sel + static_cast<long long>(b) * p.k;
  block_emit_ordered<NW, PER>(kk, vmask, Tk, need_eq, cnt, [&](int pos, int j) {
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
  else if (per <= 36) hipLaunchKernelGGL(token_merge_kernel<36>, grid, block, 0, s, p);
  else if (per <= 52) hipLaunchKernelGGL(token_merge_kernel<52>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(token_merge_kernel<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_token_select(const TokenSelectParams& p, int dtype, hipStream_t s) {
  return dtype == kBF16 ? token_select_typed<bf16_t>(p, s) : token_select_typed<float>(p, s);
}

}  // namespace tsa
