// Fused RESOLVE step of the HiSparse-style hot cache for gfx950
// ("KV卸载上主机:HiSparse、PDD与DDR4回收", paper analysis 1: hit detection, LRU
// replacement, metadata update and host fetch in one kernel; the authoritative
// KV stays in pinned host memory, HBM holds S slots per request per layer).
//
// One workgroup of 1024 threads per request:
//   1. every slot gets a 64-bit key (policy word) << 32 | slot in LDS; under
//      LRU the policy word is last_use + 1, so free slots (last_use = -1)
//      get the smallest keys;
//   2. selected tokens look up the page table; hit slots get the largest
//      policy word, which sorts them after every evictable slot;
//   3. misses are ranked in selection order (block prefix sums);
//   4. a bitonic sort of the keys in LDS orders the slots by
//      (policy word, slot); the r-th miss takes the r-th slot;
//   5. page table, slot owners and stamps are updated in place;
//   6. the missed tokens' K and V rows (all KV heads, contiguous in the host
//      copy) are read straight from host-mapped memory and stored into the
//      slots, one wave per missed token, 16 B per lane.
// Token ids outside [0, N) are ignored (slot -1) so a bad selection cannot
// address memory outside the tables.
//
// Replacement policies (the analysis compares LRU with FIFO, random and the
// offline Belady policy by miss rate) differ only in the high word of the
// slot key: LRU the last use, FIFO the fetch step (hits keep their stamp),
// random a SplitMix64 key of (seed, request, step, slot) (Steele, Lea and
// Flood, OOPSLA 2014), priority the complement of a caller-given per-token
// value (Belady: the step of the token's next selection). Free slots sort
// first and the step's hits last under every policy.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kResolveThreads = 1024;
constexpr int kResolvePer = kMaxTokenK / kResolveThreads;  // selected tokens per thread

__device__ __forceinline__ unsigned long long splitmix64(unsigned long long x) {
  unsigned long long z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// 31-bit key chained over (seed, request, step, slot).
__device__ __forceinline__ uint32_t random_key(unsigned long long seed, int b, int step, int slot) {
  unsigned long long x = splitmix64(seed);
  x = splitmix64(x + static_cast<unsigned long long>(b));
  x = splitmix64(x + static_cast<unsigned long long>(static_cast<uint32_t>(step)));
  x = splitmix64(x + static_cast<unsigned long long>(slot));
  return static_cast<uint32_t>(x >> 33);
}

// Fetch of one request's missed tokens: one wave per token (waves w0,
// w0 + wstride, ...); lanes stride over its 16-B chunks, K and V rows loaded
// together so each lane keeps four 16-B host reads in flight.
__device__ __forceinline__ void fetch_missed(const int32_t* mtok, const int32_t* mslot, int n_miss, int b, int N,
                                             int S, long long row_bytes, const void* host_k, const void* host_v,
                                             void* pool_k, void* pool_v, int w0, int wstride) {
  const int chunks = static_cast<int>(row_bytes / 16);
  const int lane = lane_id();
  const char* hk = static_cast<const char*>(host_k);
  const char* hv = static_cast<const char*>(host_v);
  char* pk = static_cast<char*>(pool_k);
  char* pv = static_cast<char*>(pool_v);
  for (int r = w0; r < n_miss; r += wstride) {
    const int tk = mtok[r], sl = mslot[r];
    if (tk < 0 || tk >= N || sl < 0 || sl >= S) continue;  // never addresses outside the arrays
    const long long src = (static_cast<long long>(b) * N + tk) * row_bytes;
    const long long dst = (static_cast<long long>(b) * S + sl) * row_bytes;
    const uint4* sk4 = reinterpret_cast<const uint4*>(hk + src);
    const uint4* sv4 = reinterpret_cast<const uint4*>(hv + src);
    uint4* dk4 = reinterpret_cast<uint4*>(pk + dst);
    uint4* dv4 = reinterpret_cast<uint4*>(pv + dst);
    for (int c = lane; c < chunks; c += 2 * kWave) {
      const bool two = c + kWave < chunks;
      const uint4 k0 = sk4[c], v0 = sv4[c];
      uint4 k1 = k0, v1 = v0;
      if (two) {
        k1 = sk4[c + kWave];
        v1 = sv4[c + kWave];
      }
      dk4[c] = k0;
      dv4[c] = v0;
      if (two) {
        dk4[c + kWave] = k1;
        dv4[c + kWave] = v1;
      }
    }
  }
}

__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(ResolveParams p, int spow2) {
  constexpr int NW = kResolveThreads / kWave;
  extern __shared__ unsigned long long lds[];
  unsigned long long* sk = lds;                                   // [spow2]
  int32_t* miss_tok = reinterpret_cast<int32_t*>(lds + spow2);     // [k]
  int32_t* miss_slot = miss_tok + p.k;                            // [k]
  __shared__ int scratch[NW];
  const int b = blockIdx.x, tid = threadIdx.x;
  int32_t* pt = p.page_table + static_cast<long long>(b) * p.N;
  int32_t* st = p.slot_token + static_cast<long long>(b) * p.S;
  int32_t* lu = p.last_use + static_cast<long long>(b) * p.S;
  const int32_t* sel = p.sel + static_cast<long long>(b) * p.k;
  const unsigned long long hit_key = 0xFFFFFFFFull << 32;  // after every evictable slot

  for (int s = tid; s < spow2; s += kResolveThreads) {
    unsigned long long key = ~0ull;
    if (s < p.S) {
      uint32_t hi;
      if (p.policy == kEvictLru || p.policy == kEvictFifo) {
        hi = static_cast<uint32_t>(lu[s] + 1);  // free slots carry -1
      } else {
        const int t = st[s];
        if (t < 0 || t >= p.N) {
          hi = 0;  // free
        } else if (p.policy == kEvictRandom) {
          hi = 1u + random_key(p.seed, b, p.step, s);
        } else {
          const int pr = min(max(p.priority[static_cast<long long>(b) * p.N + t], 0), 0x7FFFFFFF);
          hi = 1u + static_cast<uint32_t>(0x7FFFFFFF - pr);
        }
      }
      key = (static_cast<unsigned long long>(hi) << 32) | static_cast<uint32_t>(s);
    }
    sk[s] = key;
  }
  __syncthreads();

  int tok[kResolvePer], slot[kResolvePer];
#pragma unroll
  for (int j = 0; j < kResolvePer; ++j) {
    const int i = tid + j * kResolveThreads;
    tok[j] = -1;
    slot[j] = -1;
    if (i < p.k) {
      const int t = sel[i];
      if (t >= 0 && t < p.N) {
        tok[j] = t;
        const int sl = pt[t];
        slot[j] = (sl >= 0 && sl < p.S) ? sl : -1;  // a corrupt entry counts as absent
        if (slot[j] >= 0) sk[slot[j]] = hit_key | static_cast<uint32_t>(slot[j]);
      }
    }
  }
  int rank[kResolvePer];
  int n_miss = 0, n_hit = 0;
#pragma unroll
  for (int j = 0; j < kResolvePer; ++j) {
    const bool miss = tok[j] >= 0 && slot[j] < 0;
    int tot;
    rank[j] = n_miss + block_exclusive_scan<NW>(miss ? 1 : 0, scratch, &tot);
    n_miss += tot;
    n_hit += block_sum<NW>(tok[j] >= 0 && slot[j] >= 0 ? 1 : 0, scratch);
  }
  __syncthreads();

  for (int size = 2; size <= spow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (spow2 >> 1); i += kResolveThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool ascending = (lo & size) == 0;
        const unsigned long long a = sk[lo], c = sk[hi];
        if ((a > c) == ascending) {
          sk[lo] = c;
          sk[hi] = a;
        }
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int j = 0; j < kResolvePer; ++j) {
    const int i = tid + j * kResolveThreads;
    if (tok[j] < 0) {
      if (i < p.k) p.slots_out[static_cast<long long>(b) * p.k + i] = -1;
      continue;
    }
    if (slot[j] >= 0) {
      if (p.policy != kEvictFifo) lu[slot[j]] = p.step;  // FIFO keeps the fetch step
    } else {
      const int v = static_cast<int>(sk[rank[j]] & 0xffffffffu);
      const int old = st[v];
      if (old >= 0 && old < p.N) pt[old] = -1;
      pt[tok[j]] = v;
      st[v] = tok[j];
      lu[v] = p.step;
      slot[j] = v;
      miss_tok[rank[j]] = tok[j];
      miss_slot[rank[j]] = v;
    }
    p.slots_out[static_cast<long long>(b) * p.k + i] = slot[j];
  }
  if (tid == 0) {
    if (p.hits) p.hits[b] = n_hit;
    if (p.misses) p.misses[b] = n_miss;
  }
  __syncthreads();

  if (p.miss_tok) {  // the miss list, for the other layers of a layer group
    for (int r = tid; r < n_miss; r += kResolveThreads) {
      p.miss_tok[static_cast<long long>(b) * p.k + r] = miss_tok[r];
      p.miss_slot[static_cast<long long>(b) * p.k + r] = miss_slot[r];
    }
  }
  fetch_missed(miss_tok, miss_slot, n_miss, b, p.N, p.S, p.row_bytes, p.host_k, p.host_v, p.pool_k, p.pool_v,
               tid / kWave, kResolveThreads / kWave);
}

// grid (B, layers, split): workgroup z of (request, layer) takes every
// split-th wave's share of the request's misses
constexpr int kFetchThreads = 1024;
__global__ __launch_bounds__(kFetchThreads) void fetch_rows_kernel(FetchParams p) {
  constexpr int NW = kFetchThreads / kWave;
  const int b = blockIdx.x, layer = blockIdx.y, z = blockIdx.z;
  const int n = min(max(p.misses[b], 0), p.k);
  fetch_missed(p.miss_tok + static_cast<long long>(b) * p.k, p.miss_slot + static_cast<long long>(b) * p.k, n, b,
               p.N, p.S, p.row_bytes, p.host_k[layer], p.host_v[layer], p.pool_k[layer], p.pool_v[layer],
               z * NW + static_cast<int>(threadIdx.x) / kWave, p.split * NW);
}

hipError_t launch_fetch_rows(const FetchParams& p, hipStream_t s) {
  hipLaunchKernelGGL(fetch_rows_kernel, dim3(p.B, p.n_layers, p.split), dim3(kFetchThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_resolve(const ResolveParams& p, hipStream_t s) {
  int spow2 = 1;
  while (spow2 < p.S) spow2 <<= 1;
  const size_t lds = static_cast<size_t>(spow2) * sizeof(unsigned long long) +
                     2 * static_cast<size_t>(p.k) * sizeof(int32_t);
  hipLaunchKernelGGL(resolve_kernel, dim3(p.B), dim3(kResolveThreads), lds, s, p, spow2);
  return hipGetLastError();
}

}  // namespace tsa
