// Inverted-index decode with one workgroup per query head (or per share of a
// query head's rows) for small batches ([KARAT] worked example, steps 3-4:
// score the query against the centroids, take the top-k lists, attend over
// their entries; [KARAT] = paper-daily digest "Heterogeneous LLM Serving with
// General-Purpose Processing-Near-Memory for Retrieval-Based Sparse
// Attention").
//
// With few (request, KV head) groups the plan-based path (scoring, select +
// plan, gather, combine) is a chain of launches each bound by the latency of
// a few waves, and its select workgroup per group serialises the selection,
// the plan and its writes. Here the selection moves into the workgroups that
// attend:
//  1. (fused) the workgroup scores the KV group's codebook for every head of
//     the group (MFMA for bf16, vector units for fp32) into LDS as order
//     keys, next to the group's list offsets (and lengths), every load in
//     flight together. (split) the scores come from centroid_score_kernel,
//     launched before: with one CU reading some 40 GB/s, a codebook of a few
//     hundred KiB is read fastest spread over many workgroups.
//  2. a wave selects its head's top-k lists with the same code as the
//     plan-based path (so the same lists). The workgroup that writes the
//     group's union count (head 0; share 0) selects every head of the group.
//  3. the head's rows (the entries of its k lists, in list order; with
//     split, share s of S of them) are dealt to the waves a batch at a time:
//     a lane finds its row's list by a binary search over the k list starts
//     held one per lane, loads the row id, and the wave streams the K/V rows
//     (16 lanes per row, all loads of the batch in flight) into an online
//     softmax per lane group;
//  4. the lane groups merge by shuffles, the waves through LDS; fused: wave 0
//     writes o / l (zero when no row was selected); split: it writes the
//     share's partial state as record h * S + s of the group and counts in,
//     and the head's last share to count in merges its S records.
#include <type_traits>

#include "attn_rows.hpp"
#include "device_common.hpp"
#include "kernels.hpp"
#include "select_common.hpp"

namespace tsa {

// rows per lane group per batch: 4 (16 rows a wave), in bf16 and fp32 alike.
// A split share gives each wave about 16 rows, and 4-row batches measured
// faster than 8-row ones at one 100K-token request (about 0.2 us a step).
template <typename T>
constexpr int head_unroll() { return kGatherUnroll / 2; }

// Split decode, end of a share (wave 0 holding the share's merged state):
// the state goes out with agent-scope stores, which write through the XCD's
// L2, and once the wave has seen them complete it counts in on the head's
// arrival counter. The share that counts in last gets true and merges the
// head. No L2 write-back is needed, since every word of a record is written
// and read at agent scope; the counters are cleared by centroid_score_kernel,
// launched before in the same stream.
__device__ __forceinline__ bool publish_share(float* rec, const HeadState& st, int r, int e, uint32_t* arrive,
                                              int S) {
  store_state(rec, st, r, e, true);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t n = 0;
  if (lane_id() == 0) n = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __shfl(static_cast<int>(n), 0) == S - 1;
}

// The head's S records (rec0 + s * stride, s ascending) merged with the
// log-sum-exp rule, o / l written to out[128] (zero when nothing was
// selected). One wave, lane l holding o[2l], o[2l + 1]; eight records'
// words requested before the first wait, all read at agent scope.
__device__ __forceinline__ void merge_shares(const float* rec0, int S, long long stride, float* out) {
  constexpr int kU = 8;
  const int lane = lane_id();
  auto ld = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  float M = kEmptyMax, L = 0.f, O0 = 0.f, O1 = 0.f;
  for (int s0 = 0; s0 < S; s0 += kU) {
    float m[kU], l[kU], o0[kU], o1[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float* ph = rec0 + min(s0 + u, S - 1) * stride;  // clamped: straight-line loads
      m[u] = ld(ph);
      l[u] = ld(ph + 1);
      o0[u] = ld(ph + kPartO + lane * 2);
      o1[u] = ld(ph + kPartO + lane * 2 + 1);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (s0 + u >= S) break;
      const float Mn = fmaxf(M, m[u]);
      const float a = fast_exp2(M - Mn), w = fast_exp2(m[u] - Mn);
      L = L * a + l[u] * w;
      O0 = O0 * a + o0[u] * w;
      O1 = O1 * a + o1[u] * w;
      M = Mn;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float2*>(out + lane * 2) = make_float2(O0 * inv, O1 * inv);
}

template <typename T, int G, int KPL, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * kWave) void ivf_head_kernel(HeadDecodeParams p) {
  constexpr int NT = NW * kWave;
  constexpr int U = head_unroll<T>();
  constexpr int BR = 4 * U;         // rows per wave per batch
  constexpr int CM = KPL * kWave;   // lists the workgroup holds
  static_assert(BR <= kWave, "a batch's row ids are one per lane");
  __shared__ uint32_t keys[SPLIT ? 1 : G * CM];
  __shared__ uint32_t lmask[CM];
  __shared__ int loff[CM + 1];
  __shared__ int llen[CM];
  // candidate scratch of the selecting waves (0 .. min(NW, G) - 1)
  constexpr int NSEL = NW < G ? NW : G;
  __shared__ __align__(16) uint64_t cand_lds[NSEL][2 * kWave];
  __shared__ int sel_lds[kWave];
  __shared__ int ids_lds[NW][kWave];
  __shared__ float st_lds[NW][2 + kHeadDim];
  __shared__ int scratch[NW];
  const SelectParams& sp = p.s;
  const int C = sp.C, k = sp.k;
  const int S = SPLIT ? p.S : 1;
  const int bh = SPLIT ? blockIdx.x / S : blockIdx.x;
  const int share = SPLIT ? blockIdx.x % S : 0;
  const int b = bh / p.Hq, qh = bh % p.Hq;
  const int g = qh / G, h = qh % G;
  const int bg = b * sp.Hkv + g;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = lane >> 4, e = lane & 15;
  // the workgroup that writes the group's union count selects every head
  const bool all_heads = h == 0 && share == 0 && sp.uniq_out != nullptr;

  // 1. the group's list offsets (and lengths) into registers, then the scores
  const int32_t* off = sp.offsets + static_cast<long long>(bg) * (C + 1);
  const int32_t* lens = sp.lens ? sp.lens + static_cast<long long>(bg) * C : nullptr;
  constexpr int kOffPer = (CM + NT) / NT;  // C + 1 <= CM + 1 offsets
  int offv[kOffPer], lenv[kOffPer];
#pragma unroll
  for (int i = 0; i < kOffPer; ++i) offv[i] = off[min(tid + i * NT, C)];
  if (lens) {
#pragma unroll
    for (int i = 0; i < kOffPer; ++i) lenv[i] = lens[min(tid + i * NT, C - 1)];
  }
  for (int c = tid; c < C; c += NT) lmask[c] = 0u;
  const uint32_t* kg;  // [G][C] order keys of the group
  if constexpr (SPLIT) {
    kg = sp.keys + static_cast<long long>(bg) * G * C;
  } else {
    kg = keys;
    if constexpr (std::is_same<T, bf16_t>::value) {
      // CM / 16 <= 64 tiles over the waves, at most 4 per wave at 16 waves
      const int ntile = (C + 15) / 16;
      const int per_wave = (ntile + NW - 1) / NW;
      score_tiles_mfma<G, 4>(sp, b, g, wave * per_wave, min(ntile, (wave + 1) * per_wave), keys);
    } else {
      score_rows_valu<T, G, NW, 4>(sp, b, g, wave, keys);
    }
  }
  // the selecting waves' keys (split: straight from the scores in memory)
  uint32_t kk[(G + NW - 1) / NW][KPL];
  auto head_of = [&](int i) { return all_heads ? wave + i * NW : h; };
  auto selects = [&](int i) { return all_heads ? wave + i * NW < G : (wave == 0 && i == 0); };
  auto load_keys = [&] {
#pragma unroll
    for (int i = 0; i < (G + NW - 1) / NW; ++i) {
      if (!selects(i)) continue;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int c = j * kWave + lane;
        kk[i][j] = c < C ? kg[head_of(i) * C + min(c, C - 1)] : 0u;
      }
    }
  };
  if constexpr (SPLIT) load_keys();
#pragma unroll
  for (int i = 0; i < kOffPer; ++i) {
    const int c = tid + i * NT;
    if (c <= C) loff[c] = min(max(offv[i], 0), sp.n_entries);
    if (lens && c < C) llen[c] = lenv[i];
  }
  __syncthreads();
  if constexpr (!SPLIT) load_keys();
  // rows of list c: its whole range, or (dynamic index) the valid front part
  auto list_len = [&](int c) {
    const int range = max(loff[c + 1] - loff[c], 0);
    return lens ? min(max(llen[c], 0), range) : range;
  };

  // 2. top-k lists
#pragma unroll
  for (int i = 0; i < (G + NW - 1) / NW; ++i) {
    if (!selects(i)) continue;
    const int hw = head_of(i);
    topk_lists<KPL>(kk[i], k, cand_lds[wave], [&](int c, int pos) {
      atomicOr(&lmask[c], 1u << hw);
      if (hw == h) sel_lds[pos] = c;
    });
  }
  __syncthreads();

  // 3. the head's lists, lane i < k holding list i (ascending order): its
  // first entry and the head's rows before it
  int st_i = 0, len_i = 0;
  if (lane < k) {
    const int c = sel_lds[lane];
    st_i = loff[c];
    len_i = list_len(c);
  }
  const int incl = wave_inclusive_scan(len_i);
  const int pre_i = incl - len_i;
  const int R = __shfl(incl, kWave - 1);
  if (share == 0 && wave == 0) {  // the head's lists and row count (share 0 writes them)
    if (sp.sel_out && lane < k) sp.sel_out[(static_cast<long long>(b) * p.Hq + qh) * k + lane] = sel_lds[lane];
    if (sp.rows_out && lane == 0) sp.rows_out[static_cast<long long>(b) * p.Hq + qh] = R;
  }
  if (all_heads) {  // uniform over the workgroup
    int u = 0;
    for (int c = tid; c < C; c += NT) u += lmask[c] ? list_len(c) : 0;
    u = block_sum<NW>(u, scratch);
    if (tid == 0) sp.uniq_out[bg] = u;
  }
  // this workgroup's rows [r0, r1) of the head
  const int r0 = static_cast<int>(static_cast<long long>(R) * share / S);
  const int r1 = static_cast<int>(static_cast<long long>(R) * (share + 1) / S);

  // rows come from the list-major copies by entry when given, else from the
  // caches by the entry's token id
  const bool by_entry = p.kl != nullptr;
  const long long ebase = (static_cast<long long>(b) * sp.Hkv + g) * sp.n_entries;  // first entry of the group
  const long long row_stride = by_entry ? kHeadDim : static_cast<long long>(sp.Hkv) * kHeadDim;
  const T* kb = by_entry ? static_cast<const T*>(p.kl) + ebase * kHeadDim + e * 8
                         : static_cast<const T*>(p.k) + static_cast<long long>(b) * sp.N * row_stride + g * kHeadDim +
                               e * 8;
  const T* vb = by_entry ? static_cast<const T*>(p.vl) + ebase * kHeadDim + e * 8
                         : static_cast<const T*>(p.v) + static_cast<long long>(b) * sp.N * row_stride + g * kHeadDim +
                               e * 8;
  const int32_t* rid = p.ids + ebase;
  QFrag<T> qf;
  qf.load(static_cast<const T*>(sp.q) + (static_cast<long long>(b) * p.Hq + qh) * kHeadDim + e * 8);
  HeadState st;
  st.init();
  int* wid = ids_lds[wave];
  for (int base = r0 + wave * BR; base < r1; base += NT / kWave * BR) {
    // row t of this lane (clamped to a row of the share): its list is the
    // last list i < k whose first row pre_i is <= t (an empty list shares
    // its pre with the next one, so the last such list holds t)
    const int t = min(base + lane, r1 - 1);
    int li = 0;
#pragma unroll
    for (int step = kWave / 2; step > 0; step >>= 1) {
      const int cand = li + step;  // <= 63
      const int pc = __shfl(pre_i, cand);
      if (cand < k && pc <= t) li = cand;
    }
    const int s0 = __shfl(st_i, li), p0 = __shfl(pre_i, li);
    const int ent = s0 + (t - p0);
    const int id = by_entry ? ent : rid[ent];
    // ids outside [0, N) (entries outside [0, n_entries)) are skipped, never
    // dereferenced
    const bool ok = lane < BR && base + lane < r1 &&
                    static_cast<unsigned>(id) < static_cast<unsigned>(by_entry ? sp.n_entries : sp.N);
    wid[lane] = ok ? id : -1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    Batch<T, U> bt;
    issue_batch<kGatherStream>(bt, wid, 0, min(BR, r1 - base), r, kb, vb, row_stride);
    consume_batch(bt, st, qf, p.qscale);
    __builtin_amdgcn_wave_barrier();  // the next batch overwrites wid
  }

  // 4. merge: lane groups by shuffles, then the waves through LDS
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
    float o2[8];
    const float m2 = __shfl_xor(st.m, x);
    const float l2 = __shfl_xor(st.l, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) o2[i] = __shfl_xor(st.o[i], x);
    merge_into(st, m2, l2, o2);
  }
  if constexpr (NW > 1) {
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) st_lds[wave][2 + e * 8 + i] = st.o[i];
      if (e == 0) {
        st_lds[wave][0] = st.m;
        st_lds[wave][1] = st.l;
      }
    }
    __syncthreads();
    if (wave != 0) return;
    // every lane group of wave 0 folds the other waves' states into its own
    for (int w = 1; w < NW; ++w) {
      float o2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) o2[i] = st_lds[w][2 + e * 8 + i];
      merge_into(st, st_lds[w][0], st_lds[w][1], o2);
    }
  }
  if constexpr (SPLIT) {
    const long long stride = static_cast<long long>(G) * kPartStride;  // floats between records
    float* rec0 = p.partial + (static_cast<long long>(bg) * sp.smax + h * S) * stride + h * kPartStride;
    const bool last = publish_share(rec0 + share * stride, st, r, e, sp.arrive_heads + bh, S);
    if (last) merge_shares(rec0, S, stride, p.out + (static_cast<long long>(b) * p.Hq + qh) * kHeadDim);
  } else {
    if (r == 0) {
      const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
      float* o = p.out + (static_cast<long long>(b) * p.Hq + qh) * kHeadDim + e * 8;
      *reinterpret_cast<float4*>(o) = make_float4(st.o[0] * inv, st.o[1] * inv, st.o[2] * inv, st.o[3] * inv);
      *reinterpret_cast<float4*>(o + 4) = make_float4(st.o[4] * inv, st.o[5] * inv, st.o[6] * inv, st.o[7] * inv);
    }
  }
}

template <typename T, int G, int NW, bool SPLIT>
static void head_dispatch_g(const HeadDecodeParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.s.B * p.Hq * (SPLIT ? p.S : 1))), block(NW * kWave);
  if (p.s.C <= 64) hipLaunchKernelGGL((ivf_head_kernel<T, G, 1, NW, SPLIT>), grid, block, 0, s, p);
  else if (p.s.C <= 256) hipLaunchKernelGGL((ivf_head_kernel<T, G, 4, NW, SPLIT>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((ivf_head_kernel<T, G, kHeadMaxC / 64, NW, SPLIT>), grid, block, 0, s, p);
}

template <typename T, int NW, bool SPLIT>
static void head_dispatch(const HeadDecodeParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: head_dispatch_g<T, 1, NW, SPLIT>(p, s); break;
    case 2: head_dispatch_g<T, 2, NW, SPLIT>(p, s); break;
    case 4: head_dispatch_g<T, 4, NW, SPLIT>(p, s); break;
    default: head_dispatch_g<T, 8, NW, SPLIT>(p, s); break;
  }
}

hipError_t launch_fused_decode(const HeadDecodeParams& p, int dtype, int G, hipStream_t s) {
  if (dtype == kBF16) head_dispatch<bf16_t, kFusedWaves, false>(p, G, s);
  else head_dispatch<float, kFusedWaves, false>(p, G, s);
  return hipGetLastError();
}

hipError_t launch_split_decode(const HeadDecodeParams& p, int G, hipStream_t s) {
  head_dispatch<bf16_t, kSplitWaves, true>(p, G, s);
  return hipGetLastError();
}

}  // namespace tsa
