// Centroid scoring and per-head top-k list selection, shared by the select
// kernel (one workgroup per (request, KV head), followed by the gather) and
// the fused small-batch decode (one workgroup per query head).
//
// [KARAT] = paper-daily digest "Heterogeneous LLM Serving with General-Purpose
// Processing-Near-Memory for Retrieval-Based Sparse Attention".
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

// Scores of one KV group as a dense contraction on matrix cores: 16x16x32
// bf16 MFMAs, fp32 accumulation. The A operand holds the group's query heads
// in rows 0..G-1 (rows G..15 repeat head G-1 and are dropped); each
// 16-centroid B tile is read straight from memory, since every centroid row
// is used once per group. The calling wave scores tiles [t_begin, t_end),
// kSelTiles of them in flight. Lane l of a result tile holds centroid l % 16
// for heads (l / 16) * 4 .. +4; the order key of s[h][c] goes to
// keys[h * C + c]. Cosine scaling divides by |c|, summed from the same B
// fragments (each lane squares 32 of the row's elements; the four lanes of a
// column add theirs).
constexpr int kSelTiles = 8;

template <int G, int TILES = kSelTiles>
__device__ __forceinline__ void score_tiles_mfma(const SelectParams& p, int b, int g, int t_begin, int t_end,
                                                 uint32_t* keys) {
  const int C = p.C;
  const int lane = lane_id(), col = lane & 15, grp = lane >> 4;
  const bf16_t* qr = static_cast<const bf16_t*>(p.q) + (static_cast<long long>(b) * p.Hkv + g) * G * kHeadDim +
                     min(col, G - 1) * kHeadDim + grp * 8;
  bf16x8_t a[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) a[ks] = *reinterpret_cast<const bf16x8_t*>(qr + ks * 32);
  const bf16_t* cb = static_cast<const bf16_t*>(p.centroids) + b * p.cent_bstride +
                     static_cast<long long>(g) * C * kHeadDim + grp * 8;
  for (int t0 = t_begin; t0 < t_end; t0 += TILES) {
    bf16x8_t bt[TILES][4];
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
      if (t0 + u < t_end) {
        const bf16_t* row = cb + static_cast<long long>(min((t0 + u) * 16 + col, C - 1)) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) bt[u][ks] = *reinterpret_cast<const bf16x8_t*>(row + ks * 32);
      }
    }
#pragma unroll
    for (int u = 0; u < TILES; ++u) {
      if (t0 + u >= t_end) break;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], bt[u][ks], acc, 0, 0, 0);
      float inv = 1.f;
      if (p.cosine) {  // q.c / |c| (1/|q| ranks nothing differently)
        float n2 = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          Raw8<bf16_t> r;
          r.v = __builtin_bit_cast(uint4, bt[u][ks]);
          n2 += sq8(r);
        }
        n2 += __shfl_xor(n2, 16);
        n2 += __shfl_xor(n2, 32);
        inv = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
      }
      const int c = (t0 + u) * 16 + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = grp * 4 + i;
        if (h < G && c < C) keys[h * C + c] = order_key(acc[i] * inv);
      }
    }
  }
}

// The same scores on the vector units (fp32 data, or any dtype): 16 lanes
// per 128-element centroid row (8 elements each) reduced through DPP, four
// rows per wave load, U rows per lane group in flight; wave `wave` of NW
// takes rows wave * 4 + [0, 4) + j * 4 * NW.
template <typename T, int G, int NW, int U>
__device__ __forceinline__ void score_rows_valu(const SelectParams& p, int b, int g, int wave, uint32_t* keys) {
  const int C = p.C;
  const int lane = lane_id(), r = lane >> 4, e = lane & 15;
  const T* qb = static_cast<const T*>(p.q) + (static_cast<long long>(b) * p.Hkv + g) * G * kHeadDim;
  QFrag<T> qf[G];
#pragma unroll
  for (int h = 0; h < G; ++h) qf[h].load(qb + h * kHeadDim + e * 8);
  const T* cb = static_cast<const T*>(p.centroids) + b * p.cent_bstride +
                static_cast<long long>(g) * C * kHeadDim + e * 8;
  for (int c0 = wave * 4; c0 < C; c0 += 4 * NW * U) {
    Raw8<T> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u * 4 * NW + r, C - 1);  // clamped: straight-line loads
      raw[u].load(cb + static_cast<long long>(c) * kHeadDim);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 4 * NW + r;
      float inv = 1.f;
      if (p.cosine) {  // cosine similarity: q.c / |c| (1/|q| ranks nothing differently)
        const float n2 = group16_sum(sq8(raw[u]));
        inv = n2 > 0.f ? 1.f / sqrtf(n2) : 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sc = group16_sum(qf[h].dot(raw[u])) * inv;
        if (e == 0 && c < C) keys[h * C + c] = order_key(sc);
      }
    }
  }
}

// The largest t with count(t) >= k, for a count that does not grow with t
// and count(0) >= k: searched from the most significant bits down, two bits
// a step (the three candidate counts of a step are independent). The steps
// stay a loop, which keeps the kernels that inline it compact.
template <typename Count>
__device__ __forceinline__ uint32_t largest_with_count(int k, Count&& count) {
  uint32_t t = 0;
#pragma unroll 1
  for (int bit = 30; bit >= 0; bit -= 2) {
    const uint32_t c1 = t | (1u << bit), c2 = t | (2u << bit), c3 = t | (3u << bit);
    const int n1 = count(c1), n2 = count(c2), n3 = count(c3);
    t = n3 >= k ? c3 : (n2 >= k ? c2 : (n1 >= k ? c1 : t));
  }
  return t;
}

// Rank of this lane's composite value xc among v[0 .. n) (a wave-private
// LDS array, 16-byte aligned, n <= 64): how many of them are larger. Every
// lane reads the same addresses (broadcast), two values a read.
__device__ __forceinline__ int rank_among(const uint64_t* v, int n, uint64_t xc) {
  int r = 0;
#pragma unroll 4
  for (int j = 0; j < n; j += 2) {
    const ulonglong2 w = *reinterpret_cast<const ulonglong2*>(v + j);
    r += w.x > xc ? 1 : 0;
    r += j + 1 < n && w.y > xc ? 1 : 0;
  }
  return r;
}

// (key, index) as one value that orders by key, then by lower index first
// (index < 2^BITS)
template <int BITS>
__device__ __forceinline__ uint64_t key_rank_value(uint32_t key, int idx) {
  return (static_cast<uint64_t>(key) << BITS) | static_cast<uint64_t>((1 << BITS) - 1 - idx);
}
constexpr int kListBits = 12;  // list ids < kMaxCentroids = 4096
static_assert(kMaxCentroids <= (1 << kListBits), "list ids fit the rank value");

// Top-k lists of one query head ([KARAT] How: the top-k most similar
// lists), run by one wave on the head's order keys held in registers: lane
// holds keys c = j * 64 + lane (ascending c by j), 0 for "no list" (below
// every real key). The k lists with the largest keys are taken, ties to the
// lower list id; take(c, pos) runs on the lane of each taken list c, pos =
// its rank among the taken lists in ascending list order.
//
// With k <= 64 the selection ranks instead of searching: the k-th largest of
// the 64 lane maxima, t1, has at least k keys at or above it, so every key of
// the top k is among the keys >= t1. t1 comes from the ranks of the lane
// maxima among themselves (each lane counts, from LDS broadcast reads, the
// maxima above its own, ties to the lower lane); when at most 64 keys reach
// t1, each lane appends its own, with their lists, to the wave's LDS scratch
// (cl: 128 values, the upper half one spare slot a lane for the keys it
// drops) at its exclusive prefix count, and the candidates are ranked by
// (key, lower list id first). The candidate of rank k - 1 holds the k-th
// largest value T; the lists whose (key, list) value reaches T are taken, in
// ascending list order straight from the keys' own layout (ballot prefix
// counts). Otherwise (or for k > 64) thr, the k-th largest key,
// is searched bit by bit over all keys, keys above it are taken, then keys
// equal to it in ascending list order until k are taken.
template <int KPL, typename Take>
__device__ __forceinline__ void topk_lists(const uint32_t (&kk)[KPL], int k, uint64_t* cl, Take&& take) {
  const int lane = lane_id();
  if (k <= kWave) {
    if constexpr (KPL == 1) {
      // one key a lane, lane = list: rank the keys themselves
      const uint64_t xc = key_rank_value<6>(kk[0], lane);
      cl[lane] = xc;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const bool tk = rank_among(cl, kWave, xc) < k;
      const uint64_t tm = __ballot(tk);
      if (tk) take(lane, prefix_count(tm));
      __builtin_amdgcn_wave_barrier();  // a later call of this wave reuses cl
      return;
    } else {
      uint32_t lmax = kk[0];
#pragma unroll
      for (int j = 1; j < KPL; ++j) lmax = max(lmax, kk[j]);
      const uint64_t mc = key_rank_value<6>(lmax, lane);
      cl[lane] = mc;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint64_t at = __ballot(rank_among(cl, kWave, mc) == k - 1);  // one lane: ranks are distinct
      const uint32_t t1 = static_cast<uint32_t>(__shfl(lmax, static_cast<int>(__builtin_ctzll(at))));
      int n_cand = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) n_cand += __popcll(__ballot(kk[j] >= t1));
      if (n_cand <= kWave) {
        int mine = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) mine += kk[j] >= t1 ? 1 : 0;
        int idx = wave_inclusive_scan(mine) - mine;
        __builtin_amdgcn_wave_barrier();  // every lane has read the maxima
        // straight-line: a key below t1 goes to this lane's spare slot
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const bool in = kk[j] >= t1;
          const int slot = in ? idx : kWave + lane;
          cl[slot] = key_rank_value<kListBits>(kk[j], j * kWave + lane);
          idx += in ? 1 : 0;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint64_t xc = lane < n_cand ? cl[lane] : 0u;
        const int rk = lane < n_cand ? rank_among(cl, n_cand, xc) : kWave;
        // the k-th largest candidate value T (k <= n_cand: the keys >= t1
        // number at least k); the taken lists are those whose value is >= T
        const int at_k = static_cast<int>(__builtin_ctzll(__ballot(rk == k - 1)));  // one lane
        const uint64_t T = (static_cast<uint64_t>(static_cast<uint32_t>(__shfl(static_cast<int>(xc >> 32), at_k)))
                            << 32) |
                           static_cast<uint32_t>(__shfl(static_cast<int>(xc & 0xffffffffu), at_k));
        // emitted from the keys' own layout in ascending list order, placed
        // by ballot prefix counts (values are distinct, so exactly k)
        int base = 0;
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int c = j * kWave + lane;
          const bool tk = key_rank_value<kListBits>(kk[j], c) >= T;
          const uint64_t tm = __ballot(tk);
          if (tk) take(c, base + prefix_count(tm));
          base += __popcll(tm);
        }
        __builtin_amdgcn_wave_barrier();  // a later call of this wave reuses cl
        return;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  const uint32_t thr = largest_with_count(k, [&](uint32_t c) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) cnt += __popcll(__ballot(kk[j] >= c));
    return cnt;
  });
  int n_gt = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) n_gt += __popcll(__ballot(kk[j] > thr));
  const int need_eq = k - n_gt;
  int base = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int c = j * kWave + lane;
    const bool gt = kk[j] > thr;
    const bool eq = kk[j] == thr;
    const uint64_t eqm = __ballot(eq);
    const bool tk = gt || (eq && eq_seen + prefix_count(eqm) < need_eq);
    const uint64_t tm = __ballot(tk);
    if (tk) take(c, base + prefix_count(tm));
    base += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
}

}  // namespace tsa
