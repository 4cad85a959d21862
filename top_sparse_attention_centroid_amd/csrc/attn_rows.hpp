// Gathered rows scored against one query head with an online softmax: the
// pieces shared by the gather kernels and the fused small-batch decode
// ([KARAT] Eq. 2 over the retrieved rows; [KARAT] = paper-daily digest
// "Heterogeneous LLM Serving with General-Purpose Processing-Near-Memory for
// Retrieval-Based Sparse Attention"). 16 lanes cover one 256-B bf16 row (16 B
// each), a wave load instruction fetches 4 rows, and every load of a batch
// of rows is issued before any arithmetic on it.
#pragma once

#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kGatherUnroll = 8;  // rows per 16-lane group per batch
// K/V rows that one head reads are read once per call: non-temporal loads
constexpr bool kGatherStream = true;
constexpr int kBatchRows = 4 * kGatherUnroll;      // rows per wave per batch

// Online-softmax state of one query head in one 16-lane group (log2 domain).
// The running max starts at a finite sentinel instead of -inf so masked rows
// can be folded in with selects (no -inf - -inf); a state that saw no valid
// row keeps l = 0 and contributes nothing when merged.
constexpr float kEmptyMax = -1e30f;   // running max before any valid row
constexpr float kMaskedScore = -3e30f; // score of a masked row: exp2(kMasked - m) == 0

struct HeadState {
  float m, l, o[8];
  __device__ __forceinline__ void init() {
    m = kEmptyMax;
    l = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;
  }
};

__device__ __forceinline__ void merge_into(HeadState& a, float m2, float l2, const float (&o2)[8]) {
  const float M = fmaxf(a.m, m2);
  const float x = fast_exp2(a.m - M), y = fast_exp2(m2 - M);
  a.l = a.l * x + l2 * y;
#pragma unroll
  for (int i = 0; i < 8; ++i) a.o[i] = a.o[i] * x + o2[i] * y;
  a.m = M;
}

// K and V rows of one batch: lane group r = lane / 16 takes rows r, r+4, ...
// of the batch; raw bits stay in registers until scored.
template <typename T, int U = kGatherUnroll>
struct Batch {
  Raw8<T> k[U], v[U];
  bool valid[U];
};

// Straight-line issue: every lane loads, rows past the segment end or with a
// rejected id load row 0 of the request (always in bounds) and are masked at
// scoring. Without control flow around the loads the compiler keeps all of
// them in flight (a predicated load would force a wait for every earlier one).
template <bool STREAM, bool DUP = false, typename T, int U>
__device__ __forceinline__ void issue_batch(Batch<T, U>& bt, const int* ids, int base, int cnt, int r,
                                            const T* kb, const T* vb, long long row_stride,
                                            const uint32_t* dup = nullptr, int h = 0) {
  int row[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = base + u * 4 + r;
    const int id = ids[min(j, kSegRows - 1)];
    // dup: heads that attend this token through another (lower) chosen list
    bool twice = false;
    if constexpr (DUP) twice = (dup[min(j, kSegRows - 1)] >> h) & 1u;
    bt.valid[u] = (j < cnt) & (id >= 0) & !twice;
    row[u] = bt.valid[u] ? id : 0;
  }
  if constexpr (STREAM) {
#pragma unroll
    for (int u = 0; u < U; ++u) bt.k[u].load_stream(kb + row[u] * row_stride);
#pragma unroll
    for (int u = 0; u < U; ++u) bt.v[u].load_stream(vb + row[u] * row_stride);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) bt.k[u].load(kb + row[u] * row_stride);
#pragma unroll
    for (int u = 0; u < U; ++u) bt.v[u].load(vb + row[u] * row_stride);
  }
}

// Scores the batch's rows for one head, then folds them into the state with
// one max update per batch (one rescale of o instead of one per row).
template <typename T, int U>
__device__ __forceinline__ void consume_batch(const Batch<T, U>& bt, HeadState& st, const QFrag<T>& qf,
                                              float qscale) {
  float sc[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    sc[u] = bt.valid[u] ? group16_sum(qf.dot(bt.k[u])) * qscale : kMaskedScore;
  float mb = sc[0];
#pragma unroll
  for (int u = 1; u < U; ++u) mb = fmaxf(mb, sc[u]);
  const float mn = fmaxf(st.m, mb);
  const float a = fast_exp2(st.m - mn);
  st.l *= a;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.o[i] *= a;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float vx[8];
    bt.v[u].widen(vx);
    const float pw = fast_exp2(sc[u] - mn);
    st.l += pw;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.o[i] = fmaf(pw, vx[i], st.o[i]);
  }
  st.m = mn;
}

// Writes a merged state (every lane group holds the same values after the
// shuffle merge): lanes 0..15 write o, lanes 16..23 the header line
// (m, l, zeros), so each 128-byte line of the record is written in full.
// agent: every word written at agent scope (write-through past the XCD's L2),
// for a merge by another workgroup within the same launch; only m, l and o
__device__ __forceinline__ void store_state(float* ph, const HeadState& st, int r, int e, bool agent = false) {
  if (agent) {
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __hip_atomic_store(ph + kPartO + e * 8 + i, st.o[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (r == 1 && e == 0) {
      __hip_atomic_store(ph, st.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ph + 1, st.l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  if (r == 0) {
    *reinterpret_cast<float4*>(ph + kPartO + e * 8) = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
    *reinterpret_cast<float4*>(ph + kPartO + 4 + e * 8) = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
  } else if (r == 1 && e < kPartO / 4) {
    *reinterpret_cast<float4*>(ph + e * 4) = e == 0 ? make_float4(st.m, st.l, 0.f, 0.f) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

}  // namespace tsa
