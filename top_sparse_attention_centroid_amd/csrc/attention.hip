// Gathered sparse attention for gfx950 ([KARAT] Eq. 2 with -inf outside the
// retrieved set; [KARAT] = paper-daily digest "Heterogeneous LLM Serving with
// General-Purpose Processing-Near-Memory for Retrieval-Based Sparse
// Attention").
//
// gather_attn: a segment is at most kSegRows rows of one (request, KV head),
// with the head mask of the GQA group's query heads that chose them, so a row
// chosen by several heads of the group is read from HBM once. Each wave owns
// whole segments: 16 lanes cover one 256-B bf16 row (16 B each), a wave load
// instruction fetches 4 rows, and a batch of 16 rows is in flight while the
// previous batch is scored (double buffering in registers). Each lane group
// keeps an online-softmax state (running max m, sum l, output o) in the log2
// domain; the four lane groups merge by lane shuffles and the segment writes
// one partial (m, l, o) per masked head.
// combine: one wave per query head merges the partials of its segments with
// the log-sum-exp rule and writes o / l (zero when nothing was selected).
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kGatherWaves = kGatherWavesPerBlock;  // each wave owns whole segments
constexpr int kGatherUnroll = 4;  // rows per 16-lane group per batch (a batch is 16 rows per wave)
constexpr int kBatchRows = 4 * kGatherUnroll;

template <int G>
struct SoftmaxState {
  float m[G], l[G], o[G][8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }
  }
};

__device__ __forceinline__ void merge_into(float& m, float& l, float (&o)[8], float m2, float l2,
                                           const float (&o2)[8]) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  const float a = fast_exp2(m - M), c = fast_exp2(m2 - M);
  l = l * a + l2 * c;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = o[i] * a + o2[i] * c;
  m = M;
}

// K and V rows of one batch (16 rows per wave: lane group r = lane / 16 takes
// rows r, r + 4, r + 8, r + 12 of the batch), raw bits in registers.
template <typename T>
struct Batch {
  Raw8<T> k[kGatherUnroll], v[kGatherUnroll];
  int row[kGatherUnroll];
};

template <typename T>
__device__ __forceinline__ void issue_batch(Batch<T>& bt, const int* ids, int base, int cnt, int r,
                                            const T* kb, const T* vb, long long row_stride) {
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u) {
    const int j = base + u * 4 + r;
    bt.row[u] = j < cnt ? ids[j] : -1;
  }
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u)
    if (bt.row[u] >= 0) bt.k[u].load(kb + bt.row[u] * row_stride);
#pragma unroll
  for (int u = 0; u < kGatherUnroll; ++u)
    if (bt.row[u] >= 0) bt.v[u].load(vb + bt.row[u] * row_stride);
}

template <typename T, int G>
__device__ __forceinline__ void consume_batch(const Batch<T>& bt, SoftmaxState<G>& st, uint32_t mask,
                                              const float* qs, int e) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!(mask & (1u << h))) continue;
    float qf[8];
    {
      const float4 a = *reinterpret_cast<const float4*>(qs + h * kHeadDim + e * 8);
      const float4 b = *reinterpret_cast<const float4*>(qs + h * kHeadDim + e * 8 + 4);
      qf[0] = a.x; qf[1] = a.y; qf[2] = a.z; qf[3] = a.w;
      qf[4] = b.x; qf[5] = b.y; qf[6] = b.z; qf[7] = b.w;
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      if (bt.row[u] < 0) continue;
      float kx[8], vx[8];
      bt.k[u].widen(kx);
      bt.v[u].widen(vx);
      const float sc = group16_sum(dot8(qf, kx));
      const float mn = fmaxf(st.m[h], sc);
      const float a = fast_exp2(st.m[h] - mn);
      const float pw = fast_exp2(sc - mn);
      st.l[h] = fmaf(st.l[h], a, pw);
#pragma unroll
      for (int i = 0; i < 8; ++i) st.o[h][i] = fmaf(pw, vx[i], st.o[h][i] * a);
      st.m[h] = mn;
    }
  }
}

// gather_attn: every wave processes whole segments on its own (no block
// barrier after the q staging). Per segment: row ids -> wave-private LDS in
// one round trip, then K/V batches double-buffered in registers (batch i+1 in
// flight while batch i is scored), then the four lane groups merge and lanes
// 0..15 write the segment's partial state per masked head.
template <typename T, int G, bool EXPLICIT>
__global__ __launch_bounds__(kGatherWaves * kWave) void gather_attn_kernel(GatherParams p) {
  constexpr int NW = kGatherWaves;
  __shared__ float qs[G * kHeadDim];
  __shared__ int ids_lds[NW][kSegRows];
  const int bg = blockIdx.x / p.W, w0 = blockIdx.x % p.W;
  const int b = bg / p.Hkv, g = bg % p.Hkv;

  int nseg, total_rows = 0;
  if constexpr (EXPLICIT) {
    nseg = p.nseg[bg];
  } else {
    // clamp a device-side count to the planned capacity (never trusted)
    total_rows = min(max(p.counts ? p.counts[b] : p.count_const, 0), p.count_max);
    nseg = (total_rows + p.seg_rows - 1) / p.seg_rows;
  }
  if (w0 * NW >= nseg) return;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = lane >> 4, e = lane & 15;
  {
    const T* qb = static_cast<const T*>(p.q) + (static_cast<long long>(b) * p.Hkv + g) * G * kHeadDim;
    for (int i = tid; i < G * kHeadDim / 8; i += NW * kWave) {
      float x[8];
      load8(qb + i * 8, x);
#pragma unroll
      for (int t = 0; t < 8; ++t) qs[i * 8 + t] = x[t] * p.qscale;
    }
  }
  __syncthreads();

  const long long row_stride = static_cast<long long>(p.Hkv) * kHeadDim;
  const T* kb = static_cast<const T*>(p.k) + static_cast<long long>(b) * p.n_rows * row_stride +
                g * kHeadDim + e * 8;
  const T* vb = static_cast<const T*>(p.v) + static_cast<long long>(b) * p.n_rows * row_stride +
                g * kHeadDim + e * 8;
  const int32_t* rid = p.rowids + b * p.rid_bstride + g * p.rid_gstride;
  int* ids = ids_lds[wave];

  for (int s = w0 * NW + wave; s < nseg; s += p.W * NW) {
    int start, cnt;
    uint32_t mask;
    if constexpr (EXPLICIT) {
      const int4 d = p.seg[static_cast<long long>(bg) * p.smax + s];
      start = d.x;
      cnt = d.y;
      mask = static_cast<uint32_t>(d.z);
    } else {
      start = s * p.seg_rows;
      cnt = min(p.seg_rows, total_rows - start);
      mask = (1u << G) - 1u;
    }
    for (int j = lane; j < cnt; j += kWave) {
      const int id = rid[start + j];
      // ids outside [0, n_rows) are skipped, never dereferenced
      ids[j] = static_cast<unsigned long long>(id) < static_cast<unsigned long long>(p.n_rows) ? id : -1;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    SoftmaxState<G> st;
    st.init();
    Batch<T> A, Bb;
    issue_batch(A, ids, 0, cnt, r, kb, vb, row_stride);
    for (int base = 0; base < cnt; base += 2 * kBatchRows) {
      const bool has_b = base + kBatchRows < cnt;
      if (has_b) issue_batch(Bb, ids, base + kBatchRows, cnt, r, kb, vb, row_stride);
      consume_batch(A, st, mask, qs, e);
      if (has_b) {
        if (base + 2 * kBatchRows < cnt) issue_batch(A, ids, base + 2 * kBatchRows, cnt, r, kb, vb, row_stride);
        consume_batch(Bb, st, mask, qs, e);
      }
    }

    // Merge the four 16-lane row groups (lanes e, e+16, e+32, e+48) and write
    // the segment's partial for every masked head.
    float* part = p.partial + (static_cast<long long>(bg) * p.smax + s) * G * kPartStride;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!(mask & (1u << h))) continue;
#pragma unroll
      for (int x = 16; x <= 32; x <<= 1) {
        float o2[8];
        const float m2 = __shfl_xor(st.m[h], x);
        const float l2 = __shfl_xor(st.l[h], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) o2[i] = __shfl_xor(st.o[h][i], x);
        merge_into(st.m[h], st.l[h], st.o[h], m2, l2, o2);
      }
      if (r == 0) {
        float* ph = part + h * kPartStride;
        *reinterpret_cast<float4*>(ph + 4 + e * 8) = make_float4(st.o[h][0], st.o[h][1], st.o[h][2], st.o[h][3]);
        *reinterpret_cast<float4*>(ph + 8 + e * 8) = make_float4(st.o[h][4], st.o[h][5], st.o[h][6], st.o[h][7]);
        if (e == 0) {
          ph[0] = st.m[h];
          ph[1] = st.l[h];
        }
      }
    }
    // the next segment overwrites this wave's id staging area
    __builtin_amdgcn_wave_barrier();
  }
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// combine: one wave per query head. Lanes read 64 segment descriptors and
// partial (m, l) at once, so the log-sum-exp weights come from two wave
// reductions; the o vectors of the head's segments are then accumulated with
// four independent loads in flight per lane.
template <int G, bool EXPLICIT>
__global__ __launch_bounds__(512) void combine_kernel(GatherParams p) {
  const int bg = blockIdx.x;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int h = threadIdx.x / kWave, lane = lane_id();
  int nseg;
  if constexpr (EXPLICIT) {
    nseg = p.nseg[bg];
  } else {
    const int rows = min(max(p.counts ? p.counts[b] : p.count_const, 0), p.count_max);
    nseg = (rows + p.seg_rows - 1) / p.seg_rows;
  }
  float M = -INFINITY, L = 0.f, O0 = 0.f, O1 = 0.f;
  const float* base = p.partial + static_cast<long long>(bg) * p.smax * G * kPartStride + h * kPartStride;
  for (int s0 = 0; s0 < nseg; s0 += kWave) {
    const int s = s0 + lane;
    bool mine = s < nseg;
    if constexpr (EXPLICIT) {
      if (mine) mine = (static_cast<uint32_t>(p.seg[static_cast<long long>(bg) * p.smax + s].z) >> h) & 1u;
    }
    const float* ph = base + static_cast<long long>(s) * G * kPartStride;
    const float pm = mine ? ph[0] : -INFINITY;
    const float pl = mine ? ph[1] : 0.f;
    const float Mn = fmaxf(M, wave_max_f(pm));
    if (Mn == -INFINITY) continue;
    const float w = mine ? fast_exp2(pm - Mn) : 0.f;
    const float a = fast_exp2(M - Mn);
    L = L * a + wave_sum_f(pl * w);
    O0 *= a;
    O1 *= a;
    M = Mn;
    uint64_t bal = __ballot(mine && pm != -INFINITY);
    while (bal) {
      int j[4];
      float wj[4];
      float2 po[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        j[u] = bal ? __builtin_ctzll(bal) : -1;
        if (bal) bal &= bal - 1;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wj[u] = __shfl(w, j[u] < 0 ? 0 : j[u]);
        po[u] = j[u] < 0 ? make_float2(0.f, 0.f)
                         : *reinterpret_cast<const float2*>(base + static_cast<long long>(s0 + j[u]) * G * kPartStride +
                                                            4 + lane * 2);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j[u] < 0) continue;
        O0 = fmaf(wj[u], po[u].x, O0);
        O1 = fmaf(wj[u], po[u].y, O1);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* o = p.out + ((static_cast<long long>(b) * p.Hkv + g) * G + h) * kHeadDim + lane * 2;
  *reinterpret_cast<float2*>(o) = make_float2(O0 * inv, O1 * inv);
}

template <typename T, bool EXPLICIT>
static void gather_dispatch(const GatherParams& p, int G, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.B * p.Hkv * p.W)), block(kGatherWaves * kWave);
  switch (G) {
    case 1: hipLaunchKernelGGL((gather_attn_kernel<T, 1, EXPLICIT>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((gather_attn_kernel<T, 2, EXPLICIT>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((gather_attn_kernel<T, 4, EXPLICIT>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((gather_attn_kernel<T, 8, EXPLICIT>), grid, block, 0, s, p); break;
  }
}

hipError_t launch_gather(const GatherParams& p, int dtype, int G, bool explicit_plan,
                         hipStream_t s) {
  if (dtype == kBF16) {
    if (explicit_plan) gather_dispatch<bf16_t, true>(p, G, s);
    else gather_dispatch<bf16_t, false>(p, G, s);
  } else {
    if (explicit_plan) gather_dispatch<float, true>(p, G, s);
    else gather_dispatch<float, false>(p, G, s);
  }
  return hipGetLastError();
}

template <bool EXPLICIT>
static void combine_dispatch(const GatherParams& p, int G, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.B * p.Hkv)), block(G * kWave);
  switch (G) {
    case 1: hipLaunchKernelGGL((combine_kernel<1, EXPLICIT>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((combine_kernel<2, EXPLICIT>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((combine_kernel<4, EXPLICIT>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((combine_kernel<8, EXPLICIT>), grid, block, 0, s, p); break;
  }
}

hipError_t launch_combine(const GatherParams& p, int G, bool explicit_plan, hipStream_t s) {
  if (explicit_plan) combine_dispatch<true>(p, G, s);
  else combine_dispatch<false>(p, G, s);
  return hipGetLastError();
}

}  // namespace tsa
