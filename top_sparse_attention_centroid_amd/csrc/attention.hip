// Gathered sparse attention for gfx950 ([KARAT] Eq. 2 with -inf outside the
// retrieved set; [KARAT] = paper-daily digest "Heterogeneous LLM Serving with
// General-Purpose Processing-Near-Memory for Retrieval-Based Sparse
// Attention").
//
// gather_attn: one workgroup (4 waves) per segment of at most kSegRows rows of
// one (request, KV head). A segment carries a head mask: the rows are read
// once from HBM and scored for every query head of the GQA group that chose
// them. Inside a wave, 16 lanes own one 256-B bf16 row (16 B each) so a wave
// load instruction fetches 4 rows; U row groups per lane are in flight before
// any arithmetic. Each lane group keeps an online-softmax state (running max
// m, sum l, output o) in the log2 domain; states merge across the 4 lane
// groups (lane shuffles), then across waves (LDS), and the segment writes one
// partial (m, l, o) per head.
// combine: one wave per query head merges the partials of its segments with
// the log-sum-exp rule and writes o / l (zero when nothing was selected).
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

constexpr int kGatherWaves = 4;
constexpr int kGatherUnroll = 4;

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

template <typename T, int G, bool EXPLICIT>
__global__ __launch_bounds__(256) void gather_attn_kernel(GatherParams p) {
  constexpr int NW = kGatherWaves, U = kGatherUnroll;
  __shared__ float red[NW][G][kHeadDim + 2];
  const int bg = blockIdx.x / p.W, w0 = blockIdx.x % p.W;
  const int b = bg / p.Hkv, g = bg % p.Hkv;

  int nseg, total_rows = 0;
  if constexpr (EXPLICIT) {
    nseg = p.nseg[bg];
  } else {
    // clamp a device-side count to the planned capacity (never trusted)
    total_rows = min(max(p.counts ? p.counts[b] : p.count_const, 0), p.count_max);
    nseg = (total_rows + kSegRows - 1) / kSegRows;
  }
  if (w0 >= nseg) return;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = lane >> 4, e = lane & 15;
  const long long row_stride = static_cast<long long>(p.Hkv) * kHeadDim;
  const T* kb = static_cast<const T*>(p.k) + static_cast<long long>(b) * p.n_rows * row_stride +
                g * kHeadDim + e * 8;
  const T* vb = static_cast<const T*>(p.v) + static_cast<long long>(b) * p.n_rows * row_stride +
                g * kHeadDim + e * 8;
  const int32_t* rid = p.rowids + b * p.rid_bstride + g * p.rid_gstride;

  float qf[G][8];
  {
    const T* qb = static_cast<const T*>(p.q) + (static_cast<long long>(b) * p.Hkv + g) * G * kHeadDim;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      load8(qb + h * kHeadDim + e * 8, qf[h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[h][i] *= p.qscale;
    }
  }

  for (int s = w0; s < nseg; s += p.W) {
    int start, cnt;
    uint32_t mask;
    if constexpr (EXPLICIT) {
      const int4 d = p.seg[static_cast<long long>(bg) * p.smax + s];
      start = d.x;
      cnt = d.y;
      mask = static_cast<uint32_t>(d.z);
    } else {
      start = s * kSegRows;
      cnt = min(kSegRows, total_rows - start);
      mask = (1u << G) - 1u;
    }

    SoftmaxState<G> st;
    st.init();
    for (int jw = wave * 4; jw < cnt; jw += NW * 4 * U) {
      int row[U];
      Raw8<T> kr[U], vr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = jw + u * NW * 4 + r;
        const int id = j < cnt ? rid[start + j] : -1;
        // ids outside [0, n_rows) are skipped, never dereferenced
        row[u] = static_cast<unsigned long long>(id) < static_cast<unsigned long long>(p.n_rows) ? id : -1;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (row[u] >= 0) kr[u].load(kb + row[u] * row_stride);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (row[u] >= 0) vr[u].load(vb + row[u] * row_stride);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (row[u] >= 0) {
          float kx[8], vx[8];
          kr[u].widen(kx);
          vr[u].widen(vx);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (mask & (1u << h)) {
              const float sc = group16_sum(dot8(qf[h], kx));
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
      }
    }

    // Merge the four 16-lane row groups of the wave (lanes e, e+16, e+32, e+48).
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (mask & (1u << h)) {
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
#pragma unroll
          for (int i = 0; i < 8; ++i) red[wave][h][2 + e * 8 + i] = st.o[h][i];
          if (e == 0) {
            red[wave][h][0] = st.m[h];
            red[wave][h][1] = st.l[h];
          }
        }
      }
    }
    __syncthreads();
    // Merge across waves and write this segment's partial for each masked head.
    float* part = p.partial + (static_cast<long long>(bg) * p.smax + s) * G * kPartStride;
    for (int idx = tid; idx < G * kHeadDim; idx += NW * kWave) {
      const int h = idx / kHeadDim, dd = idx % kHeadDim;
      if (!(mask & (1u << h))) continue;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, red[ww][h][0]);
      float L = 0.f, O = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
          const float c = fast_exp2(red[ww][h][0] - M);
          L = fmaf(red[ww][h][1], c, L);
          O = fmaf(red[ww][h][2 + dd], c, O);
        }
      }
      float* ph = part + h * kPartStride;
      ph[4 + dd] = O;
      if (dd == 0) {
        ph[0] = M;
        ph[1] = L;
      }
    }
    __syncthreads();
  }
}

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
    nseg = (rows + kSegRows - 1) / kSegRows;
  }
  float M = -INFINITY, L = 0.f, O0 = 0.f, O1 = 0.f;
  const float* base = p.partial + static_cast<long long>(bg) * p.smax * G * kPartStride;
  for (int s = 0; s < nseg; ++s) {
    if constexpr (EXPLICIT) {
      const uint32_t mask = static_cast<uint32_t>(p.seg[static_cast<long long>(bg) * p.smax + s].z);
      if (!(mask & (1u << h))) continue;
    }
    const float* ph = base + (static_cast<long long>(s) * G + h) * kPartStride;
    const float pm = ph[0], pl = ph[1];
    const float2 po = *reinterpret_cast<const float2*>(ph + 4 + lane * 2);
    const float Mn = fmaxf(M, pm);
    if (Mn == -INFINITY) continue;
    const float a = fast_exp2(M - Mn), c = fast_exp2(pm - Mn);
    L = L * a + pl * c;
    O0 = O0 * a + po.x * c;
    O1 = O1 * a + po.y * c;
    M = Mn;
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
