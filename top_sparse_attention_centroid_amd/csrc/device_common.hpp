// Device helpers for the gfx950 kernels: element loads, wave64 cross-lane
// reductions through DPP, ballot prefix counts, order-preserving float keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsa {

constexpr int kHeadDim = 128;  // d: one row is 128 elements (256 B in bf16)
constexpr int kWave = 64;

// bf16 bit patterns are stored as uint16_t; widening to fp32 is exact.
using bf16_t = uint16_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Eight consecutive elements in flight as raw bits: 16 B for bf16, 32 B for fp32.
template <typename T>
struct Raw8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load; the streaming variant is for data touched once per call.
__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <>
struct Raw8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_stream(const bf16_t* p) { v = load16_stream(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void widen(float (&x)[8]) const {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
    x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
    x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
};

template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void load_stream(const float* p) {
    const uint4 x = load16_stream(p), y = load16_stream(p + 4);
    a = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
    b = make_float4(__uint_as_float(y.x), __uint_as_float(y.y), __uint_as_float(y.z), __uint_as_float(y.w));
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void widen(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));   // MFMA 16x16x32 bf16 operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));     // MFMA 16x16 fp32 result

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// One lane's 8 query elements, kept in the storage type. dot() returns the
// partial dot product with 8 key elements: bf16 pairs go through v_dot2 (the
// bf16 x bf16 products are exact in fp32), fp32 through FMAs.
template <typename T>
struct QFrag;

template <>
struct QFrag<bf16_t> {
  uint4 q;
  __device__ __forceinline__ void load(const bf16_t* p) { q = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float dot(const Raw8<bf16_t>& k) const {
    float acc = dot2_bf16(q.x, k.v.x, 0.f);
    acc = dot2_bf16(q.y, k.v.y, acc);
    acc = dot2_bf16(q.z, k.v.z, acc);
    return dot2_bf16(q.w, k.v.w, acc);
  }
};

template <>
struct QFrag<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ float dot(const Raw8<float>& k) const {
    float s = a.x * k.a.x;
    s = fmaf(a.y, k.a.y, s); s = fmaf(a.z, k.a.z, s); s = fmaf(a.w, k.a.w, s);
    s = fmaf(b.x, k.b.x, s); s = fmaf(b.y, k.b.y, s); s = fmaf(b.z, k.b.z, s);
    return fmaf(b.w, k.b.w, s);
  }
};

// Sum of squares of 8 elements (bf16 pairs through v_dot2, exact products).
__device__ __forceinline__ float sq8(const Raw8<bf16_t>& r) {
  float acc = dot2_bf16(r.v.x, r.v.x, 0.f);
  acc = dot2_bf16(r.v.y, r.v.y, acc);
  acc = dot2_bf16(r.v.z, r.v.z, acc);
  return dot2_bf16(r.v.w, r.v.w, acc);
}
__device__ __forceinline__ float sq8(const Raw8<float>& r) {
  float s = r.a.x * r.a.x;
  s = fmaf(r.a.y, r.a.y, s); s = fmaf(r.a.z, r.a.z, s); s = fmaf(r.a.w, r.a.w, s);
  s = fmaf(r.b.x, r.b.x, s); s = fmaf(r.b.y, r.b.y, s); s = fmaf(r.b.z, r.b.z, s);
  return fmaf(r.b.w, r.b.w, s);
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
  Raw8<T> r;
  r.load(p);
  r.widen(x);
}

__device__ __forceinline__ float dot8(const float (&a)[8], const float (&b)[8]) {
  float s = a[0] * b[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) s = fmaf(a[i], b[i], s);
  return s;
}

// DPP lane permutations inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16-lane row

// Sum over aligned groups of 8 / 16 lanes. Every lane of a group ends with the
// bitwise-same value (each step adds commutative pairs).
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x;
}
__device__ __forceinline__ float group16_sum(float x) {
  x = group8_sum(x);
  x += dpp_f<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int prefix_count(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Unsigned key whose order matches the float order (+0 and -0 collapse).
// Finite floats map to keys >= 0x00800000, so key 0 can mark "no entry".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the wave through DPP: shifts of 1, 2, 4 and 8
// lanes within each 16-lane row, then the row totals carried across rows
// (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3). Lanes
// whose source lies outside the row read 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum over a block of NW waves. `scratch` holds NW ints.
// Returns the caller's exclusive prefix; *total receives the block total.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int x = wave_inclusive_scan(v);
  if (lane == kWave - 1) scratch[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int t = scratch[w];
    before += (w < wave) ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// block_exclusive_scan of v that also returns the block total of u in the
// same two barriers. `scratch` holds 2 * NW ints.
template <int NW>
__device__ __forceinline__ int block_exclusive_scan_and_sum(int v, int u, int* scratch, int* total_v,
                                                            int* total_u) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int x = wave_inclusive_scan(v);
  u = wave_sum_i(u);
  if (lane == kWave - 1) {
    scratch[wave] = x;
    scratch[NW + wave] = u;
  }
  __syncthreads();
  int before = 0, all = 0, all_u = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = scratch[w];
    before += (w < wave) ? t : 0;
    all += t;
    all_u += scratch[NW + w];
  }
  __syncthreads();
  *total_v = all;
  *total_u = all_u;
  return before + x - v;
}

// Exclusive block scan of NC per-thread counts at once, classes placed one
// after another: pos[k] = (items of all classes below k) + (items of class k
// held by lower threads). Items therefore land class by class, each class in
// thread order. Also sums `u` over the block into *total_u and the counts
// of every class into *total. `scratch` holds NW * (NC + 1) ints; two
// barriers.
template <int NW, int NC>
__device__ __forceinline__ void block_class_scan(const int (&cnt)[NC], int (&pos)[NC], int u, int* scratch,
                                                 int* total, int* total_u) {
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int x[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) x[c] = wave_inclusive_scan(cnt[c]);
  u = wave_sum_i(u);
  if (lane == kWave - 1) {
#pragma unroll
    for (int c = 0; c < NC; ++c) scratch[wave * (NC + 1) + c] = x[c];
    scratch[wave * (NC + 1) + NC] = u;
  }
  __syncthreads();
  int base = 0, all_u = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = scratch[w * (NC + 1) + c];
      before += (w < wave) ? t : 0;
      all += t;
    }
    pos[c] = base + before + x[c] - cnt[c];
    base += all;
  }
#pragma unroll
  for (int w = 0; w < NW; ++w) all_u += scratch[w * (NC + 1) + NC];
  __syncthreads();
  *total = base;
  *total_u = all_u;
}

template <int NW>
__device__ __forceinline__ int block_sum(int v, int* scratch) {
  int total;
  block_exclusive_scan<NW>(v, scratch, &total);
  return total;
}

}  // namespace tsa
