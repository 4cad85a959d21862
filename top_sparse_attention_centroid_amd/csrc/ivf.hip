// Inverted-index kernels for gfx950: index build (nearest-centroid assignment
// and stable CSR posting lists), centroid scoring, and per-query-head top-k
// list selection fused with the gather plan of the KV group.
//
// [KARAT] = paper-daily digest "Heterogeneous LLM Serving with General-Purpose
// Processing-Near-Memory for Retrieval-Based Sparse Attention".
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"
#include "select_common.hpp"

namespace tsa {

// ============================================================================
// Index build, step 1 for fp32 data: nearest centroid of every key ([KARAT]
// How, index structure). One thread per key holds the key in registers;
// centroids stream through LDS in tiles of 32 rows. argmin_c |k - c|^2 = argmin_c (|c|^2 -
// 2 k.c); ties keep the lower centroid (strict <).
// ============================================================================
constexpr int kAssignTile = 32;

// The M best (distance, centroid) pairs seen so far, best first; order is
// lexicographic, so an equal distance keeps the lower centroid id. A new
// pair is inserted by one pass of compare-and-swap down the list (the
// displaced pair carried on), which keeps the list sorted and drops the
// worst.
template <int M>
struct TopM {
  float d[M];
  int c[M];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      d[i] = INFINITY;
      c[i] = 0x7fffffff;
    }
  }
  __device__ __forceinline__ static bool less(float d1, int c1, float d2, int c2) {
    return d1 < d2 || (d1 == d2 && c1 < c2);
  }
  __device__ __forceinline__ void push(float dd, int cc) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const bool sw = less(dd, cc, d[i], c[i]);
      const float td = d[i];
      const int tc = c[i];
      d[i] = sw ? dd : td;
      c[i] = sw ? cc : tc;
      dd = sw ? td : dd;
      cc = sw ? tc : cc;
    }
  }
};
static_assert(kMaxAssign >= 1 && kMaxAssign <= 4, "lists per key");

template <typename T, int M>
__global__ __launch_bounds__(256) void assign_kernel(AssignParams p) {
  __shared__ float4 tile[kAssignTile][kHeadDim / 4];
  __shared__ float norm2[kAssignTile];
  const int bg = blockIdx.y;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int tid = threadIdx.x;
  const int i = blockIdx.x * 256 + tid;
  const bool valid = i < p.n_assign;

  float kf[kHeadDim];
  {
    const T* kr = static_cast<const T*>(p.keys) +
                  ((static_cast<long long>(b) * p.N + (valid ? i : 0)) * p.Hkv + g) * kHeadDim;
#pragma unroll
    for (int j = 0; j < kHeadDim / 8; ++j) {
      float x[8];
      load8(kr + j * 8, x);
#pragma unroll
      for (int t = 0; t < 8; ++t) kf[j * 8 + t] = x[t];
    }
  }
  const T* cb = static_cast<const T*>(p.centroids) + b * p.cent_bstride +
                static_cast<long long>(g) * p.C * kHeadDim;
  TopM<M> top;
  top.init();
  for (int c0 = 0; c0 < p.C; c0 += kAssignTile) {
    __syncthreads();
    for (int idx = tid; idx < kAssignTile * (kHeadDim / 8); idx += 256) {
      const int row = idx / (kHeadDim / 8), part = idx % (kHeadDim / 8);
      const int c = c0 + row;
      float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (c < p.C) load8(cb + static_cast<long long>(c) * kHeadDim + part * 8, x);
      tile[row][part * 2] = make_float4(x[0], x[1], x[2], x[3]);
      tile[row][part * 2 + 1] = make_float4(x[4], x[5], x[6], x[7]);
    }
    __syncthreads();
    if (tid < kAssignTile) {
      float s = 0.f;
      for (int t = 0; t < kHeadDim / 4; ++t) {
        float4 v = tile[tid][t];
        s = fmaf(v.x, v.x, s); s = fmaf(v.y, v.y, s); s = fmaf(v.z, v.z, s); s = fmaf(v.w, v.w, s);
      }
      norm2[tid] = s;
    }
    __syncthreads();
    const int nc = min(kAssignTile, p.C - c0);
    for (int j = 0; j < nc; ++j) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int t = 0; t < kHeadDim / 4; ++t) {
        const float4 v = tile[j][t];
        a0 = fmaf(kf[4 * t + 0], v.x, a0);
        a1 = fmaf(kf[4 * t + 1], v.y, a1);
        a2 = fmaf(kf[4 * t + 2], v.z, a2);
        a3 = fmaf(kf[4 * t + 3], v.w, a3);
      }
      top.push(norm2[j] - 2.f * ((a0 + a1) + (a2 + a3)), c0 + j);
    }
  }
  if (valid) {
#pragma unroll
    for (int r = 0; r < M; ++r) p.assign[(static_cast<long long>(bg) * p.N + i) * M + r] = top.c[r];
  }
}

// ============================================================================
// Index build, step 1 on matrix cores (bf16): the same nearest-centroid search
// as a dense contraction centroids x keys^T (16x16x32 bf16 MFMA, fp32
// accumulate). Each wave keeps a 16-key tile (4 fragments cover d = 128) in
// registers as the B operand and runs 16-centroid A tiles read from LDS
// against it (rows padded so the 16 lanes of a fragment read distinct banks).
// The accumulator starts at -|c|^2 / 2, so the MFMA chain yields
// s = k.c - |c|^2 / 2 and the nearest centroid is the largest s
// (|k - c|^2 = |k|^2 - 2 s); padding rows start at -inf and never win. Lane l
// of a 16x16 result holds key column l % 16 for centroid rows (l / 16) * 4 ..
// +4, so each lane follows one key: it keeps the key's best M values of s over
// its centroids in ascending id order (strict >, so a tie keeps the lower id)
// with compares and selects only, and the four lanes that share the key merge
// their lists on d = -2 s with the lexicographic order (distance, centroid id).
// ============================================================================

constexpr int kMfmaCs = 256;      // centroids per LDS stage
constexpr int kMfmaKb = 1024;     // keys per workgroup
constexpr int kMfmaWaves = 8;
constexpr int kCentPad = 136;     // LDS row stride in elements (128 + 8)
constexpr int kAssignTiles = 4;  // 16-key tiles scored per pass over the staged centroids

__global__ __launch_bounds__(256) void centroid_norms_kernel(const bf16_t* cent, float* norms, long long rows) {
  const long long row = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) / 16;
  const int e = threadIdx.x & 15;
  float x[8];
  load8(cent + min(row, rows - 1) * kHeadDim + e * 8, x);
  float s2 = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s2 = fmaf(x[i], x[i], s2);
  s2 = group16_sum(s2);
  if (e == 0 && row < rows) norms[row] = s2;
}

// A workgroup owns kMfmaKb keys of one (request, KV head). Centroids are
// staged kMfmaCs at a time; for each stage every wave runs its 16-key tiles
// against all staged 16-centroid tiles and folds each key's best into the
// per-key best kept in LDS (strict <, so a tie keeps the earlier stage's lower
// centroid id).
template <int M>
__global__ __launch_bounds__(kMfmaWaves * kWave) void assign_mfma_kernel(AssignParams p, const float* norms) {
  __shared__ __align__(16) bf16_t cs[kMfmaCs * kCentPad];
  __shared__ __align__(16) float hn[kMfmaCs];  // -|c|^2 / 2 of the staged centroids, -inf past C
  __shared__ float best_d[kMfmaKb * M];
  __shared__ int best_c[kMfmaKb * M];
  const int bg = blockIdx.y;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int kbase = blockIdx.x * kMfmaKb;
  const bf16_t* keys = static_cast<const bf16_t*>(p.keys);
  const bf16_t* cb = static_cast<const bf16_t*>(p.centroids) + b * p.cent_bstride +
                     static_cast<long long>(g) * p.C * kHeadDim;
  const float* nb = norms + (p.cent_bstride ? (static_cast<long long>(b) * p.Hkv + g) : g) * p.C;
  for (int i = tid; i < kMfmaKb * M; i += kMfmaWaves * kWave) {
    best_d[i] = INFINITY;
    best_c[i] = 0x7fffffff;
  }
  for (int c0 = 0; c0 < p.C; c0 += kMfmaCs) {
    __syncthreads();
    for (int idx = tid; idx < kMfmaCs * 16; idx += kMfmaWaves * kWave) {
      const int row = idx / 16, part = idx % 16;
      const int c = min(c0 + row, p.C - 1);
      *reinterpret_cast<uint4*>(cs + row * kCentPad + part * 8) =
          *reinterpret_cast<const uint4*>(cb + static_cast<long long>(c) * kHeadDim + part * 8);
    }
    for (int i = tid; i < kMfmaCs; i += kMfmaWaves * kWave)
      hn[i] = c0 + i < p.C ? -0.5f * nb[c0 + i] : -INFINITY;
    __syncthreads();
    const int ntile = (min(kMfmaCs, p.C - c0) + 15) / 16;
    // A pass scores kAssignTiles of the wave's 16-key tiles (kt, kt +
    // kMfmaWaves, ...) against the staged centroids: each centroid fragment
    // read from LDS feeds kAssignTiles MFMA chains, and the tiles' keys are
    // requested together.
    constexpr int NT = kAssignTiles;
    constexpr int kTiles = kMfmaKb / 16;
    for (int kt = wave; kt < kTiles; kt += NT * kMfmaWaves) {
      if (kbase + kt * 16 >= p.n_assign) break;
      bool on[NT];
      bf16x8_t a[NT][4];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int ktj = kt + j * kMfmaWaves;
        on[j] = ktj < kTiles && kbase + ktj * 16 < p.n_assign;  // uniform over the wave
        const int key = min(kbase + min(ktj, kTiles - 1) * 16 + col, p.n_assign - 1);  // clamped: in bounds
        const bf16_t* kr = keys + ((static_cast<long long>(b) * p.N + key) * p.Hkv + g) * kHeadDim + grp * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a[j][ks] = *reinterpret_cast<const bf16x8_t*>(kr + ks * 32);
      }
      // the lane's key in tile j: its best M values of s, best first
      float bs[NT][M];
      int bc[NT][M];
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < M; ++r) {
          bs[j][r] = -INFINITY;
          bc[j][r] = 0x7fffffff;
        }
      for (int t = 0; t < ntile; ++t) {
        const bf16_t* crow = cs + (t * 16 + col) * kCentPad + grp * 8;
        bf16x8_t cfr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) cfr[ks] = *reinterpret_cast<const bf16x8_t*>(crow + ks * 32);
        const f32x4_t h = *reinterpret_cast<const f32x4_t*>(hn + t * 16 + grp * 4);
        const int cr = c0 + t * 16 + grp * 4;  // centroid of accumulator row 0
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          f32x4_t acc = h;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cfr[ks], a[j][ks], acc, 0, 0, 0);
          // rows hold ascending centroids: strict > keeps the lower id of a
          // tie; -inf padding never passes
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // insert (acc[i], cr + i) into the list, ordered by s
            // descending, then id ascending: the new id is above every id in
            // the list, so it goes before the first strictly smaller s, and
            // the entries from there on move down one place
            const float v = acc[i];
            bool gt[M];
#pragma unroll
            for (int r = 0; r < M; ++r) gt[r] = v > bs[j][r];
#pragma unroll
            for (int r = M - 1; r >= 1; --r) {
              bs[j][r] = gt[r - 1] ? bs[j][r - 1] : (gt[r] ? v : bs[j][r]);
              bc[j][r] = gt[r - 1] ? bc[j][r - 1] : (gt[r] ? cr + i : bc[j][r]);
            }
            bs[j][0] = gt[0] ? v : bs[j][0];
            bc[j][0] = gt[0] ? cr + i : bc[j][0];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (!on[j]) continue;  // uniform over the wave
        TopM<M> best;
#pragma unroll
        for (int r = 0; r < M; ++r) {
          best.d[r] = -2.f * bs[j][r];  // exact scaling: the order reverses, ties stay ties
          best.c[r] = bc[j][r];
        }
        // lanes col, col + 16, col + 32, col + 48 hold the key's disjoint
        // centroid rows: merge their lists over lane distances 16 and 32
#pragma unroll
        for (int off = 16; off < kWave; off <<= 1) {
          float od[M];
          int oc[M];
#pragma unroll
          for (int r = 0; r < M; ++r) {
            od[r] = __shfl_xor(best.d[r], off);
            oc[r] = __shfl_xor(best.c[r], off);
          }
#pragma unroll
          for (int r = 0; r < M; ++r) best.push(od[r], oc[r]);
        }
        if (grp == 0) {
          const int kl = (kt + j * kMfmaWaves) * 16 + col;
          TopM<M> tm;
#pragma unroll
          for (int r = 0; r < M; ++r) {
            tm.d[r] = best_d[kl * M + r];
            tm.c[r] = best_c[kl * M + r];
          }
#pragma unroll
          for (int r = 0; r < M; ++r) tm.push(best.d[r], best.c[r]);
#pragma unroll
          for (int r = 0; r < M; ++r) {
            best_d[kl * M + r] = tm.d[r];
            best_c[kl * M + r] = tm.c[r];
          }
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < kMfmaKb * M; i += kMfmaWaves * kWave) {
    const int key = kbase + i / M;
    if (key < p.n_assign) p.assign[(static_cast<long long>(bg) * p.N + key) * M + i % M] = best_c[i];
  }
}

// ============================================================================
// Index build, step 2 for codebooks of up to kCsrMaxC lists: the NW waves of
// a workgroup each take a contiguous share of the (token, list) entries. Per-wave LDS histograms give every wave its own cursor per list
// (lists ordered by token, waves in token order, so ids stay ascending inside
// a list); each wave places its tokens with the same ballot ranking as
// csr_kernel below, its list ids requested kCsrBatch chunks at a time. With
// STAGED (N <= kCsrStage) the ids go to an LDS copy of the (request, KV
// head)'s list, written out with coalesced stores; otherwise straight to
// memory (long contexts, where few workgroups need many waves). The
// one-wave csr_kernel placed every token itself and wrote each 4-byte id
// straight to memory (a 16-byte write each).
// ============================================================================
constexpr int kCsrStage = 32768;  // token ids staged in LDS (128 KiB)
constexpr int kCsrMaxC = 1024;    // lists with per-wave counters in LDS
constexpr int kCsrSmallC = 256;   // lists whose 16 waves' counters fit beside the LDS stage
constexpr int kCsrBatch = 16;     // 64-token chunks whose list ids a wave requests together

template <int NW, bool STAGED, int MAXC = kCsrMaxC>
__global__ __launch_bounds__(NW * kWave) void csr_waves_kernel(CsrParams p) {
  __shared__ int stage[STAGED ? kCsrStage : 1];
  __shared__ int hist[NW][MAXC];  // counts, then cursors (C <= MAXC)
  __shared__ int scan_scratch[NW];
  const int bg = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int C = p.C, m = p.m;
  const int n = p.n_assign * m;                          // (token, list) entries, token-major
  const long long cap = static_cast<long long>(p.N) * m;
  const int32_t* a = p.assign + static_cast<long long>(bg) * cap;
  int32_t* off = p.offsets + static_cast<long long>(bg) * (C + 1);
  int32_t* ids = p.ids + static_cast<long long>(bg) * cap;
  int32_t* alt = p.alt ? p.alt + static_cast<long long>(bg) * cap * (m - 1) : nullptr;
  int32_t* lens = p.lens ? p.lens + static_cast<long long>(bg) * C : nullptr;
  // entry i (token i / m's choice i % m) placed at pos: its alt row holds
  // the token's other m - 1 lists, in the token's order of preference
  auto put_alt = [&](long long pos, int i) {
    const int tok = i / m, r = i - tok * m;
    for (int q = 0; q < m - 1; ++q)
      alt[pos * (m - 1) + q] = min(max(a[static_cast<long long>(tok) * m + q + (q >= r ? 1 : 0)], 0), C - 1);
  };
  // this wave's entries, whole tokens (a multiple of m) each
  const int lo = static_cast<int>(static_cast<long long>(wave) * n / NW / m * m);
  const int hi = static_cast<int>(static_cast<long long>(wave + 1) * n / NW / m * m);
  auto put_id = [&](long long pos, int v) {
    if constexpr (STAGED) stage[pos] = v;
    else ids[pos] = v;
  };

  // list ids of kCsrBatch chunks of 64 in one round trip: -1 past the range
  auto load_batch = [&](int i0, int (&cc)[kCsrBatch]) {
    int raw[kCsrBatch];
#pragma unroll
    for (int u = 0; u < kCsrBatch; ++u) raw[u] = a[min(i0 + u * kWave + lane, hi - 1)];  // straight-line, in range
#pragma unroll
    for (int u = 0; u < kCsrBatch; ++u) cc[u] = i0 + u * kWave + lane < hi ? min(max(raw[u], 0), C - 1) : -1;
  };
  for (int i = tid; i < NW * MAXC; i += NW * kWave) hist[i / MAXC][i % MAXC] = 0;
  if constexpr (STAGED)
    for (int i = tid; i < cap; i += NW * kWave) stage[i] = -1;  // free entries and the tail stay -1
  __syncthreads();
  for (int i0 = lo; i0 < hi; i0 += kCsrBatch * kWave) {
    int cc[kCsrBatch];
    load_batch(i0, cc);
#pragma unroll
    for (int u = 0; u < kCsrBatch; ++u)
      if (cc[u] >= 0) atomicAdd(&hist[wave][cc[u]], 1);
  }
  __syncthreads();
  // list starts by one block scan of the totals (plus the free entries after
  // every list); each wave's cursor follows the lower waves' entries
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += NW * kWave) {
    const int c = c0 + tid;
    int tot_c = 0;
    for (int w = 0; w < NW; ++w) tot_c += c < C ? hist[w][c] : 0;
    int tot;
    const int ex = block_exclusive_scan<NW>(tot_c + (c < C ? p.slack : 0), scan_scratch, &tot);
    if (c < C) {
      const int start = carry + ex;
      off[c] = start;
      if (lens) lens[c] = tot_c;
      if constexpr (!STAGED)
        for (int j = tot_c; j < tot_c + p.slack; ++j) ids[start + j] = -1;  // free entries
      int run = start;
      for (int w = 0; w < NW; ++w) {
        const int cnt = hist[w][c];
        hist[w][c] = run;
        run += cnt;
      }
    }
    carry += tot;
  }
  if (tid == 0) off[C] = carry;  // n + C * slack <= N * m
  if constexpr (!STAGED)
    for (long long i = carry + tid; i < cap; i += NW * kWave) ids[i] = -1;  // entries not in use yet
  __syncthreads();
  const int nbits = C > 1 ? 32 - __clz(C - 1) : 0;
  int* cur = hist[wave];
  for (int i0 = lo; i0 < hi; i0 += kCsrBatch * kWave) {
    int cc[kCsrBatch];
    load_batch(i0, cc);
#pragma unroll
    for (int u = 0; u < kCsrBatch; ++u) {
      const int i = i0 + u * kWave + lane;
      const bool valid = cc[u] >= 0;
      const int c = valid ? cc[u] : 0;
      uint64_t same = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (c >> bit) & 1;
        const uint64_t bal = __ballot(set);
        same &= set ? bal : ~bal;
      }
      if (valid) {
        const int rank = prefix_count(same);
        const int pos = cur[c] + rank;
        put_id(pos, i / m);                  // entries of one token are adjacent: ascending ids per list
        if (alt) put_alt(pos, i);
        if (rank == static_cast<int>(__popcll(same)) - 1) cur[c] = pos + 1;
      }
    }
  }
  if constexpr (STAGED) {
    __syncthreads();
    for (int i = tid; i < cap; i += NW * kWave) ids[i] = stage[i];
  }
}

// ============================================================================
// Index build, step 2: CSR posting lists, token ids ascending inside a list.
// One workgroup per (request, KV head): LDS histogram, exclusive scan, then a
// single wave walks the tokens in order; lanes sharing a list find each other
// with one ballot per bit of the list id, which keeps the scatter stable.
// ============================================================================
__global__ __launch_bounds__(256) void csr_kernel(CsrParams p) {
  extern __shared__ int cursor[];  // [C]
  __shared__ int scan_scratch[4];
  const int bg = blockIdx.x;
  const int tid = threadIdx.x;
  const int m = p.m;
  const int n = p.n_assign * m;  // (token, list) entries, token-major
  const long long cap = static_cast<long long>(p.N) * m;
  const int32_t* a = p.assign + static_cast<long long>(bg) * cap;
  int32_t* off = p.offsets + static_cast<long long>(bg) * (p.C + 1);
  int32_t* ids = p.ids + static_cast<long long>(bg) * cap;
  int32_t* alt = p.alt ? p.alt + static_cast<long long>(bg) * cap * (m - 1) : nullptr;
  int32_t* lens = p.lens ? p.lens + static_cast<long long>(bg) * p.C : nullptr;

  for (int c = tid; c < p.C; c += 256) cursor[c] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += 256) atomicAdd(&cursor[a[i]], 1);
  __syncthreads();
  int carry = 0;
  for (int c0 = 0; c0 < p.C; c0 += 256) {
    const int c = c0 + tid;
    const int cnt = c < p.C ? cursor[c] : 0;
    int tot;
    const int ex = block_exclusive_scan<4>(cnt + (c < p.C ? p.slack : 0), scan_scratch, &tot);
    if (c < p.C) {
      const int start = carry + ex;
      off[c] = start;
      cursor[c] = start;
      if (lens) lens[c] = cnt;
      for (int j = cnt; j < cnt + p.slack; ++j) ids[start + j] = -1;  // free entries
    }
    carry += tot;
  }
  if (tid == 0) off[p.C] = carry;  // n + C * slack <= N * m
  for (long long i = carry + tid; i < cap; i += 256) ids[i] = -1;
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    const int nbits = p.C > 1 ? 32 - __clz(p.C - 1) : 0;
    for (int i0 = 0; i0 < n; i0 += kWave) {
      const int i = i0 + lane;
      const bool valid = i < n;
      const int c = valid ? a[i] : 0;
      uint64_t same = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (c >> bit) & 1;
        const uint64_t bal = __ballot(set);
        same &= set ? bal : ~bal;
      }
      if (valid) {
        const int rank = prefix_count(same);
        const int pos = cursor[c] + rank;
        ids[pos] = i / m;                       // entries of one token are adjacent: ascending ids per list
        if (alt) {                              // the token's other lists, in its order of preference
          const int tok = i / m, r = i - tok * m;
          for (int q = 0; q < m - 1; ++q) alt[static_cast<long long>(pos) * (m - 1) + q] = a[tok * m + q + (q >= r ? 1 : 0)];
        }
        if (rank == static_cast<int>(__popcll(same)) - 1) cursor[c] = pos + 1;
      }
    }
  }
}

// ============================================================================
// Centroid scoring, top-k lists per query head, and the gather plan of the
// KV group, fused in one workgroup (kSelWaves waves) per (request, KV head).
//
// Scoring ([KARAT] worked example, step 3): s[h][c] = q[h] . centroid[g][c],
// raw dot product with fp32 accumulation. bf16 data runs it on matrix cores
// (score_tiles_mfma below), inside this workgroup or, for small batches, in
// centroid_score_kernel beforehand; fp32 data on the vector units, 16 lanes
// per 128-element centroid row (8 elements each) reduced through DPP, four
// rows per wave load. Scores go to LDS as order-preserving keys, next to the
// list offsets.
//
// Top-k ([KARAT] How: the top-k most similar lists): wave w owns query heads
// w, w + NW of the group and holds that head's keys in registers, KPL per lane
// (C <= 64 * KPL). The k-th largest key T is found bit by bit (MSB first)
// with ballot counts, over a short candidate list when one suffices (see the
// kernel); keys above it are taken, then keys equal to it in ascending list
// order until k are taken (ties -> lower list id). Lists are emitted in
// ascending order through ballot prefix counts.
//
// Plan: the union of the group's chosen lists with a head bitmask per list,
// each list cut into segments of at most seg_rows rows, ascending list order.
// ============================================================================
// Scoring as its own launch, for batches too small to fill the chip with one
// workgroup per (request, KV head): grid (ceil(C / (16 * kScoreTileWaves)),
// B * Hkv), each wave one 16-centroid tile, keys to p.keys; with p.arrive_heads it also clears
// the group's arrival counters of the split decode.
constexpr int kScoreTileWaves = 2;  // 16-centroid tiles (one a wave) per scoring workgroup; 2 beat 4 and 8
template <int G>
__global__ __launch_bounds__(kScoreTileWaves * kWave) void centroid_score_kernel(SelectParams p) {
  const int bg = blockIdx.y;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  // the split decode's arrival counters of the group, for the launch after
  if (p.arrive_heads && blockIdx.x == 0 && threadIdx.x < G) p.arrive_heads[bg * G + threadIdx.x] = 0u;
  const int t = blockIdx.x * kScoreTileWaves + static_cast<int>(threadIdx.x) / kWave;
  const int ntile = (p.C + 15) / 16;
  if (t >= ntile) return;  // uniform over the wave
  score_tiles_mfma<G>(p, b, g, t, t + 1, p.keys + static_cast<long long>(bg) * G * p.C);
}

template <typename T, int G, int KPL, int NW>
__global__ __launch_bounds__(NW * kWave) void ivf_select_kernel(SelectParams p) {
  constexpr int NT = NW * kWave;
  extern __shared__ uint32_t smem[];
  const int C = p.C, k = p.k;
  uint32_t* keys = smem;                              // [G][C]
  uint32_t* lmask = smem + G * C;                     // [C]
  int* loff = reinterpret_cast<int*>(smem + (G + 1) * C);  // [C+1], clamped to [0, N]
  int* llen = loff + C + 1;                           // [C] valid entries per list (p.lens_lds only)
  __shared__ int class_scratch[NW * (G + 2)];
  __shared__ __align__(16) uint64_t cand_lds[NW][2 * kWave];
  const int bg = blockIdx.x;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = lane >> 4, e = lane & 15;

  // Every global read the selection waits on is requested before the first
  // wait: the list offsets into registers (clamped addresses, straight-line
  // loads), then the scores' operands (or the scores themselves); the
  // offsets reach LDS after the scoring.
  const int32_t* off = p.offsets + static_cast<long long>(bg) * (C + 1);
  const int32_t* lens = p.lens ? p.lens + static_cast<long long>(bg) * C : nullptr;
  constexpr int kOffPer = (KPL * kWave + NT) / NT;  // C + 1 <= 64 * KPL + 1 offsets
  int offv[kOffPer], lenv[kOffPer];
  // a dynamic index's list lengths are staged in LDS beside the offsets when
  // they fit in the 64 KiB of dynamic LDS, else read where used
  const bool lens_lds = lens && p.lens_lds;
#pragma unroll
  for (int i = 0; i < kOffPer; ++i) offv[i] = off[min(tid + i * NT, C)];
  if (lens_lds) {
#pragma unroll
    for (int i = 0; i < kOffPer; ++i) lenv[i] = lens[min(tid + i * NT, C - 1)];
  }
  for (int c = tid; c < C; c += NT) lmask[c] = 0u;
  if (p.keys) {  // scored by centroid_score_kernel: staged beside the offsets, 16 loads in flight
    const uint32_t* kg = p.keys + static_cast<long long>(bg) * G * C;
    for (int i0 = 0; i0 < G * C; i0 += 16 * NT) {
      uint32_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * NT + tid;
        v[u] = i < G * C ? kg[i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = i0 + u * NT + tid;
        if (i < G * C) keys[i] = v[u];
      }
    }
  } else if constexpr (std::is_same<T, bf16_t>::value) {
    const int ntile = (C + 15) / 16;
    const int per_wave = (ntile + NW - 1) / NW;
    score_tiles_mfma<G>(p, b, g, wave * per_wave, min(ntile, (wave + 1) * per_wave), keys);
  } else {
    score_rows_valu<T, G, NW, 16>(p, b, g, wave, keys);
  }
#pragma unroll
  for (int i = 0; i < kOffPer; ++i) {
    const int c = tid + i * NT;
    if (c <= C) loff[c] = min(max(offv[i], 0), p.n_entries);
    if (lens_lds && c < C) llen[c] = lenv[i];
  }
  __syncthreads();
  // rows of list c: its whole range, or (dynamic index) the valid front part
  auto list_len = [&](int c) {
    const int range = max(loff[c + 1] - loff[c], 0);
    return lens ? min(max(lens_lds ? llen[c] : lens[c], 0), range) : range;
  };

  for (int h = wave; h < G; h += NW) {
    const uint32_t* kh = keys + h * C;
    // lane holds keys c = j * 64 + lane (ascending c by j); 0 marks "no list"
    // and sits below every real key
    uint32_t kk[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int c = j * kWave + lane;
      kk[j] = c < C ? kh[c] : 0u;
    }
    const int qh = g * G + h;
    int32_t* sel = p.sel_out ? p.sel_out + (static_cast<long long>(b) * p.Hkv * G + qh) * k : nullptr;
    int rows = 0;
    topk_lists<KPL>(kk, k, cand_lds[wave], [&](int c, int pos) {
      if (sel) sel[pos] = c;
      atomicOr(&lmask[c], 1u << h);
      rows += list_len(c);
    });
    rows = wave_sum_i(rows);
    if (p.rows_out && lane == 0) p.rows_out[static_cast<long long>(b) * p.Hkv * G + qh] = rows;
  }
  __syncthreads();
  if (p.lmask_out)  // the chosen lists' head masks, for the gather's duplicate test
    for (int c = tid; c < C; c += NT) p.lmask_out[static_cast<long long>(bg) * C + c] = lmask[c];

  // Thread t plans lists [t * PER, (t + 1) * PER); their head masks,
  // offsets and lengths come from LDS once, all PER together, into
  // registers. For merged gather sets the segments are ordered by head
  // class: the lists only head 0 chose, then those only head 1 chose, ...,
  // then the lists several heads chose; within a class, list order.
  // Consecutive segments then mostly share one head, so a gather workgroup
  // that takes several of them merges their states into one per head.
  // Otherwise they follow list order. One block scan of the per-thread
  // counts (of every class) places them.
  int4* seg = p.seg + static_cast<long long>(bg) * p.smax;
  // plan segments are a power of two long (they halve from kSegRows)
  const int sr_log = 31 - __builtin_clz(static_cast<uint32_t>(min(max(p.seg_rows, 1), kSegRows)));
  const int sr = 1 << sr_log;
  constexpr int PER = (KPL * kWave + NT - 1) / NT;  // C <= 64 * KPL lists over NT threads
  const int c_lo = tid * PER;
  uint32_t lm[PER];
  int lst[PER], lln[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = min(c_lo + i, C - 1);
    const uint32_t m = lmask[c];
    const int len = list_len(c);
    const bool use = c_lo + i < C && m != 0u && len > 0;
    lm[i] = use ? m : 0u;
    lln[i] = use ? len : 0;
    lst[i] = loff[c];
  }
  int carry, uniq_all;
  if (p.class_order) {
    // class of a chosen list: its head if one head chose it, else G
    auto class_of = [&](uint32_t m) { return (m & (m - 1u)) == 0u ? static_cast<int>(__builtin_ctz(m)) : G; };
    int cls_segs[G + 1], cls_pos[G + 1];
#pragma unroll
    for (int x = 0; x <= G; ++x) cls_segs[x] = 0;
    int uniq = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int cl = lm[i] ? class_of(lm[i]) : G, ns = (lln[i] + sr - 1) >> sr_log;
#pragma unroll
      for (int x = 0; x <= G; ++x) cls_segs[x] += x == cl ? ns : 0;
      uniq += lln[i];
    }
    block_class_scan<NW, G + 1>(cls_segs, cls_pos, uniq, class_scratch, &carry, &uniq_all);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (lln[i] == 0) continue;
      const int cl = class_of(lm[i]), ns = (lln[i] + sr - 1) >> sr_log;
      int pos = 0;
#pragma unroll
      for (int x = 0; x <= G; ++x) {
        if (x == cl) {
          pos = cls_pos[x];
          cls_pos[x] += ns;
        }
      }
      for (int j = 0; j < ns; ++j, ++pos) {
        if (pos < p.smax)
          seg[pos] = make_int4(lst[i] + (j << sr_log), min(sr, lln[i] - (j << sr_log)), static_cast<int>(lm[i]),
                               c_lo + i);
      }
    }
  } else {
    int my_segs = 0, uniq = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      my_segs += (lln[i] + sr - 1) >> sr_log;
      uniq += lln[i];
    }
    int pos = block_exclusive_scan_and_sum<NW>(my_segs, uniq, class_scratch, &carry, &uniq_all);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ns = (lln[i] + sr - 1) >> sr_log;
      for (int j = 0; j < ns; ++j, ++pos) {
        if (pos < p.smax)
          seg[pos] = make_int4(lst[i] + (j << sr_log), min(sr, lln[i] - (j << sr_log)), static_cast<int>(lm[i]),
                               c_lo + i);
      }
    }
  }
  // Fixed token ranges attended beside the lists by every head of the group
  // (the first n_sink tokens and the last n_window before the request's
  // length), as direct segments (list -1); the gather skips list rows that
  // fall inside them, so each row is attended once.
  if (p.n_sink > 0 || p.n_window > 0) {
    const int L = p.lengths ? min(max(p.lengths[b], 0), p.N) : p.N;
    const int sink_hi = min(p.n_sink, L);
    const int win_lo = p.n_window > 0 ? max(L - p.n_window, sink_hi) : L;
    const int nsink = (sink_hi + sr - 1) >> sr_log;
    const int nwin = (L - win_lo + sr - 1) >> sr_log;
    const int all = (1 << G) - 1;
    for (int j = tid; j < nsink + nwin; j += NT) {
      const int start = j < nsink ? j << sr_log : win_lo + ((j - nsink) << sr_log);
      const int cnt = min(sr, (j < nsink ? sink_hi : L) - start);
      if (carry + j < p.smax) seg[carry + j] = make_int4(start, cnt, all, -1);
    }
    carry += nsink + nwin;
  }
  if (tid == 0) {
    p.nseg[bg] = min(carry, p.smax);
    if (p.uniq_out) p.uniq_out[bg] = uniq_all;
  }
}

// ============================================================================
// Per-step KV and index append ([KARAT] worked example, step 6: after each
// step the new KV entry is stored and added to its posting list). One
// workgroup (4 waves) per (request, KV head): the new row goes to the cache;
// its key is scored against every centroid (|c|^2 - 2 k.c, 16 lanes per
// centroid row, DPP reduction, kAppendU rows in flight per lane group), the
// M best (distance, index) pairs are merged lexicographically over lane
// groups and waves, and the id is written at the end of the valid entries of
// each of the M lists (with its other lists in alt) when every one of them
// still has a free entry, else into none.
// ============================================================================
// One workgroup per (request, KV head); its NW waves split the codebook,
// append_unroll<T>() centroids per lane group in flight. With only B * Hkv
// workgroups the scan is bound by loads in flight per CU, so small batches
// with large codebooks take up to 16 waves. The position is checked only
// after the scan, so that its load overlaps the codebook's.
template <typename T>
constexpr int append_unroll() { return sizeof(T) == 2 ? 16 : 8; }

template <typename T, int M, int NW>
__global__ __launch_bounds__(NW * kWave) void kv_append_kernel(AppendParams p) {
  constexpr int U = append_unroll<T>();
  __shared__ float wbest[NW][M];
  __shared__ int wbestc[NW][M];
  const int bg = blockIdx.x;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave, r = lane >> 4, e = lane & 15;
  const int pos = p.pos[b];
  int32_t* st = p.status ? p.status + bg : nullptr;
  const long long src = static_cast<long long>(bg) * kHeadDim + e * 8;
  QFrag<T> kq;
  kq.load(static_cast<const T*>(p.new_k) + src);
  const T* cb = static_cast<const T*>(p.centroids) + b * p.cent_bstride +
                static_cast<long long>(g) * p.C * kHeadDim + e * 8;
  TopM<M> top;  // this lane group's M nearest, by (distance, centroid)
  top.init();
  constexpr int kStep = NW * U * 4;
  for (int c0 = wave * U * 4; c0 < p.C; c0 += kStep) {
    Raw8<T> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      raw[u].load(cb + static_cast<long long>(min(c0 + u * 4 + r, p.C - 1)) * kHeadDim);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * 4 + r;
      float x[8];
      raw[u].widen(x);
      float n2 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) n2 = fmaf(x[i], x[i], n2);
      const float dot = group16_sum(kq.dot(raw[u]));
      n2 = group16_sum(n2);
      if (c < p.C) top.push(n2 - 2.f * dot, c);
    }
  }
  // merge the lane groups' lists, then the waves'
#pragma unroll
  for (int o = 16; o < kWave; o <<= 1) {
    float od[M];
    int oc[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      od[i] = __shfl_xor(top.d[i], o);
      oc[i] = __shfl_xor(top.c[i], o);
    }
#pragma unroll
    for (int i = 0; i < M; ++i) top.push(od[i], oc[i]);
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      wbest[wave][i] = top.d[i];
      wbestc[wave][i] = top.c[i];
    }
  }
  if (pos < 0 || pos >= p.N) {  // uniform: nothing is written but the status
    if (st && tid == 0) *st = 2;
    return;
  }
  if (wave == 0 && r == 0) {
    const long long dst = ((static_cast<long long>(b) * p.N + pos) * p.Hkv + g) * kHeadDim + e * 8;
    Raw8<T> kr, vr;
    kr.load(static_cast<const T*>(p.new_k) + src);
    vr.load(static_cast<const T*>(p.new_v) + src);
    *reinterpret_cast<Raw8<T>*>(static_cast<T*>(p.k_cache) + dst) = kr;
    *reinterpret_cast<Raw8<T>*>(static_cast<T*>(p.v_cache) + dst) = vr;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int i = 0; i < M; ++i) top.push(wbest[w][i], wbestc[w][i]);
    // the key joins its M lists only if every one has a free entry
    const long long cap = static_cast<long long>(p.N) * M;
    const int32_t* off = p.offsets + static_cast<long long>(bg) * (p.C + 1);
    int32_t* lens = p.lens + static_cast<long long>(bg) * p.C;
    int start[M], len[M];
    bool room = true;
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const int c = min(max(top.c[i], 0), p.C - 1);
      start[i] = off[c];
      len[i] = lens[c];
      const int end = off[c + 1];
      room = room && start[i] >= 0 && end <= cap && len[i] >= 0 && start[i] + len[i] < end;
    }
    if (room) {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const long long e = static_cast<long long>(bg) * cap + start[i] + len[i];
        p.ids[e] = pos;
        if constexpr (M > 1) {  // the token's other lists, in its order of preference
#pragma unroll
          for (int q = 0; q < M - 1; ++q) p.alt[e * (M - 1) + q] = top.c[q + (q >= i ? 1 : 0)];
        }
        lens[min(max(top.c[i], 0), p.C - 1)] = len[i] + 1;
      }
    }
    if (st) *st = room ? 0 : 1;
  }
}

// Regrow: one workgroup per kRegrowChunk output entries of one (request, KV
// head). Each workgroup scans the lists' lengths (clamped to their ranges)
// into the new offsets, in LDS; an output entry finds its list by binary
// search and copies the list's entry (and its alt row) at the same place
// from the front of the old range, or writes -1 past the valid entries.
// When the valid entries plus the free ones exceed the capacity, nothing is
// written but the status.
template <int W>  // m - 1: the alt entries per list entry
__global__ __launch_bounds__(256) void regrow_kernel(RegrowParams p) {
  __shared__ int noff[kMaxCentroids + 1];
  __shared__ int soff[kMaxCentroids];
  __shared__ int nlen[kMaxCentroids];
  __shared__ int scratch[8];
  const int bg = blockIdx.y;
  const int tid = threadIdx.x;
  const int C = p.C;
  const long long cap = p.cap;
  const int32_t* off = p.offsets + static_cast<long long>(bg) * (C + 1);
  const int32_t* lens = p.lens + static_cast<long long>(bg) * C;
  // clamped valid lengths and their total
  int my_total = 0;
  for (int c = tid; c < C; c += 256) {
    const int lo = min(max(off[c], 0), p.cap), hi = min(max(off[c + 1], lo), p.cap);
    const int n = min(max(lens[c], 0), hi - lo);
    soff[c] = lo;
    nlen[c] = n;
    my_total += n;
  }
  const int total = block_sum<4>(my_total, scratch);
  int slack = p.slack;
  if (slack < 0) slack = static_cast<int>((cap - total) / C);
  const bool fits = slack >= 0 && total + static_cast<long long>(C) * slack <= cap;
  if (!fits) {
    if (blockIdx.x == 0 && tid == 0 && p.status) p.status[bg] = 1;
    return;  // uniform over the block
  }
  // new offsets: exclusive scan of (len + slack), 256 lists per round
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int c = c0 + tid;
    int tot;
    const int ex = block_exclusive_scan<4>(c < C ? nlen[c] + slack : 0, scratch, &tot);
    if (c < C) noff[c] = carry + ex;
    carry += tot;
  }
  if (tid == 0) noff[C] = carry;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int c = tid; c <= C; c += 256) p.offsets_out[static_cast<long long>(bg) * (C + 1) + c] = noff[c];
    for (int c = tid; c < C; c += 256) p.lens_out[static_cast<long long>(bg) * C + c] = nlen[c];
    if (tid == 0 && p.status) p.status[bg] = 0;
  }
  const int32_t* ids = p.ids + static_cast<long long>(bg) * cap;
  int32_t* ids_out = p.ids_out + static_cast<long long>(bg) * cap;
  const long long e_lo = static_cast<long long>(blockIdx.x) * kRegrowChunk;
  const long long e_hi = min(cap, e_lo + kRegrowChunk);
  // every entry's source first, then all loads, then all stores, so that
  // the loads of a thread's entries are in flight together
  // list of each entry: the last list whose new offset is <= the entry, by
  // a branch-free binary search run for all of a thread's entries in step
  int top_step = 1;
  while (top_step * 2 < C) top_step *= 2;
  int li[kRegrowPer];
#pragma unroll
  for (int i = 0; i < kRegrowPer; ++i) li[i] = 0;
  for (int step = top_step; step > 0; step >>= 1) {
#pragma unroll
    for (int i = 0; i < kRegrowPer; ++i) {
      const long long e = e_lo + tid + i * 256;
      const int cand = li[i] + step;
      if (cand < C && noff[cand] <= e) li[i] = cand;
    }
  }
  int src[kRegrowPer];
#pragma unroll
  for (int i = 0; i < kRegrowPer; ++i) {
    const long long e = e_lo + tid + i * 256;
    src[i] = -1;
    if (e < e_hi && e < carry) {
      const int j = static_cast<int>(e - noff[li[i]]);
      if (j < nlen[li[i]]) src[i] = soff[li[i]] + j;
    }
  }
  int v[kRegrowPer];
#pragma unroll
  for (int i = 0; i < kRegrowPer; ++i) v[i] = src[i] >= 0 ? ids[src[i]] : -1;
#pragma unroll
  for (int i = 0; i < kRegrowPer; ++i) {
    const long long e = e_lo + tid + i * 256;
    if (e < e_hi) ids_out[e] = v[i];
  }
  if constexpr (W > 0) {
    const int32_t* alt = p.alt + static_cast<long long>(bg) * cap * W;
    int32_t* alt_out = p.alt_out + static_cast<long long>(bg) * cap * W;
    int a[kRegrowPer][W];
#pragma unroll
    for (int i = 0; i < kRegrowPer; ++i)
#pragma unroll
      for (int q = 0; q < W; ++q) a[i][q] = src[i] >= 0 ? alt[static_cast<long long>(src[i]) * W + q] : -1;
#pragma unroll
    for (int i = 0; i < kRegrowPer; ++i) {
      const long long e = e_lo + tid + i * 256;
      if (e < e_hi)
#pragma unroll
        for (int q = 0; q < W; ++q) alt_out[e * W + q] = a[i][q];
    }
  }
}

hipError_t launch_regrow(const RegrowParams& p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.cap + kRegrowChunk - 1) / kRegrowChunk), p.B * p.Hkv);
  switch (p.m) {
    case 1: hipLaunchKernelGGL(regrow_kernel<0>, grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL(regrow_kernel<1>, grid, dim3(256), 0, s, p); break;
    case 3: hipLaunchKernelGGL(regrow_kernel<2>, grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL(regrow_kernel<3>, grid, dim3(256), 0, s, p); break;
  }
  return hipGetLastError();
}

// ============================================================================
// Launchers
// ============================================================================
hipError_t launch_assign(const AssignParams& p, int dtype, float* norms, hipStream_t s) {
  if (dtype == kBF16) {
    const long long rows = (p.cent_bstride ? static_cast<long long>(p.B) : 1LL) * p.Hkv * p.C;
    hipLaunchKernelGGL(centroid_norms_kernel, dim3(static_cast<unsigned>((rows * 16 + 255) / 256)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(p.centroids), norms, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((p.n_assign + kMfmaKb - 1) / kMfmaKb, p.B * p.Hkv), block(kMfmaWaves * kWave);
    const float* nf = norms;
    switch (p.m) {
      case 1: hipLaunchKernelGGL(assign_mfma_kernel<1>, grid, block, 0, s, p, nf); break;
      case 2: hipLaunchKernelGGL(assign_mfma_kernel<2>, grid, block, 0, s, p, nf); break;
      case 3: hipLaunchKernelGGL(assign_mfma_kernel<3>, grid, block, 0, s, p, nf); break;
      default: hipLaunchKernelGGL(assign_mfma_kernel<4>, grid, block, 0, s, p, nf); break;
    }
  } else {
    dim3 grid((p.n_assign + 255) / 256, p.B * p.Hkv);
    switch (p.m) {
      case 1: hipLaunchKernelGGL((assign_kernel<float, 1>), grid, dim3(256), 0, s, p); break;
      case 2: hipLaunchKernelGGL((assign_kernel<float, 2>), grid, dim3(256), 0, s, p); break;
      case 3: hipLaunchKernelGGL((assign_kernel<float, 3>), grid, dim3(256), 0, s, p); break;
      default: hipLaunchKernelGGL((assign_kernel<float, 4>), grid, dim3(256), 0, s, p); break;
    }
  }
  return hipGetLastError();
}

template <typename T, int NW>
static void append_dispatch(const AppendParams& p, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv), block(NW * kWave);
  switch (p.m) {
    case 1: hipLaunchKernelGGL((kv_append_kernel<T, 1, NW>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((kv_append_kernel<T, 2, NW>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((kv_append_kernel<T, 3, NW>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((kv_append_kernel<T, 4, NW>), grid, block, 0, s, p); break;
  }
}

hipError_t launch_kv_append(const AppendParams& p, int dtype, hipStream_t s) {
  // A wave takes append_unroll<T>() * 4 centroids per pass. While the
  // workgroups alone do not fill the CUs, enough waves for about one pass
  // over the codebook (16 at most); otherwise 4.
  const int per_wave = (dtype == kBF16 ? append_unroll<bf16_t>() : append_unroll<float>()) * 4;
  const bool few = static_cast<long long>(p.B) * p.Hkv < 256;
  const int nw = !few || p.C <= 4 * per_wave ? 4 : (p.C <= 8 * per_wave ? 8 : 16);
  if (dtype == kBF16) {
    if (nw == 16) append_dispatch<bf16_t, 16>(p, s);
    else if (nw == 8) append_dispatch<bf16_t, 8>(p, s);
    else append_dispatch<bf16_t, 4>(p, s);
  } else {
    if (nw == 16) append_dispatch<float, 16>(p, s);
    else if (nw == 8) append_dispatch<float, 8>(p, s);
    else append_dispatch<float, 4>(p, s);
  }
  return hipGetLastError();
}

// Up to kCsrMaxC lists: the ids staged in LDS when a (request, KV head)'s ids
// fit there and no second array is written (128 KiB leaves one workgroup per
// CU: 16 waves when the counters of up to kCsrSmallC lists fit beside the
// stage, else 4), else 16 waves writing to memory; larger codebooks take
// csr_kernel.
hipError_t launch_csr(const CsrParams& p, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv);
  const long long cap = static_cast<long long>(p.N) * p.m;
  if (p.C <= kCsrSmallC && !p.alt && cap <= kCsrStage)
    hipLaunchKernelGGL((csr_waves_kernel<16, true, kCsrSmallC>), grid, dim3(16 * kWave), 0, s, p);
  else if (p.C <= kCsrMaxC && !p.alt && cap <= kCsrStage)
    hipLaunchKernelGGL((csr_waves_kernel<4, true>), grid, dim3(4 * kWave), 0, s, p);
  else if (p.C <= kCsrMaxC)
    hipLaunchKernelGGL((csr_waves_kernel<16, false>), grid, dim3(16 * kWave), 0, s, p);
  else
    hipLaunchKernelGGL(csr_kernel, grid, dim3(256), p.C * sizeof(int), s, p);
  return hipGetLastError();
}

template <typename T, int KPL, int NW>
static void select_dispatch_g(const SelectParams& p, int G, size_t lds, hipStream_t s) {
  const dim3 grid(p.B * p.Hkv), block(NW * kWave);
  switch (G) {
    case 1: hipLaunchKernelGGL((ivf_select_kernel<T, 1, KPL, NW>), grid, block, lds, s, p); break;
    case 2: hipLaunchKernelGGL((ivf_select_kernel<T, 2, KPL, NW>), grid, block, lds, s, p); break;
    case 4: hipLaunchKernelGGL((ivf_select_kernel<T, 4, KPL, NW>), grid, block, lds, s, p); break;
    default: hipLaunchKernelGGL((ivf_select_kernel<T, 8, KPL, NW>), grid, block, lds, s, p); break;
  }
}

template <typename T>
static void select_dispatch(const SelectParams& p, int G, size_t lds, hipStream_t s) {
  if (p.C <= 64) select_dispatch_g<T, 1, kSelWaves>(p, G, lds, s);
  else if (p.C <= 256) select_dispatch_g<T, 4, kSelWaves>(p, G, lds, s);
  else if (p.C <= 1024) select_dispatch_g<T, 16, kSelWaves>(p, G, lds, s);
  else select_dispatch_g<T, kMaxCentroids / 64, kSelWaves>(p, G, lds, s);
}

// ============================================================================
// List-major copy of the K/V rows ([KARAT] How: an inverted file keeps its
// entries by list, so a chosen list is read as one contiguous stream).
// Workgroup (x, bg) copies entries [x * kListCopyRows, ...) of (request, KV
// head) bg: a row is kPieces 16-byte pieces, one per lane; each thread first
// reads the token ids of its kListCopyU rows, then has all their loads in
// flight before the stores.
// ============================================================================
constexpr int kListCopyThreads = 256;
constexpr int kListCopyRows = 256;  // entries per workgroup
constexpr int kListCopyU = 4;       // rows per thread in flight

template <typename T>
__global__ __launch_bounds__(kListCopyThreads) void kv_list_major_kernel(KvListsParams p) {
  constexpr int kPieces = kHeadDimRows * static_cast<int>(sizeof(T)) / 16;  // 16 (bf16) or 32 (fp32)
  constexpr int kElems = 16 / static_cast<int>(sizeof(T));                  // elements per piece
  constexpr int kRowsPerPass = kListCopyThreads / kPieces;
  static_assert(kListCopyRows % (kRowsPerPass * kListCopyU) == 0, "whole passes");
  const int bg = blockIdx.y;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int piece = threadIdx.x % kPieces, rsub = threadIdx.x / kPieces;
  const long long row_stride = static_cast<long long>(p.Hkv) * kHeadDimRows;  // elements between tokens
  const T* kb = static_cast<const T*>(p.k) + static_cast<long long>(b) * p.N * row_stride + g * kHeadDimRows +
                piece * kElems;
  const T* vb = static_cast<const T*>(p.v) + static_cast<long long>(b) * p.N * row_stride + g * kHeadDimRows +
                piece * kElems;
  const long long gbase = static_cast<long long>(bg) * p.N;  // first entry of the group
  T* kl = static_cast<T*>(p.kl) + gbase * kHeadDimRows + piece * kElems;
  T* vl = static_cast<T*>(p.vl) + gbase * kHeadDimRows + piece * kElems;
  const int32_t* ids = p.ids + gbase;
  const int e0 = blockIdx.x * kListCopyRows;
  for (int r0 = 0; r0 < kListCopyRows; r0 += kRowsPerPass * kListCopyU) {
    int e[kListCopyU], id[kListCopyU];
#pragma unroll
    for (int u = 0; u < kListCopyU; ++u) {
      e[u] = e0 + r0 + u * kRowsPerPass + rsub;
      id[u] = e[u] < p.N ? ids[e[u]] : -1;
    }
    uint4 kv[kListCopyU], vv[kListCopyU];
#pragma unroll
    for (int u = 0; u < kListCopyU; ++u) {
      const bool ok = static_cast<unsigned>(id[u]) < static_cast<unsigned>(p.N);
      const long long off = static_cast<long long>(ok ? id[u] : 0) * row_stride;  // id 0: in bounds
      kv[u] = load16_stream(kb + off);
      vv[u] = load16_stream(vb + off);
      if (!ok) kv[u] = vv[u] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kListCopyU; ++u) {
      if (e[u] < p.N) {
        *reinterpret_cast<uint4*>(kl + static_cast<long long>(e[u]) * kHeadDimRows) = kv[u];
        *reinterpret_cast<uint4*>(vl + static_cast<long long>(e[u]) * kHeadDimRows) = vv[u];
      }
    }
  }
}

hipError_t launch_kv_list_major(const KvListsParams& p, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((p.N + kListCopyRows - 1) / kListCopyRows), p.B * p.Hkv);
  if (dtype == kBF16) hipLaunchKernelGGL(kv_list_major_kernel<bf16_t>, grid, dim3(kListCopyThreads), 0, s, p);
  else hipLaunchKernelGGL(kv_list_major_kernel<float>, grid, dim3(kListCopyThreads), 0, s, p);
  return hipGetLastError();
}

template <int G>
static void score_dispatch_g(const SelectParams& p, hipStream_t s) {
  const dim3 grid((p.C + 16 * kScoreTileWaves - 1) / (16 * kScoreTileWaves), p.B * p.Hkv);
  hipLaunchKernelGGL(centroid_score_kernel<G>, grid, dim3(kScoreTileWaves * kWave), 0, s, p);
}

hipError_t launch_centroid_score(const SelectParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: score_dispatch_g<1>(p, s); break;
    case 2: score_dispatch_g<2>(p, s); break;
    case 4: score_dispatch_g<4>(p, s); break;
    default: score_dispatch_g<8>(p, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_ivf_select(const SelectParams& p, int dtype, int G, hipStream_t s) {
  if (p.keys) {  // bf16 only (checked by the caller)
    const hipError_t e = launch_centroid_score(p, G, s);
    if (e != hipSuccess) return e;
  }
  size_t lds = (static_cast<size_t>(G + 1) * p.C + p.C + 1) * sizeof(uint32_t);
  SelectParams q = p;
  q.lens_lds = p.lens && lds + p.C * sizeof(uint32_t) <= kSelectLdsBytes;
  if (q.lens_lds) lds += p.C * sizeof(uint32_t);
  if (dtype == kBF16) select_dispatch<bf16_t>(q, G, lds, s);
  else select_dispatch<float>(q, G, lds, s);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, long long n, int32_t value) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += 256LL * gridDim.x) p[i] = value;
}

hipError_t launch_fill_i32(int32_t* p, long long n, int32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

}  // namespace tsa
