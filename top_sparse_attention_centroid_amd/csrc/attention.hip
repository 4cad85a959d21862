// Gathered sparse attention for gfx950 ([KARAT] Eq. 2 with -inf outside the
// retrieved set; [KARAT] = paper-daily digest "Heterogeneous LLM Serving with
// General-Purpose Processing-Near-Memory for Retrieval-Based Sparse
// Attention").
//
// gather_attn: a segment is at most kSegRows rows of one (request, KV head),
// with the head mask of the GQA group's query heads that chose them, so a row
// chosen by several heads of the group is read from HBM once. Each wave owns
// whole segments: 16 lanes cover one 256-B bf16 row (16 B each), a wave load
// instruction fetches 4 rows, and every load of a batch of rows is issued
// before any arithmetic on it; latency is hidden by many resident waves.
// Each lane group keeps an online-softmax state (running max m, sum l,
// output o) in the log2 domain; the four lane groups merge by lane shuffles
// and the segment writes one partial (m, l, o) per masked head.
// gather_merge (large bf16 batches of inverted-index plans): the same wave
// work, but kMergeWaves waves of a workgroup take consecutive segments and
// merge their states per head in LDS, so the set writes one partial per head.
// combine: merges each query head's partials with the log-sum-exp rule (one
// wave per head in large batches, several in small ones) and writes o / l
// (zero when nothing was selected).
#include "attn_rows.hpp"
#include "device_common.hpp"
#include "kernels.hpp"

namespace tsa {

// waves per workgroup: explicit plans (uneven segments) run one wave per
// workgroup so a finished segment frees its slot at once; row lists (equal
// segments) run several
template <bool EXPLICIT>
constexpr int gather_waves() { return EXPLICIT ? kGatherWavesExplicit : kGatherWavesRows; }
constexpr int kSegsPerWave = kGatherSegsPerWave;    // segments a wave is planned to take
constexpr int kUnrollAll = 4;                      // all-heads pass: rows per lane group per batch
constexpr int kBatchRowsAll = 4 * kUnrollAll;

// gather_attn: every wave processes whole segments on its own (no block
// barrier after the q staging); a workgroup covers up to 4 segments of one
// (request, KV head) and exits, so the hardware dispatcher balances the
// uneven segments across CUs. Per segment: row ids -> wave-private LDS in one
// round trip; then, for each query head in the segment's mask, one pass over
// the rows in batches of kBatchRows (16 lanes per row, all loads of a batch in
// flight together); segments that every head reads (in large batches, two or
// more heads) take one all-heads pass instead (every row loaded once).
// Otherwise a second head's pass re-reads the rows the first pass just
// brought into L2. The four lane groups
// then merge and lanes 0..15 write the head's partial state.
// For each query head in `mask`: one pass over the segment's rows, then the
// four 16-lane row groups merge and lanes 0..15 write the head's partial.
// One query head's pass over rows ids[0, cnt): the returned state is merged
// over the four lane groups (every lane holds it; lanes 0..15 own o).
template <bool STREAM, bool DUP, typename T>
__device__ __forceinline__ HeadState head_pass(int h, const int* ids, int cnt, int r, int e, const T* kb,
                                               const T* vb, long long row_stride, const T* qs, float qscale,
                                               const uint32_t* dup) {
  {
    QFrag<T> qf;
    qf.load(qs + h * kHeadDim + e * 8);
    HeadState st;
    st.init();
    for (int base = 0; base < cnt; base += kBatchRows) {
      Batch<T> A;
      issue_batch<STREAM, DUP>(A, ids, base, cnt, r, kb, vb, row_stride, dup, h);
      consume_batch(A, st, qf, qscale);
    }
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      float o2[8];
      const float m2 = __shfl_xor(st.m, x);
      const float l2 = __shfl_xor(st.l, x);
#pragma unroll
      for (int t = 0; t < 8; ++t) o2[t] = __shfl_xor(st.o[t], x);
      merge_into(st, m2, l2, o2);
    }
    return st;
  }
}

template <bool STREAM, bool DUP, typename T>
__device__ __forceinline__ void head_passes(uint32_t mask, const int* ids, int cnt, int r, int e, const T* kb,
                                            const T* vb, long long row_stride, const T* qs, float qscale,
                                            float* part, const uint32_t* dup) {
  for (uint32_t hm = mask; hm != 0u; hm &= hm - 1u) {
    const int h = __builtin_ctz(hm);
    const HeadState st = head_pass<STREAM, DUP>(h, ids, cnt, r, e, kb, vb, row_stride, qs, qscale, dup);
    store_state(part + h * kPartStride, st, r, e);
  }
}

// Row lists shared by every head of the group (token selections, hot-cache
// slots): one pass scores each batch of rows for all G heads, so a row is
// loaded into registers once; G online-softmax states per lane group.
// `row_heads(j)` gives the heads that attend row j (a row outside a head's
// set is scored and dropped for it); the states come back merged over the
// four lane groups.
template <int G, typename T, typename RowHeads>
__device__ __forceinline__ void all_heads_states(HeadState (&st)[G], const int* ids, int cnt, int r, int e,
                                                 const T* kb, const T* vb, long long row_stride, const T* qs,
                                                 float qscale, RowHeads row_heads) {
  QFrag<T> qf[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    qf[h].load(qs + h * kHeadDim + e * 8);
    st[h].init();
  }
  for (int base = 0; base < cnt; base += kBatchRowsAll) {
    Raw8<T> k[kUnrollAll], v[kUnrollAll];
    bool valid[kUnrollAll];
    int row[kUnrollAll];
    uint32_t heads[kUnrollAll];
#pragma unroll
    for (int u = 0; u < kUnrollAll; ++u) {
      const int j = base + u * 4 + r;
      const int id = ids[min(j, kSegRows - 1)];
      valid[u] = (j < cnt) & (id >= 0);
      row[u] = valid[u] ? id : 0;
      heads[u] = row_heads(j);
    }
#pragma unroll
    for (int u = 0; u < kUnrollAll; ++u) k[u].load_stream(kb + row[u] * row_stride);
#pragma unroll
    for (int u = 0; u < kUnrollAll; ++u) v[u].load_stream(vb + row[u] * row_stride);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc[kUnrollAll];
#pragma unroll
      for (int u = 0; u < kUnrollAll; ++u)
        sc[u] = valid[u] && ((heads[u] >> h) & 1u) ? group16_sum(qf[h].dot(k[u])) * qscale : kMaskedScore;
      float mb = sc[0];
#pragma unroll
      for (int u = 1; u < kUnrollAll; ++u) mb = fmaxf(mb, sc[u]);
      const float mn = fmaxf(st[h].m, mb);
      const float a = fast_exp2(st[h].m - mn);
      st[h].l *= a;
#pragma unroll
      for (int i = 0; i < 8; ++i) st[h].o[i] *= a;
#pragma unroll
      for (int u = 0; u < kUnrollAll; ++u) {
        float vx[8];
        v[u].widen(vx);
        const float pw = fast_exp2(sc[u] - mn);
        st[h].l += pw;
#pragma unroll
        for (int i = 0; i < 8; ++i) st[h].o[i] = fmaf(pw, vx[i], st[h].o[i]);
      }
      st[h].m = mn;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      float o2[8];
      const float m2 = __shfl_xor(st[h].m, x);
      const float l2 = __shfl_xor(st[h].l, x);
#pragma unroll
      for (int t = 0; t < 8; ++t) o2[t] = __shfl_xor(st[h].o[t], x);
      merge_into(st[h], m2, l2, o2);
    }
  }
}

template <int G, typename T>
__device__ __forceinline__ void all_heads_pass(uint32_t mask, const int* ids, int cnt, int r, int e, const T* kb,
                                               const T* vb, long long row_stride, const T* qs, float qscale,
                                               float* part) {
  HeadState st[G];
  all_heads_states<G>(st, ids, cnt, r, e, kb, vb, row_stride, qs, qscale, [](int) { return ~0u; });
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // heads outside the mask were scored with the others but are not merged
    if ((mask >> h) & 1u) store_state(part + h * kPartStride, st[h], r, e);
  }
}

// Heads of the group that attend an m-way list entry through a lower chosen
// list: the OR of the chosen-list head masks of the entry's other lists
// (alt row of w = m - 1 ids) that are numbered below `list`.
__device__ __forceinline__ uint32_t dup_heads(const int32_t* alt_row, int w, int list, const uint32_t* lmask,
                                              int C) {
  uint32_t dm = 0u;
  for (int q = 0; q < w; ++q) {
    const int other = alt_row[q];
    if (other >= 0 && other < list && other < C) dm |= lmask[other];
  }
  return dm;
}

// DUP: explicit plans over m-way lists, with per-row duplicate head masks
template <typename T, int G, bool EXPLICIT, bool DUP>
__device__ __forceinline__ void gather_attn_body(const GatherParams& p) {
  constexpr int NW = gather_waves<EXPLICIT>();
  __shared__ __align__(16) T qs[G * kHeadDim];
  __shared__ int ids_lds[NW][kSegRows];
  __shared__ uint32_t dup_lds[DUP ? NW : 1][DUP ? kSegRows : 1];
  const int bg = blockIdx.x / p.W, w0 = blockIdx.x % p.W;
  const int b = bg / p.Hkv, g = bg % p.Hkv;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = lane >> 4, e = lane & 15;
  const int s_first = w0 * NW + wave;
  const int stride = p.W * NW;

  // A wave takes segments s_first, s_first + stride, ... (about kSegsPerWave
  // of them). Everything its first rows depend on is requested together:
  // the segment count, the group's queries (block-wide, staged to LDS) and
  // the descriptors of all its segments; then the first segment's row ids.
  // While a segment's rows stream, the next segment's row ids are already
  // in flight into registers, so only the first segment waits for them.
  int nseg, total_rows = 0;
  int4 dq[kSegsPerWave];
  if constexpr (EXPLICIT) {
    nseg = p.nseg[bg];
#pragma unroll
    for (int i = 0; i < kSegsPerWave; ++i)
      dq[i] = p.seg[static_cast<long long>(bg) * p.smax + min(s_first + i * stride, p.smax - 1)];
  } else {
    // clamp a device-side count to the planned capacity (never trusted)
    total_rows = min(max(p.counts ? p.counts[b] : p.count_const, 0), p.count_max);
    nseg = (total_rows + p.seg_rows - 1) / p.seg_rows;
#pragma unroll
    for (int i = 0; i < kSegsPerWave; ++i) dq[i] = make_int4(0, 0, 0, 0);
  }
  constexpr int kQParts = G * kHeadDim / 8;  // 16-B (bf16) or 32-B (fp32) pieces of the group's queries
  constexpr int kQPer = (kQParts + NW * kWave - 1) / (NW * kWave);
  Raw8<T> qpart[kQPer];
  const T* qb = static_cast<const T*>(p.q) + (static_cast<long long>(b) * p.Hkv + g) * G * kHeadDim;
#pragma unroll
  for (int i = 0; i < kQPer; ++i)
    if (tid + i * NW * kWave < kQParts) qpart[i].load(qb + (tid + i * NW * kWave) * 8);
  if (w0 * NW >= nseg) return;  // uniform over the block

  // explicit plans: list segments read the list-major copies by entry when
  // given (every segment is then a list segment)
  const bool by_entry = EXPLICIT && p.kl != nullptr;
  const long long ebase = b * p.rid_bstride + g * p.rid_gstride;  // first row id / entry of the group
  const long long row_stride = by_entry ? kHeadDim : static_cast<long long>(p.Hkv) * kHeadDim;
  const T* kb = by_entry ? static_cast<const T*>(p.kl) + ebase * kHeadDim + e * 8
                         : static_cast<const T*>(p.k) + static_cast<long long>(b) * p.n_rows * row_stride +
                               g * kHeadDim + e * 8;
  const T* vb = by_entry ? static_cast<const T*>(p.vl) + ebase * kHeadDim + e * 8
                         : static_cast<const T*>(p.v) + static_cast<long long>(b) * p.n_rows * row_stride +
                               g * kHeadDim + e * 8;
  const long long row_limit = by_entry ? p.rid_gstride : p.n_rows;
  const int32_t* rid = p.rowids + ebase;
  int* ids = ids_lds[wave];
  // sink / window ranges of an explicit plan: attended through their own
  // direct segments, so list rows inside them are skipped (empty by default)
  int fx_sink = 0, fx_lo = 0, fx_hi = 0;
  if constexpr (EXPLICIT) {
    if (p.n_sink > 0 || p.n_window > 0) {
      const int L = p.lengths ? min(max(p.lengths[b], 0), static_cast<int>(p.n_rows)) : static_cast<int>(p.n_rows);
      fx_sink = min(p.n_sink, L);
      fx_lo = p.n_window > 0 ? max(L - p.n_window, fx_sink) : L;
      fx_hi = L;
    }
  }

  // segment s: rows [start, start + cnt) of the list or token range, its head mask
  struct Seg {
    int start, cnt;
    uint32_t mask;
    bool direct;  // a token range [start, start + cnt) instead of list entries
    int list;     // the posting list (explicit plans)
  };
  auto seg_of = [&](int s, int4 d) {
    Seg sg;
    if constexpr (EXPLICIT) {
      sg.start = d.x;
      sg.cnt = min(max(d.y, 0), kSegRows);
      sg.mask = static_cast<uint32_t>(d.z);
      sg.direct = d.w < 0;
      sg.list = d.w;
    } else {
      sg.start = s * p.seg_rows;
      sg.cnt = min(p.seg_rows, total_rows - sg.start);
      sg.mask = (1u << G) - 1u;
      sg.direct = false;
      sg.list = -1;
    }
    return sg;
  };
  // m-way lists: a token sits in m lists; for each head the entry of the
  // lowest chosen list is the one attended (per-row duplicate head masks)
  constexpr bool two_way = DUP;
  uint32_t* dup = DUP ? dup_lds[DUP ? wave : 0] : nullptr;
  const int32_t* altb = two_way ? p.alt + (b * p.rid_bstride + g * p.rid_gstride) * p.alt_w : nullptr;
  auto stage_dup = [&](const Seg& sg) {
    if constexpr (!DUP) return;
    for (int j = lane; j < sg.cnt; j += kWave) {
      uint32_t dm = 0u;
      if (!sg.direct) dm = dup_heads(altb + static_cast<long long>(sg.start + j) * p.alt_w, p.alt_w, sg.list,
                                     p.lmask + static_cast<long long>(bg) * p.C, p.C);
      dup[j] = dm;
    }
  };
  constexpr int kIdsPerLane = kSegRows / kWave;
  // a segment's row ids into registers: straight-line loads at clamped
  // positions (cnt >= 1 for every planned segment), filtered when stored
  auto load_ids = [&](const Seg& sg, int (&dst)[kIdsPerLane]) {
#pragma unroll
    for (int i = 0; i < kIdsPerLane; ++i) {
      const int j = min(lane + i * kWave, max(sg.cnt - 1, 0));
      dst[i] = sg.direct || by_entry ? sg.start + j : rid[sg.start + j];
    }
  };
  auto store_ids = [&](const Seg& sg, const int (&src)[kIdsPerLane]) {
#pragma unroll
    for (int i = 0; i < kIdsPerLane; ++i) {
      const int j = lane + i * kWave;
      const int id = src[i];
      // ids outside [0, n_rows) (entries outside the group) are skipped,
      // never dereferenced
      bool ok = static_cast<unsigned long long>(id) < static_cast<unsigned long long>(row_limit);
      if (!sg.direct) ok = ok && !(id < fx_sink || (id >= fx_lo && id < fx_hi));
      if (j < sg.cnt) ids[j] = ok ? id : -1;
    }
  };

  Seg cur = seg_of(s_first, dq[0]);
  int cid[kIdsPerLane];
  if (s_first < nseg && cur.cnt > 0) load_ids(cur, cid);
#pragma unroll
  for (int i = 0; i < kQPer; ++i)
    if (tid + i * NW * kWave < kQParts) *reinterpret_cast<Raw8<T>*>(qs + (tid + i * NW * kWave) * 8) = qpart[i];
  if (s_first < nseg && cur.cnt > 0) {
    store_ids(cur, cid);
    stage_dup(cur);
  }
  __syncthreads();

  for (int it = 0, s = s_first; s < nseg; ++it, s += stride) {
    const int cnt = cur.cnt;
    const uint32_t mask = cur.mask;
    // the next segment's row ids fly while this one's rows stream
    const int sn = s + stride;
    Seg nxt;
    int nid[kIdsPerLane];
    const bool has_next = sn < nseg;
    if (has_next) {
      int4 dn = make_int4(0, 0, 0, 0);
      if constexpr (EXPLICIT) {
        dn = it + 1 < kSegsPerWave ? dq[(it + 1) % kSegsPerWave]
                                   : p.seg[static_cast<long long>(bg) * p.smax + sn];
      }
      nxt = seg_of(sn, dn);
      if (nxt.cnt > 0) load_ids(nxt, nid);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float* part = p.partial + (static_cast<long long>(bg) * p.smax + s) * G * kPartStride;
    // Rows read by one head stream past the caches in that head's pass. Rows
    // that every head of the group reads are loaded once and scored for all
    // heads in one pass; with multi_all (large batches, bound by bandwidth)
    // so are rows that two or more heads read (heads outside the mask are
    // scored and dropped; only the mask's states are written). Otherwise such rows
    // stay cacheable, one pass per head, the later passes hitting L2: a
    // small batch is bound by the latency of its waves, which the extra
    // heads' arithmetic would lengthen. (m-way lists keep per-head passes:
    // their duplicate masks differ per head.)
    const bool all_heads =
        !EXPLICIT || (G > 1 && !two_way &&
                      (mask == (1u << G) - 1u || (p.multi_all && (mask & (mask - 1u)) != 0u)));
    if (all_heads) {
      all_heads_pass<G>(mask, ids, cnt, r, e, kb, vb, row_stride, qs, p.qscale, part);
    } else if (kGatherStream && (mask & (mask - 1u)) == 0u) {
      head_passes<true, DUP>(mask, ids, cnt, r, e, kb, vb, row_stride, qs, p.qscale, part, dup);
    } else {
      head_passes<false, DUP>(mask, ids, cnt, r, e, kb, vb, row_stride, qs, p.qscale, part, dup);
    }
    // the next segment overwrites this wave's id staging area
    __builtin_amdgcn_wave_barrier();
    if (has_next) {
      cur = nxt;
      if (cur.cnt > 0) {
        store_ids(cur, nid);
        stage_dup(cur);
      }
    }
  }
}

// gather_merge: explicit plans in large batches. A workgroup of kMergeWaves
// waves takes kMergeWaves consecutive plan segments of one (request, KV
// head), a segment per wave; the plan lists the single-head lists head by
// head, so they mostly share one head. The waves merge their states per
// head through LDS and the workgroup writes one partial state per head of
// the set instead of one per segment and head: each written state costs its
// wave a store round trip before the wave retires, and the HBM a write-back
// amid the row stream. Set t covers segments [t * kMergeWaves,
// (t + 1) * kMergeWaves); its states sit at segment slot t * kMergeWaves.
// (Splitting a set's rows evenly over the waves, or aligning each head class
// to a set with empty segments, measured slower: the first adds a barrier
// between staging and streaming, the second idle waves.)
// DUP: m-way lists, whose rows carry per-head duplicate masks (each head
// attends a token through the lowest of its chosen lists that hold it);
// every head of a segment then takes its own pass.
template <typename T, int G, bool DUP>
__device__ __forceinline__ void gather_merge_body(const GatherParams& p) {
  constexpr int NW = kMergeWaves;
  constexpr int kHeadsPerWave = (G + NW - 1) / NW;  // heads each wave merges
  __shared__ __align__(16) T qs[G * kHeadDim];
  __shared__ int ids_lds[NW][kSegRows];
  __shared__ uint32_t dup_lds[DUP ? NW : 1][DUP ? kSegRows : 1];
  __shared__ float sm_m[NW][G], sm_l[NW][G];
  __shared__ __align__(16) float sm_o[NW][G][kHeadDim];
  const int bg = blockIdx.x / p.W, w0 = blockIdx.x % p.W;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int r = lane >> 4, e = lane & 15;

  const int nseg = min(max(p.nseg[bg], 0), p.smax);
  constexpr int kQParts = G * kHeadDim / 8;
  constexpr int kQPer = (kQParts + NW * kWave - 1) / (NW * kWave);
  Raw8<T> qpart[kQPer];
  const T* qb = static_cast<const T*>(p.q) + (static_cast<long long>(b) * p.Hkv + g) * G * kHeadDim;
#pragma unroll
  for (int i = 0; i < kQPer; ++i)
    if (tid + i * NW * kWave < kQParts) qpart[i].load(qb + (tid + i * NW * kWave) * 8);
  if (w0 * NW >= nseg) return;  // uniform over the block
#pragma unroll
  for (int i = 0; i < kQPer; ++i)
    if (tid + i * NW * kWave < kQParts) *reinterpret_cast<Raw8<T>*>(qs + (tid + i * NW * kWave) * 8) = qpart[i];

  // list segments read the list-major copies by entry when given (every
  // segment is then a list segment: no sink / window ranges, m = 1)
  const bool by_entry = p.kl != nullptr;
  const long long ebase = b * p.rid_bstride + g * p.rid_gstride;  // first entry of the group
  const long long row_stride = by_entry ? kHeadDim : static_cast<long long>(p.Hkv) * kHeadDim;
  const T* kb = by_entry ? static_cast<const T*>(p.kl) + ebase * kHeadDim + e * 8
                         : static_cast<const T*>(p.k) + static_cast<long long>(b) * p.n_rows * row_stride +
                               g * kHeadDim + e * 8;
  const T* vb = by_entry ? static_cast<const T*>(p.vl) + ebase * kHeadDim + e * 8
                         : static_cast<const T*>(p.v) + static_cast<long long>(b) * p.n_rows * row_stride +
                               g * kHeadDim + e * 8;
  const long long row_limit = by_entry ? p.rid_gstride : p.n_rows;  // entries of a group, or tokens
  const int32_t* rid = p.rowids + ebase;
  int* ids = ids_lds[wave];
  uint32_t* dup = dup_lds[DUP ? wave : 0];
  const int32_t* altb = DUP ? p.alt + (b * p.rid_bstride + g * p.rid_gstride) * p.alt_w : nullptr;
  // sink / window ranges: list rows inside them are skipped (attended
  // through their own direct segments)
  int fx_sink = 0, fx_lo = 0, fx_hi = 0;
  if (p.n_sink > 0 || p.n_window > 0) {
    const int L = p.lengths ? min(max(p.lengths[b], 0), static_cast<int>(p.n_rows)) : static_cast<int>(p.n_rows);
    fx_sink = min(p.n_sink, L);
    fx_lo = p.n_window > 0 ? max(L - p.n_window, fx_sink) : L;
    fx_hi = L;
  }

  for (int t = w0; t * NW < nseg; t += p.W) {  // uniform over the block
    const int s0 = t * NW;
    // every wave reads the set's descriptors (the same addresses): its own
    // segment, and the head masks of all of them
    uint32_t msk[NW];
    int my_start = 0, my_cnt = 0, my_list = -1;
    bool my_direct = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const bool in = s0 + i < nseg;
      const int4 d = p.seg[static_cast<long long>(bg) * p.smax + min(s0 + i, nseg - 1)];
      msk[i] = in ? static_cast<uint32_t>(d.z) & ((1u << G) - 1u) : 0u;
      if (i == wave) {
        my_start = d.x;
        my_cnt = in ? min(max(d.y, 0), kSegRows) : 0;
        my_direct = d.w < 0;
        my_list = d.w;
      }
    }
    uint32_t U = 0u, my_mask = 0u;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      U |= msk[i];
      my_mask = i == wave ? msk[i] : my_mask;
    }
    // the wave's row ids into its LDS area; ids outside [0, n_rows) are
    // skipped, never dereferenced
    for (int j = lane; j < my_cnt; j += kWave) {
      const int id = my_direct || by_entry ? my_start + j : rid[my_start + j];
      bool ok = static_cast<unsigned long long>(id) < static_cast<unsigned long long>(row_limit);
      if (!my_direct) ok = ok && !(id < fx_sink || (id >= fx_lo && id < fx_hi));
      ids[j] = ok ? id : -1;
      if constexpr (DUP) {  // heads that attend this token through a lower chosen list
        dup[j] = my_direct ? 0u
                           : dup_heads(altb + static_cast<long long>(my_start + j) * p.alt_w, p.alt_w, my_list,
                                       p.lmask + static_cast<long long>(bg) * p.C, p.C);
      }
    }
    __syncthreads();  // queries staged (first set); the ids are wave-private

    auto put = [&](int h, const HeadState& st) {
      if (r == 0) {
        *reinterpret_cast<float4*>(&sm_o[wave][h][e * 8]) = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
        *reinterpret_cast<float4*>(&sm_o[wave][h][e * 8 + 4]) = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
        if (e == 0) {
          sm_m[wave][h] = st.m;
          sm_l[wave][h] = st.l;
        }
      }
    };
    if (DUP && (my_mask & (my_mask - 1u)) != 0u) {
      // several heads with per-head duplicate masks: a cacheable pass each
      for (uint32_t hm = my_mask; hm != 0u; hm &= hm - 1u) {
        const int h = __builtin_ctz(hm);
        put(h, head_pass<false, DUP>(h, ids, my_cnt, r, e, kb, vb, row_stride, qs, p.qscale, dup));
      }
    } else if (my_mask != 0u && (my_mask & (my_mask - 1u)) == 0u) {
      const int h = __builtin_ctz(my_mask);
      put(h, head_pass<kGatherStream, DUP>(h, ids, my_cnt, r, e, kb, vb, row_stride, qs, p.qscale, dup));
    } else if (my_mask != 0u) {  // a list several heads chose, or a sink / window range
      HeadState st[G];
      all_heads_states<G>(st, ids, my_cnt, r, e, kb, vb, row_stride, qs, p.qscale, [](int) { return ~0u; });
#pragma unroll
      for (int h = 0; h < G; ++h)
        if ((my_mask >> h) & 1u) put(h, st[h]);
    }
    __syncthreads();

    // wave w merges heads w, w + NW, ... of the set: log-sum-exp over the
    // states of the waves whose segment the head attended, in wave order
#pragma unroll
    for (int hh = 0; hh < kHeadsPerWave; ++hh) {
      const int h = wave + hh * NW;
      if (h >= G || !((U >> h) & 1u)) continue;  // uniform over the wave
      float M = kEmptyMax;
#pragma unroll
      for (int i = 0; i < NW; ++i) M = (msk[i] >> h) & 1u ? fmaxf(M, sm_m[i][h]) : M;
      float L = 0.f, O0 = 0.f, O1 = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        if (!((msk[i] >> h) & 1u)) continue;
        const float a = fast_exp2(sm_m[i][h] - M);
        const float2 o = *reinterpret_cast<const float2*>(&sm_o[i][h][lane * 2]);
        L = fmaf(sm_l[i][h], a, L);
        O0 = fmaf(o.x, a, O0);
        O1 = fmaf(o.y, a, O1);
      }
      float* ph = p.partial + ((static_cast<long long>(bg) * p.smax + s0) * G + h) * kPartStride;
      *reinterpret_cast<float2*>(ph + kPartO + lane * 2) = make_float2(O0, O1);
      if (lane < kPartO / 4)
        *reinterpret_cast<float4*>(ph + lane * 4) = lane == 0 ? make_float4(M, L, 0.f, 0.f) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if ((t + p.W) * NW < nseg) __syncthreads();  // the next set reuses the LDS
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

// combine: a workgroup merges GH query heads of one (request, KV head), NS
// waves per head. Wave `part` of head h takes the head's segments part,
// part + NS, ...; its lanes read 64 segment descriptors and partial (m, l)
// at once, so the log-sum-exp weights come from two wave reductions; the o
// vectors are then accumulated with eight independent loads in flight per
// lane. Large batches run GH = G heads with one wave each and read only the
// head's own (m, l). Small batches, where the merge is a chain of round
// trips, run one head per workgroup with kCombineWavesSmall waves: the
// descriptors and (m, l) are requested together, and the NS partial states
// of the head are merged through LDS in a fixed order.
constexpr int kCombineWavesSmall = 8;  // waves per head when the batch is small (8 beat 16 at 16 x 8 token selections)

// The calling wave's share of query head h's partial states in group bg:
// records part, part + NS, ... merged into (M, L, O0, O1), lane l holding
// o[2l], o[2l + 1].
template <int G, int NS, bool EXPLICIT>
__device__ __forceinline__ void combine_partials(const GatherParams& p, int bg, int h, int part, float& M, float& L,
                                                 float& O0, float& O1) {
  constexpr int kU = 8;
  const int b = bg / p.Hkv;
  const int lane = lane_id();
  // records: one per segment, or with merged sets (gather_merge_kernel) one
  // per set of kMergeWaves segments at slot set * kMergeWaves, covering the
  // heads of all its segments
  int nseg, rs = 1;
  if constexpr (EXPLICIT) {
    nseg = min(max(p.nseg[bg], 0), p.smax);
    if (p.merge) rs = kMergeWaves;
  } else {
    const int rows = min(max(p.counts ? p.counts[b] : p.count_const, 0), p.count_max);
    nseg = (rows + p.seg_rows - 1) / p.seg_rows;
  }
  const int nrec = (nseg + rs - 1) / rs;
  const int4* segs = p.seg + static_cast<long long>(bg) * p.smax;
  auto rec_heads = [&](int t) {  // heads whose state record t holds (explicit plans)
    uint32_t m = static_cast<uint32_t>(segs[t * rs].z);
    for (int i = 1; i < rs; ++i)
      if (t * rs + i < nseg) m |= static_cast<uint32_t>(segs[t * rs + i].z);
    return m;
  };
  const long long rec_stride = static_cast<long long>(rs) * G * kPartStride;  // floats between records
  M = kEmptyMax;
  L = O0 = O1 = 0.f;
  const float* base = p.partial + static_cast<long long>(bg) * p.smax * G * kPartStride + h * kPartStride;
  const int n_mine = nrec > part ? (nrec - part + NS - 1) / NS : 0;  // records part + i * NS
  for (int i0 = 0; i0 < n_mine; i0 += kWave) {
    const int s = part + (i0 + lane) * NS;
    const bool in_range = i0 + lane < n_mine;
    // descriptor and partial (m, l) requested together; the (m, l) of a
    // record whose heads leave this head out are never written and never used
    const float* ph = base + (in_range ? s : 0) * rec_stride;
    float pm = kMaskedScore, pl = 0.f;
    bool mine = in_range;
    if constexpr (NS > 1) {
      const float pm_raw = ph[0], pl_raw = ph[1];
      if constexpr (EXPLICIT) mine = mine && ((rec_heads(in_range ? s : 0) >> h) & 1u);
      pm = mine ? pm_raw : kMaskedScore;
      pl = mine ? pl_raw : 0.f;
    } else {
      if constexpr (EXPLICIT) {
        if (mine) mine = (rec_heads(s) >> h) & 1u;
      }
      if (mine) {
        pm = ph[0];
        pl = ph[1];
      }
    }
    const float Mn = fmaxf(M, wave_max_f(pm));
    const float w = mine ? fast_exp2(pm - Mn) : 0.f;
    const float a = fast_exp2(M - Mn);
    L = L * a + wave_sum_f(pl * w);
    O0 *= a;
    O1 *= a;
    M = Mn;
    uint64_t bal = __ballot(mine);
    while (bal) {
      int j[kU];
      float wj[kU];
      float2 po[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        j[u] = bal ? __builtin_ctzll(bal) : -1;
        if (bal) bal &= bal - 1;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        // j < 0: a padding slot reloads record `part` (in range, so the load
        // stays straight-line) and is never added: that record need not hold
        // this head's state, and its stale bits may be NaN (0 * NaN = NaN)
        const int jj = j[u] < 0 ? 0 : j[u];
        wj[u] = j[u] < 0 ? 0.f : __shfl(w, jj);
        po[u] = *reinterpret_cast<const float2*>(base + (j[u] < 0 ? part : part + (i0 + jj) * NS) * rec_stride +
                                                 kPartO + lane * 2);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        O0 = j[u] < 0 ? O0 : fmaf(wj[u], po[u].x, O0);
        O1 = j[u] < 0 ? O1 : fmaf(wj[u], po[u].y, O1);
      }
    }
  }
}

// o / l of query head h of group bg (zero when nothing was selected)
template <int G>
__device__ __forceinline__ void write_head_out(const GatherParams& p, int bg, int h, float L, float O0, float O1) {
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* o = p.out + (static_cast<long long>(bg) * G + h) * kHeadDim + lane_id() * 2;
  *reinterpret_cast<float2*>(o) = make_float2(O0 * inv, O1 * inv);
}

template <int G, int GH, int NS, bool EXPLICIT>
__global__ __launch_bounds__(GH * NS * kWave) void combine_kernel(GatherParams p) {
  __shared__ float sm_m[GH][NS], sm_l[GH][NS];
  __shared__ float2 sm_o[NS > 1 ? GH : 1][NS > 1 ? NS : 1][kWave];
  const int bg = blockIdx.x / (G / GH);
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int hl = wave / NS, part = wave % NS;           // head within the workgroup
  const int h = (blockIdx.x % (G / GH)) * GH + hl;      // head within the group
  float M, L, O0, O1;
  combine_partials<G, NS, EXPLICIT>(p, bg, h, part, M, L, O0, O1);
  if constexpr (NS > 1) {
    if (lane == 0) {
      sm_m[hl][part] = M;
      sm_l[hl][part] = L;
    }
    sm_o[hl][part][lane] = make_float2(O0, O1);
    __syncthreads();
    if (part != 0) return;
    M = kEmptyMax;
#pragma unroll
    for (int j = 0; j < NS; ++j) M = fmaxf(M, sm_m[hl][j]);
    L = 0.f;
    O0 = 0.f;
    O1 = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float a = fast_exp2(sm_m[hl][j] - M);
      const float2 o = sm_o[hl][j][lane];
      L = fmaf(sm_l[hl][j], a, L);
      O0 = fmaf(o.x, a, O0);
      O1 = fmaf(o.y, a, O1);
    }
  }
  write_head_out<G>(p, bg, h, L, O0, O1);
}

template <typename T, int G, bool EXPLICIT, bool DUP>
__global__ __launch_bounds__(gather_waves<EXPLICIT>() * kWave) void gather_attn_kernel(GatherParams p) {
  gather_attn_body<T, G, EXPLICIT, DUP>(p);
}

template <typename T, int G, bool DUP>
__global__ __launch_bounds__(kMergeWaves * kWave) void gather_merge_kernel(GatherParams p) {
  gather_merge_body<T, G, DUP>(p);
}

template <typename T, bool EXPLICIT, bool DUP>
static void gather_dispatch(const GatherParams& p, int G, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.B * p.Hkv * p.W)), block(gather_waves<EXPLICIT>() * kWave);
  switch (G) {
    case 1: hipLaunchKernelGGL((gather_attn_kernel<T, 1, EXPLICIT, DUP>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((gather_attn_kernel<T, 2, EXPLICIT, DUP>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((gather_attn_kernel<T, 4, EXPLICIT, DUP>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((gather_attn_kernel<T, 8, EXPLICIT, DUP>), grid, block, 0, s, p); break;
  }
}

// Merged sets run for bf16 with up to 4 query heads per KV head (the
// caller sets p.merge only then; wider states would spill registers).
hipError_t launch_gather(const GatherParams& p, int dtype, int G, bool explicit_plan,
                         hipStream_t s) {
  if (explicit_plan && p.merge) {
    if (dtype != kBF16) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(p.B * p.Hkv * p.W)), block(kMergeWaves * kWave);
    if (p.alt) {
      switch (G) {
        case 1: hipLaunchKernelGGL((gather_merge_kernel<bf16_t, 1, true>), grid, block, 0, s, p); break;
        case 2: hipLaunchKernelGGL((gather_merge_kernel<bf16_t, 2, true>), grid, block, 0, s, p); break;
        case 4: hipLaunchKernelGGL((gather_merge_kernel<bf16_t, 4, true>), grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
      }
    } else {
      switch (G) {
        case 1: hipLaunchKernelGGL((gather_merge_kernel<bf16_t, 1, false>), grid, block, 0, s, p); break;
        case 2: hipLaunchKernelGGL((gather_merge_kernel<bf16_t, 2, false>), grid, block, 0, s, p); break;
        case 4: hipLaunchKernelGGL((gather_merge_kernel<bf16_t, 4, false>), grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
      }
    }
    return hipGetLastError();
  }
  if (dtype == kBF16) {
    if (explicit_plan && p.alt) gather_dispatch<bf16_t, true, true>(p, G, s);
    else if (explicit_plan) gather_dispatch<bf16_t, true, false>(p, G, s);
    else gather_dispatch<bf16_t, false, false>(p, G, s);
  } else {
    if (explicit_plan && p.alt) gather_dispatch<float, true, true>(p, G, s);
    else if (explicit_plan) gather_dispatch<float, true, false>(p, G, s);
    else gather_dispatch<float, false, false>(p, G, s);
  }
  return hipGetLastError();
}

template <int G, int GH, int NS, bool EXPLICIT>
static void combine_launch(const GatherParams& p, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<G, GH, NS, EXPLICIT>), dim3(static_cast<unsigned>(p.B * p.Hkv * (G / GH))),
                     dim3(GH * NS * kWave), 0, s, p);
}

// One wave per head once the batch alone gives every CU a few waves.
// Otherwise several waves per head: a workgroup of kCombineWavesSmall waves
// per head when each (request, KV head) has many segments (64 or more
// planned), else the group's heads share one workgroup of
// kCombineWavesSmall waves.
template <int G, bool EXPLICIT>
static void combine_dispatch_g(const GatherParams& p, hipStream_t s) {
  constexpr int NS = kCombineWavesSmall / G;
  const long long segs = static_cast<long long>(p.W) * (EXPLICIT ? kGatherWavesExplicit : kGatherWavesRows);
  if (static_cast<long long>(p.B) * p.Hkv * G >= 1024) combine_launch<G, G, 1, EXPLICIT>(p, s);
  else if (segs >= 64) combine_launch<G, 1, kCombineWavesSmall, EXPLICIT>(p, s);
  else combine_launch<G, G, NS, EXPLICIT>(p, s);
}

template <bool EXPLICIT>
static void combine_dispatch(const GatherParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: combine_dispatch_g<1, EXPLICIT>(p, s); break;
    case 2: combine_dispatch_g<2, EXPLICIT>(p, s); break;
    case 4: combine_dispatch_g<4, EXPLICIT>(p, s); break;
    default: combine_dispatch_g<8, EXPLICIT>(p, s); break;
  }
}

hipError_t launch_combine(const GatherParams& p, int G, bool explicit_plan, hipStream_t s) {
  if (explicit_plan) combine_dispatch<true>(p, G, s);
  else combine_dispatch<false>(p, G, s);
  return hipGetLastError();
}

}  // namespace tsa
