// Internal interface between the C-ABI layer and the gfx950 kernels.
// Launchers validate nothing: the C-ABI layer checks every shape, pointer and
// size before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tsa {

constexpr int kHeadDimRows = 128;   // d: elements per row (head_dim)
constexpr int kSegRows = 256;       // max rows per attention segment (one wave's work unit)
constexpr int kRowSegRows = 64;       // shortest segment for per-request row lists (token / slot paths)
constexpr int kGatherWavesExplicit = 1;    // gather waves per workgroup, IVF plans
constexpr int kGatherWavesRows = 4;   // ... per-request row lists
constexpr int kGatherSegsPerWave = 1;  // segments each gather wave is planned to take
// A partial softmax state is five whole 128-byte lines: line 0 holds m, l and
// zero fill, lines 1-4 hold o[128]. One wave writes every byte of each line,
// so no line reaches HBM partly written (HBM3E spends its mask pins on ECC,
// so a partial line write becomes a read-modify-write in the memory
// controller). Records stay line-aligned when the workspace is 128-byte
// aligned, as every device allocation is.
constexpr int kPartStride = 160;    // floats per partial state
// waves (and plan segments) per merging gather workgroup; at the batched
// 64 x 32K decode 3 measured best (2: fewer states merged, 4 and up: a
// workgroup waits longer for its longest segment, 6 also loses occupancy)
constexpr int kMergeWaves = 3;
constexpr int kPartO = 32;          // offset of o[128] within the state
constexpr int kTokFilterTile = 4096;      // score keys filtered per workgroup
constexpr int kTokHistBits = 12;          // top bits of the score key in the threshold histogram
constexpr int kTokHistBins = 1 << kTokHistBits;
constexpr int kMaxTokFilterChunks = 4096; // N <= kTokFilterTile * kMaxTokFilterChunks
constexpr int kMaxCentroids = 4096;
constexpr int kMaxAssign = 4;          // lists per key of a multi-way index
constexpr int kMaxFixedRows = 8192;   // sink + window rows of one decode
constexpr int kMaxSlots = 4096;
constexpr int kMaxTokenK = 4096;

enum Dtype { kF32 = 0, kBF16 = 1 };

inline int esize(int dtype) { return dtype == kF32 ? 4 : 2; }

// ---------------------------------------------------------------- index build
struct AssignParams {
  const void* keys;        // [B][N][Hkv][d]
  const void* centroids;   // [Bc][Hkv][C][d]
  long long cent_bstride;  // elements between request codebooks (0 = shared)
  int32_t* assign;         // [B][Hkv][N][m]: the key's m nearest centroids, nearest first
  int B, N, Hkv, C;
  int n_assign;            // keys 0 .. n_assign-1 of every request are assigned
  int m;                   // assignments per key (1 or 2)
};
// norms: workspace for |c|^2 of every centroid row (bf16 path)
hipError_t launch_assign(const AssignParams& p, int dtype, float* norms, hipStream_t s);

struct CsrParams {
  const int32_t* assign;   // [B][Hkv][N]
  int32_t* offsets;        // [B][Hkv][C+1]: list c owns ids[offsets[c] .. offsets[c+1])
  int32_t* ids;            // [B][Hkv][N]; free entries are -1
  int32_t* lens;           // [B][Hkv][C] valid entries per list, or null
  int32_t* alt;            // [B][Hkv][N*m][m-1] (m >= 2): each entry's other lists, or null
  int B, N, Hkv, C;
  int n_assign;            // tokens 0 .. n_assign-1 go into the lists
  int slack;               // free entries after every list
  int m;                   // lists per token (ids and alt hold N * m entries)
};
hipError_t launch_csr(const CsrParams& p, hipStream_t s);

// ---------------------------------------------------------- IVF select + plan
struct SelectParams {
  const void* q;           // [B][Hq][d]
  const void* centroids;   // [Bc][Hkv][C][d]
  long long cent_bstride;  // elements between request codebooks (0 = shared)
  const int32_t* offsets;  // [B][Hkv][C+1]
  const int32_t* lens;     // [B][Hkv][C] valid entries per list, or null (whole ranges)
  int32_t* sel_out;        // [B][Hq][k] or null
  int32_t* rows_out;       // [B][Hq] or null
  int32_t* uniq_out;       // [B][Hkv] or null
  int4* seg;               // [B*Hkv][smax]: {start, count, head mask, list}; list -1 = token range
  int32_t* nseg;           // [B*Hkv]
  int B, Hkv, C, k, smax, N;
  int cosine;              // score q.c / |c| instead of q.c
  int n_sink, n_window;    // token ranges attended beside the lists
  const int32_t* lengths;  // [B] current length per request, or null (N)
  int n_entries;           // list entries per (request, KV head): N, or N * m with m lists per token
  uint32_t* lmask_out;     // [B][Hkv][C] head mask of every chosen list, or null
  int seg_rows;            // rows per plan segment (<= kSegRows)
  uint32_t* keys;          // [B*Hkv][G][C] order keys of the scores, computed by centroid_score_kernel
                           // (bf16 only), or null: the select kernel scores the centroids itself
  int class_order;         // 1: plan segments by head class (merged gather sets), 0: list order
  int lens_lds = 0;        // set by the launcher: the list lengths fit in LDS beside the offsets
  uint32_t* arrive_heads = nullptr;  // [B*Hkv][G] arrival counters of the split decode, cleared
                                     // by centroid_score_kernel, or null
};
constexpr int kSelWaves = 4;               // waves per select workgroup
constexpr size_t kSelectLdsBytes = 65536;  // dynamic LDS of a select workgroup (keys, masks, offsets, lengths)
hipError_t launch_ivf_select(const SelectParams& p, int dtype, int G, hipStream_t s);

// ------------------------------------------- per-head decode (small batches)
// Fused: one workgroup of kFusedWaves waves per (request, query head) scores
// the KV group's codebook, selects the group's heads' top-k lists, gathers its
// own head's rows and writes its output, in one launch with no workspace.
// Split: centroid_score_kernel first; then S workgroups of kSplitWaves waves
// per query head each select the head's lists from the scores and attend
// share s of its rows, writing a partial state per share (record h * S + s
// of the group); the head's last share to finish merges the S records.
struct HeadDecodeParams {
  SelectParams s;          // q, centroids, offsets, lens, the sel / rows / uniq outputs, sizes,
                           // cosine, n_entries; split: keys (the scores), smax
  const int32_t* ids;      // [B][Hkv][n_entries]
  const void* k;           // [B][N][Hkv][d]
  const void* v;
  float* out;              // [B][Hq][d] (fused)
  float* partial;          // [B*Hkv][smax][G][kPartStride] (split)
  float qscale;            // log2(e) / sqrt(d)
  int Hq;
  int S;                   // split: workgroups per query head (G * S <= smax)
  const void* kl = nullptr;  // list-major copies [B][Hkv][n_entries][d], read by entry instead of
  const void* vl = nullptr;  // k / v by row id; null: k / v
};
constexpr int kFusedWaves = 8;    // beat 16, 4 and 2 waves at one 4K-token fp32 head
constexpr int kSplitWaves = 8;    // with 16 rows a wave per share; see split_shares
constexpr int kHeadMaxC = 1024;   // lists of a group held in one workgroup's LDS
constexpr int kHeadMaxK = 64;     // chosen lists of a head, one per lane
hipError_t launch_fused_decode(const HeadDecodeParams& p, int dtype, int G, hipStream_t s);
hipError_t launch_split_decode(const HeadDecodeParams& p, int G, hipStream_t s);  // bf16 only
hipError_t launch_centroid_score(const SelectParams& p, int G, hipStream_t s);     // bf16; writes p.keys

// ------------------------------------------------------- list-major KV copy
struct KvListsParams {
  const int32_t* ids;      // [B][Hkv][N]
  const void* k;           // [B][N][Hkv][d]
  const void* v;
  void* kl;                // [B][Hkv][N][d]
  void* vl;
  int B, N, Hkv;
};
hipError_t launch_kv_list_major(const KvListsParams& p, int dtype, hipStream_t s);

// ---------------------------------------------------------- KV + index append
struct AppendParams {
  const void* new_k;       // [B][Hkv][d]
  const void* new_v;       // [B][Hkv][d]
  const int32_t* pos;      // [B] row of the new token
  const void* centroids;   // [Bc][Hkv][C][d]
  long long cent_bstride;
  void* k_cache;           // [B][N][Hkv][d]
  void* v_cache;
  const int32_t* offsets;  // [B][Hkv][C+1]
  int32_t* lens;           // [B][Hkv][C]
  int32_t* ids;            // [B][Hkv][N*m]
  int32_t* status;         // [B][Hkv] or null: 0 indexed, 1 a list full, 2 row out of range
  int B, N, Hkv, C;
  int m = 1;               // lists per key: the key joins its m nearest lists, all or none
  int32_t* alt = nullptr;  // [B][Hkv][N*m][m-1] (m >= 2): each entry's other lists
};
hipError_t launch_kv_append(const AppendParams& p, int dtype, hipStream_t s);

// Re-layout of a growing index with `slack` free entries after every list
// (slack < 0: as many as fit for every list), into separate output arrays.
struct RegrowParams {
  const int32_t* offsets;  // [B][Hkv][C+1]
  const int32_t* lens;     // [B][Hkv][C]
  const int32_t* ids;      // [B][Hkv][cap]
  const int32_t* alt;      // [B][Hkv][cap][m-1] or null (m == 1)
  int32_t* offsets_out;
  int32_t* lens_out;
  int32_t* ids_out;
  int32_t* alt_out;
  int32_t* status;         // [B][Hkv] or null: 0 done, 1 the lists do not fit (outputs untouched)
  int B, Hkv, C, cap, m, slack;
};
constexpr int kRegrowChunk = 4096;   // output entries per regrow workgroup
constexpr int kRegrowPer = kRegrowChunk / 256;   // output entries per regrow thread
hipError_t launch_regrow(const RegrowParams& p, hipStream_t s);

// --------------------------------------------------------- gather attention
struct GatherParams {
  const void* q;           // [B][Hq][d]
  const void* k;           // [B][n_rows][Hkv][d]
  const void* v;
  long long n_rows;
  const int32_t* rowids;   // row-id arrays
  long long rid_bstride;   // int32 elements between requests' row-id arrays
  long long rid_gstride;   // ... between KV heads' (0: shared by all heads)
  const int4* seg;         // explicit segments (IVF) or null
  const int32_t* nseg;     // explicit segment counts or null
  const int32_t* counts;   // implicit: rows per request, or null
  int count_const;         // implicit: rows per request when counts is null
  int count_max;           // implicit: capacity of each request's row-id array
  int seg_rows;            // implicit: rows per segment (<= kSegRows)
  float* partial;          // [B*Hkv][smax][G][kPartStride]
  int n_sink, n_window;    // explicit plans: list rows inside these ranges are skipped
  const int32_t* lengths;  // [B] or null (n_rows)
  const int32_t* alt;      // explicit plans over m-way lists: each entry's other lists
                           // ([entry][alt_w]), or null
  int alt_w;               // m - 1 (with alt)
  const uint32_t* lmask;   // [B*Hkv][C] head masks of the chosen lists (with alt)
  int C;                   // lists per (request, KV head) (with alt)
  int multi_all;           // explicit plans: segments chosen by two or more heads take one all-heads pass
  int merge;               // explicit plans: kMergeWaves consecutive segments per workgroup, rows split
                           // evenly over its waves, one partial state per head per set (0: a wave per segment)
  float* out;              // [B][Hq][d]
  int B, Hkv, smax, W;     // W: workgroups per (request, KV head)
  float qscale;            // log2(e) / sqrt(d)
  const void* kl = nullptr;  // explicit plans: list-major copies [B][Hkv][entries][d] (row of
  const void* vl = nullptr;  // entry e of (b, g) at rowids offset b * rid_bstride + g * rid_gstride + e),
                             // read instead of k / v for list segments; null: k / v by row id
};
hipError_t launch_gather(const GatherParams& p, int dtype, int G, bool explicit_plan,
                         hipStream_t s);
hipError_t launch_combine(const GatherParams& p, int G, bool explicit_plan, hipStream_t s);

// ------------------------------------------------------------ token select
struct TokenSelectParams {
  const void* q_idx;       // [B][64]
  const void* k_idx;       // [B][N][64]
  uint32_t* keys;          // [B][N] order-preserving score keys
  int32_t* hist;           // [B][kTokHistBins]
  uint32_t* cand_key;      // [B][N]: filter chunk c's candidates from c * kTokFilterTile
  int32_t* cand_id;        // [B][N]
  int32_t* cand_cnt;       // [B][nfchunk]
  int32_t* sel;            // [B][k]
  int B, N, k, nfchunk;
  hipEvent_t score_ev0 = nullptr, score_ev1 = nullptr;  // recorded around the scan launch when set
  // The scan clears the histogram itself: workgroup 0 of request b zeroes
  // hist[b] and grab[b], then publishes tag = mix(*epoch * phi + nonce) in ready[b]; the
  // other workgroups add their counts once ready[b] holds that tag. The final
  // select advances *epoch, so every call (and every replay of a captured
  // call) has a tag of its own.
  uint64_t* epoch = nullptr;  // [1]
  uint64_t* ready = nullptr;  // [B]
  uint64_t nonce = 0;         // per call, from the host
  // per-request counter of the scan's shared chunks, zeroed with hist[b]
  int32_t* grab = nullptr;    // [B]
};
hipError_t launch_token_select(const TokenSelectParams& p, int dtype, hipStream_t s);

// ---------------------------------------------------------------- resolve
struct ResolveParams {
  int32_t* page_table;     // [B][N]
  int32_t* slot_token;     // [B][S]
  int32_t* last_use;       // [B][S]
  const int32_t* sel;      // [B][k]
  const void* host_k;      // [B][N][Hkv][d] host-mapped
  const void* host_v;
  void* pool_k;            // [B][S][Hkv][d]
  void* pool_v;
  int32_t* slots_out;      // [B][k]
  int32_t* hits;           // [B] or null
  int32_t* misses;         // [B] or null
  long long row_bytes;     // Hkv * d * element size (multiple of 16)
  int B, N, S, k, step;
  int policy;              // kEvictLru / kEvictFifo / kEvictRandom / kEvictPriority
  unsigned long long seed; // random policy
  const int32_t* priority; // [B][N] priority policy: evict the largest value first
  int32_t* miss_tok;       // [B][k] or null: missed tokens in miss order
  int32_t* miss_slot;      // [B][k] or null: the slot each took
};
hipError_t launch_resolve(const ResolveParams& p, hipStream_t s);

// Copies the rows of a miss list (from a RESOLVE of the same selection) from
// the host copies of up to kMaxFetchLayers layers into their pools.
constexpr int kMaxFetchLayers = 16;
struct FetchParams {
  const int32_t* miss_tok;   // [B][k]
  const int32_t* miss_slot;  // [B][k]
  const int32_t* misses;     // [B]
  const void* host_k[kMaxFetchLayers];  // per layer [B][N][Hkv][d] host-mapped
  const void* host_v[kMaxFetchLayers];
  void* pool_k[kMaxFetchLayers];        // per layer [B][S][Hkv][d]
  void* pool_v[kMaxFetchLayers];
  int n_layers;
  int split;                 // workgroups per (request, layer)
  long long row_bytes;
  int B, N, S, k;
};
hipError_t launch_fetch_rows(const FetchParams& p, hipStream_t s);

constexpr int kEvictLru = 0, kEvictFifo = 1, kEvictRandom = 2, kEvictPriority = 3;

hipError_t launch_fill_i32(int32_t* p, long long n, int32_t value, hipStream_t s);

// ---------------------------------------------------------------- probe
int stream_read_blocks();
int stream_read_waves_per_block();
hipError_t launch_stream_read(const void* p, long long n16, uint32_t* sink, hipStream_t s);

}  // namespace tsa
