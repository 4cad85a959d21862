/*
 * tsa.h - retrieval-based sparse-attention decode for AMD Instinct MI355X
 * (gfx950). C ABI: plain integers and pointers only.
 *
 * Pages the operations come from (cited by title and section):
 *   [KARAT]  paper-daily digest "Heterogeneous LLM Serving with
 *            General-Purpose Processing-Near-Memory for Retrieval-Based
 *            Sparse Attention": How (index structure), core formulas (Eq. 2),
 *            worked example (steps 3-4).
 *   [HISPARSE-NEWS]  "KV卸载上主机:HiSparse、PDD与DDR4回收", paper analysis 1
 *            (HiSparse): hot cache of B slots per request per layer, page
 *            table + LRU, one fused RESOLVE kernel, authoritative KV in pinned
 *            host memory, exactness.
 *   [HISPARSE-NOTES] "10月14日学习笔记", HiSparse (indexer top-k selection,
 *            LRU for the locality of consecutive selections).
 *
 * Conventions shared by every entry point
 *   - Memory: every array argument is caller-owned. Pointers marked (device)
 *     are device memory of the current HIP device; (host-mapped) is pinned
 *     host memory the device can read (tsa_host_alloc). The library keeps no
 *     pointer after a call returns and allocates nothing inside a call.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream). Every kernel of a call is enqueued on it; the call returns
 *     without synchronising and results are valid once the stream reaches
 *     them. No call records a memset or a host synchronisation, so calls can
 *     be captured into a HIP graph.
 *   - Layouts are dense and row-major, innermost index last. A "row" is one
 *     token's head_dim elements for one KV head. K and V caches are
 *     [batch][n_rows][n_kv_heads][head_dim]: the rows of one token for all KV
 *     heads are contiguous. Query head h reads KV head h / (n_q_heads /
 *     n_kv_heads).
 *   - Element types: tsa_dtype selects fp32 or bf16 (bfloat16 bit patterns in
 *     uint16). Arithmetic is fp32 (products of bf16 inputs, fp32 sums);
 *     attention outputs are fp32.
 *   - Workspace: ops that need scratch take (ws, ws_bytes); the size comes
 *     from tsa_workspace_bytes for the same descriptor and k. It must be
 *     16-byte aligned. Its contents need no initialisation and are
 *     meaningless between calls.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a failing call enqueues nothing and writes no output.
 *     TSA_ERR_INVALID_ARG: null pointer, non-positive size, k out of range,
 *     misaligned pointer. TSA_ERR_UNSUPPORTED: a shape this build does not
 *     implement (head_dim != 128, idx_dim != 64, n_q_heads / n_kv_heads not
 *     in {1,2,4,8}, sizes beyond the limits stated per call).
 *     TSA_ERR_WORKSPACE: ws_bytes too small. TSA_ERR_HIP: a HIP launch
 *     failed. tsa_last_error() returns this thread's last message.
 *   - Tie rule for every top-k: the larger score wins, equal scores go to the
 *     lower index, and selections are written in ascending index order.
 */
#ifndef TSA_H
#define TSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TSA_ABI_VERSION 3

/* Size of the static device scratch of tsa_sparse_decode_noalloc. */
#define TSA_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef enum tsa_status {
  TSA_OK = 0,
  TSA_ERR_INVALID_ARG = 1,
  TSA_ERR_UNSUPPORTED = 2,
  TSA_ERR_WORKSPACE = 3,
  TSA_ERR_HIP = 4
} tsa_status;

typedef enum tsa_dtype { TSA_F32 = 0, TSA_BF16 = 1 } tsa_dtype;

/* Workspace-sized operations, for tsa_workspace_bytes. */
typedef enum tsa_op {
  TSA_OP_INDEX_BUILD = 0,
  TSA_OP_SPARSE_DECODE = 1,
  TSA_OP_TOKEN_DECODE = 2,
  TSA_OP_ATTEND_ROWS = 3,
  TSA_OP_SPARSE_DECODE_EX = 4,
  TSA_OP_INDEX_BUILD_MULTI = 5,      /* tsa_index_build_multi (m = 2; any m: tsa_workspace_bytes_multi) */
  TSA_OP_SPARSE_DECODE_EX_MULTI = 6  /* tsa_sparse_decode_ex with assign_per_key = m (likewise)       */
} tsa_op;

/* Inverted-index (centroid) problem. */
typedef struct tsa_ivf_desc {
  int32_t batch;           /* B requests                                   */
  int32_t n_tokens;        /* N cached tokens per request                  */
  int32_t n_kv_heads;      /* Hkv                                          */
  int32_t n_q_heads;       /* Hq; Hq / Hkv in {1, 2, 4, 8}                 */
  int32_t head_dim;        /* d; must be 128                               */
  int32_t n_centroids;     /* C lists per (request, KV head); C <= 4096 and
                              C * (Hq / Hkv + 2) < 16384                   */
  int32_t shared_codebook; /* 1: centroids [Hkv][C][d] for all requests;
                              0: centroids [B][Hkv][C][d]                 */
  int32_t dtype;           /* tsa_dtype of q, keys, values, centroids     */
} tsa_ivf_desc;

/* Token-indexer (DSA-style) problem. */
typedef struct tsa_token_desc {
  int32_t batch;       /* B                                    */
  int32_t n_tokens;    /* N                                    */
  int32_t n_kv_heads;  /* Hkv                                  */
  int32_t n_q_heads;   /* Hq                                   */
  int32_t head_dim;    /* d = 128                              */
  int32_t idx_dim;     /* indexer key width; must be 64        */
  int32_t dtype;       /* tsa_dtype of all inputs              */
} tsa_token_desc;

/* Hot-cache (HiSparse-style) problem: one layer. */
typedef struct tsa_cache_desc {
  int32_t batch;       /* B requests                                       */
  int32_t n_tokens;    /* N tokens in each request's host copy             */
  int32_t n_slots;     /* S hot slots per request; <= 4096                 */
  int32_t n_kv_heads;  /* Hkv                                              */
  int32_t head_dim;    /* d = 128                                          */
  int32_t dtype;       /* tsa_dtype of the K/V rows                        */
} tsa_cache_desc;

/* Attention over explicit per-request row lists shared by all heads. */
typedef struct tsa_attn_desc {
  int32_t batch;       /* B                                                */
  int32_t n_rows;      /* rows addressable per request in k/v (N, or S)    */
  int32_t n_kv_heads;  /* Hkv                                              */
  int32_t n_q_heads;   /* Hq                                               */
  int32_t head_dim;    /* d = 128                                          */
  int32_t max_rows;    /* capacity of each request's row list              */
  int32_t dtype;       /* tsa_dtype of q, k, v                             */
} tsa_attn_desc;

/* ------------------------------------------------------------------------
 * tsa_index_build - posting lists of an inverted index.
 *   [KARAT] How, index structure: each KV entry goes to a posting list by
 *   its key. Reading: every key joins exactly one list, that of its nearest
 *   centroid by squared Euclidean distance (ties -> lower centroid id).
 *   keys       (device) [B][N][Hkv][d], the K cache itself.
 *   centroids  (device) [Hkv][C][d] shared, or [B][Hkv][C][d].
 *   offsets    (device, out) int32 [B][Hkv][C+1]: list c of (b, g) holds
 *              ids[b][g][offsets[b][g][c] .. offsets[b][g][c+1]).
 *   ids        (device, out) int32 [B][Hkv][N]: token ids, ascending within
 *              each list.
 *   Workspace: tsa_workspace_bytes(TSA_OP_INDEX_BUILD, desc, 0, ...).
 *   Distances are computed in fp32; they decide the same list as exact
 *   arithmetic whenever the nearest and second-nearest squared distances
 *   differ by more than fp32 rounding.
 * ---------------------------------------------------------------------- */
tsa_status tsa_index_build(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                           int32_t* offsets, int32_t* ids, void* ws, size_t ws_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * tsa_sparse_decode - one decode step of retrieval-based sparse attention.
 *   [KARAT] worked example steps 3-4 and Eq. 2: score q against every
 *   centroid of its KV head (raw dot product), keep the k best lists, gather
 *   the K/V rows of those lists and attend over them only:
 *     out[b][h] = sum_{i in R} softmax_i(q.K_i / sqrt(d)) V_i,
 *     R = union of the k chosen lists of (b, h).
 *   q          (device) [B][Hq][d]
 *   centroids  (device) as for tsa_index_build
 *   offsets, ids (device) posting lists from tsa_index_build
 *   k_cache, v_cache (device) [B][N][Hkv][d]
 *   k          lists per query head, 1 <= k <= C
 *   out        (device, out) fp32 [B][Hq][d]; zero where R is empty
 *   sel_out    (device, out, nullable) int32 [B][Hq][k]: chosen lists,
 *              ascending
 *   rows_out   (device, out, nullable) int32 [B][Hq]: |R| per head (0 flags
 *              an empty set)
 *   uniq_out   (device, out, nullable) int32 [B][Hkv]: rows read once for the
 *              whole KV group (the union over its query heads' lists)
 *   Workspace: tsa_workspace_bytes(TSA_OP_SPARSE_DECODE, desc, k, ...).
 *   Scores are fp32; the chosen lists equal the exact top-k whenever the
 *   k-th and (k+1)-th scores differ by more than fp32 rounding. Results are
 *   bitwise reproducible for a given desc and k. How the chosen rows are
 *   grouped for the softmax merge depends on the batch shape, so one request
 *   decoded within batches of different sizes selects the same lists and
 *   gets outputs that agree to fp32 rounding.
 * ---------------------------------------------------------------------- */
tsa_status tsa_sparse_decode(const tsa_ivf_desc* desc, const void* q, const void* centroids,
                             const int32_t* offsets, const int32_t* ids, const void* k_cache,
                             const void* v_cache, int32_t k, float* out, int32_t* sel_out,
                             int32_t* rows_out, int32_t* uniq_out, void* ws, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * tsa_sparse_decode_noalloc - tsa_sparse_decode without a workspace
 *   argument, for callers that cannot allocate device memory (code under HIP
 *   graph capture, tight serving loops, harnesses that forbid allocation).
 *   Computes exactly what tsa_sparse_decode computes (bitwise the same
 *   outputs for the same desc and k), with the same arguments minus ws and
 *   ws_bytes; it calls no allocating routine.
 *   Its workspace is a static device array of TSA_NOALLOC_SCRATCH_BYTES
 *   (64 MiB) inside the library: each GPU the library runs on holds one until
 *   the process ends. A decode whose workspace
 *   (tsa_workspace_bytes(TSA_OP_SPARSE_DECODE, ...)) exceeds it is rejected
 *   with TSA_ERR_WORKSPACE before anything is enqueued; one 100K-token
 *   request (8 KV / 32 query heads, C = 1000, k = 10) or 16 requests of 32K
 *   tokens (C = 256, k = 16) fit.
 *   Every call on one GPU shares that GPU's array, and no output depends on
 *   what an earlier call left in it. Calls that overlap on one GPU (on
 *   different streams or threads, without ordering between them) race on
 *   the array and give undefined results. The stream must belong to the
 *   current device.
 * ---------------------------------------------------------------------- */
tsa_status tsa_sparse_decode_noalloc(const tsa_ivf_desc* desc, const void* q, const void* centroids,
                                     const int32_t* offsets, const int32_t* ids, const void* k_cache,
                                     const void* v_cache, int32_t k, float* out, int32_t* sel_out,
                                     int32_t* rows_out, int32_t* uniq_out, void* stream);

/* ------------------------------------------------------------------------
 * tsa_index_build_multi - posting lists in which every key joins its m
 *   nearest lists ([KARAT] How, index structure: an entry is placed into
 *   several lists by its key), 1 <= m <= 4 and m <= C (squared L2 in fp32,
 *   nearest first, ties to the lower index).
 *   offsets (device, out) int32 [B][Hkv][C+1] over N * m entries
 *   ids     (device, out) int32 [B][Hkv][N*m]: ascending token ids per list
 *   alt     (device, out) int32 [B][Hkv][N*m][m-1] (NULL for m = 1): for
 *           each entry, the token's other m - 1 lists, in the token's order
 *           of preference
 *   Workspace: tsa_workspace_bytes_multi(TSA_OP_INDEX_BUILD_MULTI, desc, 0,
 *   m, ...). Decode with tsa_sparse_decode_ex and opts->assign_per_key = m.
 *   TSA_ERR_UNSUPPORTED for m outside [1, 4] or N * m beyond int32.
 * ---------------------------------------------------------------------- */
tsa_status tsa_index_build_multi(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                                 int32_t m, int32_t* offsets, int32_t* ids, int32_t* alt, void* ws,
                                 size_t ws_bytes, void* stream);

/* tsa_workspace_bytes for the m-way operations: TSA_OP_INDEX_BUILD_MULTI
 * (k unused) and TSA_OP_SPARSE_DECODE_EX_MULTI (k = top-k) with m lists per
 * key (tsa_workspace_bytes sizes them for m = 2); other ops as
 * tsa_workspace_bytes. */
tsa_status tsa_workspace_bytes_multi(int32_t op, const void* desc, int32_t k, int32_t m, size_t* bytes);

/* ------------------------------------------------------------------------
 * Growing index: per-step KV and posting-list append.
 *   [KARAT] worked example, step 6: after each step the new KV entry is
 *   stored and added to its posting list; Limitations, item 3: keeping the
 *   index current is the cost to pay as the cache grows.
 *
 * tsa_index_build_dyn - posting lists over the first n_prefix tokens of every
 *   request, each list followed by `slack` free entries for later appends.
 *   desc->n_tokens is the capacity N (rows of the K/V cache and of ids).
 *   keys, centroids  as for tsa_index_build (rows >= n_prefix are not read)
 *   n_prefix         1 <= n_prefix <= N
 *   slack            >= 0, n_prefix + C * slack <= N
 *   offsets (device, out) int32 [B][Hkv][C+1]: list c owns
 *            ids[offsets[c] .. offsets[c+1]) (its valid entries first)
 *   lens    (device, out) int32 [B][Hkv][C]: valid entries of each list
 *   ids     (device, out) int32 [B][Hkv][N]: ascending token ids at the front
 *            of every list range; free entries (and the tail) are -1
 *   Workspace: tsa_workspace_bytes(TSA_OP_INDEX_BUILD, desc, 0, ...).
 *
 * tsa_kv_append - one decode step's append for every request: stores the new
 *   token's K and V rows at row pos[b] of the caches and adds pos[b] at the
 *   end of the valid entries of the list of the key's nearest centroid
 *   (squared L2 in fp32, ties to the lower index), if that list has a free
 *   entry. Positions should grow from step to step so that every list stays
 *   in ascending id order. No workspace.
 *   new_k, new_v (device) [B][Hkv][d], the storage dtype
 *   pos          (device) int32 [B]
 *   centroids    (device) as for tsa_index_build
 *   k_cache, v_cache (device, in/out) [B][N][Hkv][d]
 *   offsets      (device) from tsa_index_build_dyn;  lens, ids (device, in/out)
 *   status       (device, out, nullable) int32 [B][Hkv]: 0 indexed; 1 list
 *                full (rows stored, id not indexed: rebuild the index);
 *                2 pos outside [0, N) (nothing stored)
 *
 * tsa_sparse_decode_dyn - tsa_sparse_decode over a growing index: list c is
 *   ids[offsets[c] .. offsets[c] + lens[c]). Same arguments otherwise; with
 *   the same lists it gives bitwise the same output as tsa_sparse_decode.
 * ---------------------------------------------------------------------- */
tsa_status tsa_index_build_dyn(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                               int32_t n_prefix, int32_t slack, int32_t* offsets, int32_t* lens,
                               int32_t* ids, void* ws, size_t ws_bytes, void* stream);
tsa_status tsa_kv_append(const tsa_ivf_desc* desc, const void* new_k, const void* new_v,
                         const int32_t* pos, const void* centroids, void* k_cache, void* v_cache,
                         const int32_t* offsets, int32_t* lens, int32_t* ids, int32_t* status,
                         void* stream);
tsa_status tsa_sparse_decode_dyn(const tsa_ivf_desc* desc, const void* q, const void* centroids,
                                 const int32_t* offsets, const int32_t* lens, const int32_t* ids,
                                 const void* k_cache, const void* v_cache, int32_t k, float* out,
                                 int32_t* sel_out, int32_t* rows_out, int32_t* uniq_out, void* ws,
                                 size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Growing m-way index (several lists per key, [KARAT] How, index
 * structure; appended every step, worked example step 6).
 *
 * tsa_index_build_dyn_multi - tsa_index_build_dyn in which every key of the
 *   prefix joins its m nearest lists (1 <= m <= 4, m <= C). The lists hold
 *   N * m entries: n_prefix * m + C * slack <= N * m.
 *   offsets, lens  as for tsa_index_build_dyn, over N * m entries
 *   ids     (device, out) int32 [B][Hkv][N*m]; free entries -1
 *   alt     (device, out) int32 [B][Hkv][N*m][m-1] (NULL for m = 1): each
 *           valid entry's other lists (free entries are not written)
 *   Workspace: tsa_workspace_bytes_multi(TSA_OP_INDEX_BUILD_MULTI, desc, 0, m).
 *
 * tsa_kv_append_multi - tsa_kv_append into an m-way growing index: the key
 *   joins its m nearest lists, each at the end of its valid entries with
 *   its other lists in alt, when every one of them has a free entry; else
 *   it joins none (status 1; its K and V rows are stored either way).
 *   No workspace.
 *
 * tsa_index_regrow - repairs a growing index whose lists ran full: lays the
 *   same lists out again, in separate output arrays of the same shapes, each
 *   list keeping its valid entries (and alt rows) in order at the front of
 *   a range with `slack` free entries after them (slack < 0: the largest
 *   slack every list can get, (N * m - total valid) / C). Nothing is
 *   reassigned; appends that reported a full list can then be made again.
 *   m, offsets, lens, ids, alt   the index (alt NULL for m = 1)
 *   *_out   (device, out) the new index; no output may alias an input
 *   status  (device, out, nullable) int32 [B][Hkv]: 0 done; 1 the valid
 *           entries plus the free ones exceed N * m (that group's outputs
 *           are not written)
 *   Lengths are clamped to their list's range and ranges to [0, N * m).
 *   No workspace.
 *
 * Decode a growing m-way index with tsa_sparse_decode_ex, opts->lens and
 * opts->assign_per_key = m.
 * ---------------------------------------------------------------------- */
tsa_status tsa_index_build_dyn_multi(const tsa_ivf_desc* desc, const void* keys, const void* centroids,
                                     int32_t n_prefix, int32_t slack, int32_t m, int32_t* offsets,
                                     int32_t* lens, int32_t* ids, int32_t* alt, void* ws, size_t ws_bytes,
                                     void* stream);
tsa_status tsa_kv_append_multi(const tsa_ivf_desc* desc, int32_t m, const void* new_k, const void* new_v,
                               const int32_t* pos, const void* centroids, void* k_cache, void* v_cache,
                               const int32_t* offsets, int32_t* lens, int32_t* ids, int32_t* alt,
                               int32_t* status, void* stream);
tsa_status tsa_index_regrow(const tsa_ivf_desc* desc, int32_t m, const int32_t* offsets, const int32_t* lens,
                            const int32_t* ids, const int32_t* alt, int32_t slack, int32_t* offsets_out,
                            int32_t* lens_out, int32_t* ids_out, int32_t* alt_out, int32_t* status,
                            void* stream);

/* ------------------------------------------------------------------------
 * tsa_sparse_decode_ex - tsa_sparse_decode with the decode variants.
 *   [KARAT] worked example, step 3: centroids are compared with the query by
 *   cosine similarity; method details: the cores also run window-based
 *   sparse attention (StreamingLLM) beside retrieval.
 *   opts->similarity  TSA_SIM_DOT (q.c, as tsa_sparse_decode) or
 *                     TSA_SIM_COSINE (q.c / |c|; 0 for a zero centroid)
 *   opts->n_sink      the first n_sink tokens are attended by every head
 *   opts->n_window    so are the last n_window tokens before the length
 *                     (n_sink, n_window >= 0, n_sink + n_window <= 8192)
 *   opts->lengths     (device, nullable) int32 [B]: current length L of each
 *                     request (default N); both ranges are clipped to [0, L)
 *   opts->lens        (device, nullable) list lengths of a growing index, as
 *                     for tsa_sparse_decode_dyn
 *   opts->assign_per_key  0 or 1: one list per token; m in 2..4: ids and alt
 *                     come from tsa_index_build_multi (or, with lens, from
 *                     tsa_index_build_dyn_multi and tsa_kv_append_multi)
 *                     with that m ([B][Hkv][N*m]); a token in several chosen
 *                     lists of a head is attended once (through the
 *                     lowest-numbered of them)
 *   opts->alt         (device) int32 [B][Hkv][N*m][m-1] from the m-way build,
 *                     required when assign_per_key is 2 or more
 *   opts->schedule    tsa_schedule (0: AUTO)
 *   opts->k_lists, opts->v_lists  (device, nullable) list-major copies of
 *                     the caches from tsa_kv_list_major for this index: the
 *                     chosen lists' rows are read from them (plain lists
 *                     only: assign_per_key <= 1, no sink, window or lens)
 *   The attended set of a head is the union of its chosen lists' rows and
 *   the two ranges; a row in both is attended once. rows_out and uniq_out
 *   count list entries only. Workspace:
 *   tsa_workspace_bytes(TSA_OP_SPARSE_DECODE_EX, desc, k, ...), or
 *   TSA_OP_SPARSE_DECODE_EX_MULTI with assign_per_key 2. Other arguments as
 *   for tsa_sparse_decode.
 * ---------------------------------------------------------------------- */
typedef enum tsa_similarity { TSA_SIM_DOT = 0, TSA_SIM_COSINE = 1 } tsa_similarity;

/* How the launches of one decode are laid out (the results are the same
 * lists, row counts and, to rounding, outputs):
 *   TSA_SCHED_AUTO    the library's choice (below)
 *   TSA_SCHED_STAGED  scoring, top-k + gather plan per (request, KV head),
 *                     gather over plan segments, combine
 *   TSA_SCHED_FUSED   one workgroup per (request, query head) scores, selects
 *                     and attends in one launch
 *   TSA_SCHED_SPLIT   scoring, then S workgroups per (request, query head)
 *                     each select the head's lists and attend a share of its
 *                     rows; the head's last share to finish merges the
 *                     shares in that launch (bf16 only)
 * FUSED and SPLIT take plain list decodes only: one list per token, no sink
 * or window, C <= 1024, k <= 64 (else TSA_ERR_UNSUPPORTED). AUTO takes FUSED
 * when every head's work fits one CU (B * Hq <= 256, about k * N / C <= 512
 * rows a head, a codebook of at most 64 KiB per KV head), else SPLIT for bf16
 * batches of fewer than 128 (request, KV head) groups, else STAGED.
 * tsa_sparse_decode and tsa_sparse_decode_dyn use AUTO. */
typedef enum tsa_schedule {
  TSA_SCHED_AUTO = 0,
  TSA_SCHED_STAGED = 1,
  TSA_SCHED_FUSED = 2,
  TSA_SCHED_SPLIT = 3
} tsa_schedule;

typedef struct tsa_decode_opts {
  int32_t similarity;       /* tsa_similarity                               */
  int32_t n_sink;           /* leading tokens always attended               */
  int32_t n_window;         /* trailing tokens (before the length) attended */
  int32_t assign_per_key;   /* 0 or 1 .. 4 lists per token                  */
  const int32_t* lengths;   /* device [B] or NULL                           */
  const int32_t* lens;      /* device [B][Hkv][C] or NULL                   */
  const int32_t* alt;       /* device [B][Hkv][N*m][m-1] or NULL            */
  int32_t schedule;         /* tsa_schedule                                 */
  const void* k_lists;      /* device [B][Hkv][N][d] from tsa_kv_list_major */
  const void* v_lists;      /*   or NULL (both or neither)                  */
} tsa_decode_opts;

/* ------------------------------------------------------------------------
 * tsa_kv_list_major - the K and V rows of every (request, KV head) copied in
 *   posting-list order, so that each list is one contiguous run of rows.
 *   [KARAT] How, index structure: an inverted file keeps its entries by
 *   list; a decode then reads a chosen list as one stream instead of
 *   scattered rows.
 *   ids        (device) int32 [B][Hkv][N] from tsa_index_build
 *   k_cache, v_cache  (device) [B][N][Hkv][d]
 *   k_lists, v_lists  (device, out) [B][Hkv][N][d], caller-owned:
 *              k_lists[b][g][e] = k_cache[b][ids[b][g][e]][g], likewise v;
 *              a row whose id lies outside [0, N) is written as zeros.
 *   Give both to tsa_sparse_decode_ex (opts->k_lists, opts->v_lists): the
 *   rows of the chosen lists are then read from them, with the same lists,
 *   counts and outputs. They describe one static index: build them again
 *   after tsa_index_build or after the caches change. With them the decode
 *   takes one list per token, no sink or window and no growing index
 *   (else TSA_ERR_UNSUPPORTED). No workspace.
 * ---------------------------------------------------------------------- */
tsa_status tsa_kv_list_major(const tsa_ivf_desc* desc, const int32_t* ids, const void* k_cache,
                             const void* v_cache, void* k_lists, void* v_lists, void* stream);

tsa_status tsa_sparse_decode_ex(const tsa_ivf_desc* desc, const tsa_decode_opts* opts, const void* q,
                                const void* centroids, const int32_t* offsets, const int32_t* ids,
                                const void* k_cache, const void* v_cache, int32_t k, float* out,
                                int32_t* sel_out, int32_t* rows_out, int32_t* uniq_out, void* ws,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * tsa_token_decode - token-level indexer top-k and attention (DSA style).
 *   [HISPARSE-NOTES] motivation (an indexer picks the top-k tokens, O(k)
 *   work per step); [HISPARSE-NEWS] the selector states the positions each
 *   step needs; [KARAT] Eq. 2 over that set.
 *   score_i = q_idx[b] . k_idx[b][i]; the k best tokens of request b are
 *   attended by all its query heads.
 *   q_idx  (device) [B][idx_dim];  k_idx (device) [B][N][idx_dim]
 *   q      (device) [B][Hq][d];    k_cache, v_cache (device) [B][N][Hkv][d]
 *   k      1 <= k <= N, k <= 4096; N <= 4096 * 4096
 *   out    (device, out) fp32 [B][Hq][d]
 *   sel_out (device, out, nullable) int32 [B][k], ascending token ids
 *   Workspace: tsa_workspace_bytes(TSA_OP_TOKEN_DECODE, desc, k, ...). It
 *   may hold anything before a call: the scan launch clears the score
 *   histogram and its per-request chunk counters itself and marks them
 *   cleared with a tag drawn from an epoch the workspace keeps and a
 *   per-call nonce (so no earlier contents or earlier call pass for this
 *   call's mark, save by a 2^-64 coincidence). Calls that share a workspace
 *   must not overlap.
 * ---------------------------------------------------------------------- */
tsa_status tsa_token_decode(const tsa_token_desc* desc, const void* q_idx, const void* k_idx,
                            const void* q, const void* k_cache, const void* v_cache, int32_t k,
                            float* out, int32_t* sel_out, void* ws, size_t ws_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * tsa_resolve - one fused RESOLVE step of the hot cache, all requests.
 *   [HISPARSE-NEWS] paper analysis 1: hit detection, LRU replacement,
 *   metadata update and host fetch in one kernel.
 *   Batch-step LRU (the page leaves the order inside a step open):
 *     hits   = selected tokens with page_table >= 0; their slots' last_use
 *              becomes `step` (protected from eviction in this step);
 *     misses = the other selected tokens, in the order given (ascending);
 *     victims = slots with last_use < step ordered by (last_use, slot),
 *              free slots (-1) first; the r-th miss takes the r-th victim:
 *              its old token leaves the page table, page_table[miss] = slot,
 *              slot_token[slot] = miss, last_use[slot] = step, and the
 *              token's K and V rows for every KV head are copied from the
 *              host copy into the slot.
 *   page_table (device, in/out) int32 [B][N]   slot or -1
 *   slot_token (device, in/out) int32 [B][S]   token or -1
 *   last_use   (device, in/out) int32 [B][S]   step or -1
 *   sel        (device) int32 [B][k]: strictly ascending token ids in [0, N)
 *   k          1 <= k <= min(S, 4096)
 *   step       stamp of this step; larger than every stamp already stored
 *   host_k, host_v (host-mapped) [B][N][Hkv][d]: the authoritative copy
 *   pool_k, pool_v (device, in/out) [B][S][Hkv][d]: the hot slots
 *   slots_out  (device, out) int32 [B][k]: slot holding sel[b][i]
 *   hits, misses (device, out, nullable) int32 [B]
 *   No workspace. Contract violations (unsorted or repeated sel, stale
 *   step) give an undefined but in-bounds cache state.
 * ---------------------------------------------------------------------- */
tsa_status tsa_resolve(const tsa_cache_desc* desc, int32_t* page_table, int32_t* slot_token,
                       int32_t* last_use, const int32_t* sel, int32_t k, int32_t step,
                       const void* host_k, const void* host_v, void* pool_k, void* pool_v,
                       int32_t* slots_out, int32_t* hits, int32_t* misses, void* stream);

/* ------------------------------------------------------------------------
 * tsa_resolve_policy - tsa_resolve under another replacement policy.
 *   [HISPARSE-NEWS] compares LRU with FIFO, random and the offline Belady
 *   policy by miss rate (13.4 / 17.2 / 16.1 / 8.2 % at B = 4096) without
 *   defining them further. Under every policy the step's hits are kept,
 *   free slots are taken first, and the r-th miss (ascending token order)
 *   takes the r-th victim; the policies order the other slots:
 *     TSA_EVICT_LRU       (last use, slot), as tsa_resolve
 *     TSA_EVICT_FIFO      (fetch step, slot): a hit does not restamp
 *     TSA_EVICT_RANDOM    (key, slot), key = top 31 bits of SplitMix64
 *                         (Steele, Lea, Flood, OOPSLA 2014) chained over
 *                         seed, request, step and slot:
 *                         x = mix(seed); x = mix(x + b); x = mix(x + step);
 *                         x = mix(x + slot); key = x >> 33, where mix(z)
 *                         adds 0x9E3779B97F4A7C15 and applies the
 *                         generator's output function
 *     TSA_EVICT_PRIORITY  largest priority[b][token] first, then slot; with
 *                         the step of each token's next selection (INT32_MAX
 *                         for never) this is the offline Belady policy
 *   priority (device) int32 [B][N], required for TSA_EVICT_PRIORITY, else
 *            ignored (negative values count as 0)
 *   Other arguments, ownership and errors as for tsa_resolve;
 *   TSA_ERR_INVALID_ARG for an unknown policy.
 * ---------------------------------------------------------------------- */
typedef enum {
  TSA_EVICT_LRU = 0,
  TSA_EVICT_FIFO = 1,
  TSA_EVICT_RANDOM = 2,
  TSA_EVICT_PRIORITY = 3
} tsa_evict_policy;

tsa_status tsa_resolve_policy(const tsa_cache_desc* desc, int32_t* page_table, int32_t* slot_token,
                              int32_t* last_use, const int32_t* sel, int32_t k, int32_t step,
                              int32_t policy, uint64_t seed, const int32_t* priority,
                              const void* host_k, const void* host_v, void* pool_k, void* pool_v,
                              int32_t* slots_out, int32_t* hits, int32_t* misses, int32_t* miss_tok,
                              int32_t* miss_slot, void* stream);

/* ------------------------------------------------------------------------
 * Layer groups that share one selection: cross-layer prefetch.
 *   [HISPARSE-NOTES] method 3: some models reuse the indexer's selection
 *   across a group of layers, so the rows every later layer of the group
 *   needs are known exactly once the first layer's selection is; they can be
 *   fetched ahead while earlier layers attend. [HISPARSE-NEWS]: exposed host
 *   IO falls from 7-8 ms to about 3 ms per token with prefetch.
 *
 * tsa_resolve_policy's miss_tok / miss_slot (device, out, nullable, both or
 *   neither) int32 [B][k]: the step's missed tokens in miss order and the
 *   slot each took (the first misses[b] entries are valid).
 *
 * tsa_fetch_rows - copy the rows of a miss list from one more layer's host
 *   copy into that layer's pool (same slots): the fetch part of RESOLVE
 *   without the table update. Arguments as for tsa_resolve.
 *
 * tsa_hier_group_step - one decode step of a layer group sharing `sel`:
 *   RESOLVE once (tables, miss list, layer 0's rows) on `stream`; the other
 *   layers' rows on `fetch_stream`; each layer's attention over its pool on
 *   `stream` once its rows are in. Per layer j (layers[j], a host array):
 *   host_k/host_v (host-mapped [B][N][Hkv][d]), pool_k/pool_v (device
 *   [B][S][Hkv][d]), q (device [B][Hq][d]), out (device fp32 [B][Hq][d]).
 *   fetch_stream NULL: everything runs in order on `stream`. n_layers <= 17
 *   (one fetch launch covers the other layers of the group).
 *   events: two caller-created hipEvent_t (timing may be disabled): the fork
 *   to fetch_stream and the join back to `stream`; required when
 *   fetch_stream is given and n_layers > 1. misses, miss_tok, miss_slot are
 *   required when n_layers > 1.
 *   Workspace: tsa_workspace_bytes(TSA_OP_ATTEND_ROWS) of the attn desc
 *   {B, S, Hkv, n_q_heads, d, max_rows = k, dtype}.
 * ---------------------------------------------------------------------- */
tsa_status tsa_fetch_rows(const tsa_cache_desc* desc, const int32_t* miss_tok, const int32_t* miss_slot,
                          const int32_t* misses, int32_t k, const void* host_k, const void* host_v,
                          void* pool_k, void* pool_v, void* stream);

typedef struct tsa_layer_io {
  const void* host_k;
  const void* host_v;
  void* pool_k;
  void* pool_v;
  const void* q;
  float* out;
} tsa_layer_io;

tsa_status tsa_hier_group_step(const tsa_cache_desc* desc, int32_t n_q_heads, int32_t n_layers,
                               const tsa_layer_io* layers, int32_t* page_table, int32_t* slot_token,
                               int32_t* last_use, const int32_t* sel, int32_t k, int32_t step,
                               int32_t policy, uint64_t seed, const int32_t* priority,
                               int32_t* slots_out, int32_t* hits, int32_t* misses, int32_t* miss_tok,
                               int32_t* miss_slot, void* ws, size_t ws_bytes, void* stream,
                               void* fetch_stream, void* const* events);

/* tsa_cache_reset - mark every page-table entry and slot empty (-1), so the
 * next step misses every selected token ([HISPARSE-NEWS]: the hot cache is
 * disposable, the host copy is authoritative). Uses a fill kernel. */
tsa_status tsa_cache_reset(const tsa_cache_desc* desc, int32_t* page_table, int32_t* slot_token,
                           int32_t* last_use, void* stream);

/* ------------------------------------------------------------------------
 * tsa_attend_rows - attention of every query head over a per-request row
 *   list shared by all heads ([KARAT] Eq. 2; with slot ids it is the
 *   attention over the hot cache, [HISPARSE-NEWS]).
 *   q        (device) [B][Hq][d]
 *   k_rows, v_rows (device) [B][n_rows][Hkv][d]
 *   row_ids  (device) int32 [B][max_rows], entries in [0, n_rows)
 *   row_counts (device, nullable) int32 [B] rows used per request, each in
 *            [0, max_rows]; NULL means max_rows for every request
 *   out      (device, out) fp32 [B][Hq][d]; zero for an empty list
 *   Workspace: tsa_workspace_bytes(TSA_OP_ATTEND_ROWS, desc, 0, ...).
 * ---------------------------------------------------------------------- */
tsa_status tsa_attend_rows(const tsa_attn_desc* desc, const void* q, const void* k_rows,
                           const void* v_rows, const int32_t* row_ids, const int32_t* row_counts,
                           float* out, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes for `op` with `desc` (the struct matching the op) and k. */
tsa_status tsa_workspace_bytes(int32_t op, const void* desc, int32_t k, size_t* bytes);

/* Pinned, device-mapped host memory for the authoritative KV copy
 * ([HISPARSE-NEWS]: full KV in pinned host memory). tsa_host_alloc returns
 * the host pointer, which the device may read directly. Set-up calls: they
 * allocate and are not for use inside a decode step. */
tsa_status tsa_host_alloc(size_t bytes, void** host_ptr);
tsa_status tsa_host_free(void* host_ptr);

/* Timing hook: arm (ev_start, ev_stop), two hipEvent_t as void*, to be
 * recorded on the call's stream immediately before and after the next
 * gather-attention kernel launched by this thread. One-shot. */
tsa_status tsa_time_next_gather(void* ev_start, void* ev_stop);

/* The same for a chosen kernel: TSA_TIMED_GATHER (the gather-attention
 * kernel, as tsa_time_next_gather), TSA_TIMED_TOKEN_SCAN (the indexer scan
 * of the next tsa_token_decode), TSA_TIMED_APPEND (the kernel of the next
 * tsa_kv_append / tsa_kv_append_multi) or TSA_TIMED_REGROW (the kernel of
 * the next tsa_index_regrow). One-shot per kernel; a call that fails
 * validation before its launch leaves the events armed. */
enum { TSA_TIMED_GATHER = 0, TSA_TIMED_TOKEN_SCAN = 1, TSA_TIMED_APPEND = 2, TSA_TIMED_REGROW = 3 };
tsa_status tsa_time_next_launch(int32_t kernel, void* ev_start, void* ev_stop);

/* Measurement probe (not part of the decode path): reads `bytes` (a
 * multiple of 16) at device address p once with 16-byte non-temporal loads,
 * each workgroup sweeping a contiguous chunk, writing one word per wave to
 * sink (device, at least tsa_stream_read_sink_bytes() bytes; the XOR of all
 * sink words is the XOR of the buffer's 32-bit words). Timed by the caller,
 * it gives a measured HBM streaming-read ceiling for the device. */
tsa_status tsa_stream_read(const void* p, size_t bytes, uint32_t* sink, size_t sink_bytes, void* stream);
size_t tsa_stream_read_sink_bytes(void);

const char* tsa_status_str(tsa_status s);
const char* tsa_last_error(void);
int32_t tsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TSA_H */
