"""Plain fp64 CPU oracle for retrieval-based sparse-attention decode.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or run anything in this package. The product path
(the HIP library and its Python binding) never calls it and shares no code
with it: no kernels, headers, helpers, tables or pre/post-processing.

Every function here is the plain definition of what the decode path computes,
written from the pages:

  [KARAT]  paper-daily digest "Heterogeneous LLM Serving with General-Purpose
           Processing-Near-Memory for Retrieval-Based Sparse Attention":
           How (index structure: posting lists under centroids), core
           formulas (Eq. 2, masked sparse attention), worked example
           (steps 3-4: centroid similarity, top-10 lists, scan of the lists).
  [HISPARSE-NEWS]  "KV卸载上主机:HiSparse、PDD与DDR4回收", paper analysis 1
           (HiSparse): two-tier KV, hot cache of B slots per request per layer,
           page table + LRU, one fused RESOLVE step, exact by construction.
  [HISPARSE-NOTES] "10月14日学习笔记", HiSparse (motivation: an indexer picks
           the top-k tokens so the work falls from O(context) to O(k);
           method: LRU fits the locality of consecutive selections).

Arithmetic is fp64 on inputs widened exactly from their stored dtype
(bf16 or fp32). Selections use a full sort with ties broken by the lower
index. Softmax is two-pass (max, then normalised exponentials).

Modules:
  ivf    index build, centroid scoring, top-k lists, gather set, attention
  token  per-token indexer scoring and top-k
  cache  batch-step LRU over a fixed slot pool (RESOLVE), cache-mediated
         attention
  append per-step KV and posting-list append with per-list free entries
  variants cosine similarity; sink and window tokens beside the lists

Parity pins: every function is checked by tests marked ``not gpu`` against
closed forms, brute force on tiny inputs, a library routine for the dense
special case, and the op counts the KARAT worked example prints.
"""

from . import ivf, token, cache, append, variants  # noqa: F401
