"""Retrieval-based sparse-attention decode for AMD Instinct MI355X (gfx950).

The compute path is libtsa.so (hand-written HIP kernels behind the C ABI in
include/tsa.h); this package is its thin Python binding plus the seeded
synthetic workload generators. The library is loaded on first use and any
entry point raises ImportError when it has not been built.
"""

from . import workloads  # noqa: F401
from .binding import (  # noqa: F401
    BoundCall,
    HostArray,
    TsaError,
    abi_version,
    attend_rows,
    cache_reset,
    fetch_rows,
    hier_group_step,
    index_build,
    index_build_dyn,
    index_build_multi,
    index_build_dyn_multi,
    index_regrow,
    kv_append,
    kv_list_major,
    lib_path,
    load,
    resolve,
    sparse_decode,
    sparse_decode_dyn,
    sparse_decode_ex,
    sparse_decode_noalloc,
    time_next_gather,
    time_next_launch,
    stream_read,
    token_decode,
    workspace_bytes,
)

__all__ = [
    "workloads", "load", "lib_path", "abi_version", "index_build", "index_build_dyn", "index_build_multi", "index_build_dyn_multi", "index_regrow", "kv_append", "kv_list_major", "sparse_decode",
    "sparse_decode_dyn", "sparse_decode_ex", "sparse_decode_noalloc", "token_decode",
    "attend_rows", "resolve", "cache_reset", "fetch_rows", "hier_group_step", "HostArray", "time_next_gather", "time_next_launch", "stream_read", "workspace_bytes",
    "TsaError", "BoundCall",
]
