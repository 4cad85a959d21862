"""ctypes binding over libtsa.so (include/tsa.h). Argument marshalling only:
torch supplies device memory and the current stream; every step of the decode
path runs in the library's HIP kernels. Loading fails loudly when the library
has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsa.so")

TSA_OK, TSA_ERR_INVALID_ARG, TSA_ERR_UNSUPPORTED, TSA_ERR_WORKSPACE, TSA_ERR_HIP = range(5)
TSA_F32, TSA_BF16 = 0, 1
(OP_INDEX_BUILD, OP_SPARSE_DECODE, OP_TOKEN_DECODE, OP_ATTEND_ROWS, OP_SPARSE_DECODE_EX, OP_INDEX_BUILD_MULTI,
 OP_SPARSE_DECODE_EX_MULTI) = range(7)
SIMILARITY = {"dot": 0, "cosine": 1}
SCHEDULE = {"auto": 0, "staged": 1, "fused": 2, "split": 3}
ABI_VERSION = 3  # TSA_ABI_VERSION of include/tsa.h
EVICT_POLICIES = {"lru": 0, "fifo": 1, "random": 2, "priority": 3}

_I32 = ctypes.c_int32
_P = ctypes.c_void_p


class IvfDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("n_tokens", _I32), ("n_kv_heads", _I32), ("n_q_heads", _I32),
                ("head_dim", _I32), ("n_centroids", _I32), ("shared_codebook", _I32), ("dtype", _I32)]


class TokenDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("n_tokens", _I32), ("n_kv_heads", _I32), ("n_q_heads", _I32),
                ("head_dim", _I32), ("idx_dim", _I32), ("dtype", _I32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("n_tokens", _I32), ("n_slots", _I32), ("n_kv_heads", _I32),
                ("head_dim", _I32), ("dtype", _I32)]


class DecodeOpts(ctypes.Structure):
    _fields_ = [("similarity", _I32), ("n_sink", _I32), ("n_window", _I32), ("assign_per_key", _I32),
                ("lengths", _P), ("lens", _P), ("alt", _P), ("schedule", _I32), ("k_lists", _P),
                ("v_lists", _P)]


class LayerIO(ctypes.Structure):
    _fields_ = [("host_k", _P), ("host_v", _P), ("pool_k", _P), ("pool_v", _P), ("q", _P), ("out", _P)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", _I32), ("n_rows", _I32), ("n_kv_heads", _I32), ("n_q_heads", _I32),
                ("head_dim", _I32), ("max_rows", _I32), ("dtype", _I32)]


# name -> argument types (all return tsa_status except where noted)
_SIGNATURES = {
    "tsa_index_build": [ctypes.POINTER(IvfDesc), _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_sparse_decode": [ctypes.POINTER(IvfDesc), _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                          ctypes.c_size_t, _P],
    "tsa_sparse_decode_noalloc": [ctypes.POINTER(IvfDesc), _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P],
    "tsa_sparse_decode_ex": [ctypes.POINTER(IvfDesc), ctypes.POINTER(DecodeOpts), _P, _P, _P, _P, _P, _P, _I32,
                             _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_index_build_multi": [ctypes.POINTER(IvfDesc), _P, _P, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_kv_list_major": [ctypes.POINTER(IvfDesc), _P, _P, _P, _P, _P, _P],
    "tsa_index_build_dyn": [ctypes.POINTER(IvfDesc), _P, _P, _I32, _I32, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_kv_append": [ctypes.POINTER(IvfDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "tsa_sparse_decode_dyn": [ctypes.POINTER(IvfDesc), _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                              ctypes.c_size_t, _P],
    "tsa_token_decode": [ctypes.POINTER(TokenDesc), _P, _P, _P, _P, _P, _I32, _P, _P, _P,
                         ctypes.c_size_t, _P],
    "tsa_resolve": [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P],
    "tsa_resolve_policy": [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _I32, _I32, _I32, ctypes.c_uint64, _P,
                           _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "tsa_fetch_rows": [ctypes.POINTER(CacheDesc), _P, _P, _P, _I32, _P, _P, _P, _P, _P],
    "tsa_hier_group_step": [ctypes.POINTER(CacheDesc), _I32, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32,
                            ctypes.c_uint64, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P],
    "tsa_cache_reset": [ctypes.POINTER(CacheDesc), _P, _P, _P, _P],
    "tsa_attend_rows": [ctypes.POINTER(AttnDesc), _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "tsa_workspace_bytes": [_I32, _P, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "tsa_workspace_bytes_multi": [_I32, _P, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "tsa_index_build_dyn_multi": [ctypes.POINTER(IvfDesc), _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P],
    "tsa_kv_append_multi": [ctypes.POINTER(IvfDesc), _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "tsa_index_regrow": [ctypes.POINTER(IvfDesc), _I32, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P],
    "tsa_host_alloc": [ctypes.c_size_t, ctypes.POINTER(_P)],
    "tsa_host_free": [_P],
    "tsa_time_next_gather": [_P, _P],
    "tsa_time_next_launch": [_I32, _P, _P],
    "tsa_stream_read": [_P, ctypes.c_size_t, _P, ctypes.c_size_t, _P],
}

_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libtsa.so (once). Raises ImportError when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m top_sparse_attention_centroid_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, args in _SIGNATURES.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = _I32
    lib.tsa_status_str.argtypes = [_I32]
    lib.tsa_status_str.restype = ctypes.c_char_p
    lib.tsa_last_error.argtypes = []
    lib.tsa_last_error.restype = ctypes.c_char_p
    lib.tsa_abi_version.argtypes = []
    lib.tsa_abi_version.restype = _I32
    lib.tsa_stream_read_sink_bytes.argtypes = []
    lib.tsa_stream_read_sink_bytes.restype = ctypes.c_size_t
    if lib.tsa_abi_version() != ABI_VERSION:  # the structs below follow one layout
        raise ImportError(f"{_LIB_PATH} has ABI {lib.tsa_abi_version()}, this binding expects {ABI_VERSION}; "
                          "rebuild it")
    _lib = lib
    return lib


class TsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{load().tsa_status_str(status).decode()}: {msg}")
        self.status = status


def _check(status: int):
    if status != TSA_OK:
        raise TsaError(status, load().tsa_last_error().decode())


class BoundCall:
    """A library call whose arguments were checked and marshalled once (the
    decode functions below with bind=True). Calling it issues the same C call
    again -- same tensors, sizes and stream -- with no Python-side checks; the
    C entry point still validates its arguments, and a failure status raises
    TsaError. Every kernel of the call runs on each call; only the host work
    shrinks, to the one foreign call (a serving loop that calls the C ABI
    directly gets the same). Holds references to what it points at; the
    tensors' contents may change between calls, their storage may not."""
    __slots__ = ("_fn", "_args", "_keep", "result")

    def __init__(self, fn, args, keep, result):
        self._fn, self._args, self._keep, self.result = fn, args, keep, result

    def __call__(self):
        status = self._fn(*self._args)
        if status:
            _check(status)
        return self.result


def _issue(bind: bool, fn, args: tuple, keep: tuple, result):
    """Run the C call now, or (bind) return it as a BoundCall."""
    if bind:
        return BoundCall(fn, args, keep, result)
    _check(fn(*args))
    return result


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return TSA_F32
    if t == torch.bfloat16:
        return TSA_BF16
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libtsa must be contiguous")
    return t.data_ptr()


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _i32(t: Optional[torch.Tensor], name: str, shape):
    if t is None:
        return
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be int32 {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")


def workspace_bytes(op: int, desc, k: int = 0, m: Optional[int] = None) -> int:
    """Workspace of an operation; m (lists per key) for the m-way operations."""
    n = ctypes.c_size_t()
    if m is None:
        _check(load().tsa_workspace_bytes(op, ctypes.cast(ctypes.pointer(desc), _P), k, ctypes.byref(n)))
    else:
        _check(load().tsa_workspace_bytes_multi(op, ctypes.cast(ctypes.pointer(desc), _P), k, m, ctypes.byref(n)))
    return n.value


def _workspace(op, desc, k, ws, device, m: Optional[int] = None) -> torch.Tensor:
    need = workspace_bytes(op, desc, k, m)
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace has {ws.numel() * ws.element_size()} bytes, needs {need}")
    return ws


# ----------------------------------------------------------------------------
# descriptors
# ----------------------------------------------------------------------------

def ivf_desc(keys: torch.Tensor, centroids: torch.Tensor, n_q_heads: int) -> IvfDesc:
    B, N, Hkv, d = keys.shape
    Bc, Hkv2, C, d2 = centroids.shape
    if Hkv2 != Hkv or d2 != d or Bc not in (1, B):
        raise ValueError(f"centroids {tuple(centroids.shape)} do not match keys {tuple(keys.shape)}")
    return IvfDesc(B, N, Hkv, n_q_heads, d, C, 1 if Bc == 1 else 0, _dtype_code(keys.dtype))


def token_desc(k_idx: torch.Tensor, k_cache: torch.Tensor, n_q_heads: int) -> TokenDesc:
    B, N, Hkv, d = k_cache.shape
    if tuple(k_idx.shape[:2]) != (B, N):
        raise ValueError("k_idx and k_cache disagree on batch / tokens")
    return TokenDesc(B, N, Hkv, n_q_heads, d, k_idx.shape[2], _dtype_code(k_cache.dtype))


def cache_desc(host_k: torch.Tensor, n_slots: int) -> CacheDesc:
    B, N, Hkv, d = host_k.shape
    return CacheDesc(B, N, n_slots, Hkv, d, _dtype_code(host_k.dtype))


def attn_desc(k_rows: torch.Tensor, n_q_heads: int, max_rows: int) -> AttnDesc:
    B, R, Hkv, d = k_rows.shape
    return AttnDesc(B, R, Hkv, n_q_heads, d, max_rows, _dtype_code(k_rows.dtype))


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI, without the tsa_ prefix)
# ----------------------------------------------------------------------------

def index_build(keys, centroids, *, offsets=None, ids=None, ws=None, stream=None):
    """Posting lists of the K cache: returns (offsets [B][Hkv][C+1], ids [B][Hkv][N])."""
    _dev(keys, "keys"), _dev(centroids, "centroids")
    if centroids.dtype != keys.dtype:
        raise ValueError("keys and centroids must share a dtype")
    desc = ivf_desc(keys, centroids, keys.shape[2])
    B, N, Hkv, _ = keys.shape
    C = centroids.shape[2]
    if offsets is None:
        offsets = torch.empty((B, Hkv, C + 1), dtype=torch.int32, device=keys.device)
    if ids is None:
        ids = torch.empty((B, Hkv, N), dtype=torch.int32, device=keys.device)
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(ids, "ids", (B, Hkv, N))
    ws = _workspace(OP_INDEX_BUILD, desc, 0, ws, keys.device)
    _check(load().tsa_index_build(ctypes.byref(desc), _ptr(keys), _ptr(centroids), _ptr(offsets),
                                  _ptr(ids), _ptr(ws), ws.numel(), _stream(stream)))
    return offsets, ids


def index_build_dyn(keys, centroids, n_prefix: int, slack: Optional[int] = None, *, offsets=None, lens=None,
                    ids=None, ws=None, stream=None):
    """Growing index over the first n_prefix tokens, `slack` free entries per
    list (default: the spare capacity shared evenly). Returns (offsets, lens, ids)."""
    _dev(keys, "keys"), _dev(centroids, "centroids")
    if centroids.dtype != keys.dtype:
        raise ValueError("keys and centroids must share a dtype")
    desc = ivf_desc(keys, centroids, keys.shape[2])
    B, N, Hkv, _ = keys.shape
    C = centroids.shape[2]
    if slack is None:
        slack = (N - n_prefix) // C
    if offsets is None:
        offsets = torch.empty((B, Hkv, C + 1), dtype=torch.int32, device=keys.device)
    if lens is None:
        lens = torch.empty((B, Hkv, C), dtype=torch.int32, device=keys.device)
    if ids is None:
        ids = torch.empty((B, Hkv, N), dtype=torch.int32, device=keys.device)
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(lens, "lens", (B, Hkv, C))
    _i32(ids, "ids", (B, Hkv, N))
    ws = _workspace(OP_INDEX_BUILD, desc, 0, ws, keys.device)
    _check(load().tsa_index_build_dyn(ctypes.byref(desc), _ptr(keys), _ptr(centroids), n_prefix, slack,
                                      _ptr(offsets), _ptr(lens), _ptr(ids), _ptr(ws), ws.numel(), _stream(stream)))
    return offsets, lens, ids


def kv_append(new_k, new_v, pos, centroids, k_cache, v_cache, offsets, lens, ids, *, alt=None, status=None,
              stream=None, bind: bool = False):
    """Store one new token per request at row pos[b] and add it to its posting
    list (with `alt`, an m-way index: to its m nearest lists, all or none).
    Returns status [B][Hkv] int32 (0 indexed, 1 a list full, 2 bad row);
    bind=True: the call as a BoundCall, not run."""
    for t, n in ((new_k, "new_k"), (new_v, "new_v"), (centroids, "centroids"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _dev(t, n)
    if not (new_k.dtype == new_v.dtype == centroids.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("new rows, centroids and caches must share a dtype")
    desc = ivf_desc(k_cache, centroids, k_cache.shape[2])
    B, N, Hkv, d = k_cache.shape
    C = desc.n_centroids
    if tuple(new_k.shape) != (B, Hkv, d) or tuple(new_v.shape) != (B, Hkv, d):
        raise ValueError("new_k / new_v must be [B][Hkv][d]")
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache and v_cache shapes differ")
    m = _lists_per_key(alt, B, Hkv, N)
    _i32(pos, "pos", (B,))
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(lens, "lens", (B, Hkv, C))
    _i32(ids, "ids", (B, Hkv, N * m))
    if status is None:
        status = torch.empty((B, Hkv), dtype=torch.int32, device=k_cache.device)
    _i32(status, "status", (B, Hkv))
    args = (ctypes.byref(desc), m, _ptr(new_k), _ptr(new_v), _ptr(pos), _ptr(centroids), _ptr(k_cache),
            _ptr(v_cache), _ptr(offsets), _ptr(lens), _ptr(ids), _ptr(alt), _ptr(status), _stream(stream))
    keep = (desc, new_k, new_v, pos, centroids, k_cache, v_cache, offsets, lens, ids, alt)
    return _issue(bind, load().tsa_kv_append_multi, args, keep, status)


def _alt_shape(B, Hkv, N, m):
    return (B, Hkv, N * m, m - 1)


def _lists_per_key(alt, B, Hkv, N) -> int:
    """m of an m-way index from its alt array ([B][Hkv][N*m][m-1]; None: 1)."""
    if alt is None:
        return 1
    if alt.dim() != 4 or alt.shape[3] < 1:
        raise ValueError(f"alt must be int32 [B][Hkv][N*m][m-1], got {tuple(alt.shape)}")
    m = alt.shape[3] + 1
    _i32(alt, "alt", _alt_shape(B, Hkv, N, m))
    return m


def index_build_multi(keys, centroids, m: int = 2, *, offsets=None, ids=None, alt=None, ws=None, stream=None):
    """Posting lists where every key joins its m nearest lists (1 <= m <= 4).
    Returns (offsets [B][Hkv][C+1], ids [B][Hkv][N*m], alt [B][Hkv][N*m][m-1] or None)."""
    _dev(keys, "keys"), _dev(centroids, "centroids")
    if centroids.dtype != keys.dtype:
        raise ValueError("keys and centroids must share a dtype")
    desc = ivf_desc(keys, centroids, keys.shape[2])
    B, N, Hkv, _ = keys.shape
    C = centroids.shape[2]
    if offsets is None:
        offsets = torch.empty((B, Hkv, C + 1), dtype=torch.int32, device=keys.device)
    if ids is None:
        ids = torch.empty((B, Hkv, N * m), dtype=torch.int32, device=keys.device)
    if alt is None and m > 1:
        alt = torch.empty(_alt_shape(B, Hkv, N, m), dtype=torch.int32, device=keys.device)
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(ids, "ids", (B, Hkv, N * m))
    if m > 1:
        _i32(alt, "alt", _alt_shape(B, Hkv, N, m))
    ws = _workspace(OP_INDEX_BUILD_MULTI, desc, 0, ws, keys.device, m)
    _check(load().tsa_index_build_multi(ctypes.byref(desc), _ptr(keys), _ptr(centroids), m, _ptr(offsets), _ptr(ids),
                                        _ptr(alt if m > 1 else None), _ptr(ws), ws.numel(), _stream(stream)))
    return offsets, ids, (alt if m > 1 else None)


def index_build_dyn_multi(keys, centroids, n_prefix: int, m: int, slack: Optional[int] = None, *, offsets=None,
                          lens=None, ids=None, alt=None, ws=None, stream=None):
    """Growing m-way index over the first n_prefix tokens with `slack` free
    entries per list (default: the spare entries shared evenly).
    Returns (offsets, lens, ids [B][Hkv][N*m], alt [B][Hkv][N*m][m-1] or None)."""
    _dev(keys, "keys"), _dev(centroids, "centroids")
    if centroids.dtype != keys.dtype:
        raise ValueError("keys and centroids must share a dtype")
    desc = ivf_desc(keys, centroids, keys.shape[2])
    B, N, Hkv, _ = keys.shape
    C = centroids.shape[2]
    if slack is None:
        slack = (N * m - n_prefix * m) // C
    dev = keys.device
    offsets = torch.empty((B, Hkv, C + 1), dtype=torch.int32, device=dev) if offsets is None else offsets
    lens = torch.empty((B, Hkv, C), dtype=torch.int32, device=dev) if lens is None else lens
    ids = torch.empty((B, Hkv, N * m), dtype=torch.int32, device=dev) if ids is None else ids
    if alt is None and m > 1:
        alt = torch.empty(_alt_shape(B, Hkv, N, m), dtype=torch.int32, device=dev)
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(lens, "lens", (B, Hkv, C))
    _i32(ids, "ids", (B, Hkv, N * m))
    if m > 1:
        _i32(alt, "alt", _alt_shape(B, Hkv, N, m))
    ws = _workspace(OP_INDEX_BUILD_MULTI, desc, 0, ws, dev, m)
    _check(load().tsa_index_build_dyn_multi(ctypes.byref(desc), _ptr(keys), _ptr(centroids), n_prefix, slack, m,
                                            _ptr(offsets), _ptr(lens), _ptr(ids), _ptr(alt if m > 1 else None),
                                            _ptr(ws), ws.numel(), _stream(stream)))
    return offsets, lens, ids, (alt if m > 1 else None)


def index_regrow(offsets, lens, ids, alt=None, slack: int = -1, *, out=None, status=None, stream=None):
    """Lay a growing index out again with `slack` free entries after every
    list (-1: as many as fit for every list), into new arrays (or `out`, a
    tuple (offsets, lens, ids, alt)). Returns ((offsets, lens, ids, alt), status)."""
    for t, n in ((offsets, "offsets"), (lens, "lens"), (ids, "ids")):
        _dev(t, n)
    B, Hkv, C1 = offsets.shape
    C = C1 - 1
    cap = ids.shape[2]
    m = 1 if alt is None else alt.shape[3] + 1
    if cap % m:
        raise ValueError("ids must hold N * m entries")
    N = cap // m
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(lens, "lens", (B, Hkv, C))
    _i32(ids, "ids", (B, Hkv, cap))
    if alt is not None:
        _i32(alt, "alt", _alt_shape(B, Hkv, N, m))
    if out is None:
        out = (torch.empty_like(offsets), torch.empty_like(lens), torch.empty_like(ids),
               None if alt is None else torch.empty_like(alt))
    if status is None:
        status = torch.empty((B, Hkv), dtype=torch.int32, device=ids.device)
    _i32(status, "status", (B, Hkv))
    desc = IvfDesc(B, N, Hkv, Hkv, 128, C, 1, 1)
    _check(load().tsa_index_regrow(ctypes.byref(desc), m, _ptr(offsets), _ptr(lens), _ptr(ids), _ptr(alt), slack,
                                   _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(out[3]), _ptr(status),
                                   _stream(stream)))
    return out, status


def sparse_decode_ex(q, centroids, offsets, ids, k_cache, v_cache, k: int, *, similarity: str = "dot",
                     n_sink: int = 0, n_window: int = 0, lengths=None, lens=None, alt=None, out=None,
                     sel_out=None, rows_out=None, uniq_out=None, ws=None, stream=None, schedule: str = "auto",
                     k_lists=None, v_lists=None, bind: bool = False):
    """Decode with the variants: cosine similarity and/or the first n_sink and
    last n_window tokens (before lengths[b]) attended beside the lists; with
    `alt` (an m-way index from index_build_multi or index_build_dyn_multi)
    every token sits in m lists and is attended once per head; with `lens`,
    a growing index. `schedule`: "auto", "staged" (scoring, select + plan,
    gather, combine launches), "fused" (one launch) or "split" (scoring, a
    select + attend launch over shares of each head's rows, combine); fused
    and split take plain decodes (one list per key, no sink or window,
    C <= 1024, k <= 64), split bf16 only. k_lists / v_lists: list-major
    copies of the caches from kv_list_major for this index, from which the
    chosen lists' rows are then read (plain lists only). bind=True returns
    the call as a BoundCall instead of running it."""
    for t, n in ((q, "q"), (centroids, "centroids"), (offsets, "offsets"), (ids, "ids"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    if not (q.dtype == centroids.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, centroids, k_cache and v_cache must share a dtype")
    if similarity not in SIMILARITY:
        raise ValueError(f"similarity must be one of {sorted(SIMILARITY)}")
    if schedule not in SCHEDULE:
        raise ValueError(f"schedule must be one of {sorted(SCHEDULE)}")
    B, Hq, d = q.shape
    desc = ivf_desc(k_cache, centroids, Hq)
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("q / k_cache / v_cache shapes disagree")
    Hkv, C, N = desc.n_kv_heads, desc.n_centroids, desc.n_tokens
    m = _lists_per_key(alt, B, Hkv, N)
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(ids, "ids", (B, Hkv, N * m))
    _i32(lengths, "lengths", (B,))
    _i32(lens, "lens", (B, Hkv, C))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, d):
        raise ValueError("out must be fp32 [B][Hq][d]")
    _i32(sel_out, "sel_out", (B, Hq, k))
    _i32(rows_out, "rows_out", (B, Hq))
    _i32(uniq_out, "uniq_out", (B, Hkv))
    for t, n in ((k_lists, "k_lists"), (v_lists, "v_lists")):
        if t is not None:
            _dev(t, n)
            if t.dtype != k_cache.dtype or tuple(t.shape) != (B, Hkv, N, d):
                raise ValueError(f"{n} must be {k_cache.dtype} [B][Hkv][N][d] = {(B, Hkv, N, d)}")
    opts = DecodeOpts(SIMILARITY[similarity], n_sink, n_window, m, _ptr(lengths), _ptr(lens), _ptr(alt),
                      SCHEDULE[schedule], _ptr(k_lists), _ptr(v_lists))
    ws = (_workspace(OP_SPARSE_DECODE_EX_MULTI, desc, k, ws, q.device, m) if m > 1
          else _workspace(OP_SPARSE_DECODE_EX, desc, k, ws, q.device))
    args = (ctypes.byref(desc), ctypes.byref(opts), _ptr(q), _ptr(centroids), _ptr(offsets), _ptr(ids),
            _ptr(k_cache), _ptr(v_cache), k, _ptr(out), _ptr(sel_out), _ptr(rows_out), _ptr(uniq_out), _ptr(ws),
            ws.numel(), _stream(stream))
    keep = (desc, opts, q, centroids, offsets, ids, k_cache, v_cache, lengths, lens, alt, sel_out, rows_out,
            uniq_out, ws, k_lists, v_lists)
    return _issue(bind, load().tsa_sparse_decode_ex, args, keep, out)


def kv_list_major(ids, k_cache, v_cache, *, k_lists=None, v_lists=None, stream=None):
    """List-major copies of the caches for a static index: k_lists[b][g][e] =
    k_cache[b][ids[b][g][e]][g] (zeros for an id outside [0, N)), likewise v.
    Returns (k_lists, v_lists), each [B][Hkv][N][d] of the caches' dtype."""
    for t, n in ((ids, "ids"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    if k_cache.dtype != v_cache.dtype or tuple(k_cache.shape) != tuple(v_cache.shape):
        raise ValueError("k_cache and v_cache must share a dtype and a shape")
    B, N, Hkv, d = k_cache.shape
    _i32(ids, "ids", (B, Hkv, N))
    if k_lists is None:
        k_lists = torch.empty((B, Hkv, N, d), dtype=k_cache.dtype, device=k_cache.device)
    if v_lists is None:
        v_lists = torch.empty((B, Hkv, N, d), dtype=k_cache.dtype, device=k_cache.device)
    for t, n in ((k_lists, "k_lists"), (v_lists, "v_lists")):
        _dev(t, n)
        if t.dtype != k_cache.dtype or tuple(t.shape) != (B, Hkv, N, d):
            raise ValueError(f"{n} must be {k_cache.dtype} [B][Hkv][N][d] = {(B, Hkv, N, d)}")
    desc = IvfDesc(B, N, Hkv, Hkv, d, 1, 1, _dtype_code(k_cache.dtype))
    _check(load().tsa_kv_list_major(ctypes.byref(desc), _ptr(ids), _ptr(k_cache), _ptr(v_cache), _ptr(k_lists),
                                    _ptr(v_lists), _stream(stream)))
    return k_lists, v_lists


def sparse_decode_dyn(q, centroids, offsets, lens, ids, k_cache, v_cache, k: int, **kw):
    """sparse_decode over a growing index (list c = ids[offsets[c] : offsets[c] + lens[c]])."""
    return sparse_decode(q, centroids, offsets, ids, k_cache, v_cache, k, lens=lens, **kw)


def sparse_decode(q, centroids, offsets, ids, k_cache, v_cache, k: int, *, out=None, sel_out=None,
                  rows_out=None, uniq_out=None, ws=None, stream=None, lens=None, bind: bool = False):
    """One retrieval-based sparse-attention decode step. Returns out [B][Hq][d]
    fp32 (bind=True: the call as a BoundCall, not run)."""
    for t, n in ((q, "q"), (centroids, "centroids"), (offsets, "offsets"), (ids, "ids"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    if not (q.dtype == centroids.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, centroids, k_cache and v_cache must share a dtype")
    B, Hq, d = q.shape
    desc = ivf_desc(k_cache, centroids, Hq)
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("q / k_cache / v_cache shapes disagree")
    Hkv, C, N = desc.n_kv_heads, desc.n_centroids, desc.n_tokens
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(ids, "ids", (B, Hkv, N))
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, d):
        raise ValueError("out must be fp32 [B][Hq][d]")
    _i32(sel_out, "sel_out", (B, Hq, k))
    _i32(rows_out, "rows_out", (B, Hq))
    _i32(uniq_out, "uniq_out", (B, Hkv))
    ws = _workspace(OP_SPARSE_DECODE, desc, k, ws, q.device)
    keep = (desc, q, centroids, offsets, ids, k_cache, v_cache, lens, sel_out, rows_out, uniq_out, ws)
    tail = (_ptr(k_cache), _ptr(v_cache), k, _ptr(out), _ptr(sel_out), _ptr(rows_out), _ptr(uniq_out), _ptr(ws),
            ws.numel(), _stream(stream))
    if lens is None:
        return _issue(bind, load().tsa_sparse_decode,
                      (ctypes.byref(desc), _ptr(q), _ptr(centroids), _ptr(offsets), _ptr(ids)) + tail, keep, out)
    _i32(lens, "lens", (B, Hkv, C))
    return _issue(bind, load().tsa_sparse_decode_dyn,
                  (ctypes.byref(desc), _ptr(q), _ptr(centroids), _ptr(offsets), _ptr(lens), _ptr(ids)) + tail,
                  keep, out)


def sparse_decode_noalloc(q, centroids, offsets, ids, k_cache, v_cache, k: int, *, out, sel_out=None,
                          rows_out=None, uniq_out=None, stream=None):
    """sparse_decode with the library's static device scratch instead of a
    workspace: the call allocates nothing, so `out` must be given."""
    for t, n in ((q, "q"), (centroids, "centroids"), (offsets, "offsets"), (ids, "ids"),
                 (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _dev(t, n)
    if not (q.dtype == centroids.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q, centroids, k_cache and v_cache must share a dtype")
    B, Hq, d = q.shape
    desc = ivf_desc(k_cache, centroids, Hq)
    if tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("q / k_cache / v_cache shapes disagree")
    Hkv, C, N = desc.n_kv_heads, desc.n_centroids, desc.n_tokens
    _i32(offsets, "offsets", (B, Hkv, C + 1))
    _i32(ids, "ids", (B, Hkv, N))
    if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, d):
        raise ValueError("out must be fp32 [B][Hq][d]")
    _i32(sel_out, "sel_out", (B, Hq, k))
    _i32(rows_out, "rows_out", (B, Hq))
    _i32(uniq_out, "uniq_out", (B, Hkv))
    _check(load().tsa_sparse_decode_noalloc(ctypes.byref(desc), _ptr(q), _ptr(centroids), _ptr(offsets), _ptr(ids),
                                            _ptr(k_cache), _ptr(v_cache), k, _ptr(out), _ptr(sel_out),
                                            _ptr(rows_out), _ptr(uniq_out), _stream(stream)))
    return out


def token_decode(q_idx, k_idx, q, k_cache, v_cache, k: int, *, out=None, sel_out=None, ws=None,
                 stream=None, bind: bool = False):
    """Token-indexer top-k + attention. Returns out [B][Hq][d] fp32
    (bind=True: the call as a BoundCall, not run)."""
    for t, n in ((q_idx, "q_idx"), (k_idx, "k_idx"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    if not (q_idx.dtype == k_idx.dtype == q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("all inputs must share a dtype")
    B, Hq, d = q.shape
    desc = token_desc(k_idx, k_cache, Hq)
    if tuple(q_idx.shape) != (B, desc.idx_dim) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q_idx / v_cache shapes disagree")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _i32(sel_out, "sel_out", (B, k))
    ws = _workspace(OP_TOKEN_DECODE, desc, k, ws, q.device)
    args = (ctypes.byref(desc), _ptr(q_idx), _ptr(k_idx), _ptr(q), _ptr(k_cache), _ptr(v_cache), k, _ptr(out),
            _ptr(sel_out), _ptr(ws), ws.numel(), _stream(stream))
    return _issue(bind, load().tsa_token_decode, args, (desc, q_idx, k_idx, q, k_cache, v_cache, sel_out, ws), out)


def attend_rows(q, k_rows, v_rows, row_ids, row_counts=None, *, out=None, ws=None, stream=None):
    """Attention of every query head over per-request row lists. row_ids [B][max_rows]."""
    for t, n in ((q, "q"), (k_rows, "k_rows"), (v_rows, "v_rows"), (row_ids, "row_ids")):
        _dev(t, n)
    B, Hq, d = q.shape
    max_rows = row_ids.shape[1]
    desc = attn_desc(k_rows, Hq, max_rows)
    _i32(row_ids, "row_ids", (B, max_rows))
    _i32(row_counts, "row_counts", (B,))
    if tuple(v_rows.shape) != tuple(k_rows.shape) or k_rows.shape[0] != B:
        raise ValueError("k_rows / v_rows / q shapes disagree")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    ws = _workspace(OP_ATTEND_ROWS, desc, 0, ws, q.device)
    _check(load().tsa_attend_rows(ctypes.byref(desc), _ptr(q), _ptr(k_rows), _ptr(v_rows), _ptr(row_ids),
                                  _ptr(row_counts), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def resolve(page_table, slot_token, last_use, sel, step: int, host_k, host_v, pool_k, pool_v, *,
            slots_out=None, hits=None, misses=None, stream=None, policy: str = "lru", seed: int = 0,
            priority=None):
    """One RESOLVE step for all requests. Returns (slots_out, hits, misses).

    policy: "lru" (default), "fifo", "random" (seeded) or "priority"
    (evict the largest priority[b][token] first; Belady with next-use steps)."""
    B, N, Hkv, d = host_k.shape
    S = pool_k.shape[1]
    k = sel.shape[1]
    desc = cache_desc(host_k, S)
    _i32(page_table, "page_table", (B, N))
    _i32(slot_token, "slot_token", (B, S))
    _i32(last_use, "last_use", (B, S))
    _i32(sel, "sel", (B, k))
    if tuple(pool_k.shape) != (B, S, Hkv, d) or tuple(pool_v.shape) != (B, S, Hkv, d):
        raise ValueError("pool shapes must be [B][S][Hkv][d]")
    if host_k.is_cuda or host_v.is_cuda:
        raise ValueError("host_k / host_v must be host-mapped memory (host_alloc)")
    dev = pool_k.device
    if slots_out is None:
        slots_out = torch.empty((B, k), dtype=torch.int32, device=dev)
    if hits is None:
        hits = torch.empty((B,), dtype=torch.int32, device=dev)
    if misses is None:
        misses = torch.empty((B,), dtype=torch.int32, device=dev)
    if policy not in EVICT_POLICIES:
        raise ValueError(f"unknown policy {policy!r}; one of {sorted(EVICT_POLICIES)}")
    if policy == "lru":
        _check(load().tsa_resolve(ctypes.byref(desc), _ptr(page_table), _ptr(slot_token), _ptr(last_use),
                                  _ptr(sel), k, step, _ptr(host_k), _ptr(host_v), _ptr(pool_k), _ptr(pool_v),
                                  _ptr(slots_out), _ptr(hits), _ptr(misses), _stream(stream)))
        return slots_out, hits, misses
    if policy == "priority":
        if priority is None:
            raise ValueError("policy 'priority' needs priority [B][N] int32")
        _dev(priority, "priority")
        _i32(priority, "priority", (B, N))
    _check(load().tsa_resolve_policy(ctypes.byref(desc), _ptr(page_table), _ptr(slot_token), _ptr(last_use),
                                     _ptr(sel), k, step, EVICT_POLICIES[policy], seed & ((1 << 64) - 1),
                                     _ptr(priority), _ptr(host_k), _ptr(host_v), _ptr(pool_k), _ptr(pool_v),
                                     _ptr(slots_out), _ptr(hits), _ptr(misses), None, None, _stream(stream)))
    return slots_out, hits, misses


def fetch_rows(miss_tok, miss_slot, misses, host_k, host_v, pool_k, pool_v, *, stream=None):
    """Copy the rows of a miss list from one more layer's host copy into its pool."""
    B, N, Hkv, d = host_k.shape
    S = pool_k.shape[1]
    k = miss_tok.shape[1]
    desc = cache_desc(host_k, S)
    _i32(miss_tok, "miss_tok", (B, k))
    _i32(miss_slot, "miss_slot", (B, k))
    _i32(misses, "misses", (B,))
    if host_k.is_cuda or host_v.is_cuda:
        raise ValueError("host_k / host_v must be host-mapped memory (host_alloc)")
    _check(load().tsa_fetch_rows(ctypes.byref(desc), _ptr(miss_tok), _ptr(miss_slot), _ptr(misses), k,
                                 _ptr(host_k), _ptr(host_v), _ptr(pool_k), _ptr(pool_v), _stream(stream)))


def hier_group_step(layers, page_table, slot_token, last_use, sel, step: int, *, policy: str = "lru",
                    seed: int = 0, priority=None, slots_out=None, hits=None, misses=None, miss_tok=None,
                    miss_slot=None, ws=None, stream=None, fetch_stream=None, events=None):
    """One decode step of a layer group sharing `sel`. layers: list of dicts
    with host_k, host_v (host-mapped), pool_k, pool_v, q, out (device). With
    fetch_stream (and two events) the later layers' rows are fetched on that
    stream while the first layer attends. Returns (slots, hits, misses)."""
    L0 = layers[0]
    B, N, Hkv, d = L0["host_k"].shape
    S = L0["pool_k"].shape[1]
    Hq = L0["q"].shape[1]
    k = sel.shape[1]
    desc = cache_desc(L0["host_k"], S)
    dev = L0["pool_k"].device
    if policy not in EVICT_POLICIES:
        raise ValueError(f"unknown policy {policy!r}")
    for name, t in (("slots_out", slots_out), ("miss_tok", miss_tok), ("miss_slot", miss_slot)):
        _i32(t, name, (B, k))
    slots_out = torch.empty((B, k), dtype=torch.int32, device=dev) if slots_out is None else slots_out
    hits = torch.empty((B,), dtype=torch.int32, device=dev) if hits is None else hits
    misses = torch.empty((B,), dtype=torch.int32, device=dev) if misses is None else misses
    if len(layers) > 1:
        miss_tok = torch.empty((B, k), dtype=torch.int32, device=dev) if miss_tok is None else miss_tok
        miss_slot = torch.empty((B, k), dtype=torch.int32, device=dev) if miss_slot is None else miss_slot
    arr = (LayerIO * len(layers))()
    for j, L in enumerate(layers):
        if L["host_k"].is_cuda or L["host_v"].is_cuda:
            raise ValueError("host_k / host_v must be host-mapped memory (host_alloc)")
        if tuple(L["pool_k"].shape) != (B, S, Hkv, d) or tuple(L["out"].shape) != (B, Hq, d):
            raise ValueError(f"layer {j}: pool or out shape disagrees with layer 0")
        arr[j] = LayerIO(_ptr(L["host_k"]), _ptr(L["host_v"]), _ptr(L["pool_k"]), _ptr(L["pool_v"]),
                         _ptr(L["q"]), _ptr(L["out"]))
    adesc = attn_desc(L0["pool_k"], Hq, k)
    ws = _workspace(OP_ATTEND_ROWS, adesc, 0, ws, dev)
    ev_arr = None
    if fetch_stream is not None and len(layers) > 1:
        if events is None or len(events) < 2:
            raise ValueError("fetch_stream needs two events (fork and join)")
        for ev in events[:2]:
            if not ev.cuda_event:
                ev.record()
        ev_arr = (_P * 2)(events[0].cuda_event, events[1].cuda_event)
    _check(load().tsa_hier_group_step(ctypes.byref(desc), Hq, len(layers), ctypes.cast(arr, _P), _ptr(page_table),
                                      _ptr(slot_token), _ptr(last_use), _ptr(sel), k, step, EVICT_POLICIES[policy],
                                      seed & ((1 << 64) - 1), _ptr(priority), _ptr(slots_out), _ptr(hits),
                                      _ptr(misses), _ptr(miss_tok), _ptr(miss_slot), _ptr(ws), ws.numel(),
                                      _stream(stream), _stream(fetch_stream) if fetch_stream is not None else None,
                                      ctypes.cast(ev_arr, _P) if ev_arr is not None else None))
    return slots_out, hits, misses


def cache_reset(page_table, slot_token, last_use, stream=None):
    B, N = page_table.shape
    S = slot_token.shape[1]
    desc = CacheDesc(B, N, S, 1, 128, TSA_BF16)
    _check(load().tsa_cache_reset(ctypes.byref(desc), _ptr(page_table), _ptr(slot_token), _ptr(last_use),
                                  _stream(stream)))


class HostArray:
    """Pinned, device-readable host memory from tsa_host_alloc, viewed as a
    torch CPU tensor (``.tensor``). Freed when this object is collected."""

    def __init__(self, shape, dtype: torch.dtype):
        nbytes = int(torch.Size(shape).numel()) * torch.empty((), dtype=dtype).element_size()
        p = _P()
        _check(load().tsa_host_alloc(max(nbytes, 1), ctypes.byref(p)))
        self._ptr = p.value
        buf = (ctypes.c_uint8 * max(nbytes, 1)).from_address(self._ptr)
        self.tensor = torch.frombuffer(buf, dtype=torch.uint8)[:nbytes].view(dtype).view(shape)

    def __del__(self):
        if getattr(self, "_ptr", None):
            self.tensor = None
            load().tsa_host_free(self._ptr)
            self._ptr = None


def time_next_gather(ev_start: torch.cuda.Event, ev_stop: torch.cuda.Event):
    """Have the next gather-attention launch of this thread record the two
    events around itself (on the stream of that call)."""
    for ev in (ev_start, ev_stop):
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record()
    _check(load().tsa_time_next_gather(_P(ev_start.cuda_event), _P(ev_stop.cuda_event)))


TIMED_GATHER, TIMED_TOKEN_SCAN, TIMED_APPEND, TIMED_REGROW = 0, 1, 2, 3


def time_next_launch(kernel: int, ev_start: torch.cuda.Event, ev_stop: torch.cuda.Event):
    """Have the next launch of `kernel` (TIMED_GATHER, TIMED_TOKEN_SCAN,
    TIMED_APPEND or TIMED_REGROW) by this thread record the two events around
    itself (on that call's stream)."""
    for ev in (ev_start, ev_stop):
        if not ev.cuda_event:
            ev.record()
    _check(load().tsa_time_next_launch(kernel, _P(ev_start.cuda_event), _P(ev_stop.cuda_event)))


def stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Measurement probe: read every byte of the device tensor `buf` once with
    non-temporal 16-byte loads (no decode work). Returns the sink words."""
    _dev(buf, "buf")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    nbytes = buf.numel() * buf.element_size()
    need = load().tsa_stream_read_sink_bytes()
    if sink is None:
        sink = torch.empty(need // 4, dtype=torch.int32, device=buf.device)
    _check(load().tsa_stream_read(_ptr(buf), nbytes, _ptr(sink), sink.numel() * 4, _stream(stream)))
    return sink


def abi_version() -> int:
    return load().tsa_abi_version()
