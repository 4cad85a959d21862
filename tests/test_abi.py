"""The C-ABI library: it loads, exports every symbol include/tsa.h declares, and
rejects bad arguments on the host before touching a device (no GPU needed)."""

import ctypes
import os
import re

import pytest

from top_sparse_attention_centroid_amd import binding as B

# floats per partial softmax state in the workspace: five whole 128-byte
# lines (m, l and zero fill; then o[128])
PART_FLOATS = 160

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        from top_sparse_attention_centroid_amd import build
        build.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsa_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("tsa_index_build", "tsa_sparse_decode", "tsa_token_decode", "tsa_resolve",
              "tsa_attend_rows", "tsa_cache_reset", "tsa_workspace_bytes", "tsa_status_str",
              "tsa_last_error", "tsa_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert lib.tsa_abi_version() == B.ABI_VERSION == 3
    assert lib.tsa_status_str(B.TSA_ERR_WORKSPACE) == b"TSA_ERR_WORKSPACE"
    assert lib.tsa_status_str(99) == b"TSA_ERR_UNKNOWN"


def _status(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_workspace_sizes_and_validation(lib):
    d = B.IvfDesc(64, 32768, 8, 32, 128, 256, 1, B.TSA_BF16)
    n = B.workspace_bytes(B.OP_SPARSE_DECODE, d, 16)
    G, smax = 4, 4 * 16 + 32768 // 256
    assert n >= 64 * 8 * smax * G * PART_FLOATS * 4
    # 512 groups fill the chip with 256-row plan segments: no finer cut (128-row
    # segments would need this many partial states)
    assert n < 64 * 8 * (4 * 16 + 32768 // 128) * G * PART_FLOATS * 4
    # one request with 100-row lists: 8 groups x 40 lists would give 320 waves, so
    # lists are cut into 32-row segments (the shortest), and the scores get a
    # buffer of their own
    one = B.IvfDesc(1, 100_000, 8, 32, 128, 1000, 0, B.TSA_BF16)
    n1 = B.workspace_bytes(B.OP_SPARSE_DECODE, one, 10)
    assert n1 >= 8 * (4 * 10 + 100_000 // 32) * G * PART_FLOATS * 4 + 8 * G * 1000 * 4
    assert n1 < 8 * (4 * 10 + 100_000 // 16) * G * PART_FLOATS * 4
    assert B.workspace_bytes(B.OP_INDEX_BUILD, d) >= 64 * 8 * 32768 * 4
    with pytest.raises(B.TsaError, match="INVALID_ARG"):
        B.workspace_bytes(B.OP_SPARSE_DECODE, d, 0)
    with pytest.raises(B.TsaError, match="INVALID_ARG"):
        B.workspace_bytes(B.OP_SPARSE_DECODE, d, 257)
    for bad, code in ((B.IvfDesc(1, 10, 8, 32, 64, 16, 1, 1), "UNSUPPORTED"),    # d != 128
                      (B.IvfDesc(1, 10, 8, 24, 128, 16, 1, 1), "UNSUPPORTED"),   # G = 3
                      (B.IvfDesc(1, 10, 8, 32, 128, 5000, 1, 1), "UNSUPPORTED"), # C too big
                      (B.IvfDesc(1, 10, 8, 32, 128, 16, 1, 7), "UNSUPPORTED"),   # dtype
                      (B.IvfDesc(0, 10, 8, 32, 128, 16, 1, 1), "INVALID_ARG")):
        with pytest.raises(B.TsaError, match=code):
            B.workspace_bytes(B.OP_SPARSE_DECODE, bad, 4)
    t = B.TokenDesc(16, 200_000, 8, 32, 128, 64, B.TSA_BF16)
    assert B.workspace_bytes(B.OP_TOKEN_DECODE, t, 2048) > 0
    with pytest.raises(B.TsaError, match="UNSUPPORTED"):
        B.workspace_bytes(B.OP_TOKEN_DECODE, B.TokenDesc(1, 1000, 8, 32, 128, 32, 1), 10)
    # 2M tokens are fine now; the limit is 4096 filter chunks of 4096 keys
    assert B.workspace_bytes(B.OP_TOKEN_DECODE, B.TokenDesc(1, 2_000_000, 8, 32, 128, 64, 1), 4096) > 0
    with pytest.raises(B.TsaError, match="UNSUPPORTED"):
        B.workspace_bytes(B.OP_TOKEN_DECODE, B.TokenDesc(1, 4096 * 4096 + 1, 8, 32, 128, 64, 1), 4096)
    a = B.AttnDesc(32, 4096, 8, 32, 128, 2048, B.TSA_BF16)
    # 32 x 8 row lists of 2048 rows: 256-row segments (2048 of them), G = 4 partial states each
    assert B.workspace_bytes(B.OP_ATTEND_ROWS, a) == 32 * 8 * (2048 // 256) * 4 * PART_FLOATS * 4
    small = B.AttnDesc(2, 4096, 8, 32, 128, 2048, B.TSA_BF16)   # few lists: 64-row segments
    assert B.workspace_bytes(B.OP_ATTEND_ROWS, small) == 2 * 8 * (2048 // 64) * 4 * PART_FLOATS * 4


def test_calls_reject_bad_arguments_before_any_launch(lib):
    d = B.IvfDesc(2, 100, 2, 8, 128, 8, 1, B.TSA_BF16)
    fake = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: validation fails first
    fake2 = ctypes.c_void_p(0x20000)       # a second such pointer
    odd = ctypes.c_void_p(0x10001)
    args = [ctypes.byref(d), fake, fake, fake, fake, fake, fake]
    ws_need = B.workspace_bytes(B.OP_SPARSE_DECODE, d, 4)
    # null q
    st = lib.tsa_sparse_decode(ctypes.byref(d), None, fake, fake, fake, fake, fake, 4, fake, None, None,
                               None, fake, ws_need, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"q is NULL" in lib.tsa_last_error()
    # misaligned k_cache
    st = lib.tsa_sparse_decode(ctypes.byref(d), fake, fake, fake, fake, odd, fake, 4, fake, None, None,
                               None, fake, ws_need, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"aligned" in lib.tsa_last_error()
    # k out of range
    st = lib.tsa_sparse_decode(*args, 9, fake, None, None, None, fake, ws_need, None)
    assert st == B.TSA_ERR_INVALID_ARG
    # workspace too small
    st = lib.tsa_sparse_decode(*args, 4, fake, None, None, None, fake, ws_need - 1, None)
    assert st == B.TSA_ERR_WORKSPACE
    # resolve: k larger than the slot pool, too many slots
    c = B.CacheDesc(2, 1000, 64, 8, 128, B.TSA_BF16)
    st = lib.tsa_resolve(ctypes.byref(c), fake, fake, fake, fake, 65, 0, fake, fake, fake, fake, fake,
                         None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG
    c2 = B.CacheDesc(2, 10000, 8192, 8, 128, B.TSA_BF16)
    st = lib.tsa_resolve(ctypes.byref(c2), fake, fake, fake, fake, 16, 0, fake, fake, fake, fake, fake,
                         None, None, None)
    assert st == B.TSA_ERR_UNSUPPORTED
    st = lib.tsa_resolve(ctypes.byref(c), fake, fake, fake, fake, 16, -1, fake, fake, fake, fake, fake,
                         None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG
    # decode variants: bad similarity, too many fixed rows, null opts
    ws_ex = B.workspace_bytes(B.OP_SPARSE_DECODE_EX, d, 4)
    assert ws_ex > ws_need
    for opts in (B.DecodeOpts(2, 0, 0, 0, None, None, None), B.DecodeOpts(0, 5000, 4000, 0, None, None, None),
                 B.DecodeOpts(0, -1, 0, 0, None, None, None), B.DecodeOpts(0, 0, 0, 2, None, None, None),
                 B.DecodeOpts(0, 0, 0, 3, None, None, None)):
        st = lib.tsa_sparse_decode_ex(ctypes.byref(d), ctypes.byref(opts), fake, fake, fake, fake, fake, fake, 4,
                                      fake, None, None, None, fake, ws_ex, None)
        assert st == B.TSA_ERR_INVALID_ARG
    # schedule: an unknown value; the fused schedule for decodes it does not take
    for bad in (-1, 4):
        opts = B.DecodeOpts(0, 0, 0, 0, None, None, None, bad)
        st = lib.tsa_sparse_decode_ex(ctypes.byref(d), ctypes.byref(opts), fake, fake, fake, fake, fake, fake, 4,
                                      fake, None, None, None, fake, ws_ex, None)
        assert st == B.TSA_ERR_INVALID_ARG and b"unknown schedule" in lib.tsa_last_error()
    d_f32 = B.IvfDesc(2, 100, 2, 8, 128, 8, 1, B.TSA_F32)
    opts = B.DecodeOpts(0, 0, 0, 0, None, None, None, B.SCHEDULE["split"])
    st = lib.tsa_sparse_decode_ex(ctypes.byref(d_f32), ctypes.byref(opts), fake, fake, fake, fake, fake, fake, 4,
                                  fake, None, None, None, fake, 1 << 30, None)
    assert st == B.TSA_ERR_UNSUPPORTED and b"bf16" in lib.tsa_last_error()
    fused = B.SCHEDULE["fused"]
    d_wide = B.IvfDesc(2, 5000, 2, 8, 128, 2000, 1, B.TSA_BF16)
    ws_wide = B.workspace_bytes(B.OP_SPARSE_DECODE_EX, d_wide, 65)
    for desc, opts, kk in ((d, B.DecodeOpts(0, 4, 0, 0, None, None, None, fused), 4),     # sink rows
                           (d, B.DecodeOpts(0, 0, 2, 0, None, None, None, fused), 4),     # window rows
                           (d, B.DecodeOpts(0, 0, 0, 2, None, None, 0x30000, fused), 4),  # two lists per key
                           (d_wide, B.DecodeOpts(0, 0, 0, 0, None, None, None, fused), 4),    # C > 1024
                           (d_wide, B.DecodeOpts(0, 0, 0, 0, None, None, None, fused), 65)):  # k > 64
        st = lib.tsa_sparse_decode_ex(ctypes.byref(desc), ctypes.byref(opts), fake, fake, fake, fake, fake, fake,
                                      kk, fake, None, None, None, fake, ws_wide, None)
        assert st == B.TSA_ERR_UNSUPPORTED and b"fused and split" in lib.tsa_last_error(), (opts.n_sink, kk)
        opts.schedule = B.SCHEDULE["split"]
        st = lib.tsa_sparse_decode_ex(ctypes.byref(desc), ctypes.byref(opts), fake, fake, fake, fake, fake, fake,
                                      kk, fake, None, None, None, fake, ws_wide, None)
        assert st == B.TSA_ERR_UNSUPPORTED and b"fused and split" in lib.tsa_last_error(), (opts.n_sink, kk)
    # list-major copies: both or neither, aligned, plain lists only
    fake3, fake4 = ctypes.c_void_p(0x30000), ctypes.c_void_p(0x40000)
    for opts, want, msg in ((B.DecodeOpts(0, 0, 0, 0, None, None, None, 0, fake3, None), B.TSA_ERR_INVALID_ARG,
                             b"both or neither"),
                            (B.DecodeOpts(0, 0, 0, 0, None, None, None, 0, odd, fake4), B.TSA_ERR_INVALID_ARG,
                             b"aligned"),
                            (B.DecodeOpts(0, 4, 0, 0, None, None, None, 0, fake3, fake4), B.TSA_ERR_UNSUPPORTED,
                             b"plain lists"),
                            (B.DecodeOpts(0, 0, 2, 0, None, None, None, 0, fake3, fake4), B.TSA_ERR_UNSUPPORTED,
                             b"plain lists"),
                            (B.DecodeOpts(0, 0, 0, 0, None, fake2, None, 0, fake3, fake4), B.TSA_ERR_UNSUPPORTED,
                             b"plain lists"),
                            (B.DecodeOpts(0, 0, 0, 2, None, None, 0x50000, 0, fake3, fake4),
                             B.TSA_ERR_UNSUPPORTED, b"plain lists")):
        st = lib.tsa_sparse_decode_ex(ctypes.byref(d), ctypes.byref(opts), fake, fake, fake, fake, fake, fake, 4,
                                      fake, None, None, None, fake, 1 << 30, None)
        assert st == want and msg in lib.tsa_last_error(), lib.tsa_last_error()
    st = lib.tsa_kv_list_major(ctypes.byref(d), fake, fake, fake2, None, fake4, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"k_lists is NULL" in lib.tsa_last_error()
    st = lib.tsa_kv_list_major(ctypes.byref(d), fake, fake, fake2, fake3, fake3, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"separate" in lib.tsa_last_error()
    st = lib.tsa_kv_list_major(ctypes.byref(d), fake, fake, fake2, fake, fake4, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"separate" in lib.tsa_last_error()
    st = lib.tsa_kv_list_major(ctypes.byref(d), fake, fake, fake2, odd, fake4, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"aligned" in lib.tsa_last_error()
    d_big = B.IvfDesc(8192, 100, 16, 16, 128, 8, 1, B.TSA_BF16)
    st = lib.tsa_kv_list_major(ctypes.byref(d_big), fake, fake, fake2, fake3, fake4, None)
    assert st == B.TSA_ERR_UNSUPPORTED
    assert B.workspace_bytes(B.OP_SPARSE_DECODE_EX_MULTI, d, 4) > ws_ex
    assert B.workspace_bytes(B.OP_INDEX_BUILD_MULTI, d) > B.workspace_bytes(B.OP_INDEX_BUILD, d)
    for m in (0, 5):
        st = lib.tsa_index_build_multi(ctypes.byref(d), fake, fake, m, fake, fake, fake, fake, 1 << 30, None)
        assert st == B.TSA_ERR_UNSUPPORTED
    for m in (2, 3, 4):
        st = lib.tsa_index_build_multi(ctypes.byref(d), fake, fake, m, fake, fake, None, fake, 1 << 30, None)
        assert st == B.TSA_ERR_INVALID_ARG and b"alt is NULL" in lib.tsa_last_error()
    # m-way workspaces grow with m; m outside [1, 4] is refused
    ws_m = [B.workspace_bytes(B.OP_INDEX_BUILD_MULTI, d, 0, m) for m in (1, 2, 3, 4)]
    assert ws_m[0] == B.workspace_bytes(B.OP_INDEX_BUILD, d) and ws_m == sorted(ws_m) and len(set(ws_m)) == 4
    assert B.workspace_bytes(B.OP_INDEX_BUILD_MULTI, d, 0, 2) == B.workspace_bytes(B.OP_INDEX_BUILD_MULTI, d)
    assert B.workspace_bytes(B.OP_SPARSE_DECODE_EX_MULTI, d, 4, 4) > B.workspace_bytes(B.OP_SPARSE_DECODE_EX_MULTI, d, 4)
    n = ctypes.c_size_t()
    assert lib.tsa_workspace_bytes_multi(B.OP_INDEX_BUILD_MULTI, ctypes.cast(ctypes.pointer(d), ctypes.c_void_p), 0,
                                         5, ctypes.byref(n)) == B.TSA_ERR_UNSUPPORTED
    # growing m-way index: capacity N * m, alt and lens required
    st = lib.tsa_index_build_dyn_multi(ctypes.byref(d), fake, fake, 10, d.n_tokens, 2, fake, fake, fake, fake,
                                       fake, 1 << 30, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"exceeds" in lib.tsa_last_error()
    st = lib.tsa_index_build_dyn_multi(ctypes.byref(d), fake, fake, 10, 0, 3, fake, fake, fake, None, fake,
                                       1 << 30, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"alt is NULL" in lib.tsa_last_error()
    st = lib.tsa_index_build_dyn_multi(ctypes.byref(d), fake, fake, 10, 0, 2, fake, None, fake, fake, fake,
                                       1 << 30, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"lens is NULL" in lib.tsa_last_error()
    st = lib.tsa_kv_append_multi(ctypes.byref(d), 2, fake, fake, fake, fake, fake, fake, fake, fake, fake, None,
                                 None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"alt is NULL" in lib.tsa_last_error()
    st = lib.tsa_kv_append_multi(ctypes.byref(d), 5, fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                 None, None)
    assert st == B.TSA_ERR_UNSUPPORTED
    # regrow: separate outputs, alt for m >= 2
    st = lib.tsa_index_regrow(ctypes.byref(d), 1, fake, fake, fake, None, -1, fake2, fake2, fake, None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"alias" in lib.tsa_last_error()
    st = lib.tsa_index_regrow(ctypes.byref(d), 2, fake, fake, fake, None, -1, fake2, fake2, fake2, fake2, None,
                              None)
    assert st == B.TSA_ERR_INVALID_ARG and b"alt is NULL" in lib.tsa_last_error()
    st = lib.tsa_sparse_decode_ex(ctypes.byref(d), None, fake, fake, fake, fake, fake, fake, 4, fake, None, None,
                                  None, fake, ws_ex, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"opts is NULL" in lib.tsa_last_error()
    # replacement policy: unknown policy, priority policy without priorities
    st = lib.tsa_resolve_policy(ctypes.byref(c), fake, fake, fake, fake, 16, 0, 4, 0, None, fake, fake, fake,
                                fake, fake, None, None, None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"policy" in lib.tsa_last_error()
    st = lib.tsa_resolve_policy(ctypes.byref(c), fake, fake, fake, fake, 16, 0, 3, 0, None, fake, fake, fake,
                                fake, fake, None, None, None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"priority is NULL" in lib.tsa_last_error()
    st = lib.tsa_resolve_policy(ctypes.byref(c), fake, fake, fake, fake, 16, 0, 0, 0, None, fake, fake, fake,
                                fake, fake, None, None, fake, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"miss_tok and miss_slot" in lib.tsa_last_error()
    # layer group: no layers, a NULL layer pointer, events missing for a fetch stream
    io = (B.LayerIO * 2)(B.LayerIO(fake, fake, fake, fake, fake, fake), B.LayerIO(fake, None, fake, fake, fake, fake))
    ws_at = B.workspace_bytes(B.OP_ATTEND_ROWS, B.AttnDesc(2, 64, 8, 32, 128, 16, B.TSA_BF16))
    st = lib.tsa_hier_group_step(ctypes.byref(c), 32, 0, ctypes.cast(io, ctypes.c_void_p), fake, fake, fake, fake,
                                 16, 0, 0, 0, None, fake, fake, fake, fake, fake, fake, ws_at, None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"n_layers" in lib.tsa_last_error()
    st = lib.tsa_hier_group_step(ctypes.byref(c), 32, 2, ctypes.cast(io, ctypes.c_void_p), fake, fake, fake, fake,
                                 16, 0, 0, 0, None, fake, fake, fake, fake, fake, fake, ws_at, None, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"layers[1]" in lib.tsa_last_error()
    st = lib.tsa_hier_group_step(ctypes.byref(c), 32, 2, ctypes.cast(io, ctypes.c_void_p), fake, fake, fake, fake,
                                 16, 0, 0, 0, None, fake, fake, fake, fake, fake, fake, ws_at, None, fake, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"events is NULL" in lib.tsa_last_error()
    # token decode: k > N
    t = B.TokenDesc(1, 100, 8, 32, 128, 64, B.TSA_BF16)
    st = lib.tsa_token_decode(ctypes.byref(t), fake, fake, fake, fake, fake, 101, fake, None, fake, 1 << 30, None)
    assert st == B.TSA_ERR_INVALID_ARG
    # growing index: prefix and slack must fit the capacity; append needs lens
    ws_ix = B.workspace_bytes(B.OP_INDEX_BUILD, d)
    st = lib.tsa_index_build_dyn(ctypes.byref(d), fake, fake, 0, 0, fake, fake, fake, fake, ws_ix, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"n_prefix" in lib.tsa_last_error()
    st = lib.tsa_index_build_dyn(ctypes.byref(d), fake, fake, 60, 6, fake, fake, fake, fake, ws_ix, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"slack" in lib.tsa_last_error()   # 60 + 8 * 6 > 100
    st = lib.tsa_index_build_dyn(ctypes.byref(d), fake, fake, 60, 5, fake, None, fake, fake, ws_ix, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"lens is NULL" in lib.tsa_last_error()
    st = lib.tsa_kv_append(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, None, fake, None, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"lens is NULL" in lib.tsa_last_error()
    st = lib.tsa_sparse_decode_dyn(ctypes.byref(d), fake, fake, fake, None, fake, fake, fake, 4, fake, None, None,
                                   None, fake, ws_need, None)
    assert st == B.TSA_ERR_INVALID_ARG and b"lens is NULL" in lib.tsa_last_error()
    # timing hook needs both events
    assert lib.tsa_time_next_gather(fake, None) == B.TSA_ERR_INVALID_ARG
    assert lib.tsa_time_next_gather(None, None) == B.TSA_OK
    for kind in (B.TIMED_GATHER, B.TIMED_TOKEN_SCAN, B.TIMED_APPEND, B.TIMED_REGROW):
        assert lib.tsa_time_next_launch(kind, None, fake) == B.TSA_ERR_INVALID_ARG
        assert lib.tsa_time_next_launch(kind, None, None) == B.TSA_OK     # disarms
    assert lib.tsa_time_next_launch(4, None, None) == B.TSA_ERR_INVALID_ARG
    assert b"unknown timed kernel" in lib.tsa_last_error()


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 4, 1, 128), dtype=torch.bfloat16)
    c = torch.zeros((1, 1, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        B.index_build(x, c)


def test_bound_call_reissues_its_call_and_raises_a_failure_status(lib):
    """BoundCall issues the stored foreign call with the stored arguments on
    every call, returns the stored result, and turns a failure status into
    TsaError as the direct calls do."""
    seen = []

    def fn(*args):
        seen.append(args)
        return B.TSA_OK if len(seen) < 3 else B.TSA_ERR_INVALID_ARG

    keep = object()
    call = B.BoundCall(fn, (7, None, 3.5), (keep,), "result")
    assert call() == "result" and call() == "result"
    with pytest.raises(B.TsaError, match="TSA_ERR_INVALID_ARG"):
        call()
    assert seen == [(7, None, 3.5)] * 3


def _ivf_ws(B_, N, Hkv, Hq, C, k, rows, keys):
    """Workspace bytes of a plain sparse decode whose lists are cut into
    `rows`-row plan segments (layout: descriptors, counts, partial states,
    and for bf16 the score keys of a scoring launch of its own, which the
    staged path's small batches and every split decode use, and the split
    decode's arrival counters, one per query head; each region 256-B
    aligned)."""
    def al(x):
        return (x + 255) // 256 * 256
    G, bh = Hq // Hkv, B_ * Hkv
    smax = G * k + -(-N // rows)
    return (al(bh * smax * 16) + al(bh * 4) + al(bh * smax * G * PART_FLOATS * 4)
            + (al(bh * G * C * 4) + al(bh * G * 4) if keys else 0))


@pytest.mark.parametrize("k,rows", [(8, 64), (12, 128), (16, 256)])
def test_plan_segment_length_follows_the_expected_wave_count(lib, k, rows):
    # 2 requests x 8 KV heads, lists of ~200 rows (N / C): the longest segment
    # length for which 16 groups x 4k lists give >= 2048 segments
    d = B.IvfDesc(2, 6400, 8, 32, 128, 32, 1, B.TSA_BF16)
    assert B.workspace_bytes(B.OP_SPARSE_DECODE, d, k) == _ivf_ws(2, 6400, 8, 32, 32, k, rows, keys=True)


def test_plan_segment_length_at_the_benchmark_shapes(lib):
    big = B.IvfDesc(64, 32768, 8, 32, 128, 256, 1, B.TSA_BF16)
    assert B.workspace_bytes(B.OP_SPARSE_DECODE, big, 16) == _ivf_ws(64, 32768, 8, 32, 256, 16, 256, keys=True)
    one = B.IvfDesc(1, 100_000, 8, 32, 128, 1000, 0, B.TSA_BF16)
    assert B.workspace_bytes(B.OP_SPARSE_DECODE, one, 10) == _ivf_ws(1, 100_000, 8, 32, 1000, 10, 32, keys=True)
