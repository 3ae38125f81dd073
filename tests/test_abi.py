"""The C-ABI library loads, exports every symbol include/hga.h declares, and
rejects bad arguments on the host with status codes (no GPU needed: every
path exercised here returns before anything is launched)."""
import ctypes
import os
import re

import pytest

from long_context_fine_amd import hga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "hga.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hga_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hga._LIB_PATH):
        from long_context_fine_amd import build
        build.build()
    return hga.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert set(names) == set(hga.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert L.hga_abi_version() == 4
    assert L.hga_status_string(0) == b"HGA_OK"
    assert L.hga_status_string(3) == b"HGA_ERR_WORKSPACE"
    assert L.hga_status_string(99) == b"HGA_ERR_UNKNOWN"


def _shape(**kw):
    s = hga.make_shape(32, 8, 128, 14336, 2048, 16, 32)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


FAKE = 0x10000  # never dereferenced: validation fails first


@pytest.mark.parametrize("field,value,status", [
    ("n_q_heads", 0, hga.HGA_ERR_INVALID_ARG),
    ("n_q_heads", 30, hga.HGA_ERR_INVALID_ARG),          # not a multiple of n_kv
    ("head_dim", 96, hga.HGA_ERR_UNSUPPORTED),
    ("head_dim", -1, hga.HGA_ERR_INVALID_ARG),
    ("chunk", 32, hga.HGA_ERR_UNSUPPORTED),
    ("group", 16, hga.HGA_ERR_UNSUPPORTED),
    ("block_q", 128, hga.HGA_ERR_UNSUPPORTED),
    ("top_k_chunks", 0, hga.HGA_ERR_INVALID_ARG),
    ("top_k_groups", 513, hga.HGA_ERR_UNSUPPORTED),
    ("hist_len", 100, hga.HGA_ERR_INVALID_ARG),          # H % 64 != 0
    ("hist_len", -64, hga.HGA_ERR_INVALID_ARG),
    ("seg_len", 100, hga.HGA_ERR_INVALID_ARG),           # S % 64 != 0
    ("seg_len", 0, hga.HGA_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), hga.HGA_ERR_INVALID_ARG),
    ("softmax_scale", 0.0, hga.HGA_ERR_INVALID_ARG),
    ("dtype", 7, hga.HGA_ERR_INVALID_ARG),
    ("hist_loc", 5, hga.HGA_ERR_INVALID_ARG),
    ("hist_stride", 14336 - 64, hga.HGA_ERR_INVALID_ARG),   # below hist_len
    ("hist_stride", 14336 + 8, hga.HGA_ERR_INVALID_ARG),    # not a multiple of 64
    ("hist_stride", -64, hga.HGA_ERR_INVALID_ARG),
    ("n_sink_chunks", -1, hga.HGA_ERR_INVALID_ARG),
    ("local_window", -5, hga.HGA_ERR_INVALID_ARG),
])
def test_invalid_shapes_are_rejected(L, field, value, status):
    s = _shape(**{field: value})
    st = L.hga_route(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status
    assert L.hga_last_error() != b""
    assert L.hga_workspace_size(ctypes.byref(s), hga.HGA_OP_ROUTE) == 0


def test_history_stride_is_accepted(L):
    """A history buffer with room to grow: stride above hist_len is valid and
    does not change any workspace size."""
    s = _shape()
    grown = _shape(hist_stride=14336 + 2048)
    for op in (hga.HGA_OP_ROUTE, hga.HGA_OP_ATTN_FWD, hga.HGA_OP_ATTN_BWD):
        assert L.hga_workspace_size(ctypes.byref(grown), op) == L.hga_workspace_size(ctypes.byref(s), op)
    assert grown.hist_rows == 14336 + 2048 and s.hist_rows == 14336


def test_null_shape_and_null_pointers(L):
    assert L.hga_attn_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) \
        == hga.HGA_ERR_INVALID_ARG
    s = _shape()
    assert L.hga_route(ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) \
        == hga.HGA_ERR_INVALID_ARG
    assert L.hga_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 0,
                          None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_attn_bwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                          FAKE, None, FAKE, FAKE, 1 << 30, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_gather_groups(ctypes.byref(s), FAKE, FAKE, None, FAKE, FAKE, None) \
        == hga.HGA_ERR_INVALID_ARG


def test_workspace_sizes_and_undersized_workspace(L):
    s = _shape()
    n_route = L.hga_workspace_size(ctypes.byref(s), hga.HGA_OP_ROUTE)
    # chunk scores [32][8][224] f32
    assert n_route == 32 * 8 * 224 * 4
    assert L.hga_workspace_size(ctypes.byref(s), hga.HGA_OP_ATTN_FWD) == 0
    # Dvec and LSE*log2(e) [32][2048] f32 each + dK/dV partials of the 2 head groups
    # [2][2][8][2048][128] f32
    assert L.hga_workspace_size(ctypes.byref(s), hga.HGA_OP_ATTN_BWD) == \
        2 * 32 * 2048 * 4 + 2 * 2 * 8 * 2048 * 128 * 4
    assert L.hga_workspace_size(ctypes.byref(s), 9) == 0
    st = L.hga_route(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n_route - 1, None)
    assert st == hga.HGA_ERR_WORKSPACE
    st = L.hga_route(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, n_route, None)
    assert st == hga.HGA_ERR_WORKSPACE                    # misaligned
    st = L.hga_attn_bwd(ctypes.byref(s), *([FAKE] * 13), 16, None)
    assert st == hga.HGA_ERR_WORKSPACE
    host = _shape(hist_loc=hga.HGA_HIST_HOST_PINNED)
    n_fwd = L.hga_workspace_size(ctypes.byref(host), hga.HGA_OP_ATTN_FWD)
    assert n_fwd == 2 * (32 * 8 * 32 * 8 * 128 * 2)       # {K,V} rows of all 32 blocks
    st = L.hga_attn_fwd(ctypes.byref(host), *([FAKE] * 8), FAKE, n_fwd - 1, None)
    assert st == hga.HGA_ERR_WORKSPACE
    # backward over host history: + {K, V} routed rows of all 32 blocks,
    # [32][8][32*8][128] bf16 each, copied over the host link before dQ
    n_bwd_dev = L.hga_workspace_size(ctypes.byref(s), hga.HGA_OP_ATTN_BWD)
    n_bwd_host = L.hga_workspace_size(ctypes.byref(host), hga.HGA_OP_ATTN_BWD)
    assert n_bwd_host == n_bwd_dev + 2 * (32 * 8 * 256 * 128 * 2)
    st = L.hga_attn_bwd(ctypes.byref(host), *([FAKE] * 13), n_bwd_host - 1, None)
    assert st == hga.HGA_ERR_WORKSPACE
    # the staged backward reads the forward's workspace: it needs a pinned-host
    # shape, the forward's full workspace and only the kernels' own workspace
    staged = lambda sh, fwd_bytes, bwd_bytes: L.hga_attn_bwd_staged(  # noqa: E731
        ctypes.byref(sh), FAKE, FAKE, fwd_bytes, *([FAKE] * 9), FAKE, bwd_bytes, None)
    assert staged(s, n_fwd, n_bwd_dev) == hga.HGA_ERR_INVALID_ARG          # device history
    assert staged(host, n_fwd - 1, n_bwd_dev) == hga.HGA_ERR_WORKSPACE
    assert staged(host, n_fwd, n_bwd_dev - 1) == hga.HGA_ERR_WORKSPACE
    assert L.hga_attn_bwd_staged(ctypes.byref(host), FAKE, None, n_fwd, *([FAKE] * 9), FAKE, n_bwd_dev,
                                 None) == hga.HGA_ERR_WORKSPACE
    assert L.hga_attn_bwd_staged(ctypes.byref(host), FAKE, FAKE + 8, n_fwd, *([FAKE] * 9), FAKE, n_bwd_dev,
                                 None) == hga.HGA_ERR_WORKSPACE            # misaligned
    assert L.hga_attn_bwd_staged(ctypes.byref(host), FAKE, FAKE, n_fwd, *([FAKE] * 8), None, FAKE, n_bwd_dev,
                                 None) == hga.HGA_ERR_INVALID_ARG          # dv_seg NULL
    # sink rows staged per call: + {K, V} x [8][2*64][128] bf16; the sink is
    # clamped to the history (224 chunks)
    sink = _shape(hist_loc=hga.HGA_HIST_HOST_PINNED, n_sink_chunks=2, local_window=1024)
    assert L.hga_workspace_size(ctypes.byref(sink), hga.HGA_OP_ATTN_FWD) == n_fwd + 2 * (8 * 128 * 128 * 2)
    huge = _shape(hist_loc=hga.HGA_HIST_HOST_PINNED, n_sink_chunks=1000)
    assert L.hga_workspace_size(ctypes.byref(huge), hga.HGA_OP_ATTN_FWD) == n_fwd + 2 * (8 * 14336 * 128 * 2)
    assert L.hga_workspace_size(ctypes.byref(sink), hga.HGA_OP_ATTN_BWD) == n_bwd_host + 2 * (8 * 128 * 128 * 2)
    # no history: nothing to copy
    empty = _shape(hist_loc=hga.HGA_HIST_HOST_PINNED, hist_len=0)
    assert L.hga_workspace_size(ctypes.byref(empty), hga.HGA_OP_ATTN_BWD) == n_bwd_dev
    # a device-resident sink or a window needs no workspace of its own
    dev = _shape(n_sink_chunks=4, local_window=512)
    for op in (hga.HGA_OP_ROUTE, hga.HGA_OP_ATTN_FWD, hga.HGA_OP_ATTN_BWD):
        assert L.hga_workspace_size(ctypes.byref(dev), op) == L.hga_workspace_size(ctypes.byref(s), op)


def test_group_summary_cache_sizes_and_checks(L):
    s = _shape()                                          # H = 14336: 224 chunks, 8 KV heads
    a = lambda x: (x + 255) // 256 * 256
    assert L.hga_gcache_bytes(ctypes.byref(s), 512) == \
        a(8 * 224 * 4) + a(8 * 512 * 4) + a(8 * 4) + 8 * 512 * 8 * 128 * 4
    assert L.hga_gcache_bytes(ctypes.byref(s), 0) == 0
    assert L.hga_gcache_bytes(ctypes.byref(s), 16385) == 0
    assert L.hga_workspace_size(ctypes.byref(s), hga.HGA_OP_ROUTE_CACHED) == \
        32 * 8 * 224 * 4 + 32 * 8 * 128 * 4                # chunk scores + block queries
    n_ws = 1 << 30
    # 32 blocks x 16 kept chunks need 512 slots
    st = L.hga_route_cached(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 511, FAKE, FAKE, None, FAKE, n_ws, None)
    assert st == hga.HGA_ERR_INVALID_ARG and b"511" in L.hga_last_error()
    st = L.hga_route_cached(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 512, FAKE, FAKE, None, FAKE, 16, None)
    assert st == hga.HGA_ERR_WORKSPACE
    st = L.hga_route_cached(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE + 8, 512, FAKE, FAKE, None, FAKE, n_ws,
                            None)
    assert st == hga.HGA_ERR_INVALID_ARG                  # misaligned cache
    long = _shape(seg_len=65536)                           # 1024 blocks x 16 chunks > 8192
    st = L.hga_route_cached(ctypes.byref(long), FAKE, FAKE, FAKE, FAKE, 16384, FAKE, FAKE, None, FAKE, n_ws,
                            None)
    assert st == hga.HGA_ERR_UNSUPPORTED
    huge = _shape(hist_len=131072 * 64 + 64)              # chunk ids beyond the dedupe bitmap
    st = L.hga_route_cached(ctypes.byref(huge), FAKE, FAKE, FAKE, FAKE, 512, FAKE, FAKE, None, FAKE, n_ws,
                            None)
    assert st == hga.HGA_ERR_UNSUPPORTED
    assert L.hga_route_cached(ctypes.byref(s), FAKE, FAKE, FAKE, None, 512, FAKE, FAKE, None, FAKE, n_ws,
                              None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_gcache_reset(ctypes.byref(s), None, 512, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_gcache_reset(ctypes.byref(s), FAKE, 0, None) == hga.HGA_ERR_INVALID_ARG


def test_summary_range_checks(L):
    s = _shape()
    assert L.hga_build_summaries(ctypes.byref(s), FAKE, 64, 32, FAKE, FAKE, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_build_summaries(ctypes.byref(s), FAKE, 0, 14336 + 64, FAKE, FAKE, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_build_summaries(ctypes.byref(s), FAKE, 0, 100, FAKE, FAKE, None) == hga.HGA_ERR_INVALID_ARG
    # summaries are written 16 bytes at a time: misaligned outputs are refused
    assert L.hga_build_summaries(ctypes.byref(s), FAKE, 0, 64, FAKE + 4, FAKE, None) == hga.HGA_ERR_INVALID_ARG
    assert b"16-byte aligned" in L.hga_last_error()
    assert L.hga_build_summaries(ctypes.byref(s), FAKE, 0, 64, FAKE, FAKE + 8, None) == hga.HGA_ERR_INVALID_ARG
    # an empty range is a no-op that touches nothing
    assert L.hga_build_summaries(ctypes.byref(s), None, 128, 128, None, None, None) == hga.HGA_OK
    assert L.hga_last_error() == b""


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hga, "_lib", None)
    monkeypatch.setattr(hga, "_LIB_PATH", str(tmp_path / "libhga.so"))
    with pytest.raises(RuntimeError, match="missing"):
        hga.lib()


def test_route_noalloc_rejects_shapes_beyond_its_scratch(L):
    # 1,024 query blocks x 8 KV heads x 4,160 chunks of scores: 136 MB > 16 MiB
    s = hga.make_shape(32, 8, 128, 4160 * 64, 65536, 16, 32)
    assert hga.hga_workspace_size(s, hga.HGA_OP_ROUTE) > 16 * 2 ** 20
    st = L.hga_route_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == hga.HGA_ERR_WORKSPACE
    assert b"static scratch" in L.hga_last_error()
    s = _shape(top_k_chunks=0)
    assert L.hga_route_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None) == hga.HGA_ERR_INVALID_ARG


def test_binding_host_tensors_must_be_pinned_unless_empty():
    """Host-side history tensors go through the pinned check, except an empty
    one (a history of zero tokens is never read)."""
    import torch
    assert hga._ptr(torch.empty(0, dtype=torch.bfloat16), name="k_hist", device=False) is not None
    with pytest.raises(ValueError, match="pinned host tensor"):
        hga._ptr(torch.empty(4, dtype=torch.bfloat16), name="k_hist", device=False)


def test_decode_arguments_and_workspace(L):
    """hga_decode's host checks: batch and n_new ranges, at most 16 query rows
    per KV head, workspace size (history in host memory adds the K and V
    copies of every (sequence, KV head)'s sink rows and routed groups)."""
    s = _shape()                                 # capacity 14,336, open segment 2,048
    n = L.hga_decode_workspace_size(ctypes.byref(s), 4, 1)
    assert n > 0 and n % 256 == 0
    assert L.hga_decode_workspace_size(ctypes.byref(s), 0, 1) == 0       # batch < 1
    assert L.hga_decode_workspace_size(ctypes.byref(s), 4, 0) == 0       # n_new < 1
    assert L.hga_decode_workspace_size(ctypes.byref(s), 4, 5) == 0       # 4 x 5 rows > 16
    host = _shape(hist_loc=hga.HGA_HIST_HOST_PINNED)
    # + {K, V} x [4 sequences][8 KV heads][32 groups x 8][128] bf16
    assert L.hga_decode_workspace_size(ctypes.byref(host), 4, 1) == n + 2 * (4 * 8 * 256 * 128 * 2)
    # with a 2-chunk sink the attention also has more keys; the copies add the
    # sink's 128 rows per (sequence, KV head)
    ns = L.hga_decode_workspace_size(ctypes.byref(_shape(n_sink_chunks=2)), 4, 1)
    sink = _shape(hist_loc=hga.HGA_HIST_HOST_PINNED, n_sink_chunks=2)
    assert L.hga_decode_workspace_size(ctypes.byref(sink), 4, 1) == ns + 2 * (4 * 8 * (128 + 256) * 128 * 2)
    dec = lambda sh, batch, n_new, ws, nbytes: L.hga_decode(  # noqa: E731
        ctypes.byref(sh), batch, n_new, *([FAKE] * 13), ws, nbytes, None)
    assert dec(s, 0, 1, FAKE, n) == hga.HGA_ERR_INVALID_ARG
    assert dec(s, 4, 2049, FAKE, n) == hga.HGA_ERR_INVALID_ARG            # n_new > seg_len
    assert dec(s, 4, 5, FAKE, n) == hga.HGA_ERR_UNSUPPORTED
    assert dec(s, 4, 1, FAKE, n - 1) == hga.HGA_ERR_WORKSPACE
    assert dec(s, 4, 1, FAKE + 8, n) == hga.HGA_ERR_WORKSPACE              # misaligned
    assert dec(s, 4, 1, None, n) == hga.HGA_ERR_WORKSPACE
    nh = L.hga_decode_workspace_size(ctypes.byref(host), 4, 1)
    assert dec(host, 4, 1, FAKE, nh - 1) == hga.HGA_ERR_WORKSPACE


def test_decode_twopass_and_bf16_copy_arguments(L):
    """hga_decode_twopass: hga_decode's checks plus a non-NULL, 16-byte aligned
    bf16 copy of the chunk summaries; hga_summaries_to_bf16: n a multiple of 8,
    aligned pointers. All rejected on the host before any launch."""
    s = _shape()
    n = L.hga_decode_workspace_size(ctypes.byref(s), 4, 1)
    dec2 = lambda sh, batch, n_new, lo, ws, nbytes: L.hga_decode_twopass(  # noqa: E731
        ctypes.byref(sh), batch, n_new, *([FAKE] * 4), lo, *([FAKE] * 9), ws, nbytes, None)
    assert dec2(s, 4, 1, None, FAKE, n) == hga.HGA_ERR_INVALID_ARG          # no bf16 copy
    assert dec2(s, 4, 1, FAKE + 2, FAKE, n) == hga.HGA_ERR_INVALID_ARG      # misaligned copy
    assert b"chunk_sum_bf16" in L.hga_last_error()
    assert dec2(s, 0, 1, FAKE, FAKE, n) == hga.HGA_ERR_INVALID_ARG          # the hga_decode checks follow
    assert dec2(s, 4, 5, FAKE, FAKE, n) == hga.HGA_ERR_UNSUPPORTED
    assert dec2(s, 4, 1, FAKE, FAKE, n - 1) == hga.HGA_ERR_WORKSPACE
    assert L.hga_summaries_to_bf16(None, None, 0, None) == hga.HGA_OK       # nothing to do
    assert L.hga_summaries_to_bf16(FAKE, FAKE, 12, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_summaries_to_bf16(FAKE, FAKE, -8, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_summaries_to_bf16(None, FAKE, 16, None) == hga.HGA_ERR_INVALID_ARG
    assert L.hga_summaries_to_bf16(FAKE, FAKE + 4, 16, None) == hga.HGA_ERR_INVALID_ARG
