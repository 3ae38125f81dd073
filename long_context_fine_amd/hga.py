"""Python binding of libhga.so (the C ABI in include/hga.h).

Argument marshalling only: every function checks tensor shapes, dtypes and
devices, then hands raw pointers and the current HIP stream to the library.
All computation happens in the library's HIP kernels; there is no fallback.
If libhga.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhga.so")

HGA_OK, HGA_ERR_INVALID_ARG, HGA_ERR_UNSUPPORTED, HGA_ERR_WORKSPACE, HGA_ERR_HIP = range(5)
HGA_F32, HGA_BF16 = 0, 1
HGA_HIST_DEVICE, HGA_HIST_HOST_PINNED = 0, 1
HGA_OP_ROUTE, HGA_OP_ATTN_FWD, HGA_OP_ATTN_BWD, HGA_OP_ROUTE_CACHED = 0, 1, 2, 3

EXPORTS = ("hga_build_summaries", "hga_route", "hga_attn_fwd", "hga_attn_bwd",
           "hga_gather_groups", "hga_workspace_size", "hga_status_string",
           "hga_last_error", "hga_abi_version", "hga_set_kernel_events",
           "hga_gcache_bytes", "hga_gcache_reset", "hga_route_cached",
           "hga_decode_workspace_size", "hga_decode", "hga_route_noalloc", "hga_attn_bwd_staged",
           "hga_decode_twopass", "hga_summaries_to_bf16")

KERNELS = ("summaries", "route", "gather", "attn_fwd", "bwd_dq", "bwd_dkdv", "gcache", "decode")


class HGAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("group", ctypes.c_int32), ("block_q", ctypes.c_int32),
        ("top_k_chunks", ctypes.c_int32), ("top_k_groups", ctypes.c_int32),
        ("hist_len", ctypes.c_int64), ("seg_len", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("hist_loc", ctypes.c_int32), ("hist_stride", ctypes.c_int64),
        ("n_sink_chunks", ctypes.c_int32), ("local_window", ctypes.c_int32),
    ]

    @property
    def hist_rows(self) -> int:
        """Rows per KV head of the history buffers (hist_stride, else hist_len)."""
        return self.hist_stride or self.hist_len

    @property
    def n_blocks(self) -> int:
        return self.seg_len // self.block_q

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == HGA_BF16 else torch.float32


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhga.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m long_context_fine_amd.build` (needs hipcc)")
    L = ctypes.CDLL(_LIB_PATH)
    P, SZ, I32, I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    SP = ctypes.POINTER(Shape)
    sig = {
        "hga_build_summaries": [SP, P, I64, I64, P, P, P],
        "hga_route": [SP, P, P, P, P, P, P, SZ, P],
        "hga_route_noalloc": [SP, P, P, P, P, P, P],
        "hga_attn_fwd": [SP, P, P, P, P, P, P, P, P, P, SZ, P],
        "hga_attn_bwd": [SP, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "hga_attn_bwd_staged": [SP, P, P, SZ, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "hga_gather_groups": [SP, P, P, P, P, P, P],
        "hga_gcache_reset": [SP, P, I32, P],
        "hga_route_cached": [SP, P, P, P, P, I32, P, P, P, P, SZ, P],
        "hga_decode": [SP, I32, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "hga_decode_twopass": [SP, I32, I32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "hga_summaries_to_bf16": [P, P, ctypes.c_int64, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.hga_workspace_size.argtypes = [SP, I32]
    L.hga_workspace_size.restype = SZ
    L.hga_gcache_bytes.argtypes = [SP, I32]
    L.hga_gcache_bytes.restype = SZ
    L.hga_decode_workspace_size.argtypes = [SP, I32, I32]
    L.hga_decode_workspace_size.restype = SZ
    L.hga_status_string.argtypes = [I32]
    L.hga_status_string.restype = ctypes.c_char_p
    L.hga_last_error.argtypes = []
    L.hga_last_error.restype = ctypes.c_char_p
    L.hga_set_kernel_events.argtypes = [I32, P, P]
    L.hga_set_kernel_events.restype = ctypes.c_int
    L.hga_abi_version.argtypes = []
    L.hga_abi_version.restype = I32
    _lib = L
    return L


def make_shape(n_q_heads: int, n_kv_heads: int, head_dim: int, hist_len: int, seg_len: int,
               top_k_chunks: int, top_k_groups: int, dtype=torch.bfloat16,
               softmax_scale: float | None = None, hist_on_host: bool = False,
               hist_stride: int = 0, n_sink_chunks: int = 0, local_window: int = 0) -> Shape:
    return Shape(n_q_heads, n_kv_heads, head_dim, 64, 8, 64, top_k_chunks, top_k_groups,
                 hist_len, seg_len,
                 softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(head_dim),
                 HGA_BF16 if dtype == torch.bfloat16 else HGA_F32,
                 HGA_HIST_HOST_PINNED if hist_on_host else HGA_HIST_DEVICE, hist_stride,
                 n_sink_chunks, local_window)


def _check(status: int) -> None:
    if status != HGA_OK:
        L = lib()
        raise HGAError(status, f"{L.hga_status_string(status).decode()}: "
                               f"{L.hga_last_error().decode()}")


def _ptr(t: torch.Tensor | None, shape=None, dtype=None, name="", device=True) -> int | None:
    if t is None:
        return None
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    # an empty host tensor (no history) is never read; torch does not report
    # a zero-size allocation as pinned
    if not device and (t.is_cuda or (t.numel() > 0 and not t.is_pinned())):
        raise ValueError(f"{name}: must be a pinned host tensor")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def hga_set_kernel_events(kernel: int | str, ev_start=None, ev_stop=None) -> None:
    """Bracket every launch of `kernel` with two caller-owned HIP events
    (torch.cuda.Event objects or raw hipEvent_t handles); None turns it off."""
    kid = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)

    def h(e):
        if e is None:
            return None
        return e.cuda_event if hasattr(e, "cuda_event") else int(e)

    _check(lib().hga_set_kernel_events(kid, h(ev_start), h(ev_stop)))


def hga_workspace_size(shape: Shape, op: int) -> int:
    return int(lib().hga_workspace_size(ctypes.byref(shape), op))


def alloc_workspace(shape: Shape, op: int, device="cuda") -> torch.Tensor:
    n = hga_workspace_size(shape, op)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def hga_build_summaries(shape: Shape, k_hist, chunk_sum, group_sum, tok_begin=0, tok_end=None,
                        stream=None) -> None:
    H, kv, d = shape.hist_rows, shape.n_kv_heads, shape.head_dim
    tok_end = shape.hist_len if tok_end is None else tok_end
    host = shape.hist_loc == HGA_HIST_HOST_PINNED
    _check(lib().hga_build_summaries(
        ctypes.byref(shape), _ptr(k_hist, (kv, H, d), shape.torch_dtype, "k_hist", not host),
        tok_begin, tok_end,
        _ptr(chunk_sum, (kv, H // 64, d), torch.float32, "chunk_sum"),
        _ptr(group_sum, (kv, H // 8, d), torch.float32, "group_sum", group_sum.is_cuda),
        _stream(stream)))


def hga_route(shape: Shape, q, chunk_sum, group_sum, sel_chunks, sel_groups, ws=None,
              stream=None) -> None:
    H, kv, d, S = shape.hist_rows, shape.n_kv_heads, shape.head_dim, shape.seg_len
    if ws is None:
        ws = alloc_workspace(shape, HGA_OP_ROUTE, q.device)
    _check(lib().hga_route(
        ctypes.byref(shape), _ptr(q, (shape.n_q_heads, S, d), shape.torch_dtype, "q"),
        _ptr(chunk_sum, (kv, H // 64, d), torch.float32, "chunk_sum"),
        _ptr(group_sum, (kv, H // 8, d), torch.float32, "group_sum"),
        _ptr(sel_chunks, (shape.n_blocks, kv, shape.top_k_chunks), torch.int32, "sel_chunks"),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def hga_route_noalloc(shape: Shape, q, chunk_sum, group_sum, sel_chunks, sel_groups,
                      stream=None) -> None:
    """hga_route with the library's static per-device scratch as its workspace."""
    H, kv, d, S = shape.hist_rows, shape.n_kv_heads, shape.head_dim, shape.seg_len
    _check(lib().hga_route_noalloc(
        ctypes.byref(shape), _ptr(q, (shape.n_q_heads, S, d), shape.torch_dtype, "q"),
        _ptr(chunk_sum, (kv, H // 64, d), torch.float32, "chunk_sum"),
        _ptr(group_sum, (kv, H // 8, d), torch.float32, "group_sum"),
        _ptr(sel_chunks, (shape.n_blocks, kv, shape.top_k_chunks), torch.int32, "sel_chunks"),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _stream(stream)))


def hga_attn_fwd(shape: Shape, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse, ws=None,
                 stream=None) -> None:
    H, kv, d, S, nq = shape.hist_rows, shape.n_kv_heads, shape.head_dim, shape.seg_len, shape.n_q_heads
    dt = shape.torch_dtype
    host = shape.hist_loc == HGA_HIST_HOST_PINNED
    if ws is None and hga_workspace_size(shape, HGA_OP_ATTN_FWD) > 0:
        ws = alloc_workspace(shape, HGA_OP_ATTN_FWD, q.device)
    _check(lib().hga_attn_fwd(
        ctypes.byref(shape), _ptr(q, (nq, S, d), dt, "q"),
        _ptr(k_hist, (kv, H, d), dt, "k_hist", not host),
        _ptr(v_hist, (kv, H, d), dt, "v_hist", not host),
        _ptr(k_seg, (kv, S, d), dt, "k_seg"), _ptr(v_seg, (kv, S, d), dt, "v_seg"),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _ptr(o, (nq, S, d), dt, "o"), _ptr(lse, (nq, S), torch.float32, "lse"),
        None if ws is None else ws.data_ptr(),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def hga_attn_bwd(shape: Shape, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse, d_o,
                 dq, dk_seg, dv_seg, ws=None, stream=None) -> None:
    H, kv, d, S, nq = shape.hist_rows, shape.n_kv_heads, shape.head_dim, shape.seg_len, shape.n_q_heads
    dt = shape.torch_dtype
    host = shape.hist_loc == HGA_HIST_HOST_PINNED
    if ws is None:
        ws = alloc_workspace(shape, HGA_OP_ATTN_BWD, q.device)
    _check(lib().hga_attn_bwd(
        ctypes.byref(shape), _ptr(q, (nq, S, d), dt, "q"),
        _ptr(k_hist, (kv, H, d), dt, "k_hist", not host),
        _ptr(v_hist, (kv, H, d), dt, "v_hist", not host),
        _ptr(k_seg, (kv, S, d), dt, "k_seg"), _ptr(v_seg, (kv, S, d), dt, "v_seg"),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _ptr(o, (nq, S, d), dt, "o"), _ptr(lse, (nq, S), torch.float32, "lse"),
        _ptr(d_o, (nq, S, d), dt, "d_o"), _ptr(dq, (nq, S, d), dt, "dq"),
        _ptr(dk_seg, (kv, S, d), dt, "dk_seg"), _ptr(dv_seg, (kv, S, d), dt, "dv_seg"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def hga_attn_bwd_staged(shape: Shape, q, fwd_ws, k_seg, v_seg, sel_groups, o, lse, d_o,
                        dq, dk_seg, dv_seg, ws=None, stream=None) -> None:
    """hga_attn_bwd for pinned-host history, reading the routed rows that the
    forward left in its workspace `fwd_ws` (same shape and selections)."""
    kv, d, S, nq = shape.n_kv_heads, shape.head_dim, shape.seg_len, shape.n_q_heads
    dt = shape.torch_dtype
    if ws is None:
        ws = alloc_workspace(shape, HGA_OP_ATTN_BWD, q.device)
    _check(lib().hga_attn_bwd_staged(
        ctypes.byref(shape), _ptr(q, (nq, S, d), dt, "q"),
        _ptr(fwd_ws, None, None, "fwd_ws"),
        0 if fwd_ws is None else fwd_ws.numel() * fwd_ws.element_size(),
        _ptr(k_seg, (kv, S, d), dt, "k_seg"), _ptr(v_seg, (kv, S, d), dt, "v_seg"),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _ptr(o, (nq, S, d), dt, "o"), _ptr(lse, (nq, S), torch.float32, "lse"),
        _ptr(d_o, (nq, S, d), dt, "d_o"), _ptr(dq, (nq, S, d), dt, "dq"),
        _ptr(dk_seg, (kv, S, d), dt, "dk_seg"), _ptr(dv_seg, (kv, S, d), dt, "dv_seg"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def hga_gather_groups(shape: Shape, k_hist, v_hist, sel_groups, k_out, v_out, stream=None) -> None:
    H, kv, d = shape.hist_rows, shape.n_kv_heads, shape.head_dim
    dt = shape.torch_dtype
    host = shape.hist_loc == HGA_HIST_HOST_PINNED
    out_shape = (shape.n_blocks, kv, shape.top_k_groups * 8, d)
    _check(lib().hga_gather_groups(
        ctypes.byref(shape), _ptr(k_hist, (kv, H, d), dt, "k_hist", not host),
        _ptr(v_hist, (kv, H, d), dt, "v_hist", not host),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _ptr(k_out, out_shape, dt, "k_out"), _ptr(v_out, out_shape, dt, "v_out"), _stream(stream)))


def hga_gcache_bytes(shape: Shape, n_slots: int) -> int:
    return int(lib().hga_gcache_bytes(ctypes.byref(shape), n_slots))


def hga_gcache_reset(shape: Shape, cache, n_slots: int, stream=None) -> None:
    _check(lib().hga_gcache_reset(ctypes.byref(shape), _ptr(cache, name="cache"), n_slots,
                                  _stream(stream)))


def hga_route_cached(shape: Shape, q, chunk_sum, group_sum_host, cache, n_slots: int, sel_chunks,
                     sel_groups, stats=None, ws=None, stream=None) -> None:
    H, kv, d, S = shape.hist_rows, shape.n_kv_heads, shape.head_dim, shape.seg_len
    if ws is None:
        ws = alloc_workspace(shape, HGA_OP_ROUTE_CACHED, q.device)
    _check(lib().hga_route_cached(
        ctypes.byref(shape), _ptr(q, (shape.n_q_heads, S, d), shape.torch_dtype, "q"),
        _ptr(chunk_sum, (kv, H // 64, d), torch.float32, "chunk_sum"),
        _ptr(group_sum_host, (kv, H // 8, d), torch.float32, "group_sum_host", False),
        _ptr(cache, name="cache"), n_slots,
        _ptr(sel_chunks, (shape.n_blocks, kv, shape.top_k_chunks), torch.int32, "sel_chunks"),
        _ptr(sel_groups, (shape.n_blocks, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _ptr(stats, (kv, 2), torch.int32, "stats"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def hga_decode_workspace_size(shape: Shape, batch: int, n_new: int) -> int:
    return int(lib().hga_decode_workspace_size(ctypes.byref(shape), batch, n_new))


def _decode_call(entry, shape: Shape, q, k_hist, v_hist, chunk_sum, chunk_sum_bf16, group_sum, k_tail,
                 v_tail, hist_lens, tail_lens, sel_chunks, sel_groups, o, lse, ws, stream) -> None:
    B, nq, n_new, d = q.shape
    kv, P, T, dt = shape.n_kv_heads, shape.hist_rows, shape.seg_len, shape.torch_dtype
    if ws is None:
        n = hga_decode_workspace_size(shape, B, n_new)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    lo = () if chunk_sum_bf16 is False else (
        _ptr(chunk_sum_bf16, (B, kv, P // 64, d), torch.bfloat16, "chunk_sum_bf16"),)
    _check(entry(
        ctypes.byref(shape), B, n_new, _ptr(q, (B, shape.n_q_heads, n_new, d), dt, "q"),
        _ptr(k_hist, (B, kv, P, d), dt, "k_hist", shape.hist_loc != HGA_HIST_HOST_PINNED),
        _ptr(v_hist, (B, kv, P, d), dt, "v_hist", shape.hist_loc != HGA_HIST_HOST_PINNED),
        _ptr(chunk_sum, (B, kv, P // 64, d), torch.float32, "chunk_sum"), *lo,
        _ptr(group_sum, (B, kv, P // 8, d), torch.float32, "group_sum"),
        _ptr(k_tail, (B, kv, T, d), dt, "k_tail"), _ptr(v_tail, (B, kv, T, d), dt, "v_tail"),
        _ptr(hist_lens, (B,), torch.int32, "hist_lens"), _ptr(tail_lens, (B,), torch.int32, "tail_lens"),
        _ptr(sel_chunks, (B, kv, shape.top_k_chunks), torch.int32, "sel_chunks"),
        _ptr(sel_groups, (B, kv, shape.top_k_groups), torch.int32, "sel_groups"),
        _ptr(o, (B, nq, n_new, d), dt, "o"), _ptr(lse, (B, nq, n_new), torch.float32, "lse"),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def hga_decode(shape: Shape, q, k_hist, v_hist, chunk_sum, group_sum, k_tail, v_tail, hist_lens,
               tail_lens, sel_chunks, sel_groups, o, lse, ws=None, stream=None) -> None:
    """One decode step for a batch (layouts of include/hga.h: q [B][n_q][n_new][d],
    history [B][n_kv][P][d], open segment [B][n_kv][T][d], lengths int32 [B] on the GPU)."""
    _decode_call(lib().hga_decode, shape, q, k_hist, v_hist, chunk_sum, False, group_sum, k_tail, v_tail,
                 hist_lens, tail_lens, sel_chunks, sel_groups, o, lse, ws, stream)


def hga_decode_twopass(shape: Shape, q, k_hist, v_hist, chunk_sum, chunk_sum_bf16, group_sum, k_tail,
                       v_tail, hist_lens, tail_lens, sel_chunks, sel_groups, o, lse, ws=None,
                       stream=None) -> None:
    """hga_decode with the two-pass chunk route; chunk_sum_bf16 (torch.bfloat16, the
    layout of chunk_sum) holds hga_summaries_to_bf16 of chunk_sum."""
    _decode_call(lib().hga_decode_twopass, shape, q, k_hist, v_hist, chunk_sum, chunk_sum_bf16, group_sum,
                 k_tail, v_tail, hist_lens, tail_lens, sel_chunks, sel_groups, o, lse, ws, stream)


def hga_summaries_to_bf16(src, dst, stream=None) -> None:
    """dst (torch.bfloat16) = src (torch.float32, same shape) rounded to nearest even."""
    _check(lib().hga_summaries_to_bf16(_ptr(src, tuple(src.shape), torch.float32, "src"),
                                       _ptr(dst, tuple(src.shape), torch.bfloat16, "dst"),
                                       src.numel(), _stream(stream)))


def summaries_to_bf16(src):
    """Allocate and fill the bf16 copies of fp32 summaries."""
    dst = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    hga_summaries_to_bf16(src, dst)
    return dst


def decode(shape: Shape, q, k_hist, v_hist, chunk_sum, group_sum, k_tail, v_tail, hist_lens, tail_lens,
           ws=None, chunk_sum_bf16=None):
    """Allocate the outputs and run hga_decode, or hga_decode_twopass when
    chunk_sum_bf16 is given: (o, lse, sel_chunks, sel_groups)."""
    B, nq, n_new, _ = q.shape
    dev = q.device
    sc = torch.empty((B, shape.n_kv_heads, shape.top_k_chunks), dtype=torch.int32, device=dev)
    sg = torch.empty((B, shape.n_kv_heads, shape.top_k_groups), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, nq, n_new), dtype=torch.float32, device=dev)
    if chunk_sum_bf16 is None:
        hga_decode(shape, q, k_hist, v_hist, chunk_sum, group_sum, k_tail, v_tail, hist_lens, tail_lens,
                   sc, sg, o, lse, ws)
    else:
        hga_decode_twopass(shape, q, k_hist, v_hist, chunk_sum, chunk_sum_bf16, group_sum, k_tail, v_tail,
                           hist_lens, tail_lens, sc, sg, o, lse, ws)
    return o, lse, sc, sg


class GroupSummaryCache:
    """One device buffer holding the group-summary cache of a history with the
    shape's KV heads, head_dim and row capacity (hist_stride or hist_len)."""

    def __init__(self, shape: Shape, n_slots: int, device="cuda"):
        self.n_slots, self.n_kv, self.d = n_slots, shape.n_kv_heads, shape.head_dim
        self.chunk_rows = shape.hist_rows // 64
        n = hga_gcache_bytes(shape, n_slots)
        if n == 0:
            _check(HGA_ERR_INVALID_ARG)
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        self.reset(shape)

    def reset(self, shape: Shape, stream=None) -> None:
        hga_gcache_reset(shape, self.buf, self.n_slots, stream)

    def route(self, shape: Shape, q, chunk_sum, group_sum_host, sel_chunks, sel_groups, stats=None,
              ws=None, stream=None) -> None:
        hga_route_cached(shape, q, chunk_sum, group_sum_host, self.buf, self.n_slots, sel_chunks,
                         sel_groups, stats, ws, stream)

    def tables(self):
        """Views of the buffer's parts (layout of include/hga.h): slot_of_chunk
        [n_kv][rows/64], chunk_of_slot [n_kv][n_slots], hand [n_kv], data
        [n_kv][n_slots][8][d]."""
        def a256(x):
            return (x + 255) // 256 * 256
        kv, ns = self.n_kv, self.n_slots
        o1 = a256(4 * kv * self.chunk_rows)
        o2 = o1 + a256(4 * kv * ns)
        o3 = o2 + a256(4 * kv)
        b = self.buf
        return (b[:4 * kv * self.chunk_rows].view(torch.int32).view(kv, self.chunk_rows),
                b[o1:o1 + 4 * kv * ns].view(torch.int32).view(kv, ns),
                b[o2:o2 + 4 * kv].view(torch.int32),
                b[o3:o3 + 4 * kv * ns * 8 * self.d].view(torch.float32).view(kv, ns, 8, self.d))


# ---------------------------------------------------------------------------
# conveniences built from the calls above (allocation + call order only)
# ---------------------------------------------------------------------------
def summaries(shape: Shape, k_hist, device="cuda"):
    """Allocate and build the chunk / group summaries of the whole history."""
    H, kv, d = shape.hist_rows, shape.n_kv_heads, shape.head_dim
    C = torch.empty((kv, H // 64, d), dtype=torch.float32, device=device)
    G = torch.empty((kv, H // 8, d), dtype=torch.float32, device=device)
    hga_build_summaries(shape, k_hist, C, G)
    return C, G


def route(shape: Shape, q, chunk_sum, group_sum, ws=None):
    """Allocate the selection lists and route every query block."""
    dev = q.device
    sc = torch.empty((shape.n_blocks, shape.n_kv_heads, shape.top_k_chunks), dtype=torch.int32, device=dev)
    sg = torch.empty((shape.n_blocks, shape.n_kv_heads, shape.top_k_groups), dtype=torch.int32, device=dev)
    hga_route(shape, q, chunk_sum, group_sum, sc, sg, ws)
    return sc, sg


def attn_fwd(shape: Shape, q, k_hist, v_hist, k_seg, v_seg, sel_groups, ws=None):
    o = torch.empty_like(q)
    lse = torch.empty((shape.n_q_heads, shape.seg_len), dtype=torch.float32, device=q.device)
    hga_attn_fwd(shape, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse, ws)
    return o, lse


def attn_bwd(shape: Shape, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse, d_o, ws=None):
    dq = torch.empty_like(q)
    dk = torch.empty_like(k_seg)
    dv = torch.empty_like(v_seg)
    hga_attn_bwd(shape, q, k_hist, v_hist, k_seg, v_seg, sel_groups, o, lse, d_o, dq, dk, dv, ws)
    return dq, dk, dv


class HGAAttention(torch.autograd.Function):
    """Routed exact-token attention as an autograd op: forward routes with the
    given summaries and attends; backward returns grads for q, k_seg, v_seg
    only (history, summaries and routing get none)."""

    @staticmethod
    def forward(ctx, shape, q, k_seg, v_seg, k_hist, v_hist, chunk_sum, group_sum):
        _, sel_g = route(shape, q, chunk_sum, group_sum)
        ws_f = None
        if shape.hist_loc == HGA_HIST_HOST_PINNED and shape.hist_len > 0:
            # kept for the backward: it holds the routed rows the forward
            # brought over the host link
            ws_f = alloc_workspace(shape, HGA_OP_ATTN_FWD, q.device)
        o, lse = attn_fwd(shape, q, k_hist, v_hist, k_seg, v_seg, sel_g, ws_f)
        ctx.shape = shape
        ctx.ws_f = ws_f
        ctx.save_for_backward(q, k_seg, v_seg, k_hist, v_hist, sel_g, o, lse)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k_seg, v_seg, k_hist, v_hist, sel_g, o, lse = ctx.saved_tensors
        d_o = d_o.contiguous()
        if ctx.ws_f is not None:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k_seg), torch.empty_like(v_seg)
            hga_attn_bwd_staged(ctx.shape, q, ctx.ws_f, k_seg, v_seg, sel_g, o, lse, d_o, dq, dk, dv)
            ctx.ws_f = None
        else:
            dq, dk, dv = attn_bwd(ctx.shape, q, k_hist, v_hist, k_seg, v_seg, sel_g, o, lse, d_o)
        return None, dq, dk, dv, None, None, None, None
