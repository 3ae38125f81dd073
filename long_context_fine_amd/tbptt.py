"""Segment-wise (truncated-BPTT) driver for one HGA attention layer.

The pages train over a long sequence segment by segment: only the active
segment is differentiable, and once a segment closes its keys and values are
detached and join the history, whose chunk and group summaries are built once
(gist.science Technical Summary §2.2, "Segment-wise Backward and Tiered
Storage"; pith.science review, Figure 2 caption). `LayerHistory` keeps that
state for one layer and sequences the library's calls around it:

    o, lse = h.forward(q, k_seg, v_seg)          # route over the history, attend
    dq, dk, dv = h.backward(q, k_seg, v_seg, o, lse, d_o)
    h.close_segment(k_seg, v_seg)                # detach: append K/V, summarise

With `group_cache_slots` > 0 the group summaries live in page-locked host
memory and routing reads them through an HBM cache of that many chunk slots
per KV head (`hga_route_cached`; per-call hits and misses in `cache_stats`).

The first `n_sink_chunks` history chunks form a fixed sink attended by every
query, and `local_window` limits the segment keys each query sees (0: the
whole causal segment).

History K/V live in one buffer per tensor with room for `max_hist` tokens per
KV head ([n_kv][max_hist][d], device memory or page-locked host memory), and the
summaries in [n_kv][max_hist/64][d] / [n_kv][max_hist/8][d]; the library reads
them through `hist_stride`, so the history grows in place without repacking.
Every computation runs in the library's kernels; this module only allocates,
copies segments into the history and orders the calls. With history in host
memory the forward gathers routed groups over the host link into its
workspace, and the backward reads them there (`hga_attn_bwd_staged`), so each
segment moves its routed groups over the link once. `backward` must therefore
follow the `forward` of the same segment.
"""
from __future__ import annotations

import torch

from . import hga


class LayerHistory:
    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int, seg_len: int,
                 max_hist: int, top_k_chunks: int, top_k_groups: int,
                 dtype=torch.bfloat16, softmax_scale: float | None = None,
                 hist_on_host: bool = False, device="cuda", n_sink_chunks: int = 0,
                 local_window: int = 0, group_cache_slots: int = 0):
        if max_hist <= 0 or max_hist % 64 or seg_len % 64:
            raise ValueError("max_hist must be a positive multiple of 64 and seg_len a multiple of 64")
        self.n_q, self.n_kv, self.d, self.seg_len = n_q_heads, n_kv_heads, head_dim, seg_len
        self.max_hist, self.k_c, self.k_g = max_hist, top_k_chunks, top_k_groups
        self.dtype, self.scale, self.on_host = dtype, softmax_scale, hist_on_host
        self.n_sink, self.window = n_sink_chunks, local_window
        self.device = torch.device(device)
        kv = (n_kv_heads, max_hist, head_dim)
        if hist_on_host:
            self.k_hist = torch.empty(kv, dtype=dtype, pin_memory=True)
            self.v_hist = torch.empty(kv, dtype=dtype, pin_memory=True)
        else:
            self.k_hist = torch.empty(kv, dtype=dtype, device=self.device)
            self.v_hist = torch.empty(kv, dtype=dtype, device=self.device)
        self.chunk_sum = torch.zeros((n_kv_heads, max_hist // 64, head_dim), dtype=torch.float32,
                                     device=self.device)
        if group_cache_slots:
            # group summaries in page-locked host memory behind an HBM cache
            self.group_sum = torch.zeros((n_kv_heads, max_hist // 8, head_dim), dtype=torch.float32,
                                         pin_memory=True)
        else:
            self.group_sum = torch.zeros((n_kv_heads, max_hist // 8, head_dim), dtype=torch.float32,
                                         device=self.device)
        self.hist_len = 0
        n_blocks = seg_len // 64
        self.sel_chunks = torch.empty((n_blocks, n_kv_heads, top_k_chunks), dtype=torch.int32,
                                      device=self.device)
        self.sel_groups = torch.empty((n_blocks, n_kv_heads, top_k_groups), dtype=torch.int32,
                                      device=self.device)
        full = self.shape(max_hist)           # workspaces sized for the full history
        self.gcache = hga.GroupSummaryCache(full, group_cache_slots, self.device) if group_cache_slots else None
        self.cache_stats = torch.zeros((n_kv_heads, 2), dtype=torch.int32, device=self.device)
        self.ws_route = hga.alloc_workspace(
            full, hga.HGA_OP_ROUTE_CACHED if group_cache_slots else hga.HGA_OP_ROUTE, self.device)
        self.ws_fwd = hga.alloc_workspace(full, hga.HGA_OP_ATTN_FWD, self.device)
        # the backward's own workspace (with host history it reads the routed
        # rows from ws_fwd, so it needs no staging of its own)
        self.ws_bwd = hga.alloc_workspace(self.shape(max_hist, hist_on_host=False), hga.HGA_OP_ATTN_BWD,
                                          self.device)

    def shape(self, hist_len: int | None = None, hist_on_host: bool | None = None) -> hga.Shape:
        return hga.make_shape(self.n_q, self.n_kv, self.d,
                              self.hist_len if hist_len is None else hist_len, self.seg_len,
                              self.k_c, self.k_g, self.dtype, self.scale,
                              self.on_host if hist_on_host is None else hist_on_host,
                              hist_stride=self.max_hist, n_sink_chunks=self.n_sink,
                              local_window=self.window)

    def forward(self, q, k_seg, v_seg):
        """Route the segment's query blocks over the current history and run
        exact-token attention; returns (o, lse). The selections stay in
        `sel_groups` for the backward."""
        s = self.shape()
        if self.gcache is not None:
            self.gcache.route(s, q, self.chunk_sum, self.group_sum, self.sel_chunks, self.sel_groups,
                              self.cache_stats, self.ws_route)
        else:
            hga.hga_route(s, q, self.chunk_sum, self.group_sum, self.sel_chunks, self.sel_groups,
                          self.ws_route)
        o = torch.empty_like(q)
        lse = torch.empty((self.n_q, self.seg_len), dtype=torch.float32, device=q.device)
        hga.hga_attn_fwd(s, q, self.k_hist, self.v_hist, k_seg, v_seg, self.sel_groups, o, lse,
                         self.ws_fwd)
        return o, lse

    def backward(self, q, k_seg, v_seg, o, lse, d_o):
        """Gradients of sum(o * d_o) for the segment: (dq, dk_seg, dv_seg); the
        history is detached and receives none."""
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k_seg), torch.empty_like(v_seg)
        if self.on_host:
            # the forward of this segment left every block's routed rows in
            # its workspace: no second trip over the host link
            hga.hga_attn_bwd_staged(self.shape(), q, self.ws_fwd, k_seg, v_seg, self.sel_groups,
                                    o, lse, d_o, dq, dk, dv, self.ws_bwd)
        else:
            hga.hga_attn_bwd(self.shape(), q, self.k_hist, self.v_hist, k_seg, v_seg, self.sel_groups,
                             o, lse, d_o, dq, dk, dv, self.ws_bwd)
        return dq, dk, dv

    def close_segment(self, k_seg, v_seg) -> None:
        """Detach the segment: copy its K/V into the history (a device copy, or
        device-to-host into the page-locked buffer) and build the summaries of
        its chunks, all on the current stream."""
        H, S = self.hist_len, self.seg_len
        if H + S > self.max_hist:
            raise ValueError(f"history full: {H} + {S} tokens exceed max_hist {self.max_hist}")
        self.k_hist[:, H:H + S].copy_(k_seg.detach(), non_blocking=True)
        self.v_hist[:, H:H + S].copy_(v_seg.detach(), non_blocking=True)
        hga.hga_build_summaries(self.shape(H + S), self.k_hist, self.chunk_sum, self.group_sum,
                                H, H + S)
        self.hist_len = H + S
