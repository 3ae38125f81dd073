"""Segment-wise driver (long_context_fine_amd.tbptt) on the GPU: the history
grows in place (hist_stride), summaries are built incrementally per closed
segment, and every segment's routing, attention and gradients match the
oracle run on the history accumulated so far."""
import math

import numpy as np
import pytest
import torch

from long_context_fine_amd import hga, synth, tbptt
from oracle import hga_oracle as orc

pytestmark = pytest.mark.gpu

N_Q, N_KV, D, S, K_C, K_G, N_SEG = 8, 2, 128, 128, 3, 12, 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


def _sequence(seed):
    """Q, K, V, dO for N_SEG consecutive segments (bf16), from the shared
    generator: the workload's history+segment K/V span all segments."""
    w = synth.Workload("tbptt", N_Q, N_KV, D, (N_SEG - 1) * S, S, K_C, K_G, "bf16",
                       1.0 / math.sqrt(D), backward=True)
    inp = synth.make_inputs(w, seed, with_grad_out=True)
    k = torch.cat([inp["k_hist"], inp["k_seg"]], dim=1)
    v = torch.cat([inp["v_hist"], inp["v_seg"]], dim=1)
    g = torch.Generator().manual_seed(seed + 100)
    segs = []
    for i in range(N_SEG):
        q = (torch.randn((N_Q, S, D), generator=g) / math.sqrt(D)).to(torch.bfloat16)
        d_o = torch.randn((N_Q, S, D), generator=g).to(torch.bfloat16)
        segs.append(dict(q=q, k=k[:, i * S:(i + 1) * S].contiguous(),
                         v=v[:, i * S:(i + 1) * S].contiguous(), d_o=d_o))
    return segs, k, v


def _f32(t):
    return t.detach().float().cpu().numpy()


def _close(name, got, ref, tol=2e-2):
    err, rel = orc.error_stats(got, ref)
    print(f"  {name}: max|d|={err:.3e} rel_l2={rel:.3e}", flush=True)
    ok = orc.lse_within(got, ref) if name == "LSE" else orc.within_tolerance(got, ref, tol)
    assert ok, (name, err, rel)


@pytest.mark.parametrize("sink,window", [(0, 0), (1, 96)])
def test_segments_match_oracle_on_growing_history(sink, window):
    segs, k_all, v_all = _sequence(5)
    h = tbptt.LayerHistory(N_Q, N_KV, D, S, max_hist=4 * S, top_k_chunks=K_C, top_k_groups=K_G,
                           n_sink_chunks=sink, local_window=window)
    extra = dict(n_sink_tokens=64 * sink, window=window or None)
    scale = 1.0 / math.sqrt(D)
    for i, sg in enumerate(segs):
        print(f"[case] tbptt segment {i} history {h.hist_len} sink {sink} window {window}", flush=True)
        g = {k: v.cuda() for k, v in sg.items()}
        o, lse = h.forward(g["q"], g["k"], g["v"])
        dq, dk, dv = h.backward(g["q"], g["k"], g["v"], o, lse, g["d_o"])
        torch.cuda.synchronize()
        H = i * S
        kh = _f32(k_all[:, :H]) if H else np.zeros((N_KV, 0, D), np.float32)
        vh = _f32(v_all[:, :H]) if H else np.zeros((N_KV, 0, D), np.float32)
        if H:
            C_ref, G_ref = orc.chunk_summaries(kh), orc.group_summaries(kh)
            # incrementally built summaries = summaries of the whole history
            kmax = float(np.abs(kh).max())
            assert np.max(np.abs(_f32(h.chunk_sum[:, :H // 64]) - C_ref)) <= 2e-6 * kmax
            assert np.max(np.abs(_f32(h.group_sum[:, :H // 8]) - G_ref)) <= 2e-6 * kmax
            qbar = orc.block_queries(_f32(sg["q"]), N_KV)
            rep = orc.check_selection(qbar, C_ref, G_ref, h.sel_chunks.cpu().numpy(),
                                      h.sel_groups.cpu().numpy(), K_C, K_G, n_sink=sink)
            assert rep["ok"], rep["failures"][:3]
        sel = h.sel_groups.cpu().numpy()
        O_ref, L_ref = orc.attn_fwd(_f32(sg["q"]), kh, vh, _f32(sg["k"]), _f32(sg["v"]), sel, scale,
                                    **extra)
        _close("O", _f32(o), O_ref)
        _close("LSE", _f32(lse), L_ref)
        dQ, dK, dV = orc.attn_bwd(_f32(sg["q"]), kh, vh, _f32(sg["k"]), _f32(sg["v"]), sel, scale,
                                  _f32(sg["d_o"]), **extra)
        _close("dQ", _f32(dq), dQ)
        _close("dK", _f32(dk), dK)
        _close("dV", _f32(dv), dV)
        h.close_segment(g["k"], g["v"])
    torch.cuda.synchronize()
    assert h.hist_len == N_SEG * S
    assert torch.equal(h.k_hist[:, :N_SEG * S].cpu(), k_all)


def test_group_summary_cache_gives_identical_segments():
    # group summaries in host memory behind a 6-slot HBM cache (the 2 blocks x
    # 3 chunks of one call; later segments evict)
    segs, _, _ = _sequence(7)
    dev = tbptt.LayerHistory(N_Q, N_KV, D, S, max_hist=4 * S, top_k_chunks=K_C, top_k_groups=K_G)
    cached = tbptt.LayerHistory(N_Q, N_KV, D, S, max_hist=4 * S, top_k_chunks=K_C, top_k_groups=K_G,
                                group_cache_slots=6)
    for i, sg in enumerate(segs):
        print(f"[case] tbptt group-summary cache segment {i}", flush=True)
        g = {k: v.cuda() for k, v in sg.items()}
        o1, l1 = dev.forward(g["q"], g["k"], g["v"])
        o2, l2 = cached.forward(g["q"], g["k"], g["v"])
        torch.cuda.synchronize()
        assert torch.equal(dev.sel_chunks, cached.sel_chunks)
        assert torch.equal(dev.sel_groups, cached.sel_groups)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        print(f"  hits/misses {cached.cache_stats.cpu().tolist()}", flush=True)
        dev.close_segment(g["k"], g["v"])
        cached.close_segment(g["k"], g["v"])
    torch.cuda.synchronize()
    assert torch.equal(dev.group_sum.cpu(), cached.group_sum)


@pytest.mark.parametrize("sink,window", [(0, 0), (1, 96)])
def test_pinned_host_history_is_bit_identical(sink, window):
    """Segment by segment, forward and backward with the history in
    page-locked host memory equal the device-history driver bit for bit (which
    the test above checks against the oracle)."""
    segs, _, _ = _sequence(6)
    kw = dict(top_k_chunks=K_C, top_k_groups=K_G, n_sink_chunks=sink, local_window=window)
    dev = tbptt.LayerHistory(N_Q, N_KV, D, S, max_hist=4 * S, **kw)
    host = tbptt.LayerHistory(N_Q, N_KV, D, S, max_hist=4 * S, hist_on_host=True, **kw)
    for i, sg in enumerate(segs):
        print(f"[case] tbptt pinned-host segment {i} sink {sink} window {window}", flush=True)
        g = {k: v.cuda() for k, v in sg.items()}
        o1, l1 = dev.forward(g["q"], g["k"], g["v"])
        o2, l2 = host.forward(g["q"], g["k"], g["v"])
        torch.cuda.synchronize()
        assert torch.equal(dev.sel_groups, host.sel_groups)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        g1 = dev.backward(g["q"], g["k"], g["v"], o1, l1, g["d_o"])
        g2 = host.backward(g["q"], g["k"], g["v"], o2, l2, g["d_o"])
        torch.cuda.synchronize()
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)
        dev.close_segment(g["k"], g["v"])
        host.close_segment(g["k"], g["v"])
    torch.cuda.synchronize()
    assert torch.equal(dev.chunk_sum, host.chunk_sum) and torch.equal(dev.group_sum, host.group_sum)
