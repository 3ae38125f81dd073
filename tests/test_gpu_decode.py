"""Decode step on the GPU (hga_decode, through the C ABI) against the oracle's
decode_step, per sequence of a ragged batch: routing through the selection
checker (exact up to near-ties), outputs with the oracle fed the GPU's own
selection, to the same tolerance as the training path."""
import math

import numpy as np
import pytest
import torch

from long_context_fine_amd import hga, synth
from oracle import hga_oracle as orc

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


def _f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def run_decode(n_q, n_kv, d, P, T, k_c, k_g, dtype, hist_lens, tail_lens, n_new, seed, sink=0,
               window=0, check_outputs=True):
    print(f"[case] decode nq={n_q} nkv={n_kv} d={d} P={P} T={T} kc={k_c} kg={k_g} {dtype} "
          f"hist={list(hist_lens)} tail={list(tail_lens)} n_new={n_new} sink={sink} W={window}",
          flush=True)
    w = synth.Workload("decode", n_q, n_kv, d, P, T, k_c, k_g, dtype,
                       1.0 if dtype == "f32" else 1.0 / math.sqrt(d))
    inp = synth.make_decode_inputs(w, hist_lens, tail_lens, n_new, seed)
    g = {k: v.cuda() for k, v in inp.items()}
    B = len(hist_lens)
    s = hga.make_shape(n_q, n_kv, d, P, T, k_c, k_g, w.torch_dtype, w.softmax_scale,
                       n_sink_chunks=sink, local_window=window)
    C = torch.zeros((B, n_kv, P // 64, d), dtype=torch.float32, device="cuda")
    G = torch.zeros((B, n_kv, P // 8, d), dtype=torch.float32, device="cuda")
    for b in range(B):
        if hist_lens[b]:
            sb = hga.make_shape(n_q, n_kv, d, hist_lens[b], T, k_c, k_g, w.torch_dtype,
                                hist_stride=P)
            hga.hga_build_summaries(sb, g["k_hist"][b], C[b], G[b])
    o, lse, sc, sg = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                                g["hist_lens"], g["tail_lens"])
    torch.cuda.synchronize()
    tol = TOL[dtype]
    for b in range(B):
        H, Tb = hist_lens[b], tail_lens[b]
        qb = _f64(inp["q"][b])
        kh, vh = _f64(inp["k_hist"][b][:, :H]), _f64(inp["v_hist"][b][:, :H])
        kt, vt = _f64(inp["k_tail"][b][:, :Tb]), _f64(inp["v_tail"][b][:, :Tb])
        sc_b, sg_b = sc[b].cpu().numpy(), sg[b].cpu().numpy()
        if H:
            qbar = orc.decode_query_mean(qb, n_kv)[None]
            rep = orc.check_selection(qbar, orc.chunk_summaries(kh), orc.group_summaries(kh),
                                      sc_b[None], sg_b[None], k_c, k_g, n_sink=sink)
            print(f"  seq {b}: route ok={rep['ok']} exemptions={rep['chunk_exemptions']}/"
                  f"{rep['group_exemptions']}", flush=True)
            assert rep["ok"], rep["failures"][:3]
        else:
            assert (sc_b == -1).all() and (sg_b == -1).all()
        if not check_outputs:
            continue
        _, _, O_ref, L_ref = orc.decode_step(qb, kh, vh, kt, vt, k_c, k_g, w.softmax_scale,
                                             n_sink=sink, window=window or None, sel_groups=sg_b)
        for name, got, ref in (("O", _f64(o[b]), O_ref), ("LSE", _f64(lse[b]), L_ref)):
            err, rel = orc.error_stats(got, ref)
            print(f"  seq {b} {name}: max|d|={err:.3e} rel_l2={rel:.3e}", flush=True)
            assert orc.within_tolerance(got, ref, tol), (b, name, err, rel)
    return o, lse, sc, sg


def test_decode_ragged_batch_one_new_token():
    run_decode(8, 2, 128, 1024, 256, 4, 16, "bf16", [1024, 512, 0, 64, 960], [256, 1, 130, 77, 200],
               n_new=1, seed=0)


def test_decode_two_new_tokens_with_sink_and_window():
    run_decode(8, 2, 128, 2048, 192, 5, 13, "bf16", [2048, 640, 128], [192, 50, 3], n_new=2, seed=1,
               sink=1, window=50)


def test_decode_sixteen_query_rows_d64():
    # r = 4 heads x 4 new tokens; a window of 1 keeps only each token itself
    run_decode(8, 2, 64, 1024, 128, 3, 20, "bf16", [1024, 320], [128, 4], n_new=4, seed=2)
    run_decode(8, 2, 64, 1024, 128, 3, 20, "bf16", [704, 64], [100, 9], n_new=4, seed=3, window=1)


def test_decode_fp32_mha():
    run_decode(2, 2, 64, 512, 128, 3, 10, "f32", [512, 256], [128, 65], n_new=1, seed=4)


def test_decode_lengths_are_clamped_to_the_buffers():
    # a history beyond the capacity reads as full, a ragged one as whole chunks
    # and an open segment shorter than n_new as n_new tokens
    w = dict(n_q=4, n_kv=1, d=128, P=512, T=128, k_c=2, k_g=8, dtype="bf16")
    a = run_decode(**w, hist_lens=[512, 448], tail_lens=[128, 2], n_new=2, seed=5, check_outputs=False)
    inp_lens = [(10 ** 6, 1000), (490, 1)]
    wl = synth.Workload("decode", 4, 1, 128, 512, 128, 2, 8, "bf16", 1.0 / math.sqrt(128))
    inp = synth.make_decode_inputs(wl, [512, 448], [128, 2], 2, 5)
    g = {k: v.cuda() for k, v in inp.items()}
    g["hist_lens"] = torch.tensor([x for x, _ in inp_lens], dtype=torch.int32, device="cuda")
    g["tail_lens"] = torch.tensor([y for _, y in inp_lens], dtype=torch.int32, device="cuda")
    s = hga.make_shape(4, 1, 128, 512, 128, 2, 8, torch.bfloat16)
    C = torch.zeros((2, 1, 8, 128), dtype=torch.float32, device="cuda")
    G = torch.zeros((2, 1, 64, 128), dtype=torch.float32, device="cuda")
    for b, H in enumerate([512, 448]):
        hga.hga_build_summaries(hga.make_shape(4, 1, 128, H, 128, 2, 8, torch.bfloat16, hist_stride=512),
                                g["k_hist"][b], C[b], G[b])
    o, lse, sc, sg = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                                g["hist_lens"], g["tail_lens"])
    torch.cuda.synchronize()
    assert torch.equal(o, a[0]) and torch.equal(lse, a[1]) and torch.equal(sg, a[3])


# Small batches split the chunk scan of each (sequence, KV head) over several
# workgroups (history capacity of 32,768+ tokens and fewer than 256
# (sequence, KV head) pairs): ragged histories from full to empty, some with
# fewer chunks than parts, against the oracle.
@pytest.mark.parametrize("n_new,sink,window", [(1, 0, 0), (2, 1, 40)])
def test_decode_split_route_ragged(n_new, sink, window):
    run_decode(8, 2, 128, 32768, 256, 16, 32, "bf16", [32768, 20032, 192, 0], [256, 100, 7, 40],
               n_new=n_new, seed=10 + n_new, sink=sink, window=window)


def test_decode_split_route_matches_unsplit():
    # the same four sequences alone (32 (sequence, KV head) pairs: split
    # route) and tiled to a batch of 32 (256 pairs: one workgroup each) give
    # bit-identical selections; the attention splits the keys into pieces of
    # 128 (small batch) or 256, so its outputs agree to rounding
    n_q, n_kv, d, P, T = 32, 8, 128, 32768, 256
    hist, tail = [32768, 26624, 4096, 64], [256, 33, 128, 1]
    w = synth.Workload("decode", n_q, n_kv, d, P, T, 16, 32, "bf16", 1.0 / math.sqrt(d))
    print(f"[case] decode split vs unsplit P={P} hist={hist}", flush=True)
    inp = synth.make_decode_inputs(w, hist, tail, 1, 21)
    g = {k: v.cuda() for k, v in inp.items()}
    s = hga.make_shape(n_q, n_kv, d, P, T, 16, 32, torch.bfloat16, w.softmax_scale)
    C = torch.zeros((4, n_kv, P // 64, d), dtype=torch.float32, device="cuda")
    G = torch.zeros((4, n_kv, P // 8, d), dtype=torch.float32, device="cuda")
    for b in range(4):
        sb = hga.make_shape(n_q, n_kv, d, hist[b], T, 16, 32, torch.bfloat16, hist_stride=P)
        hga.hga_build_summaries(sb, g["k_hist"][b], C[b], G[b])
    o4, lse4, sc4, sg4 = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                                    g["hist_lens"], g["tail_lens"])
    rep = lambda x: x.repeat((8,) + (1,) * (x.dim() - 1))
    o32, lse32, sc32, sg32 = hga.decode(s, rep(g["q"]), rep(g["k_hist"]), rep(g["v_hist"]), rep(C), rep(G),
                                        rep(g["k_tail"]), rep(g["v_tail"]), rep(g["hist_lens"]),
                                        rep(g["tail_lens"]))
    torch.cuda.synchronize()
    assert torch.equal(sc32[:4], sc4) and torch.equal(sg32[:4], sg4)
    o_ref = o4.float()
    assert (o32[:4].float() - o_ref).abs().max() <= 1e-2 * o_ref.abs().max()
    assert (lse32[:4] - lse4).abs().max() <= 1e-5 * lse4.abs().max()


def test_decode_qwen3_8b_131k():
    # Qwen3-8B layer shapes, 129,024-token history capacity, 2,048-token open
    # segment, one new token per sequence, ragged lengths
    run_decode(32, 8, 128, 129024, 2048, 16, 32, "bf16", [129024, 100032], [2048, 517], n_new=1,
               seed=6)


def test_decode_retrieves_a_planted_needle():
    # retrieval: one history chunk of sequence 0, far back, gets keys aligned
    # with the new token's query; routing must select it and most attention
    # mass must land on it (the output moves toward that chunk's values)
    n_q, n_kv, d, P, T = 8, 2, 128, 8192, 128
    w = synth.Workload("decode", n_q, n_kv, d, P, T, 4, 16, "bf16", 1.0 / math.sqrt(d))
    inp = synth.make_decode_inputs(w, [P], [T], 1, 9)
    needle = 17                                  # chunk 17 of 128
    r = n_q // n_kv
    for j in range(n_kv):
        qdir = inp["q"][0, j * r:(j + 1) * r, 0].float().mean(0)
        qdir = qdir / qdir.norm()
        inp["k_hist"][0, j, 64 * needle:64 * needle + 64] = (qdir * 200.0).to(torch.bfloat16)
        inp["v_hist"][0, j, 64 * needle:64 * needle + 64] = 1.0
    g = {k: v.cuda() for k, v in inp.items()}
    s = hga.make_shape(n_q, n_kv, d, P, T, 4, 16, torch.bfloat16)
    C = torch.zeros((1, n_kv, P // 64, d), dtype=torch.float32, device="cuda")
    G = torch.zeros((1, n_kv, P // 8, d), dtype=torch.float32, device="cuda")
    hga.hga_build_summaries(s, g["k_hist"][0], C[0], G[0])
    o, lse, sc, sg = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                                g["hist_lens"], g["tail_lens"])
    torch.cuda.synchronize()
    print("[case] decode needle: chunks", sc[0].tolist(), flush=True)
    for j in range(n_kv):
        assert needle in sc[0, j].tolist()
        assert set(range(8 * needle, 8 * needle + 8)) <= set(sg[0, j].tolist())
    # the needle's values (all ones) dominate: every output coordinate near 1
    assert float(o.float().mean()) > 0.9
    _, _, O_ref, L_ref = orc.decode_step(_f64(inp["q"][0]), _f64(inp["k_hist"][0]), _f64(inp["v_hist"][0]),
                                         _f64(inp["k_tail"][0]), _f64(inp["v_tail"][0]), 4, 16,
                                         w.softmax_scale, sel_groups=sg[0].cpu().numpy())
    assert orc.within_tolerance(_f64(o[0]), O_ref, TOL["bf16"])
    assert orc.within_tolerance(_f64(lse[0]), L_ref, TOL["bf16"])
