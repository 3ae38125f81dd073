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
               window=0, check_outputs=True, pinned_host=False, twopass=True):
    """Decode one ragged batch, check it against the oracle sequence by
    sequence; with pinned_host, run it again with the history in page-locked
    host memory and require bit-identical results; with twopass, run it again
    through hga_decode_twopass (bf16 copies of the chunk summaries) and
    require bit-identical results."""
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
    lo = _assert_twopass_identical(s, g, C, G, (o, lse, sc, sg)) if twopass else None
    if pinned_host:
        print("  the same batch with the history in pinned host memory", flush=True)
        kh_p = torch.empty(inp["k_hist"].shape, dtype=w.torch_dtype, pin_memory=True)
        vh_p = torch.empty(inp["v_hist"].shape, dtype=w.torch_dtype, pin_memory=True)
        kh_p.copy_(inp["k_hist"])
        vh_p.copy_(inp["v_hist"])
        sh = hga.make_shape(n_q, n_kv, d, P, T, k_c, k_g, w.torch_dtype, w.softmax_scale, True,
                            n_sink_chunks=sink, local_window=window)
        o2, lse2, sc2, sg2 = hga.decode(sh, g["q"], kh_p, vh_p, C, G, g["k_tail"], g["v_tail"],
                                        g["hist_lens"], g["tail_lens"])
        torch.cuda.synchronize()
        assert torch.equal(sc2, sc) and torch.equal(sg2, sg)
        assert torch.equal(o2, o) and torch.equal(lse2, lse)
        if lo is not None:
            print("  pinned host memory with the two-pass route", flush=True)
            out = hga.decode(sh, g["q"], kh_p, vh_p, C, G, g["k_tail"], g["v_tail"], g["hist_lens"],
                             g["tail_lens"], chunk_sum_bf16=lo)
            torch.cuda.synchronize()
            for name, a, b in zip(("o", "lse", "sel_chunks", "sel_groups"), out, (o, lse, sc, sg)):
                assert torch.equal(a, b), name
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
            ok = orc.lse_within(got, ref) if name == "LSE" else orc.within_tolerance(got, ref, tol)
            assert ok, (b, name, err, rel)
    return o, lse, sc, sg


def _assert_twopass_identical(s, g, C, G, ref):
    """hga_decode_twopass on bf16 copies of C gives hga_decode's outputs bit for
    bit; the copies themselves are torch's round-to-nearest-even of C."""
    print("  two-pass chunk route on bf16 copies", flush=True)
    lo = hga.summaries_to_bf16(C)
    fin = torch.isfinite(C)
    assert torch.equal(lo[fin], C[fin].to(torch.bfloat16))
    assert torch.isnan(lo[torch.isnan(C)].float()).all()
    out = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                     g["hist_lens"], g["tail_lens"], chunk_sum_bf16=lo)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "lse", "sel_chunks", "sel_groups"), out, ref):
        assert torch.equal(a, b), name
    return lo


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
# workgroups (history capacity of 32,768+ tokens and at most 64
# (sequence, KV head) pairs): ragged histories from full to empty, some with
# fewer chunks than parts, against the oracle.
@pytest.mark.parametrize("n_new,sink,window", [(1, 0, 0), (2, 1, 40)])
def test_decode_split_route_ragged(n_new, sink, window):
    run_decode(8, 2, 128, 32768, 256, 16, 32, "bf16", [32768, 20032, 192, 0], [256, 100, 7, 40],
               n_new=n_new, seed=10 + n_new, sink=sink, window=window)


def test_decode_split_route_matches_unsplit():
    # the same four sequences alone (32 (sequence, KV head) pairs: the chunk
    # scan split in 8 parts), tiled to a batch of 8 (64 pairs: 4 parts) and to
    # a batch of 32 (256 pairs: one workgroup each) give bit-identical
    # selections; the attention splits the keys into pieces of 128 (small
    # batch) or 256, so its outputs agree to rounding
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
    rep2 = lambda x: x.repeat((2,) + (1,) * (x.dim() - 1))
    o8, lse8, sc8, sg8 = hga.decode(s, rep2(g["q"]), rep2(g["k_hist"]), rep2(g["v_hist"]), rep2(C), rep2(G),
                                    rep2(g["k_tail"]), rep2(g["v_tail"]), rep2(g["hist_lens"]),
                                    rep2(g["tail_lens"]))
    torch.cuda.synchronize()
    assert torch.equal(sc32[:4], sc4) and torch.equal(sg32[:4], sg4)
    assert torch.equal(sc32[:8], sc8) and torch.equal(sg32[:8], sg8)
    o_ref = o4.float()
    assert (o32[:4].float() - o_ref).abs().max() <= 1e-2 * o_ref.abs().max()
    assert (lse32[:4] - lse4).abs().max() <= 1e-5 * lse4.abs().max()


def test_decode_qwen3_8b_131k():
    # Qwen3-8B layer shapes, 129,024-token history capacity, 2,048-token open
    # segment, one new token per sequence, ragged lengths; again with the
    # history in pinned host memory
    run_decode(32, 8, 128, 129024, 2048, 16, 32, "bf16", [129024, 100032], [2048, 517], n_new=1,
               seed=6, pinned_host=True)


# History in page-locked host memory: each (sequence, KV head)'s sink rows and
# routed groups are copied over the host link before the attention; the
# results equal the device-history decode bit for bit. One and four new
# tokens (VALU and MFMA P.V), a sink and window, ragged lengths down to empty,
# fp32 at d = 64.
@pytest.mark.parametrize("n_q,d,n_new,sink,window,dtype", [
    (8, 128, 1, 0, 0, "bf16"), (8, 128, 4, 1, 40, "bf16"), (4, 64, 2, 2, 0, "f32")])
def test_decode_pinned_host_history(n_q, d, n_new, sink, window, dtype):
    run_decode(n_q, 2, d, 2048, 256, 5, 13, dtype, [2048, 704, 0, 128], [256, 31, 9, 64], n_new=n_new,
               seed=30 + n_new, sink=sink, window=window, pinned_host=True)


def test_decode_qwen3_8b_131k_four_new_tokens():
    # the same shapes with four new tokens: 16 query rows per KV head, whose
    # P.V runs on MFMA over 128-key pieces
    run_decode(32, 8, 128, 129024, 2048, 16, 32, "bf16", [129024, 64064], [2048, 1029], n_new=4,
               seed=8)


def test_decode_gqa8_two_new_tokens_with_sink_and_window():
    # GQA ratio 8 x 2 new tokens: 16 query rows (MFMA P.V) at d = 128, with a
    # sink and a window that cuts into the open segment
    run_decode(16, 2, 128, 2048, 256, 6, 24, "bf16", [2048, 704, 64], [256, 31, 2], n_new=2, seed=9,
               sink=2, window=100)


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
    assert orc.lse_within(_f64(lse[0]), L_ref)


def _random_decode_cases(n=10, seed=20261204):
    """Seeded random ragged batches, every axis drawn at once: GQA ratio and KV
    heads, new tokens per sequence (r * n_new <= 16), head dim, capacities,
    history lengths in whole chunks (0 included), open-segment lengths, budgets,
    sink, window, dtype."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        r = int(rng.choice([1, 2, 4, 8]))
        n_kv = int(rng.choice([1, 2, 4]))
        n_new = int(rng.integers(1, 5))
        while r * n_new > 16:
            n_new -= 1
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        P = 64 * int(rng.integers(1, 48))
        T = 64 * int(rng.integers(1, 9))
        B = int(rng.integers(1, 6))
        hist = [64 * int(rng.integers(0, P // 64 + 1)) for _ in range(B)]
        tail = [int(rng.integers(n_new, T + 1)) for _ in range(B)]
        k_c = int(rng.integers(1, 9))
        k_g = int(rng.integers(1, 8 * k_c + 9))
        sink = int(rng.integers(1, 3)) if rng.random() < 0.4 else 0
        window = int(rng.integers(1, T + 1)) if rng.random() < 0.5 else 0
        out.append((f"rdec{i}", r * n_kv, n_kv, d, P, T, k_c, k_g, dtype, hist, tail, n_new, sink, window))
    return out


RANDOM_DECODE = _random_decode_cases()


@pytest.mark.parametrize("case", RANDOM_DECODE, ids=[c[0] for c in RANDOM_DECODE])
def test_decode_random_batches(case):
    _, n_q, n_kv, d, P, T, k_c, k_g, dtype, hist, tail, n_new, sink, window = case
    run_decode(n_q, n_kv, d, P, T, k_c, k_g, dtype, hist, tail, n_new=n_new, seed=7, sink=sink,
               window=window)


def _random_split_cases(n=4, seed=20261208):
    """Seeded random small batches with long histories (32K-128K capacity), so
    the chunk scan is split over several workgroups per (sequence, KV head)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        n_kv = int(rng.choice([1, 2, 4]))
        r = int(rng.choice([1, 2, 4]))
        n_new = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        P = 64 * int(rng.integers(512, 2049))
        T = 64 * int(rng.integers(1, 5))
        B = int(rng.integers(1, 5))
        hist = [64 * int(rng.integers(P // 128, P // 64 + 1)) for _ in range(B)]
        tail = [int(rng.integers(n_new, T + 1)) for _ in range(B)]
        k_c = int(rng.integers(4, 17))
        k_g = int(rng.integers(8, 8 * k_c + 1))
        sink = int(rng.integers(1, 3)) if rng.random() < 0.4 else 0
        window = int(rng.integers(1, T + 1)) if rng.random() < 0.5 else 0
        out.append((f"rsplit{i}", r * n_kv, n_kv, d, P, T, k_c, k_g, "bf16", hist, tail, n_new, sink, window))
    return out


RANDOM_SPLIT = _random_split_cases()


@pytest.mark.parametrize("case", RANDOM_SPLIT, ids=[c[0] for c in RANDOM_SPLIT])
def test_decode_random_long_histories(case):
    _, n_q, n_kv, d, P, T, k_c, k_g, dtype, hist, tail, n_new, sink, window = case
    run_decode(n_q, n_kv, d, P, T, k_c, k_g, dtype, hist, tail, n_new=n_new, seed=8, sink=sink,
               window=window)


def _twopass_variants(C, seed):
    """Chunk summaries built to stress the two-pass bound: the real ones,
    identical rows (every chunk ties), rows equal in bf16 but apart in fp32
    (the order is decided by fp32 alone), zeros, huge and subnormal scales
    (fallback and absolute-bound paths), a NaN and an infinite row."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    B, kv, R, d = C.shape
    base = C[:, :, :1].clone()
    yield "real", C
    yield "identical", base.expand(-1, -1, R, -1).contiguous()
    tie = base.expand(-1, -1, R, -1).clone()
    # chunks differ in one coordinate by less than a quarter of a bf16 ulp
    # (relative 2^-9), in shuffled order: their copies mostly coincide
    perm = torch.randperm(R, generator=gen).to(C.device).view(1, 1, R).float()
    tie[..., 0] = tie[..., 0] * (1 + perm * 2.0 ** -20)
    yield "bf16-ties", tie.contiguous()
    yield "zeros", torch.zeros_like(C)
    yield "huge", (C * 1e35).contiguous()
    yield "subnormal", (C * 1e-39).contiguous()
    bad = C.clone()
    bad[0, 0, R // 3, 5] = float("nan")
    bad[-1, -1, R // 2, 7] = float("inf")
    yield "nan-inf", bad


@pytest.mark.parametrize("B,P", [(4, 16384), (4, 32768), (9, 32768)],
                         ids=["unsplit-256", "split-8x64", "unsplit-512"])
def test_decode_twopass_adversarial_summaries(B, P):
    """hga_decode_twopass equals hga_decode bit for bit on chunk summaries made
    to defeat the bf16 bound: 256 chunks in one workgroup, 512 chunks split in
    8 parts of 64 (a split scan reads no copies: both run the fp32 scan), and
    512 chunks in one workgroup (every chunk a candidate: the fp32 scan)."""
    n_q, n_kv, d, T = 8, 8, 64, 64
    hist = [P - 64 * b for b in range(B)]
    tail = [64 - b for b in range(B)]
    w = synth.Workload("decode", n_q, n_kv, d, P, T, 16, 32, "bf16", 1.0 / math.sqrt(d))
    print(f"[case] decode two-pass adversarial B={B} P={P}", flush=True)
    inp = synth.make_decode_inputs(w, hist, tail, 1, 31 + B)
    g = {k: v.cuda() for k, v in inp.items()}
    s = hga.make_shape(n_q, n_kv, d, P, T, 16, 32, torch.bfloat16, w.softmax_scale)
    C = torch.zeros((B, n_kv, P // 64, d), dtype=torch.float32, device="cuda")
    G = torch.zeros((B, n_kv, P // 8, d), dtype=torch.float32, device="cuda")
    for b in range(B):
        sb = hga.make_shape(n_q, n_kv, d, hist[b], T, 16, 32, torch.bfloat16, hist_stride=P)
        hga.hga_build_summaries(sb, g["k_hist"][b], C[b], G[b])
    for name, Cv in _twopass_variants(C, 7 + B):
        print(f"  summaries: {name}", flush=True)
        ref = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], Cv, G, g["k_tail"], g["v_tail"],
                         g["hist_lens"], g["tail_lens"])
        torch.cuda.synchronize()
        _assert_twopass_identical(s, g, Cv, G, ref)


def test_summaries_to_bf16_special_values_and_ragged_length():
    """hga_summaries_to_bf16 rounds to nearest even like torch: zeros of both
    signs, subnormals, halfway cases, values that overflow to infinity,
    infinities and NaN; a length of 8 * 1001 elements leaves a ragged last
    workgroup, and an empty call does nothing."""
    print("[case] bf16 copies: special values, 8008 elements", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(5)
    x = torch.randn(8 * 1001, generator=gen)
    special = torch.tensor([0.0, -0.0, 1e-40, -1e-40, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.39e38, 3.4e38,
                            -3.4e38, float("inf"), float("-inf"), float("nan")])
    x[: special.numel()] = special
    x[100:200] *= 1e-39
    src = x.cuda()
    dst = torch.full(src.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    hga.hga_summaries_to_bf16(src, dst)
    hga.hga_summaries_to_bf16(src[:0], dst[:0])
    torch.cuda.synchronize()
    want = x.to(torch.bfloat16)
    got = dst.cpu()
    nan = torch.isnan(x)
    assert torch.isnan(got[nan].float()).all()
    assert torch.equal(got[~nan].view(torch.int16), want[~nan].view(torch.int16))


def test_decode_twopass_over_a_growing_history():
    """A decode loop whose history grows: at every step some sequences close a
    chunk, whose summaries are built on their own and whose sequence's bf16
    copies are refreshed; hga_decode_twopass equals hga_decode bit for bit at
    every step, and the incrementally built summaries equal a full build."""
    n_q, n_kv, d, P, T, B = 8, 8, 64, 32768, 64, 9
    hist = [P - 64 * (4 + b) for b in range(B)]
    tail = [64 - 3 * b for b in range(B)]
    w = synth.Workload("decode", n_q, n_kv, d, P, T, 16, 32, "bf16", 1.0 / math.sqrt(d))
    print(f"[case] decode two-pass, growing history B={B} P={P}", flush=True)
    inp = synth.make_decode_inputs(w, hist, tail, 1, 41)
    g = {k: v.cuda() for k, v in inp.items()}
    s = hga.make_shape(n_q, n_kv, d, P, T, 16, 32, torch.bfloat16, w.softmax_scale)
    C = torch.zeros((B, n_kv, P // 64, d), dtype=torch.float32, device="cuda")
    G = torch.zeros((B, n_kv, P // 8, d), dtype=torch.float32, device="cuda")

    def close(b, t0, t1):
        sb = hga.make_shape(n_q, n_kv, d, t1, T, 16, 32, torch.bfloat16, hist_stride=P)
        hga.hga_build_summaries(sb, g["k_hist"][b], C[b], G[b], t0, t1)

    for b in range(B):
        close(b, 0, hist[b])
    lo = hga.summaries_to_bf16(C)
    for step in range(4):
        for b in range(B):
            if (b + step) % 2 == 0:
                hist[b] += 64
                close(b, hist[b] - 64, hist[b])
                hga.hga_summaries_to_bf16(C[b], lo[b])
        g["hist_lens"] = torch.tensor(hist, dtype=torch.int32, device="cuda")
        print(f"  step {step}: hist={hist}", flush=True)
        ref = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                         g["hist_lens"], g["tail_lens"])
        out = hga.decode(s, g["q"], g["k_hist"], g["v_hist"], C, G, g["k_tail"], g["v_tail"],
                         g["hist_lens"], g["tail_lens"], chunk_sum_bf16=lo)
        torch.cuda.synchronize()
        for name, a, b_ in zip(("o", "lse", "sel_chunks", "sel_groups"), out, ref):
            assert torch.equal(a, b_), (step, name)
    C2 = torch.zeros_like(C)
    G2 = torch.zeros_like(G)
    for b in range(B):
        sb = hga.make_shape(n_q, n_kv, d, hist[b], T, 16, 32, torch.bfloat16, hist_stride=P)
        hga.hga_build_summaries(sb, g["k_hist"][b], C2[b], G2[b])
    torch.cuda.synchronize()
    assert torch.equal(C, C2) and torch.equal(G, G2)
