"""Pins for the CPU oracle, each against something other than the oracle itself:
closed forms, brute force, torch's scaled-dot-product attention and autograd
(independent library implementations of dense attention), finite differences
and negative controls. CPU only.
"""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import hga_oracle as orc
from long_context_fine_amd import synth


def _small(**kw):
    base = dict(name="small", n_q_heads=4, n_kv_heads=2, head_dim=16, hist_len=512,
                seg_len=128, top_k_chunks=3, top_k_groups=6, dtype="f32",
                input_scale=1.0, backward=True)
    base.update(kw)
    return synth.Workload(**base)


def _np(inp):
    return {k: synth.to_numpy64(v) for k, v in inp.items()}


# ---------------------------------------------------------------------------
# summaries and block queries: closed forms and invariants
# ---------------------------------------------------------------------------
def test_summary_of_constant_keys_is_the_constant():
    rng = np.random.default_rng(1)
    # bf16-representable constants: every partial sum k*c (k <= 64) is exact in fp32
    c = torch.from_numpy(rng.standard_normal((3, 1, 16)).astype(np.float32)).bfloat16().float().numpy()
    k = np.broadcast_to(c, (3, 256, 16)).copy()
    C = orc.chunk_summaries(k)
    G = orc.group_summaries(k)
    assert C.shape == (3, 4, 16) and G.shape == (3, 32, 16)
    assert np.array_equal(C, np.broadcast_to(c, C.shape))
    assert np.array_equal(G, np.broadcast_to(c, G.shape))


def test_summary_of_token_ramp_closed_form():
    n_kv, H, d = 2, 512, 8
    t = np.arange(H, dtype=np.float64)[None, :, None]
    j = np.arange(n_kv, dtype=np.float64)[:, None, None]
    e = np.arange(d, dtype=np.float64)[None, None, :]
    k = t + 1000.0 * j + 10000.0 * e
    C = orc.chunk_summaries(k)
    G = orc.group_summaries(k)
    m = np.arange(H // 64, dtype=np.float64)[None, :, None]
    n = np.arange(H // 8, dtype=np.float64)[None, :, None]
    # mean of 64m..64m+63 is 64m + 31.5; mean of 8n..8n+7 is 8n + 3.5
    assert np.array_equal(C, (64 * m + 31.5 + 1000.0 * j + 10000.0 * e).astype(np.float32))
    assert np.array_equal(G, (8 * n + 3.5 + 1000.0 * j + 10000.0 * e).astype(np.float32))


def test_chunk_summary_is_mean_of_its_group_summaries():
    inp = _np(synth.make_inputs(_small(), seed=3))
    C = orc.chunk_summaries(inp["k_hist"])
    G = orc.group_summaries(inp["k_hist"])
    G8 = G.reshape(G.shape[0], -1, 8, G.shape[2]).astype(np.float64).mean(axis=2)
    assert np.allclose(C, G8, rtol=0, atol=1e-6 * np.abs(C).max())


def test_summary_invariant_under_token_permutation_within_chunk():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, 256, 16)).astype(np.float32)
    perm = np.concatenate([64 * c + rng.permutation(64) for c in range(4)])
    a = orc.chunk_summaries(k)
    b = orc.chunk_summaries(k[:, perm])
    assert np.allclose(a, b, rtol=0, atol=1e-6)


def test_block_query_closed_form():
    n_q, n_kv, S, d = 8, 2, 192, 4
    r = n_q // n_kv
    h = np.arange(n_q, dtype=np.float64)[:, None, None]
    i = np.arange(S, dtype=np.float64)[None, :, None]
    e = np.arange(d, dtype=np.float64)[None, None, :]
    q = i + 100.0 * h + 0.25 * e
    qbar = orc.block_queries(q, n_kv)
    assert qbar.shape == (S // 64, n_kv, d)
    for b in range(S // 64):
        for j in range(n_kv):
            # mean over i in 64b..64b+63 and h in jr..jr+r-1
            want = 64 * b + 31.5 + 100.0 * (j * r + (r - 1) / 2) + 0.25 * np.arange(d)
            assert np.array_equal(qbar[b, j], want.astype(np.float32))


# ---------------------------------------------------------------------------
# top-k: brute force, ties, NaN / signed zero
# ---------------------------------------------------------------------------
def _bruteforce_topk(s, k):
    """The unique k-subset whose every member beats every non-member under
    (higher score, then lower index); found by enumerating all subsets."""
    n = len(s)
    k = min(k, n)

    def beats(x, y):
        return s[x] > s[y] or (s[x] == s[y] and x < y)

    hits = [set(c) for c in itertools.combinations(range(n), k)
            if all(beats(x, y) for x in c for y in range(n) if y not in c)]
    assert len(hits) == 1
    return sorted(hits[0])


@pytest.mark.parametrize("seed", range(40))
def test_topk_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    k = int(rng.integers(1, 11))
    # few distinct values so that ties are frequent
    s = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.5)
    got = orc.topk_lowest_index(s, k).tolist()
    assert got == _bruteforce_topk(s.tolist(), k)


def test_topk_nan_is_last_and_signed_zeros_tie():
    s = np.array([np.nan, -0.0, 0.0, -1.0, np.nan, 0.0], dtype=np.float32)
    assert orc.topk_lowest_index(s, 1).tolist() == [1]        # -0 ties +0: lowest index
    assert orc.topk_lowest_index(s, 3).tolist() == [1, 2, 5]
    assert orc.topk_lowest_index(s, 4).tolist() == [1, 2, 3, 5]
    assert orc.topk_lowest_index(s, 5).tolist() == [0, 1, 2, 3, 5]


def test_route_exact_ties_choose_lowest_index():
    # integer-valued keys with identical chunks: every score ties exactly
    n_kv, H, d, S, n_q = 1, 1024, 8, 128, 2
    k = np.ones((n_kv, H, d))
    q = np.ones((n_q, S, d))
    sel_c, sel_g, _ = orc.route(q, k, n_kv, k_c=4, k_g=8)
    assert (sel_c == np.arange(4)).all()
    assert (sel_g == np.arange(8)).all()
    # make chunk 9 and its group 75 strictly better; the rest still tie
    k[0, 9 * 64:10 * 64] = 2.0
    k[0, 75 * 8:76 * 8] = 3.0
    sel_c, sel_g, _ = orc.route(q, k, n_kv, k_c=4, k_g=8)
    assert sel_c[0, 0].tolist() == [0, 1, 2, 9]
    # group 75 first, then chunk 9's other groups (score 2), then lowest-index ones
    assert sel_g[0, 0].tolist() == [72, 73, 74, 75, 76, 77, 78, 79]


def test_route_planted_chunk_ranks_first():
    w = synth.WORKLOADS["tiny_f32"]
    inp = _np(synth.make_inputs(w, seed=5))
    qbar = orc.block_queries(inp["q"], 1)
    for b, m_star in [(0, 7), (1, 12)]:
        k = inp["k_hist"].copy()
        # offset every key of chunk m* along block b's query direction
        k[0, 64 * m_star: 64 * (m_star + 1)] += 50.0 * qbar[b, 0]
        sel_c, sel_g, aux = orc.route(inp["q"], k, 1, w.top_k_chunks, w.top_k_groups)
        sc = aux["chunk_scores"][b, 0]
        assert int(np.argmax(sc)) == m_star and m_star in sel_c[b, 0]
        assert sel_g[b, 0].tolist() == list(range(8 * m_star, 8 * m_star + 8))


@pytest.mark.parametrize("name", ["tiny_f32", "small"])
def test_route_invariants(name):
    w = synth.WORKLOADS["tiny_f32"] if name == "tiny_f32" else _small()
    inp = _np(synth.make_inputs(w, seed=6))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], w.n_kv_heads,
                                w.top_k_chunks, w.top_k_groups)
    n_C = w.hist_len // 64
    for b in range(w.seg_len // 64):
        for j in range(w.n_kv_heads):
            c, g = sel_c[b, j], sel_g[b, j]
            assert len(c) == w.top_k_chunks and (c >= 0).all() and (np.diff(c) > 0).all()
            assert len(g) == w.top_k_groups and (g >= 0).all() and (np.diff(g) > 0).all()
            # every selected index precedes the query block (lies in history)
            assert (c < n_C).all() and (8 * g + 7 < w.hist_len).all()
            # every group lies inside a selected chunk
            assert set((g // 8).tolist()) <= set(c.tolist())


def test_route_budget_larger_than_candidates_pads():
    w = _small(hist_len=128, top_k_chunks=5, top_k_groups=40)
    inp = _np(synth.make_inputs(w, seed=7))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 5, 40)
    assert (sel_c[:, :, :2] == [0, 1]).all() and (sel_c[:, :, 2:] == -1).all()
    assert (sel_g[:, :, :16] == np.arange(16)).all() and (sel_g[:, :, 16:] == -1).all()


# ---------------------------------------------------------------------------
# attention forward vs torch SDPA (float64, independent implementation)
# ---------------------------------------------------------------------------
def _sdpa_with_key_mask(q, k_all, v_all, allowed, scale):
    """q [n_q,S,d]; k_all/v_all [n_kv,T,d]; allowed bool [n_q,S,T]."""
    n_q, n_kv = q.shape[0], k_all.shape[0]
    r = n_q // n_kv
    kq = torch.from_numpy(k_all).repeat_interleave(r, dim=0)
    vq = torch.from_numpy(v_all).repeat_interleave(r, dim=0)
    out = F.scaled_dot_product_attention(torch.from_numpy(q), kq, vq,
                                         attn_mask=torch.from_numpy(allowed), scale=scale)
    s = scale * torch.from_numpy(q) @ kq.transpose(1, 2)
    lse = torch.logsumexp(s.masked_fill(~torch.from_numpy(allowed), -math.inf), dim=-1)
    return out.numpy(), lse.numpy()


def _mask_for_selection(sel_groups, n_q, n_kv, H, S):
    """allowed[h, i, t]: t < H history token of a group selected for (i//64, h//r),
    t >= H segment token with t - H <= i."""
    r = n_q // n_kv
    allowed = np.zeros((n_q, S, H + S), bool)
    for h in range(n_q):
        for i in range(S):
            for n in sel_groups[i // 64, h // r]:
                if n >= 0:
                    allowed[h, i, 8 * n: 8 * n + 8] = True
            allowed[h, i, H: H + i + 1] = True
    return allowed


def test_full_budget_equals_dense_causal_attention():
    # router disabled: every history group selected -> dense causal attention
    w = _small(hist_len=256, top_k_chunks=4, top_k_groups=32)
    inp = _np(synth.make_inputs(w, seed=8))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 4, 32)
    assert (sel_g == np.arange(32)).all()
    O, LSE = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"],
                          inp["v_seg"], sel_g, w.softmax_scale)
    k_all = np.concatenate([inp["k_hist"], inp["k_seg"]], axis=1)
    v_all = np.concatenate([inp["v_hist"], inp["v_seg"]], axis=1)
    H, S = w.hist_len, w.seg_len
    # causal over the full context, queries at positions H .. H+S-1
    pos_q = H + np.arange(S)[:, None]
    allowed = np.broadcast_to(np.arange(H + S)[None, :] <= pos_q, (w.n_q_heads, S, H + S)).copy()
    ref, ref_lse = _sdpa_with_key_mask(inp["q"], k_all, v_all, allowed, w.softmax_scale)
    assert np.max(np.abs(O - ref)) < 1e-12
    assert np.max(np.abs(LSE - ref_lse)) < 1e-12


def test_zero_history_is_causal_attention_over_the_segment():
    w = _small(hist_len=0, top_k_chunks=2, top_k_groups=4)
    inp = _np(synth.make_inputs(w, seed=9))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 2, 4)
    assert (sel_c == -1).all() and (sel_g == -1).all()
    O, _ = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"],
                        inp["v_seg"], sel_g, w.softmax_scale)
    r = w.n_q_heads // w.n_kv_heads
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(inp["q"]),
        torch.from_numpy(inp["k_seg"]).repeat_interleave(r, 0),
        torch.from_numpy(inp["v_seg"]).repeat_interleave(r, 0),
        is_causal=True, scale=w.softmax_scale).numpy()
    assert np.max(np.abs(O - ref)) < 1e-12


@pytest.mark.parametrize("seed", [10, 11])
def test_arbitrary_selection_matches_explicit_key_list(seed):
    w = _small()
    inp = _np(synth.make_inputs(w, seed=seed))
    rng = np.random.default_rng(seed)
    n_B, n_G = w.seg_len // 64, w.hist_len // 8
    sel = np.full((n_B, w.n_kv_heads, 6), -1, np.int32)
    for b in range(n_B):
        for j in range(w.n_kv_heads):
            cnt = int(rng.integers(0, 7))          # includes empty and padded lists
            sel[b, j, :cnt] = np.sort(rng.choice(n_G, cnt, replace=False))
    O, LSE = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"],
                          inp["v_seg"], sel, w.softmax_scale)
    allowed = _mask_for_selection(sel, w.n_q_heads, w.n_kv_heads, w.hist_len, w.seg_len)
    k_all = np.concatenate([inp["k_hist"], inp["k_seg"]], axis=1)
    v_all = np.concatenate([inp["v_hist"], inp["v_seg"]], axis=1)
    ref, ref_lse = _sdpa_with_key_mask(inp["q"], k_all, v_all, allowed, w.softmax_scale)
    assert np.max(np.abs(O - ref)) < 1e-12
    assert np.max(np.abs(LSE - ref_lse)) < 1e-12


def test_uniform_values_give_that_value():
    w = _small()
    inp = _np(synth.make_inputs(w, seed=12))
    v = np.linspace(-2, 3, w.head_dim)
    vh = np.broadcast_to(v, inp["v_hist"].shape).copy()
    vs = np.broadcast_to(v, inp["v_seg"].shape).copy()
    _, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 3, 6)
    O, LSE = orc.attn_fwd(inp["q"], inp["k_hist"], vh, inp["k_seg"], vs, sel_g,
                          w.softmax_scale)
    assert np.max(np.abs(O - v)) < 1e-12


# ---------------------------------------------------------------------------
# attention backward: finite differences and torch autograd
# ---------------------------------------------------------------------------
def _loss(inp, sel, scale, q=None, ks=None, vs=None):
    O, _ = orc.attn_fwd(inp["q"] if q is None else q, inp["k_hist"], inp["v_hist"],
                        inp["k_seg"] if ks is None else ks,
                        inp["v_seg"] if vs is None else vs, sel, scale)
    return float(np.sum(O * inp["d_o"]))


@pytest.mark.parametrize("wname", ["tiny_f32", "gqa"])
def test_backward_matches_central_finite_differences(wname):
    w = synth.WORKLOADS["tiny_f32"] if wname == "tiny_f32" else _small()
    inp = _np(synth.make_inputs(w, seed=13, with_grad_out=True))
    _, sel, _ = orc.route(inp["q"], inp["k_hist"], w.n_kv_heads, w.top_k_chunks,
                          w.top_k_groups)
    dQ, dK, dV = orc.attn_bwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"],
                              inp["v_seg"], sel, w.softmax_scale, inp["d_o"])
    rng = np.random.default_rng(14)
    eps = 1e-6
    for key, grad in (("q", dQ), ("k_seg", dK), ("v_seg", dV)):
        fd, an = [], []
        for _ in range(24):
            idx = tuple(int(rng.integers(0, n)) for n in inp[key].shape)
            plus, minus = inp[key].copy(), inp[key].copy()
            plus[idx] += eps
            minus[idx] -= eps
            kw_p = {{"q": "q", "k_seg": "ks", "v_seg": "vs"}[key]: plus}
            kw_m = {{"q": "q", "k_seg": "ks", "v_seg": "vs"}[key]: minus}
            fd.append((_loss(inp, sel, w.softmax_scale, **kw_p)
                       - _loss(inp, sel, w.softmax_scale, **kw_m)) / (2 * eps))
            an.append(grad[idx])
        fd, an = np.array(fd), np.array(an)
        assert np.linalg.norm(fd - an) <= 1e-6 * np.linalg.norm(an), key


def test_backward_full_budget_matches_torch_autograd():
    w = _small(hist_len=256, top_k_chunks=4, top_k_groups=32)
    inp = _np(synth.make_inputs(w, seed=15))
    _, sel, _ = orc.route(inp["q"], inp["k_hist"], 2, 4, 32)
    dQ, dK, dV = orc.attn_bwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"],
                              inp["v_seg"], sel, w.softmax_scale, inp["d_o"])
    q = torch.from_numpy(inp["q"]).requires_grad_(True)
    ks = torch.from_numpy(inp["k_seg"]).requires_grad_(True)
    vs = torch.from_numpy(inp["v_seg"]).requires_grad_(True)
    kh = torch.from_numpy(inp["k_hist"])        # detached history
    vh = torch.from_numpy(inp["v_hist"])
    r = w.n_q_heads // w.n_kv_heads
    k_all = torch.cat([kh, ks], 1).repeat_interleave(r, 0)
    v_all = torch.cat([vh, vs], 1).repeat_interleave(r, 0)
    H, S = w.hist_len, w.seg_len
    allowed = torch.arange(H + S)[None, :] <= (H + torch.arange(S))[:, None]
    out = F.scaled_dot_product_attention(q, k_all, v_all, attn_mask=allowed,
                                         scale=w.softmax_scale)
    (out * torch.from_numpy(inp["d_o"])).sum().backward()
    assert np.max(np.abs(q.grad.numpy() - dQ)) < 1e-12
    assert np.max(np.abs(ks.grad.numpy() - dK)) < 1e-12
    assert np.max(np.abs(vs.grad.numpy() - dV)) < 1e-12


# ---------------------------------------------------------------------------
# sink and local window: explicit key sets, closed forms, autograd
# ---------------------------------------------------------------------------
def _mask_sink_window(sel_groups, n_q, n_kv, H, S, n_sink_tokens, W):
    """allowed[h, i, t]: history token t < n_sink_tokens, or in a group selected
    for (i//64, h//r); segment token t = H + u with i - W < u <= i."""
    r = n_q // n_kv
    allowed = np.zeros((n_q, S, H + S), bool)
    for h in range(n_q):
        for i in range(S):
            allowed[h, i, :min(n_sink_tokens, H)] = True
            for n in sel_groups[i // 64, h // r]:
                if n >= 0:
                    allowed[h, i, 8 * n: 8 * n + 8] = True
            allowed[h, i, H + max(0, i - W + 1): H + i + 1] = True
    return allowed


@pytest.mark.parametrize("n_sink,W", [(1, 128), (2, 64), (0, 96), (3, 1), (8, 200)])
def test_sink_and_window_match_explicit_key_sets(n_sink, W):
    w = _small(seg_len=192)
    inp = _np(synth.make_inputs(w, seed=20 + n_sink))
    sel_c, sel_g, aux = orc.route(inp["q"], inp["k_hist"], 2, 3, 6, n_sink=n_sink)
    O, LSE = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"],
                          sel_g, w.softmax_scale, n_sink_tokens=64 * n_sink, window=W)
    allowed = _mask_sink_window(sel_g, w.n_q_heads, w.n_kv_heads, w.hist_len, w.seg_len,
                                64 * n_sink, W)
    k_all = np.concatenate([inp["k_hist"], inp["k_seg"]], axis=1)
    v_all = np.concatenate([inp["v_hist"], inp["v_seg"]], axis=1)
    ref, ref_lse = _sdpa_with_key_mask(inp["q"], k_all, v_all, allowed, w.softmax_scale)
    assert np.max(np.abs(O - ref)) < 1e-12
    assert np.max(np.abs(LSE - ref_lse)) < 1e-12


def test_sink_chunks_are_never_routed():
    # the history's best chunk lies inside the sink: routing must pick others
    w = _small(hist_len=512, n_kv_heads=1, n_q_heads=1, seg_len=64)
    inp = _np(synth.make_inputs(w, seed=30))
    qbar = orc.block_queries(inp["q"], 1)[0, 0]
    kh = inp["k_hist"].copy()
    kh[0, 0:64] += 50.0 * qbar / np.linalg.norm(qbar)      # chunk 0: best by far
    sel_c0, _, _ = orc.route(inp["q"], kh, 1, 3, 6)
    assert 0 in sel_c0[0, 0]
    sel_c, sel_g, aux = orc.route(inp["q"], kh, 1, 3, 6, n_sink=2)
    ids = [int(x) for x in sel_c[0, 0] if x >= 0]
    assert len(ids) == 3 and min(ids) >= 2
    # the same selection as ranking the non-sink chunks by brute force
    sc = aux["chunk_scores"][0, 0]
    ref = sorted(sorted(range(2, 8), key=lambda m: (-sc[m], m))[:3])
    assert ids == ref
    assert all(int(n) // 8 >= 2 for n in sel_g[0, 0] if n >= 0)


def test_sink_longer_than_history_routes_nothing():
    w = _small(hist_len=128)
    inp = _np(synth.make_inputs(w, seed=31))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 3, 6, n_sink=4)
    assert (sel_c == -1).all() and (sel_g == -1).all()


def test_window_of_one_attends_only_itself_closed_form():
    # no history, W = 1: each query sees exactly its own key, so O = V_i and
    # LSE = scale * q_i . k_i
    w = _small(hist_len=0)
    inp = _np(synth.make_inputs(w, seed=32))
    sel = np.full((w.seg_len // 64, w.n_kv_heads, 6), -1, np.int32)
    O, LSE = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"],
                          sel, w.softmax_scale, window=1)
    r = w.n_q_heads // w.n_kv_heads
    for h in range(w.n_q_heads):
        assert np.max(np.abs(O[h] - inp["v_seg"][h // r])) < 1e-15
        lse = w.softmax_scale * np.einsum("sd,sd->s", inp["q"][h], inp["k_seg"][h // r])
        assert np.max(np.abs(LSE[h] - lse)) < 1e-12


def test_window_covering_the_segment_changes_nothing():
    w = _small()
    inp = _np(synth.make_inputs(w, seed=33))
    _, sel, _ = orc.route(inp["q"], inp["k_hist"], 2, 3, 6)
    a = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"], sel,
                     w.softmax_scale)
    b = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"], sel,
                     w.softmax_scale, window=w.seg_len)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("n_sink,W", [(2, 64), (1, 100)])
def test_backward_with_sink_and_window_matches_torch_autograd(n_sink, W):
    w = _small(seg_len=192)
    inp = _np(synth.make_inputs(w, seed=40 + W))
    _, sel, _ = orc.route(inp["q"], inp["k_hist"], 2, 3, 6, n_sink=n_sink)
    dQ, dK, dV = orc.attn_bwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"],
                              sel, w.softmax_scale, inp["d_o"], n_sink_tokens=64 * n_sink, window=W)
    q = torch.from_numpy(inp["q"]).requires_grad_(True)
    ks = torch.from_numpy(inp["k_seg"]).requires_grad_(True)
    vs = torch.from_numpy(inp["v_seg"]).requires_grad_(True)
    r = w.n_q_heads // w.n_kv_heads
    k_all = torch.cat([torch.from_numpy(inp["k_hist"]), ks], 1).repeat_interleave(r, 0)
    v_all = torch.cat([torch.from_numpy(inp["v_hist"]), vs], 1).repeat_interleave(r, 0)
    allowed = torch.from_numpy(_mask_sink_window(sel, w.n_q_heads, w.n_kv_heads, w.hist_len,
                                                 w.seg_len, 64 * n_sink, W))
    out = F.scaled_dot_product_attention(q, k_all, v_all, attn_mask=allowed, scale=w.softmax_scale)
    (out * torch.from_numpy(inp["d_o"])).sum().backward()
    assert np.max(np.abs(q.grad.numpy() - dQ)) < 1e-12
    assert np.max(np.abs(ks.grad.numpy() - dK)) < 1e-12
    assert np.max(np.abs(vs.grad.numpy() - dV)) < 1e-12


def test_selection_checker_honours_the_sink():
    w = _small()
    inp = _np(synth.make_inputs(w, seed=34))
    sel_c, sel_g, aux = orc.route(inp["q"], inp["k_hist"], 2, 3, 6, n_sink=2)
    ok = orc.check_selection(aux["qbar"], aux["C"], aux["G"], sel_c, sel_g, 3, 6, n_sink=2)
    assert ok["ok"]
    bad = sel_c.copy()
    bad[0, 0, 0] = 0                                   # a sink chunk may not be routed
    bad[0, 0] = np.sort(bad[0, 0])
    assert not orc.check_selection(aux["qbar"], aux["C"], aux["G"], bad, sel_g, 3, 6,
                                   n_sink=2)["ok"]


# ---------------------------------------------------------------------------
# the parity criteria: selection checker and non-vacuous output tolerance
# ---------------------------------------------------------------------------
def test_selection_checker_accepts_oracle_and_rejects_clear_swaps():
    w = synth.WORKLOADS["tiny_f32"]
    inp = _np(synth.make_inputs(w, seed=16))
    sel_c, sel_g, aux = orc.route(inp["q"], inp["k_hist"], 1, 4, 8)
    rep = orc.check_selection(aux["qbar"], aux["C"], aux["G"], sel_c, sel_g, 4, 8)
    assert rep["ok"] and rep["chunk_exemptions"] == 0 and rep["group_exemptions"] == 0
    # replace the best chunk by the worst one: far from a tie, must be rejected
    sc = aux["chunk_scores"][0, 0]
    bad_c = sel_c.copy()
    row = set(bad_c[0, 0].tolist())
    row.discard(int(np.argmax(sc)))
    row.add(int(np.argmin(sc)))
    bad_c[0, 0] = sorted(row)
    assert not orc.check_selection(aux["qbar"], aux["C"], aux["G"], bad_c, sel_g, 4, 8)["ok"]
    # a group outside the selected chunks must be rejected
    bad_g = sel_g.copy()
    outside = [n for n in range(128) if n // 8 not in sel_c[0, 0]][0]
    bad_g[0, 0, 0] = outside
    bad_g[0, 0] = np.sort(bad_g[0, 0])
    assert not orc.check_selection(aux["qbar"], aux["C"], aux["G"], sel_c, bad_g, 4, 8)["ok"]


def test_selection_checker_accepts_an_exact_tie_swap():
    n_kv, H, d = 1, 1024, 8
    k = np.ones((n_kv, H, d))
    q = np.ones((2, 128, d))
    sel_c, sel_g, aux = orc.route(q, k, 1, 4, 8)
    alt = sel_c.copy()
    alt[0, 0] = [0, 1, 2, 15]                  # chunk 15 ties chunk 3 exactly
    alt_g = sel_g.copy()
    rep = orc.check_selection(aux["qbar"], aux["C"], aux["G"], alt, alt_g, 4, 8)
    assert rep["ok"] and rep["chunk_exemptions"] == 1


def test_output_tolerance_is_not_vacuous():
    """At Qwen3-8B-like magnitudes |O| is ~2e-2, the size of the plain 2e-2
    max-abs bar itself, so that bar alone barely separates a correct output
    from an all-zero one. The relative part of the criterion must reject the
    zero output, dense attention, local-only attention and selections shifted
    by one chunk (forward, and dQ / dK of the backward), and accept the
    reference rounded to bf16."""
    w = synth.Workload("neg", 8, 2, 128, 2048, 256, 8, 16, "bf16", 1 / math.sqrt(128),
                       backward=True)
    inp = _np(synth.make_inputs(w, seed=17))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 8, 16)
    args = (inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"])
    ref, _ = orc.attn_fwd(*args, sel_g, w.softmax_scale)
    tol = 2e-2
    assert np.abs(ref).max() < 0.05
    rounded = torch.from_numpy(ref).bfloat16().double().numpy()
    assert orc.within_tolerance(rounded, ref, tol)
    assert not orc.within_tolerance(np.zeros_like(ref), ref, tol)
    all_groups = np.ascontiguousarray(
        np.broadcast_to(np.arange(w.hist_len // 8), sel_g.shape[:2] + (w.hist_len // 8,)))
    shifted = np.sort((sel_g + 8) % (w.hist_len // 8), axis=-1)
    none = np.full_like(sel_g, -1)
    for sel in (all_groups, none, shifted):
        wrong, _ = orc.attn_fwd(*args, sel, w.softmax_scale)
        assert not orc.within_tolerance(wrong, ref, tol)
    g_ref = orc.attn_bwd(*args, sel_g, w.softmax_scale, inp["d_o"])
    for sel in (all_groups, shifted):
        g_bad = orc.attn_bwd(*args, sel, w.softmax_scale, inp["d_o"])
        for i in (0, 1):                                 # dQ, dK
            assert not orc.within_tolerance(g_bad[i], g_ref[i], tol)
        assert orc.within_tolerance(torch.from_numpy(g_ref[i]).bfloat16().double().numpy(),
                                    g_ref[i], tol)


# ---------------------------------------------------------------------------
# decode step: pinned to the training block, to SDPA and to a closed form
# ---------------------------------------------------------------------------
def test_decode_query_mean_closed_form():
    # q[h][i] = (h * n_new + i) * 1 -> mean over the r heads of KV head j and
    # the n_new rows = j * r * n_new + (r * n_new - 1) / 2
    n_q, n_kv, n_new, d = 6, 2, 3, 8
    q = np.zeros((n_q, n_new, d))
    for h in range(n_q):
        for i in range(n_new):
            q[h, i] = h * n_new + i
    qbar = orc.decode_query_mean(q, n_kv)
    r = n_q // n_kv
    for j in range(n_kv):
        assert np.all(qbar[j] == np.float32(j * r * n_new + (r * n_new - 1) / 2))


def test_decode_of_a_full_block_equals_the_training_block():
    # 64 new tokens at the end of a 128-token open segment are query block 1
    # of training with that segment: same routing, same outputs
    w = _small(hist_len=512, seg_len=128, top_k_chunks=3, top_k_groups=6)
    inp = _np(synth.make_inputs(w, seed=31))
    sel_c, sel_g, _ = orc.route(inp["q"], inp["k_hist"], 2, 3, 6, n_sink=1)
    O, LSE = orc.attn_fwd(inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"],
                          sel_g, w.softmax_scale, n_sink_tokens=64, window=100)
    dc, dg, Od, Ld = orc.decode_step(inp["q"][:, 64:], inp["k_hist"], inp["v_hist"], inp["k_seg"],
                                     inp["v_seg"], 3, 6, w.softmax_scale, n_sink=1, window=100)
    assert np.array_equal(dc, sel_c[1]) and np.array_equal(dg, sel_g[1])
    assert np.max(np.abs(Od - O[:, 64:])) < 1e-12 and np.max(np.abs(Ld - LSE[:, 64:])) < 1e-12


@pytest.mark.parametrize("T,n_new,n_sink,W", [(77, 1, 0, None), (77, 3, 1, 20), (5, 2, 2, 3),
                                              (130, 4, 0, 1)])
def test_decode_matches_sdpa_with_explicit_keys(T, n_new, n_sink, W):
    # ragged open segment; keys: sink, selected groups, window of the open
    # segment ending at each new token
    rng = np.random.default_rng(T * 7 + n_new)
    n_q, n_kv, d, H = 4, 2, 16, 512
    q = rng.standard_normal((n_q, n_new, d))
    kh, vh = rng.standard_normal((n_kv, H, d)), rng.standard_normal((n_kv, H, d))
    kt, vt = rng.standard_normal((n_kv, T, d)), rng.standard_normal((n_kv, T, d))
    scale = 0.25
    sc, sg, O, LSE = orc.decode_step(q, kh, vh, kt, vt, 3, 7, scale, n_sink=n_sink, window=W)
    r = n_q // n_kv
    Wd = T if W is None else W
    allowed = np.zeros((n_q, n_new, H + T), bool)
    for h in range(n_q):
        for i in range(n_new):
            allowed[h, i, :64 * n_sink] = True
            for n in sg[h // r]:
                if n >= 0:
                    allowed[h, i, 8 * n:8 * n + 8] = True
            p = T - n_new + i
            allowed[h, i, H + max(0, p - Wd + 1):H + p + 1] = True
    ref, ref_lse = _sdpa_with_key_mask(q, np.concatenate([kh, kt], 1), np.concatenate([vh, vt], 1),
                                       allowed, scale)
    assert np.max(np.abs(O - ref)) < 1e-12 and np.max(np.abs(LSE - ref_lse)) < 1e-12
    # the sink is never routed; routed groups lie inside routed chunks
    assert (sc[sc >= 0] >= n_sink).all()
    for j in range(n_kv):
        assert set(int(g) // 8 for g in sg[j] if g >= 0) <= set(int(c) for c in sc[j] if c >= 0)


def test_decode_full_budget_is_dense_causal_attention():
    rng = np.random.default_rng(3)
    n_q, n_kv, d, H, T, n_new = 4, 1, 16, 256, 40, 2
    q = rng.standard_normal((n_q, n_new, d))
    kh, vh = rng.standard_normal((n_kv, H, d)), rng.standard_normal((n_kv, H, d))
    kt, vt = rng.standard_normal((n_kv, T, d)), rng.standard_normal((n_kv, T, d))
    sc, sg, O, LSE = orc.decode_step(q, kh, vh, kt, vt, 4, 32, 0.3)
    assert (sg[0] == np.arange(32)).all()
    pos = H + T - n_new + np.arange(n_new)[:, None]
    allowed = np.broadcast_to(np.arange(H + T)[None, :] <= pos, (n_q, n_new, H + T)).copy()
    ref, ref_lse = _sdpa_with_key_mask(q, np.concatenate([kh, kt], 1), np.concatenate([vh, vt], 1),
                                       allowed, 0.3)
    assert np.max(np.abs(O - ref)) < 1e-12 and np.max(np.abs(LSE - ref_lse)) < 1e-12


def test_decode_without_history_attends_the_open_segment():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 1, 8))
    kt, vt = rng.standard_normal((1, 9, 8)), rng.standard_normal((1, 9, 8))
    empty = np.zeros((1, 0, 8))
    sc, sg, O, _ = orc.decode_step(q, empty, empty, kt, vt, 2, 4, 1.0)
    assert (sc == -1).all() and (sg == -1).all()
    for h in range(2):
        s = kt[0] @ q[h, 0]
        p = np.exp(s - s.max())
        assert np.allclose(O[h, 0], p @ vt[0] / p.sum(), rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# localized errors: the per-slice part of the criterion and the LSE bar
# ---------------------------------------------------------------------------
def test_one_wrong_slice_fails_among_a_thousand():
    """32 heads x 32 query blocks, as at the Qwen3-8B layer: one (head, block)
    slice 50% off moves the whole-tensor relative L2 by only ~1.6%, under the
    2e-2 bar, so only the per-slice part catches it; so do 8 zeroed rows of
    one slice and a single row with its sign flipped."""
    rng = np.random.default_rng(21)
    ref = 0.01 * rng.standard_normal((32, 2048, 16))
    tol = 2e-2
    assert orc.within_tolerance(torch.from_numpy(ref).bfloat16().double().numpy(), ref, tol)
    bad = ref.copy()
    bad[3, 5 * 64:6 * 64] *= 1.5
    assert orc.error_stats(bad, ref)[1] < tol          # the whole-tensor part alone passes
    assert not orc.within_tolerance(bad, ref, tol)
    rows = ref.copy()
    rows[17, 64 * 30 + 3:64 * 30 + 11] = 0.0
    assert orc.error_stats(rows, ref)[1] < tol
    assert not orc.within_tolerance(rows, ref, tol)
    flip = ref.copy()
    flip[0, 2047] *= -1.0
    assert not orc.within_tolerance(flip, ref, tol)
    sl = orc.slice_rel_l2(bad, ref)
    assert sl.shape == (32, 32) and sl[3, 5] == pytest.approx(0.5, rel=0.1)
    assert np.delete(sl.ravel(), 3 * 32 + 5).max() == 0


def test_slices_follow_the_head_and_block_axes():
    # LSE-like [n][T] arrays and ragged T: the last slice is the partial run
    ref = np.ones((2, 130))
    got = ref.copy()
    got[1, 64:128] = 1.25
    sl = orc.slice_rel_l2(got, ref)
    assert sl.shape == (2, 3)
    assert sl[1, 1] == pytest.approx(0.25) and sl[0].max() == 0 and sl[1, 0] == 0 and sl[1, 2] == 0
    # a slice far smaller than the typical one is measured against the
    # root-mean-square slice norm (here 8: 64 ones per slice)
    got = ref.copy()
    got[1, 128:] = 2.0                                   # the 2-row tail, 100% off
    sl = orc.slice_rel_l2(got, ref)
    rms = math.sqrt((64 + 64 + 2) / 3)
    assert sl[1, 2] == pytest.approx(math.sqrt(2) / rms)


def test_small_slices_admit_bf16_rounding_of_o_and_ds():
    """With no history and a 70-token window, the first query block's rows see
    1..64 keys that share one chunk offset, and dQ cancels that offset almost
    exactly. Rounding the forward output O (which enters dS through
    D = dO . O) and dS itself to bf16, as a bf16 kernel stores and multiplies
    them, then moves those slices by ~2% of their own norm (half the typical
    slice norm); the criterion must accept that rounding and still reject a
    5%-wrong slice there."""
    w = synth.Workload("bf16_nohist_w70", 4, 2, 128, 0, 256, 4, 8, "bf16", 1 / math.sqrt(128),
                       backward=True, n_sink_chunks=2, local_window=70)
    a = _np(synth.make_inputs(w, seed=3, with_grad_out=True))
    sel = np.full((4, 2, 8), -1, np.int32)
    dQ, _, _ = orc.attn_bwd(a["q"], a["k_hist"], a["v_hist"], a["k_seg"], a["v_seg"], sel,
                            w.softmax_scale, a["d_o"], window=70)

    def bf(x):
        return torch.from_numpy(np.asarray(x)).to(torch.bfloat16).double().numpy()

    rounded = np.zeros_like(dQ)
    for h in range(4):
        for b in range(4):
            rows = slice(64 * b, 64 * b + 64)
            Kc, Vc, nh, loc0, nl = orc._block_keys(a["k_hist"], a["v_hist"], a["k_seg"], a["v_seg"],
                                                   sel, b, h // 2, 0, 70)
            P, _ = orc._block_probs(a["q"][h, rows], Kc, nh, loc0, nl, b, w.softmax_scale, 70)
            D = (a["d_o"][h, rows] * bf(P @ Vc)).sum(axis=1, keepdims=True)
            dS = bf(P * (a["d_o"][h, rows] @ Vc.T - D))
            rounded[h, rows] = w.softmax_scale * (dS @ Kc)
    own = max(np.linalg.norm(rounded[h, :64] - dQ[h, :64]) / np.linalg.norm(dQ[h, :64]) for h in range(4))
    assert own > 0.01                                    # the effect is real
    assert orc.within_tolerance(rounded, dQ, 2e-2)
    # an error of 5% of the typical slice norm, placed in a small first-block slice
    rms = np.sqrt(np.mean([np.sum(dQ[h, 64 * s:64 * s + 64] ** 2) for h in range(4) for s in range(4)]))
    bad = dQ.copy()
    bad[0, :64] += 0.05 * rms * dQ[0, :64] / np.linalg.norm(dQ[0, :64])
    assert not orc.within_tolerance(bad, dQ, 2e-2)


def test_lse_is_held_to_the_fp32_bar():
    rng = np.random.default_rng(22)
    ref = 7.0 + rng.standard_normal((8, 256))
    assert orc.lse_within(ref.astype(np.float32).astype(np.float64), ref)
    off = ref.copy()
    off[2, 100] += 2e-3                                   # 2.5e-4 relative at |LSE| ~ 8
    assert not orc.lse_within(off, ref)
    # bf16 rounding of an LSE of ~7 moves it by up to 0.016: far outside the bar
    assert not orc.lse_within(torch.from_numpy(ref).bfloat16().double().numpy(), ref)
    small = np.full((1, 4), 0.25)
    assert orc.lse_within(small + 0.9e-4, small) and not orc.lse_within(small + 1.1e-4, small)


# ---------------------------------------------------------------------------
# routing with several KV heads: brute force and per-head plants
# ---------------------------------------------------------------------------
def _bruteforce_route(q, k, n_kv, k_c, k_g):
    """Route written out with Python loops over explicit head lists, float64
    arithmetic and full sorts: query head h belongs to KV head h // r; the
    block query of (b, j) averages rows 64b..64b+63 of heads jr..jr+r-1; chunk
    m averages keys 64m..64m+63 of KV head j; ranking is higher score, then
    lower index."""
    n_q, S, d = q.shape
    H = k.shape[1]
    r = n_q // n_kv
    n_B, n_C = S // 64, H // 64
    sel_c = np.full((n_B, n_kv, k_c), -1, np.int64)
    sel_g = np.full((n_B, n_kv, k_g), -1, np.int64)
    for b in range(n_B):
        for j in range(n_kv):
            heads = [h for h in range(n_q) if h // r == j]
            qb = [sum(float(q[h, i, e]) for h in heads for i in range(64 * b, 64 * b + 64)) / (64 * len(heads))
                  for e in range(d)]
            def score(lo, n):
                return sum(qb[e] * sum(float(k[j, t, e]) for t in range(lo, lo + n)) / n for e in range(d))
            ranked = sorted(range(n_C), key=lambda m: (-score(64 * m, 64), m))[:k_c]
            chunks = sorted(ranked)
            sel_c[b, j, :len(chunks)] = chunks
            cand = [8 * m + u for m in chunks for u in range(8)]
            top = sorted(sorted(cand, key=lambda n: (-score(8 * n, 8), n))[:k_g])
            sel_g[b, j, :len(top)] = top
    return sel_c, sel_g


@pytest.mark.parametrize("n_q,n_kv", [(6, 3), (4, 2), (8, 2)])
def test_route_several_kv_heads_matches_bruteforce(n_q, n_kv):
    """Small-integer inputs keep every sum exact in float32 and float64 alike,
    so the oracle's selections must equal the brute force's for every
    (block, KV head), ties (frequent with so few values) included."""
    rng = np.random.default_rng(n_q * 10 + n_kv)
    d, H, S = 4, 512, 128
    q = rng.integers(0, 3, (n_q, S, d)).astype(np.float64)
    k = rng.integers(-1, 3, (n_kv, H, d)).astype(np.float64)
    k[:, 64 * 2:64 * 3] = 1.0                 # whole-chunk ties across heads
    k[:, 64 * 5:64 * 6] = 1.0
    got_c, got_g, _ = orc.route(q, k, n_kv, 3, 5)
    want_c, want_g = _bruteforce_route(q, k, n_kv, 3, 5)
    assert np.array_equal(got_c, want_c)
    assert np.array_equal(got_g, want_g)


def test_route_planted_chunk_differs_per_kv_head():
    """KV head j gets its own planted chunk m_j and group g_j along its own
    query direction u_j; every block of head j must route to exactly them
    (top-1 chunk, top-1 group) and never to another head's plant."""
    n_q, n_kv, d, H, S = 6, 3, 16, 1024, 192
    rng = np.random.default_rng(23)
    q = 0.1 * rng.standard_normal((n_q, S, d))
    k = 0.1 * rng.standard_normal((n_kv, H, d))
    u = np.linalg.qr(rng.standard_normal((d, n_kv)))[0].T          # orthonormal directions
    plant_c, plant_g = [3, 11, 7], [3 * 8 + 5, 11 * 8 + 0, 7 * 8 + 7]
    for h in range(n_q):
        q[h] += 2.0 * u[h // (n_q // n_kv)]
    for j in range(n_kv):
        k[j, 64 * plant_c[j]:64 * plant_c[j] + 64] += 3.0 * u[j]
        k[j, 8 * plant_g[j]:8 * plant_g[j] + 8] += 3.0 * u[j]
    sel_c, sel_g, aux = orc.route(q, k, n_kv, 1, 1)
    for b in range(S // 64):
        for j in range(n_kv):
            assert sel_c[b, j].tolist() == [plant_c[j]]
            assert sel_g[b, j].tolist() == [plant_g[j]]
            assert int(np.argmax(aux["chunk_scores"][b, j])) == plant_c[j]
