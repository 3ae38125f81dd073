"""CPU oracle for the HGA route + exact-token attention path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module. The product path (the HIP library
and its Python binding) never calls it, and it shares no code with them: it
reads plain numpy arrays and computes every step with plain loops and library
primitives (sum, matmul, sort), in the order the pages describe the method.

Sources (all five pages share the title "Long-Context Fine-Tuning with Limited
VRAM"):
  [gist 2.1]  gist.science, Technical Summary §2.1 "Hierarchical Global
              Attention (HGA)": chunk selection over 64-token chunk summaries,
              group selection over 8-token group summaries inside the chosen
              chunks, exact-token attention over the selected groups, routing
              without gradient, no router weights.
  [gist 2.2]  same page, §2.2 "Segment-wise Backward and Tiered Storage":
              history K/V is detached at the segment boundary.
  [pith F1]   pith.science review, Figure 1 caption: summaries select regions,
              the final attention uses exact token K/V only.
  [pith core] pith.science review, "Core claim": the router is built from the
              model's projected keys; only exact K/V of selected groups enter
              the working set.

Readings where the pages are silent (each listed in the design notes):
  * summary vector = arithmetic mean of the keys of the chunk / group;
  * block query = mean of the block's 64 queries over the r query heads that
    share one KV head (grouped-query attention, head h uses KV head h // r);
  * score = unscaled fp32 dot product, no softmax;
  * top-k order = score descending, then index ascending (lowest index wins a
    tie); NaN counts as -inf, -0 equals +0;
  * selections are emitted in ascending index order, padded with -1;
  * every history chunk (all lie before the segment) is eligible, except the
    sink: the first n_sink history chunks are attended in full by every query
    (the "fixed sink" window beside the routed chunks [gist 2.1]) and are
    therefore not ranked, so no token is counted twice;
  * the local window is the W most recent segment tokens, causal: query i
    attends segment keys t with i - W < t <= i (W = S by default, the whole
    segment); routing covers the closed history only, so with W < S older
    segment tokens are not attended;
  * the gathered history is detached: no gradient reaches K_hist / V_hist.

Precision: the routing decisions (summaries, block queries, scores) are taken
in float32, the precision the kernels decide them in; attention forward and
backward run in float64.

Decode: the step's query block is the n_new newest tokens (their mean query
routes); the open segment (not yet summarised) plays the role of the active
segment, and the history is every closed chunk.

Parity pins live in tests/test_oracle.py (dense-attention equivalence through
torch's SDPA, brute-force top-k, closed forms, finite differences). No function
here is left unpinned.
"""
from __future__ import annotations

import numpy as np

CHUNK = 64     # tokens per chunk [gist 2.1]
GROUP = 8      # tokens per group [gist 2.1]
BLOCK = 64     # queries per routed query block (one routing decision)

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------
# Summaries [gist 2.1 "Chunk Selection" / "Group Selection"; pith core]
# ---------------------------------------------------------------------------
def _segmented_mean(k_hist: np.ndarray, width: int) -> np.ndarray:
    """Mean over consecutive runs of ``width`` tokens, summed in token order."""
    n_kv, H, d = k_hist.shape
    if H % width:
        raise ValueError(f"history length {H} is not a multiple of {width}")
    k = np.asarray(k_hist, dtype=F32).reshape(n_kv, H // width, width, d)
    acc = np.zeros((n_kv, H // width, d), dtype=F32)
    for u in range(width):                 # sequential sum over the run
        acc += k[:, :, u, :]
    return acc * F32(1.0 / width)


def chunk_summaries(k_hist: np.ndarray) -> np.ndarray:
    """C[j][m] = mean of K_hist[j][64m .. 64m+63]; float32 [n_kv][H/64][d]."""
    return _segmented_mean(k_hist, CHUNK)


def group_summaries(k_hist: np.ndarray) -> np.ndarray:
    """G[j][n] = mean of K_hist[j][8n .. 8n+7]; float32 [n_kv][H/8][d]."""
    return _segmented_mean(k_hist, GROUP)


# ---------------------------------------------------------------------------
# Block query [gist 2.1 "the current query block scores these summaries"]
# ---------------------------------------------------------------------------
def block_queries(q: np.ndarray, n_kv: int) -> np.ndarray:
    """qbar[b][j] = mean of Q[h][64b .. 64b+63] over the r heads h of KV head j.

    Returns float32 [S/64][n_kv][d].
    """
    n_q, S, d = q.shape
    if n_q % n_kv or S % BLOCK:
        raise ValueError("bad query shape")
    r = n_q // n_kv
    qq = np.asarray(q, dtype=F32).reshape(n_kv, r, S // BLOCK, BLOCK, d)
    acc = np.zeros((n_kv, S // BLOCK, d), dtype=F32)
    for h in range(r):
        for i in range(BLOCK):
            acc += qq[:, h, :, i, :]
    acc *= F32(1.0 / (BLOCK * r))
    return np.ascontiguousarray(acc.transpose(1, 0, 2))


# ---------------------------------------------------------------------------
# Top-k with lowest-index tie-break
# ---------------------------------------------------------------------------
def topk_lowest_index(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k best scores: score descending, index ascending on ties.

    NaN ranks as -inf; -0 and +0 compare equal. Returned in ascending index
    order (the selection is a set; ascending keeps later gathers monotone).
    """
    s = np.asarray(scores, dtype=F32).copy()
    s[np.isnan(s)] = -np.inf
    idx = np.arange(s.shape[0])
    order = np.lexsort((idx, -s))          # primary: -score, secondary: index
    return np.sort(order[: min(k, s.shape[0])])


def chunk_scores(qbar: np.ndarray, C: np.ndarray) -> np.ndarray:
    """sc[b][j][m] = qbar[b][j] . C[j][m] in float32; [n_B][n_kv][n_C]."""
    n_B, n_kv, d = qbar.shape
    out = np.empty((n_B, n_kv, C.shape[1]), dtype=F32)
    for j in range(n_kv):
        out[:, j, :] = np.asarray(qbar[:, j, :], F32) @ np.asarray(C[j], F32).T
    return out


def route_chunks(qbar: np.ndarray, C: np.ndarray, k_c: int, n_sink: int = 0):
    """Chunk selection [gist 2.1 "Chunk Selection"].

    Every history chunk precedes the active segment; the candidates are the
    chunks after the sink, m in [n_sink, n_C), for every query block (the sink
    chunks are attended in full anyway). Returns (sel int32 [n_B][n_kv][k_c]
    ascending, -1 padded; scores float32 [n_B][n_kv][n_C] of all chunks).
    """
    sc = chunk_scores(qbar, C)
    n_B, n_kv, n_C = sc.shape
    s0 = min(n_sink, n_C)
    sel = np.full((n_B, n_kv, k_c), -1, dtype=np.int32)
    for b in range(n_B):
        for j in range(n_kv):
            top = s0 + topk_lowest_index(sc[b, j, s0:], k_c)
            sel[b, j, : top.shape[0]] = top
    return sel, sc


def group_candidates(chunks: np.ndarray) -> np.ndarray:
    """Groups 8m .. 8m+7 of every selected chunk m (ascending chunks)."""
    ch = [int(m) for m in chunks if m >= 0]
    return np.array([8 * m + u for m in ch for u in range(CHUNK // GROUP)],
                    dtype=np.int64)


def route_groups_one(qbar_bj: np.ndarray, G_j: np.ndarray, chunks: np.ndarray,
                     k_g: int):
    """Group selection for one (query block, KV head) [gist 2.1 "Group Selection"].

    Returns (selected group ids ascending, candidate ids, candidate scores).
    """
    cand = group_candidates(chunks)
    if cand.shape[0] == 0:
        return cand.astype(np.int32), cand, np.zeros(0, F32)
    sg = np.asarray(G_j[cand], F32) @ np.asarray(qbar_bj, F32)
    top = topk_lowest_index(sg, k_g)       # positions in cand (ascending)
    return cand[top].astype(np.int32), cand, sg


def route_groups(qbar: np.ndarray, G: np.ndarray, sel_chunks: np.ndarray, k_g: int):
    """sel_groups int32 [n_B][n_kv][k_g], ascending, -1 padded."""
    n_B, n_kv, _ = sel_chunks.shape
    sel = np.full((n_B, n_kv, k_g), -1, dtype=np.int32)
    for b in range(n_B):
        for j in range(n_kv):
            g, _, _ = route_groups_one(qbar[b, j], G[j], sel_chunks[b, j], k_g)
            sel[b, j, : g.shape[0]] = g
    return sel


def route(q, k_hist, n_kv, k_c, k_g, n_sink: int = 0):
    """The whole routing step from raw inputs: summaries, block queries,
    chunk top-k, group top-k. Returns (sel_chunks, sel_groups, aux)."""
    C = chunk_summaries(k_hist)
    G = group_summaries(k_hist)
    qbar = block_queries(q, n_kv)
    sel_c, sc = route_chunks(qbar, C, k_c, n_sink)
    sel_g = route_groups(qbar, G, sel_c, k_g)
    return sel_c, sel_g, dict(C=C, G=G, qbar=qbar, chunk_scores=sc)


# ---------------------------------------------------------------------------
# Exact-token attention [gist 2.1 "Exact-Token Attention"; pith F1]
# ---------------------------------------------------------------------------
def attended_history_tokens(sel_groups_bj: np.ndarray, n_sink_tokens: int = 0) -> np.ndarray:
    """History token ids: the sink tokens 0 .. n_sink_tokens-1, then
    8n .. 8n+7 of every selected group n >= 0."""
    return np.array(list(range(n_sink_tokens)) +
                    [GROUP * int(n) + u for n in sel_groups_bj if n >= 0
                     for u in range(GROUP)], dtype=np.int64)


def _window(window, S):
    return S if window is None or window <= 0 else min(int(window), S)


def _block_keys(k_hist, v_hist, k_seg, v_seg, sel_groups, b, j, n_sink_tokens=0, window=None):
    """Keys of query block b: the history tokens, then the segment keys any
    of its 64 rows may attend, [loc0, 64b+63]."""
    hist = attended_history_tokens(sel_groups[b, j], min(n_sink_tokens, k_hist.shape[1]))
    W = _window(window, k_seg.shape[1])
    loc0 = max(0, BLOCK * b - W + 1)
    loc1 = BLOCK * (b + 1)
    Kc = np.concatenate([np.asarray(k_hist[j][hist], F64),
                         np.asarray(k_seg[j][loc0:loc1], F64)], axis=0)
    Vc = np.concatenate([np.asarray(v_hist[j][hist], F64),
                         np.asarray(v_seg[j][loc0:loc1], F64)], axis=0)
    return Kc, Vc, hist.shape[0], loc0, loc1 - loc0


def _block_probs(Qb, Kc, n_hist, loc0, n_loc, b, scale, W):
    """Softmax over [history || segment window] for 64 query rows: row i may
    attend segment key t iff i - W < t <= i."""
    s = scale * (Qb @ Kc.T)                          # (64, n_hist + n_loc)
    qpos = BLOCK * b + np.arange(BLOCK)[:, None]     # segment position of row
    kpos = loc0 + np.arange(n_loc)[None, :]
    allowed = np.concatenate([np.ones((BLOCK, n_hist), bool),
                              (kpos <= qpos) & (kpos > qpos - W)], axis=1)
    s = np.where(allowed, s, -np.inf)
    M = s.max(axis=1, keepdims=True)
    e = np.exp(s - M)
    ell = e.sum(axis=1, keepdims=True)
    return e / ell, (M + np.log(ell))[:, 0]


def attn_fwd(q, k_hist, v_hist, k_seg, v_seg, sel_groups, scale, n_sink_tokens=0, window=None):
    """O[h][i] = softmax(scale * Q[h][i] . K_t) weighted sum of V_t over
    t in {sink tokens} U {selected history tokens of block i//64, KV head h//r}
    U {segment keys i-W+1 .. i} (W = window, default the whole segment).

    Returns (O float64 [n_q][S][d], LSE float64 [n_q][S]).
    """
    n_q, S, d = q.shape
    n_kv = k_seg.shape[0]
    r = n_q // n_kv
    O = np.zeros((n_q, S, d), F64)
    LSE = np.zeros((n_q, S), F64)
    for h in range(n_q):
        j = h // r
        for b in range(S // BLOCK):
            Kc, Vc, n_hist, loc0, n_loc = _block_keys(k_hist, v_hist, k_seg, v_seg, sel_groups,
                                                      b, j, n_sink_tokens, window)
            Qb = np.asarray(q[h, BLOCK * b: BLOCK * (b + 1)], F64)
            P, lse = _block_probs(Qb, Kc, n_hist, loc0, n_loc, b, scale, _window(window, S))
            O[h, BLOCK * b: BLOCK * (b + 1)] = P @ Vc
            LSE[h, BLOCK * b: BLOCK * (b + 1)] = lse
    return O, LSE


def attn_bwd(q, k_hist, v_hist, k_seg, v_seg, sel_groups, scale, d_o, n_sink_tokens=0,
             window=None):
    """Gradients of sum(O * dO) w.r.t. Q, K_seg, V_seg [gist 2.1, gist 2.2].

    The history K/V is detached (no gradient); routing is a stop-gradient step,
    so the selections are constants. Uses the softmax Jacobian directly:
    dS = P * (dP - sum_t P_t dP_t). Returns float64 (dQ, dK_seg, dV_seg).
    """
    n_q, S, d = q.shape
    n_kv = k_seg.shape[0]
    r = n_q // n_kv
    dQ = np.zeros((n_q, S, d), F64)
    dK = np.zeros((n_kv, S, d), F64)
    dV = np.zeros((n_kv, S, d), F64)
    for h in range(n_q):
        j = h // r
        for b in range(S // BLOCK):
            rows = slice(BLOCK * b, BLOCK * (b + 1))
            Kc, Vc, n_hist, loc0, n_loc = _block_keys(k_hist, v_hist, k_seg, v_seg, sel_groups,
                                                      b, j, n_sink_tokens, window)
            Qb = np.asarray(q[h, rows], F64)
            dOb = np.asarray(d_o[h, rows], F64)
            P, _ = _block_probs(Qb, Kc, n_hist, loc0, n_loc, b, scale, _window(window, S))
            dP = dOb @ Vc.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[h, rows] = scale * (dS @ Kc)
            dK[j, loc0:loc0 + n_loc] += scale * (dS[:, n_hist:].T @ Qb)
            dV[j, loc0:loc0 + n_loc] += P[:, n_hist:].T @ dOb
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# Decode / retrieval step [gist §3 "Key Contributions": the trained adapter can
# run with HGA for retrieval and generation; gist 2.1 for the routing and the
# key set; gist 2.2 for the closed history and the open segment]
# ---------------------------------------------------------------------------
def decode_query_mean(q_new: np.ndarray, n_kv: int) -> np.ndarray:
    """qbar[j] = mean of the n_new newest queries over the r heads of KV head
    j: the decode step's query block. float32 [n_kv][d]."""
    n_q, n_new, d = q_new.shape
    if n_q % n_kv:
        raise ValueError("bad query shape")
    r = n_q // n_kv
    acc = np.zeros((n_kv, d), dtype=F32)
    for j in range(n_kv):
        for h in range(j * r, (j + 1) * r):
            for i in range(n_new):
                acc[j] += np.asarray(q_new[h, i], F32)
    acc *= F32(1.0 / (n_new * r))
    return acc


def decode_step(q_new, k_hist, v_hist, k_tail, v_tail, k_c, k_g, scale, n_sink=0, window=None,
                sel_groups=None):
    """One decode step of one sequence.

    The history (k_hist / v_hist [n_kv][H][d], H a multiple of 64) is closed
    and summarised; the open segment (k_tail / v_tail [n_kv][T][d], not yet
    summarised) ends with the n_new tokens whose queries are q_new
    [n_q][n_new][d], at open-segment positions T - n_new .. T - 1. Routing as
    in training, with the n_new queries as the query block; query i at
    position p attends the sink tokens, the tokens of the selected groups and
    the open-segment tokens t with p - W < t <= p (W = window, default the
    whole open segment). sel_groups [n_kv][k_g], if given, replaces the
    routed selection in the attention (to check a kernel's outputs against its
    own selection).

    Returns (sel_chunks int32 [n_kv][k_c], sel_groups int32 [n_kv][k_g],
    O float64 [n_q][n_new][d], LSE float64 [n_q][n_new]).
    """
    n_q, n_new, d = q_new.shape
    n_kv, T, _ = k_tail.shape
    H = k_hist.shape[1]
    if n_new > T:
        raise ValueError("the open segment must hold the new tokens")
    r = n_q // n_kv
    qbar = decode_query_mean(q_new, n_kv)[None]           # one query block
    if H:
        sel_c, _ = route_chunks(qbar, chunk_summaries(k_hist), k_c, n_sink)
        sel_g = route_groups(qbar, group_summaries(k_hist), sel_c, k_g)
    else:
        sel_c = np.full((1, n_kv, k_c), -1, np.int32)
        sel_g = np.full((1, n_kv, k_g), -1, np.int32)
    use = sel_g[0] if sel_groups is None else np.asarray(sel_groups)
    W = T if window is None or window <= 0 else min(int(window), T)
    sink_tok = min(n_sink * CHUNK, H)
    O = np.zeros((n_q, n_new, d), F64)
    LSE = np.zeros((n_q, n_new), F64)
    for h in range(n_q):
        j = h // r
        hist = attended_history_tokens(use[j], sink_tok)
        for i in range(n_new):
            p = T - n_new + i
            loc = np.arange(max(0, p - W + 1), p + 1)
            K = np.concatenate([np.asarray(k_hist[j][hist], F64), np.asarray(k_tail[j][loc], F64)])
            V = np.concatenate([np.asarray(v_hist[j][hist], F64), np.asarray(v_tail[j][loc], F64)])
            sc = scale * (K @ np.asarray(q_new[h, i], F64))
            m = sc.max()
            e = np.exp(sc - m)
            O[h, i] = (e @ V) / e.sum()
            LSE[h, i] = m + np.log(e.sum())
    return sel_c[0], sel_g[0], O, LSE


# ---------------------------------------------------------------------------
# Parity criteria used by the tests
# ---------------------------------------------------------------------------
def error_stats(got: np.ndarray, ref: np.ndarray):
    """(max|got-ref|, ||got-ref||_2 / ||ref||_2)."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    if ref.size == 0:
        return 0.0, 0.0
    diff = got - ref
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return float(np.max(np.abs(diff))), rel


def slice_rel_l2(got, ref, rows: int = BLOCK) -> np.ndarray:
    """L2 error of every slice (index along axis 0, run of ``rows`` consecutive
    indices along axis 1) of arrays shaped [n][T] or [n][T][...], relative to
    the larger of that slice's reference norm and the root-mean-square
    reference norm of all slices: for O, dQ and LSE a slice is one (query
    head, query block), for dK and dV one (KV head, 64-key tile).

    The floor keeps a slice that is much smaller than its tensor's typical
    slice from being held to a tighter absolute bar than the others. Such
    slices occur where a query row sees few keys: dQ then cancels a common key
    component (the synthetic per-chunk key offsets) almost exactly, so the
    rounding of bf16 outputs and operands is large relative to the slice
    itself. A slice of typical size that is wrong by a fraction f reports about
    f. Returns float64 [n][ceil(T / rows)]."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    n, T = ref.shape[0], ref.shape[1]
    n_sl = -(-T // rows)
    num = np.zeros((n, n_sl), F64)
    den = np.zeros((n, n_sl), F64)
    for a in range(n):
        for s in range(n_sl):
            rs = slice(s * rows, min(T, (s + 1) * rows))
            num[a, s] = np.linalg.norm(got[a, rs] - ref[a, rs])
            den[a, s] = np.linalg.norm(ref[a, rs])
    floor = float(np.sqrt(np.mean(den ** 2)))
    den = np.maximum(den, floor)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def within_tolerance(got, ref, tol: float, rows: int = BLOCK) -> bool:
    """Pass iff max|got - ref| <= tol * max(1, max|ref|),
    ||got - ref||_2 <= tol * ||ref||_2 over the whole tensor, and the same
    relative L2 bound holds on every slice of ``slice_rel_l2`` (arrays of two
    or more dimensions).

    tol is the stated bar (2e-2 for bf16 outputs, 1e-4 for fp32). The max part
    is that bar as an absolute bound for tensors of magnitude <= 1; above 1 it
    scales with the tensor, because a bf16 value of magnitude m is only stored
    to within 2^-9 m (at |x| ~ 6 that is already 0.016). The relative L2 parts
    keep the check meaningful when |ref| is itself of the order of tol
    (attention outputs at these shapes are ~1e-2): an all-zero output, dense
    attention, local-only attention or a selection shifted by one chunk fail
    the whole-tensor part; one wrong (head, block) slice, or a few wrong rows
    of one, fail the per-slice part even among a thousand correct slices.
    The per-slice part measures each slice against max(its own norm, the
    root-mean-square slice norm): see ``slice_rel_l2``.
    """
    err, rel = error_stats(got, ref)
    mx = float(np.max(np.abs(np.asarray(ref, F64)))) if np.size(ref) else 0.0
    if not (err <= tol * max(1.0, mx) and rel <= tol):
        return False
    if np.ndim(ref) >= 2 and np.size(ref):
        return bool(np.max(slice_rel_l2(got, ref, rows)) <= tol)
    return True


LSE_TOL = 1e-4


def lse_within(got, ref, tol: float = LSE_TOL) -> bool:
    """LSE is an fp32 output whatever the input dtype (the scores are fp32 sums
    of products of the stored inputs), so it is held to the fp32 bar element
    by element: |got_i - ref_i| <= tol * max(1, |ref_i|)."""
    got = np.asarray(got, F64)
    ref = np.asarray(ref, F64)
    if ref.size == 0:
        return True
    return bool(np.all(np.abs(got - ref) <= tol * np.maximum(1.0, np.abs(ref))))


def check_selection(qbar, C, G, sel_chunks, sel_groups, k_c, k_g, gap=1e-5, n_sink=0):
    """Validate a selection against this oracle, allowing near-tie swaps.

    Per (block b, KV head j):
      chunks: the set must have min(k_c, n_C) distinct ascending valid ids,
        -1 padded; every id in the symmetric difference with the oracle's set
        must score within ``gap`` of the oracle's k-th best chunk score.
      groups: the oracle's group step is re-run on the given chunk set, then
        the same rule applies; every group must lie inside a given chunk.
    Returns dict(ok, failures[list], chunk_exemptions, group_exemptions).
    """
    sc = chunk_scores(qbar, C)
    n_B, n_kv, n_C = sc.shape
    fails, ex_c, ex_g = [], 0, 0
    for b in range(n_B):
        for j in range(n_kv):
            got_c = [int(x) for x in sel_chunks[b, j]]
            s0 = min(n_sink, n_C)
            want_n = min(k_c, n_C - s0)
            ids = [x for x in got_c if x >= 0]
            if (len(ids) != want_n or got_c[len(ids):] != [-1] * (k_c - len(ids))
                    or any(x >= n_C or x < s0 for x in ids)
                    or any(ids[i] >= ids[i + 1] for i in range(len(ids) - 1))):
                fails.append((b, j, "chunk set malformed", got_c))
                continue
            ref_c = s0 + topk_lowest_index(sc[b, j, s0:], k_c)
            tau = float(np.min(sc[b, j][ref_c])) if ref_c.size else 0.0
            diff = set(ids) ^ set(int(x) for x in ref_c)
            bad = [m for m in diff if not abs(float(sc[b, j, m]) - tau) < gap]
            if bad:
                fails.append((b, j, "chunk mismatch", sorted(diff)))
                continue
            ex_c += len(diff) // 2
            ref_g, cand, sg = route_groups_one(qbar[b, j], G[j], np.array(ids), k_g)
            got_g = [int(x) for x in sel_groups[b, j]]
            gids = [x for x in got_g if x >= 0]
            want_g = min(k_g, cand.shape[0])
            cset = set(ids)
            if (len(gids) != want_g or got_g[len(gids):] != [-1] * (k_g - len(gids))
                    or any(gids[i] >= gids[i + 1] for i in range(len(gids) - 1))
                    or any((x // (CHUNK // GROUP)) not in cset for x in gids)):
                fails.append((b, j, "group set malformed", got_g))
                continue
            score_of = {int(n): float(s) for n, s in zip(cand, sg)}
            tau_g = min(score_of[int(n)] for n in ref_g) if ref_g.size else 0.0
            diff_g = set(gids) ^ set(int(x) for x in ref_g)
            bad_g = [n for n in diff_g if not abs(score_of[n] - tau_g) < gap]
            if bad_g:
                fails.append((b, j, "group mismatch", sorted(diff_g)))
                continue
            ex_g += len(diff_g) // 2
    return dict(ok=not fails, failures=fails, chunk_exemptions=ex_c,
                group_exemptions=ex_g)
