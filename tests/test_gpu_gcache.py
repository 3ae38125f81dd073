"""Group-summary cache on the GPU: with the group summaries in page-locked host
memory, hga_route_cached must select exactly what hga_route selects from
device-resident summaries (same fp32 rows, same arithmetic), and the cache
tables must follow the documented policy, replayed here by a plain model:
the union of the chunks kept by a call's blocks is looked up per KV head;
cached chunks are hits and keep their slots; each miss, in ascending chunk
order, takes the next slot in clock order from the hand that no hit holds."""
import math

import numpy as np
import pytest
import torch

from long_context_fine_amd import hga, synth
from oracle import hga_oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hga.lib()


class ClockModel:
    """The replacement policy of the cache, on the host."""

    def __init__(self, n_kv, n_slots):
        self.n_slots = n_slots
        self.slot_of = [dict() for _ in range(n_kv)]
        self.chunk_of = [[-1] * n_slots for _ in range(n_kv)]
        self.hand = [0] * n_kv

    def call(self, sel_chunks):
        stats = []
        for j in range(len(self.hand)):
            needed = sorted({int(c) for c in sel_chunks[:, j, :].ravel() if c >= 0})
            hits = [c for c in needed if c in self.slot_of[j]]
            misses = [c for c in needed if c not in self.slot_of[j]]
            pinned = {self.slot_of[j][c] for c in hits}
            order = [(self.hand[j] + i) % self.n_slots for i in range(self.n_slots)]
            free = [p for p in order if p not in pinned]
            for k, c in enumerate(misses):
                p = free[k]
                old = self.chunk_of[j][p]
                if old >= 0:
                    del self.slot_of[j][old]
                self.slot_of[j][c] = p
                self.chunk_of[j][p] = c
            if misses:
                self.hand[j] = (free[len(misses) - 1] + 1) % self.n_slots
            stats.append((len(hits), len(misses)))
        return np.array(stats, dtype=np.int32)


def _check_tables(cache, model, G_host, n_chunk_rows):
    soc, cos, hand, data = (t.cpu() for t in cache.tables())
    for j in range(len(model.hand)):
        exp_soc = np.full(n_chunk_rows, -1, np.int32)
        for c, p in model.slot_of[j].items():
            exp_soc[c] = p
        assert np.array_equal(soc[j].numpy(), exp_soc), f"slot_of_chunk, KV head {j}"
        assert cos[j].tolist() == model.chunk_of[j], f"chunk_of_slot, KV head {j}"
        assert int(hand[j]) == model.hand[j], f"hand, KV head {j}"
        for c, p in model.slot_of[j].items():
            assert torch.equal(data[j, p], G_host[j, 8 * c:8 * c + 8]), f"slot {p} rows, chunk {c}"


def _inputs(n_q, n_kv, d, H, S, seed, dtype="bf16"):
    w = synth.Workload("gcache", n_q, n_kv, d, H, S, 1, 1, dtype, 1.0 / math.sqrt(d))
    return synth.make_inputs(w, seed)


def _run_sequence(n_q, n_kv, d, H, S, k_c, k_g, n_slots, seeds, sink=0, check_oracle=True, dtype="bf16"):
    base = _inputs(n_q, n_kv, d, H, S, seeds[0], dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s = hga.make_shape(n_q, n_kv, d, H, S, k_c, k_g, tdt, n_sink_chunks=sink)
    k_hist = base["k_hist"].cuda()
    C, G_dev = hga.summaries(s, k_hist)
    G_host = torch.empty(G_dev.shape, dtype=torch.float32, pin_memory=True)
    C2 = torch.empty_like(C)
    hga.hga_build_summaries(s, k_hist, C2, G_host)     # group rows written to host memory
    torch.cuda.synchronize()
    assert torch.equal(C2, C) and torch.equal(G_host, G_dev.cpu())
    cache = hga.GroupSummaryCache(s, n_slots)
    model = ClockModel(n_kv, n_slots)
    n_B = S // 64
    stats = torch.empty((n_kv, 2), dtype=torch.int32, device="cuda")
    history = []
    for i, seed in enumerate(seeds):
        print(f"[case] gcache H={H} S={S} kc={k_c} slots={n_slots} sink={sink} call {i} seed {seed}",
              flush=True)
        q = _inputs(n_q, n_kv, d, H, S, seed, dtype)["q"].cuda()
        sc = torch.empty((n_B, n_kv, k_c), dtype=torch.int32, device="cuda")
        sg = torch.empty((n_B, n_kv, k_g), dtype=torch.int32, device="cuda")
        cache.route(s, q, C, G_host, sc, sg, stats)
        ref_c, ref_g = hga.route(s, q, C, G_dev)
        torch.cuda.synchronize()
        assert torch.equal(sc, ref_c) and torch.equal(sg, ref_g)
        exp = model.call(sc.cpu().numpy())
        got = stats.cpu().numpy()
        print(f"  hits/misses per KV head: {got.tolist()}", flush=True)
        assert np.array_equal(got, exp)
        history.append(got)
        _check_tables(cache, model, G_host, H // 64)
        if check_oracle:
            qbar = orc.block_queries(q.float().cpu().numpy(), n_kv)
            rep = orc.check_selection(qbar, orc.chunk_summaries(k_hist.float().cpu().numpy()),
                                      orc.group_summaries(k_hist.float().cpu().numpy()),
                                      sc.cpu().numpy(), sg.cpu().numpy(), k_c, k_g, n_sink=sink)
            assert rep["ok"], rep["failures"][:3]
    return history


def test_cache_with_evictions_matches_resident_route():
    # the smallest cache (8 blocks x 4 chunks = 32 slots) over 128 chunks: new
    # queries evict; the repeated query (last) hits everything it kept
    st = _run_sequence(8, 2, 128, 8192, 512, 4, 16, 32, seeds=[0, 1, 2, 3, 3])
    assert st[4][:, 1].sum() == 0


def test_cache_larger_than_a_call_keeps_earlier_chunks():
    # 4 blocks x 3 chunks = at most 12 new chunks a call: two calls fit in 40
    # slots, so repeating the first query misses nothing
    st = _run_sequence(4, 2, 64, 4096, 256, 3, 10, 40, seeds=[5, 6, 5, 7])
    assert st[0][:, 0].sum() == 0 and st[0][:, 1].min() > 0      # cold: all misses
    assert st[2][:, 1].sum() == 0 and st[2][:, 0].min() > 0      # repeat: all hits


def test_cache_with_sink_ranks_after_it():
    _run_sequence(8, 2, 128, 4096, 320, 5, 13, 25, seeds=[8, 9], sink=2)


def test_cache_with_fp32_inputs():
    # fp32 queries and keys (the fp32 instances of the route kernel)
    _run_sequence(4, 2, 64, 4096, 256, 4, 12, 32, seeds=[11, 12, 11], dtype="f32")


def test_cache_at_131k_full_size():
    # Qwen3-8B layer, 129,024 history tokens, 512 slots per KV head (16 MiB of
    # cached rows instead of 63 MiB of group summaries)
    _run_sequence(32, 8, 128, 129024, 2048, 16, 32, 512, seeds=[0, 1, 1], check_oracle=False)


def test_reset_empties_the_cache():
    s = hga.make_shape(8, 2, 128, 4096, 256, 4, 16, torch.bfloat16)
    cache = hga.GroupSummaryCache(s, 64)
    soc, cos, hand, _ = cache.tables()
    torch.cuda.synchronize()
    assert bool((soc == -1).all()) and bool((cos == -1).all()) and bool((hand == 0).all())


def _random_cache_cases(n=6, seed=20261206):
    """Seeded random shapes for the cached route: GQA ratio, KV heads, head
    dim, history, segment, budgets, sink, dtype, and a cache between the
    smallest allowed ((S/64) * k_c slots) and twice that; three calls, the
    last repeating the first query."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        r = int(rng.choice([1, 2, 4, 8]))
        n_kv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        H = 64 * int(rng.integers(2, 65))
        S = 64 * int(rng.integers(1, 9))
        k_c = int(rng.integers(1, 9))
        k_g = int(rng.integers(1, 8 * k_c + 9))
        n_slots = (S // 64) * k_c + int(rng.integers(0, (S // 64) * k_c + 1))
        sink = int(rng.integers(1, 3)) if rng.random() < 0.3 else 0
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        out.append((f"rcache{i}", r * n_kv, n_kv, d, H, S, k_c, k_g, n_slots, sink, dtype))
    return out


RANDOM_CACHE = _random_cache_cases()


@pytest.mark.parametrize("case", RANDOM_CACHE, ids=[c[0] for c in RANDOM_CACHE])
def test_cache_random_shapes(case):
    _, n_q, n_kv, d, H, S, k_c, k_g, n_slots, sink, dtype = case
    _run_sequence(n_q, n_kv, d, H, S, k_c, k_g, n_slots, seeds=[21, 22, 21], sink=sink, dtype=dtype)
