"""hga_route_noalloc (the route with the library's static per-device scratch
as its workspace) against hga_route with a caller workspace: bit-identical
selections on two calls in a row, the second with a smaller input, both with
more than 4,096 chunks per KV head so that the chunk scores go through the
workspace."""
import math
import sys

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


def _route_both(n_q, n_kv, d, H, S, kc, kg, seed):
    print(f"[case] route_noalloc H={H} S={S} nq={n_q} nkv={n_kv} d={d} kc={kc} kg={kg}", flush=True)
    sys.stdout.flush()
    w = synth.Workload("noalloc", n_q, n_kv, d, H, S, kc, kg, "bf16", 1 / math.sqrt(d), backward=False)
    inp = synth.make_inputs(w, seed)
    q, k = inp["q"].cuda(), inp["k_hist"].cuda()
    s = hga.make_shape(n_q, n_kv, d, H, S, kc, kg, torch.bfloat16)
    assert 256 * 2 ** 10 < hga.hga_workspace_size(s, hga.HGA_OP_ROUTE) <= 16 * 2 ** 20
    C, G = hga.summaries(s, k)
    ref_c, ref_g = hga.route(s, q, C, G)
    got_c = torch.full_like(ref_c, -7)
    got_g = torch.full_like(ref_g, -7)
    hga.hga_route_noalloc(s, q, C, G, got_c, got_g)
    torch.cuda.synchronize()
    assert torch.equal(got_c, ref_c) and torch.equal(got_g, ref_g)
    return inp, s, got_c, got_g


def test_route_noalloc_matches_route_on_two_calls():
    # first call: 2 KV heads x 32 blocks x 4,160 chunks of scores in the scratch
    inp, s, c1, g1 = _route_both(4, 2, 64, 4160 * 64, 2048, 8, 16, 31)
    # second call, smaller: 16 blocks x 4,097 chunks, on top of the first call's contents
    inp2, s2, c2, g2 = _route_both(4, 2, 64, 4097 * 64, 1024, 8, 16, 32)
    # and the second call's selections are the oracle's (near-ties excepted)
    a = {k: v.float().numpy() for k, v in inp2.items()}
    qbar = orc.block_queries(a["q"], 2)
    rep = orc.check_selection(qbar, orc.chunk_summaries(a["k_hist"]), orc.group_summaries(a["k_hist"]),
                              c2.cpu().numpy(), g2.cpu().numpy(), 8, 16)
    assert rep["ok"], rep["failures"][:3]
