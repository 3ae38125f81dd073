"""The stored fixture under tests/golden/ (written by tests/golden/make_golden.py
from the CPU oracle on the tiny fp32 workload, seed 0).

* CPU: the oracle, run again, still gives the stored values (a regression pin:
  any change to the oracle's arithmetic has to rewrite the fixture in the same
  commit).
* GPU: the HIP path, through the C ABI, matches the stored values without an
  oracle run: selections exactly, sampled outputs and row sums within the fp32
  tolerance 1e-4 (relative to max(1, max|ref|), row sums over d terms).
"""
import importlib.util
import json
import os

import numpy as np
import pytest
import torch

from long_context_fine_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FIXTURE = os.path.join(GOLDEN, "tiny_f32_seed0.json")
TOL = 1e-4


def _load():
    with open(FIXTURE) as f:
        return json.load(f)


def _make_golden():
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _same_summary(name, got: dict, ref: dict, rtol: float, atol: float):
    assert got["shape"] == ref["shape"], name
    assert got["sample_index"] == ref["sample_index"], name
    np.testing.assert_allclose(got["row_sums"], ref["row_sums"], rtol=rtol, atol=atol, err_msg=name)
    np.testing.assert_allclose(got["sample"], ref["sample"], rtol=rtol, atol=atol, err_msg=name)


def test_oracle_reproduces_the_stored_fixture():
    ref = _load()
    got = _make_golden().compute()
    assert got["workload"] == ref["workload"]
    assert got["sel_chunks"] == ref["sel_chunks"]
    assert got["sel_groups"] == ref["sel_groups"]
    np.testing.assert_allclose(got["lse"], ref["lse"], rtol=1e-12, atol=1e-12)
    for k in ("chunk_summaries", "group_summaries", "o", "dq", "dk_seg", "dv_seg"):
        _same_summary(k, got[k], ref[k], rtol=1e-9, atol=1e-12)


def test_fixture_is_consistent():
    """Structure the pages fix: selections ascending, k_c chunks and k_g
    groups per block, every selected group inside a selected chunk."""
    ref = _load()
    w = ref["workload"]
    sc = np.asarray(ref["sel_chunks"])
    sg = np.asarray(ref["sel_groups"])
    n_blocks = w["seg_len"] // 64
    assert sc.shape == (n_blocks, w["n_kv_heads"], w["top_k_chunks"])
    assert sg.shape == (n_blocks, w["n_kv_heads"], w["top_k_groups"])
    for b in range(n_blocks):
        for j in range(w["n_kv_heads"]):
            c, g = sc[b, j], sg[b, j]
            assert list(c) == sorted(c) and list(g) == sorted(g)
            assert set((g // 8).tolist()) <= set(c.tolist())
            assert c.max() < w["hist_len"] // 64


def _summary(x: np.ndarray, idx) -> dict:
    flat = x.reshape(-1)
    return {"shape": list(x.shape), "row_sums": x.reshape(-1, x.shape[-1]).sum(-1),
            "sample": flat[idx]}


@pytest.mark.gpu
def test_hip_path_matches_the_stored_fixture():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_fine_amd import hga
    ref = _load()
    w = synth.WORKLOADS["tiny_f32"]
    print(f"[case] golden {w.name} seed=0", flush=True)
    inp = {k: v.cuda() for k, v in synth.make_inputs(w, 0, with_grad_out=True).items()}
    s = hga.make_shape(w.n_q_heads, w.n_kv_heads, w.head_dim, w.hist_len, w.seg_len,
                       w.top_k_chunks, w.top_k_groups, w.torch_dtype, w.softmax_scale)
    C, G = hga.summaries(s, inp["k_hist"])
    sel_c, sel_g = hga.route(s, inp["q"], C, G)
    o, lse = hga.attn_fwd(s, inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"], sel_g)
    dq, dk, dv = hga.attn_bwd(s, inp["q"], inp["k_hist"], inp["v_hist"], inp["k_seg"], inp["v_seg"],
                              sel_g, o, lse, inp["d_o"])
    torch.cuda.synchronize()
    assert sel_c.cpu().numpy().tolist() == ref["sel_chunks"]
    assert sel_g.cpu().numpy().tolist() == ref["sel_groups"]
    lse_ref = np.asarray(ref["lse"])
    assert np.abs(lse.double().cpu().numpy().reshape(-1) - lse_ref).max() <= TOL * max(1.0, np.abs(lse_ref).max())
    for name, t in (("chunk_summaries", C), ("group_summaries", G), ("o", o), ("dq", dq),
                    ("dk_seg", dk), ("dv_seg", dv)):
        r = ref[name]
        got = _summary(t.double().cpu().numpy(), r["sample_index"])
        assert got["shape"] == r["shape"], name
        scale = max(1.0, float(np.abs(r["sample"]).max()))
        d = got["shape"][-1]
        err_s = np.abs(got["sample"] - np.asarray(r["sample"])).max()
        err_r = np.abs(got["row_sums"] - np.asarray(r["row_sums"])).max()
        print(f"  {name}: sample max|d|={err_s:.2e} row-sum max|d|={err_r:.2e}", flush=True)
        assert err_s <= TOL * scale, name
        assert err_r <= TOL * scale * d, name
