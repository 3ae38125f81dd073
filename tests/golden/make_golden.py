"""Write the stored oracle outputs under tests/golden/.

The pages print no worked example and no per-kernel value for the route or
the attention (every number they give is an end-to-end fine-tuning metric), so
nothing here is quoted from them. The fixture is the CPU oracle (oracle/) run
on the tiny fp32 workload's seeded inputs (long_context_fine_amd.synth, which
only draws random numbers): exact selections plus sampled and row-summed
outputs. It pins the oracle's results against unnoticed change (a change to
its arithmetic must rewrite this file in the same commit) and gives the GPU
tests a stored reference that needs no oracle run.

This script calls only oracle/ and the seeded generator. Run from the
repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from long_context_fine_amd import synth  # noqa: E402
from oracle import hga_oracle as orc  # noqa: E402

WORKLOAD = "tiny_f32"
SEED = 0
N_SAMPLE = 64
OUT = os.path.join(HERE, "tiny_f32_seed0.json")


def sample_index(n: int) -> list:
    """N_SAMPLE flat positions spread evenly over an array of n elements."""
    return [int(x) for x in np.linspace(0, n - 1, N_SAMPLE).round()]


def summarise(x: np.ndarray) -> dict:
    flat = np.asarray(x, np.float64).reshape(-1)
    idx = sample_index(flat.size)
    return {
        "shape": list(x.shape),
        "row_sums": [float(v) for v in np.asarray(x, np.float64).reshape(-1, x.shape[-1]).sum(-1)],
        "sample_index": idx,
        "sample": [float(flat[i]) for i in idx],
    }


def compute() -> dict:
    w = synth.WORKLOADS[WORKLOAD]
    inp = synth.make_inputs(w, SEED, with_grad_out=True)
    a = {k: synth.to_numpy64(v) for k, v in inp.items()}
    sel_c, sel_g, aux = orc.route(a["q"], a["k_hist"], w.n_kv_heads, w.top_k_chunks, w.top_k_groups)
    O, LSE = orc.attn_fwd(a["q"], a["k_hist"], a["v_hist"], a["k_seg"], a["v_seg"], sel_g,
                          w.softmax_scale)
    dQ, dK, dV = orc.attn_bwd(a["q"], a["k_hist"], a["v_hist"], a["k_seg"], a["v_seg"], sel_g,
                              w.softmax_scale, a["d_o"])
    return {
        "about": ("CPU oracle outputs on synth.make_inputs(WORKLOADS['tiny_f32'], seed=0, "
                  "with_grad_out=True); written by tests/golden/make_golden.py"),
        "workload": {"name": w.name, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                     "head_dim": w.head_dim, "hist_len": w.hist_len, "seg_len": w.seg_len,
                     "top_k_chunks": w.top_k_chunks, "top_k_groups": w.top_k_groups,
                     "softmax_scale": w.softmax_scale, "seed": SEED},
        "sel_chunks": np.asarray(sel_c).tolist(),
        "sel_groups": np.asarray(sel_g).tolist(),
        "chunk_summaries": summarise(aux["C"]),
        "group_summaries": summarise(aux["G"]),
        "lse": [float(v) for v in np.asarray(LSE).reshape(-1)],
        "o": summarise(O),
        "dq": summarise(dQ),
        "dk_seg": summarise(dK),
        "dv_seg": summarise(dV),
    }


if __name__ == "__main__":
    rec = compute()
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("wrote", OUT)
