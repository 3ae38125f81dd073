"""Host-side pieces of bench.py (no GPU): the algorithmic work each roofline
is computed from, pinned to the per-layer figures derived by hand for the
Qwen3-8B workloads (32 query / 8 KV heads, d = 128, S = 2,048, top-16 chunks
then top-32 groups), and the guards around the child processes that time the
other workloads."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_fine_amd import synth  # noqa: E402

MIB = 2 ** 20


def _work(name, **kw):
    w = synth.WORKLOADS[name]
    if kw:
        w = w.replace(**kw)
    return bench.kernel_work(w, None)


def test_route_bytes_16k_and_131k():
    # Q of the segment (bf16) + every ranked chunk summary once (fp32) + the
    # 8 * 16 candidate group summaries per (block, KV head) + the selections
    q = 32 * 2048 * 128 * 2
    cand = 32 * 8 * (8 * 16) * 128 * 4
    sel = 32 * 8 * (16 + 32) * 4
    assert _work("qwen3_8b_16k_fwdbwd")["route"] == ("hbm", q + 8 * 224 * 128 * 4 + cand + sel)
    assert round(_work("qwen3_8b_16k_fwdbwd")["route"][1] / MIB, 1) == 32.9
    assert _work("qwen3_8b_131k_fwd")["route"] == ("hbm", q + 8 * 2016 * 128 * 4 + cand + sel)
    assert round(_work("qwen3_8b_131k_fwd")["route"][1] / MIB, 1) == 39.9


def test_attention_flops_16k():
    # per query head: 2,048 queries x 256 routed history keys, plus the
    # causal segment pairs 2,048 * 2,049 / 2
    hist, causal = 2048 * 256, 2048 * 2049 // 2
    w = _work("qwen3_8b_16k_fwdbwd")
    assert w["attn_fwd"] == ("mfma", 4 * 128 * 32 * (hist + causal))
    assert round(w["attn_fwd"][1] / 1e9, 2) == 42.97
    assert w["bwd_dq"] == ("mfma", 6 * 128 * 32 * (hist + causal))
    assert w["bwd_dkdv"] == ("mfma", 4 * 128 * 32 * causal)
    # the whole backward: 10 d per causal pair, 6 d per history pair, no pair twice
    assert round((w["bwd_dq"][1] + w["bwd_dkdv"][1]) / 1e9, 1) == 98.8
    # the dK/dV kernel executes S and dP again: twice its algorithmic work
    ex = bench.kernel_executed_work(synth.WORKLOADS["qwen3_8b_16k_fwdbwd"])
    assert ex["bwd_dkdv"] == 2 * w["bwd_dkdv"][1]


def test_forward_only_has_no_backward_work():
    w = _work("qwen3_8b_16k_fwd")
    assert "bwd_dq" not in w and "bwd_dkdv" not in w
    assert bench.kernel_executed_work(synth.WORKLOADS["qwen3_8b_16k_fwd"]) == {}


def test_host_tier_moves_routed_rows_over_the_link():
    # 32 blocks x 8 KV heads x 256 routed tokens x (K and V rows of 256 B)
    w = _work("qwen3_8b_131k_fwd_host")
    assert w["gather"] == ("host", 32 * 8 * 256 * 128 * 2 * 2)
    assert w["gather"][1] == 32 * MIB


def test_window_and_sink_change_the_attended_pairs():
    # a window of 1,024: query i sees min(i + 1, 1024) segment keys; one sink
    # chunk adds 64 keys to every query
    w = _work("qwen3_8b_16k_fwdbwd", n_sink_chunks=1, local_window=1024)
    causal = 1024 * 1025 // 2 + (2048 - 1024) * 1024
    hist = 2048 * (256 + 64)
    assert w["attn_fwd"] == ("mfma", 4 * 128 * 32 * (hist + causal))
    assert w["bwd_dkdv"] == ("mfma", 4 * 128 * 32 * causal)


class _Args:
    def __init__(self, also="auto", workload="qwen3_8b_16k_fwdbwd"):
        self.also, self.workload = also, workload
        self.steps, self.warmup, self.seed = 2, 1, 0


def test_other_configs_only_for_the_default_workload(monkeypatch):
    monkeypatch.delenv("ROCPROF_OUTPUT_PATH", raising=False)
    assert bench.other_configs(_Args(also="none")) is None
    assert bench.other_configs(_Args(workload="qwen3_8b_131k_fwd")) is None


def test_other_configs_start_nothing_under_the_profiler(monkeypatch):
    monkeypatch.setenv("ROCPROF_OUTPUT_PATH", "/tmp/x")
    assert bench.other_configs(_Args()) == {"skipped": "running under rocprofv3"}


def test_failed_child_is_recorded_not_raised(monkeypatch):
    # without a GPU the child exits with an error; the parent records it
    monkeypatch.setattr(bench, "ALSO_DEFAULT", ("qwen3_8b_16k_fwd",))
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the child would run")
    res = bench.other_configs(_Args())
    assert set(res) == {"qwen3_8b_16k_fwd"} and res["qwen3_8b_16k_fwd"]["error"] == "exit 1"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr
