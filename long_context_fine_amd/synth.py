"""Seeded synthetic inputs for the HGA route + exact-token attention path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic, so both the HIP path and the CPU oracle may consume what it
produces without sharing any computation.

The pages measure on Qwen3-8B activations over PG19 text (gist.science,
"Long-Context Fine-Tuning with Limited VRAM", Technical Summary §4). Neither the
weights nor the corpus are available, so seeded Gaussian tensors with Qwen3-8B
layer shapes (32 query heads, 8 KV heads, head dim 128) stand in for them.
Every 64-token chunk of keys gets a shared random offset so that chunk-level
content routing has something to find.

Recipe (fixed draw order so every consumer sees identical values):
  rng = numpy.random.default_rng(seed)
  Q  ~ N(0,1) [n_q, S, d]        K ~ N(0,1) [n_kv, H+S, d]
  V  ~ N(0,1) [n_kv, H+S, d]     off ~ N(0, 0.5^2) [n_kv, (H+S)/64, d]
  dO ~ N(0,1) [n_q, S, d]        (drawn last, used by the backward)
  Q, K, V *= a  (a = 1 for the tiny fp32 case, 1/sqrt(128) otherwise)
  K += off repeated over the 64 tokens of each chunk
  bf16 workloads: round-to-nearest-even cast of every tensor (dO unscaled).
  K, V split into history [:, :H] and active segment [:, H:].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

CHUNK_TOKENS = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hist_len: int
    seg_len: int
    top_k_chunks: int
    top_k_groups: int
    dtype: str            # "f32" or "bf16"
    input_scale: float
    backward: bool = False
    hist_on_host: bool = False
    n_sink_chunks: int = 0  # history chunks attended in full (fixed sink)
    local_window: int = 0   # segment tokens each query sees (0: the whole causal segment)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_QWEN3_8B = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, seg_len=2048,
                 top_k_chunks=16, top_k_groups=32, dtype="bf16",
                 input_scale=1.0 / math.sqrt(128))

WORKLOADS = {
    # tiny fp32 case: 1 KV head, 1 query head, d = 64, 1,024 history tokens
    "tiny_f32": Workload("tiny_f32", 1, 1, 64, 1024, 128, 4, 8, "f32", 1.0,
                         backward=True),
    # Qwen3-8B layer at 16,384 tokens of context (14,336 history + 2,048 segment)
    "qwen3_8b_16k_fwd": Workload("qwen3_8b_16k_fwd", hist_len=14336, **_QWEN3_8B),
    "qwen3_8b_16k_fwdbwd": Workload("qwen3_8b_16k_fwdbwd", hist_len=14336,
                                    backward=True, **_QWEN3_8B),
    # 131,072 tokens of context: 129,024 history tokens + 2,048 segment
    "qwen3_8b_131k_fwd": Workload("qwen3_8b_131k_fwd", hist_len=129024, **_QWEN3_8B),
    "qwen3_8b_131k_fwd_host": Workload("qwen3_8b_131k_fwd_host", hist_len=129024,
                                       hist_on_host=True, **_QWEN3_8B),
}


def _round(x: np.ndarray, w: Workload) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(w.torch_dtype).contiguous()


def make_inputs(w: Workload, seed: int = 0, with_grad_out: bool | None = None) -> dict:
    """Draw the inputs of workload ``w`` from ``seed``; returns CPU torch tensors.

    Keys: q [n_q,S,d], k_hist/v_hist [n_kv,H,d], k_seg/v_seg [n_kv,S,d] and,
    when the workload has a backward (or ``with_grad_out``), d_o [n_q,S,d].
    """
    if (w.hist_len + w.seg_len) % CHUNK_TOKENS:
        raise ValueError("context length must be a multiple of 64 tokens")
    rng = np.random.default_rng(seed)
    total = w.hist_len + w.seg_len
    f32 = np.float32
    q = rng.standard_normal((w.n_q_heads, w.seg_len, w.head_dim), dtype=f32)
    k = rng.standard_normal((w.n_kv_heads, total, w.head_dim), dtype=f32)
    v = rng.standard_normal((w.n_kv_heads, total, w.head_dim), dtype=f32)
    off = rng.standard_normal((w.n_kv_heads, total // CHUNK_TOKENS, w.head_dim),
                              dtype=f32) * f32(0.5)
    want_do = w.backward if with_grad_out is None else with_grad_out
    d_o = (rng.standard_normal((w.n_q_heads, w.seg_len, w.head_dim), dtype=f32)
           if want_do else None)
    a = f32(w.input_scale)
    if a != 1:
        q *= a
        k *= a
        v *= a
    k = k.reshape(w.n_kv_heads, total // CHUNK_TOKENS, CHUNK_TOKENS, w.head_dim)
    k += off[:, :, None, :]
    k = k.reshape(w.n_kv_heads, total, w.head_dim)
    H = w.hist_len
    out = {
        "q": _round(q, w),
        "k_hist": _round(k[:, :H], w),
        "v_hist": _round(v[:, :H], w),
        "k_seg": _round(k[:, H:], w),
        "v_seg": _round(v[:, H:], w),
    }
    if d_o is not None:
        out["d_o"] = _round(d_o, w)
    return out


def make_decode_inputs(w: Workload, hist_lens, tail_lens, n_new: int, seed: int = 0) -> dict:
    """A decode batch: sequence b is make_inputs(w, seed + b) with history
    capacity w.hist_len and open-segment capacity w.seg_len; its
    hist_lens[b] oldest history tokens and tail_lens[b] open-segment tokens are
    the live ones, and its new tokens' queries are the segment queries at
    positions tail_lens[b] - n_new .. tail_lens[b] - 1. CPU tensors:
    q [B,n_q,n_new,d], k_hist/v_hist [B,n_kv,P,d], k_tail/v_tail [B,n_kv,T,d],
    hist_lens/tail_lens int32 [B]."""
    seqs = [make_inputs(w, seed + b) for b in range(len(hist_lens))]
    q = torch.stack([x["q"][:, t - n_new:t] for x, t in zip(seqs, tail_lens)]).contiguous()
    return {
        "q": q,
        "k_hist": torch.stack([x["k_hist"] for x in seqs]).contiguous(),
        "v_hist": torch.stack([x["v_hist"] for x in seqs]).contiguous(),
        "k_tail": torch.stack([x["k_seg"] for x in seqs]).contiguous(),
        "v_tail": torch.stack([x["v_seg"] for x in seqs]).contiguous(),
        "hist_lens": torch.tensor(list(hist_lens), dtype=torch.int32),
        "tail_lens": torch.tensor(list(tail_lens), dtype=torch.int32),
    }


def to_numpy64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU tensor (fp32 or bf16) to float64 numpy."""
    return t.detach().to(torch.float64).numpy()
