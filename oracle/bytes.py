"""Byte and gap model of one decode step.  TEST INFRASTRUCTURE ONLY.

Restates, in this project's own terms, the estimate of the handbook chapter on PDL and
megakernels (section "how large are the gaps: an estimate"):

* decode work is memory bound, so a kernel takes (bytes it reads and writes) / (effective
  bandwidth); the effective bandwidth is 85 % of an H100's 3.35 TB/s;
* every kernel boundary on the GPU costs a gap of g microseconds (0.5, 1, 2 or 3);
* issued one by one from the CPU (no graph), every kernel costs 5 us of CPU time, and the
  GPU cannot finish before the CPU has issued the last kernel;
* the per-layer kernel split follows vLLM's fusion: residual add + RMSNorm is one kernel,
  QK-norm + RoPE another; the step ends with the final norm, lm_head and sampling.

The page prints the resulting table; ``tests/golden/decode_gaps_table.txt`` holds it and
``tests/test_oracle_bytes.py`` checks this model against it.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple


@dataclasses.dataclass(frozen=True)
class DecoderShape:
    """Dimensions of a decoder-only model (the two Qwen3 sizes the page uses)."""
    hidden: int
    inter: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    vocab: int

    @property
    def q_width(self) -> int:
        return self.q_heads * self.head_dim

    @property
    def kv_width(self) -> int:
        return self.kv_heads * self.head_dim


SHAPES = {
    "Qwen3-0.6B": DecoderShape(hidden=1024, inter=3072, layers=28, q_heads=16, kv_heads=8, head_dim=128, vocab=151936),
    "Qwen3-8B": DecoderShape(hidden=4096, inter=12288, layers=36, q_heads=32, kv_heads=8, head_dim=128, vocab=151936),
}

GB_PER_S_EFFECTIVE = 0.85 * 3.35e12  # bytes / s the page assumes a memory-bound kernel reaches
HOST_ISSUE_US = 5.0                  # CPU time per kernel launched without a graph
GAP_LEVELS_US = (0.5, 1.0, 2.0, 3.0)


def layer_traffic(s: DecoderShape, batch: int, context: int, elem: int = 2) -> List[Tuple[str, int]]:
    """Bytes moved by each kernel of one layer, in chain order (step names of this project).

    Norm kernels read and write both the hidden state and the residual; projections are
    dominated by their weights; the KV read covers the whole context of every request; the
    cache write stores one K row and one V row per request; SiLU-mul reads gate and up and
    writes their product."""
    hidden_vec = batch * s.hidden * elem
    norm = 2 * (2 * hidden_vec)  # read x and residual, write both
    return [
        ("add_norm_attn", norm),
        ("proj_qkv", s.hidden * (s.q_width + 2 * s.kv_width) * elem),
        ("qk_norm_rope", 2 * batch * (s.q_width + s.kv_width) * elem),
        ("cache_write", 2 * batch * s.kv_width * elem),
        ("attention_kv_read", batch * context * 2 * s.kv_width * elem),
        ("proj_o", s.q_width * s.hidden * elem),
        ("add_norm_mlp", norm),
        ("proj_gate_up", 2 * s.inter * s.hidden * elem),
        ("silu_mul", 3 * batch * s.inter * elem),
        ("proj_down", s.hidden * s.inter * elem),
    ]


def tail_traffic(s: DecoderShape, batch: int, elem: int = 2) -> List[Tuple[str, int]]:
    """The step's last kernels: final norm (read + write the hidden state), lm_head (its
    weights), sampling (fp32 logits of every request)."""
    return [
        ("final_norm", 2 * batch * s.hidden * elem),
        ("lm_head", s.vocab * s.hidden * elem),
        ("sample", 4 * batch * s.vocab),
    ]


def step_traffic(s: DecoderShape, batch: int, context: int) -> List[Tuple[str, int]]:
    """Every kernel of one decode step: the layer list once per layer, then the tail."""
    return layer_traffic(s, batch, context) * s.layers + tail_traffic(s, batch)


def memory_time_us(nbytes: float) -> float:
    return nbytes / GB_PER_S_EFFECTIVE * 1e6


def graph_time_us(t_mem: float, n_kernels: int, gap_us: float) -> float:
    """Replayed as a graph: the data time plus one gap per kernel."""
    return t_mem + n_kernels * gap_us


def eager_time_us(t_mem: float, n_kernels: int) -> float:
    """Launched kernel by kernel: the step ends when both the host has issued every kernel and
    the GPU has run them with the smallest gap."""
    host_done = n_kernels * HOST_ISSUE_US
    gpu_done = graph_time_us(t_mem, n_kernels, min(GAP_LEVELS_US))
    return max(host_done, gpu_done)


def decode_estimate(model_name: str, batch: int, context: int) -> Dict[str, object]:
    """The page's per-scenario figures: kernel count, data time, eager time, graph time and
    the share of the step spent in gaps at each gap level, kernels under 1 us, mean kernel time."""
    kernels = step_traffic(SHAPES[model_name], batch, context)
    per_kernel_us = [memory_time_us(b) for _, b in kernels]
    n = len(kernels)
    t_mem = sum(per_kernel_us)
    graph = {g: graph_time_us(t_mem, n, g) for g in GAP_LEVELS_US}
    return {
        "kernels": n,
        "data_us": t_mem,
        "eager_us": eager_time_us(t_mem, n),
        "graph_us": graph,
        "gap_share": {g: n * g / graph[g] for g in GAP_LEVELS_US},
        "small_kernels": sum(t < 1.0 for t in per_kernel_us),
        "mean_kernel_us": t_mem / n,
    }
