"""Byte accounting for the decode chain.

``decode_estimate`` restates the handbook's decode gap estimate (the PDL/megakernel
chapter, "how large are the gaps"): every decode kernel is memory bound, so its
time is its bytes over an effective bandwidth; each kernel boundary adds a gap of g
microseconds; launching kernel by kernel without a graph costs 5 us of CPU time per
kernel.  The per-layer kernel list fuses residual-add + RMSNorm and QK-norm + RoPE,
as vLLM does; the tail is final norm, lm_head and sampling.

"""
from __future__ import annotations

from typing import Dict, List, Tuple

QWEN3 = {
    "Qwen3-0.6B": dict(hidden=1024, inter=3072, layers=28, heads=16, kv_heads=8, head_dim=128, vocab=151936),
    "Qwen3-8B": dict(hidden=4096, inter=12288, layers=36, heads=32, kv_heads=8, head_dim=128, vocab=151936),
}
H100_EFFECTIVE_BW = 3.35e12 * 0.85
CPU_LAUNCH_US = 5.0


def decode_kernels(model: dict, batch: int, context: int, nbytes: int = 2) -> List[Tuple[str, int]]:
    h, inter = model["hidden"], model["inter"]
    q = model["heads"] * model["head_dim"]
    kv = model["kv_heads"] * model["head_dim"]
    act = batch * h * nbytes
    per_layer = [
        ("add_rmsnorm", 4 * act),                       # read x and residual, write both
        ("qkv_proj", h * (q + 2 * kv) * nbytes),        # weight bytes dominate
        ("qk_norm_rope", 2 * batch * (q + kv) * nbytes),
        ("kv_cache_write", 2 * batch * kv * nbytes),
        ("attention", batch * context * 2 * kv * nbytes),
        ("o_proj", q * h * nbytes),
        ("add_rmsnorm", 4 * act),
        ("gate_up_proj", h * 2 * inter * nbytes),
        ("silu_mul", 3 * batch * inter * nbytes),
        ("down_proj", inter * h * nbytes),
    ]
    tail = [("final_norm", 2 * act), ("lm_head", h * model["vocab"] * nbytes), ("sample", batch * model["vocab"] * 4)]
    out: List[Tuple[str, int]] = []
    for _ in range(model["layers"]):
        out.extend(per_layer)
    return out + tail


def decode_estimate(model_name: str, batch: int, context: int, gaps_us=(0.5, 1.0, 2.0, 3.0),
                    bw: float = H100_EFFECTIVE_BW) -> Dict[str, object]:
    ks = decode_kernels(QWEN3[model_name], batch, context)
    n = len(ks)
    t_data = sum(b for _, b in ks) / bw * 1e6
    res = {"kernels": n, "data_us": t_data,
           "eager_us": max(n * CPU_LAUNCH_US, t_data + n * gaps_us[0]),
           "graph_us": {g: t_data + n * g for g in gaps_us},
           "gap_share": {g: n * g / (t_data + n * g) for g in gaps_us},
           "small_kernels": sum(1 for _, b in ks if b / bw * 1e6 < 1.0),
           "mean_kernel_us": t_data / n}
    return res
