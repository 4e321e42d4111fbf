"""Workload definitions and seeded synthetic input generators.

This module is shared by the CPU oracle side (tests, the CPU baseline leg of the
benchmark) and the GPU side.  It holds shapes and random draws only: no step of
the decode-layer computation is performed here (no normalisation, no
projection, no rounding to a compute format, no FP8 encoding).

* bf16 tensors are produced as raw ``uint16`` bit patterns by keeping the upper
  half of float32 draws (round toward zero, a property of the synthetic
  distribution, not of the method).
* FP8 e4m3 tensors are produced directly as code bytes, field by field
  (sign, exponent field, mantissa field), never by quantising real values;
  the NaN codes 0x7F / 0xFF are never drawn.  Their fp32 scales are drawn too.

The workloads follow the decode-layer chain described on the MegaRTP page
(section 4, the M=16 / KV=8192 attention-pre plan) and the Qwen3 shapes used by
the handbook's decode byte model (the ``decode_gaps.py`` model table).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = ["Config", "CONFIGS", "get_config", "make_inputs", "f32_to_bf16_bits_trunc", "algorithmic_bytes"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    workload: str  # "qwen3_layer" | "qwen3_step" | "indexer_front"
    hidden: int
    inter: int = 0
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 128
    num_layers: int = 1
    vocab: int = 0
    n_requests: int = 1
    tokens_per_request: int = 1
    context: int = 512  # context length per request, including the current token(s)
    page_size: int = 16
    random_pages: bool = False
    weight_fp8: bool = False
    act_fp8: bool = False
    # indexer front
    idx_q_rank: int = 0
    idx_heads: int = 0
    idx_head_dim: int = 0
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    residual_zero: bool = False  # r_in == 0 (full decode step)
    topk: int = 0  # indexer front: positions each token selects after the score (0: no top-k)
    mla_heads: int = 0  # indexer front: heads of the main-MLA query half D0 -> D2 (0: none)
    rotary_dim: int = 0  # dims of a head the RoPE rotates (0: all of them)
    tile_params: tuple = ()  # the plan's tile sizes (rows per task, split tokens); () or 0: the planner's rule

    @property
    def m(self) -> int:
        return self.n_requests * self.tokens_per_request

    @property
    def pages_per_request(self) -> int:
        return -(-self.context // self.page_size)

    @property
    def num_phys_pages(self) -> int:
        return self.n_requests * self.pages_per_request


CONFIGS: Dict[str, Config] = {
    # Qwen3-0.6B-shaped single decode layer, batch 1, context 512 in 16-token pages.
    "qwen3_0p6b_layer": Config("qwen3_0p6b_layer", "qwen3_layer", hidden=1024, inter=3072,
                               n_q_heads=16, n_kv_heads=8, context=512, page_size=16),
    # Qwen3-0.6B-shaped full 28-layer decode step + final norm + lm_head + greedy argmax.
    "qwen3_0p6b_step": Config("qwen3_0p6b_step", "qwen3_step", hidden=1024, inter=3072,
                              n_q_heads=16, n_kv_heads=8, num_layers=28, vocab=151936,
                              context=2048, page_size=16, residual_zero=True),
    # Qwen3-8B-shaped layer, 16 requests x 1 token, context 4096 in 64-token pages.
    "qwen3_8b_layer": Config("qwen3_8b_layer", "qwen3_layer", hidden=4096, inter=12288,
                             n_q_heads=32, n_kv_heads=8, n_requests=16, context=4096,
                             page_size=64),
    # Same with FP8 e4m3 weights (128x128 block scales) and FP8 activations, context 8192,
    # randomised page tables.
    "qwen3_8b_layer_fp8": Config("qwen3_8b_layer_fp8", "qwen3_layer", hidden=4096, inter=12288,
                                 n_q_heads=32, n_kv_heads=8, n_requests=16, context=8192,
                                 page_size=64, random_pages=True, weight_fp8=True, act_fp8=True),
    # Qwen3-8B-shaped layer at a larger batch: 64 requests x 1 token (four 16-row groups), context
    # 4096 in 64-token pages, randomised page tables.
    "qwen3_8b_layer_m64": Config("qwen3_8b_layer_m64", "qwen3_layer", hidden=4096, inter=12288,
                                 n_q_heads=32, n_kv_heads=8, n_requests=64, context=4096,
                                 page_size=64, random_pages=True),
    # Indexer-style pre-attention front: 2 requests x 8 tokens, KV 8192, 64 heads x 128.
    "indexer_front": Config("indexer_front", "indexer_front", hidden=6144, n_requests=2,
                            tokens_per_request=8, context=8192, page_size=64, random_pages=True,
                            weight_fp8=True, act_fp8=True, idx_q_rank=1536, idx_heads=64,
                            idx_head_dim=128),
    # The same front followed by the per-token Top-2048 over its 8192 scores (the MegaRTP page's
    # next step after the paged indexer score).
    "indexer_front_topk": Config("indexer_front_topk", "indexer_front", hidden=6144, n_requests=2,
                                 tokens_per_request=8, context=8192, page_size=64, random_pages=True,
                                 weight_fp8=True, act_fp8=True, idx_q_rank=1536, idx_heads=64,
                                 idx_head_dim=128, topk=2048),
    # The page's whole attention-pre graph: the indexer front plus the main-MLA query half,
    # D0 Main-Q (64 heads x 128 no-RoPE dims from the normalised q_a) -> D2 Q-BMM (per head, into
    # a 512-wide latent).
    "attention_pre": Config("attention_pre", "indexer_front", hidden=6144, n_requests=2,
                            tokens_per_request=8, context=8192, page_size=64, random_pages=True,
                            weight_fp8=True, act_fp8=True, idx_q_rank=1536, idx_heads=64,
                            idx_head_dim=128, mla_heads=64),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    return cfg


def f32_to_bf16_bits_trunc(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values (round toward zero): the synthetic bf16 draw."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a.reshape(-1).view(np.uint16)[1::2].reshape(a.shape)  # little-endian: the upper half words


def _bf16_normal(rng: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    chunk = 1 << 24
    for s in range(0, flat.size, chunk):
        n = min(chunk, flat.size - s)
        v = rng.standard_normal(n, dtype=np.float32)
        v *= np.float32(std)
        if mean:
            v += np.float32(mean)
        flat[s:s + n] = v.view(np.uint16)[1::2]  # upper 16 bits (little-endian)
    return out


def _binade_probs(sigma: float) -> np.ndarray:
    """P(|v| falls in the e4m3 binade of exponent field e), e = 0..15, for v ~ N(0, sigma^2) in
    code units: field 0 holds [0, 2^-6), field e >= 1 holds [2^(e-7), 2^(e-6)), and field 15 also
    every larger magnitude (the top binade takes the tail)."""
    edges = [0.0] + [2.0 ** (e - 7) for e in range(1, 16)] + [math.inf]
    cdf = [math.erf(x / (sigma * math.sqrt(2.0))) if math.isfinite(x) else 1.0 for x in edges]
    p = np.diff(np.array(cdf))
    return p / p.sum()


def _fp8_codes(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """e4m3 code bytes drawn field by field so that the decoded values spread like a normal
    N(0, sigma^2) in code units: sign uniform, exponent field from the normal's binade
    probabilities, mantissa uniform in [0, 7] (the NaN pattern, exponent 15 with mantissa 7, is
    drawn as mantissa 6)."""
    probs = _binade_probs(sigma)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    chunk = 1 << 24
    for s in range(0, n, chunk):
        k = min(chunk, n - s)
        sign = rng.integers(0, 2, k, dtype=np.uint8)
        e = rng.choice(16, size=k, p=probs).astype(np.uint8)
        m = rng.integers(0, 8, k, dtype=np.uint8)
        m = np.where((e == 15) & (m == 7), np.uint8(6), m)
        out[s:s + k] = (sign << 7) | (e << 3) | m
    return out.reshape(shape)


# Spread of the codes, as a per-group amax -> 448 mapping of normal values would give them: a
# 128 x 128 weight block's amax is about 4 standard deviations (codes ~ N(0, 112^2)), a 128-wide
# key row's about 2.6 (codes ~ N(0, 172^2)).  The scales then make the effective values
# N(0, 0.02^2) for weights and N(0, 1) for keys.
_FP8_W_SIGMA, _FP8_K_SIGMA = 112.0, 172.0
_FP8_W_SCALE = 0.02 / _FP8_W_SIGMA
_FP8_K_SCALE = 1.0 / _FP8_K_SIGMA


def _page_table(rng: np.random.Generator, cfg: Config) -> np.ndarray:
    n = cfg.num_phys_pages
    pages = rng.permutation(n).astype(np.int32) if cfg.random_pages else np.arange(n, dtype=np.int32)
    return pages.reshape(cfg.n_requests, cfg.pages_per_request)


def make_inputs(cfg: Config, seed: int = 0, layers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Seeded synthetic inputs for one workload.  The draw order is fixed and listed
    below; every tensor is stored in the layout the library consumes:

    qwen3_layer / qwen3_step (L = num_layers, stacked on a leading layer axis):
      w_qkv  [L, (Hq+2Hkv)d, H]   bf16 bits (or e4m3 codes + s_qkv [L, ceil(N/128), ceil(H/128)] f32)
      w_o    [L, H, Hq d]
      w_gu   [L, 2I, H]           rows [0, I) gate, [I, 2I) up
      w_down [L, H, I]
      g_attn, g_mlp [L, H]; g_q, g_k [L, d]   bf16 bits, 1 + N(0, 0.02)
      k_cache, v_cache [L, pages, P, Hkv, d]  bf16 bits ~ N(0, 1) (slots < ctx-1 hold prior tokens)
      block_table [R, pages_per_request] int32; context_lens [R] int32
      x [M, H] bf16 bits ~ N(0,1); r_in [M, H] f32 ~ N(0,1) (zeros for the full step)
      step only: g_final [H], w_lm [V, H]
    indexer_front:
      w_qa [1536, H], w_w [64, H], w_k [128, H], w_qi [64*128, 1536]: e4m3 codes + block scales
      g_norm [H], g_qa [1536] bf16 bits; x [16, H] bf16 bits; r_in [16, H] f32
      key_cache [pages, 64, 128] e4m3 codes, key_scale [pages, 64] f32; block_table, context_lens
      main-MLA half (mla_heads = nm > 0), drawn last: w_qb [nm 128, 1536] e4m3 codes + s_qb,
      w_uk [nm 512, 128] bf16 bits ~ N(0, 0.05)
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, np.ndarray] = {}
    if cfg.workload in ("qwen3_layer", "qwen3_step"):
        L = cfg.num_layers if layers is None else layers
        H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
        nq, nkv = cfg.n_q_heads * d, cfg.n_kv_heads * d
        shapes = [("w_qkv", (nq + 2 * nkv, H)), ("w_o", (H, nq)), ("w_gu", (2 * I, H)), ("w_down", (H, I))]
        for name, (n, k) in shapes:
            if cfg.weight_fp8:
                out[name] = _fp8_codes(rng, (L, n, k), _FP8_W_SIGMA)
                nb, kb = -(-n // 128), -(-k // 128)
                out["s_" + name[2:]] = (rng.uniform(0.8, 1.25, (L, nb, kb)) * _FP8_W_SCALE).astype(np.float32)
            else:
                out[name] = _bf16_normal(rng, (L, n, k), 0.02)
        out["g_attn"] = _bf16_normal(rng, (L, H), 0.02, 1.0)
        out["g_mlp"] = _bf16_normal(rng, (L, H), 0.02, 1.0)
        out["g_q"] = _bf16_normal(rng, (L, d), 0.02, 1.0)
        out["g_k"] = _bf16_normal(rng, (L, d), 0.02, 1.0)
        bt = _page_table(rng, cfg)
        out["block_table"] = bt
        out["context_lens"] = np.full(cfg.n_requests, cfg.context, dtype=np.int32)
        cache_shape = (L, cfg.num_phys_pages, cfg.page_size, cfg.n_kv_heads, d)
        out["k_cache"] = _bf16_normal(rng, cache_shape, 1.0)
        out["v_cache"] = _bf16_normal(rng, cache_shape, 1.0)
        out["x"] = _bf16_normal(rng, (cfg.m, H), 1.0)
        if cfg.residual_zero:
            out["r_in"] = np.zeros((cfg.m, H), dtype=np.float32)
        else:
            out["r_in"] = rng.standard_normal((cfg.m, H), dtype=np.float32)
        if cfg.workload == "qwen3_step":
            out["g_final"] = _bf16_normal(rng, (H,), 0.02, 1.0)
            out["w_lm"] = _bf16_normal(rng, (cfg.vocab, H), 0.02)
    elif cfg.workload == "indexer_front":
        H = cfg.hidden
        qr, nh, hd = cfg.idx_q_rank, cfg.idx_heads, cfg.idx_head_dim
        for name, (n, k) in [("w_qa", (qr, H)), ("w_w", (nh, H)), ("w_k", (hd, H)), ("w_qi", (nh * hd, qr))]:
            out[name] = _fp8_codes(rng, (n, k), _FP8_W_SIGMA)
            out["s_" + name[2:]] = (rng.uniform(0.8, 1.25, (-(-n // 128), -(-k // 128))) * _FP8_W_SCALE).astype(np.float32)
        out["g_norm"] = _bf16_normal(rng, (H,), 0.02, 1.0)
        out["g_qa"] = _bf16_normal(rng, (qr,), 0.02, 1.0)
        bt = _page_table(rng, cfg)
        out["block_table"] = bt
        out["context_lens"] = np.full(cfg.n_requests, cfg.context, dtype=np.int32)
        out["key_cache"] = _fp8_codes(rng, (cfg.num_phys_pages, cfg.page_size, hd), _FP8_K_SIGMA)
        out["key_scale"] = (rng.uniform(0.8, 1.25, (cfg.num_phys_pages, cfg.page_size)) * _FP8_K_SCALE).astype(np.float32)
        out["x"] = _bf16_normal(rng, (cfg.m, H), 1.0)
        out["r_in"] = rng.standard_normal((cfg.m, H), dtype=np.float32)
        if cfg.mla_heads:  # drawn last: the indexer's inputs are the same with or without this half
            n = cfg.mla_heads * 128
            out["w_qb"] = _fp8_codes(rng, (n, qr), _FP8_W_SIGMA)
            out["s_qb"] = (rng.uniform(0.8, 1.25, (-(-n // 128), -(-qr // 128))) * _FP8_W_SCALE).astype(np.float32)
            out["w_uk"] = _bf16_normal(rng, (cfg.mla_heads * 512, 128), 0.05)
    else:
        raise ValueError(cfg.workload)
    return out


def algorithmic_bytes(cfg) -> Dict[str, int]:
    """Bytes one pass of the workload must move at least: every weight, scale and norm gain
    once, the prior KV cache (or indexer keys) once, the new cache rows, and the external
    inputs and outputs.  Intermediates and redundant re-reads are excluded."""
    parts: Dict[str, int] = {}
    if cfg.workload in ("qwen3_layer", "qwen3_step"):
        H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
        nq, nkv = cfg.n_q_heads * d, cfg.n_kv_heads * d
        L, M = cfg.num_layers, cfg.m
        wel = 1 if cfg.weight_fp8 else 2
        mats = [(nq + 2 * nkv, H), (H, nq), (2 * I, H), (H, I)]
        parts["weights"] = L * sum(n * k * wel for n, k in mats)
        if cfg.weight_fp8:
            parts["scales"] = L * sum((-(-n // 128)) * (-(-k // 128)) * 4 for n, k in mats)
        parts["norms"] = L * (2 * H + 2 * d) * 2
        prior = cfg.n_requests * (cfg.context - 1)
        parts["kv_read"] = L * prior * 2 * nkv * 2
        parts["kv_write"] = L * cfg.n_requests * 2 * nkv * 2
        parts["act_in"] = M * H * (2 + 4)
        if cfg.workload == "qwen3_step":
            parts["lm_head"] = cfg.vocab * H * 2 + H * 2
            parts["logits_out"] = M * cfg.vocab * 4 + M * 4
        else:
            parts["act_out"] = M * H * (2 + 4)
    elif cfg.workload == "indexer_front":
        H, qr, nh, hd = cfg.hidden, cfg.idx_q_rank, cfg.idx_heads, cfg.idx_head_dim
        mats = [(qr, H), (nh, H), (hd, H), (nh * hd, qr)]
        parts["weights"] = sum(n * k for n, k in mats)
        parts["scales"] = sum((-(-n // 128)) * (-(-k // 128)) * 4 for n, k in mats)
        parts["norms"] = (H + qr) * 2
        M = cfg.m
        prior = cfg.n_requests * (cfg.context - cfg.tokens_per_request)
        parts["keys_read"] = prior * (hd + 4)
        parts["keys_write"] = M * (hd + 4)
        parts["act_in"] = M * H * (2 + 4)
        parts["score_out"] = M * cfg.context * 4
        if cfg.topk:
            parts["topk_out"] = M * cfg.topk * 4  # the scores it reads are this workload's own output
        if cfg.mla_heads:
            n = cfg.mla_heads * 128
            parts["mla_weights"] = n * qr + (-(-n // 128)) * (-(-qr // 128)) * 4 + cfg.mla_heads * 512 * 128 * 2
            parts["qlat_out"] = M * cfg.mla_heads * 512 * 2
    parts["total"] = sum(parts.values())
    return parts
