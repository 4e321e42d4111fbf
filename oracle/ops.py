"""One plain float64 function per step of the decode-layer chain.

Every function computes its step's plain definition; nothing is blocked, fused or
reordered beyond what the definition states.  Inputs that the chain materialises
in a storage format (bf16, e4m3) are passed in already decoded to float64.

Sources (pages):
  * handbook "PDL and megakernels", decode estimate: the per-layer kernel list
    (fused residual-add + RMSNorm, QKV projection, fused QK-norm + RoPE, KV-cache
    write, attention, O projection, gate-up projection, SiLU-mul, down projection;
    final norm, lm_head and sampling at the tail).
  * MegaRTP page, section 4: Add + RMSNorm + Quant (A0), the FP8 GEMM branches,
    RoPE + cache write (B1), the paged indexer score (E1) over block_table /
    context_lens.
  * "kernel prologue/epilogue" page, section 4 (attention epilogue): online softmax
    starts from m = -inf, l = 0; a fully masked row has l = 0; split-KV writes
    (O_i, lse_i) per split and the combine weights are w_i = exp(lse_i - lse).
"""
from __future__ import annotations

import numpy as np

from .numerics import round_f32


def add_residual(x: np.ndarray, r_in: np.ndarray) -> np.ndarray:
    """r1 = fp32(r_in + x): the residual stream is kept in fp32."""
    return round_f32(np.asarray(r_in, np.float64) + np.asarray(x, np.float64))


def rmsnorm(r: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """h = r / sqrt(mean(r^2) + eps) * gamma over the last axis (float64, unrounded)."""
    r = np.asarray(r, np.float64)
    ms = np.mean(r * r, axis=-1, keepdims=True)
    return r / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def linear(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Y = H W^T with W stored [N, K] (float64; exact products, one rounding per add)."""
    return np.asarray(h, np.float64) @ np.asarray(w, np.float64).T


def linear_w8a8(qa: np.ndarray, sa: np.ndarray, qw: np.ndarray, sw: np.ndarray, block: int = 128) -> np.ndarray:
    """Block-scaled FP8 projection:
        Y[m, n] = sa[m] * sum_kb sw[n // 128, kb] * sum_{k in kb} qa[m, k] * qw[n, k]
    qa, qw are decoded e4m3 values; each inner block sum is exact in float64."""
    qa = np.asarray(qa, np.float64)
    qw = np.asarray(qw, np.float64)
    m, k = qa.shape
    n = qw.shape[0]
    kb_n = -(-k // block)
    sw_rows = np.repeat(np.asarray(sw, np.float64), block, axis=0)[:n]  # [N, kb]
    y = np.zeros((m, n))
    for kb in range(kb_n):
        part = qa[:, kb * block:(kb + 1) * block] @ qw[:, kb * block:(kb + 1) * block].T
        y += part * sw_rows[:, kb][None, :]
    return y * np.asarray(sa, np.float64)[:, None]


def rope_neox(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE over the full last axis (d even):
        angle_i = pos * theta^(-2i/d),  i < d/2
        (x_i, x_{i+d/2}) -> (x_i cos - x_{i+d/2} sin, x_{i+d/2} cos + x_i sin)
    ``pos`` broadcasts against x[..., 0]."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half) / d)
    ang = np.asarray(pos, np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def cache_slots(block_table: np.ndarray, positions: np.ndarray, request_of_row: np.ndarray, page_size: int):
    """Physical (page, offset) for each new row: page = bt[r][p // P], offset = p % P."""
    pos = np.asarray(positions, np.int64)
    req = np.asarray(request_of_row, np.int64)
    page = np.asarray(block_table, np.int64)[req, pos // page_size]
    return page, pos % page_size


def token_slots(block_table_row: np.ndarray, n_tokens: int, page_size: int) -> np.ndarray:
    """The page walk: physical slot page * P + offset of tokens 0..n_tokens-1 of one request, with
    page = block_table_row[t // P] and offset = t % P (the block table maps logical to physical pages)."""
    t = np.arange(n_tokens)
    return np.asarray(block_table_row, np.int64)[t // page_size] * page_size + t % page_size


def gather_tokens(cache: np.ndarray, block_table_row: np.ndarray, n_tokens: int, page_size: int) -> np.ndarray:
    """Tokens 0..n_tokens-1 of one request from a paged cache [pages, P, ...] via its page walk."""
    slots = token_slots(block_table_row, n_tokens, page_size)
    return cache[slots // page_size, slots % page_size]


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """One query row against T keys/values of its kv head: o = softmax(q k^T / sqrt(d)) v."""
    d = q.shape[-1]
    s = (k @ q) / np.sqrt(d)
    return softmax(s) @ v


def attention_partial(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """One split of split-KV attention: (O_i normalised within the split, lse_i).
    An empty split returns (0, -inf)."""
    d = q.shape[-1]
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1]), -np.inf
    s = (k @ q) / np.sqrt(d)
    m = np.max(s)
    e = np.exp(s - m)
    l = np.sum(e)
    return (e @ v) / l, m + np.log(l)


def combine_splits(os: np.ndarray, lses: np.ndarray) -> np.ndarray:
    """o = sum_i exp(lse_i - lse) O_i with lse = log sum_i exp(lse_i); empty splits weigh 0."""
    lses = np.asarray(lses, np.float64)
    mx = np.max(lses)
    lse = mx + np.log(np.sum(np.exp(lses - mx)))
    w = np.exp(lses - lse)
    return np.tensordot(w, np.asarray(os, np.float64), axes=(0, 0))


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """m = g * sigmoid(g) * u = g / (1 + exp(-g)) * u."""
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, np.float64)


def argmax_first(logits: np.ndarray) -> int:
    """Greedy token: the smallest index attaining the maximum."""
    logits = np.asarray(logits)
    return int(np.flatnonzero(logits == np.max(logits))[0])


def indexer_score(qi: np.ndarray, w: np.ndarray, kq: np.ndarray, sk: np.ndarray, pos: int) -> np.ndarray:
    """Paged indexer score for one query token over T keys:
        score[t] = sum_h w[h] * max(0, sk[t] * (qi[h] . kq[t]))   for t <= pos, -inf otherwise
    qi [heads, d], w [heads], kq [T, d] decoded key values, sk [T] key scales."""
    T = kq.shape[0]
    dots = np.asarray(qi, np.float64) @ np.asarray(kq, np.float64).T  # [heads, T]
    relu = np.maximum(0.0, dots * np.asarray(sk, np.float64)[None, :])
    score = np.asarray(w, np.float64) @ relu
    score = np.where(np.arange(T) <= pos, score, -np.inf)
    return score


def topk_positions(scores: np.ndarray, n_valid: int, k: int) -> np.ndarray:
    """Top-k selection after the indexer score (MegaRTP page: the Top-2048 that follows the paged
    indexer score): the positions of the k largest of scores[:n_valid], ties to the smaller
    position, listed in ascending order; -1 fills the k entries past n_valid.  (The pages fix
    neither the tie rule nor the output order; these are the plainest.)"""
    s = np.asarray(scores[:n_valid], np.float64)
    pos = np.arange(n_valid)
    order = np.lexsort((pos, -s))  # by score descending, then by position ascending
    out = np.full(k, -1, np.int64)
    sel = np.sort(order[:k])
    out[:len(sel)] = sel
    return out
