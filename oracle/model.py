"""The workloads, composed op by op from ``oracle.ops`` in the chain's order.

Qwen3-shaped decode layer (handbook decode estimate, per-layer kernel list):
    r1 = fp32(r_in + x);  h1 = RMSNorm(r1) * g_attn          -> bf16 (FP8 path: per-token e4m3)
    qkv = h1 W_qkv^T;  q | k | v column split, head h at columns [h d, (h+1) d)
    q, k: per-head RMSNorm over d (g_q, g_k), then rotate-half RoPE at pos   -> bf16
    cache write: K[bt[r][p // P], p % P, hk] = k, V likewise (p = ctx_r - 1)
    o_h = softmax(q_h K^T / sqrt(d)) V over t < ctx_r, kv head hk = h // (Hq / Hkv) -> bf16 (FP8: e4m3)
    a = bf16(o W_o^T);  r2 = fp32(r1 + a);  h2 = RMSNorm(r2) * g_mlp  -> bf16 (FP8: e4m3)
    [G U] = h2 W_gu^T;  m = G sigmoid(G) U                     -> bf16 (FP8: e4m3)
    y = bf16(m W_down^T);   the layer returns (y, r2)
Full decode step: layers chained with x_{l+1} = y_l, r_in,{l+1} = r2_l; then
    r_f = fp32(r2 + y);  h_f = bf16(RMSNorm(r_f) g_final);  logits = fp32(h_f W_lm^T);
    token = smallest index of the maximum.
Indexer front (MegaRTP page, section 4, the A0 -> {B0, C0, B1} -> D1 -> E1 DAG):
    A0: r1 = fp32(r_in + x); (hq, sh) = e4m3 per token of RMSNorm(r1) g_norm
    B0: q_a = W8A8(hq, W_qa); (qaq, sqa) = e4m3 per token of RMSNorm(q_a) g_qa
    C0: w = fp32(W8A8(hq, W_w))                               [M, heads]
    B1: k = RoPE(W8A8(hq, W_k), pos); (kq, sk) = e4m3 per token; key cache write at
        (bt[r][pos // P], pos % P)
    D1: qi = bf16(RoPE(W8A8(qaq, W_qi) as [M, heads, d], pos))
    E1: score[m, t] = sum_h w[m, h] ReLU(sk[t] (qi[m, h] . kq[t])) for t <= pos(m), else -inf
    top-k (optional, the step after E1): the positions of the k largest fp32 scores t <= pos(m)
    D0 / D2 (optional, the main-MLA query half): q_nope = bf16(W8A8(qaq, W_qb)) per head, then
        q_lat[m, h] = bf16(W_uk[h] q_nope[m, h])

Every materialised tensor is returned both before (``*_pre``) and after its storage
rounding; the next step consumes the rounded value.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import ops
from .numerics import (bf16_admissible, bf16_bits_to_f64, dequant_per_token, dequant_weight_blocks, e4m3_ambiguous, e4m3_decode,
                       e4m3_other_code, f64_to_bf16_bits, quant_per_token, round_bf16, round_f32)


def _w(inp: Dict[str, np.ndarray], name: str, layer: int, cfg) -> np.ndarray:
    """Decoded weight of one layer (bf16 bits, or e4m3 codes x block scales)."""
    if cfg.weight_fp8:
        return dequant_weight_blocks(inp[name][layer], inp["s_" + name[2:]][layer])
    return bf16_bits_to_f64(inp[name][layer])


def _quant(pre: np.ndarray, key: str, ties, out: Dict[str, np.ndarray]) -> tuple:
    """Per-token e4m3 quantisation of ``pre`` (round to nearest even in the fp32 ratio pre / s).

    ``ties`` (optional) resolves the oracle's own ambiguous decisions and nothing else.  A
    value that lies within delta of the midpoint between two e4m3 codes may be coded either way
    by an evaluation that reproduces it only to within delta (an fp32 evaluation that sums in
    another order); one code step at the top binade is 1/14 of the row's largest value and
    reaches every output of the next projection.  The oracle marks those elements itself:
    ``ties.delta(key)`` gives (delta_rel, delta_abs) in code units and the ambiguous set is
    {|v - midpoint| <= delta_rel |v| + delta_abs}.  ``ties.choose(key, v, codes, s, ambiguous)``
    returns where to take the other code of the enclosing pair; a choice outside the ambiguous
    set is an error.  Without ``ties`` every decision is the oracle's own."""
    codes, s = quant_per_token(pre)
    if ties is None:
        return codes, s
    v = round_f32(pre / s[..., None])
    amb = e4m3_ambiguous(v, *ties.delta(key))
    other = np.asarray(ties.choose(key, v, codes, s, amb), dtype=bool)
    if np.any(other & ~amb):
        raise ValueError(f"{key}: a code choice outside the oracle's ambiguity set")
    out[key + "_ambiguous"] = amb
    return np.where(other, e4m3_other_code(v, codes), codes), s


def _round_bf16(pre: np.ndarray, key: str, ties) -> np.ndarray:
    """bf16 materialisation of ``pre`` (round to nearest even).  Like ``_quant`` for the e4m3
    codes: an evaluation that reproduces ``pre`` only to within delta may round it to any bf16
    value that some value within delta of it rounds to, and one step of q, k or v moves that
    head's logits and outputs.  ``ties`` (optional, with bf16 entries) gives delta from the
    oracle's own values (``ties.bf16_delta(key, pre)``); where more than one bf16 value is
    admissible the oracle takes the value ``ties.choose_bf16`` returns, and a value that is not
    admissible, or differs where only one is, is an error."""
    rne = round_bf16(pre)
    if ties is None or not getattr(ties, "has_bf16", lambda k: False)(key):
        return rne
    lo, hi = bf16_admissible(pre, ties.bf16_delta(key, pre))
    amb = lo != hi
    chosen = np.asarray(ties.choose_bf16(key, pre, rne, amb), dtype=np.float64)
    if np.any((chosen != rne) & ~amb) or np.any((chosen < lo) | (chosen > hi)):
        raise ValueError(f"{key}: a bf16 value the oracle does not admit")
    return chosen


def _w8a8(cfg, inp, name, layer, codes, scale):
    return ops.linear_w8a8(e4m3_decode(codes), scale, e4m3_decode(inp[name][layer]), inp["s_" + name[2:]][layer])


def qwen3_layer(cfg, inp: Dict[str, np.ndarray], layer: int, x: np.ndarray, r_in: np.ndarray,
                k_cache: np.ndarray, v_cache: np.ndarray, ties=None) -> Dict[str, np.ndarray]:
    """One decode layer.  x: decoded bf16 values [M, H]; r_in: fp32 values [M, H].
    k_cache / v_cache: this layer's decoded caches [pages, P, Hkv, d] (updated in place
    with the new rows).  Rows are requests (one token per request).
    ties: optional resolution of ambiguous FP8 decisions at "h1q", "oq", "h2q", "mq" (``_quant``) and
    of the bf16 roundings of "q", "k", "v" (``_round_bf16``)."""
    H, d = cfg.hidden, cfg.head_dim
    Hq, Hkv = cfg.n_q_heads, cfg.n_kv_heads
    g = Hq // Hkv
    M = x.shape[0]
    ctx = inp["context_lens"].astype(np.int64)
    pos = ctx - 1
    req = np.arange(M)
    out: Dict[str, np.ndarray] = {}
    fp8 = cfg.weight_fp8

    r1 = ops.add_residual(x, r_in)
    h1_pre = ops.rmsnorm(r1, bf16_bits_to_f64(inp["g_attn"][layer]), cfg.rms_eps)
    out["r1"] = r1
    out["h1_pre"] = h1_pre
    if fp8:
        h1q, s1 = _quant(h1_pre, "h1q", ties, out)
        out["h1q"], out["s1"] = h1q, s1
        qkv = _w8a8(cfg, inp, "w_qkv", layer, h1q, s1)
    else:
        h1 = round_bf16(h1_pre)
        out["h1"] = h1
        qkv = ops.linear(h1, _w(inp, "w_qkv", layer, cfg))
    out["qkv"] = qkv
    q = qkv[:, :Hq * d].reshape(M, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(M, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(M, Hkv, d)
    qn = ops.rmsnorm(q, bf16_bits_to_f64(inp["g_q"][layer]), cfg.rms_eps)
    kn = ops.rmsnorm(k, bf16_bits_to_f64(inp["g_k"][layer]), cfg.rms_eps)
    q_pre = ops.rope_neox(qn, pos[:, None], cfg.rope_theta)
    k_pre = ops.rope_neox(kn, pos[:, None], cfg.rope_theta)
    out["q_pre"], out["k_pre"], out["v_pre"] = q_pre, k_pre, v
    qb, kb, vb = _round_bf16(q_pre, "q", ties), _round_bf16(k_pre, "k", ties), _round_bf16(v, "v", ties)
    out["q"], out["k"], out["v"] = qb, kb, vb

    page, off = ops.cache_slots(inp["block_table"], pos, req, cfg.page_size)
    out["slot_page"], out["slot_off"] = page, off
    k_cache[page, off] = kb
    v_cache[page, off] = vb

    o_pre = np.zeros((M, Hq, d))
    for mi in range(M):
        K = ops.gather_tokens(k_cache, inp["block_table"][mi], int(ctx[mi]), cfg.page_size)  # [T, Hkv, d]
        V = ops.gather_tokens(v_cache, inp["block_table"][mi], int(ctx[mi]), cfg.page_size)
        for h in range(Hq):
            hk = h // g
            o_pre[mi, h] = ops.attention_decode(qb[mi, h], K[:, hk], V[:, hk])
    o_pre = o_pre.reshape(M, Hq * d)
    out["o_pre"] = o_pre
    if fp8:
        oq, so = _quant(o_pre, "oq", ties, out)
        out["oq"], out["so"] = oq, so
        a_pre = _w8a8(cfg, inp, "w_o", layer, oq, so)
    else:
        o = round_bf16(o_pre)
        out["o"] = o
        a_pre = ops.linear(o, _w(inp, "w_o", layer, cfg))
    a = round_bf16(a_pre)
    out["a_pre"], out["a"] = a_pre, a
    r2 = ops.add_residual(a, r1)
    out["r2"] = r2
    h2_pre = ops.rmsnorm(r2, bf16_bits_to_f64(inp["g_mlp"][layer]), cfg.rms_eps)
    out["h2_pre"] = h2_pre
    I = cfg.inter
    if fp8:
        h2q, s2 = _quant(h2_pre, "h2q", ties, out)
        out["h2q"], out["s2"] = h2q, s2
        gu = _w8a8(cfg, inp, "w_gu", layer, h2q, s2)
    else:
        h2 = round_bf16(h2_pre)
        out["h2"] = h2
        gu = ops.linear(h2, _w(inp, "w_gu", layer, cfg))
    m_pre = ops.silu_mul(gu[:, :I], gu[:, I:])
    out["m_pre"] = m_pre
    if fp8:
        mq, sm = _quant(m_pre, "mq", ties, out)
        out["mq"], out["sm"] = mq, sm
        y_pre = _w8a8(cfg, inp, "w_down", layer, mq, sm)
    else:
        mb = round_bf16(m_pre)
        out["m"] = mb
        y_pre = ops.linear(mb, _w(inp, "w_down", layer, cfg))
    out["y_pre"] = y_pre
    out["y"] = round_bf16(y_pre)
    return out


def run_qwen3_layer(cfg, inp: Dict[str, np.ndarray], layer: int = 0, ties=None) -> Dict[str, np.ndarray]:
    """Single-layer workload: returns the layer outputs and the updated caches (decoded)."""
    k_cache = bf16_bits_to_f64(inp["k_cache"][layer])
    v_cache = bf16_bits_to_f64(inp["v_cache"][layer])
    out = qwen3_layer(cfg, inp, layer, bf16_bits_to_f64(inp["x"]), inp["r_in"].astype(np.float64),
                      k_cache, v_cache, ties)
    out["k_cache"], out["v_cache"] = k_cache, v_cache
    return out


def run_qwen3_step(cfg, inp: Dict[str, np.ndarray], keep_layers: bool = False) -> Dict[str, np.ndarray]:
    """Full decode step: num_layers layers, final norm, lm_head, greedy argmax.
    Caches are decoded one layer at a time to bound memory."""
    x = bf16_bits_to_f64(inp["x"])
    r = inp["r_in"].astype(np.float64)
    res: Dict[str, np.ndarray] = {"layers": []}
    for l in range(cfg.num_layers):
        kc = bf16_bits_to_f64(inp["k_cache"][l])
        vc = bf16_bits_to_f64(inp["v_cache"][l])
        o = qwen3_layer(cfg, inp, l, x, r, kc, vc)
        if keep_layers:
            res["layers"].append(o)
        else:
            res["layers"].append({k2: o[k2] for k2 in ("y_pre", "y", "r2", "slot_page", "slot_off", "k", "v",
                                                            "k_pre", "v_pre")})
        x, r = o["y"], o["r2"]
    r_f = ops.add_residual(x, r)
    hf_pre = ops.rmsnorm(r_f, bf16_bits_to_f64(inp["g_final"]), cfg.rms_eps)
    hf = round_bf16(hf_pre)
    logits_pre = ops.linear(hf, bf16_bits_to_f64(inp["w_lm"]))
    logits = round_f32(logits_pre)
    res.update(r_f=r_f, hf_pre=hf_pre, hf=hf, logits_pre=logits_pre, logits=logits,
               token=np.array([ops.argmax_first(logits[i]) for i in range(logits.shape[0])], dtype=np.int64))
    return res


def run_indexer_front(cfg, inp: Dict[str, np.ndarray], ties=None) -> Dict[str, np.ndarray]:
    """ties: optional resolution of ambiguous FP8 decisions at "hq", "qaq", "kq" (``_quant``)."""
    H, qr, nh, hd = cfg.hidden, cfg.idx_q_rank, cfg.idx_heads, cfg.idx_head_dim
    R, T = cfg.n_requests, cfg.tokens_per_request
    M = R * T
    ctx = inp["context_lens"].astype(np.int64)
    req = np.repeat(np.arange(R), T)
    pos = ctx[req] - T + np.tile(np.arange(T), R)
    out: Dict[str, np.ndarray] = {"pos": pos}

    def w8a8(name, codes, scale):
        return ops.linear_w8a8(e4m3_decode(codes), scale, e4m3_decode(inp[name]), inp["s_" + name[2:]])

    r1 = ops.add_residual(bf16_bits_to_f64(inp["x"]), inp["r_in"].astype(np.float64))
    h_pre = ops.rmsnorm(r1, bf16_bits_to_f64(inp["g_norm"]), cfg.rms_eps)
    hq, sh = _quant(h_pre, "hq", ties, out)
    out.update(r1=r1, h_pre=h_pre, hq=hq, sh=sh)
    # B0
    qa = w8a8("w_qa", hq, sh)
    qa_n = ops.rmsnorm(qa, bf16_bits_to_f64(inp["g_qa"]), cfg.rms_eps)
    qaq, sqa = _quant(qa_n, "qaq", ties, out)
    out.update(qa=qa, qa_n=qa_n, qaq=qaq, sqa=sqa)
    # C0
    w_pre = w8a8("w_w", hq, sh)
    w = round_f32(w_pre)
    out.update(w_pre=w_pre, w=w)
    # B1
    k_lin = w8a8("w_k", hq, sh)
    k_pre = ops.rope_neox(k_lin, pos, cfg.rope_theta)
    kq, sk = _quant(k_pre, "kq", ties, out)
    out.update(k_lin=k_lin, k_pre=k_pre, kq=kq, sk=sk)
    page, off = ops.cache_slots(inp["block_table"], pos, req, cfg.page_size)
    key_cache = inp["key_cache"].copy()
    key_scale = inp["key_scale"].astype(np.float64).copy()
    key_cache[page, off] = kq
    key_scale[page, off] = sk
    out.update(slot_page=page, slot_off=off, key_cache=key_cache, key_scale=key_scale)
    # D1
    qi_lin = w8a8("w_qi", qaq, sqa).reshape(M, nh, hd)
    qi_pre = ops.rope_neox(qi_lin, pos[:, None], cfg.rope_theta)
    qi = round_bf16(qi_pre)
    out.update(qi_pre=qi_pre, qi=qi)
    # E1
    ctx_max = int(ctx.max())
    score_pre = np.full((M, ctx_max), -np.inf)
    for mi in range(M):
        r = req[mi]
        K = ops.gather_tokens(e4m3_decode(key_cache), inp["block_table"][r], int(ctx[r]), cfg.page_size)
        S = ops.gather_tokens(key_scale, inp["block_table"][r], int(ctx[r]), cfg.page_size)
        score_pre[mi, :ctx[r]] = ops.indexer_score(qi[mi], w[mi], K, S, int(pos[mi]))
    out["score_pre"] = score_pre
    out["score"] = round_f32(score_pre)
    # main-MLA query half (the D0 -> D2 edge of the MegaRTP page's attention-pre graph, section 4):
    # D0 q_nope[h] = bf16(W8A8(qaq, W_qb) rows h 128 .. h 128 + 127); D2 q_lat[h] = bf16(q_nope[h] W_uk[h]^T)
    nm = getattr(cfg, "mla_heads", 0)
    if nm:
        qn_pre = w8a8("w_qb", qaq, sqa).reshape(M, nm, 128)
        qn = round_bf16(qn_pre)
        w_uk = bf16_bits_to_f64(inp["w_uk"]).reshape(nm, 512, 128)
        ql_pre = np.einsum("mhk,hnk->mhn", qn, w_uk)
        out.update(qn_pre=qn_pre, qn=qn, qlat_pre=ql_pre, qlat=round_bf16(ql_pre))
    # top-k over each token's keys t <= pos, on the scores as stored (fp32)
    if getattr(cfg, "topk", 0):
        out["topk"] = np.stack([ops.topk_positions(out["score"][mi], int(pos[mi]) + 1, cfg.topk) for mi in range(M)])
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return f64_to_bf16_bits(x)


def dequant(codes, s):
    return dequant_per_token(codes, s)
