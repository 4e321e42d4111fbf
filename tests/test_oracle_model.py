"""The composed oracle workloads against an independent torch-CPU formulation on small
shapes (torch's rms_norm, matmul and scaled_dot_product_attention with GQA; FP8 codes made and
read by torch's own float8_e4m3fn conversion, not by the oracle's codec), plus the cache-write
slots: the bf16 layer, the FP8 (W8A8) layer, the decode step with its tail (final add, norm,
lm_head, argmax) and the indexer front."""
import dataclasses

import numpy as np
import torch
import torch.nn.functional as F

from oracle import model, numerics as nu
from workloads import get_config, make_inputs


def _small_cfg(**kw):
    base = dict(hidden=256, inter=384, n_q_heads=4, n_kv_heads=2, head_dim=64, n_requests=2,
                context=40, page_size=16, random_pages=True)
    base.update(kw)
    return dataclasses.replace(get_config("qwen3_0p6b_layer"), **base)


def _t_e4m3(codes):
    """torch's decoding of e4m3fn code bytes."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64)


def _t_quant(pre):
    """Per-token FP8 with torch's conversion: s = fp32(amax / 448) (1 for an all-zero row), codes =
    float8_e4m3fn(fp32(pre / s)) after clamping to +-448.  Returns (code bytes, dequantised values)."""
    amax = pre.abs().amax(-1, keepdim=True)
    s = torch.where(amax > 0, (amax / 448).to(torch.float32).to(torch.float64), torch.ones_like(amax))
    f8 = (pre / s).to(torch.float32).clamp(-448, 448).to(torch.float8_e4m3fn)
    return f8.view(torch.uint8).numpy(), f8.to(torch.float64) * s


def _t_weight(inp, name, layer=None):
    """Decoded weight: bf16 bits, or e4m3 codes times their 128 x 128 block scales."""
    w = inp[name] if layer is None else inp[name][layer]
    sname = "s_" + name[2:]
    if sname not in inp:
        return torch.from_numpy(nu.bf16_bits_to_f64(w))
    s = torch.from_numpy(np.asarray(inp[sname] if layer is None else inp[sname][layer], np.float64))
    n, k = w.shape
    return _t_e4m3(w) * s.repeat_interleave(128, 0).repeat_interleave(128, 1)[:n, :k]


def _t_rope(t, pos, theta):
    d = t.shape[-1]
    inv = theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = pos[..., None].to(torch.float64) * inv
    cos, sin = torch.cat([ang.cos(), ang.cos()], -1), torch.cat([ang.sin(), ang.sin()], -1)
    return t * cos + torch.cat([-t[..., d // 2:], t[..., :d // 2]], -1) * sin


def _torch_layer(cfg, inp, layer=0, x=None, r_in=None):
    dt = torch.float64
    bf = lambda a: torch.from_numpy(nu.bf16_bits_to_f64(a))
    rb = lambda t: torch.from_numpy(nu.round_bf16(t.numpy()))
    fp8 = cfg.weight_fp8
    codes = {}

    def act(t, key):  # a materialised projection input: bf16, or per-token e4m3 on the FP8 path
        if not fp8:
            return rb(t)
        codes[key], v = _t_quant(t)
        return v

    H, d, Hq, Hkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    x = bf(inp["x"]) if x is None else x
    r_in = torch.from_numpy(inp["r_in"].astype(np.float64)) if r_in is None else r_in
    r1 = (x + r_in).to(torch.float32).to(dt)
    h1 = act(F.rms_norm(r1, (H,), bf(inp["g_attn"][layer]), eps=cfg.rms_eps), "h1q")
    qkv = h1 @ _t_weight(inp, "w_qkv", layer).T
    M = x.shape[0]
    q = qkv[:, :Hq * d].view(M, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].view(M, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].view(M, Hkv, d)
    q = F.rms_norm(q, (d,), bf(inp["g_q"][layer]), eps=cfg.rms_eps)
    k = F.rms_norm(k, (d,), bf(inp["g_k"][layer]), eps=cfg.rms_eps)
    pos = torch.from_numpy(inp["context_lens"].astype(np.int64) - 1)[:, None]
    q = rb(_t_rope(q, pos, cfg.rope_theta))
    k = rb(_t_rope(k, pos, cfg.rope_theta))
    v = rb(v)
    kc, vc = bf(inp["k_cache"][layer]).clone(), bf(inp["v_cache"][layer]).clone()
    bt = torch.from_numpy(inp["block_table"].astype(np.int64))
    outs = []
    for m in range(M):
        ctx = int(inp["context_lens"][m])
        p = ctx - 1
        kc[bt[m, p // cfg.page_size], p % cfg.page_size] = k[m]
        vc[bt[m, p // cfg.page_size], p % cfg.page_size] = v[m]
        t = torch.arange(ctx)
        K = kc[bt[m, t // cfg.page_size], t % cfg.page_size].permute(1, 0, 2)[None]
        V = vc[bt[m, t // cfg.page_size], t % cfg.page_size].permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(q[m][None, :, None, :], K, V, enable_gqa=True)
        outs.append(o[0, :, 0, :].reshape(-1))
    o = act(torch.stack(outs), "oq")
    a = rb(o @ _t_weight(inp, "w_o", layer).T)
    r2 = (r1 + a).to(torch.float32).to(dt)
    h2 = act(F.rms_norm(r2, (H,), bf(inp["g_mlp"][layer]), eps=cfg.rms_eps), "h2q")
    gu = h2 @ _t_weight(inp, "w_gu", layer).T
    mm = act(F.silu(gu[:, :cfg.inter]) * gu[:, cfg.inter:], "mq")
    y = mm @ _t_weight(inp, "w_down", layer).T
    return {"y_pre": y.numpy(), "y": rb(y), "r2": r2, "o": o.numpy(), "k": k.numpy(), "codes": codes}


def test_layer_matches_torch_formulation():
    cfg = _small_cfg()
    inp = make_inputs(cfg, seed=3)
    o = model.run_qwen3_layer(cfg, inp)
    t = _torch_layer(cfg, inp)
    assert np.max(np.abs(o["r2"] - t["r2"].numpy())) < 1e-6
    assert np.max(np.abs(o["o"] - t["o"])) <= 2 * 2.0 ** -8 * np.max(np.abs(t["o"]))
    assert np.max(np.abs(o["y_pre"] - t["y_pre"])) < 1e-3
    # cache rows written at the page-table slots
    for m in range(cfg.n_requests):
        p = cfg.context - 1
        page = inp["block_table"][m, p // cfg.page_size]
        assert np.array_equal(o["k_cache"][page, p % cfg.page_size], o["k"][m])


def test_fp8_layer_matches_torch_formulation():
    """W8A8 layer: every per-token code (h1, o, h2, m) equals torch's float8_e4m3fn conversion of
    torch's own values, and y / r2 agree; the weights are decoded by torch from their code bytes."""
    cfg = dataclasses.replace(_small_cfg(), weight_fp8=True, act_fp8=True, hidden=256, inter=512)
    for seed in (9, 10):
        inp = make_inputs(cfg, seed=seed)
        o = model.run_qwen3_layer(cfg, inp)
        t = _torch_layer(cfg, inp)
        for key in ("h1q", "oq", "h2q", "mq"):
            assert np.array_equal(o[key], t["codes"][key]), (seed, key, int(np.sum(o[key] != t["codes"][key])))
        assert np.max(np.abs(o["r2"] - t["r2"].numpy())) < 1e-6
        assert np.max(np.abs(o["y_pre"] - t["y_pre"])) < 1e-9 * max(1.0, np.max(np.abs(t["y_pre"])))


def test_step_tail_matches_torch_formulation():
    """Three chained layers and the tail (r_f = fp32(r2 + y), bf16 RMSNorm with g_final, fp32
    logits over the vocabulary, first index of the maximum), each side computing its own layers."""
    cfg = dataclasses.replace(_small_cfg(n_requests=2, random_pages=True), workload="qwen3_step",
                              num_layers=3, vocab=700, residual_zero=True)
    inp = make_inputs(cfg, seed=12)
    res = model.run_qwen3_step(cfg, inp)
    x = torch.from_numpy(nu.bf16_bits_to_f64(inp["x"]))
    r = torch.from_numpy(inp["r_in"].astype(np.float64))
    for l in range(cfg.num_layers):
        t = _torch_layer(cfg, inp, l, x, r)
        x, r = t["y"], t["r2"]
    r_f = (x + r).to(torch.float32).to(torch.float64)
    g = torch.from_numpy(nu.bf16_bits_to_f64(inp["g_final"]))
    hf = torch.from_numpy(nu.round_bf16(F.rms_norm(r_f, (cfg.hidden,), g, eps=cfg.rms_eps).numpy()))
    logits = (hf @ torch.from_numpy(nu.bf16_bits_to_f64(inp["w_lm"])).T).to(torch.float32).to(torch.float64)
    assert np.max(np.abs(res["r_f"] - r_f.numpy())) < 1e-6
    assert np.max(np.abs(res["logits"] - logits.numpy())) < 1e-5
    assert np.array_equal(res["token"], torch.argmax(logits, dim=-1).numpy())
    # the tail is not the identity on the last layer: dropping its residual changes the logits
    hf_wrong = F.rms_norm(x.to(torch.float32).to(torch.float64), (cfg.hidden,), g, eps=cfg.rms_eps)
    assert np.max(np.abs(res["hf_pre"] - hf_wrong.numpy())) > 1e-2


def _torch_indexer(cfg, inp):
    """The indexer front in torch on dequantised codes: A0 add + rms_norm + e4m3, B0 q_a + rms_norm +
    e4m3, C0 head weights, B1 key + rotate-half RoPE at ctx - T + j + e4m3 into the paged key cache,
    D1 query heads + RoPE -> bf16, E1 sum over heads of w * ReLU(q . key), masked after the token."""
    H, qr, nh, hd, eps = cfg.hidden, cfg.idx_q_rank, cfg.idx_heads, cfg.idx_head_dim, cfg.rms_eps
    R, T, P = cfg.n_requests, cfg.tokens_per_request, cfg.page_size
    bf = lambda a: torch.from_numpy(nu.bf16_bits_to_f64(a))
    ctx = torch.from_numpy(inp["context_lens"].astype(np.int64))
    req = torch.arange(R).repeat_interleave(T)
    pos = ctx[req] - T + torch.arange(T).repeat(R)
    M = R * T
    r1 = (bf(inp["x"]) + torch.from_numpy(inp["r_in"].astype(np.float64))).to(torch.float32).to(torch.float64)
    hq, h = _t_quant(F.rms_norm(r1, (H,), bf(inp["g_norm"]), eps=eps))
    qaq, qa = _t_quant(F.rms_norm(h @ _t_weight(inp, "w_qa").T, (qr,), bf(inp["g_qa"]), eps=eps))
    w = (h @ _t_weight(inp, "w_w").T).to(torch.float32).to(torch.float64)
    kq, k = _t_quant(_t_rope(h @ _t_weight(inp, "w_k").T, pos, cfg.rope_theta))
    qi = _t_rope((qa @ _t_weight(inp, "w_qi").T).view(M, nh, hd), pos[:, None], cfg.rope_theta)
    qi = torch.from_numpy(nu.round_bf16(qi.numpy()))
    keys = _t_e4m3(inp["key_cache"]) * torch.from_numpy(inp["key_scale"].astype(np.float64))[..., None]
    bt = torch.from_numpy(inp["block_table"].astype(np.int64))
    keys[bt[req, pos // P], pos % P] = k
    score = torch.full((M, int(ctx.max())), -torch.inf, dtype=torch.float64)
    for m in range(M):
        t = torch.arange(int(pos[m]) + 1)
        K = keys[bt[req[m], t // P], t % P]  # [t, hd]
        score[m, :len(t)] = (w[m][:, None] * torch.relu(qi[m] @ K.T)).sum(0)
    out = {"hq": hq, "qaq": qaq, "kq": kq, "score_pre": score.numpy()}
    if cfg.mla_heads:  # D0 Main-Q per head from the normalised q_a, then D2's per-head BMM into the latent
        nm = cfg.mla_heads
        qn = torch.from_numpy(nu.round_bf16((qa @ _t_weight(inp, "w_qb").T).view(M, nm, 128).numpy()))
        w_uk = torch.from_numpy(nu.bf16_bits_to_f64(inp["w_uk"])).view(nm, 512, 128)
        out["qlat_pre"] = torch.bmm(qn.transpose(0, 1), w_uk.transpose(1, 2).contiguous()).transpose(0, 1).numpy()
        out["qn"] = qn.numpy()
    return out


def test_indexer_front_matches_torch_formulation():
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=512, idx_q_rank=256, idx_heads=4,
                              idx_head_dim=64, context=200, page_size=64, mla_heads=3)
    for seed, ctx in ((5, [200, 200]), (6, [9, 131])):  # 9 keys: a request of new keys and one older
        inp = make_inputs(cfg, seed=seed)
        inp["context_lens"] = np.array(ctx, dtype=np.int32)
        o = model.run_indexer_front(cfg, inp)
        t = _torch_indexer(cfg, inp)
        for key in ("hq", "qaq", "kq"):
            assert np.array_equal(o[key], t[key]), (seed, key)
        fin = np.isfinite(t["score_pre"])
        assert np.array_equal(fin, np.isfinite(o["score_pre"]))
        ref = t["score_pre"][fin]
        assert np.max(np.abs(o["score_pre"][fin] - ref)) < 1e-9 * max(1.0, np.max(np.abs(ref)))
        # the main-MLA half: D0's bf16 q_nope bit for bit, D2's latent to rounding
        assert np.array_equal(o["qn"], t["qn"]), seed
        assert np.max(np.abs(o["qlat_pre"] - t["qlat_pre"])) < 1e-9 * max(1.0, np.max(np.abs(t["qlat_pre"])))


def test_step_chains_layers():
    cfg = dataclasses.replace(_small_cfg(n_requests=1, random_pages=False), workload="qwen3_step",
                              num_layers=3, vocab=500, residual_zero=True)
    inp = make_inputs(cfg, seed=4)
    res = model.run_qwen3_step(cfg, inp, keep_layers=True)
    # the second layer run alone on the first layer's outputs gives the same result
    kc = nu.bf16_bits_to_f64(inp["k_cache"][1])
    vc = nu.bf16_bits_to_f64(inp["v_cache"][1])
    l0 = res["layers"][0]
    l1 = model.qwen3_layer(cfg, inp, 1, l0["y"], l0["r2"], kc, vc)
    assert np.array_equal(l1["y"], res["layers"][1]["y"])
    assert res["token"][0] == int(np.argmax(res["logits"][0]))


def test_indexer_front_consistency():
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=512, idx_q_rank=256, idx_heads=4,
                              idx_head_dim=64, context=200, page_size=64)
    inp = make_inputs(cfg, seed=5)
    o = model.run_indexer_front(cfg, inp)
    assert o["score"].shape == (16, 200)
    # causal mask within each request's 8 new tokens
    for mi in range(16):
        p = o["pos"][mi]
        assert np.all(np.isinf(o["score"][mi, p + 1:])) and np.all(np.isfinite(o["score"][mi, :p + 1]))
    # key rows written at their page-table slots, with their scales
    for mi in range(16):
        assert np.array_equal(o["key_cache"][o["slot_page"][mi], o["slot_off"][mi]], o["kq"][mi])
    # score of the newest key equals the direct formula on that token
    mi = 15
    kq = nu.e4m3_decode(o["kq"][mi]) * o["sk"][mi]
    ref = np.sum(o["w"][mi] * np.maximum(0, o["qi"][mi] @ kq))
    assert abs(o["score"][mi, o["pos"][mi]] - ref) < 1e-3 * max(1, abs(ref))


class _Ties:
    """Takes the other enclosing code at the listed elements of the listed points (and nowhere else)."""

    def __init__(self, flips, delta=(0.0, 1e9)):
        self.flips, self._delta = flips, delta

    def delta(self, key):
        return self._delta

    def choose(self, key, v, codes, s, amb):
        take = np.zeros(codes.shape, bool)
        for (r, c) in self.flips.get(key, ()):
            take[r, c] = True
        return take


def test_fp8_ambiguity_resolution_is_exact_and_linear():
    """The FP8 layer with a resolution that takes no choice is the independent layer bit for bit;
    taking the other code of one mq element changes y by that code step times the dequantised
    down-projection column (the layer is linear in the down projection's input), and nothing else."""
    cfg = dataclasses.replace(_small_cfg(), weight_fp8=True, act_fp8=True, hidden=256, inter=512)
    inp = make_inputs(cfg, seed=9)
    own = model.run_qwen3_layer(cfg, inp)
    same = model.run_qwen3_layer(cfg, inp, ties=_Ties({}))
    for key in ("y_pre", "r2", "o_pre", "m_pre", "qkv", "h1q", "oq", "h2q", "mq"):
        assert np.array_equal(same[key], own[key]), key
    row, col = 1, int(np.argmax(np.abs(nu.e4m3_decode(own["mq"][1]) * (np.abs(nu.e4m3_decode(own["mq"][1])) < 448))))
    moved = model.run_qwen3_layer(cfg, inp, ties=_Ties({"mq": [(row, col)]}))
    code, new = int(own["mq"][row, col]), int(moved["mq"][row, col])
    assert new != code and np.sum(moved["mq"] != own["mq"]) == 1
    step = nu.e4m3_decode(np.array([new], np.uint8))[0] - nu.e4m3_decode(np.array([code], np.uint8))[0]
    v = own["m_pre"][row, col] / own["sm"][row]
    lo, hi = nu.e4m3_enclosing(np.array([v]))
    assert abs(step) == hi[0] - lo[0]  # the other member of the enclosing pair
    w_col = nu.dequant_weight_blocks(inp["w_down"][0], inp["s_down"][0])[:, col]
    want = own["y_pre"].copy()
    want[row] += step * own["sm"][row] * w_col
    assert np.allclose(moved["y_pre"], want, rtol=0, atol=1e-12)
    assert np.array_equal(moved["y_pre"][0], own["y_pre"][0])  # other rows untouched
