"""The composed oracle workloads against an independent torch-CPU formulation on small
shapes (torch's rms_norm, matmul and scaled_dot_product_attention with GQA), plus the
cache-write slots."""
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


def _torch_layer(cfg, inp, layer=0):
    dt = torch.float64
    bf = lambda a: torch.from_numpy(nu.bf16_bits_to_f64(a))
    rb = lambda t: t.to(torch.bfloat16).to(dt) if False else torch.from_numpy(nu.round_bf16(t.numpy()))
    H, d, Hq, Hkv = cfg.hidden, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    x, r_in = bf(inp["x"]), torch.from_numpy(inp["r_in"].astype(np.float64))
    r1 = (x + r_in).to(torch.float32).to(dt)
    h1 = rb(F.rms_norm(r1, (H,), bf(inp["g_attn"][layer]), eps=cfg.rms_eps))
    qkv = h1 @ bf(inp["w_qkv"][layer]).T
    M = x.shape[0]
    q = qkv[:, :Hq * d].view(M, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].view(M, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].view(M, Hkv, d)
    q = F.rms_norm(q, (d,), bf(inp["g_q"][layer]), eps=cfg.rms_eps)
    k = F.rms_norm(k, (d,), bf(inp["g_k"][layer]), eps=cfg.rms_eps)
    pos = torch.from_numpy(inp["context_lens"].astype(np.float64) - 1)
    inv = cfg.rope_theta ** (-torch.arange(0, d, 2, dtype=dt) / d)
    ang = pos[:, None] * inv[None, :]
    cos = torch.cat([ang.cos(), ang.cos()], -1)[:, None, :]
    sin = torch.cat([ang.sin(), ang.sin()], -1)[:, None, :]
    rot = lambda t: torch.cat([-t[..., d // 2:], t[..., :d // 2]], -1)
    q = rb(q * cos + rot(q) * sin)
    k = rb(k * cos + rot(k) * sin)
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
    o = rb(torch.stack(outs))
    a = rb(o @ bf(inp["w_o"][layer]).T)
    r2 = (r1 + a).to(torch.float32).to(dt)
    h2 = rb(F.rms_norm(r2, (H,), bf(inp["g_mlp"][layer]), eps=cfg.rms_eps))
    gu = h2 @ bf(inp["w_gu"][layer]).T
    mm = rb(F.silu(gu[:, :cfg.inter]) * gu[:, cfg.inter:])
    y = mm @ bf(inp["w_down"][layer]).T
    return {"y_pre": y.numpy(), "r2": r2.numpy(), "o": o.numpy(), "k": k.numpy()}


def test_layer_matches_torch_formulation():
    cfg = _small_cfg()
    inp = make_inputs(cfg, seed=3)
    o = model.run_qwen3_layer(cfg, inp)
    t = _torch_layer(cfg, inp)
    assert np.max(np.abs(o["r2"] - t["r2"])) < 1e-6
    assert np.max(np.abs(o["o"] - t["o"])) <= 2 * 2.0 ** -8 * np.max(np.abs(t["o"]))
    assert np.max(np.abs(o["y_pre"] - t["y_pre"])) < 1e-3
    # cache rows written at the page-table slots
    for m in range(cfg.n_requests):
        p = cfg.context - 1
        page = inp["block_table"][m, p // cfg.page_size]
        assert np.array_equal(o["k_cache"][page, p % cfg.page_size], o["k"][m])


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
