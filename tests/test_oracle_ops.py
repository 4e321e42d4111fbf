"""Pins of the per-step oracle functions: closed forms, invariants, brute-force loops."""
import math

import numpy as np
import pytest

from oracle import ops


def test_add_rmsnorm_brute_force_and_unit_rms():
    rng = np.random.default_rng(0)
    x, r, g = rng.standard_normal(8), rng.standard_normal(8), rng.uniform(0.5, 1.5, 8)
    r1 = ops.add_residual(x, r)
    assert np.all(r1 == (r + x).astype(np.float32))
    ms = 0.0
    for i in range(8):
        ms += r1[i] * r1[i]
    ms /= 8
    ref = [r1[i] / math.sqrt(ms + 1e-6) * g[i] for i in range(8)]
    assert np.allclose(ops.rmsnorm(r1, g, 1e-6), ref, rtol=1e-14, atol=0)
    h = ops.rmsnorm(r1, np.ones(8), 1e-6)
    assert abs(np.sqrt(np.mean(h * h)) - np.sqrt(ms / (ms + 1e-6))) < 1e-14
    assert np.allclose(ops.rmsnorm(3.5 * r1, g, 0.0), ops.rmsnorm(r1, g, 0.0), rtol=1e-14)


def test_rope_closed_form_and_invariants():
    # d = 2: a plain rotation by pos radians (theta_0 = pos * base^0)
    out = ops.rope_neox(np.array([1.0, 0.0]), math.pi / 2, 1e6)
    assert np.allclose(out, [0.0, 1.0], atol=1e-15)
    out = ops.rope_neox(np.array([0.0, 1.0]), math.pi / 2, 1e6)
    assert np.allclose(out, [-1.0, 0.0], atol=1e-15)
    rng = np.random.default_rng(1)
    d = 128
    x, q, k = rng.standard_normal((3, d))
    assert np.array_equal(ops.rope_neox(x, 0, 1e6), x)
    y = ops.rope_neox(x, 777, 1e6)
    half = d // 2
    assert np.allclose(x[:half] ** 2 + x[half:] ** 2, y[:half] ** 2 + y[half:] ** 2, rtol=1e-12)
    assert np.allclose(ops.rope_neox(ops.rope_neox(x, 100, 1e6), 23, 1e6), ops.rope_neox(x, 123, 1e6), atol=1e-12)
    a = np.dot(ops.rope_neox(q, 900, 1e6), ops.rope_neox(k, 250, 1e6))
    b = np.dot(ops.rope_neox(q, 650, 1e6), k)
    assert abs(a - b) < 1e-10
    # pair i uses frequency base^(-2i/d): pair 1 of d=4 at pos 1, base 100 rotates by 0.1 rad
    v = ops.rope_neox(np.array([0.0, 1.0, 0.0, 0.0]), 1.0, 100.0)
    assert np.allclose(v, [0.0, math.cos(0.1), 0.0, math.sin(0.1)], atol=1e-15)


def test_softmax_and_attention_special_cases():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((4, 37)) * 5
    assert np.allclose(ops.softmax(s).sum(axis=1), 1.0, atol=1e-15)
    d = 16
    q, k, v = rng.standard_normal(d), rng.standard_normal((1, d)), rng.standard_normal((1, d))
    assert np.array_equal(ops.attention_decode(q, k, v), v[0])  # one key: o = v exactly
    K = np.tile(rng.standard_normal(d), (9, 1))
    V = rng.standard_normal((9, d))
    assert np.allclose(ops.attention_decode(q, K, V), V.mean(axis=0), atol=1e-14)
    # brute force
    K, V = rng.standard_normal((23, d)), rng.standard_normal((23, d))
    sc = [sum(q[i] * K[t, i] for i in range(d)) / math.sqrt(d) for t in range(23)]
    mx = max(sc)
    e = [math.exp(x - mx) for x in sc]
    ref = [sum(e[t] * V[t, i] for t in range(23)) / sum(e) for i in range(d)]
    assert np.allclose(ops.attention_decode(q, K, V), ref, atol=1e-13)


def test_split_kv_combine_equals_unsplit():
    rng = np.random.default_rng(3)
    d, T = 32, 100
    q, K, V = rng.standard_normal(d), rng.standard_normal((T, d)), rng.standard_normal((T, d))
    full = ops.attention_decode(q, K, V)
    bounds = [0, 7, 7, 40, 64, 100]  # includes an empty split
    parts = [ops.attention_partial(q, K[a:b], V[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    assert parts[1][1] == -np.inf and not parts[1][0].any()
    o = ops.combine_splits(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
    assert np.max(np.abs(o - full)) < 1e-12


def test_linear_brute_force_and_w8a8_exact_integers():
    rng = np.random.default_rng(4)
    h, w = rng.standard_normal((3, 5)), rng.standard_normal((4, 5))
    ref = np.array([[sum(h[m, k] * w[n, k] for k in range(5)) for n in range(4)] for m in range(3)])
    assert np.allclose(ops.linear(h, w), ref, atol=1e-14)
    # integer-valued e4m3 operands, unit scales: exact integer result
    qa = rng.integers(-8, 9, (2, 300)).astype(float)
    qw = rng.integers(-8, 9, (3, 300)).astype(float)
    y = ops.linear_w8a8(qa, np.ones(2), qw, np.ones((1, 3)))
    assert np.array_equal(y, qa @ qw.T)
    # scales: brute force over blocks
    sa, sw = np.array([0.5, 2.0]), np.array([[1.0, 0.25, 4.0]])
    y = ops.linear_w8a8(qa, sa, qw, sw)
    for m in range(2):
        for n in range(3):
            acc = 0.0
            for kb in range(3):
                acc += sw[0, kb] * sum(qa[m, k] * qw[n, k] for k in range(kb * 128, min(300, kb * 128 + 128)))
            assert y[m, n] == sa[m] * acc


def test_silu_mul_closed_form():
    assert ops.silu_mul(0.0, 5.0) == 0.0
    assert abs(ops.silu_mul(40.0, 1.0) - 40.0) < 1e-12
    g = np.linspace(-6, 6, 25)
    assert np.allclose(ops.silu_mul(g, 2.0), 2 * g * (1 / (1 + np.exp(-g))), rtol=1e-15)


def test_cache_slots_bit_exact():
    rng = np.random.default_rng(5)
    bt = rng.permutation(64).astype(np.int32).reshape(4, 16)
    pos = np.array([0, 15, 16, 255])
    req = np.array([0, 1, 2, 3])
    page, off = ops.cache_slots(bt, pos, req, 16)
    for i in range(4):
        assert page[i] == bt[req[i], pos[i] // 16] and off[i] == pos[i] % 16
    cache = np.arange(64 * 16).reshape(64, 16)
    tok = ops.gather_tokens(cache, bt[2], 40, 16)
    assert [int(t) for t in tok] == [int(bt[2][t // 16]) * 16 + t % 16 for t in range(40)]
    # the page walk: one physical slot per logical token, brute force; with a permutation table the
    # walks of all requests over their full page lists visit every physical slot exactly once
    walk = ops.token_slots(bt[1], 37, 16)
    for t in range(37):
        page = None
        for logical, phys in enumerate(bt[1]):
            if logical == t // 16:
                page = int(phys)
        assert walk[t] == page * 16 + (t - (t // 16) * 16)
    every = np.concatenate([ops.token_slots(bt[r], 256, 16) for r in range(4)])
    assert np.array_equal(np.sort(every), np.arange(64 * 16))


def test_argmax_ties_smallest_index():
    assert ops.argmax_first(np.array([1.0, 3.0, 3.0, -1.0])) == 1
    assert ops.argmax_first(np.array([5.0])) == 0


def test_indexer_score_brute_force_and_reductions():
    rng = np.random.default_rng(6)
    nh, d, T = 3, 8, 11
    qi, w, kq, sk = rng.standard_normal((nh, d)), rng.standard_normal(nh), rng.standard_normal((T, d)), rng.uniform(0.1, 2, T)
    pos = 6
    s = ops.indexer_score(qi, w, kq, sk, pos)
    for t in range(T):
        if t > pos:
            assert s[t] == -np.inf
            continue
        ref = sum(w[h] * max(0.0, sk[t] * sum(qi[h, i] * kq[t, i] for i in range(d))) for h in range(nh))
        assert abs(s[t] - ref) < 1e-12
    onehot = np.array([0.0, 1.0, 0.0])
    s1 = ops.indexer_score(qi, onehot, kq, sk, T)
    assert np.allclose(s1, sk * np.maximum(0, kq @ qi[1]), atol=1e-14)


def _topk_valid(scores, n_valid, k, got):
    """The defining property, checked pair by pair: min(k, n_valid) distinct positions < n_valid in
    ascending order, -1 after them, and every selected position beats every unselected one (a
    larger score, or an equal score and a smaller position)."""
    n = min(k, n_valid)
    sel = [int(v) for v in got[:n]]
    assert all(v == -1 for v in got[n:])
    assert sel == sorted(set(sel)) and all(0 <= v < n_valid for v in sel)
    rest = [t for t in range(n_valid) if t not in set(sel)]
    for i in sel:
        for j in rest:
            assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j), (i, j)


def test_topk_brute_force_and_special_cases():
    rng = np.random.default_rng(3)
    for trial in range(200):  # small rows with many ties (values from a set of 4)
        n = int(rng.integers(1, 12))
        s = rng.integers(0, 4, n).astype(np.float64) - 1.5
        nv = int(rng.integers(0, n + 1))
        k = int(rng.integers(1, n + 2))
        got = ops.topk_positions(s, nv, k)
        assert got.shape == (k,)
        _topk_valid(s, nv, k, got)
        # brute force: the selected set is the unique one of its size with that property
        if nv <= 8:
            from itertools import combinations
            m = min(k, nv)
            good = [c for c in combinations(range(nv), m)
                    if all(s[i] > s[j] or (s[i] == s[j] and i < j) for i in c for j in range(nv) if j not in c)]
            assert len(good) == 1 and list(good[0]) == [int(v) for v in got[:m]]
    # fewer keys than k: every key, then -1
    assert list(ops.topk_positions(np.array([5.0, -1.0, 2.0]), 3, 5)) == [0, 1, 2, -1, -1]
    # all equal: the first k positions
    assert list(ops.topk_positions(np.zeros(10), 10, 4)) == [0, 1, 2, 3]
    # increasing scores: the last k positions; keys past n_valid are ignored
    assert list(ops.topk_positions(np.arange(10.0), 7, 3)) == [4, 5, 6]
    # -inf and negative scores order below everything finite
    assert list(ops.topk_positions(np.array([-np.inf, -3.0, 0.0, -np.inf]), 4, 2)) == [1, 2]
