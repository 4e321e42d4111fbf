"""The C++ planner (through the C ABI, host-only) against the oracle queue builder:
bit-exact queues, thresholds and counts."""
import dataclasses

import numpy as np
import pytest

from oracle import queue as oq
from workloads import get_config


def _both(cfg, W, ctx=None):
    import persistent_megakernel_amd as mk
    plan = mk.Plan(cfg, context_lens=ctx, num_workers=W)
    ref = oq.build_queue(cfg, W, ctx)
    return plan, ref


@pytest.mark.parametrize("name", ["qwen3_0p6b_layer", "qwen3_0p6b_step", "qwen3_8b_layer", "qwen3_8b_layer_fp8",
                                  "qwen3_8b_layer_m64", "indexer_front", "indexer_front_topk",
                                  "attention_pre"])
@pytest.mark.parametrize("W", [1, 7, 148, 256])
def test_queue_bit_exact(name, W):
    cfg = get_config(name)
    plan, ref = _both(cfg, W)
    q = plan.queue()
    assert q.shape == ref["queue"].shape
    assert np.array_equal(q, ref["queue"])
    assert np.array_equal(plan.thresholds(), ref["thresholds"])
    info = plan.info()
    assert info["n_tasks"] == ref["n_tasks"] and info["n_ops"] == ref["n_ops"] and info["n_arrivals"] == ref["n_arrivals"]
    plan.close()


@pytest.mark.parametrize("ctx", [[1], [5], [37], [511], [513], [2048]])
def test_ragged_contexts_bit_exact(ctx):
    cfg = dataclasses.replace(get_config("qwen3_0p6b_layer"), context=max(ctx[0], 16))
    for W in (5, 64, 256):
        plan, ref = _both(cfg, W, ctx)
        assert np.array_equal(plan.queue(), ref["queue"])
        assert np.array_equal(plan.thresholds(), ref["thresholds"])
        oq.check_invariants(ref)
        plan.close()


def test_small_shapes_bit_exact():
    cfg = dataclasses.replace(get_config("qwen3_0p6b_step"), hidden=256, inter=384, n_q_heads=4, n_kv_heads=2,
                              num_layers=3, vocab=1000, context=40)
    for W in (3, 16, 256):
        plan, ref = _both(cfg, W)
        assert np.array_equal(plan.queue(), ref["queue"])
        plan.close()


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("R", [17, 40, 64, 256])
def test_row_groups_bit_exact(fp8, R):
    """Multi-row plans beyond 16 rows (16-row groups), ragged contexts, two layers."""
    cfg = dataclasses.replace(get_config("qwen3_8b_layer_fp8" if fp8 else "qwen3_8b_layer"), hidden=1024,
                              inter=2048, n_q_heads=8, n_kv_heads=2, n_requests=R, context=300, page_size=16,
                              num_layers=2)
    rng = np.random.default_rng(R)
    ctx = [int(c) for c in rng.integers(1, 301, R)]
    for W in (5, 37, 256):
        plan, ref = _both(cfg, W, ctx)
        assert np.array_equal(plan.queue(), ref["queue"])
        assert np.array_equal(plan.thresholds(), ref["thresholds"])
        oq.check_invariants(ref)
        plan.close()


def test_row_group_limits():
    import persistent_megakernel_amd as mk
    base = get_config("qwen3_8b_layer")
    with pytest.raises(mk.MkError, match="at most 256 rows"):
        mk.Plan(dataclasses.replace(base, n_requests=257), num_workers=256)
    mk.Plan(dataclasses.replace(base, n_requests=256), num_workers=256).close()


@pytest.mark.parametrize("topk,mla", [(0, 0), (64, 0), (0, 3), (64, 2)])
def test_indexer_ragged_bit_exact(topk, mla):
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, idx_heads=64,
                              n_requests=2, tokens_per_request=3, context=300, topk=topk, mla_heads=mla)
    for ctx in ([300, 3], [129, 256]):
        for W in (5, 64, 256):
            plan, ref = _both(cfg, W, ctx)
            assert np.array_equal(plan.queue(), ref["queue"])
            assert np.array_equal(plan.thresholds(), ref["thresholds"])
            oq.check_invariants(ref)
            plan.close()


@pytest.mark.parametrize("W", [3, 7, 100, 256])
def test_multi_row_attention_chains(W):
    """Multi-row attention: bit-exact queues with ragged contexts, and the chains of splits they
    encode.  A task continues a chain exactly when the worker's previous instruction is a split of
    the same (request, kv head); it ends one exactly when the next is not; only chain ends signal;
    each pair's chains have slots 0 .. n-1 and cover its splits once; its combine reduces n."""
    ctx = [700, 1, 129, 384, 513]
    cfg = dataclasses.replace(get_config("qwen3_8b_layer"), n_requests=len(ctx), context=max(ctx), num_layers=2)
    plan, ref = _both(cfg, W, ctx)
    assert np.array_equal(plan.queue(), ref["queue"])
    assert np.array_equal(plan.thresholds(), ref["thresholds"])
    plan.close()
    oq.check_invariants(ref)
    q, thr = ref["queue"], ref["thresholds"]
    st = ref["params"]["s_tok"]
    chains, splits, comb = {}, {}, {}
    for w in range(q.shape[0]):
        for i in range(q.shape[1]):
            t = q[w, i]
            if t[0] == oq.OP_COMB:
                comb[tuple(int(v) for v in t[20:23])] = (int(t[23]), int(t[7]))
            if t[0] != oq.OP_ATTN:
                continue
            key = tuple(int(v) for v in t[20:23])
            same = lambda j: 0 <= j < q.shape[1] and q[w, j][0] == oq.OP_ATTN and tuple(int(v) for v in q[w, j][20:23]) == key
            flags, slot = int(t[30]), int(t[31])
            assert bool(flags & 1) == same(i - 1) and bool(flags & 2) == (not same(i + 1))
            assert int(t[2]) == (1 if flags & 2 else 0)
            if flags & 2:
                assert int(t[15]) == 1
            s, t0, t1 = int(t[23]), int(t[24]), int(t[25])
            r = key[1]
            assert (t0, t1) == (s * st, min(ctx[r], (s + 1) * st)) and int(t[29]) == -(-ctx[r] // st)
            splits.setdefault(key, []).append(s)
            chains.setdefault(key, set()).add(slot)
    for key, ss in splits.items():
        assert sorted(ss) == list(range(-(-ctx[key[1]] // st)))
        n = len(chains[key])
        assert chains[key] == set(range(n)) and comb[key] == (n, n)


@pytest.mark.parametrize("name", ["qwen3_8b_layer", "qwen3_8b_layer_fp8"])
def test_multi_row_attention_chain_lengths(name):
    """At the full sizes on 256 workers the splits of each (request, kv head) form chains of equal
    length covering contiguous token ranges: 4096 / 128 = 32 splits in two chains of 16 (8192: two
    of 32), one chain per worker."""
    cfg = get_config(name)
    ref = oq.build_queue(cfg, 256)
    q = ref["queue"]
    ns = -(-cfg.context // ref["params"]["s_tok"])
    for w in range(256):
        att = [q[w, i] for i in range(q.shape[1]) if q[w, i][0] == oq.OP_ATTN]
        assert len(att) == ns // 2
        assert len({tuple(int(v) for v in t[20:23]) for t in att}) == 1
        s = [int(t[23]) for t in att]
        assert s == list(range(s[0], s[0] + ns // 2)) and s[0] % (ns // 2) == 0
        assert [int(t[30]) for t in att] == [0] + [1] * (ns // 2 - 2) + [3] and len({int(t[31]) for t in att}) == 1


def test_topk_plan_shape_and_limits():
    """The top-k adds one task per token row after its request's score tasks and leaves the rest of
    the plan as without it; more than 8192 keys per row is refused."""
    import persistent_megakernel_amd as mk
    base = get_config("indexer_front")
    with_k = get_config("indexer_front_topk")
    a, b = oq.build_queue(base, 256), oq.build_queue(with_k, 256)
    assert b["n_tasks"] == a["n_tasks"] + with_k.m
    tasks = b["queue"].reshape(-1, 32)
    topk = tasks[tasks[:, 0] == oq.OP_TOPK]
    assert sorted(int(t[21]) for t in topk) == list(range(with_k.m))
    assert all(int(t[7]) == 8192 // 128 for t in topk)
    with pytest.raises(mk.MkError, match="8192 keys"):
        mk.Plan(dataclasses.replace(with_k, context=8200), num_workers=256)
    with pytest.raises(mk.MkError, match="indexer front"):
        mk.Plan(dataclasses.replace(get_config("qwen3_0p6b_layer"), topk=4), num_workers=256)


def test_main_mla_half_plan():
    """D0: 2 tiles of 64 rows per head x the q-rank K chunks, a finalize per head waiting for all
    of them; D2: 8 tiles of 64 latent rows per head, each waiting only for its own head's finalize
    (one event of threshold 1 per head), reading that head's 128 columns.  The half is one run of
    tasks between D1's finalizes and E1; without it the plan is the indexer front's, task for task,
    up to a renumbering of ids, operand rows and events that keeps which tasks share an event."""
    base, cfg = get_config("indexer_front"), get_config("attention_pre")
    a, b = oq.build_queue(base, 256), oq.build_queue(cfg, 256)
    ta, tb = oq_tasks(a), oq_tasks(b)
    mla = ((tb[:, 0] == oq.OP_GEMM) | (tb[:, 0] == oq.OP_FIN)) & np.isin(tb[:, 21], [oq.K_QB, oq.K_UK])
    at = np.flatnonzero(mla)
    assert np.array_equal(at, np.arange(at[0], at[0] + len(at)))
    assert tb[at[0] - 1, 0] == oq.OP_FIN and tb[at[-1] + 1, 0] == oq.OP_SCORE
    extra, rest = tb[mla], tb[~mla]
    assert rest.shape == ta.shape
    same = [0, 1, 2, 4, 7, 9, 11, 13, 15, 18] + list(range(20, 32))
    assert np.array_equal(rest[:, same], ta[:, same])
    emap = {}
    for x, y in zip(ta, rest):
        for k in range(int(x[1])):
            assert emap.setdefault(int(x[6 + 2 * k]), int(y[6 + 2 * k])) == int(y[6 + 2 * k])
        for k in range(int(x[2])):
            assert emap.setdefault(int(x[14 + 3 * k]), int(y[14 + 3 * k])) == int(y[14 + 3 * k])
    assert len(set(emap.values())) == len(emap)
    nk = cfg.idx_q_rank // b["params"]["kc_q"]
    d0 = extra[(extra[:, 0] == oq.OP_GEMM) & (extra[:, 21] == oq.K_QB)]
    fin = extra[extra[:, 0] == oq.OP_FIN]
    d2 = extra[(extra[:, 0] == oq.OP_GEMM) & (extra[:, 21] == oq.K_UK)]
    assert len(d0) == 64 * 2 * nk and len(fin) == 64 and len(d2) == 64 * 8
    thr = b["thresholds"]
    for h in range(64):
        f = fin[fin[:, 22] == h][0]
        assert thr[f[6]] == 2 * nk and f[2] == 1 and thr[f[14]] == 1
        heads = d2[(d2[:, 23] // 512) == h]
        assert len(heads) == 8 and all(t[6] == f[14] and t[7] == 1 and t[27] == 128 * h for t in heads)


def oq_tasks(plan):
    t = plan["queue"].reshape(-1, 32)
    t = t[t[:, 0] != 0]
    return t[np.argsort(t[:, 5])]


@pytest.mark.parametrize("name,tp,W", [
    ("qwen3_0p6b_layer", (8, 2, 6, 4, 0, 64), 256),
    ("qwen3_0p6b_layer", (16, 16, 2, 1, 0, 4), 37),
    ("qwen3_0p6b_step", (0, 0, 0, 0, 1000, 128), 256),
    ("qwen3_0p6b_step", (16, 8, 12, 8, 7, 32), 9),
    ("qwen3_8b_layer", (0, 0, 0, 0, 0, 64), 256),
    ("qwen3_8b_layer_m64", (0, 0, 0, 0, 0, 32), 148)])
def test_tile_params_bit_exact(name, tp, W):
    """Caller-fixed tile sizes (mk_config.tile_params) reach both builders alike."""
    cfg = dataclasses.replace(get_config(name), tile_params=tp, num_layers=min(2, get_config(name).num_layers),
                              vocab=min(5000, get_config(name).vocab))
    plan, ref = _both(cfg, W)
    assert np.array_equal(plan.queue(), ref["queue"])
    assert np.array_equal(plan.thresholds(), ref["thresholds"])
    p = ref["params"]
    for key, idx in (("r_qkv", 0), ("r_o", 1), ("r_gu", 2), ("r_down", 3), ("r_lm", 4), ("s_tok", 5)):
        if tp[idx]:
            assert p[key] == tp[idx]
    plan.close()


@pytest.mark.parametrize("name,tp,field", [
    ("qwen3_0p6b_layer", (3,), "QKV rows, not a power of two"),
    ("qwen3_0p6b_layer", (256,), "QKV rows above head_dim"),
    ("qwen3_0p6b_layer", (0, 3), "O rows not dividing hidden"),
    ("qwen3_0p6b_layer", (0, 256), "O rows above 128"),
    ("qwen3_0p6b_layer", (0, 0, 5), "odd gate/up rows"),
    ("qwen3_0p6b_layer", (0, 0, 96), "gate/up rows beyond one lease"),
    ("qwen3_0p6b_layer", (0, 0, 0, 7), "down rows not dividing hidden"),
    ("qwen3_0p6b_layer", (0, 0, 0, 0, 10), "lm_head rows outside the decode step"),
    ("qwen3_0p6b_layer", (0, 0, 0, 0, 0, 256), "split above 128 tokens"),
    ("qwen3_0p6b_layer", (0, 0, 0, 0, 0, 48), "split not a power of two"),
    ("qwen3_0p6b_layer", (0, 0, 0, 0, 0, 0, 1), "reserved entry"),
    ("qwen3_8b_layer", (64,), "row tiles of a multi-row plan"),
    ("indexer_front", (0, 0, 0, 0, 0, 128), "any entry of an indexer plan")])
def test_tile_params_refused(name, tp, field):
    import persistent_megakernel_amd as mk
    cfg = dataclasses.replace(get_config(name), tile_params=tp)
    with pytest.raises(mk.MkError) as e:
        mk.Plan(cfg, num_workers=256)
    assert e.value.status == mk.MK_ERR_UNSUPPORTED, field


@pytest.mark.parametrize("name,rd,ok", [("qwen3_0p6b_layer", 0, True), ("qwen3_0p6b_layer", 128, True),
                                        ("qwen3_0p6b_layer", 64, False), ("indexer_front", 128, True),
                                        ("indexer_front", 32, False)])
def test_rotary_dim(name, rd, ok):
    """RoPE over the whole head only: rotary_dim 0 or the head dim; a partial rotary is refused."""
    import persistent_megakernel_amd as mk
    cfg = dataclasses.replace(get_config(name), rotary_dim=rd)
    if ok:
        mk.Plan(cfg, num_workers=256).close()
    else:
        with pytest.raises(mk.MkError) as e:
            mk.Plan(cfg, num_workers=256)
        assert e.value.status == mk.MK_ERR_UNSUPPORTED
