"""Pins of the oracle queue builder: invariants, deadlock freedom under random worker
speeds (a CPU simulation of the worker loop), and the page's worked packing example."""
import dataclasses

import numpy as np
import pytest

from oracle import queue as oq
from workloads import get_config


@pytest.mark.parametrize("name", ["qwen3_0p6b_layer", "qwen3_0p6b_step", "qwen3_8b_layer", "qwen3_8b_layer_fp8",
                                  "qwen3_8b_layer_m64", "indexer_front", "indexer_front_topk",
                                  "attention_pre"])
@pytest.mark.parametrize("W", [1, 7, 148, 256])
def test_invariants(name, W):
    cfg = get_config(name)
    plan = oq.build_queue(cfg, W)
    oq.check_invariants(plan)
    assert plan["queue"].shape == (W, -(-plan["n_tasks"] // W), 32)


def test_small_layer_counts():
    plan = oq.build_queue(get_config("qwen3_0p6b_layer"), 256)
    p = plan["params"]
    assert (p["r_qkv"], p["r_o"], p["r_gu"], p["r_down"], p["s_tok"]) == (16, 4, 12, 4, 32)
    # 256 QKV + 8 heads x 16 splits + 256 + 256 + 256
    assert plan["n_tasks"] == 1152 and plan["queue"].shape == (256, 5, 32)
    assert list(plan["thresholds"]) == [32] * 8 + [8, 256, 256, 256]


def simulate(plan, seed=0, max_steps=10 ** 7):
    """Workers advance in random order; a task runs only when its waits are met."""
    rng = np.random.default_rng(seed)
    q = plan["queue"]
    W, L, _ = q.shape
    cnt = np.zeros(len(plan["thresholds"]), dtype=np.int64)
    arrivals = {}
    pc = np.zeros(W, dtype=np.int64)
    steps = 0
    while (pc < L).any():
        steps += 1
        assert steps < max_steps
        live = np.flatnonzero(pc < L)
        progressed = False
        for w in rng.permutation(live):
            words = q[w, pc[w]]
            if all(cnt[words[6 + 2 * k]] >= words[7 + 2 * k] for k in range(int(words[1]))):
                total = int(words[27])
                fire = True
                if words[0] != oq.OP_NOOP and total:
                    g = int(words[26])
                    arrivals[g] = arrivals.get(g, 0) + 1
                    fire = arrivals[g] == total
                if fire:
                    for k in range(int(words[2])):
                        cnt[words[14 + 3 * k]] += words[15 + 3 * k]
                pc[w] += 1
                progressed = True
        assert progressed, "deadlock"
    assert np.array_equal(cnt, plan["thresholds"].astype(np.int64))


@pytest.mark.parametrize("W", [3, 64, 256])
def test_no_deadlock_random_speeds(W):
    cfg = dataclasses.replace(get_config("qwen3_0p6b_step"), num_layers=2)
    plan = oq.build_queue(cfg, W)
    for seed in range(3):
        simulate(plan, seed)


def test_page_packing_example():
    # MegaRTP page, section 4 (KernelPlan): 732 tile tasks dealt round-robin onto 148 worker
    # queues give 140 workers with 5 instructions and 8 with 4 + one NoOp, shape [148, 5, 32].
    counts = {"A0": 16, "B0": 84, "C0": 48, "B1": 8, "D1": 128, "D0": 128, "D2": 256, "E1": 64}
    assert sum(counts.values()) == 732
    b = oq._Builder()
    for i, (op, n) in enumerate(counts.items()):
        row = b.op_row()
        for j in range(n):
            b.task(i + 1, row, 0, [], [], [j])
    T, W = len(b.tasks), 148
    L = -(-T // W)
    q = np.zeros((W, L, 32), dtype=np.uint32)
    for tid, words in enumerate(b.tasks):
        q[tid % W, tid // W] = words
    assert q.shape == (148, 5, 32)
    live = (q[:, :, 0] != 0).sum(axis=1)
    assert (live == 5).sum() == 140 and (live == 4).sum() == 8
    # the page's events are derived from its graph by the lowering in tests/test_oracle_taskgraph.py


def _tasks(plan):
    q = plan["queue"]
    return [q[w, i] for i in range(q.shape[1]) for w in range(q.shape[0]) if q[w, i][0] != oq.OP_NOOP]


@pytest.mark.parametrize("name", ["qwen3_8b_layer", "qwen3_8b_layer_fp8", "qwen3_8b_layer_m64"])
def test_multi_row_tiles_cover_each_projection_once(name):
    """Each projection's (row, K) grid is covered exactly once by its GEMM tiles, and its
    (row, 16-row group) pairs exactly once by finalize tasks whose chunk count matches the tiles."""
    cfg = get_config(name)
    plan = oq.build_queue(cfg, 256)
    p = plan["params"]
    H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
    shapes = {oq.K_QKV: ((cfg.n_q_heads + 2 * cfg.n_kv_heads) * d, H), oq.K_O: (H, cfg.n_q_heads * d),
              oq.K_GU: (I, H), oq.K_DOWN: (H, I)}
    kc = p["kc"]
    assert kc * (1 if cfg.weight_fp8 else 2) * oq.M16_ROWS == 64 * 1024
    ops = [int(t[0]) for t in _tasks(plan)]
    assert set(ops) <= {oq.OP_NORM, oq.OP_GEMM, oq.OP_FIN, oq.OP_QUANT, oq.OP_ATTN, oq.OP_COMB}
    assert ops.count(oq.OP_COMB) == cfg.n_requests * cfg.n_kv_heads
    for kind, (N, K) in shapes.items():
        G = -(-cfg.m // 16)
        grid = np.zeros((N, K // kc), dtype=np.int64)
        fin = np.zeros((N, G), dtype=np.int64)
        for t in _tasks(plan):
            pl = t[20:]  # payload words follow the header
            if t[0] == oq.OP_GEMM and pl[1] == kind:
                n0, rows, k0 = int(pl[3]), int(pl[4]), int(pl[5])
                assert int(pl[6]) == kc and k0 % kc == 0
                grid[n0:n0 + rows, k0 // kc] += 1
            if t[0] == oq.OP_FIN and pl[1] == kind:
                n0, rows, nk, gi = int(pl[3]), int(pl[4]), int(pl[5]), int(pl[9])
                assert nk == K // kc
                fin[n0:n0 + rows, gi] += 1
        assert (grid == 1).all() and (fin == 1).all(), kind
    n_norm = ops.count(oq.OP_NORM)
    n_quant = ops.count(oq.OP_QUANT)
    assert n_norm == 2 * cfg.m and n_quant == (2 * cfg.m if cfg.act_fp8 else 0)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("R", [3, 40])
def test_multi_row_no_deadlock_random_speeds(fp8, R):
    cfg = dataclasses.replace(get_config("qwen3_8b_layer_fp8" if fp8 else "qwen3_8b_layer"),
                              hidden=512, inter=1024, n_q_heads=4, n_kv_heads=2, n_requests=R,
                              context=200, num_layers=2)
    plan = oq.build_queue(cfg, 37)
    assert plan["params"]["spec"] == 1
    oq.check_invariants(plan)
    for seed in range(2):
        simulate(plan, seed)


def test_row_groups_wait_for_their_own_group():
    """Beyond 16 rows: an attention split waits for its request's 16-row group of its kv group's
    QKV finalizes, a row's second norm for its group's O finalizes, the next layer's first norm
    for its group's down finalizes; every finalize signals exactly one of those events."""
    cfg = dataclasses.replace(get_config("qwen3_8b_layer"), hidden=512, inter=1024, n_q_heads=4,
                              n_kv_heads=2, n_requests=40, context=100, num_layers=2)
    plan = oq.build_queue(cfg, 37)
    tasks = _tasks(plan)
    fin_ev = {}
    for t in tasks:
        if t[0] == oq.OP_FIN:
            fin_ev.setdefault((int(t[20]), int(t[21]), int(t[29])), set()).add(int(t[14]))
    for (l, kind, gi), evs in fin_ev.items():
        if kind != oq.K_QKV:
            assert len(evs) == 1 or kind == oq.K_GU, (l, kind, gi)
    for t in tasks:
        if t[0] == oq.OP_ATTN:
            l, r, hk = int(t[20]), int(t[21]), int(t[22])
            assert int(t[6]) in fin_ev[(l, oq.K_QKV, r // 16)]
        if t[0] == oq.OP_NORM and int(t[21]) == 1:
            l, m = int(t[20]), int(t[22])
            assert fin_ev[(l, oq.K_O, m // 16)] == {int(t[6])}
        if t[0] == oq.OP_NORM and int(t[21]) == 0 and int(t[20]) > 0:
            l, m = int(t[20]), int(t[22])
            assert fin_ev[(l - 1, oq.K_DOWN, m // 16)] == {int(t[6])}


def test_indexer_front_counts_and_no_deadlock():
    """Indexer front at its configured size: 16 norm rows, tiles of 64 rows x one K chunk for
    B0 (1536 rows), C0 (64), B1 (128) over K = 6144 (chunk 1024) and D1 (8192 rows) over K = 1536
    (chunk 768), per-tile finalizes (D1: per head), 16 q_a norm rows, one key-cache task, and
    one score task per 128 keys of each request."""
    cfg = get_config("indexer_front")
    plan = oq.build_queue(cfg, 256)
    ops = [int(t[0]) for t in _tasks(plan)]
    assert ops.count(oq.OP_NORM) == 2 * 16
    assert ops.count(oq.OP_GEMM) == (1536 // 64 + 1 + 2) * 6 + (8192 // 64) * 2
    assert ops.count(oq.OP_FIN) == 1536 // 64 + 1 + 2 + 64
    assert ops.count(oq.OP_KCACHE) == 1 and ops.count(oq.OP_SCORE) == 2 * 8192 // 128
    assert plan["n_tasks"] == 670
    small = dataclasses.replace(cfg, hidden=1024, idx_q_rank=512, context=300)
    for topk in (0, 64):
        for W in (3, 64):
            p = oq.build_queue(dataclasses.replace(small, topk=topk), W)
            oq.check_invariants(p)
            for seed in range(2):
                simulate(p, seed)


@pytest.mark.parametrize("vocab,W", [(151936, 256), (3000, 9), (100, 256), (4099, 37), (7, 7)])
def test_lm_head_tasks_cover_the_vocabulary_once(vocab, W):
    """The step's lm_head tasks: at most one per worker, task j takes the rows j, j + n, j + 2n, ...
    (n tasks), so every vocabulary row is computed exactly once; every task publishes its worker's
    maximum into its own slot of one arrival group (the last arriver takes the argmax)."""
    cfg = dataclasses.replace(get_config("qwen3_0p6b_step"), num_layers=1, vocab=vocab, context=64)
    plan = oq.build_queue(cfg, W)
    lm = [t for t in _tasks(plan) if t[0] == oq.OP_LMHEAD]
    n = len(lm)
    assert 1 <= n <= W
    rows = []
    for t in lm:
        j, nr, stride = int(t[21]), int(t[22]), int(t[23])  # first row, row count, row stride
        assert stride == n and int(t[24]) == cfg.hidden
        rows.extend(range(j, j + nr * stride, stride))
    assert sorted(rows) == list(range(vocab))
    assert sorted(int(t[28]) for t in lm) == list(range(n))  # a slot each
    assert {int(t[26]) for t in lm} == {int(lm[0][26])} and all(int(t[27]) == n for t in lm)
    # every lm_head task sits on a worker of its own
    q = plan["queue"]
    per_worker = [(q[w, :, 0] == oq.OP_LMHEAD).sum() for w in range(W)]
    assert max(per_worker) == 1
