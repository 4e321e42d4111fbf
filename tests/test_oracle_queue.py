"""Pins of the oracle queue builder: invariants, deadlock freedom under random worker
speeds (a CPU simulation of the worker loop), and the page's worked packing example."""
import dataclasses

import numpy as np
import pytest

from oracle import queue as oq
from workloads import get_config


@pytest.mark.parametrize("name", ["qwen3_0p6b_layer", "qwen3_0p6b_step", "qwen3_8b_layer"])
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
    # the page's 70 events: 16, 16, 16, 48, 64 x 2 (D0 -> D2 pairs), 32, 1
    thr = [16, 16, 16, 48] + [2] * 64 + [32, 1]
    assert len(thr) == 70 and sum(1 for t in thr if t == 2) == 128 // 2
