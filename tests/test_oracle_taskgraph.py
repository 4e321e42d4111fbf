"""The op-graph lowering (oracle/taskgraph.py) against the worked plan of the MegaRTP page
("Kernel-Mega-PDL", section 4: the M=16, KV=8192 attention-pre graph, its tile counts, its events
and its KernelPlan), and against its pairing rules on small graphs.

Printed on the page, and checked here:
* tile tasks: A0 16, B0 84 (21 N tiles x split-K 4), C0 48 (12 N x 4), B1 8 (split-K 8),
  D1 128 (32 heads x 4), D0 128 (64 heads x 2 N tiles), D2 256 (64 x 4), E1 64 (4 Q-blocks x 16
  KV tasks): 732 in all, dealt round-robin onto 148 queues -> [148, 5, 32], 140 queues with 5 live
  instructions and 8 with 4 plus a NoOp;
* 70 events: event0 >= 16 (A0's hidden FP8/scale rows, for B0 and B1), event1 >= 16 (A0's norm
  rows, for C0), event2 >= 16 (B0's final Q/scale rows), event3 >= 48 (C0's gate partials; D1
  waits for event2 and event3), 64 events of threshold 2 (D0's head tiles pairwise, for D2),
  event68 >= 32 (D1's head tiles), event69 >= 1 (B1's cache write); E1 waits for event68 and
  event69 and reads operand row 7;
* the operand pointer table [8, 16] of 8-byte addresses = 1024 bytes.
The graph below restates the page's data flow (which op reads which op's output and how each is
split); the events and thresholds are what the lowering derives from it, not a list written here.
"""
import numpy as np
import pytest

from oracle import taskgraph as tg
from oracle.taskgraph import Op, Pub, Region, Tile

ROWS = 16  # M = 16 token rows


def _rows(lo=0, hi=ROWS):
    return (lo, hi)


def page_attention_pre_graph():
    K = 8  # hidden size in units: B0 and C0 split it in 4, B1 in 8
    QW = 4  # width of B0's final Q rows in units: D1 splits it in 4
    ops = []
    # A0: Add + RMSNorm + quant, one row per tile; publishes the FP8 hidden (+ scale) and the norm output
    ops.append(Op("A0", [Tile(reads=[Region("x", (_rows(m, m + 1), (0, K)))],
                              pubs=[Pub(Region("hidden_fp8", (_rows(m, m + 1), (0, K)))),
                                    Pub(Region("norm", (_rows(m, m + 1), (0, K))))], payload=[m])
                         for m in range(ROWS)]))
    # B0: q_a GEMM, 21 N tiles x split-K 4 over the FP8 hidden; its finalize publishes the 16 Q/scale rows
    b0 = [Tile(reads=[Region("hidden_fp8", (_rows(), (2 * k, 2 * k + 2)))], payload=[n, k])
          for n in range(21) for k in range(4)]
    ops.append(Op("B0", b0, finalize=[(list(range(len(b0))),
                                       [Pub(Region("q", (_rows(m, m + 1), (0, QW)))) for m in range(ROWS)])]))
    # C0: head-weight (gate) GEMM, 12 N tiles x split-K 4 over the norm output; partials reduce in place
    ops.append(Op("C0", [Tile(reads=[Region("norm", (_rows(), (2 * k, 2 * k + 2)))],
                              pubs=[Pub(Region("gate", (_rows(), (n, n + 1))), reduce=True)], payload=[n, k])
                         for n in range(12) for k in range(4)]))
    # B1: indexer key GEMM, split-K 8; its finalize writes the key cache once
    b1 = [Tile(reads=[Region("hidden_fp8", (_rows(), (k, k + 1)))], payload=[k]) for k in range(8)]
    ops.append(Op("B1", b1, finalize=[(list(range(8)), [Pub(Region("key_cache", ((0, 1),)))])]))
    # D1: indexer Q GEMM, 32 heads x split-K 4 over B0's Q, joined with C0's gate; a head's finalize
    # publishes its Indexer-Q / head-weight tile
    d1 = [Tile(reads=[Region("q", (_rows(), (k, k + 1))), Region("gate", (_rows(), (0, 12)))], payload=[h, k])
          for h in range(32) for k in range(4)]
    ops.append(Op("D1", d1, finalize=[([4 * h + k for k in range(4)], [Pub(Region("index_q", ((h, h + 1),)))])
                                      for h in range(32)]))
    # D0: main Q GEMM, 64 heads x 2 N tiles over B0's Q
    ops.append(Op("D0", [Tile(reads=[Region("q", (_rows(), (0, QW)))],
                              pubs=[Pub(Region("main_q", ((h, h + 1), (j, j + 1))))], payload=[h, j])
                         for h in range(64) for j in range(2)]))
    # D2: per-head Q-BMM, 64 heads x 4 N tiles, each reading its head's whole D0 output
    ops.append(Op("D2", [Tile(reads=[Region("main_q", ((h, h + 1), (0, 2)))],
                              pubs=[Pub(Region("q_bmm", ((h, h + 1), (j, j + 1))))], payload=[h, j])
                         for h in range(64) for j in range(4)]))
    # E1: paged indexer score, 4 Q-blocks x 16 KV tasks, reading every head's Indexer-Q and the key cache
    ops.append(Op("E1", [Tile(reads=[Region("index_q", ((0, 32),)), Region("key_cache", ((0, 1),))],
                              pubs=[Pub(Region("score", ((b, b + 1), (s, s + 1))))], payload=[b, s])
                         for b in range(4) for s in range(16)]))
    strategies = {("A0", "B0"): "tile_cover", ("A0", "C0"): "tile_cover", ("A0", "B1"): "tile_cover",
                  ("B0", "D1"): "tile_cover", ("C0", "D1"): "tile_reduce", ("B0", "D0"): "tile_cover",
                  ("D0", "D2"): "tile_cover", ("D1", "E1"): "tile_cover", ("B1", "E1"): "exact"}
    return ops, strategies


def test_page_plan_tasks_and_packing():
    ops, strategies = page_attention_pre_graph()
    assert [len(o.tiles) for o in ops] == [16, 84, 48, 8, 128, 128, 256, 64]
    g = tg.lower(ops, strategies)
    assert len(g["tasks"]) == 732
    q = tg.kernel_plan(ops, g, 148)
    assert q.shape == (148, 5, 32)
    live = (q[:, :, 0] != 0).sum(axis=1)
    assert (live == 5).sum() == 140 and (live == 4).sum() == 8
    assert len(ops) * 16 * 8 == 1024  # the operand pointer table [8, 16] of 8-byte addresses


def test_page_plan_events():
    ops, strategies = page_attention_pre_graph()
    g = tg.lower(ops, strategies)
    thr = g["thresholds"]
    assert len(thr) == 70
    assert list(thr[:4]) == [16, 16, 16, 48]
    assert list(thr[4:68]) == [2] * 64
    assert list(thr[68:]) == [32, 1]
    by_op = {}
    for t in g["tasks"]:
        by_op.setdefault(ops[t["op"]].name, []).append(t)
    assert all(t["waits"] == [(0, 16)] for t in by_op["B0"] + by_op["B1"])
    assert all(t["waits"] == [(1, 16)] for t in by_op["C0"])
    assert all(t["waits"] == [(2, 16), (3, 48)] for t in by_op["D1"])  # the B0 + C0 join
    assert all(t["waits"] == [(2, 16)] for t in by_op["D0"])
    assert [t["waits"] for t in by_op["D2"]] == [[(4 + h, 2)] for h in range(64) for _ in range(4)]
    assert all(t["waits"] == [(68, 32), (69, 1)] for t in by_op["E1"])
    q = tg.kernel_plan(ops, g, 148)
    e1 = [w for w in q.reshape(-1, 32) if w[0] == 8]
    assert len(e1) == 64 and all(w[3] == 7 for w in e1)  # E1's operand row is row 7
    # executing the packed signal words (finalize groups signal once) meets every threshold exactly
    assert np.array_equal(tg.run_counters(ops, q), thr)


def test_unregistered_pair_falls_back_to_whole():
    ops, strategies = page_attention_pre_graph()
    del strategies[("D0", "D2")]
    g = tg.lower(ops, strategies)
    # every D2 tile now waits for all 128 D0 tiles: one shared event instead of 64 of threshold 2
    assert len(g["thresholds"]) == 70 - 64 + 1
    d2 = [t for t in g["tasks"] if ops[t["op"]].name == "D2"]
    assert all(t["waits"] == [(4, 128)] for t in d2)


def test_pairing_checks_reject_bad_regions():
    # a row missing from a cover
    ops = [Op("P", [Tile(pubs=[Pub(Region("t", ((m, m + 1),)))]) for m in range(3)]),
           Op("C", [Tile(reads=[Region("t", ((0, 4),))])])]
    with pytest.raises(tg.LoweringError, match="cover"):
        tg.lower(ops, {("P", "C"): "tile_cover"})
    # overlapping pieces in a cover
    ops = [Op("P", [Tile(pubs=[Pub(Region("t", ((0, 2),)))]), Tile(pubs=[Pub(Region("t", ((1, 3),)))])]),
           Op("C", [Tile(reads=[Region("t", ((0, 3),))])])]
    with pytest.raises(tg.LoweringError, match="overlapping"):
        tg.lower(ops, {("P", "C"): "tile_cover"})
    # a reduction read over complete publications, and uneven reductions
    ops = [Op("P", [Tile(pubs=[Pub(Region("t", ((0, 1),)))])]), Op("C", [Tile(reads=[Region("t", ((0, 1),))])])]
    with pytest.raises(tg.LoweringError, match="complete"):
        tg.lower(ops, {("P", "C"): "tile_reduce"})
    ops = [Op("P", [Tile(pubs=[Pub(Region("t", ((0, 1),)), reduce=True)]),
                    Tile(pubs=[Pub(Region("t", ((0, 1),)), reduce=True)]),
                    Tile(pubs=[Pub(Region("t", ((1, 2),)), reduce=True)])]),
           Op("C", [Tile(reads=[Region("t", ((0, 2),))])])]
    with pytest.raises(tg.LoweringError, match="different numbers"):
        tg.lower(ops, {("P", "C"): "tile_reduce"})
    # exact needs one equal publication
    ops = [Op("P", [Tile(pubs=[Pub(Region("t", ((0, 2),)))])]), Op("C", [Tile(reads=[Region("t", ((0, 1),))])])]
    with pytest.raises(tg.LoweringError, match="exactly"):
        tg.lower(ops, {("P", "C"): "exact"})
    # a consumer before its producer
    ops = [Op("C", [Tile(reads=[Region("t", ((0, 1),))])]), Op("P", [Tile(pubs=[Pub(Region("t", ((0, 1),)))])])]
    with pytest.raises(tg.LoweringError, match="before"):
        tg.lower(ops, {})
