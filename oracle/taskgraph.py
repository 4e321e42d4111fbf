"""Generic lowering of an op graph into counter events and worker queues.  TEST INFRASTRUCTURE ONLY.

Written from the MegaRTP page ("Kernel-Mega-PDL"), section 4:

* OpGraph -> TaskGraph: every op is expanded into tiles; a tile reads tensor regions and, when it
  (or the finalizing member of its group) completes, publishes regions.  For every tensor edge
  (producer op, consumer op) the host looks up a registered pairing strategy and falls back to
  ``whole`` when none is registered:
    - ``whole``: wait until every publication of the producer op is done;
    - ``tile_cover``: the producer's publications that meet the region a consumer tile reads are
      disjoint pieces that together cover exactly that region (concatenation);
    - ``tile_reduce``: they are partial contributions to whole sub-regions that together cover the
      region (a reduction: the counter counts contributions, it does not add values);
    - ``exact``: the publication equals the region read.
  Each such (producer, set of publications) pair becomes one counter event whose threshold is the
  number of those publications; consumers reading through the same set share the event.  The
  device only waits for counter >= threshold before its first read.
* Ops whose tiles are split along K publish their finalized regions through a finalize group: the
  group's last finishing member publishes them; in the instruction stream every member carries
  the signal (event, increment = publications of that event it completes, publication id).
* KernelPlan: tasks numbered in op order, tile order; dealt round-robin onto W queues padded
  with NoOp to [W, L, 32]; one operand-table row per op (table [ops, 16] of 8-byte addresses).

The instruction words follow the project's layout (w0 opcode, w1 wait count, w2 signal count,
w3 operand row, w4 spec id, w5 task id, w6..w13 waits, w14..w19 signals, w20.. payload).
"""
from __future__ import annotations

import dataclasses
import itertools
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

Box = Tuple[Tuple[int, int], ...]  # half-open range per dimension


@dataclasses.dataclass(frozen=True)
class Region:
    tensor: str
    box: Box


@dataclasses.dataclass(frozen=True)
class Pub:
    """A region a task publishes; ``reduce`` marks a partial contribution to it."""
    region: Region
    reduce: bool = False


@dataclasses.dataclass
class Tile:
    reads: Sequence[Region] = ()
    pubs: Sequence[Pub] = ()  # published when this tile completes
    payload: Sequence[int] = ()


@dataclasses.dataclass
class Op:
    name: str
    tiles: List[Tile]
    # finalize groups: (member tile indices, regions the group's last member publishes)
    finalize: List[Tuple[Sequence[int], Sequence[Pub]]] = dataclasses.field(default_factory=list)


def _meet(a: Box, b: Box) -> Optional[Box]:
    out = []
    for (a0, a1), (b0, b1) in zip(a, b):
        lo, hi = max(a0, b0), min(a1, b1)
        if lo >= hi:
            return None
        out.append((lo, hi))
    return tuple(out)


def _volume(b: Box) -> int:
    v = 1
    for lo, hi in b:
        v *= hi - lo
    return v


class LoweringError(ValueError):
    pass


def _pubs_of(op: Op):
    """Every publication of an op: (pub id, pub, publishing group) with group = tuple of tile indices."""
    out = []
    for i, t in enumerate(op.tiles):
        for p in t.pubs:
            out.append((len(out), p, (i,)))
    for members, pubs in op.finalize:
        for p in pubs:
            out.append((len(out), p, tuple(members)))
    return out


def _check_cover(pieces: List[Box], box: Box, what: str) -> None:
    for x, y in itertools.combinations(pieces, 2):
        if _meet(x, y) is not None:
            raise LoweringError(f"{what}: overlapping pieces {x} {y}")
    if sum(_volume(p) for p in pieces) != _volume(box):
        raise LoweringError(f"{what}: the pieces do not cover the region read")


def _select(strategy: str, prod: Op, pubs, region: Region, what: str) -> List[int]:
    """Publications of ``prod`` a consumer reading ``region`` waits for, checked against the strategy."""
    if strategy == "whole":
        return [pid for pid, _, _ in pubs]
    hits = [(pid, p, _meet(p.region.box, region.box)) for pid, p, _ in pubs if p.region.tensor == region.tensor]
    hits = [(pid, p, m) for pid, p, m in hits if m is not None]
    if not hits:
        raise LoweringError(f"{what}: no publication of {prod.name} meets the region read")
    if strategy == "exact":
        if len(hits) != 1 or hits[0][1].region.box != region.box:
            raise LoweringError(f"{what}: not exactly one publication equal to the region read")
    elif strategy == "tile_cover":
        if any(p.reduce for _, p, _ in hits):
            raise LoweringError(f"{what}: tile_cover over partial contributions")
        _check_cover([m for _, _, m in hits], region.box, what)
    elif strategy == "tile_reduce":
        if not all(p.reduce for _, p, _ in hits):
            raise LoweringError(f"{what}: tile_reduce over complete publications")
        groups: Dict[Box, int] = {}
        for _, p, m in hits:
            if m != p.region.box:
                raise LoweringError(f"{what}: a reduced region sticks out of the region read")
            groups[m] = groups.get(m, 0) + 1
        if len(set(groups.values())) != 1:
            raise LoweringError(f"{what}: reductions with different numbers of contributions")
        _check_cover(list(groups), region.box, what)
    else:
        raise LoweringError(f"unknown strategy {strategy}")
    return [pid for pid, _, _ in hits]


def lower(ops: List[Op], strategies: Dict[Tuple[str, str], str]):
    """TaskGraph of an op graph: events (thresholds) and per-task waits and signals, in task order."""
    owner: Dict[str, int] = {}  # tensor -> producing op
    all_pubs = [_pubs_of(op) for op in ops]
    for k, pubs in enumerate(all_pubs):
        for _, p, _ in pubs:
            if owner.setdefault(p.region.tensor, k) != k:
                raise LoweringError(f"tensor {p.region.tensor} published by two ops")
    events: List[int] = []
    event_of: Dict[Tuple[int, frozenset], int] = {}
    members_of: Dict[int, Tuple[int, List[int]]] = {}  # event -> (producer op, pub ids)
    tasks = []  # (op index, tile index, waits [(event, threshold)])
    for k, op in enumerate(ops):
        for i, t in enumerate(op.tiles):
            waits: List[Tuple[int, int]] = []
            for region in t.reads:
                if region.tensor not in owner:
                    continue  # an input of the whole graph: nothing to wait for
                pk = owner[region.tensor]
                if pk >= k:
                    raise LoweringError(f"{op.name} reads {region.tensor} before {ops[pk].name} runs")
                strategy = strategies.get((ops[pk].name, op.name), "whole")
                ids = _select(strategy, ops[pk], all_pubs[pk], region, f"{ops[pk].name} -> {op.name}")
                key = (pk, frozenset(ids))
                if key not in event_of:
                    event_of[key] = len(events)
                    events.append(len(ids))
                    members_of[event_of[key]] = (pk, ids)
                e = event_of[key]
                if all(w[0] != e for w in waits):
                    waits.append((e, events[e]))
            if len(waits) > 4:
                raise LoweringError(f"{op.name} tile {i}: more than four waits")
            tasks.append((k, i, waits))
    # signals: every member of a publishing group carries (event, publications of that event it completes)
    sig: Dict[Tuple[int, int], Dict[int, int]] = {}
    for e, (pk, ids) in members_of.items():
        pubs = all_pubs[pk]
        for pid in ids:
            group = pubs[pid][2]
            for i in group:
                d = sig.setdefault((pk, i), {})
                d[e] = d.get(e, 0) + 1
    out = []
    tid = 0
    for k, i, waits in tasks:
        signals = sorted(sig.get((k, i), {}).items())
        if len(signals) > 2:
            raise LoweringError(f"{ops[k].name} tile {i}: more than two signals")
        out.append({"op": k, "tile": i, "task": tid, "waits": waits, "signals": signals})
        tid += 1
    return {"thresholds": np.array(events, dtype=np.int64), "tasks": out, "event_members": members_of}


def kernel_plan(ops: List[Op], tg, W: int) -> np.ndarray:
    """Deal the tasks round-robin onto W worker queues padded with NoOp: uint32 [W, L, 32]."""
    T = len(tg["tasks"])
    L = -(-T // W)
    q = np.zeros((W, L, 32), dtype=np.uint32)
    for t in tg["tasks"]:
        w = np.zeros(32, dtype=np.uint32)
        w[0], w[1], w[2], w[3], w[4], w[5] = t["op"] + 1, len(t["waits"]), len(t["signals"]), t["op"], 0, t["task"]
        for j, (e, thr) in enumerate(t["waits"]):
            w[6 + 2 * j], w[7 + 2 * j] = e, thr
        for j, (e, inc) in enumerate(t["signals"]):
            w[14 + 3 * j], w[15 + 3 * j], w[16 + 3 * j] = e, inc, t["task"]
        payload = list(ops[t["op"]].tiles[t["tile"]].payload)[:12]
        for j, v in enumerate(payload):
            w[20 + j] = v
        q[t["task"] % W, t["task"] // W] = w
    return q


def run_counters(ops: List[Op], queue: np.ndarray) -> np.ndarray:
    """Execute the packed queue's signal words once, in any order (the counters only add): a task of
    an op without finalize groups issues its own signals; of a finalize group only the last finishing
    member issues the group's signals (every member carries the same words).  Returns the counters."""
    words = queue.reshape(-1, 32)
    words = words[words[:, 0] != 0]
    n_events = int(max([words[:, 6 + 2 * j].max() for j in range(4)] + [words[:, 14 + 3 * j].max() for j in range(2)])) + 1
    cnt = np.zeros(n_events, dtype=np.int64)
    last_of_group = {}
    for k, op in enumerate(ops):
        for members in (m for m, _ in op.finalize):
            for i in members:
                last_of_group[(k, i)] = max(members)
    first_task = {}
    for w in words:
        first_task.setdefault(int(w[3]), int(w[5]))
    for w in sorted(words, key=lambda w: int(w[5])):
        k, tile = int(w[3]), int(w[5]) - first_task[int(w[3])]
        if (k, tile) in last_of_group and last_of_group[(k, tile)] != tile:
            continue  # not the group's last member: its copy of the group's signals is not issued
        for j in range(int(w[2])):
            cnt[int(w[14 + 3 * j])] += int(w[15 + 3 * j])
    return cnt
