"""Chrome trace-event (Perfetto) export of an MK_FLAG_TRACE run.

``events(queue, trace)`` turns the instruction queue ``[W, L, 32]`` and the trace ``[W, L, 16]``
(``Plan.queue()``, ``Plan.read_trace()``) into trace events: one track per worker, and for each
instruction four slices -- wait (seen until its waits are met), stage (until the compute-start
barrier), body (between the two compute barriers) and epilogue (until done) -- named by opcode and
layer.  Stamps are the low 32
bits of the 100 MHz clock; they are unwrapped relative to the run's first stamp.  ``write(path,
queue, trace)`` stores the JSON that ui.perfetto.dev and chrome://tracing open.  Host tooling only:
nothing here takes part in a run.
"""
from __future__ import annotations

import json
from typing import Dict, List

import numpy as np

OPCODES = {1: "QKV", 2: "attention", 3: "O", 4: "gate/up", 5: "down", 6: "lm_head", 7: "norm", 8: "GEMM",
           9: "finalize", 10: "quantise", 11: "combine", 12: "key cache", 13: "score", 14: "top-k"}


def events(queue: np.ndarray, trace: np.ndarray) -> List[Dict]:
    q = np.asarray(queue)
    tr = np.asarray(trace).astype(np.int64)
    live = q[:, :, 0] != 0
    if not live.any():
        return []
    # the run's first stamp: the one after the widest gap between seen-stamps on the 2^32 circle
    seen = np.sort(tr[:, :, 0][live])
    gaps = np.diff(np.append(seen, seen[0] + (1 << 32)))
    t0 = int(seen[(int(np.argmax(gaps)) + 1) % len(seen)])
    ticks = lambda v: (int(v) - t0) % (1 << 32)  # 100 MHz ticks since t0
    out: List[Dict] = [{"name": "thread_name", "ph": "M", "pid": 0, "tid": int(w), "args": {"name": f"worker {w}"}}
                       for w in range(q.shape[0])]
    for w, i in zip(*np.nonzero(live)):
        op = int(q[w, i, 0])
        name = f"{OPCODES.get(op, op)} l{int(q[w, i, 20])}"
        stamps = tr[w, i]
        args = {"instruction": int(i), "task": int(q[w, i, 5]), "repolls": int(stamps[8])}
        for label, a, b in (("wait", 0, 1), ("stage", 1, 3), ("body", 3, 4), ("epilogue", 4, 7)):
            ts, te = ticks(stamps[a]), ticks(stamps[b])
            if te >= ts:
                out.append({"name": f"{name} {label}", "cat": label, "ph": "X", "ts": ts / 100, "dur": (te - ts) / 100,
                            "pid": 0, "tid": int(w), "args": args})
    return out


def write(path: str, queue: np.ndarray, trace: np.ndarray) -> None:
    with open(path, "w") as f:
        json.dump({"traceEvents": events(queue, trace), "displayTimeUnit": "ns"}, f)
