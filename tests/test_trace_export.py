"""The Perfetto export of a trace (host tooling) on a synthetic queue and trace: four slices per
live instruction in its worker's track, microseconds from the run's first stamp, a wrapped clock
unwrapped, NoOp slots skipped."""
import json

import numpy as np

from persistent_megakernel_amd import trace as tx


def test_events_from_a_synthetic_trace(tmp_path):
    q = np.zeros((2, 3, 32), dtype=np.uint32)
    q[0, 0, 0], q[0, 0, 20], q[0, 0, 5] = 1, 0, 0      # QKV layer 0
    q[1, 0, 0], q[1, 0, 20], q[1, 0, 5] = 2, 0, 1      # attention layer 0
    q[0, 1, 0], q[0, 1, 20], q[0, 1, 5] = 5, 3, 2      # down layer 3; slot (1, 1) and (*, 2) are NoOp
    tr = np.zeros((2, 3, 16), dtype=np.uint32)
    base = (1 << 32) - 150                              # the clock wraps during the run
    stamp = lambda *v: [(base + x) % (1 << 32) for x in v]
    tr[0, 0, [0, 1, 3, 4, 7]] = stamp(0, 100, 120, 220, 270)
    tr[1, 0, [0, 1, 3, 4, 7]] = stamp(50, 300, 310, 510, 560)
    tr[1, 0, 8] = 3
    tr[0, 1, [0, 1, 3, 4, 7]] = stamp(280, 400, 410, 500, 520)
    ev = [e for e in tx.events(q, tr) if e["ph"] == "X"]
    assert len(ev) == 12
    get = lambda n: [e for e in ev if e["name"] == n][0]
    assert get("QKV l0 wait")["ts"] == 0.0 and get("QKV l0 wait")["dur"] == 1.0 and get("QKV l0 wait")["tid"] == 0
    assert get("QKV l0 stage")["ts"] == 1.0 and abs(get("QKV l0 stage")["dur"] - 0.2) < 1e-12
    body = get("attention l0 body")
    assert body["ts"] == 3.1 and body["dur"] == 2.0 and body["args"]["repolls"] == 3 and body["tid"] == 1
    assert get("down l3 epilogue")["ts"] == 5.0 and get("down l3 epilogue")["dur"] == 0.2
    path = tmp_path / "t.json"
    tx.write(str(path), q, tr)
    assert len(json.loads(path.read_text())["traceEvents"]) == 12 + 2  # slices + one name per worker
