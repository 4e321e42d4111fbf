"""Pins the byte / gap estimate against the table the handbook page prints."""
import os

from oracle import bytes as ob

GOLD = os.path.join(os.path.dirname(__file__), "golden", "decode_gaps_table.txt")


def _rows():
    rows = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        rows.setdefault(f[0], []).append(f[1:])
    return rows


def test_printed_table_reproduced():
    rows = _rows()
    for model in ("Qwen3-0.6B", "Qwen3-8B"):
        for f in rows[model]:
            batch, ctx = int(f[0]), int(f[1])
            r = ob.decode_estimate(model, batch, ctx)
            assert r["kernels"] == int(f[2])
            assert round(r["data_us"]) == int(f[3])
            assert round(r["eager_us"]) == int(f[4])
            for i, g in enumerate((0.5, 1.0, 2.0, 3.0)):
                assert round(r["graph_us"][g]) == int(f[5 + 2 * i])
                assert round(100 * r["gap_share"][g]) == int(f[6 + 2 * i])


def test_small_kernel_line_and_exercise():
    rows = _rows()
    small = rows["small"][0]
    r = ob.decode_estimate("Qwen3-0.6B", 1, 1024)
    assert r["small_kernels"] == int(small[0]) and r["kernels"] == int(small[1])
    assert round(r["mean_kernel_us"], 2) == float(small[2])
    ex = rows["exercise"][0]
    n_fused = 28 * 6 + 3
    assert n_fused == int(ex[0])
    assert round(r["data_us"] + n_fused * 2.0) == int(ex[1])
    assert round(r["data_us"] + n_fused * 1.0) == int(ex[2])


def test_algorithmic_bytes_small_layer():
    from workloads import algorithmic_bytes, get_config
    b = algorithmic_bytes(get_config("qwen3_0p6b_layer"))
    # weights: (4096 + 1024*2048/1024 ...) spelled out per matrix
    assert b["weights"] == 2 * (4096 * 1024 + 1024 * 2048 + 6144 * 1024 + 1024 * 3072)
    assert b["kv_read"] == 511 * 2 * 8 * 128 * 2
    assert b["total"] == sum(v for k, v in b.items() if k != "total")
