"""Benchmark: microseconds per decode layer-step and achieved HBM bandwidth on one MI355X.

Default workload: the Qwen3-0.6B-shaped full decode step (28 layers, batch 1, context
2048 in 16-token pages, final RMSNorm, lm_head over 151936 rows, greedy argmax) with
seeded synthetic bf16 weights and caches, run as ONE persistent megakernel launch per
step.  The same op bodies are also timed as a single-stream and a multi-stream hipGraph
(one kernel per op), without cross-instruction prefetch, and with every op body skipped
(the framework alone).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBPS = 8000.0


def _kernel_source_sha16() -> str:
    import hashlib
    d = os.path.join(ROOT, "persistent_megakernel_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(d)):
        with open(os.path.join(d, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_traffic(workload: str):
    """HBM bytes per launch from the committed profiler counter summary of this workload, or
    None when there is none or the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"mk_worker_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            k, sep, v = line.partition(":")
            if sep and k.strip() in ("source_sha16", "traffic_bytes_per_launch"):
                fields[k.strip()] = v.strip().strip("()`")
    if fields.get("source_sha16") != _kernel_source_sha16() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_0p6b_step",
                    choices=["qwen3_0p6b_step", "qwen3_0p6b_layer", "qwen3_8b_layer", "qwen3_8b_layer_fp8", "qwen3_8b_layer_m64",
                             "indexer_front", "indexer_front_topk", "attention_pre"])
    ap.add_argument("--rotate", type=int, default=0, help="copies of weights/caches cycled per run (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-diagnostics", action="store_true", help="skip the traced pass and the stream-peak copy")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="time a plain device-to-device copy of this many bytes instead (calibrates the "
                         "HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs the decode chain on a single MI355X "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_bytes:
        return copy_calibration(args, torch)

    import persistent_megakernel_amd as mk
    from gpu_helpers import to_device
    from workloads import algorithmic_bytes, get_config, make_inputs

    cfg = get_config(args.workload)
    # rotation copies keep the timed runs from being served out of the 256 MiB MALL: the full step
    # and the 16-token layers are larger than it on their own (two copies for the layers)
    indexer = cfg.workload == "indexer_front"
    rotate = args.rotate or (1 if cfg.workload == "qwen3_step" else 20 if indexer else 2 if cfg.m > 1 else 16)
    _log(f"bench: workload {cfg.name}, rotate {rotate}, generating inputs")
    t0 = time.time()
    inp = make_inputs(cfg, seed=0)
    _log(f"bench: inputs generated in {time.time() - t0:.1f}s")
    step = cfg.workload == "qwen3_step"
    stream = torch.cuda.Stream()
    M, H = cfg.m, cfg.hidden

    def device_set(seed_shift: int):
        t = {k: to_device(v) for k, v in inp.items()}
        if seed_shift:  # a distinct copy: same values, other addresses (defeats cache residency)
            t = {k: v.clone() for k, v in t.items()}
        return t

    base = device_set(0)
    sets = [base] + [device_set(i) for i in range(1, rotate)]
    plans = {}

    def plan(flags=0):
        if flags not in plans:
            plans[flags] = mk.Plan(cfg, flags=flags)
        return plans[flags]

    p0 = plan(0)
    ws_bytes = p0.workspace_bytes() + 256
    tensor_sets = []
    for s in sets:
        s = dict(s)
        if indexer:  # scores [M, context], the workspace and, with a top-k, its positions [M, k]
            s["score_out"] = torch.zeros(M * cfg.context, dtype=torch.float32, device="cuda")
            s["workspace"] = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
            if cfg.topk:
                s["topk_out"] = torch.zeros(M * cfg.topk, dtype=torch.int32, device="cuda")
            if cfg.mla_heads:
                s["qlat_out"] = torch.zeros(M * cfg.mla_heads * 512, dtype=torch.int16, device="cuda")
            tensor_sets.append(mk.indexer_pointers(s))
            continue
        s["y_out"] = torch.zeros(M * H, dtype=torch.int16, device="cuda")
        s["r2_out"] = torch.zeros(M * H, dtype=torch.float32, device="cuda")
        s["workspace"] = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
        if step:
            s["logits_out"] = torch.zeros(M * cfg.vocab, dtype=torch.float32, device="cuda")
            s["token_out"] = torch.zeros(M, dtype=torch.int32, device="cuda")
        tensor_sets.append(mk.qwen3_pointers(s, step))
    torch.cuda.synchronize()

    def timed(fn, p, steps, warmup, per_step=None, sets=None):
        sets = sets or tensor_sets
        for i in range(warmup):
            fn(p, sets[i % len(sets)])
        p.sync(stream)
        torch.cuda.synchronize()
        # one event before every step and one after the last, all on the launch stream: the bracket
        # gives the mean, consecutive events each step's own duration
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            fn(p, sets[i % len(sets)])
            ev[i + 1].record(stream)
        p.sync(stream)
        torch.cuda.synchronize()
        if per_step is not None:
            per_step.extend(ev[i].elapsed_time(ev[i + 1]) * 1000.0 for i in range(steps))
        return ev[0].elapsed_time(ev[steps]) / steps  # ms per run

    run_mk = lambda p, t: p.run(t, stream)
    run_g1 = lambda p, t: p.run_graph(t, False, stream)
    run_gm = lambda p, t: p.run_graph(t, True, stream)

    _log("bench: megakernel")
    env_before = _gpu_state()
    per_step = []
    with torch.cuda.stream(stream):
        ms = timed(run_mk, p0, args.steps, args.warmup, per_step)
    env_after = _gpu_state()
    hot_ms = None
    if rotate > 1:  # the same work on one resident copy: the cache-resident (MALL / L2) figure
        _log("bench: megakernel, one resident copy")
        with torch.cuda.stream(stream):
            hot_ms = timed(run_mk, p0, max(10, args.steps // 2), 3, sets=tensor_sets[:1])
    variants = {}
    if not args.no_variants:
        for name, fn, flags in (("graph_single_stream", run_g1, 0), ("graph_multi_stream", run_gm, 0),
                                ("megakernel_no_prefetch", run_mk, mk.MK_FLAG_NO_PREFETCH),
                                ("megakernel_empty_framework", run_mk, mk.MK_FLAG_NOOP_ONLY),
                                ("graph_empty_framework", run_g1, mk.MK_FLAG_NOOP_ONLY)):
            _log(f"bench: {name}")
            with torch.cuda.stream(stream):
                variants[name] = round(timed(fn, plan(flags), max(10, args.steps // 2), 3) * 1000.0, 3)
    ab = algorithmic_bytes(cfg)
    nbytes = ab["total"]
    step_us = ms * 1000.0
    layers = cfg.num_layers
    achieved = nbytes / (ms * 1e-3) / 1e9
    out = {
        "metric": "us per decode layer-step and achieved HBM GB/s (% of MI355X peak)",
        "value": round(step_us / layers, 3),
        "unit": "us/layer-step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (bf16 MFMA products, fp32 sums)" if cfg.weight_fp8 else "bf16",
        "data": "synthetic (seeded random weights and KV caches of the workload's shapes)",
        "config": ({"workload": cfg.name, "hidden": cfg.hidden, "q_rank": cfg.idx_q_rank, "heads": cfg.idx_heads,
                    "head_dim": cfg.idx_head_dim, "requests": cfg.n_requests, "tokens_per_request": cfg.tokens_per_request,
                    "context": cfg.context, "page_size": cfg.page_size, "topk": cfg.topk, "mla_heads": cfg.mla_heads,
                    "rotation_copies": rotate,
                    "workers": int(p0.queue().shape[0])} if indexer else
                   {"workload": cfg.name, "layers": layers, "hidden": cfg.hidden, "inter": cfg.inter,
                    "q_heads": cfg.n_q_heads, "kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                    "batch": cfg.n_requests, "context": cfg.context, "page_size": cfg.page_size,
                    "vocab": cfg.vocab, "rotation_copies": rotate, "workers": int(p0.queue().shape[0])}),
        "step_us": round(step_us, 3),
        "achieved_GBps": round(achieved, 1),
        "hbm_frac_of_8TBps": round(achieved / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": _counter_traffic(cfg.name),
                     "kernel": "mk_worker<%s> (persistent megakernel, one launch per step)" % (
                         "0, false, false" if cfg.m == 1 else "1, false, false" if indexer else
                         "1, true, true" if cfg.m > 16 else "1, true, false")},
        "variants_us_per_step": variants,
        "step_us_stats": _stats(per_step),
        "hot_step_us": round(hot_ms * 1000.0, 3) if hot_ms is not None else
                       ("same as step_us: one copy, larger than the 256 MiB last-level cache" if step else None),
        "gpu_state": {"before": env_before, "after": env_after},
    }
    if variants:
        out["gain_split_us"] = {
            "branch_parallelism": round(variants["graph_single_stream"] - variants["graph_multi_stream"], 3),
            "in_kernel_scheduling": round(variants["graph_multi_stream"] - step_us, 3),
            "prefetch": round(variants["megakernel_no_prefetch"] - step_us, 3),
            # the same nodes with no op work (bodies skipped, loads of the leases not issued): what the
            # graph's kernel boundaries and per-node set-up cost beyond the megakernel's own framework
            "graph_fixed_cost_over_megakernel_framework": round(
                variants["graph_empty_framework"] - variants["megakernel_empty_framework"], 3),
        }
    if not args.no_diagnostics:
        out["diagnostics"] = _diagnostics(cfg, mk, plans, tensor_sets[0], stream, torch, step, step_us)
        if step and "tail_us" in out["diagnostics"]:
            tail = out["diagnostics"]["tail_us"] * step_us / out["diagnostics"]["traced_step_us"]
            out["us_per_layer_excluding_tail"] = round((step_us - tail) / layers, 3)
        out["stream_peak"] = _stream_peak(torch)
    if not args.no_cpu_baseline:
        _log("bench: CPU oracle baseline")
        from oracle import model as omodel
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            threads = os.cpu_count() or 1
        def one_pass():
            t0 = time.perf_counter()
            if step:
                omodel.run_qwen3_step(cfg, inp)
            elif indexer:
                omodel.run_indexer_front(cfg, inp)
            else:
                omodel.run_qwen3_layer(cfg, inp)
            return time.perf_counter() - t0

        runs = sorted(one_pass() for _ in range(3))
        dt = runs[1]
        one_thread = None
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                one_thread = one_pass()
        except Exception:
            pass
        out["cpu_baseline"] = {"value": round(dt * 1e6 / layers, 1), "unit": "us/layer-step", "cores": threads,
                               "kind": "oracle",
                               "one_thread_value": round(one_thread * 1e6 / layers, 1) if one_thread else None,
                               "sample": f"full passes of {cfg.name} ({layers} layer(s){' + lm_head' if step else ''}) "
                                         f"in float64 NumPy: median of 3 ({', '.join(f'{r:.2f}' for r in runs)} s) with "
                                         f"{threads} BLAS threads, then one pass on 1 thread "
                                         f"({one_thread or float('nan'):.2f} s); host cpu_count {os.cpu_count()}"}
    print(json.dumps(out), flush=True)
    for p in plans.values():
        p.close()
    return 0


def _stats(us):
    if not us:
        return None
    v = sorted(us)
    pick = lambda q: v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
    return {"median": round(pick(0.5), 3), "p10": round(pick(0.1), 3), "p90": round(pick(0.9), 3),
            "min": round(v[0], 3), "max": round(v[-1], 3), "steps": len(v)}


def _gpu_state():
    """Shader / memory clocks, power and performance level as rocm-smi reports them (None if unavailable,
    and not asked for under a profiler, whose preloaded library would follow rocm-smi's re-exec)."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--showperflevel", "--json"],
                           capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
    except Exception:
        return None
    card = next(iter(d.values())) if d else {}
    keep = {}
    for k, v in card.items():
        kl = k.lower()
        if any(t in kl for t in ("sclk", "mclk", "fclk", "power", "perf")):
            keep[k] = v
    return keep or None


def _diagnostics(cfg, mk, plans, tensors, stream, torch, step, step_us):
    """A traced pass after the timed region (perturbs timing, so reported apart): the share of
    instruction time the controllers spent polling for inputs and, for the decode step, the tail
    (final norm, lm_head, argmax) from the end of the last layer to the end of the step."""
    import numpy as np
    p = mk.Plan(cfg, flags=mk.MK_FLAG_TRACE)
    plans[-1] = p
    with torch.cuda.stream(stream):
        for _ in range(3):
            p.run(tensors, stream)
        p.sync(stream)
    torch.cuda.synchronize()
    tr = p.read_trace().astype(np.int64)
    q = p.queue()
    live = q[:, :, 0] != 0
    dur = (tr[:, :, 7] - tr[:, :, 0])[live]
    wait = (tr[:, :, 1] - tr[:, :, 0])[live]
    out = {"input_wait_share": round(float(wait.sum() / max(1, dur.sum())), 4),
           "repolls_per_instruction": round(float(tr[:, :, 8][live].mean()), 3),
           "traced_step_us": round(float((tr[:, :, 7][live].max() - tr[:, :, 0][live].min()) / 100.0), 2),
           "note": "from an MK_FLAG_TRACE pass: the time from a controller reaching an instruction to its inputs "
                   "being staged and current (waiting on producers, polling, staging), over the summed time of "
                   "every instruction; and the staging rounds repeated because a tag was stale"}
    if step:
        lm = live & (q[:, :, 0] == 6)
        layers_end = tr[:, :, 7][live & ~lm].max()
        out["tail_us"] = round(float((tr[:, :, 7][lm].max() - layers_end) / 100.0), 2)
        out["cross_layer_prefetch"] = _cross_layer(q, tr, live, cfg.num_layers)
    return out


def _cross_layer(q, tr, live, layers):
    """Leases of the next layer issued during this one: for every worker and layer boundary, the
    time from the issue of its first layer-(l+1) instruction's lease (trace word 9) to the end of its
    last layer-l instruction, and to the end of layer l's last down tile on any worker."""
    import numpy as np
    layer = q[:, :, 20].astype(np.int64)
    down_end = [tr[:, :, 7][live & (q[:, :, 0] == 5) & (layer == l)].max() for l in range(layers)]
    own, glob = [], []
    for w in range(q.shape[0]):
        idx = np.flatnonzero(live[w] & (q[w, :, 0] != 6))
        for a, b in zip(idx[:-1], idx[1:]):
            if layer[w, b] == layer[w, a] + 1 and tr[w, b, 9] != 0:
                own.append(tr[w, a, 7] - tr[w, b, 9])
                glob.append(down_end[layer[w, a]] - tr[w, b, 9])
    own, glob = np.array(own) / 100.0, np.array(glob) / 100.0
    if not len(own):
        return None
    return {"boundaries": int(len(own)), "share_issued_before_own_layer_end": round(float((own > 0).mean()), 3),
            "median_lead_over_own_layer_end_us": round(float(np.median(own)), 2),
            "share_issued_before_layer_done": round(float((glob > 0).mean()), 3),
            "median_lead_over_layer_done_us": round(float(np.median(glob)), 2)}


def _stream_peak(torch):
    """Measured HBM rates of plain torch kernels over 2 GiB: a device-to-device copy (read + write
    bytes) and sums (read bytes), best of 5.  The float64 sum is the fastest reader torch has here
    (fp32 sums read at about 4 TB/s, fp64 sums at about 6.1); a hand-written loop of 16-byte
    non-temporal loads reads about 7.1 TB/s on MI355X, so no torch figure is the hardware's peak."""
    n = 1 << 29  # 2 GiB of fp32
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)

    def best(fn, nbytes):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        return round(nbytes / min(t) / 1e9, 1)

    a64 = a.view(torch.float64)
    res = {"copy_GBps_read_plus_write": best(lambda: b.copy_(a), 2 * 4 * n),
           "sum_GBps_read": best(lambda: a.sum(), 4 * n),
           "sum_f64_GBps_read": best(lambda: a64.sum(), 4 * n), "bytes": 4 * n}
    del a, b
    torch.cuda.empty_cache()
    return res


def copy_calibration(args, torch) -> int:
    """Plain copy of a known size: its profiler byte counters give the scale factor that turns
    counter readings of the megakernel into HBM bytes."""
    n = args.copy_bytes // 16 * 16
    src = torch.empty(n // 4, dtype=torch.int32, device="cuda").random_()
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"copy_bytes": n, "read_bytes": n, "write_bytes": n, "ms_per_copy": round(ms, 5),
                      "GBps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
