"""GPU parity of the multi-row (16-token) decode layer -- bf16 and W8A8 FP8 -- against the CPU
oracle, through the C ABI: megakernel and both graph baselines.

Tolerances: max abs error 2e-2 (bf16) and 6e-2 (FP8 weights and activations) on the layer outputs
y and r2 and on the intermediates, against the oracle value before its output rounding; a value
the layer materialises in bf16 passes when it is the bf16 rounding of a value within that error
(bf16 spacing alone exceeds 2e-2 from |v| >= 8).  Cache writes: the written slot set is exact
(every other byte of both caches is unchanged bit for bit).
FP8 decisions (tests/fp8_check.py): at each of the four per-token quantisation points the GPU's
code equals the oracle's round-to-nearest-even code except inside the ambiguity set the oracle
computes from its own values (within delta of a rounding midpoint); there it is one of the two
enclosing codes, and the oracle continues with that choice -- nowhere else.  The fully
independent oracle (no choice taken from the GPU) is run too: r2 is compared with it at the
tolerance, and its y error is reported (a code taken the other way at an ambiguous point of o
moves the next projection's inputs and cascades; measured in the design notes).
At the full sizes the oracle runs request by request in chunks: the rows of the layer are
independent requests, so a request's outputs depend only on its own row, its own cache pages and
the shared weights; a chunk's pages are copied into a compact pool with a remapped block table.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import model
from oracle.numerics import bf16_bits_to_f64, e4m3_decode
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _tol(cfg):
    return 6e-2 if cfg.act_fp8 else 2e-2


def opnd_bf16_rows(buf: np.ndarray, K: int) -> np.ndarray:
    """[16 G, K] float64 from the bf16 matrix-core operand order: 16-row groups one after the
    other; inside a group, per K step of 32, lane m + 16 * ((k % 32) // 8) holds 8 consecutive k of
    row m of the group."""
    u = buf.view(np.uint16)
    G = len(u) // (16 * K)
    a = u[:G * 16 * K].reshape(G, K // 32, 4, 16, 8).transpose(0, 3, 1, 2, 4).reshape(16 * G, K)
    return bf16_bits_to_f64(a)


def opnd_fp8_rows(buf: np.ndarray, K: int) -> np.ndarray:
    """[16 G, K] e4m3 codes from the FP8 operand order: 16-row groups one after the other; inside
    a group, per K step of 64, lane m + 16 * ((k % 64) // 16) holds 16 consecutive k of row m."""
    u = buf.view(np.uint8)
    G = len(u) // (16 * K)
    return u[:G * 16 * K].reshape(G, K // 64, 4, 16, 16).transpose(0, 3, 1, 2, 4).reshape(16 * G, K)


def _run(cfg, inp, W=0):
    from gpu_helpers import QwenRun
    # the plan is built for the inputs' context lengths (tile counts and RoPE positions follow them)
    run = QwenRun(cfg, inp, num_workers=W, ctx=[int(c) for c in inp["context_lens"]])
    run.inp_block_table, run.inp_ctx = inp["block_table"], inp["context_lens"]
    return run


def _ws(run, name, dtype=torch.uint8):
    return run.region(name, dtype).cpu().numpy()


def _decisions(run, rows):
    """The FP8 path's per-token codes and scales at its four quantisation points, for the given rows."""
    cfg = run.cfg
    H, I, q = cfg.hidden, cfg.inter, cfg.n_q_heads * cfg.head_dim
    dec = {}
    for key, name, sname, K in (("h1q", "h1", "s1", H), ("oq", "oq", "so", q), ("h2q", "h2", "s2", H),
                                ("mq", "mq", "sm", I)):
        codes = opnd_fp8_rows(_ws(run, name), K)[rows]
        s = _ws(run, sname).view(np.float32)[:cfg.m].astype(np.float64)[rows]
        dec[key] = (codes, s)
    return dec


def _bf16_decisions(run, rows):
    """The kernel's bf16 q (as its attention materialised it, from the workspace), k and v (the
    cache rows it wrote at the new tokens' slots), for the given rows: the oracle resolves its
    ambiguous bf16 roundings of q, k, v from these (tests/fp8_check.py)."""
    cfg = run.cfg
    Hq, Hkv, d, P = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.page_size
    qb = bf16_bits_to_f64(_ws(run, "qb").view(np.uint16)[:cfg.m * Hq * d]).reshape(cfg.m, Hq, d)[rows]
    kc = run.t["k_cache"].cpu().numpy().view(np.uint16)[0]
    vc = run.t["v_cache"].cpu().numpy().view(np.uint16)[0]
    bt, ctx = run.inp_block_table, run.inp_ctx
    slots = [(bt[r][(int(ctx[r]) - 1) // P], (int(ctx[r]) - 1) % P) for r in rows]
    k = np.stack([bf16_bits_to_f64(kc[p, o]) for p, o in slots]).reshape(len(rows), Hkv, d)
    v = np.stack([bf16_bits_to_f64(vc[p, o]) for p, o in slots]).reshape(len(rows), Hkv, d)
    return {"q": qb, "k": k, "v": v}


def _oracle(cfg, inp, run, rows):
    """(resolved, independent) oracle layers for the given rows (inputs already restricted to them).
    bf16: both are the plain oracle.  FP8: ``resolved`` checks every GPU code against the oracle's
    own at each quantisation point and continues with the GPU's choice only inside the oracle's
    ambiguity set; ``independent`` takes no choice from the GPU."""
    from fp8_check import KernelTies
    if not cfg.act_fp8:
        ref = model.run_qwen3_layer(cfg, inp)
        return ref, ref
    ties = KernelTies(_decisions(run, rows), bf16=_bf16_decisions(run, rows))
    ref = model.run_qwen3_layer(cfg, inp, ties=ties)
    _say(f"  FP8 decisions: {ties.summary()}")
    ind = model.run_qwen3_layer(cfg, inp) if ties.any_flip else ref
    return ref, ind


def _check_outputs(run, ref, ind, rows, tag):
    """y, r2 of the given GPU rows against the oracle rows 0.. of ref (and r2 against the
    independent oracle)."""
    from gpu_helpers import bf16_excess, bf16_to_f64
    cfg, tol = run.cfg, _tol(run.cfg)
    y = bf16_to_f64(run.t["y_out"]).reshape(cfg.m, cfg.hidden)[rows]
    r2 = run.t["r2_out"].cpu().numpy().astype(np.float64).reshape(cfg.m, cfg.hidden)[rows]
    ey, er = np.max(np.abs(y - ref["y_pre"])), np.max(np.abs(r2 - ref["r2"]))
    eyi, eri = np.max(np.abs(y - ind["y_pre"])), np.max(np.abs(r2 - ind["r2"]))
    _say(f"  {tag}: y err {ey:.3e} (max |y| {np.abs(ref['y_pre']).max():.3g}) r2 err {er:.3e}; "
         f"independent oracle: y err {eyi:.3e} r2 err {eri:.3e}")
    assert bf16_excess(y, ref["y_pre"], tol) <= 0 and er <= tol, f"{tag}: y err {ey}, r2 err {er}"
    assert eri <= tol, f"{tag}: r2 err {eri} against the independent oracle"


def _check_slot_set(run, inp, k_before, v_before, tag):
    """Only the slots of the new tokens changed: every other byte of both caches is unchanged."""
    cfg = run.cfg
    kc = run.t["k_cache"].cpu().numpy().view(np.uint16)[0]
    vc = run.t["v_cache"].cpu().numpy().view(np.uint16)[0]
    mask = np.ones(kc.shape[:2], dtype=bool)
    ctx = inp["context_lens"]
    for r in range(cfg.n_requests):
        p = int(ctx[r]) - 1
        mask[inp["block_table"][r][p // cfg.page_size], p % cfg.page_size] = False
    assert np.array_equal(kc[mask], k_before[mask]) and np.array_equal(vc[mask], v_before[mask]), tag
    return kc, vc


def _check_written_rows(run, kc, vc, inp, ref, rows, tag):
    """The rows written at the new tokens' slots match the oracle's k and v (before rounding)."""
    cfg, tol = run.cfg, _tol(run.cfg)
    from gpu_helpers import bf16_excess
    ctx = inp["context_lens"]
    for i, r in enumerate(rows):
        p = int(ctx[r]) - 1
        page, off = inp["block_table"][r][p // cfg.page_size], p % cfg.page_size
        assert bf16_excess(bf16_bits_to_f64(kc[page, off]), ref["k_pre"][i], tol) <= 0, tag
        assert bf16_excess(bf16_bits_to_f64(vc[page, off]), ref["v_pre"][i], tol) <= 0, tag


def _check_cache(run, inp, ref, rows, k_before, v_before, tag):
    """The written slots are exactly the oracle's; their rows match; nothing else changed."""
    kc, vc = _check_slot_set(run, inp, k_before, v_before, tag)
    _check_written_rows(run, kc, vc, inp, ref, rows, tag)


def _check_intermediates(run, ref, tag):
    """Every workspace intermediate of a run covering all rows (reduced shapes)."""
    cfg, tol = run.cfg, _tol(run.cfg)
    M, H, I, q = cfg.m, cfg.hidden, cfg.inter, cfg.n_q_heads * cfg.head_dim
    qkv = run.payload_f32("qkv").reshape(M, -1)
    assert np.max(np.abs(qkv - ref["qkv"])) <= tol, tag
    r1 = _ws(run, "r1").view(np.float32).astype(np.float64)[:M * H].reshape(M, H)
    assert np.max(np.abs(r1 - ref["r1"])) <= 1e-5, tag  # an fp32 add: rounding only
    r2 = _ws(run, "r2").view(np.float32).astype(np.float64)[:M * H].reshape(M, H)
    assert np.max(np.abs(r2 - ref["r2"])) <= tol, tag
    if cfg.act_fp8:
        from fp8_check import SCALE_RTOL
        # codes: exactly the resolved oracle's (its own RNE codes, the GPU's choice only at ambiguous
        # points of the first run: every later mode must reproduce them); scales within SCALE_RTOL
        for name, K, key, skey in (("h1", H, "h1q", "s1"), ("h2", H, "h2q", "s2"), ("oq", q, "oq", "so"),
                                   ("mq", I, "mq", "sm")):
            s = _ws(run, skey).view(np.float32)[:M].astype(np.float64)
            assert np.max(np.abs(s / ref[skey] - 1)) <= SCALE_RTOL, f"{tag} {skey}"
            codes = opnd_fp8_rows(_ws(run, name), K)[:M]
            assert np.array_equal(e4m3_decode(codes), e4m3_decode(ref[key])), f"{tag} {name}"
        o = _ws(run, "o").view(np.float32)[:M * q].astype(np.float64).reshape(M, q)
        assert np.max(np.abs(o - ref["o_pre"])) <= tol, tag
        m = _ws(run, "m").view(np.float32)[:M * I].astype(np.float64).reshape(M, I)
        assert np.max(np.abs(m - ref["m_pre"])) <= tol, tag
        pad = [opnd_fp8_rows(_ws(run, n), K)[M:] for n, K in (("h1", H), ("h2", H), ("oq", q), ("mq", I))]
    else:
        from gpu_helpers import bf16_excess
        for name, K, key in (("h1", H, "h1_pre"), ("h2", H, "h2_pre"), ("o", q, "o_pre"), ("m", I, "m_pre")):
            v = opnd_bf16_rows(_ws(run, name), K)
            assert bf16_excess(v[:M], ref[key], tol) <= 0, f"{tag} {name}"
        pad = [opnd_bf16_rows(_ws(run, n), K)[M:] for n, K in (("h1", H), ("h2", H), ("o", q), ("m", I))]
    assert all(np.all(p == 0) for p in pad), f"{tag}: padding rows of the operand-order inputs were written"


def _reduced(fp8, R, ctx):
    base = get_config("qwen3_8b_layer_fp8" if fp8 else "qwen3_8b_layer")
    return dataclasses.replace(base, hidden=1024, inter=2048 if fp8 else 1536, n_q_heads=8, n_kv_heads=2,
                               n_requests=R, context=max(ctx), page_size=16)


@pytest.mark.parametrize("R", [5, 40, 256])
@pytest.mark.parametrize("fp8", [False, True])
def test_m16_reduced_layer_all_modes(fp8, R):
    """Every intermediate and output at reduced shapes; 40 requests take three 16-row groups (the
    last one ragged), 256 the most a plan takes (sixteen groups)."""
    ctx = [1, 37, 300, 513, 64] if R == 5 else [int(c) for c in np.random.default_rng(R).integers(1, 514, R)]
    cfg = _reduced(fp8, len(ctx), ctx)
    inp = make_inputs(cfg, seed=3)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    k0, v0 = inp["k_cache"][0].copy(), inp["v_cache"][0].copy()
    rows = list(range(cfg.m))
    for W in (0, 37):
        run = _run(cfg, inp, W)
        assert run.plan.queue()[0, 0, 4] == 1  # the multi-row plan
        outs = []
        ref = None
        for mode, ms in (("mk", False), ("graph", False), ("graph", True), ("mk", False)):
            _say(f"case: reduced multi-row fp8={fp8} W={W} {mode} multistream={ms}")
            run.t["y_out"].zero_()
            run.t["r2_out"].zero_()
            run.run(mode, ms)
            if ref is None:  # every mode gives the same bits (checked below)
                ref, ind = _oracle(cfg, inp, run, rows)
            _check_outputs(run, ref, ind, rows, f"{mode}/{ms}")
            _check_cache(run, inp, ref, rows, k0, v0, f"{mode}/{ms}")
            _check_intermediates(run, ref, f"W={W} {mode}/{ms}")
            outs.append((run.t["y_out"].clone(), run.t["r2_out"].clone()))
        # fixed-order reductions: every mode gives the same bits
        for y, r in outs[1:]:
            assert torch.equal(y, outs[0][0]) and torch.equal(r, outs[0][1])


def _sample_inputs(cfg, inp, rows):
    """Inputs of a layer restricted to some requests, their cache pages copied into a compact pool."""
    bt = inp["block_table"][rows]
    pages = np.unique(bt)
    remap = np.full(cfg.num_phys_pages, -1, dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    sub = dict(inp)
    sub["block_table"] = remap[bt].astype(np.int32)
    sub["context_lens"] = inp["context_lens"][rows]
    sub["x"], sub["r_in"] = inp["x"][rows], inp["r_in"][rows]
    sub["k_cache"], sub["v_cache"] = inp["k_cache"][:, pages], inp["v_cache"][:, pages]
    scfg = dataclasses.replace(cfg, n_requests=len(rows))
    return scfg, sub


@pytest.mark.timeout(900)
def test_m64_full_size_sampled_requests():
    """The 64-request layer (four 16-row groups, random page tables) at full size: the written slot
    set exact, y / r2 and the written rows of eight requests spread over the four groups (both ends
    of each) against the oracle; the graph modes bitwise equal to the megakernel."""
    name = "qwen3_8b_layer_m64"
    cfg = get_config(name)
    _say(f"case: {name} full size, inputs")
    inp = make_inputs(cfg, seed=0)
    k0, v0 = inp["k_cache"][0].copy(), inp["v_cache"][0].copy()
    run = _run(cfg, inp)
    _say(f"case: {name} megakernel W=all")
    run.run("mk")
    kc, vc = _check_slot_set(run, inp, k0, v0, f"{name} mk")
    for rows in ([0, 15, 16, 31], [32, 47, 48, 63]):
        scfg, sub = _sample_inputs(cfg, inp, rows)
        _say(f"case: {name} oracle on requests {rows}")
        ref, ind = _oracle(scfg, sub, run, rows)
        _check_outputs(run, ref, ind, rows, f"{name} mk requests {rows}")
        _check_written_rows(run, kc, vc, inp, ref, rows, f"{name} mk")
    y_mk, r2_mk = run.t["y_out"].clone(), run.t["r2_out"].clone()
    for ms in (False, True):
        _say(f"case: {name} graph multistream={ms}")
        run.t["y_out"].zero_()
        run.t["r2_out"].zero_()
        run.run("graph", ms)
        assert torch.equal(run.t["y_out"], y_mk) and torch.equal(run.t["r2_out"], r2_mk)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["qwen3_8b_layer", "qwen3_8b_layer_fp8"])
def test_m16_full_size_all_requests(name):
    """Every one of the 16 requests at full size, the oracle run on chunks of four requests."""
    cfg = get_config(name)
    _say(f"case: {name} full size, inputs")
    inp = make_inputs(cfg, seed=0)
    k0, v0 = inp["k_cache"][0].copy(), inp["v_cache"][0].copy()
    run = _run(cfg, inp)
    _say(f"case: {name} megakernel W=all")
    run.run("mk")
    kc, vc = _check_slot_set(run, inp, k0, v0, f"{name} mk")
    for rows in ([0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11], [12, 13, 14, 15]):
        scfg, sub = _sample_inputs(cfg, inp, rows)
        _say(f"case: {name} oracle on requests {rows}")
        ref, ind = _oracle(scfg, sub, run, rows)
        _check_outputs(run, ref, ind, rows, f"{name} mk requests {rows}")
        _check_written_rows(run, kc, vc, inp, ref, rows, f"{name} mk")
    y_mk, r2_mk = run.t["y_out"].clone(), run.t["r2_out"].clone()
    for ms in (False, True):
        _say(f"case: {name} graph multistream={ms}")
        run.t["y_out"].zero_()
        run.t["r2_out"].zero_()
        run.run("graph", ms)
        assert torch.equal(run.t["y_out"], y_mk) and torch.equal(run.t["r2_out"], r2_mk)
