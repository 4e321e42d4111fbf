"""GPU parity of the indexer front (A0 -> {B0, C0, B1} -> D1 -> E1) against the CPU oracle, through
the C ABI: megakernel and both graph baselines.

Tolerance: max abs error 6e-2 (the FP8 path) on the scores and the fp32 intermediates, against the
oracle value before its output rounding; bf16 q passes when it is the bf16 rounding of a value within
that error.  Scores are compared with the fully independent oracle (no value taken from the GPU).
e4m3 decisions at hq, qaq and the new keys (tests/fp8_check.py): each GPU code is the oracle's
round-to-nearest-even code except inside the ambiguity set the oracle computes from its own values,
where it is one of the two enclosing codes.  Key-cache writes: the written slot set is exact (every
other byte of the cache and its scales is unchanged).  Scores: -inf exactly for keys after a token's
position; all modes give the same bits.

Top-k (plans with cfg.topk): a selection decided in floating point, so two checks.  Validity on the
kernel's own fp32 scores, exactly: min(k, keys) distinct positions <= the token's position in
ascending order, -1 after them, and every selected key beats every unselected one (a larger score,
or an equal score and a smaller position).  Against the independent oracle: the kernel's set and
the oracle's (computed on the oracle's own scores) may differ only in keys whose oracle score lies
within 2 x TOL of the oracle's k-th largest score (a key outside that window is above or below the
kernel's own threshold too, since every kernel score is within TOL of the oracle's).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import model
from oracle.numerics import e4m3_decode
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu
TOL = 6e-2


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def opnd_fp8_rows(buf: np.ndarray, K: int) -> np.ndarray:
    return buf.view(np.uint8)[:16 * K].reshape(K // 64, 4, 16, 16).transpose(2, 0, 1, 3).reshape(16, K)


def qi_rows(buf: np.ndarray, nh: int) -> np.ndarray:
    """[16, nh, 128] float64 from the score's A-operand order: per (token, 16-head block, step f)
    1 KiB, lane (h % 16) + 16 g holding dims 64 (f // 2) + 16 g + 8 (f % 2) + 0..7."""
    a = buf.view(np.uint16)[:16 * nh * 128].reshape(16, nh // 16, 4, 4, 16, 8)  # [m, hb, f, g, hh, e]
    d = np.arange(128)
    f, g, e = 2 * (d // 64) + (d % 16) // 8, (d % 64) // 16, d % 8
    out = a[:, :, f, g, :, e]  # [128 d, 16 m, hb, 16 hh] after advanced indexing
    out = np.moveaxis(out, 0, -1).reshape(16, nh, 128)
    return (out.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ws(run, name, dtype=torch.uint8):
    return run.region(name, dtype).cpu().numpy()


def _kernel_decisions(run, ref_slots):
    cfg = run.cfg
    M, H, qr = cfg.m, cfg.hidden, cfg.idx_q_rank
    page, off = ref_slots["slot_page"], ref_slots["slot_off"]
    return {"hq": (opnd_fp8_rows(_ws(run, "hq"), H)[:M], _ws(run, "sh").view(np.float32)[:M].astype(np.float64)),
            "qaq": (opnd_fp8_rows(_ws(run, "qaq"), qr)[:M], _ws(run, "sqa").view(np.float32)[:M].astype(np.float64)),
            "kq": (run.t["key_cache"].cpu().numpy()[page, off],
                   run.t["key_scale"].cpu().numpy().astype(np.float64)[page, off])}


def _oracle(run, inp):
    """(resolved, independent): the independent oracle takes nothing from the GPU; the resolved one
    checks every GPU code at hq, qaq and the new keys against the oracle's own and continues with the
    GPU's choice only inside the oracle's ambiguity set."""
    from fp8_check import KernelTies
    cfg = run.cfg
    ind = model.run_indexer_front(cfg, inp)
    ties = KernelTies(_kernel_decisions(run, ind))
    ref = model.run_indexer_front(cfg, inp, ties=ties)
    _say(f"  FP8 decisions: {ties.summary()}")
    return ref, ind


def _check(run, inp, ref, ind, tag, intermediates=True):
    from gpu_helpers import bf16_excess
    cfg = run.cfg
    M, H, qr, nh = cfg.m, cfg.hidden, cfg.idx_q_rank, cfg.idx_heads
    ctx = inp["context_lens"]
    pos = ref["pos"]
    score = run.t["score_out"].cpu().numpy().astype(np.float64).reshape(M, run.smax)
    worst = worst_res = 0.0
    for m in range(M):
        c = int(ctx[m // cfg.tokens_per_request])
        row = score[m, :c]
        fin = np.arange(c) <= pos[m]
        assert np.all(np.isneginf(row[~fin])), f"{tag}: row {m} keys after the position are not -inf"
        assert np.all(np.isfinite(row[fin])), f"{tag}: row {m}"
        worst = max(worst, float(np.max(np.abs(row[fin] - ind["score_pre"][m, :c][fin]))))
        worst_res = max(worst_res, float(np.max(np.abs(row[fin] - ref["score_pre"][m, :c][fin]))))
    big = np.abs(ind['score_pre'][np.isfinite(ind['score_pre'])]).max()
    _say(f"  {tag}: score err {worst:.3e} against the independent oracle, {worst_res:.3e} resolved "
         f"(max |score| {big:.3g})")
    assert worst <= TOL and worst_res <= TOL, f"{tag}: score err {worst} / {worst_res}"
    if not intermediates:
        return
    from fp8_check import SCALE_RTOL
    sh = _ws(run, "sh").view(np.float32)[:M].astype(np.float64)
    assert np.max(np.abs(sh / ref["sh"] - 1)) <= SCALE_RTOL, tag
    assert np.array_equal(e4m3_decode(opnd_fp8_rows(_ws(run, "hq"), H)[:M]), e4m3_decode(ref["hq"])), tag
    qa = _ws(run, "qa").view(np.float32)[:M * qr].astype(np.float64).reshape(M, qr)
    assert np.max(np.abs(qa - ref["qa"])) <= TOL, tag
    sqa = _ws(run, "sqa").view(np.float32)[:M].astype(np.float64)
    assert np.max(np.abs(sqa / ref["sqa"] - 1)) <= SCALE_RTOL, tag
    assert np.array_equal(e4m3_decode(opnd_fp8_rows(_ws(run, "qaq"), qr)[:M]), e4m3_decode(ref["qaq"])), tag
    w = _ws(run, "w").view(np.float32)[:M * nh].astype(np.float64).reshape(M, nh)
    assert np.max(np.abs(w - ref["w_pre"])) <= TOL, tag
    k = _ws(run, "k").view(np.float32)[:M * 128].astype(np.float64).reshape(M, 128)
    assert np.max(np.abs(k - ref["k_lin"])) <= TOL, tag
    qi = qi_rows(_ws(run, "qi"), nh)
    assert bf16_excess(qi[:M], ref["qi_pre"], TOL) <= 0, tag
    assert np.all(qi[M:] == 0), tag


def _check_cache(run, inp, ref, kc0, ks0, tag):
    cfg = run.cfg
    kc = run.t["key_cache"].cpu().numpy()
    ks = run.t["key_scale"].cpu().numpy().astype(np.float64)
    mask = np.ones(kc.shape[:2], dtype=bool)
    page, off = ref["slot_page"], ref["slot_off"]
    mask[page, off] = False
    assert np.array_equal(kc[mask], kc0[mask]) and np.array_equal(ks[mask], ks0[mask]), f"{tag}: other slots changed"
    from fp8_check import SCALE_RTOL
    assert np.max(np.abs(ks[page, off] / ref["sk"] - 1)) <= SCALE_RTOL, tag
    assert np.array_equal(e4m3_decode(kc[page, off]), e4m3_decode(ref["kq"])), tag


def _check_topk(run, ind, tag):
    cfg = run.cfg
    M, k = cfg.m, cfg.topk
    got = run.t["topk_out"].cpu().numpy().astype(np.int64).reshape(M, k)
    score = run.t["score_out"].cpu().numpy().astype(np.float64).reshape(M, run.smax)
    window = 0
    for m in range(M):
        nv = int(ind["pos"][m]) + 1
        n = min(k, nv)
        sel = got[m, :n]
        assert np.all(got[m, n:] == -1), f"{tag}: row {m} padding"
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < nv, f"{tag}: row {m} positions"
        s = score[m, :nv]
        chosen = np.zeros(nv, bool)
        chosen[sel] = True
        if n < nv:  # every selected key beats every unselected one
            lo = s[chosen].min()
            assert s[~chosen].max() <= lo, f"{tag}: row {m} an unselected score above the selection"
            tie_sel = np.flatnonzero(chosen & (s == lo))
            tie_out = np.flatnonzero(~chosen & (s == lo))
            assert tie_out.size == 0 or tie_out.min() > tie_sel.max(), f"{tag}: row {m} ties not to the smaller position"
        # against the independent oracle: differences only near its k-th largest score
        os_ = ind["score"][m, :nv]
        kth = np.sort(os_)[::-1][n - 1]
        ref = np.zeros(nv, bool)
        ref[ind["topk"][m, :n]] = True
        diff = np.flatnonzero(ref != chosen)
        assert np.all(np.abs(os_[diff] - kth) <= 2 * TOL), f"{tag}: row {m} differs from the oracle away from its threshold"
        window += int(np.sum(np.abs(os_ - kth) <= 2 * TOL))
        assert len(diff) <= 2 * np.sum(np.abs(os_ - kth) <= 2 * TOL)
    _say(f"  {tag}: top-{k} valid on the kernel's scores; {window} keys of {M} rows within the oracle's threshold window")


def _check_mla(run, ref, ind, tag):
    """The main-MLA half: D0's q_nope (bf16, D2's operand order in the workspace) and D2's q_lat
    (bf16 output) against the oracle before their roundings, with the FP8 tolerance; q_lat against
    the independent oracle too."""
    from gpu_helpers import bf16_excess, bf16_to_f64
    cfg = run.cfg
    M, nm = cfg.m, cfg.mla_heads
    qn_buf = _ws(run, "qn").view(np.uint16)[:16 * nm * 128]
    k = np.arange(nm * 128)
    rows = []
    for m in range(M):  # operand order: step k // 32 of 1 KiB, lane m + 16 ((k % 32) // 8), element k % 8
        idx = (k // 32) * 512 + (m + 16 * ((k % 32) // 8)) * 8 + k % 8
        rows.append(qn_buf[idx])
    qn = (np.array(rows).astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(M, nm, 128)
    assert bf16_excess(qn, ref["qn_pre"], TOL) <= 0, f"{tag}: q_nope"
    ql = bf16_to_f64(run.t["qlat_out"]).reshape(M, nm, 512)
    assert bf16_excess(ql, ref["qlat_pre"], TOL) <= 0, f"{tag}: q_lat against the resolved oracle"
    err = float(np.max(np.abs(ql - ind["qlat_pre"])))
    _say(f"  {tag}: q_lat err {err:.3e} against the independent oracle (max |q_lat| {np.max(np.abs(ind['qlat_pre'])):.3g})")
    assert bf16_excess(ql, ind["qlat_pre"], TOL) <= 0, f"{tag}: q_lat against the independent oracle"


def _case(cfg, ctx, seed, modes=(("mk", False), ("graph", False), ("graph", True), ("mk", False)),
          W=0, intermediates=True, edit=None):
    from gpu_helpers import IndexerRun
    inp = make_inputs(cfg, seed=seed)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    if edit is not None:
        edit(inp)
    kc0, ks0 = inp["key_cache"].copy(), inp["key_scale"].astype(np.float64).copy()
    run = IndexerRun(cfg, inp, num_workers=W)
    outs, outs_k = [], []
    ref = None
    for mode, ms in modes:
        _say(f"case: {cfg.name} R={cfg.n_requests} T={cfg.tokens_per_request} ctx={ctx} W={W} {mode} ms={ms}")
        run.t["score_out"].fill_(float("nan"))
        run.run(mode, ms)
        if ref is None:  # every mode gives the same bits (checked below)
            ref, ind = _oracle(run, inp)
        _check(run, inp, ref, ind, f"{mode}/{ms}", intermediates)
        _check_cache(run, inp, ref, kc0, ks0, f"{mode}/{ms}")
        outs.append(run.t["score_out"].clone())
        if cfg.topk:
            _check_topk(run, ind, f"{mode}/{ms}")
            outs_k.append(run.t["topk_out"].clone())
            run.t["topk_out"].fill_(-7)
        if cfg.mla_heads:
            _check_mla(run, ref, ind, f"{mode}/{ms}")
            outs_k.append(run.t["qlat_out"].clone())
            run.t["qlat_out"].fill_(-1)
    for o in outs[1:]:
        assert torch.equal(torch.nan_to_num(o), torch.nan_to_num(outs[0]))
    nk = len(outs_k) // len(modes)  # per mode: [top-k], [q_lat]
    for i in range(nk, len(outs_k)):
        assert torch.equal(outs_k[i], outs_k[i % nk])
    return outs_k[0] if cfg.topk else None


@pytest.mark.parametrize("R,T,ctx,W", [(2, 8, [300, 133], 0), (3, 5, [64, 196, 5], 37)])
def test_indexer_reduced(R, T, ctx, W):
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, n_requests=R,
                              tokens_per_request=T, context=max(ctx))
    _case(cfg, ctx, seed=11, W=W)


@pytest.mark.timeout(600)
def test_indexer_full_size():
    cfg = get_config("indexer_front")
    _case(cfg, [cfg.context] * cfg.n_requests, seed=0, modes=(("mk", False), ("graph", False), ("graph", True)))


@pytest.mark.parametrize("R,T,ctx,W,k", [(2, 8, [300, 133], 0, 64), (3, 5, [64, 196, 5], 37, 100)])
def test_indexer_topk_reduced(R, T, ctx, W, k):
    """Top-k after the score, with rows that have more keys than k and rows that have fewer."""
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, n_requests=R,
                              tokens_per_request=T, context=max(ctx), topk=k)
    _case(cfg, ctx, seed=12, W=W, intermediates=False)


@pytest.mark.parametrize("k", [64, 250])
def test_indexer_topk_ties(k):
    """Every prior key of every request identical (the same e4m3 codes and scale): each token's
    scores over its prior keys are exactly equal, so its selection is decided by the tie rule --
    the prior keys it takes are the first ones, positions 0, 1, ... -- besides its own request's
    new keys, whichever of them score above the tie."""
    R, T, ctx = 2, 8, [300, 133]
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, n_requests=R,
                              tokens_per_request=T, context=max(ctx), topk=k)

    def same_keys(inp):
        inp["key_cache"][:] = inp["key_cache"].reshape(-1, inp["key_cache"].shape[-1])[0]
        inp["key_scale"][:] = inp["key_scale"].reshape(-1)[0]

    got = _case(cfg, ctx, seed=14, intermediates=False, edit=same_keys, modes=(("mk", False), ("graph", False)))
    sel = got.cpu().numpy().astype(np.int64).reshape(cfg.m, k)
    for m in range(cfg.m):
        r, j = divmod(m, T)
        prior = int(ctx[r]) - T  # keys before the request's new tokens
        p = sel[m][(sel[m] >= 0) & (sel[m] < prior)]
        assert np.array_equal(p, np.arange(len(p))), f"row {m}: tied prior keys not taken from position 0"
        assert len(p) == min(k, prior + j + 1) - np.sum((sel[m] >= prior)), f"row {m}: selection size"


@pytest.mark.timeout(600)
def test_indexer_topk_full_size():
    cfg = get_config("indexer_front_topk")  # Top-2048 of 8192 keys per token, 16 tokens
    _case(cfg, [cfg.context] * cfg.n_requests, seed=0, modes=(("mk", False), ("graph", False)), intermediates=False)


@pytest.mark.parametrize("R,T,ctx,W,nm", [(2, 8, [300, 133], 0, 3), (3, 5, [64, 196, 5], 37, 2)])
def test_attention_pre_reduced(R, T, ctx, W, nm):
    """The indexer front with the main-MLA query half (D0 -> D2): all of the indexer's checks, plus
    q_nope and q_lat."""
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, n_requests=R,
                              tokens_per_request=T, context=max(ctx), mla_heads=nm)
    _case(cfg, ctx, seed=13, W=W)


@pytest.mark.timeout(600)
def test_attention_pre_full_size():
    cfg = get_config("attention_pre")  # 64 main-MLA heads: D0 over q rank 1536, D2 into a 512 latent
    _case(cfg, [cfg.context] * cfg.n_requests, seed=0, modes=(("mk", False), ("graph", False), ("graph", True)),
          intermediates=False)
