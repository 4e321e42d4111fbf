"""Error paths of the megakernel through the C ABI, each forced from the host so that every kernel still
exits normally:

* a block-table entry outside the page pool: the kernels read it as page 0 (no access leaves the cache
  pool) and record it; mk_sync reports MK_ERR_INVALID, the plan's counters are reset, and the next run
  with a valid table matches the oracle;
* a wait that expires (MK_FLAG_DEBUG_SHORT_WATCHDOG shrinks the kernel's own bounded wait to one clock
  tick): the worker records a timeout, the others abandon their waits, mk_sync reports MK_ERR_TIMEOUT,
  and a plan without the flag then runs correctly on the same tensors.
Covered for the single-token family, the multi-row family with loader waves, and the indexer front."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from oracle import model
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _qwen_cases():
    small = dataclasses.replace(get_config("qwen3_0p6b_layer"), random_pages=True, context=300)
    ctx = [37, 300, 513, 64]
    m16 = dataclasses.replace(get_config("qwen3_8b_layer"), hidden=1024, inter=1536, n_q_heads=8, n_kv_heads=2,
                              n_requests=len(ctx), context=max(ctx), page_size=16, random_pages=True)
    return [(small, [300]), (m16, ctx)]


def _check_layer(run, ref, tag):
    from gpu_helpers import bf16_excess, bf16_to_f64
    cfg = run.cfg
    y = bf16_to_f64(run.t["y_out"]).reshape(cfg.m, cfg.hidden)
    r2 = run.t["r2_out"].cpu().numpy().astype(np.float64).reshape(cfg.m, cfg.hidden)
    assert bf16_excess(y, ref["y_pre"], 2e-2) <= 0 and np.max(np.abs(r2 - ref["r2"])) <= 2e-2, tag


def _expect(run_fn, status, text):
    import persistent_megakernel_amd as mk
    with pytest.raises(mk.MkError) as ei:
        run_fn()
    assert ei.value.status == status and text in str(ei.value), str(ei.value)


@pytest.mark.parametrize("case", [0, 1])
def test_bad_block_table_entry_is_reported(case):
    import persistent_megakernel_amd as mk
    from gpu_helpers import QwenRun
    cfg, ctx = _qwen_cases()[case]
    inp = make_inputs(cfg, seed=5)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    ref = model.run_qwen3_layer(cfg, inp)
    run = QwenRun(cfg, inp, ctx=ctx)
    good = run.t["block_table"].clone()
    bad = good.clone()
    bad[0, 1] = 1_000_000  # a page far beyond the pool, inside the first request's context
    for mode in ("mk", "graph"):
        _say(f"case: bad block table {cfg.name} M={cfg.m} {mode}")
        run.t["block_table"].copy_(bad)
        _expect(lambda: run.run(mode), mk.MK_ERR_INVALID, "block table entry 1000000")
        run.t["block_table"].copy_(good)
        run.run(mode)
        _check_layer(run, ref, f"{mode} after a bad table")


def test_bad_block_table_entry_indexer():
    import persistent_megakernel_amd as mk
    from gpu_helpers import IndexerRun
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, context=300)
    inp = make_inputs(cfg, seed=11)
    inp["context_lens"] = np.array([300, 133], dtype=np.int32)
    ref = model.run_indexer_front(cfg, inp)
    run = IndexerRun(cfg, inp)
    good = run.t["block_table"].clone()
    bad = good.clone()
    bad[0, 1] = -7  # negative: outside the pool as an unsigned page number too
    for mode in ("mk", "graph"):
        _say(f"case: bad block table indexer {mode}")
        run.t["block_table"].copy_(bad)
        _expect(lambda: run.run(mode), mk.MK_ERR_INVALID, "block table entry -7")
        run.t["block_table"].copy_(good)
        run.t["score_out"].fill_(float("nan"))
        run.run(mode)
        score = run.t["score_out"].cpu().numpy().astype(np.float64).reshape(cfg.m, run.smax)
        for m in range(cfg.m):
            c = int(inp["context_lens"][m // cfg.tokens_per_request])
            fin = np.isfinite(ref["score_pre"][m, :c])
            assert np.max(np.abs(score[m, :c][fin] - ref["score_pre"][m, :c][fin])) <= 6e-2, mode


def test_watchdog_expiry_aborts_the_run():
    import persistent_megakernel_amd as mk
    from gpu_helpers import QwenRun
    for cfg, ctx in _qwen_cases():
        inp = make_inputs(cfg, seed=6)
        inp["context_lens"] = np.array(ctx, dtype=np.int32)
        ref = model.run_qwen3_layer(cfg, inp)
        _say(f"case: short watchdog {cfg.name} M={cfg.m}")
        run = QwenRun(cfg, inp, ctx=ctx, flags=mk.MK_FLAG_DEBUG_SHORT_WATCHDOG)
        _expect(lambda: run.run("mk"), mk.MK_ERR_TIMEOUT, "watchdog")
        normal = QwenRun(cfg, inp, ctx=ctx)
        normal.t = run.t  # the same tensors, which the aborted run left half written
        normal.tensors = run.tensors
        normal.run("mk")
        _check_layer(normal, ref, "after an aborted run")
