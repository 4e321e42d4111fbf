"""mk_run_layer_noalloc (the entry point for callers that cannot allocate) against mk_run_layer, through
the C ABI: each no-allocation run must reproduce the existing entry point's outputs bit for bit (the
same kernels on the same inputs; the workspace only moves into the library's static scratch).  Calls
follow one another on one stream with different plans, the later ones smaller, so the scratch is
re-cleared and its pointer table rewritten between them, and one plan is called twice in a row (the
scratch then keeps its table)."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _qwen_outputs(run, noalloc):
    import persistent_megakernel_amd as mk
    run.t["y_out"].zero_()
    run.t["r2_out"].zero_()
    t = dict(run.t)
    if noalloc:
        t["workspace"] = torch.zeros(0, dtype=torch.uint8, device="cuda")  # ignored: any address will do
        ptrs = mk.qwen3_pointers(t, run.step)
        ptrs.ptr[mk.QWEN3_TENSORS.index("workspace")] = 0
        run.plan.run_noalloc(ptrs)
    else:
        run.plan.run(run.tensors)
    run.plan.sync()
    torch.cuda.synchronize()
    out = {"y": run.t["y_out"].clone(), "r2": run.t["r2_out"].clone()}
    if run.step:
        out["logits"] = run.t["logits_out"].clone()
        out["token"] = run.t["token_out"].clone()
    return out


def _indexer_outputs(run, noalloc):
    import persistent_megakernel_amd as mk
    run.t["score_out"].fill_(float("nan"))
    if noalloc:
        ptrs = mk.indexer_pointers(run.t)
        ptrs.ptr[mk.INDEXER_TENSORS.index("workspace")] = 0
        run.plan.run_noalloc(ptrs)
    else:
        run.plan.run(run.tensors)
    run.plan.sync()
    torch.cuda.synchronize()
    return {"score": torch.nan_to_num(run.t["score_out"].clone())}


def _same(a, b, tag):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{tag}: {k} differs from mk_run_layer's"


def test_noalloc_matches_run_layer_over_consecutive_calls():
    from gpu_helpers import IndexerRun, QwenRun
    # 1: a 16-row FP8 layer (the larger scratch use)
    ctx = [37, 300, 513, 64, 200]
    big = dataclasses.replace(get_config("qwen3_8b_layer_fp8"), hidden=1024, inter=2048, n_q_heads=8, n_kv_heads=2,
                              n_requests=len(ctx), context=max(ctx), page_size=16)
    inp = make_inputs(big, seed=3)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    run_big = QwenRun(big, inp, ctx=ctx)
    _say(f"case: noalloc 1: multi-row FP8 layer, workspace {run_big.plan.workspace_bytes()} B")
    want_big = _qwen_outputs(run_big, noalloc=False)
    _same(_qwen_outputs(run_big, noalloc=True), want_big, "multi-row FP8 layer")
    # 2: a smaller single-token layer, twice in a row (the second keeps the scratch's table)
    small = dataclasses.replace(get_config("qwen3_0p6b_layer"), context=300)
    inp_s = make_inputs(small, seed=1)
    inp_s["context_lens"] = np.array([300], dtype=np.int32)
    run_small = QwenRun(small, inp_s, ctx=[300])
    assert run_small.plan.workspace_bytes() < run_big.plan.workspace_bytes()
    _say(f"case: noalloc 2: single-token layer, workspace {run_small.plan.workspace_bytes()} B, twice")
    want_small = _qwen_outputs(run_small, noalloc=False)
    _same(_qwen_outputs(run_small, noalloc=True), want_small, "single-token layer")
    _same(_qwen_outputs(run_small, noalloc=True), want_small, "single-token layer, second call")
    # 3: the indexer front (another op family), then the first plan again
    ic = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, context=300)
    inp_i = make_inputs(ic, seed=11)
    inp_i["context_lens"] = np.array([300, 133], dtype=np.int32)
    run_i = IndexerRun(ic, inp_i)
    _say("case: noalloc 3: indexer front")
    want_i = _indexer_outputs(run_i, noalloc=False)
    _same(_indexer_outputs(run_i, noalloc=True), want_i, "indexer front")
    _say("case: noalloc 4: the multi-row FP8 layer again")
    _same(_qwen_outputs(run_big, noalloc=True), want_big, "multi-row FP8 layer, again")


def test_noalloc_full_step():
    """The 28-layer step (the headline workload) through the no-allocation entry point."""
    from gpu_helpers import QwenRun
    cfg = get_config("qwen3_0p6b_step")
    inp = make_inputs(cfg, seed=0)
    run = QwenRun(cfg, inp)
    _say("case: noalloc full step")
    want = _qwen_outputs(run, noalloc=False)
    _same(_qwen_outputs(run, noalloc=True), want, "full step")
