"""The per-instruction trace of an MK_FLAG_TRACE megakernel run (mk_read_trace), on the GPU.

Checked on the three kernel instances (single-token step, multi-row layer with loader waves,
indexer front without them):
- a traced run gives the same outputs, bit for bit, as an untraced one;
- every live instruction is stamped, in order: seen <= inputs ready <= after the compute-start
  barrier <= after the compute-end barrier <= done, and a worker's instruction is done before it
  sees its next one (stamps are the low 32 bits of the 100 MHz clock: compared as int32
  differences);
- instances without loader waves stamp when the compute waves issued an instruction's lease
  (word 9), before that instruction's compute-start barrier;
- the Perfetto export gives four slices per live instruction (every stamp pair is ordered);
- on the single-token step the leases of a layer's first instructions are issued while the
  previous layer still runs on that worker (the queue-order lookahead crosses layer boundaries);
  the share is reported, and must be a majority.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import persistent_megakernel_amd as mk
from persistent_megakernel_amd import trace as tx
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _d(a, b):
    """b - a for 32-bit clock stamps (int64 arrays), as a signed difference."""
    return ((b - a + (1 << 31)) % (1 << 32)) - (1 << 31)


def _check_order(q, tr, tag):
    live = q[:, :, 0] != 0
    for a, b in ((0, 1), (1, 3), (3, 4), (4, 7)):
        d = _d(tr[:, :, a], tr[:, :, b])[live]
        assert (d >= 0).all(), f"{tag}: word {a} after word {b} in {(d < 0).sum()} instructions"
    for w in range(q.shape[0]):
        idx = np.flatnonzero(live[w])
        if len(idx) > 1:
            assert (_d(tr[w, idx[:-1], 7], tr[w, idx[1:], 0]) >= 0).all(), f"{tag}: worker {w} out of order"
    ev = tx.events(q, tr)
    assert sum(e["ph"] == "X" for e in ev) == 4 * int(live.sum()), f"{tag}: export lost slices"
    return live


def _run_pair(make_run, cfg, inp, outs):
    plain = make_run(cfg, inp, 0)
    plain.run("mk")
    ref = [plain.t[k].clone() for k in outs]
    traced = make_run(cfg, inp, mk.MK_FLAG_TRACE)
    traced.run("mk")
    for k, r in zip(outs, ref):
        assert torch.equal(torch.nan_to_num(traced.t[k]), torch.nan_to_num(r)), f"trace changed {k}"
    return traced.plan.queue(), traced.plan.read_trace().astype(np.int64)


def test_trace_single_token_step():
    from gpu_helpers import QwenRun
    cfg = dataclasses.replace(get_config("qwen3_0p6b_step"), num_layers=3, vocab=3000, context=300)
    _say("case: trace, single-token step, 3 layers")
    inp = make_inputs(cfg, seed=5)
    q, tr = _run_pair(lambda c, i, f: QwenRun(c, i, flags=f), cfg, inp, ["logits_out", "token_out"])
    live = _check_order(q, tr, "step")
    # every instruction that streams weights or KV has a lease stamp before its compute starts
    leased = live & np.isin(q[:, :, 0], [1, 2, 3, 4, 5, 6])
    assert (tr[:, :, 9][leased] != 0).all()
    assert (_d(tr[:, :, 9], tr[:, :, 3])[leased] >= 0).all()
    # the first instruction of layer l + 1 on a worker: leased before its layer-l work ended
    layer = q[:, :, 20].astype(np.int64)
    ahead = []
    for w in range(q.shape[0]):
        idx = np.flatnonzero(live[w] & (q[w, :, 0] != 6))
        for a, b in zip(idx[:-1], idx[1:]):
            if layer[w, b] == layer[w, a] + 1:
                ahead.append(_d(tr[w, b, 9], tr[w, a, 7]) > 0)
    share = float(np.mean(ahead))
    _say(f"  {len(ahead)} layer boundaries, next layer's lease issued before the previous layer ended: {share:.3f}")
    assert len(ahead) and share > 0.5


def test_trace_multi_row_layer():
    from gpu_helpers import QwenRun
    ctx = [1, 37, 300, 64, 513]
    cfg = dataclasses.replace(get_config("qwen3_8b_layer"), hidden=1024, inter=1536, n_q_heads=8, n_kv_heads=2,
                              n_requests=len(ctx), context=max(ctx), page_size=16)
    _say("case: trace, multi-row layer (loader waves)")
    inp = make_inputs(cfg, seed=6)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    q, tr = _run_pair(lambda c, i, f: QwenRun(c, i, flags=f, ctx=ctx), cfg, inp, ["y_out", "r2_out"])
    live = _check_order(q, tr, "multi-row")
    # events met (word 14) between seeing the instruction and its inputs being ready
    assert (_d(tr[:, :, 0], tr[:, :, 14])[live] >= 0).all() and (_d(tr[:, :, 14], tr[:, :, 1])[live] >= 0).all()


def test_trace_indexer_front():
    from gpu_helpers import IndexerRun
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, n_requests=2,
                              tokens_per_request=8, context=300)
    _say("case: trace, indexer front (no loader waves)")
    inp = make_inputs(cfg, seed=7)
    inp["context_lens"] = np.array([300, 133], dtype=np.int32)
    q, tr = _run_pair(lambda c, i, f: IndexerRun(c, i, flags=f), cfg, inp, ["score_out"])
    live = _check_order(q, tr, "indexer")
    stamped = live & (tr[:, :, 9] != 0)
    assert stamped.any() and (_d(tr[:, :, 9], tr[:, :, 3])[stamped] >= 0).all()
