"""The C++ planner (through the C ABI, host-only) against the oracle queue builder:
bit-exact queues, thresholds and counts."""
import dataclasses

import numpy as np
import pytest

from oracle import queue as oq
from workloads import get_config


def _both(cfg, W, ctx=None):
    import persistent_megakernel_amd as mk
    plan = mk.Plan(cfg, context_lens=ctx, num_workers=W)
    ref = oq.build_queue(cfg, W, ctx)
    return plan, ref


@pytest.mark.parametrize("name", ["qwen3_0p6b_layer", "qwen3_0p6b_step", "qwen3_8b_layer", "qwen3_8b_layer_fp8",
                                  "indexer_front"])
@pytest.mark.parametrize("W", [1, 7, 148, 256])
def test_queue_bit_exact(name, W):
    cfg = get_config(name)
    plan, ref = _both(cfg, W)
    q = plan.queue()
    assert q.shape == ref["queue"].shape
    assert np.array_equal(q, ref["queue"])
    assert np.array_equal(plan.thresholds(), ref["thresholds"])
    info = plan.info()
    assert info["n_tasks"] == ref["n_tasks"] and info["n_ops"] == ref["n_ops"] and info["n_arrivals"] == ref["n_arrivals"]
    plan.close()


@pytest.mark.parametrize("ctx", [[1], [5], [37], [511], [513], [2048]])
def test_ragged_contexts_bit_exact(ctx):
    cfg = dataclasses.replace(get_config("qwen3_0p6b_layer"), context=max(ctx[0], 16))
    for W in (5, 64, 256):
        plan, ref = _both(cfg, W, ctx)
        assert np.array_equal(plan.queue(), ref["queue"])
        assert np.array_equal(plan.thresholds(), ref["thresholds"])
        oq.check_invariants(ref)
        plan.close()


def test_small_shapes_bit_exact():
    cfg = dataclasses.replace(get_config("qwen3_0p6b_step"), hidden=256, inter=384, n_q_heads=4, n_kv_heads=2,
                              num_layers=3, vocab=1000, context=40)
    for W in (3, 16, 256):
        plan, ref = _both(cfg, W)
        assert np.array_equal(plan.queue(), ref["queue"])
        plan.close()


def test_indexer_ragged_bit_exact():
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, idx_heads=64,
                              n_requests=2, tokens_per_request=3, context=300)
    for ctx in ([300, 3], [129, 256]):
        for W in (5, 64, 256):
            plan, ref = _both(cfg, W, ctx)
            assert np.array_equal(plan.queue(), ref["queue"])
            assert np.array_equal(plan.thresholds(), ref["thresholds"])
            oq.check_invariants(ref)
            plan.close()
