"""Page-table indexing, bit-exact: the physical cache slot of every K / V row and indexer key a run
gathers through the block table (MK_FLAG_DEBUG_GATHER, mk_read_gather) against the oracle's page walk
(``oracle.ops.token_slots``: slot = bt[r][t // P] * P + t % P), through the C ABI, megakernel and graph
baseline, with randomly permuted page tables and ragged contexts.

What a record holds (mk.h): for the decode layers, per (layer, request, kv head) and for K and V
separately, the slot fetched for every token t < ctx - 1 (the new token's row is the run's own); the
last 4-row block of a request's last split re-fetches its first row for rows past the context, so the
entries from ctx - 1 to the end of that block hold the block's first slot; every other entry is -1.
For the indexer front, per request, the slot of every key t < ctx - T written before the run; -1
elsewhere."""
import dataclasses
import sys

import numpy as np
import pytest

from oracle import ops
from workloads import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _expected_attention(cfg, inp):
    """[layers][R][Hkv][2][max_pages * P] from the oracle's page walk."""
    P, tokens = cfg.page_size, cfg.pages_per_request * cfg.page_size
    exp = np.full((cfg.num_layers, cfg.n_requests, cfg.n_kv_heads, 2, tokens), -1, dtype=np.int64)
    for r in range(cfg.n_requests):
        ctx = int(inp["context_lens"][r])
        walk = ops.token_slots(inp["block_table"][r], tokens, P)
        n = ctx - 1
        exp[:, r, :, :, :n] = walk[:n]
        if n > 0 and n % 4:
            start = (n - 1) // 4 * 4  # the last gathered block: rows past the context re-fetch its first row
            exp[:, r, :, :, n:start + 4] = walk[start]
    return exp


def _check_attention(run, inp, tag):
    got = run.plan.read_gather().astype(np.int64)
    exp = _expected_attention(run.cfg, inp)
    bad = np.argwhere(got != exp)
    assert bad.size == 0, f"{tag}: {len(bad)} gather entries differ, first at {tuple(bad[0])}: " \
                          f"{got[tuple(bad[0])]} != {exp[tuple(bad[0])]}"
    _say(f"  {tag}: {int(np.sum(exp >= 0))} gathered slots bit-exact")


def _qwen_case(cfg, ctx, W, seed, modes=(("mk", False), ("graph", False))):
    import persistent_megakernel_amd as mk
    from gpu_helpers import QwenRun
    inp = make_inputs(cfg, seed=seed)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    run = QwenRun(cfg, inp, num_workers=W, flags=mk.MK_FLAG_DEBUG_GATHER, ctx=ctx)
    for mode, ms in modes:
        _say(f"case: gather {cfg.name} layers={cfg.num_layers} R={cfg.n_requests} ctx={ctx} W={W} {mode} ms={ms}")
        run.run(mode, ms)
        _check_attention(run, inp, f"{mode}/{ms}")


@pytest.mark.parametrize("W,ctx", [(0, 512), (13, 203), (7, 2), (64, 66)])
def test_gather_single_token_layer_random_pages(W, ctx):
    cfg = dataclasses.replace(get_config("qwen3_0p6b_layer"), random_pages=True, context=ctx)
    _qwen_case(cfg, [ctx], W, seed=W + ctx)


def test_gather_single_token_step_random_pages():
    cfg = dataclasses.replace(get_config("qwen3_0p6b_step"), num_layers=3, vocab=3000, context=300, random_pages=True)
    _qwen_case(cfg, [300], 0, seed=4, modes=(("mk", False), ("graph", True)))


def test_gather_full_step():
    cfg = get_config("qwen3_0p6b_step")
    _qwen_case(cfg, [cfg.context], 0, seed=0, modes=(("mk", False),))


@pytest.mark.parametrize("R", [6, 35])
@pytest.mark.parametrize("fp8", [False, True])
def test_gather_multi_row_reduced_random_pages(fp8, R):
    ctx = [1, 37, 300, 513, 64, 6] if R == 6 else [int(c) for c in np.random.default_rng(35).integers(1, 514, R)]
    base = get_config("qwen3_8b_layer_fp8" if fp8 else "qwen3_8b_layer")
    cfg = dataclasses.replace(base, hidden=1024, inter=2048 if fp8 else 1536, n_q_heads=8, n_kv_heads=2,
                              n_requests=len(ctx), context=max(ctx), page_size=16, random_pages=True)
    _qwen_case(cfg, ctx, 37, seed=6, modes=(("mk", False), ("graph", False), ("graph", True)))


@pytest.mark.timeout(600)
def test_gather_multi_row_full_size_random_pages():
    cfg = get_config("qwen3_8b_layer_fp8")  # 16 requests x 8192 tokens over a permuted 2048-page pool
    _qwen_case(cfg, [cfg.context] * cfg.n_requests, 0, seed=0, modes=(("mk", False),))


def _indexer_case(cfg, ctx, W, seed):
    import persistent_megakernel_amd as mk
    from gpu_helpers import IndexerRun
    inp = make_inputs(cfg, seed=seed)
    inp["context_lens"] = np.array(ctx, dtype=np.int32)
    run = IndexerRun(cfg, inp, num_workers=W, flags=mk.MK_FLAG_DEBUG_GATHER)
    T, P = cfg.tokens_per_request, cfg.page_size
    tokens = cfg.pages_per_request * P
    exp = np.full((cfg.n_requests, tokens), -1, dtype=np.int64)
    for r in range(cfg.n_requests):
        n = int(ctx[r]) - T
        exp[r, :n] = ops.token_slots(inp["block_table"][r], tokens, P)[:n]
    for mode, ms in (("mk", False), ("graph", False)):
        _say(f"case: gather indexer R={cfg.n_requests} T={T} ctx={ctx} W={W} {mode}")
        run.run(mode, ms)
        got = run.plan.read_gather().astype(np.int64)
        assert np.array_equal(got, exp), f"{mode}: {int(np.sum(got != exp))} key slots differ"


@pytest.mark.parametrize("R,T,ctx,W", [(2, 8, [300, 133], 0), (3, 5, [64, 196, 5], 37)])
def test_gather_indexer_reduced(R, T, ctx, W):
    cfg = dataclasses.replace(get_config("indexer_front"), hidden=1024, idx_q_rank=512, n_requests=R,
                              tokens_per_request=T, context=max(ctx))
    _indexer_case(cfg, ctx, W, seed=11)


def test_gather_indexer_full_size():
    cfg = get_config("indexer_front")
    _indexer_case(cfg, [cfg.context] * cfg.n_requests, 0, seed=0)
