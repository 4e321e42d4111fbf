"""The C-ABI library loads and exports every entry point include/mk.h declares (no GPU calls)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_header_symbols():
    import persistent_megakernel_amd as mk
    header = open(os.path.join(ROOT, "include", "mk.h")).read()
    names = set(re.findall(r"^\s*(?:mk_status|const char\*|void)\s+(mk_\w+)\s*\(", header, re.M))
    assert {"mk_build_queue", "mk_run_layer", "mk_run_graph_baseline"} <= names
    lib = ctypes.CDLL(mk.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n


def test_host_only_plan_rejects_runs():
    import persistent_megakernel_amd as mk
    from workloads import get_config
    plan = mk.Plan(get_config("qwen3_0p6b_layer"), num_workers=16)
    t = mk.Plan.tensors([256] * 17)
    try:
        plan.run(t, stream=0)
        raised = False
    except mk.MkError as e:
        raised = e.status == mk.MK_ERR_INVALID
    assert raised
    plan.close()


def test_invalid_shapes_rejected():
    import dataclasses
    import persistent_megakernel_amd as mk
    from workloads import get_config
    bad = dataclasses.replace(get_config("qwen3_0p6b_layer"), n_q_heads=15)
    try:
        mk.Plan(bad, num_workers=8)
        ok = False
    except mk.MkError as e:
        ok = e.status == mk.MK_ERR_INVALID
    assert ok


def test_noalloc_run_rejects_a_workspace_beyond_the_scratch():
    """mk_run_layer_noalloc refuses, before anything else, a plan whose workspace and pointer table
    exceed the static scratch (here a 16-request layer at context 16384: 57.6 MiB > 40 MiB)."""
    import dataclasses
    import persistent_megakernel_amd as mk
    from workloads import get_config
    cfg = dataclasses.replace(get_config("qwen3_8b_layer"), context=16384)
    plan = mk.Plan(cfg, num_workers=256)
    assert plan.workspace_bytes() > mk.MK_SCRATCH_MAX_BYTES
    try:
        plan.run_noalloc(mk.Plan.tensors([256] * 17), stream=0)
        status = None
    except mk.MkError as e:
        status, msg = e.status, str(e)
    assert status == mk.MK_ERR_INVALID and "exceed the no-allocation scratch" in msg
    plan.close()
