"""Python binding of the decode-layer megakernel C ABI (include/mk.h).

Argument marshalling only: every step of the path runs in the HIP library
``libmk.so`` built next to this file.  Importing this package fails loudly when the
library has not been built -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

try:  # PyTorch first: libmk.so then binds to the HIP / HSA runtime PyTorch loaded (one runtime per
    import torch  # noqa: F401  process); loaded the other way round, PyTorch finds no GPU
except ImportError:  # pragma: no cover - the library itself does not need PyTorch
    pass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmk.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python persistent_megakernel_amd/build.py` "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

MK_OK, MK_ERR_INVALID, MK_ERR_UNSUPPORTED, MK_ERR_HIP, MK_ERR_NOMEM, MK_ERR_TIMEOUT = 0, -1, -2, -3, -4, -5
MK_QWEN3_LAYER, MK_QWEN3_STEP, MK_INDEXER_FRONT = 0, 1, 2
MK_FLAG_NO_PREFETCH, MK_FLAG_NOOP_ONLY, MK_FLAG_TRACE, MK_FLAG_DEBUG_GATHER, MK_FLAG_DEBUG_SHORT_WATCHDOG = 1, 2, 4, 8, 16
MK_MAX_TENSORS = 32
MK_TILE_PARAMS = 8
MK_TP_ROWS_QKV, MK_TP_ROWS_O, MK_TP_ROWS_GATEUP, MK_TP_ROWS_DOWN, MK_TP_ROWS_LMHEAD, MK_TP_SPLIT_TOKENS = 0, 1, 2, 3, 4, 5
MK_SCRATCH_MAX_BYTES = 40 << 20
QWEN3_TENSORS = ["w_qkv", "w_o", "w_gu", "w_down", "g_attn", "g_mlp", "g_q", "g_k", "k_cache", "v_cache",
                 "block_table", "context_lens", "x", "r_in", "y_out", "r2_out", "workspace",
                 "g_final", "w_lm", "logits_out", "token_out",
                 "s_qkv", "s_o", "s_gu", "s_down"]
INDEXER_TENSORS = ["w_qa", "s_qa", "w_w", "s_w", "w_k", "s_k", "w_qi", "s_qi", "g_norm", "g_qa", "key_cache",
                   "key_scale", "block_table", "context_lens", "x", "r_in", "score_out", "workspace", "topk_out",
                   "w_qb", "s_qb", "w_uk", "qlat_out"]
_WORKLOADS = {"qwen3_layer": MK_QWEN3_LAYER, "qwen3_step": MK_QWEN3_STEP, "indexer_front": MK_INDEXER_FRONT}


class MkConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "workload", "weight_fp8", "act_fp8", "hidden", "inter", "n_q_heads", "n_kv_heads", "head_dim",
        "num_layers", "vocab", "n_requests", "tokens_per_request", "page_size", "max_pages_per_req",
        "num_phys_pages", "idx_q_rank", "idx_heads", "idx_head_dim")] + [
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float), ("num_workers", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("topk", ctypes.c_int32), ("mla_heads", ctypes.c_int32),
        ("rotary_dim", ctypes.c_int32), ("tile_params", ctypes.c_int32 * MK_TILE_PARAMS)]


class MkTensors(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_uint64 * MK_MAX_TENSORS), ("n", ctypes.c_int32)]


_P = ctypes.c_void_p
_lib.mk_last_error.restype = ctypes.c_char_p
_lib.mk_build_queue.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(_P)]
_lib.mk_plan_queue.argtypes = [_P, ctypes.POINTER(ctypes.POINTER(ctypes.c_uint32)), ctypes.POINTER(ctypes.c_int32),
                               ctypes.POINTER(ctypes.c_int32)]
_lib.mk_plan_events.argtypes = [_P, ctypes.POINTER(ctypes.POINTER(ctypes.c_uint32)), ctypes.POINTER(ctypes.c_int32)]
_lib.mk_plan_info.argtypes = [_P] + [ctypes.POINTER(ctypes.c_int32)] * 3
_lib.mk_plan_workspace_bytes.argtypes = [_P, ctypes.POINTER(ctypes.c_size_t)]
_lib.mk_plan_workspace_region.argtypes = [_P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
_lib.mk_run_layer.argtypes = [_P, ctypes.POINTER(MkTensors), _P]
_lib.mk_run_layer_noalloc.argtypes = [_P, ctypes.POINTER(MkTensors), _P]
_lib.mk_run_graph_baseline.argtypes = [_P, ctypes.POINTER(MkTensors), ctypes.c_int32, _P]
_lib.mk_sync.argtypes = [_P, _P]
_lib.mk_read_trace.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32), ctypes.c_size_t]
_lib.mk_read_gather.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), ctypes.c_size_t]
_lib.mk_plan_destroy.argtypes = [_P]
_lib.mk_plan_destroy.restype = None
for _f in ("mk_build_queue", "mk_plan_queue", "mk_plan_events", "mk_plan_info", "mk_plan_workspace_bytes",
           "mk_plan_workspace_region", "mk_run_layer", "mk_run_layer_noalloc", "mk_run_graph_baseline", "mk_sync",
           "mk_read_trace", "mk_read_gather"):
    getattr(_lib, _f).restype = ctypes.c_int


class MkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {_lib.mk_last_error().decode()}")


def _check(status: int, where: str) -> None:
    if status != MK_OK:
        raise MkError(status, where)


def make_config(cfg, num_workers: int = 0, flags: int = 0) -> MkConfig:
    """mk_config from a workload description (any object with the workload attributes)."""
    c = MkConfig()
    c.workload = _WORKLOADS[cfg.workload]
    c.weight_fp8, c.act_fp8 = int(cfg.weight_fp8), int(cfg.act_fp8)
    for n in ("hidden", "inter", "n_q_heads", "n_kv_heads", "head_dim", "num_layers", "vocab", "n_requests",
              "tokens_per_request", "page_size", "idx_q_rank", "idx_heads", "idx_head_dim"):
        setattr(c, n, int(getattr(cfg, n)))
    c.max_pages_per_req = int(cfg.pages_per_request)
    c.num_phys_pages = int(cfg.num_phys_pages)
    c.rms_eps, c.rope_theta = float(cfg.rms_eps), float(cfg.rope_theta)
    c.num_workers, c.flags = int(num_workers), int(flags)
    c.topk = int(getattr(cfg, "topk", 0))
    c.mla_heads = int(getattr(cfg, "mla_heads", 0))
    c.rotary_dim = int(getattr(cfg, "rotary_dim", 0))
    tp = tuple(getattr(cfg, "tile_params", ()) or ())
    if len(tp) > MK_TILE_PARAMS:
        raise ValueError(f"tile_params holds at most {MK_TILE_PARAMS} entries")
    for i, v in enumerate(tp):
        c.tile_params[i] = int(v)
    return c


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


class Plan:
    """Owns an mk_plan: mk_build_queue on construction, mk_plan_destroy on close."""

    def __init__(self, cfg, context_lens: Optional[Sequence[int]] = None, num_workers: int = 0, flags: int = 0):
        self.cfg = cfg
        ctx = list(context_lens) if context_lens is not None else [cfg.context] * cfg.n_requests
        self._ctx = (ctypes.c_int32 * len(ctx))(*ctx)
        self._c = make_config(cfg, num_workers, flags)
        h = _P()
        _check(_lib.mk_build_queue(ctypes.byref(self._c), self._ctx, ctypes.byref(h)), "mk_build_queue")
        self._h = h
        self._keep = []

    def close(self) -> None:
        if getattr(self, "_h", None) and _lib is not None:
            _lib.mk_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def queue(self) -> np.ndarray:
        q = ctypes.POINTER(ctypes.c_uint32)()
        W, L = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.mk_plan_queue(self._h, ctypes.byref(q), ctypes.byref(W), ctypes.byref(L)), "mk_plan_queue")
        return np.ctypeslib.as_array(q, shape=(W.value, L.value, 32)).copy()

    def thresholds(self) -> np.ndarray:
        t = ctypes.POINTER(ctypes.c_uint32)()
        n = ctypes.c_int32()
        _check(_lib.mk_plan_events(self._h, ctypes.byref(t), ctypes.byref(n)), "mk_plan_events")
        return np.ctypeslib.as_array(t, shape=(n.value,)).copy() if n.value else np.zeros(0, np.uint32)

    def info(self) -> Dict[str, int]:
        a, b, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.mk_plan_info(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "mk_plan_info")
        return {"n_tasks": a.value, "n_ops": b.value, "n_arrivals": c.value}

    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(_lib.mk_plan_workspace_bytes(self._h, ctypes.byref(n)), "mk_plan_workspace_bytes")
        return n.value

    def region(self, name: str):
        off, n = ctypes.c_size_t(), ctypes.c_size_t()
        _check(_lib.mk_plan_workspace_region(self._h, name.encode(), ctypes.byref(off), ctypes.byref(n)),
               "mk_plan_workspace_region")
        return off.value, n.value

    @staticmethod
    def tensors(ptrs: Sequence[int]) -> MkTensors:
        t = MkTensors()
        for i, p in enumerate(ptrs):
            t.ptr[i] = int(p)
        t.n = len(ptrs)
        return t

    def run(self, tensors: MkTensors, stream=None) -> None:
        _check(_lib.mk_run_layer(self._h, ctypes.byref(tensors), _P(_stream_handle(stream))), "mk_run_layer")

    def run_noalloc(self, tensors: MkTensors, stream=None) -> None:
        """mk_run_layer_noalloc: the same run with the library's static device scratch as workspace."""
        _check(_lib.mk_run_layer_noalloc(self._h, ctypes.byref(tensors), _P(_stream_handle(stream))),
               "mk_run_layer_noalloc")

    def run_graph(self, tensors: MkTensors, multistream: bool = False, stream=None) -> None:
        _check(_lib.mk_run_graph_baseline(self._h, ctypes.byref(tensors), int(bool(multistream)),
                                          _P(_stream_handle(stream))), "mk_run_graph_baseline")

    def sync(self, stream=None) -> None:
        _check(_lib.mk_sync(self._h, _P(_stream_handle(stream))), "mk_sync")

    def read_trace(self) -> np.ndarray:
        q = self.queue()
        W, L = q.shape[:2]
        out = np.zeros((W, L, 16), dtype=np.uint32)
        _check(_lib.mk_read_trace(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), out.size),
               "mk_read_trace")
        return out


    def read_gather(self) -> np.ndarray:
        """The gather record of the last run (MK_FLAG_DEBUG_GATHER), shaped as mk_read_gather lays it out."""
        c = self.cfg
        tokens = int(c.pages_per_request) * int(c.page_size)
        if c.workload == "indexer_front":
            shape = (c.n_requests, tokens)
        else:
            shape = (c.num_layers, c.n_requests, c.n_kv_heads, 2, tokens)
        out = np.zeros(shape, dtype=np.int32)
        _check(_lib.mk_read_gather(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), out.size),
               "mk_read_gather")
        return out


def qwen3_pointers(t: Dict[str, "object"], step: bool) -> MkTensors:
    """mk_tensors in the ABI order from a dict of device tensors (torch) keyed by QWEN3_TENSORS;
    entries a workload does not use (the step's tail for a layer, the FP8 scales for bf16) are 0."""
    fp8 = "s_qkv" in t
    last = len(QWEN3_TENSORS) if fp8 else QWEN3_TENSORS.index("token_out" if step else "workspace") + 1
    return Plan.tensors([t[n].data_ptr() if n in t else 0 for n in QWEN3_TENSORS[:last]])


def exported_symbols():
    return [n for n in dir(_lib) if n.startswith("mk_")]


def indexer_pointers(t: Dict[str, "object"]) -> MkTensors:
    """mk_tensors in the indexer front's ABI order from a dict of device tensors keyed by INDEXER_TENSORS
    ("topk_out" only for plans with a top-k, the main-MLA tensors only with that half: 0 when absent)."""
    return Plan.tensors([t[n].data_ptr() if n in t else 0 for n in INDEXER_TENSORS])
