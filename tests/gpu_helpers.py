"""Device-side setup shared by the GPU tests: upload seeded inputs, allocate outputs and the
workspace, build the mk_tensors block."""
import numpy as np
import torch

import persistent_megakernel_amd as mk


def to_device(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |v| (8 significant bits; the smallest normal spacing below)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def bf16_excess(gpu: np.ndarray, pre: np.ndarray, tol: float) -> float:
    """How far a bf16 output is from being the bf16 rounding of a value within tol of the
    oracle's value before rounding: max(|gpu - pre| - tol - half ulp), <= 0 when it is."""
    allow = tol + np.maximum(bf16_half_ulp(gpu), bf16_half_ulp(pre))
    return float(np.max(np.abs(gpu - pre) - allow)) if gpu.size else 0.0


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    b = t.detach().cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


class QwenRun:
    """Inputs, outputs and workspace of one Qwen3 layer / step plan on cuda:0."""

    def __init__(self, cfg, inp, num_workers=0, flags=0, ctx=None):
        self.cfg = cfg
        self.step = cfg.workload == "qwen3_step"
        self.plan = mk.Plan(cfg, context_lens=ctx, num_workers=num_workers, flags=flags)
        M, H = cfg.m, cfg.hidden
        t = {k: to_device(v) for k, v in inp.items() if k in mk.QWEN3_TENSORS or k in ("x", "r_in")}
        t["y_out"] = torch.zeros(M * H, dtype=torch.int16, device="cuda")
        t["r2_out"] = torch.zeros(M * H, dtype=torch.float32, device="cuda")
        t["workspace"] = torch.zeros(self.plan.workspace_bytes() + 256, dtype=torch.uint8, device="cuda")
        if self.step:
            t["logits_out"] = torch.zeros(M * cfg.vocab, dtype=torch.float32, device="cuda")
            t["token_out"] = torch.full((M,), -1, dtype=torch.int32, device="cuda")
        self.t = t
        self.tensors = mk.qwen3_pointers(t, self.step)

    def region(self, name, dtype):
        off, n = self.plan.region(name)
        return self.t["workspace"][off:off + n].view(dtype)

    def records(self, name):
        """A workspace vector of tagged records: (payload words uint32, tags uint32)."""
        w = self.region(name, torch.int32).cpu().numpy().view(np.uint32)
        return w[0::2].copy(), w[1::2].copy()

    def payload_f32(self, name):
        return self.records(name)[0].view(np.float32).astype(np.float64)

    def payload_bf16(self, name):
        """bf16 pairs per record (low half first), as float64."""
        p = self.records(name)[0]
        pairs = np.stack([p & 0xFFFF, p >> 16], axis=1).reshape(-1).astype(np.uint32) << 16
        return pairs.view(np.float32).astype(np.float64)

    def run(self, mode="mk", multistream=False):
        if mode == "mk":
            self.plan.run(self.tensors)
        else:
            self.plan.run_graph(self.tensors, multistream=multistream)
        self.plan.sync()
        torch.cuda.synchronize()


class IndexerRun:
    """Inputs, score output and workspace of one indexer-front plan on cuda:0."""

    def __init__(self, cfg, inp, num_workers=0, flags=0):
        self.cfg = cfg
        ctx = [int(c) for c in inp["context_lens"]]
        self.plan = mk.Plan(cfg, context_lens=ctx, num_workers=num_workers, flags=flags)
        t = {k: to_device(v) for k, v in inp.items() if k in mk.INDEXER_TENSORS}
        self.smax = max(ctx)
        t["score_out"] = torch.full((cfg.m * self.smax,), float("nan"), dtype=torch.float32, device="cuda")
        t["workspace"] = torch.zeros(self.plan.workspace_bytes() + 256, dtype=torch.uint8, device="cuda")
        if getattr(cfg, "topk", 0):
            t["topk_out"] = torch.full((cfg.m * cfg.topk,), -7, dtype=torch.int32, device="cuda")
        if getattr(cfg, "mla_heads", 0):
            t["qlat_out"] = torch.full((cfg.m * cfg.mla_heads * 512,), -1, dtype=torch.int16, device="cuda")
        self.t = t
        self.tensors = mk.indexer_pointers(t)

    def region(self, name, dtype):
        off, n = self.plan.region(name)
        return self.t["workspace"][off:off + n].view(dtype)

    def run(self, mode="mk", multistream=False):
        if mode == "mk":
            self.plan.run(self.tensors)
        else:
            self.plan.run_graph(self.tensors, multistream=multistream)
        self.plan.sync()
        torch.cuda.synchronize()
