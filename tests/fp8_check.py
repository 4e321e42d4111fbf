"""Checks of the kernel's per-token FP8 (e4m3) decisions against the oracle's.

A code is an integer decided in floating point.  The oracle decides in float64 arithmetic
rounded to fp32 at the ratio value / scale; the kernel decides on fp32 values that reproduce the
oracle's only to within the error of its fp32 sums.  So the rule checked here is:

* the kernel's per-token scale equals the oracle's to SCALE_RTOL;
* wherever the oracle's ratio v lies farther than delta(v) = delta_rel |v| + delta_abs from
  the midpoint of the two e4m3 codes enclosing it, the kernel's code is the oracle's
  round-to-nearest-even code exactly (a truncating or round-toward-zero codec differs from it
  on about half of all elements, and fails);
* inside that ambiguity set (computed by the oracle from its own values) the kernel's code is
  one of the two enclosing codes, and the oracle continues the chain with the kernel's choice
  there -- and only there (``oracle.model._quant``);
* the ambiguity set is small: at most MAX_AMBIGUOUS of a point's elements.

delta per point, in code units (value / scale).  The bounds follow the fp32 error of what each
point's value goes through on the kernel side; the measured deviations of the kernel's exposed
fp32 values (o, m) from the oracle's are quoted for comparison:

* h1q, hq -- RMSNorm of inputs both sides hold bit for bit: an fp32 mean square over at most
  6144 terms summed in a tree (relative error <= (log2 n + 8) 2^-24, about 1.3e-6), one reciprocal
  square root and three roundings: relative 2^-16 leaves a margin of ten and more;
* oq -- attention output: the kernel carries the softmax weights as three bf16 parts (24
  significant bits) summed in fp32 over up to 8192 tokens: absolute 2^-8 code units (measured
  before the bf16 decisions below were resolved: largest deviation 3.1e-3, rms 2e-4 code units);
* h2q, mq, qaq, kq -- fp32 projection sums over <= 12288 products (per 128-block partials times
  the block scales), then RMSNorm, SiLU-mul or RoPE in fp32: relative 2^-14 plus absolute 2^-12
  code units (measured for m: largest deviation 8.9e-5, rms 4e-6).
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from oracle.numerics import bf16_admissible, e4m3_decode, e4m3_other_code

DELTA: Dict[str, Tuple[float, float]] = {
    "h1q": (2.0 ** -16, 2.0 ** -20), "hq": (2.0 ** -16, 2.0 ** -20),
    "oq": (2.0 ** -14, 2.0 ** -8),
    "h2q": (2.0 ** -14, 2.0 ** -12), "mq": (2.0 ** -14, 2.0 ** -12),
    "qaq": (2.0 ** -14, 2.0 ** -12), "kq": (2.0 ** -14, 2.0 ** -12),
}
SCALE_RTOL = 2e-6
MAX_AMBIGUOUS = 0.02

# bf16 decisions on the way to a quantisation point: q and k after QK-norm and RoPE, v as
# projected, each materialised in bf16 on both sides.  A value within fp32 error of a bf16
# midpoint may round either way (measured at 256 rows: one element in about 12,000 of k and v, and
# a q element taken the other way moved a token's attention output by 1e-4 of its largest element,
# fifty times SCALE_RTOL at oq).  The kernel's q (written to the workspace as it materialises it),
# k and v (the written cache rows) are checked like the codes: its value must be the bf16 rounding
# of some value within delta of the oracle's (the oracle's own round-to-nearest-even value wherever
# that admits only one), and the oracle continues with the kernel's value where several are
# admissible.  delta = delta_rel |x| + delta_abs rms(head).  The flip rate measured at 256 rows (one
# value in about 12,000 of k and v rounded the other way) puts the kernel's error near 2^-23 of a
# value: q, k (an RMSNorm over 128 dims and a rotation in fp32): 2^-18 relative and 2^-19 of the
# head's rms for the rotation's cancellation, which leaves elements near zero with several
# admissible values; v (an fp32 projection sum over the hidden size): 2^-17 and 2^-20.
BF16_DELTA: Dict[str, Tuple[float, float]] = {"q": (2.0 ** -18, 2.0 ** -19), "k": (2.0 ** -18, 2.0 ** -19),
                                              "v": (2.0 ** -17, 2.0 ** -20)}
MAX_AMBIGUOUS_BF16 = 0.04


class KernelTies:
    """The oracle's ``ties`` argument for one kernel run: at each quantisation point it checks
    the kernel's codes and scales (the rule above) and takes the kernel's choice inside the
    oracle's ambiguity set.  ``kernel``: {point: (codes [rows, K] uint8, scales [rows])}."""

    def __init__(self, kernel: Dict[str, Tuple[np.ndarray, np.ndarray]], delta=None,
                 bf16: Dict[str, np.ndarray] = None):
        self.kernel = kernel
        self._delta = dict(DELTA if delta is None else delta)
        self.bf16 = dict(bf16 or {})  # {"q" | "k" | "v": the kernel's bf16 values as float64}
        self.report: Dict[str, Dict[str, int]] = {}

    def has_bf16(self, key: str) -> bool:
        return key in self.bf16

    def bf16_delta(self, key: str, pre: np.ndarray) -> np.ndarray:
        rel, ab = BF16_DELTA[key]
        rms = np.sqrt(np.mean(np.square(pre), axis=-1, keepdims=True))
        return rel * np.abs(pre) + ab * rms

    def choose_bf16(self, key, pre, rne, ambiguous):
        kv = np.asarray(self.bf16[key], dtype=np.float64)
        assert kv.shape == rne.shape, f"{key}: shapes {kv.shape} {rne.shape}"
        differ = kv != rne
        outside = int(np.sum(differ & ~ambiguous))
        assert outside == 0, (f"{key}: {outside} of {rne.size} bf16 values differ from the oracle's "
                              f"round-to-nearest-even value where it admits no other")
        lo, hi = bf16_admissible(pre, self.bf16_delta(key, pre))
        bad = int(np.sum(differ & ((kv < lo) | (kv > hi))))
        assert bad == 0, f"{key}: {bad} values are not the rounding of any value within delta of the oracle's"
        n_amb = int(np.sum(ambiguous))
        self.report[key] = {"flipped": int(np.sum(differ)), "ambiguous": n_amb, "elements": int(rne.size)}
        assert n_amb <= MAX_AMBIGUOUS_BF16 * rne.size, f"{key}: ambiguity set {n_amb} of {rne.size} is too large"
        return np.where(differ, kv, rne)

    def delta(self, key: str) -> Tuple[float, float]:
        return self._delta[key]

    def choose(self, key, v, codes, s, ambiguous):
        kc, ks = self.kernel[key]
        kc = np.asarray(kc, dtype=np.uint8)
        ks = np.asarray(ks, dtype=np.float64)
        assert kc.shape == codes.shape and ks.shape == s.shape, f"{key}: shapes {kc.shape} {codes.shape}"
        dev = float(np.max(np.abs(ks / s - 1.0))) if s.size else 0.0
        assert dev <= SCALE_RTOL, f"{key}: per-token scale differs from the oracle's by {dev:.2e} (relative)"
        differ = e4m3_decode(kc) != e4m3_decode(codes)  # +0 and -0 are one value
        outside = int(np.sum(differ & ~ambiguous))
        assert outside == 0, (f"{key}: {outside} of {codes.size} codes differ from the oracle's round-to-nearest-even "
                              f"code away from any rounding midpoint")
        other = e4m3_other_code(v, codes)
        bad = int(np.sum(differ & (e4m3_decode(kc) != e4m3_decode(other))))
        assert bad == 0, f"{key}: {bad} ambiguous codes are neither of the two enclosing codes"
        n_amb = int(np.sum(ambiguous))
        self.report[key] = {"flipped": int(np.sum(differ)), "ambiguous": n_amb, "elements": int(codes.size)}
        assert n_amb <= MAX_AMBIGUOUS * codes.size, f"{key}: ambiguity set {n_amb} of {codes.size} is too large"
        return differ

    @property
    def any_flip(self) -> bool:
        return any(r["flipped"] for r in self.report.values())

    def summary(self) -> str:
        return "; ".join(f"{k}: {r['flipped']} taken of {r['ambiguous']} ambiguous / {r['elements']}"
                         for k, r in self.report.items())
