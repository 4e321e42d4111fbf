"""Number formats used by the chain, written from their format definitions.

* bf16: 1 sign, 8 exponent, 7 stored significand bits (same exponent range as
  IEEE binary32); rounding from float64 is round-to-nearest, ties to even, done
  in one step (no intermediate binary32 rounding).
* fp32: IEEE binary32 round-to-nearest-even (NumPy's float64 -> float32 cast).
* e4m3 (OCP 8-bit floating point, "E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa
  bits; no infinities; S.1111.111 is NaN; the largest finite magnitude is
  1.75 * 2**8 = 448; exponent field 0 holds subnormals m/8 * 2**-6.  Encoding here
  clamps to [-448, 448] first and then rounds to nearest-even ("satfinite"), so
  it never produces NaN.

The FP8 per-token and per-block quantisation rules (scale = amax / 448, amax 0 ->
scale 1) are the reading of the indexer front's "Add + RMSNorm + Quant" step on the
MegaRTP page (section 4, event0 publishes "hidden FP8/scale") and of the block-scaled
FP8 GEMMs it feeds (section 4, DeepGEMM GEMM specs).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _rne_to_grid(x: np.ndarray, mant_bits: int, min_exp: int) -> np.ndarray:
    """Round float64 x to the binary grid with ``mant_bits`` fraction bits whose
    smallest normal exponent is ``min_exp`` (below it the quantum stays 2**(min_exp-mant_bits))."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    # guard the floor(log2) of values a hair below a power of two
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > ax, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= ax, e + 1, e)
    e = np.maximum(e, min_exp)
    q = np.ldexp(1.0, (e - mant_bits).astype(np.int64))
    return np.round(x / q) * q  # np.round: half to even; x/q and *q are exact (powers of two)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (RNE), returned as float64; overflow -> +-inf."""
    r = _rne_to_grid(x, 7, -126)
    bf16_max = (2 - 2.0 ** -7) * 2.0 ** 127
    return np.where(np.abs(r) > bf16_max, np.sign(r) * np.inf, r)


def bf16_enclosing(x: np.ndarray):
    """(lo, hi): the adjacent bf16 magnitudes with lo <= |x| < hi (the finite range)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(np.ldexp(1.0, e.astype(np.int64)) > a, e - 1, e)
    e = np.where(np.ldexp(1.0, (e + 1).astype(np.int64)) <= a, e + 1, e)
    q = np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64))  # the bf16 spacing at |x|
    lo = np.floor(a / q) * q
    return lo, lo + q


def bf16_midpoint_margin(x: np.ndarray) -> np.ndarray:
    """Distance from |x| to the midpoint of its enclosing bf16 pair, where round-to-nearest
    changes its choice."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    lo, hi = bf16_enclosing(a)
    return np.abs(a - 0.5 * (lo + hi))


def bf16_other(x: np.ndarray, chosen: np.ndarray) -> np.ndarray:
    """The other member of the bf16 pair enclosing x (with x's sign): the value a rounding on the
    other side of the midpoint gives."""
    x = np.asarray(x, dtype=np.float64)
    lo, hi = bf16_enclosing(x)
    other = np.where(np.abs(np.asarray(chosen, dtype=np.float64)) == lo, hi, lo)
    return np.where(np.signbit(x), -other, other)


def bf16_admissible(x: np.ndarray, delta: np.ndarray):
    """(lo, hi): the least and greatest bf16 values that round-to-nearest gives for some value
    within delta of x (rounding is monotone, so every bf16 value between them is one too)."""
    x = np.asarray(x, dtype=np.float64)
    return round_bf16(x - delta), round_bf16(x + delta)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    r = round_bf16(x).astype(np.float32)  # exact: r has at most 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """The format definition, code by code: sign, exponent field (bias 7; 0 = subnormal), mantissa."""
    c = np.asarray(c, dtype=np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


_E4M3_VALUES = _e4m3_value(np.arange(256))  # all 256 codes, decoded once


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Clamp to [-448, 448] and round to the nearest e4m3 value (ties to even)."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    return _rne_to_grid(x, 3, -6)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Saturating RNE encode of float64 values to e4m3 code bytes (sign kept on zero)."""
    x = np.asarray(x, dtype=np.float64)
    v = e4m3_round(x)
    a = np.abs(v)
    sign = (np.signbit(x) & ~np.isnan(x)).astype(np.int64) << 7
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    normal = a >= 2.0 ** -6
    ef = np.where(normal, e + 7, 0)
    mant = np.where(normal, np.round((a / np.ldexp(1.0, e) - 1.0) * 8.0), np.round(a / 2.0 ** -9))
    code = sign | (ef << 3) | mant.astype(np.int64)
    return code.astype(np.uint8)


def quant_scale(amax: np.ndarray) -> np.ndarray:
    """Per-group FP8 scale: fp32(amax / 448), or 1 where amax is 0."""
    amax = np.asarray(amax, dtype=np.float64)
    return np.where(amax > 0, round_f32(amax / E4M3_MAX), 1.0)


def quant_per_token(h: np.ndarray):
    """Per-row FP8 quantisation of [M, K] values: returns (codes uint8 [M,K], scale f64 [M]).

    The scale division is taken in fp32 (the precision the kernel takes the code
    decision in): q = e4m3(fp32(h / s))."""
    h = np.asarray(h, dtype=np.float64)
    s = quant_scale(np.max(np.abs(h), axis=-1))
    ratio = round_f32(h / s[..., None])
    return e4m3_encode(ratio), s


def dequant_per_token(codes: np.ndarray, s: np.ndarray) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(s, dtype=np.float64)[..., None]


def quant_weight_blocks(w: np.ndarray, block: int = 128):
    """Per 128x128 block of an [N, K] matrix: s[nb, kb] = fp32(amax / 448); codes = e4m3(w / s).
    Edge blocks are partial."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    nb, kb = -(-n // block), -(-k // block)
    s = np.ones((nb, kb))
    codes = np.zeros((n, k), dtype=np.uint8)
    for i in range(nb):
        for j in range(kb):
            blk = w[i * block:(i + 1) * block, j * block:(j + 1) * block]
            sc = quant_scale(np.max(np.abs(blk)))
            s[i, j] = sc
            codes[i * block:(i + 1) * block, j * block:(j + 1) * block] = e4m3_encode(round_f32(blk / sc))
    return codes, s


def dequant_weight_blocks(codes: np.ndarray, s: np.ndarray, block: int = 128) -> np.ndarray:
    v = e4m3_decode(codes)
    n, k = v.shape
    sf = np.repeat(np.repeat(np.asarray(s, dtype=np.float64), block, axis=0), block, axis=1)[:n, :k]
    return v * sf


# ---------------------------------------------------------------------------------------------
# Rounding margins.  A value that an fp32 evaluation reproduces only to within delta may round
# to either code of the pair enclosing it when it lies within delta of that pair's midpoint;
# everywhere else round-to-nearest-even fixes the code.  These helpers give the oracle's own
# measure of that: they are the format definition (the grid, its midpoints) and nothing else.

_E4M3_GRID = np.unique(np.abs(_E4M3_VALUES[~np.isnan(_E4M3_VALUES)]))  # 0, 2^-9, ..., 448 ascending


def e4m3_enclosing(v: np.ndarray):
    """(lo, hi): the adjacent e4m3 magnitudes with lo <= |v| < hi; lo = hi = 448 from 448 up."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    i = np.searchsorted(_E4M3_GRID, a, side="right")
    top = len(_E4M3_GRID) - 1
    lo = _E4M3_GRID[np.clip(i - 1, 0, top)]
    hi = _E4M3_GRID[np.clip(i, 0, top)]
    return lo, hi


def e4m3_midpoint_margin(v: np.ndarray) -> np.ndarray:
    """Distance from |v| to the midpoint of its enclosing pair (the point where round-to-nearest
    changes its choice); infinite from 448 up, where the satfinite clamp decides."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    lo, hi = e4m3_enclosing(a)
    return np.where(a >= E4M3_MAX, np.inf, np.abs(a - 0.5 * (lo + hi)))


def e4m3_ambiguous(v: np.ndarray, delta_rel: float, delta_abs: float) -> np.ndarray:
    """True where |v| lies within delta_rel |v| + delta_abs of a rounding midpoint."""
    v = np.asarray(v, dtype=np.float64)
    return e4m3_midpoint_margin(v) <= delta_rel * np.abs(v) + delta_abs


def e4m3_other_code(v: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """The code of the other member of the pair enclosing v (same sign as v): the code a rounding
    on the other side of the midpoint gives.  From 448 up the pair is (448, 448)."""
    v = np.asarray(v, dtype=np.float64)
    lo, hi = e4m3_enclosing(v)
    chosen = np.abs(e4m3_decode(codes))
    other = np.where(chosen == lo, hi, lo)
    return e4m3_encode(np.where(np.signbit(v), -other, other))
