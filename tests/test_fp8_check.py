"""The FP8 decision checker (tests/fp8_check.py) against codecs planted on the CPU: it accepts a
round-to-nearest-even codec whose inputs carry fp32-sized errors, and rejects truncation, rounding
toward zero, rounding away from zero, a wrong scale and a code two steps away.  It also checks that
the oracle refuses a choice outside its own ambiguity set."""
import numpy as np
import pytest

from fp8_check import DELTA, KernelTies
from oracle import model
from oracle.numerics import (e4m3_decode, e4m3_encode, e4m3_enclosing, e4m3_midpoint_margin, e4m3_other_code,
                             quant_per_token, round_f32)


def _pre(seed=0, rows=8, k=1024):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, k)) * rng.uniform(0.5, 2.0, (rows, 1))


def _ratio(pre):
    _, s = quant_per_token(pre)
    return round_f32(pre / s[:, None]), s


def _run(pre, kernel_codes, kernel_s, key="mq"):
    ties = KernelTies({key: (kernel_codes, kernel_s)})
    out = {}
    codes, s = model._quant(pre, key, ties, out)
    return ties, codes, out


def test_margin_and_other_code_are_the_grid():
    v = np.array([1.0, 1.0625, 1.06, 1.07, 448.0, 600.0, -3.3, 2.0 ** -10])
    lo, hi = e4m3_enclosing(v)
    assert list(lo) == [1.0, 1.0, 1.0, 1.0, 448.0, 448.0, 3.25, 0.0]
    assert list(hi) == [1.125, 1.125, 1.125, 1.125, 448.0, 448.0, 3.5, 2.0 ** -9]
    m = e4m3_midpoint_margin(v)
    assert m[1] == 0.0 and m[7] == 0.0 and np.isinf(m[4]) and np.isinf(m[5])  # ties sit on a midpoint
    assert abs(m[2] - 0.0025) < 1e-12
    c = e4m3_encode(v)
    o = e4m3_other_code(v, c)
    assert list(e4m3_decode(o)) == [1.125, 1.125, 1.125, 1.0, 448.0, 448.0, -3.5, 2.0 ** -9]


def test_rne_with_fp32_sized_errors_passes():
    pre = _pre()
    rng = np.random.default_rng(1)
    noisy = pre * (1.0 + rng.uniform(-2e-7, 2e-7, pre.shape))  # an fp32 evaluation of the same values
    k_codes, k_s = quant_per_token(noisy)
    ties, codes, out = _run(pre, k_codes, k_s)
    assert np.array_equal(e4m3_decode(codes), e4m3_decode(k_codes))  # the kernel's choice where ambiguous
    r = ties.report["mq"]
    assert r["ambiguous"] <= 0.02 * pre.size and r["flipped"] <= r["ambiguous"]
    assert out["mq_ambiguous"].sum() == r["ambiguous"]


@pytest.mark.parametrize("codec", ["truncate", "toward_zero_plus_one_ulp_up", "away_from_zero"])
def test_wrong_rounding_is_rejected(codec):
    pre = _pre(seed=2)
    v, s = _ratio(pre)
    lo, hi = e4m3_enclosing(v)
    sign = np.where(np.signbit(v), -1.0, 1.0)
    if codec == "truncate":  # round toward zero
        mag = lo
    elif codec == "toward_zero_plus_one_ulp_up":  # round up in magnitude (ceiling)
        mag = np.where(np.abs(v) == lo, lo, hi)
    else:  # round half away from zero instead of half to even: differs only at exact ties, so
        # make every value an exact tie
        mid = 0.5 * (lo + hi)
        v = np.where(np.abs(v) < 448, sign * mid, v)
        pre = v * s[:, None]
        mag = np.where(np.abs(v) < 448, hi, lo)
    k_codes = e4m3_encode(sign * mag)
    if codec == "away_from_zero":
        # exact ties sit on a midpoint, ambiguous under any delta, so a tie-breaking rule cannot be
        # seen element by element; a draw made of ties is refused by the bound on the ambiguity set
        with pytest.raises(AssertionError, match="too large"):
            _run(pre, k_codes, s)
        return
    with pytest.raises(AssertionError, match="away from any rounding midpoint"):
        _run(pre, k_codes, s)


def test_wrong_scale_is_rejected():
    pre = _pre(seed=3)
    k_codes, k_s = quant_per_token(pre)
    with pytest.raises(AssertionError, match="scale"):
        _run(pre, k_codes, k_s * (1 + 1e-4))


def test_code_two_steps_away_is_rejected():
    pre = _pre(seed=4)
    v, s = _ratio(pre)
    codes = e4m3_encode(v)
    amb = np.argwhere(e4m3_midpoint_margin(v) <= DELTA["mq"][0] * np.abs(v) + DELTA["mq"][1])
    assert len(amb), "the draw has an ambiguous element"
    i, j = amb[0]
    bad = codes.copy()
    step = 2 if (bad[i, j] & 0x7F) < 0x7C else -2
    bad[i, j] = np.uint8(int(bad[i, j]) + step)
    with pytest.raises(AssertionError, match="neither"):
        _run(pre, bad, s)


def test_oracle_refuses_a_choice_outside_its_ambiguity_set():
    pre = _pre(seed=5)

    class Greedy:  # tries to flip every element
        def delta(self, key):
            return DELTA["mq"]

        def choose(self, key, v, codes, s, amb):
            return np.ones(codes.shape, bool)

    with pytest.raises(ValueError, match="outside the oracle's ambiguity set"):
        model._quant(pre, "mq", Greedy(), {})


# --- bf16 decisions (q, k, v on the way to the oq quantisation) ---

def test_bf16_enclosing_margin_and_other():
    from oracle.numerics import bf16_enclosing, bf16_midpoint_margin, bf16_other, round_bf16
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -9, -3.0, 255.5, 2.0 ** -130])
    lo, hi = bf16_enclosing(x)
    assert list(lo) == [1.0, 1.0, 1.0, 3.0, 255.0, 2.0 ** -130]
    assert list(hi) == [1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7, 3.0 + 2.0 ** -6, 256.0, 2.0 ** -130 + 2.0 ** -133]
    assert list(bf16_midpoint_margin(x)) == [2.0 ** -8, 0.0, 2.0 ** -9, 2.0 ** -7, 0.0, 2.0 ** -134]
    assert list(bf16_other(x, round_bf16(x))) == [1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7, -(3.0 + 2.0 ** -6),
                                                  255.0, 2.0 ** -130 + 2.0 ** -133]
    rng = np.random.default_rng(4)
    y = rng.standard_normal(10000) * 10.0 ** rng.uniform(-3, 3, 10000)
    r = round_bf16(y)
    lo, hi = bf16_enclosing(y)
    assert np.all((np.abs(r) == lo) | (np.abs(r) == hi))  # RNE picks one of the pair
    o = bf16_other(y, r)
    assert np.all(np.abs(o) != np.abs(r)) and np.all(np.sign(o) == np.sign(y))
    assert np.all(np.abs(np.abs(y) - np.abs(r)) <= np.abs(np.abs(y) - np.abs(o)))  # RNE is the nearer one


def _bf16_run(pre, kernel_vals, key="q"):
    ties = KernelTies({}, bf16={key: kernel_vals})
    return ties, model._round_bf16(pre, key, ties)


def test_bf16_rne_with_fp32_sized_errors_passes_and_is_followed():
    from oracle.numerics import round_bf16
    rng = np.random.default_rng(5)
    pre = rng.standard_normal((16, 8, 128))
    noisy = pre * (1.0 + rng.uniform(-2e-7, 2e-7, pre.shape))  # an fp32 evaluation of the same values
    k = round_bf16(noisy)
    ties, got = _bf16_run(pre, k)
    assert np.array_equal(got, k)  # the kernel's choice where ambiguous, the oracle's own elsewhere (equal)
    r = ties.report["q"]
    assert r["flipped"] <= r["ambiguous"] <= 0.04 * pre.size


def test_bf16_near_zero_admits_several_values():
    """An element whose size is comparable to the absolute evaluation error admits more than the
    enclosing pair: a value two bf16 steps from the oracle's there is accepted and followed."""
    from oracle.numerics import bf16_admissible, round_bf16
    rng = np.random.default_rng(8)
    pre = rng.standard_normal((2, 2, 128))
    pre[0, 0, 5] = 3e-7  # rms ~ 1: delta_abs 2^-18 ~ 3.8e-6 spans many bf16 steps here
    ties = KernelTies({}, bf16={"q": round_bf16(pre)})
    lo, hi = bf16_admissible(pre, ties.bf16_delta("q", pre))
    k = round_bf16(pre)
    k[0, 0, 5] = lo[0, 0, 5]  # several steps below the oracle's value, still admissible
    assert k[0, 0, 5] != round_bf16(pre)[0, 0, 5]
    ties = KernelTies({}, bf16={"q": k})
    got = model._round_bf16(pre, "q", ties)
    assert got[0, 0, 5] == lo[0, 0, 5] and np.array_equal(np.delete(got, 5), np.delete(round_bf16(pre), 5))


@pytest.mark.parametrize("codec", ["truncate", "two_steps", "away"])
def test_bf16_wrong_rounding_is_rejected(codec):
    from oracle.numerics import bf16_enclosing, bf16_other, round_bf16
    rng = np.random.default_rng(6)
    pre = rng.standard_normal((16, 8, 128))
    lo, hi = bf16_enclosing(pre)
    if codec == "truncate":
        k = np.sign(pre) * lo
    elif codec == "away":
        k = np.sign(pre) * hi
    else:  # the RNE value moved by two spacings on one element far from any midpoint
        k = round_bf16(pre)
        k.flat[7] += 2 * (hi.flat[7] - lo.flat[7]) * np.sign(pre.flat[7])
    with pytest.raises(AssertionError):
        _bf16_run(pre, k)


def test_bf16_choice_outside_the_ambiguity_set_is_refused():
    from oracle.numerics import round_bf16

    from oracle.numerics import bf16_other

    class Rogue(KernelTies):
        def choose_bf16(self, key, pre, rne, ambiguous):
            return np.where(ambiguous, rne, bf16_other(pre, rne))  # every unambiguous element the other way

    pre = np.random.default_rng(7).standard_normal((4, 2, 128))
    with pytest.raises(ValueError):
        model._round_bf16(pre, "k", Rogue({}, bf16={"k": round_bf16(pre)}))
