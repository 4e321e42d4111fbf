"""Pins of the number formats: exhaustive e4m3 codec facts, RNE ties, saturation, and the
special case where a library cast implements the same single rounding."""
import numpy as np
import pytest
import torch

from oracle import numerics as nu


def test_e4m3_code_table_facts():
    v = nu.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = ~np.isnan(v)
    assert fin.sum() == 254  # 0x7F and 0xFF are NaN
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    pos = v[(v > 0) & fin]
    assert pos.min() == 2.0 ** -9  # smallest subnormal
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9
    codes = np.arange(256, dtype=np.uint8)[fin]
    assert np.array_equal(nu.e4m3_encode(v[fin]), codes)  # decode then encode is the identity


def test_e4m3_rounding_ties_and_saturation():
    # between 1.0 (m=0) and 1.125 (m=1) the tie 1.0625 goes to even mantissa 0
    assert nu.e4m3_round(np.array([1.0625]))[0] == 1.0
    assert nu.e4m3_round(np.array([1.1875]))[0] == 1.25  # tie between m=1 and m=2 -> m=2
    assert nu.e4m3_round(np.array([500.0, -1e9, 464.0]))[0] == 448.0
    assert nu.e4m3_round(np.array([-1e9]))[0] == -448.0
    assert nu.e4m3_round(np.array([2.0 ** -10]))[0] == 0.0  # tie to even (0)
    assert nu.e4m3_round(np.array([3 * 2.0 ** -10]))[0] == 2.0 ** -8


def test_e4m3_error_bound_and_torch_agreement():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * 60
    r = nu.e4m3_round(x)
    xc = np.clip(x, -448, 448)
    ax = np.maximum(np.abs(xc), 2.0 ** -6)
    half_q = np.ldexp(1.0, np.floor(np.log2(ax)).astype(int) - 4)
    assert np.all(np.abs(r - xc) <= half_q + 1e-300)
    th = torch.from_numpy(xc).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(r, th)


def test_bf16_rne_and_torch_on_fp32_inputs():
    assert nu.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert nu.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert nu.bf16_bits_to_f64(np.array([0x3F80, 0xC000], dtype=np.uint16)).tolist() == [1.0, -2.0]
    x = (np.random.default_rng(1).standard_normal(100000) * 7).astype(np.float32).astype(np.float64)
    th = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(nu.round_bf16(x), th)
    bits = nu.f64_to_bf16_bits(x)
    assert np.array_equal(nu.bf16_bits_to_f64(bits), th)


def test_quant_per_token_rules():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((5, 300))
    h[3] = 0.0
    codes, s = nu.quant_per_token(h)
    assert s[3] == 1.0 and not codes[3].any()
    deq = nu.dequant_per_token(codes, s)
    amax = np.max(np.abs(h), axis=1)
    for i in (0, 1, 2, 4):
        j = np.argmax(np.abs(h[i]))
        assert abs(nu.e4m3_decode(codes[i, j])) == 448.0  # amax maps to +-448 exactly
        assert np.all(np.abs(deq[i] - h[i]) <= amax[i] / 448 * 16 + 1e-12)  # half the top quantum (32)


def test_weight_block_quant_partial_edges():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((200, 300)) * 0.02
    codes, s = nu.quant_weight_blocks(w)
    assert s.shape == (2, 3)
    assert s[1, 2] == nu.round_f32(np.max(np.abs(w[128:, 256:])) / 448)
    deq = nu.dequant_weight_blocks(codes, s)
    assert np.max(np.abs(deq - w)) <= np.max(s) * 16
