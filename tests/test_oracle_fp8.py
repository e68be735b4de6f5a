"""Pins of the FP8 (E4M3) oracle: the code values against the format's fixed points and
torch's float8_e4m3fn conversion for all 256 codes, the quantizer's rounding (ties to even),
saturation and scale, and attention over a dequantised cache. Planted mistakes in the FP8
code must fail a pin."""
import inspect
import math
import types

import numpy as np
import pytest
import torch

import gen
import oracle
import oracle.fp8 as of8


def test_fixed_points_of_the_format():
    v = of8.e4m3_value(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x39, 0x40, 0x7E, 0xFE,
                                 0x7F, 0xFF, 0x77]))
    np.testing.assert_array_equal(v[:10], [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0,
                                           1.125, 2.0, 448.0, -448.0])
    assert math.copysign(1.0, v[1]) < 0
    assert np.isnan(v[10]) and np.isnan(v[11])
    assert v[12] == 1.875 * 2.0 ** 7                     # e = 14, m = 7: 240


def test_all_codes_match_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    mine = of8.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()


def test_quantizer_round_trip_ties_saturation_and_scale():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = of8.e4m3_value(codes)
    back = of8.e4m3_quantize(vals, 1.0)
    np.testing.assert_array_equal(of8.e4m3_value(back), vals)      # every value is a fixed point
    # ties: 1.0625 is halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1) -> 1.0;
    # 1.1875 between 1.125 (1) and 1.25 (2) -> 1.25; same for negatives and subnormals
    t = of8.e4m3_quantize(np.array([1.0625, 1.1875, -1.0625, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9]), 1.0)
    np.testing.assert_array_equal(of8.e4m3_value(t), [1.0, 1.25, -1.0, 2.0 ** -8, 2.0 ** -8])
    # just off a tie (by one fp32 step, the precision of the quotient) goes to the nearer code
    t = of8.e4m3_quantize(np.array([1.0625 + 2.0 ** -23, 1.1875 - 2.0 ** -23]), 1.0)
    np.testing.assert_array_equal(of8.e4m3_value(t), [1.125, 1.125])
    s = of8.e4m3_quantize(np.array([464.0, 1e6, -1e30, 500.0]), 1.0)  # beyond 448 saturates
    np.testing.assert_array_equal(s, [0x7E, 0x7E, 0xFE, 0x7E])
    np.testing.assert_array_equal(of8.e4m3_quantize(np.array([3.0, -0.5]), 2.0),
                                  of8.e4m3_quantize(np.array([1.5, -0.25]), 1.0))
    assert of8.e4m3_quantize(np.array([np.nan]), 1.0)[0] in (0x7F, 0xFF)


def test_quantizer_matches_torch_inside_the_range():
    x = np.random.default_rng(3).normal(size=20000) * 60
    x = x[np.abs(x) < 440]
    mine = of8.e4m3_quantize(x, 1.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)


def test_attention_over_a_dequantised_cache():
    b = gen.make_batch("fp8", num_heads=4, num_kv_heads=2, head_size=8, block_size=16,
                       dtype="f32", query_lens=[1, 1, 1], seq_lens=[20, 45, 7],
                       passes=[(True, 0)], seed=4, pool_factor=2)
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(2, b.num_blocks, 16, 2, 8)).astype(np.uint8)
    codes[codes == 0x7F] = 0x3F
    codes[codes == 0xFF] = 0xBF
    q = rng.normal(size=(3, 4, 8))
    ks, vs = 0.03, 0.5
    o, l = oracle.attention_fp8_kv(q, codes, ks, vs, b.block_table, b.query_start_loc,
                                   b.seq_lens, 0.3, True)
    kv = np.stack([of8.e4m3_value(codes[0]) * ks, of8.e4m3_value(codes[1]) * vs])
    o2, l2 = oracle.attention(q, kv, b.block_table, b.query_start_loc, b.seq_lens, 0.3, True)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    # v_scale scales the output, k_scale acts like the softmax scale
    o3, l3 = oracle.attention_fp8_kv(q, codes, ks * 2, vs * 3, b.block_table, b.query_start_loc,
                                     b.seq_lens, 0.15, True)
    np.testing.assert_allclose(o3, 3 * o, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(l3, l, rtol=0, atol=1e-13)


MUTATIONS = {
    "bias_8": ("np.ldexp(1.0 + m / 8.0, (e - 7)", "np.ldexp(1.0 + m / 8.0, (e - 8)"),
    "subnormal_scale": ("sub = sign * m * 2.0 ** -9", "sub = sign * m * 2.0 ** -10"),
    "ties_away": ("pick_hi | (tie & even_hi)", "pick_hi | tie"),
    "overflow_to_nan": ("code = np.where(np.isnan(y), 0x7F",
                        "code = np.where(np.isnan(y) | (np.abs(y) > E4M3_MAX), 0x7F"),
    "v_scale_on_k": ("kv[0] = e4m3_value(codes[0]) * float(k_scale)",
                     "kv[0] = e4m3_value(codes[0]) * float(v_scale)"),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_a_planted_fp8_mistake_fails_some_pin(mutation, monkeypatch):
    before, after = MUTATIONS[mutation]
    src = inspect.getsource(of8)
    assert before in src
    mod = types.ModuleType("oracle_fp8_mutant")
    src = src.replace("from .naive_attention import attention", "from oracle import attention")
    exec(compile(src.replace(before, after, 1), "oracle_fp8_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(of8, "e4m3_value", mod.e4m3_value)
    monkeypatch.setattr(of8, "e4m3_quantize", mod.e4m3_quantize)
    monkeypatch.setattr(oracle, "attention_fp8_kv", mod.attention_fp8_kv)
    pins = [test_fixed_points_of_the_format, test_all_codes_match_torch_float8_e4m3fn,
            test_quantizer_round_trip_ties_saturation_and_scale,
            test_quantizer_matches_torch_inside_the_range, test_attention_over_a_dequantised_cache]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"no pin caught mutation {mutation}"
