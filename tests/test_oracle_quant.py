"""Pins of the oracle's int8 quantisation (the W8A8 activations and the int8 KV cache):
hand-worked codes, ties to even, the zero slice, the error bound that the definition
fixes, slices that quantise independently, inputs already on the grid, and the W8A8
linear against an exact integer product.  Planted mistakes (scale by amax instead of
amax / 127, truncation instead of rounding, ties away from zero, no clamp) each fail one
of them.
"""
import dataclasses

import numpy as np
import pytest

import bloom_inputs as bi
import oracle
from oracle import bloom_oracle as bo


def test_hand_worked_codes():
    q, s = oracle.quantize_int8(np.array([[0.5, -1.27, 0.3, 0.0]]))
    np.testing.assert_array_equal(q, [[50, -127, 30, 0]])
    assert s.dtype == np.float32 and s[0, 0] == np.float32(np.float32(1.27) / np.float32(127))


def test_ties_go_to_even():
    # amax 127: the multiplier is exactly 1, so x.5 values are exact ties
    q, s = oracle.quantize_int8(np.array([127.0, 0.5, 1.5, 2.5, -0.5, -2.5, -3.5, 126.5]))
    np.testing.assert_array_equal(q, [127, 0, 2, 2, 0, -2, -4, 126])
    assert s[0] == 1.0


def test_zero_slice():
    q, s = oracle.quantize_int8(np.zeros((2, 5)))
    assert not q.any() and not s.any()
    assert not oracle.int8_rows(np.zeros(7)).any()


def test_error_bound_and_range():
    rng = np.random.default_rng(5)
    a = rng.normal(size=(64, 333)) * rng.uniform(0.01, 100, size=(64, 1))
    q, s = oracle.quantize_int8(a)
    assert q.min() >= -127 and q.max() <= 127
    # every row reaches +-127 at its largest value
    assert np.all(np.abs(q).max(axis=1) == 127)
    err = np.abs(oracle.dequantize_int8(q, s) - a)
    # half a step, plus the float32 rounding of the input and the multiplier
    assert np.all(err <= s * (0.5 + 1e-5) + np.abs(a) * 2e-7)


def test_slices_quantise_independently():
    rng = np.random.default_rng(6)
    a = rng.normal(size=(3, 4, 64))
    q, s = oracle.quantize_int8(a)
    for i in range(3):
        for j in range(4):
            qi, si = oracle.quantize_int8(a[i, j])
            np.testing.assert_array_equal(q[i, j], qi)
            assert s[i, j, 0] == si[0]


def test_values_on_the_grid_survive_exactly():
    rng = np.random.default_rng(7)
    codes = rng.integers(-127, 128, size=(5, 40))
    codes[:, 0] = 127                         # amax = 127 * step exactly
    step = np.float32(2.0 ** -7)
    a = codes.astype(np.float64) * np.float64(step)
    np.testing.assert_array_equal(oracle.int8_rows(a), a)


def test_scaling_by_a_power_of_two_keeps_the_codes():
    rng = np.random.default_rng(8)
    a = rng.normal(size=(6, 50))
    q1, s1 = oracle.quantize_int8(a)
    q2, s2 = oracle.quantize_int8(a * 8.0)
    np.testing.assert_array_equal(q1, q2)
    np.testing.assert_array_equal(s2, s1 * 8)


def test_w8a8_linear_equals_an_integer_product():
    """The W8A8 linear (oracle: the weight-only linear applied to the dequantised
    activations) against s_a * s_w * (q_a . q_w) computed in exact integer arithmetic."""
    m = dataclasses.replace(bi.TINY, weight_dtype="int8", init_std=0.3)
    T = bi.model_tensors(m)
    lw = T["layers"][0]
    qw = lw["w_up"].astype(np.int64)
    sw = bi.f16_to_f32(lw["s_up"]).astype(np.float64)
    W = oracle.Int8RowScale(lw["w_up"], bi.f16_to_f32(lw["s_up"]))
    rng = np.random.default_rng(9)
    a = rng.normal(size=(5, m.hidden))
    qa, sa = oracle.quantize_int8(a)
    ref = sa.astype(np.float64) * sw[None, :] * (qa.astype(np.int64) @ qw.T).astype(np.float64)
    got = oracle.linear(oracle.int8_rows(a), W)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def _scale_by_amax(a):
    f = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(f), axis=-1, keepdims=True)
    inv = np.where(amax > 0, 1 / amax, 0).astype(np.float32)
    return np.clip(np.rint(f * inv), -127, 127).astype(np.int8), amax.astype(np.float32)


def _truncate(a):
    f = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(f), axis=-1, keepdims=True)
    inv = np.where(amax > 0, 127 / amax, 0).astype(np.float32)
    return np.clip(np.trunc(f * inv), -127, 127).astype(np.int8), (amax / 127).astype(np.float32)


def _ties_away(a):
    f = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(f), axis=-1, keepdims=True)
    inv = np.where(amax > 0, 127 / amax, 0).astype(np.float32)
    x = f * inv
    return (np.clip(np.sign(x) * np.floor(np.abs(x) + 0.5), -127, 127).astype(np.int8),
            (amax / 127).astype(np.float32))


def _no_clamp_wraps(a):
    # a scale from a smaller amax (the first half of the slice): codes past 127 wrap
    f = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(f[..., : f.shape[-1] // 2]), axis=-1, keepdims=True)
    inv = np.where(amax > 0, 127 / amax, 0).astype(np.float32)
    return np.rint(f * inv).astype(np.int64).astype(np.int8), (amax / 127).astype(np.float32)


@pytest.mark.parametrize("mutant", [_scale_by_amax, _truncate, _ties_away, _no_clamp_wraps])
def test_planted_quantiser_mistakes_fail_a_pin(mutant, monkeypatch):
    monkeypatch.setattr(bo, "quantize_int8", mutant)
    monkeypatch.setattr(oracle, "quantize_int8", mutant)
    pins = [test_hand_worked_codes, test_ties_go_to_even, test_error_bound_and_range,
            test_values_on_the_grid_survive_exactly]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"{mutant.__name__} passed every pin"


@pytest.mark.parametrize("act, kv", [("int8", "int8"), ("bf16", "int8"), ("int8", "bf16")])
def test_int8_modes_keep_incremental_decode_equal_to_a_rerun(act, kv):
    """Quantisation is per token (activations) and per token and head (keys, values), so
    the KV-cached steps still equal a full causal re-run of the prefix, and the modes
    change the result (the quantisation is applied)."""
    m = dataclasses.replace(bi.TINY, weight_dtype="int8", init_std=0.3, activations=act,
                            kv_cache=kv)
    T = bi.model_tensors(m)
    om = oracle.OracleModel.from_storage(m, T)
    assert (om.act_round is not None) == (act == "int8")
    assert (om.kv_round is not None) == (kv == "int8")
    ids, valid = bi.prompts(m, 2, 8, (8, 5))
    g = oracle.greedy_generate(om, ids, valid, 6)
    for t in range(6):
        seq = np.concatenate([ids, g.tokens[:, :t]], axis=1)
        full = oracle.forward(om, seq, 0, 8 - valid, oracle.new_cache(om, 2))[:, -1]
        np.testing.assert_allclose(g.hidden[t], full, rtol=1e-12, atol=1e-12)
    exact = oracle.OracleModel.from_storage(dataclasses.replace(m, activations="bf16",
                                                                kv_cache="bf16"), T)
    h_exact = oracle.greedy_generate(exact, ids, valid, 2, forced=g.tokens).hidden
    rel = np.linalg.norm(h_exact - g.hidden[:2]) / np.linalg.norm(h_exact)
    assert 1e-5 < rel < 5e-2
