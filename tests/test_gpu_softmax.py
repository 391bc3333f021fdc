"""GPU parity of alibi_masked_softmax against the CPU oracle.

Workload: bf16 scores [32, 14, 1, 2048] ~ N(0, 4) (also std 2), per-row left-pad
valid lengths uniform in [64, 2048], slopes of global heads 0..13 of a 112-head model
("Hugging Face BLOOM Inference Optimization", Custom CUDA Kernels and Hardware
Acceleration).  Gate: absolute error <= 1e-3 on the float32 output; masked entries
exactly 0.  Adversarial variants catch a kernel that ignores the mask (the ALiBi
decay alone would hide it): huge scores in masked slots, valid length 1 and K,
several queries with a causal mask, rows with nothing visible, ragged K.
"""
import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle

pytestmark = pytest.mark.gpu

BF16_MAX_BITS = 0x7F7F


def _run(scores_bits_or_f32, valid, H=14, n_total=112, off=0, out="f32", Q=1, offset=0):
    import transformer_bloom_decode_amd as tb

    if scores_bits_or_f32.dtype == np.uint16:
        s = torch.from_numpy(scores_bits_or_f32.view(np.int16)).cuda()
        in_dt = tb.BLOOM_BF16
    else:
        s = torch.from_numpy(scores_bits_or_f32).cuda()
        in_dt = tb.BLOOM_F32
    B, Hh, Qq, K = scores_bits_or_f32.shape
    odt = torch.float32 if out == "f32" else torch.bfloat16
    p = torch.full((B * Hh * Qq * K + offset,), float("nan"), dtype=odt, device="cuda")
    if offset:  # misaligned input and output pointers
        s = torch.cat([s.flatten()[:1], s.flatten()])[1:]
    pv = p[offset:]
    vl = torch.from_numpy(np.asarray(valid, np.int32)).cuda()
    tb.alibi_masked_softmax(s, in_dt, vl, B, Hh, Qq, K, n_total, off, pv,
                            tb.BLOOM_F32 if out == "f32" else tb.BLOOM_BF16)
    torch.cuda.synchronize()
    return pv.float().cpu().numpy().reshape(B, Hh, Qq, K)


def _ref(scores, valid, n_total=112, off=0):
    vals = bi.bf16_to_f32(scores) if scores.dtype == np.uint16 else scores
    return oracle.alibi_masked_softmax(vals, valid, n_total, off)


def _check(got, ref, valid, Q=1):
    K = got.shape[-1]
    err = np.abs(got - ref).max()
    assert err <= 1e-3, err
    for b, vl in enumerate(valid):
        assert np.all(got[b, :, :, : K - vl] == 0.0)       # masked: exactly zero
    return err


@pytest.mark.parametrize("std", [4.0, 2.0])
def test_softmax_workload_shape(std):
    scores, valid = bi.softmax_inputs(std=std)
    got = _run(scores, valid)
    ref = _ref(scores, valid)
    err = _check(got, ref, valid)
    print(f"softmax [32,14,1,2048] std={std}: max abs err {err:.3e}")
    rows = got.sum(-1)
    np.testing.assert_allclose(rows, 1.0, atol=2048 * 2 ** -24 * 4)


def test_softmax_masked_slots_hold_huge_scores():
    scores, valid = bi.softmax_inputs()
    evil = scores.copy()
    for b, vl in enumerate(valid):
        evil[b, :, :, : 2048 - vl] = BF16_MAX_BITS
    got = _run(evil, valid)
    _check(got, _ref(scores, valid), valid)


@pytest.mark.parametrize("vl", [1, 2, 2048])
def test_softmax_extreme_lengths(vl):
    scores, _ = bi.softmax_inputs()
    valid = np.full((32,), vl, np.int32)
    got = _run(scores, valid)
    _check(got, _ref(scores, valid), valid)
    if vl == 1:
        assert np.all(got[:, :, 0, -1] == 1.0)               # one visible key: one-hot


def test_softmax_zero_valid_rows_are_zero():
    scores, valid = bi.softmax_inputs()
    valid = valid.copy()
    valid[::3] = 0
    got = _run(scores, valid)
    assert np.all(got[::3] == 0.0)
    _check(got, _ref(scores, valid), valid)


def test_softmax_causal_queries_and_other_heads():
    rng = np.random.default_rng(0)
    B, H, Q, K = 3, 5, 4, 300
    scores = bi.f32_to_bf16(rng.standard_normal((B, H, Q, K)).astype(np.float32) * 4)
    valid = np.array([300, 3, 150], np.int32)
    got = _run(scores, valid, H=H, n_total=40, off=17, Q=Q)
    ref = _ref(scores, valid, n_total=40, off=17)
    _check(got, ref, valid)
    for i in range(Q):                                        # keys after the query: 0
        assert np.all(got[:, :, i, K - Q + i + 1:] == 0.0)


@pytest.mark.parametrize("K", [2047, 4100, 7])
def test_softmax_ragged_and_long_rows(K):
    rng = np.random.default_rng(K)
    B, H = 2, 3
    scores = rng.standard_normal((B, H, 1, K)).astype(np.float32) * 4
    valid = np.array([K, max(1, K // 3)], np.int32)
    got = _run(scores, valid, H=H, n_total=8)
    _check(got, _ref(scores, valid, n_total=8), valid)


def test_softmax_misaligned_pointers():
    scores, valid = bi.softmax_inputs()
    got = _run(scores, valid, offset=1)
    _check(got, _ref(scores, valid), valid)


def test_softmax_bf16_output_within_rounding():
    scores, valid = bi.softmax_inputs()
    got = _run(scores, valid, out="bf16")
    ref = _ref(scores, valid)
    # bf16 keeps 8 significant bits: round-to-nearest is within 2^-8 relative (half an
    # ulp, i.e. 2^-9 absolute on [0.5, 1)), plus the fp32 noise of the softmax itself
    assert np.all(np.abs(got - ref) <= 2 ** -8 * np.abs(ref) + 1e-6)
    for b, vl in enumerate(valid):
        assert np.all(got[b, :, :, : 2048 - vl] == 0.0)


def test_softmax_power_of_two_head_slopes_exact():
    """8 heads: slopes 2^-1 .. 2^-8 exactly; with zero scores and K keys all visible the
    row is a geometric distribution whose ratios are exp(slope)."""
    K = 16
    scores = np.zeros((1, 8, 1, K), np.float32)
    got = _run(scores, np.array([K], np.int32), H=8, n_total=8)
    ratios = got[0, :, 0, 1:] / got[0, :, 0, :-1]
    expect = np.exp(2.0 ** -np.arange(1, 9))[:, None]
    np.testing.assert_allclose(ratios, np.broadcast_to(expect, ratios.shape), rtol=2e-6)
