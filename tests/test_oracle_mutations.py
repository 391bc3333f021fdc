"""Plant plausible mistakes in the CPU oracle and check that the pins catch them.

Each mutation patches one function of ``oracle.bloom_oracle`` for the duration of a
test (on the CPU only); the Hugging Face float64 comparison must then fail by a wide
margin, showing that the pin is sensitive to that kind of slip.
"""
import math

import numpy as np
import pytest
import scipy.special

import bloom_inputs as bi
import oracle
from oracle import bloom_oracle as bo


def _gelu_erf(x):
    return 0.5 * x * (1 + scipy.special.erf(x / math.sqrt(2)))


def _slopes_sign_flipped(n, dtype=np.float64):
    return -_ORIG["alibi_slopes"](n, dtype)


def _slopes_even_terms(n, dtype=np.float64):
    c = 1 << (n.bit_length() - 1)
    s = list(_ORIG["alibi_slopes"](c, dtype))
    s += [2.0 ** (-8.0 * k / (2 * c)) for k in range(2, 2 * (n - c) + 1, 2)]
    return np.array(s, dtype)


def _slopes_zero(n, dtype=np.float64):
    return np.zeros(n, dtype)


def _ln_unbiased(x, g, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = x.var(axis=-1, ddof=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def _ln_no_eps(x, g, b, eps):
    return _ORIG["layer_norm"](x, g, b, 0.0)


def _attention_scale_1_over_d(q, k, v, slopes, pad, start):
    return _ORIG["attention"](q / math.sqrt(q.shape[-1]), k, v, slopes, pad, start)


def _attention_excludes_self(q, k, v, slopes, pad, start):
    # causal mask off by one: the current token does not see itself
    B, S, H, d = q.shape
    T = k.shape[2]
    scores = np.einsum("bshd,bhtd->bhst", q, k) / math.sqrt(d)
    j = np.arange(T)
    p = start + np.arange(S)
    bias = slopes[None, :, None, None] * (j[None, :] - pad[:, None])[:, None, None, :]
    valid = (j[None, None, None, :] >= pad[:, None, None, None]) & \
            (j[None, None, None, :] < p[None, None, :, None])
    probs = bo.masked_softmax(scores + bias, valid)
    return np.einsum("bhst,bhtd->bshd", probs, v)


def _attention_unmasked_pad(q, k, v, slopes, pad, start):
    return _ORIG["attention"](q, k, v, slopes, np.zeros_like(pad), start)


_ORIG = {n: getattr(bo, n) for n in ("alibi_slopes", "layer_norm", "attention", "gelu_tanh")}

MUTATIONS = {
    "gelu_erf_form": ("gelu_tanh", _gelu_erf),
    "alibi_sign_flipped": ("alibi_slopes", _slopes_sign_flipped),
    "alibi_dropped": ("alibi_slopes", _slopes_zero),
    "layernorm_unbiased_variance": ("layer_norm", _ln_unbiased),
    "layernorm_without_eps": ("layer_norm", _ln_no_eps),
    "attention_scale_1_over_d": ("attention", _attention_scale_1_over_d),
    "causal_mask_off_by_one": ("attention", _attention_excludes_self),
    "left_pad_not_masked": ("attention", _attention_unmasked_pad),
}


def _hf_mismatch(n_head=8, valid=(8, 5), seed=0):
    import dataclasses

    import hf_pin

    m = dataclasses.replace(bi.TINY, n_head_total=n_head, n_head_local=n_head, head_dim=8,
                            hidden=8 * n_head, ffn=32 * n_head)
    T = bi.model_tensors(m, seed=seed)
    om = oracle.OracleModel.from_storage(m, T)
    hf = hf_pin.hf_bloom(m, T)
    ids, valid = bi.prompts(m, len(valid), 8, valid)
    pad = 8 - valid
    h = oracle.forward(om, ids, 0, pad, oracle.new_cache(om, len(valid)))
    worst = 0.0
    for b in range(len(valid)):
        ref = hf_pin.hf_hidden(hf, ids[b: b + 1, pad[b]:], [valid[b]])[0]
        got = h[b, pad[b]:]
        worst = max(worst, np.linalg.norm(got - ref) / np.linalg.norm(ref))
    return worst


def test_unmutated_oracle_agrees(hf_available):
    assert _hf_mismatch() < 1e-7
    assert _hf_mismatch(n_head=12, valid=(8, 3)) < 1e-7


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pin_catches_planted_mistake(name, monkeypatch, hf_available):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(bo, attr, fn)
    # 12 heads exercises the non-power-of-two slope branch; (8, 3) a padded row
    worst = max(_hf_mismatch(), _hf_mismatch(n_head=12, valid=(8, 3)))
    # the model pin (test_model_hidden_matches_hf_bloom) accepts at most 1e-7
    assert worst > 1e-7, f"mutation {name} went unnoticed (rel err {worst:.2e})"


def test_pin_catches_even_extra_slopes(monkeypatch, hf_available):
    monkeypatch.setattr(bo, "alibi_slopes", _slopes_even_terms)
    assert _hf_mismatch(n_head=12, valid=(8, 3)) > 1e-7
