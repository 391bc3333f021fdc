"""Pins of the oracle's per-row sampling (temperature + nucleus / top-p, then a draw
from the kept tokens): hand-worked cases, brute force over tiny vocabularies, the
frequencies a uniform grid of draws produces, and invariances of the definition
(Holtzman et al., "The Curious Case of Neural Text Degeneration", Section 3.1; the
pages name per-row sampling and top-p in the custom generation loop of "Hugging Face
BLOOM Inference Optimization", Webserver Architecture and Request Handling).
"""
import itertools

import numpy as np
import pytest

import oracle


def _one(logits, T, p, u):
    r = oracle.sample_tokens(np.asarray([logits], dtype=np.float64), [T], [p], [u])
    return int(r.tokens[0]), r


def test_hand_worked_four_tokens():
    # q = (1, 2, 3, 4) / 10.  top_p 0.5: 0.4 < 0.5 <= 0.4 + 0.3, so the nucleus is ids
    # {3, 2} with mass 0.7; in id order id 2 covers u in [0, 3/7), id 3 [3/7, 1).
    lg = np.log([1.0, 2.0, 3.0, 4.0])
    for u, want in ((0.0, 2), (0.42, 2), (0.43, 3), (0.999, 3)):
        tok, r = _one(lg, 1.0, 0.5, u)
        assert tok == want, (u, tok)
        assert r.nucleus_size[0] == 2
    _, r = _one(lg, 1.0, 0.5, 0.42)
    assert abs(r.keep_margin[0] - 0.1) < 1e-12          # min(0.5 - 0.4, 0.7 - 0.5)
    assert abs(r.draw_margin[0] - (3 / 7 - 0.42)) < 1e-12
    # top_p exactly at a cumulative boundary keeps the shorter prefix
    tok, r = _one(lg, 1.0, 0.4, 0.9)
    assert tok == 3 and r.nucleus_size[0] == 1


def test_greedy_rows_take_the_lowest_id_of_the_maximum():
    for T in (0.0, -1.0):
        tok, _ = _one([1.0, 3.0, 3.0, 2.0], T, 0.9, 0.7)
        assert tok == 1


def test_vanishing_temperature_tends_to_the_argmax():
    # softmax(logits / T) -> the one-hot of the largest logit as T -> 0: a small T that
    # still has a float32 reciprocal (the sampling branch) and one whose reciprocal
    # overflows float32 (taken as greedy) both give the argmax, for any u and top_p
    lg = [0.5, 2.0, 1.999, -3.0]
    for T in (1e-6, 1e-30, 1e-39):
        for u, p in ((0.0, 0.9), (0.999, 1.0), (0.5, 0.3)):
            tok, _ = _one(lg, T, p, u)
            assert tok == 1, (T, u, p, tok)


def test_ties_at_the_boundary_are_all_kept():
    # four equal tokens, top_p 0.3: the first token taken (0.25 < 0.3) is not enough,
    # the boundary value 0.25 is shared by all four, so all are kept
    tok, r = _one([0.5, 0.5, 0.5, 0.5], 1.0, 0.3, 0.6)
    assert r.nucleus_size[0] == 4
    assert tok == 2                                   # F = 0.25, 0.5, 0.75, 1


def test_tiny_top_p_is_the_argmax_and_top_p_one_keeps_everything():
    rng = np.random.default_rng(3)
    lg = rng.normal(0, 2, size=(1, 300))
    am = int(np.argmax(lg[0]))
    for u in (0.0, 0.3, 0.999):
        r = oracle.sample_tokens(lg, [0.8], [1e-12], [u])
        assert r.tokens[0] == am
        r = oracle.sample_tokens(lg, [0.8], [0.0], [u])
        assert r.tokens[0] == am
    r = oracle.sample_tokens(lg, [0.8], [1.0], [0.5])
    assert r.nucleus_size[0] == 300


def test_nucleus_is_the_smallest_set_reaching_top_p_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(40):
        V = 6
        lg = rng.normal(0, 1.5, size=V)
        if trial % 5 == 0:
            lg[1] = lg[4]                              # a tie somewhere
        T = float(rng.uniform(0.3, 2.0))
        p = float(rng.uniform(0.05, 0.98))
        q = np.exp(lg / T - np.max(lg / T))
        q /= q.sum()
        best = None
        for k in range(1, V + 1):
            for sub in itertools.combinations(range(V), k):
                if q[list(sub)].sum() >= p:
                    best = k
                    break
            if best:
                break
        # the nucleus: the best-size set of largest q, plus every token tied with its
        # smallest member
        thr = np.sort(q)[::-1][best - 1]
        want = set(np.nonzero(q >= thr)[0].tolist())
        r = oracle.sample_tokens(lg[None], [T], [p], [0.5])
        assert r.nucleus_size[0] == len(want), (trial, best, want)
        for u in np.linspace(0, 0.999, 7):
            tok = int(oracle.sample_tokens(lg[None], [T], [p], [u]).tokens[0])
            assert tok in want


@pytest.mark.parametrize("T,p", [(1.0, 1.0), (0.7, 0.8), (2.0, 0.3)])
def test_draw_frequencies_on_a_uniform_grid(T, p):
    """A grid of N evenly spaced u must pick each kept token a fraction of times equal
    to its renormalised probability (within one grid step)."""
    rng = np.random.default_rng(5)
    V = 40
    lg = rng.normal(0, 1.0, size=V)
    N = 4000
    us = (np.arange(N) + 0.5) / N
    r = oracle.sample_tokens(np.repeat(lg[None], N, 0), np.full(N, T), np.full(N, p), us)
    counts = np.bincount(r.tokens, minlength=V) / N
    q = np.exp(lg / T - np.max(lg / T))
    q /= q.sum()
    order = np.argsort(-q)
    cum = np.cumsum(q[order])
    k = int(np.argmax(cum >= p - 1e-15)) if p < 1 else V - 1
    kept = np.zeros(V, bool)
    kept[q >= q[order][k]] = True
    want = np.where(kept, q, 0.0)
    want /= want.sum()
    assert np.all(counts[~kept] == 0)
    assert np.max(np.abs(counts - want)) <= 1.0 / N + 1e-12


def test_temperature_is_a_logit_scale():
    rng = np.random.default_rng(8)
    lg = rng.normal(0, 3, size=(6, 500))
    us = rng.uniform(0, 1, size=6)
    ps = rng.uniform(0.2, 0.95, size=6)
    a = oracle.sample_tokens(lg, np.full(6, 2.0), ps, us).tokens
    b = oracle.sample_tokens(lg / 2.0, np.full(6, 1.0), ps, us).tokens
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# planted mistakes: each plausible slip in the sampler must fail one of the pins above
# ---------------------------------------------------------------------------

def _mutant(kind):
    from oracle import bloom_oracle as bo
    orig = bo.sample_tokens

    def sample(logits, temperature, top_p, uniform):
        logits = np.asarray(logits, dtype=np.float64)
        T = np.asarray(temperature, dtype=np.float64).reshape(-1)
        if kind == "temperature_multiplies":
            return orig(logits * T[:, None] * T[:, None], temperature, top_p, uniform)
        if kind == "draw_in_probability_order":
            # same nucleus, but the draw walks it from the most probable token down
            r = orig(logits, temperature, top_p, uniform)
            out = r.tokens.copy()
            for b in range(len(out)):
                if not T[b] > 0:
                    continue
                z = logits[b] / T[b]
                q = np.exp(z - z.max())
                q /= q.sum()
                order = np.argsort(-q, kind="stable")[: int(r.nucleus_size[b])]
                F = np.cumsum(q[order]) / q[order].sum()
                j = min(int(np.searchsorted(F, float(np.asarray(uniform).reshape(-1)[b]),
                                            side="right")), len(order) - 1)
                out[b] = order[j]
            return bo.SampleResult(out, r.keep_margin, r.draw_margin, r.nucleus_size)
        if kind == "boundary_token_dropped":
            # the nucleus stops before the token that makes its mass reach top_p
            P = np.asarray(top_p, dtype=np.float64).reshape(-1)
            U = np.asarray(uniform, dtype=np.float64).reshape(-1)
            r = orig(logits, temperature, top_p, uniform)
            out = r.tokens.copy()
            size = r.nucleus_size.copy()
            for b in range(len(out)):
                if not T[b] > 0 or P[b] >= 1:
                    continue
                z = logits[b] / T[b]
                q = np.exp(z - z.max())
                q /= q.sum()
                last = np.sort(q)[::-1][int(r.nucleus_size[b]) - 1]
                keep = q > last
                if not keep.any():
                    keep = q >= q.max()
                idx = np.nonzero(keep)[0]
                F = np.cumsum(q[idx]) / q[idx].sum()
                out[b] = idx[min(int(np.searchsorted(F, U[b], side="right")), len(idx) - 1)]
                size[b] = len(idx)
            return bo.SampleResult(out, r.keep_margin, r.draw_margin, size)
        raise ValueError(kind)
    return sample


PINS = [test_hand_worked_four_tokens, test_ties_at_the_boundary_are_all_kept,
        test_nucleus_is_the_smallest_set_reaching_top_p_brute_force,
        test_temperature_is_a_logit_scale]


def _frequency_pin():
    test_draw_frequencies_on_a_uniform_grid(0.7, 0.8)


@pytest.mark.parametrize("kind", ["temperature_multiplies", "draw_in_probability_order",
                                  "boundary_token_dropped"])
def test_planted_sampler_mistakes_fail_a_pin(kind, monkeypatch):
    monkeypatch.setattr(oracle, "sample_tokens", _mutant(kind))
    caught = 0
    for pin in PINS + [_frequency_pin]:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin caught the planted mistake {kind}"
