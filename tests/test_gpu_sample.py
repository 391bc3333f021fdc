"""Per-row sampling (bloom_sample_tokens) and the LM-head logits it samples from
(bloom_lm_logits) against the CPU oracle, through the C ABI.

Which token a nucleus draw picks is decided by sums over up to 250880 probabilities:
float32 (the kernel) and float64 (the oracle) agree on it unless the top_p boundary or
the drawn point u lies within rounding of an edge.  The oracle reports both distances
(in units of the normalised mass); rows where both exceed MARGIN must give the oracle's
token exactly, the others a token of the oracle's nucleus for top_p + MARGIN (every
token that rounding can put in), and enough rows must fall in the first group for the
test to mean something.  Greedy rows (temperature <= 0) are exact: an argmax of the
same float32 values.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb
from gpu_util import upload

pytestmark = pytest.mark.gpu

MARGIN = 2e-5   # float32 sums of <= 250880 terms: relative error well under 1e-6


def _gpu_sample(logits, T, P, u):
    B, V = logits.shape
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tb.bloom_sample_tokens(d(logits), B, V, d(T), d(P), d(u), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_rows(logits, T, P, u, min_exact_frac):
    got = _gpu_sample(logits, T, P, u)
    ref = oracle.sample_tokens(logits, T, P, u)
    clear = (ref.keep_margin > MARGIN) & (ref.draw_margin > MARGIN)
    assert clear.mean() >= min_exact_frac, f"only {clear.sum()} of {len(clear)} rows clear"
    bad = np.nonzero(clear & (got != ref.tokens))[0]
    assert bad.size == 0, (bad, got[bad], ref.tokens[bad], ref.keep_margin[bad],
                           ref.draw_margin[bad])
    for b in np.nonzero(~clear)[0]:
        wide = oracle.sample_tokens(logits[b:b + 1], T[b:b + 1],
                                    [min(1.0, float(P[b]) + MARGIN)], [0.5])
        q = np.exp((logits[b].astype(np.float64) - logits[b].max()) / max(float(T[b]), 1e-30))
        order = np.argsort(-q, kind="stable")
        kept = set(order[: int(wide.nucleus_size[0])].tolist())
        assert int(got[b]) in kept, (b, got[b])
    return got, ref, clear


def test_sampling_full_vocabulary_rows():
    logits, T, P, u = bi.sampling_inputs(48, 250880)
    got, ref, clear = _check_rows(logits, T, P, u, 0.4)
    print(f"\n{clear.sum()} of {len(clear)} rows compared exactly; nucleus sizes "
          f"{sorted(ref.nucleus_size.tolist())[:8]} ... {max(ref.nucleus_size)}")


def test_sampling_ragged_vocabularies_and_edges():
    for V in (1, 7, 1000, 1023, 1025, 4099):
        logits, T, P, u = bi.sampling_inputs(12, V, seed=9)
        # edge values of top_p and u on some rows
        P[0], P[1], P[2] = 1.0, 0.0, 1e-7
        u[3], u[4] = 0.0, np.float32(1.0 - 2 ** -24)
        # a positive temperature whose reciprocal overflows float32 is greedy
        T[5] = np.float32(1e-39)
        got, ref, _ = _check_rows(logits, T, P, u, 0.0)
        am = np.argmax(logits, axis=1)
        assert got[1] == am[1] and got[2] == am[2]     # only the largest logit kept
        assert got[5] == am[5] and ref.tokens[5] == am[5]
        assert np.all((got >= 0) & (got < V))


def test_greedy_rows_and_ties():
    V = 250880
    logits, T, P, u = bi.sampling_inputs(8, V, seed=5)
    T[:] = 0.0
    T[5] = -1.0
    mx = logits.max(axis=1)
    logits[2, 17] = mx[2] + 1.0        # a planted unique maximum at a low id
    logits[3, 1000] = mx[3] + 1.0      # a tie of two maxima: the lower id wins
    logits[3, 90000] = mx[3] + 1.0
    got = _gpu_sample(logits, T, P, u)
    np.testing.assert_array_equal(got, np.argmax(logits, axis=1))
    assert got[2] == 17 and got[3] == 1000


def test_sampling_is_deterministic_and_a_temperature_scale():
    logits, T, P, u = bi.sampling_inputs(16, 50000, seed=7)
    a = _gpu_sample(logits, T, P, u)
    b = _gpu_sample(logits, T, P, u)
    np.testing.assert_array_equal(a, b)
    # T = 2 on logits equals T = 1 on logits / 2 up to rounding of the scaled logits:
    # compare on the rows the oracle calls clear
    ref = oracle.sample_tokens(logits, np.full(16, 2.0), P, u)
    c = _gpu_sample(logits, np.full(16, 2.0, np.float32), P, u)
    d = _gpu_sample((logits / 2).astype(np.float32), np.ones(16, np.float32), P, u)
    clear = (ref.keep_margin > MARGIN) & (ref.draw_margin > MARGIN)
    np.testing.assert_array_equal(c[clear], d[clear])
    np.testing.assert_array_equal(c[clear], ref.tokens[clear])


def test_draw_frequencies_match_the_renormalised_nucleus():
    """Many draws of one row on a uniform grid of u: the token counts must follow the
    oracle's renormalised nucleus probabilities (within one grid step per token, plus
    the rows whose u sits within rounding of an interval edge)."""
    V, N = 64, 4096
    logits, T, P, u = bi.sampling_inputs(1, V, sigmas=(1.5,), seed=21)
    L = np.repeat(logits, N, 0)
    Ts = np.full(N, 0.9, np.float32)
    Ps = np.full(N, 0.85, np.float32)
    us = ((np.arange(N) + 0.5) / N).astype(np.float32)
    got = _gpu_sample(L, Ts, Ps, us)
    ref = oracle.sample_tokens(L, Ts, Ps, us)
    clear = ref.draw_margin > MARGIN
    np.testing.assert_array_equal(got[clear], ref.tokens[clear])
    counts = np.bincount(got, minlength=V) / N
    want = np.bincount(ref.tokens, minlength=V) / N
    assert np.max(np.abs(counts - want)) <= (np.sum(~clear) + 1) / N


@pytest.mark.parametrize("wdt", ["bf16", "int8"])
def test_lm_logits_reproduce_the_greedy_token(wdt):
    """bloom_lm_logits on the final-LayerNorm states that a decode step returns gives the
    logits its greedy LM head ranked: the argmax equals the step's token exactly, and the
    values match the oracle's LM head (float64) on the same bf16-rounded states."""
    shape = dataclasses.replace(bi.BLOOM_560M.truncated(2), weight_dtype=wdt)
    T, dw, cfg = upload(shape)
    B, P = 5, 16
    prompt, valid = bi.prompts(shape, B, P)
    kv = tb.KVCache(cfg, B, P + 2)
    ws = tb.workspace(cfg, B, P)
    tok = torch.from_numpy(prompt).cuda()
    vl = torch.from_numpy(valid).cuda()
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    hid = torch.empty(B, shape.hidden, dtype=torch.float32, device="cuda")
    tb.bloom_prefill(cfg, dw, kv, B, P, tok, vl, nxt, hid, ws)
    # one decode step with the LM head, one without it (hidden states only)
    nxt2 = torch.empty_like(nxt)
    hid2 = torch.empty_like(hid)
    tb.bloom_decode_step(cfg, dw, kv, B, nxt, vl, nxt2, hid2, ws)
    hid3 = torch.empty_like(hid)
    kv.struct.len -= 1
    tb.bloom_decode_step(cfg, dw, kv, B, nxt, vl, None, hid3, ws)
    logits = torch.empty(B, shape.vocab, dtype=torch.float32, device="cuda")
    tb.bloom_lm_logits(cfg, dw, B, hid2, logits, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(hid3.cpu().numpy(), hid2.cpu().numpy())
    lg = logits.cpu().numpy()
    np.testing.assert_array_equal(np.argmax(lg, axis=1), nxt2.cpu().numpy())
    om = oracle.OracleModel.from_storage(shape, T)
    h16 = oracle.round_bf16(hid2.cpu().numpy().astype(np.float64))
    ref = oracle.lm_logits(om, h16)
    rel = np.linalg.norm(lg - ref) / np.linalg.norm(ref)
    assert rel < 1e-5, rel
    # greedy rows of bloom_sample_tokens on these logits give the same tokens
    z = torch.zeros(B, dtype=torch.float32, device="cuda")
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    tb.bloom_sample_tokens(logits, B, shape.vocab, z, z + 1, z, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), nxt2.cpu().numpy())


def test_workspace_contents_need_no_initialisation():
    logits, T, P, u = bi.sampling_inputs(6, 250880, seed=13)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    n = tb.bloom_sample_workspace_bytes(6, 250880)
    outs = []
    for fill in (0, 255, 17):
        ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
        out = torch.empty(6, dtype=torch.int32, device="cuda")
        tb.bloom_sample_tokens(d(logits), 6, 250880, d(T), d(P), d(u), out, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])
