"""bloom_generate with per-row sampling (temperature, top-p, caller-supplied uniform
numbers) against the eager loop built from the same entry points (bloom_prefill /
bloom_decode_step without their LM head, bloom_lm_logits, bloom_sample_tokens) and,
teacher-forced, against the oracle's sampler on the oracle's own logits.

The graph replays run the same kernels on the same values as the eager loop, so the
tokens and final-LayerNorm states must agree bit for bit; greedy rows (temperature 0)
must give the tokens of plain greedy generation.  Against the oracle a step's token must
be the oracle's draw wherever both decision margins exceed MARGIN (see
test_gpu_sample.py), and a token of the oracle's widened nucleus elsewhere.
"""
import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb
from gpu_util import upload

pytestmark = pytest.mark.gpu

MARGIN = 2e-5


def _inputs(B, n_new, seed=31, T=(0.8, 0.0, 1.2, 0.6), P=(0.9, 1.0, 0.5, 1.0)):
    T = np.array(T[:B], dtype=np.float32)
    P = np.array(P[:B], dtype=np.float32)
    u = (bi.ids(seed, 3, (n_new, B), 0, 1 << 24).astype(np.float64) / (1 << 24)).astype(np.float32)
    return T, P, u


def _sampled_graph(cfg, dw, prompt, valid, n_new, T, P, u):
    B, Pl = prompt.shape
    kv = tb.KVCache(cfg, B, Pl + n_new, fill=float("nan"))
    ws = tb.workspace(cfg, B, Pl)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    ids = torch.empty((n_new, B), dtype=torch.int32, device="cuda")
    hid = torch.empty((n_new, B, cfg.hidden), dtype=torch.float32, device="cuda")
    tb.bloom_generate(cfg, dw, kv, B, Pl, d(prompt), d(valid), n_new, ids, hid, ws,
                      temperature=d(T), top_p=d(P), uniform=d(u))
    torch.cuda.synchronize()
    return ids.cpu().numpy(), hid.cpu().numpy()


def _sampled_eager(cfg, dw, prompt, valid, n_new, T, P, u):
    B, Pl = prompt.shape
    kv = tb.KVCache(cfg, B, Pl + n_new, fill=float("nan"))
    ws = tb.workspace(cfg, B, Pl)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    Td, Pd, ud = d(T), d(P), d(u)
    hid = torch.empty((B, cfg.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, cfg.vocab), dtype=torch.float32, device="cuda")
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    ids, hids = [], []
    vl = d(valid)
    tb.bloom_prefill(cfg, dw, kv, B, Pl, d(prompt), vl, None, hid, ws)
    for t in range(n_new):
        if t > 0:
            tb.bloom_decode_step(cfg, dw, kv, B, tok, vl, None, hid, ws)
        tb.bloom_lm_logits(cfg, dw, B, hid, logits, ws)
        tb.bloom_sample_tokens(logits, B, cfg.vocab, Td, Pd, ud[t], tok)
        ids.append(tok.cpu().numpy().copy())
        hids.append(hid.cpu().numpy().copy())
    return np.stack(ids), np.stack(hids)


def test_sampled_graph_loop_equals_eager_loop_and_greedy_rows():
    shape = bi.BLOOM_560M.truncated(2)
    _, dw, cfg = upload(shape)
    B, n_new = 3, 7
    prompt, valid = bi.prompts(shape, B, 16, (16, 11, 3))
    # random-weight models put most of the mass on one token; row 0 is made nearly
    # uniform (temperature 50, no truncation) so that its draws leave the greedy path
    T, P, u = _inputs(B, n_new, T=(50.0, 0.0, 1.2), P=(1.0, 1.0, 0.5))
    ids_g, hid_g = _sampled_graph(cfg, dw, prompt, valid, n_new, T, P, u)
    ids_e, hid_e = _sampled_eager(cfg, dw, prompt, valid, n_new, T, P, u)
    np.testing.assert_array_equal(ids_g, ids_e)
    np.testing.assert_array_equal(hid_g, hid_e)
    # the greedy row is plain greedy generation
    kv = tb.KVCache(cfg, B, 16 + n_new)
    ws = tb.workspace(cfg, B, 16)
    g_ids, _ = tb.greedy_generate(cfg, dw, kv, torch.from_numpy(prompt).cuda(),
                                  torch.from_numpy(valid).cuda(), n_new, ws, graph=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids_g[:, 1], g_ids.cpu().numpy()[:, 1])
    # the nearly uniform row did sample: its tokens leave the greedy path
    assert np.any(ids_g[:, 0] != g_ids.cpu().numpy()[:, 0])


def test_sampled_generation_matches_the_oracle_teacher_forced():
    """The float32 tiny model, whose logits match the oracle's to rounding, so the draws
    can be compared (the bf16 models' logits differ from float64 by their own tolerance,
    far more than a draw's margin)."""
    m = bi.TINY
    Tn, dw, cfg = upload(m, seed=2)
    B, n_new = 4, 12
    prompt, valid = bi.prompts(m, B, 8, (8, 5, 8, 2), seed=3)
    T, P, u = _inputs(B, n_new)
    ids, _ = _sampled_graph(cfg, dw, prompt, valid, n_new, T, P, u)
    om = oracle.OracleModel.from_storage(m, Tn)
    pad = 8 - valid.astype(np.int64)
    cache = oracle.new_cache(om, B)
    h = oracle.forward(om, prompt, 0, pad, cache)[:, -1]
    exact = 0
    for t in range(n_new):
        lg = oracle.lm_logits(om, h)
        ref = oracle.sample_tokens(lg, T, P, u[t])
        clear = (ref.keep_margin > MARGIN) & (ref.draw_margin > MARGIN)
        for b in range(B):
            if clear[b]:
                assert ids[t, b] == ref.tokens[b], (t, b, ids[t, b], ref.tokens[b])
                exact += 1
            else:
                wide = oracle.sample_tokens(lg[b:b + 1], T[b:b + 1],
                                            [min(1.0, float(P[b]) + MARGIN)], [0.5])
                q = lg[b] / max(float(T[b]), 1e-30)
                order = np.argsort(-q, kind="stable")
                assert ids[t, b] in set(order[: int(wide.nucleus_size[0])].tolist())
        if t + 1 < n_new:
            h = oracle.forward(om, ids[t][:, None].astype(np.int32), 8 + t, pad, cache)[:, 0]
    assert exact >= 0.75 * B * n_new, exact


def test_sampled_generation_with_end_token_and_row_limits():
    """The stop rule applies to sampled tokens as to greedy ones: each row's ids equal
    the unconstrained sampled run's up to its end (its end token, or its token limit),
    then the pad id; token counts are reported."""
    shape = bi.BLOOM_560M.truncated(2)
    _, dw, cfg = upload(shape)
    B, n_new = 3, 8
    prompt, valid = bi.prompts(shape, B, 16, (16, 9, 12))
    T, P, u = _inputs(B, n_new, T=(50.0, 40.0, 0.0), P=(1.0, 0.95, 1.0))
    free, _ = _sampled_graph(cfg, dw, prompt, valid, n_new, T, P, u)
    eos = int(free[3, 0])                      # row 0 ends at step 3 (or earlier)
    max_new = np.array([n_new, 5, n_new], dtype=np.int32)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv = tb.KVCache(cfg, B, 16 + n_new)
    ws = tb.workspace(cfg, B, 16)
    ids = torch.empty((n_new, B), dtype=torch.int32, device="cuda")
    out_len = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    tb.bloom_generate(cfg, dw, kv, B, 16, d(prompt), d(valid), n_new, ids, None, ws,
                      eos_id=eos, pad_id=3, max_new=d(max_new), out_len=out_len,
                      temperature=d(T), top_p=d(P), uniform=d(u))
    torch.cuda.synchronize()
    want, lengths = oracle.stop_rule(free.T, eos, max_new, 3)
    np.testing.assert_array_equal(ids.cpu().numpy().T, want)
    np.testing.assert_array_equal(out_len.cpu().numpy(), lengths)
