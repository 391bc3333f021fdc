"""bloom_generate (the prompt pass, one eager decode step, then replays of one captured
decode step) against the eager bloom_prefill + bloom_decode_step loop and the oracle.

The graph replays run the same kernels on the same inputs as the eager loop, so ids,
final-LayerNorm states and the KV cache must agree bit for bit; the oracle checks the
result to the usual gates.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb
from gpu_util import compare, upload

pytestmark = pytest.mark.gpu


def _run(cfg, dw, prompt, valid, n_new, graph, max_len=None, want_hidden=True):
    B, P = prompt.shape
    kv = tb.KVCache(cfg, B, max_len or (P + n_new), fill=float("nan"))
    ws = tb.workspace(cfg, B, P)
    tok = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    vl = torch.from_numpy(np.ascontiguousarray(valid, dtype=np.int32)).cuda()
    ids, hid = tb.greedy_generate(cfg, dw, kv, tok, vl, n_new, ws, want_hidden=want_hidden,
                                  graph=graph)
    torch.cuda.synchronize()
    return (ids.cpu().numpy().T.copy(), None if hid is None else hid.cpu().numpy(), kv)


def _same(a, b):
    ia, ha, ka = a
    ib, hb, kb = b
    np.testing.assert_array_equal(ia, ib)
    if ha is not None:
        assert np.array_equal(ha.view(np.uint32), hb.view(np.uint32))
    assert ka.len == kb.len and ka.prompt_len == kb.prompt_len
    for x, y in ((ka.k, kb.k), (ka.v, kb.v)):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def test_tiny_fp32_graph_matches_oracle_exactly():
    w = bi.WORKLOADS["tiny"]
    m = w.model
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, 2, w.prompt_len, w.valid_lens)
    g = _run(cfg, dw, prompt, valid, w.new_tokens, graph=True)
    res = oracle.greedy_generate(oracle.OracleModel.from_storage(m, T), prompt, valid,
                                 w.new_tokens)
    np.testing.assert_array_equal(g[0], res.tokens)
    rel = np.linalg.norm(g[1] - res.hidden) / np.linalg.norm(res.hidden)
    assert rel <= 1e-5
    _same(g, _run(cfg, dw, prompt, valid, w.new_tokens, graph=False))


@pytest.mark.parametrize("n_new", [1, 2, 3, 40])
def test_bloom560m_graph_equals_eager_bitwise(n_new):
    m = bi.BLOOM_560M.truncated(4)
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, 3, 16, (16, 9, 2))
    g = _run(cfg, dw, prompt, valid, n_new, graph=True, max_len=64)
    e = _run(cfg, dw, prompt, valid, n_new, graph=False, max_len=64)
    _same(g, e)
    assert np.isnan(g[2].k[:, :3, :, 16 + n_new - 1:].float().cpu().numpy()).all()


def test_graph_without_hidden_and_consecutive_calls():
    """Two bloom_generate calls in a row on one workspace, the second with a smaller
    batch and prompt, and without hidden output: each equals its eager loop."""
    m = bi.BLOOM_560M.truncated(3)
    T, dw, cfg = upload(m, seed=5)
    p1, v1 = bi.prompts(m, 8, 16, None, seed=6)
    p2, v2 = bi.prompts(m, 2, 7, (7, 3), seed=7)
    kv1 = tb.KVCache(cfg, 8, 16 + 24)
    ws = tb.workspace(cfg, 8, 16)
    out = []
    for (p, v, n), kv in (((p1, v1, 25), kv1), ((p2, v2, 11), tb.KVCache(cfg, 8, 40))):
        tok = torch.from_numpy(p.astype(np.int32)).cuda()
        vl = torch.from_numpy(np.asarray(v, dtype=np.int32)).cuda()
        ids, _ = tb.greedy_generate(cfg, dw, kv, tok, vl, n, ws, want_hidden=False, graph=True)
        torch.cuda.synchronize()
        out.append(ids.cpu().numpy().T.copy())
    for got, (p, v, n) in zip(out, ((p1, v1, 25), (p2, v2, 11))):
        e = _run(cfg, dw, p, v, n, graph=False, want_hidden=False)
        np.testing.assert_array_equal(got, e[0])


def test_tp_share_176b_graph_two_layers_oracle():
    m = bi.BLOOM_176B_TP8_RANK0.truncated(2)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, 1, 16)
    g = _run(cfg, dw, prompt, vl, 6, graph=True)
    from gpu_util import GpuRun
    v = compare(m, T, prompt, vl, GpuRun(g[0], g[1], g[2], cfg), 1e-2, widen_embed=True)
    print(f"176b rank-0 share L2 B1 graph: hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    _same(g, _run(cfg, dw, prompt, vl, 6, graph=False))


def test_dynamic_batch_extraction_compacts_kv_cache():
    """Four rows decode together; two of them are extracted after 5 tokens
    (kv_cache_compact keeps rows 0 and 2) and the other two go on alone as a batch of 2.
    The compacted cache holds the kept rows' slots bit for bit, and the kept rows' whole
    generation matches the oracle."""
    m = bi.BLOOM_560M.truncated(3)
    T, dw, cfg = upload(m, seed=71)
    B, P, n1, n2 = 4, 12, 5, 6
    prompt, valid = bi.prompts(m, B, P, (12, 7, 12, 3), seed=72)
    kv = tb.KVCache(cfg, B, P + n1 + n2, fill=float("nan"))
    ws = tb.workspace(cfg, B, P)
    tok = torch.from_numpy(prompt.astype(np.int32)).cuda()
    vl = torch.from_numpy(np.asarray(valid, dtype=np.int32)).cuda()
    ids1 = torch.empty((n1, B), dtype=torch.int32, device="cuda")
    hid1 = torch.empty((n1, B, m.hidden), dtype=torch.float32, device="cuda")
    tb.bloom_prefill(cfg, dw, kv, B, P, tok, vl, ids1[0], hid1[0], ws)
    for t in range(1, n1):
        tb.bloom_decode_step(cfg, dw, kv, B, ids1[t - 1], vl, ids1[t], hid1[t], ws)
    keep = [0, 2]
    L = kv.len
    k_before, v_before = kv.k.clone(), kv.v.clone()
    tb.kv_cache_compact(cfg, kv, B, keep)
    torch.cuda.synchronize()
    for new, old in ((kv.k, k_before), (kv.v, v_before)):
        for i, r in enumerate(keep):
            assert torch.equal(new[:, i, :, :L].view(torch.int16),
                               old[:, r, :, :L].view(torch.int16))
    assert kv.len == L
    vl2 = vl[keep].contiguous()
    cur = ids1[n1 - 1, keep].contiguous()
    ids2 = torch.empty((n2, 2), dtype=torch.int32, device="cuda")
    hid2 = torch.empty((n2, 2, m.hidden), dtype=torch.float32, device="cuda")
    for t in range(n2):
        tb.bloom_decode_step(cfg, dw, kv, 2, cur if t == 0 else ids2[t - 1], vl2, ids2[t],
                             hid2[t], ws)
    torch.cuda.synchronize()
    ids = np.concatenate([ids1.cpu().numpy()[:, keep], ids2.cpu().numpy()], axis=0).T.copy()
    hid = np.concatenate([hid1.cpu().numpy()[:, keep], hid2.cpu().numpy()], axis=0)
    from gpu_util import GpuRun
    v = compare(m, T, prompt[keep], np.asarray(valid)[keep], GpuRun(ids, hid, kv, cfg), 1e-2,
                widen_embed=True)
    print(f"extraction 4 -> 2 rows: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    assert kv.len == P + n1 + n2 - 1


def test_generation_control_eos_and_row_limits():
    """bloom_generate with an end token and per-row limits: each row's tokens are those
    of plain greedy generation up to its end (its own end token kept, or its limit),
    pad after; the token counts are reported; the hidden states (pad-fed after a row's
    end) match the oracle teacher-forced on the same tokens."""
    m = bi.BLOOM_560M.truncated(3)
    T, dw, cfg = upload(m, seed=81)
    B, P, n_new, pad = 3, 10, 14, 3
    prompt, valid = bi.prompts(m, B, P, (10, 6, 10), seed=82)
    base = _run(cfg, dw, prompt, valid, n_new, graph=True)[0]            # [B, n_new]
    # greedy decoding of this random-weight model repeats one token per row, so the end
    # token is row 2's (row 2 ends on its first token), row 1 ends on its limit of 6
    # tokens and row 0 runs to n_new (the rule's mid-sequence cases are pinned on the
    # CPU, test_stop_rule_hand_worked)
    eos = int(base[2, 0])
    assert eos not in base[:2]
    max_new = np.array([n_new, 6, n_new], dtype=np.int32)
    expected, lengths = oracle.stop_rule(base, eos, max_new, pad)

    kv = tb.KVCache(cfg, B, P + n_new, fill=float("nan"))
    ws = tb.workspace(cfg, B, P)
    tok = torch.from_numpy(prompt.astype(np.int32)).cuda()
    vl = torch.from_numpy(np.asarray(valid, dtype=np.int32)).cuda()
    ids = torch.empty((n_new, B), dtype=torch.int32, device="cuda")
    hid = torch.empty((n_new, B, m.hidden), dtype=torch.float32, device="cuda")
    out_len = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    tb.bloom_generate(cfg, dw, kv, B, P, tok, vl, n_new, ids, hid, ws, eos_id=eos, pad_id=pad,
                      max_new=torch.from_numpy(max_new).cuda(), out_len=out_len)
    got = ids.cpu().numpy().T
    np.testing.assert_array_equal(got, expected)
    np.testing.assert_array_equal(out_len.cpu().numpy(), lengths)
    assert kv.len == P + n_new - 1

    om = oracle.OracleModel.from_storage(m, T)
    om.embed = np.asarray(om.embed, dtype=np.float64)
    res = oracle.greedy_generate(om, prompt, valid, n_new, forced=got)
    h = hid.cpu().numpy()
    rel = float(np.linalg.norm(h - res.hidden) / np.linalg.norm(res.hidden))
    print(f"generation control: ends {lengths.tolist()}, hidden rel {rel:.2e}")
    assert rel <= 1e-2
    for b in range(B):
        for t in range(int(lengths[b])):
            assert res.chosen[t, b] >= res.top1[t, b] - 3e-2 * res.rms[t, b]
