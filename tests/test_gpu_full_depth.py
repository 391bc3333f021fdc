"""Full depth of the 176B tensor-parallel rank-0 share (70 layers, hidden 14336, 14 of
112 heads; the workload bench.py times at batch 1).

1. Parity with the oracle, teacher-forced: the prompt pass and 3 decode steps of the
   GPU against one causal oracle pass over the prompt and the GPU's tokens (teacher
   forcing fixes every input token, so the KV-cached steps equal that pass, pinned by
   test_incremental_decode_equals_full_rerun).  The oracle does not hold the 70 layers
   at once (about 86 GB in float64): it regenerates and widens one layer at a time.
   * float32 activations: hidden rel-L2 <= 1e-2, the spec gate, and <= 1e-3 (the
     bf16-pair operands keep every activation to 2^-17; the float64 oracle with
     float32-rounded activations is 5e-7 from the exact one at 70 layers).
   * fp16 activations and KV cache: <= 1e-2 (the float64 oracle with fp16-rounded
     activations and KV is 3.0e-3 from the exact one at 70 layers), also with the
     LayerNorms of the decode steps folded into the QKV / MLP-up GEMVs (bloom_ln_fold,
     the benchmarked configuration).
   * bf16 activations do not meet 1e-2 at this depth: the float64 oracle with its
     activations rounded to bf16 at the same points is itself 2.5e-2 from the exact
     oracle (attention scores spread ~6 with these weights, so a rounding of q or k
     moves the softmax by ~1%, and the stack amplifies it).  That run is kept as a
     regression check against the bf16-activation oracle: no further than 1.25x its
     distance (two computations that round at the same points, in different order,
     are statistically equally far from the exact result), with every id by the
     teacher-forced near-tie rule.
2. Self-invariants of the path at full depth (float32 activations):
   * the decode step at position P + t equals a prompt pass over the (P + t + 1)-token
     prefix (vector-ALU GEMV steps against the MFMA prompt pass), within 1e-3;
   * a KV cache saved after some steps and restored later reproduces the continuation
     bit for bit (tokens and final-LayerNorm states).
"""
import dataclasses
import sys
import time

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb

pytestmark = pytest.mark.gpu

M_SHARE = bi.BLOOM_176B_TP8_RANK0
P = 16


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def share_weights():
    """The 70-layer share's weights in HBM, generated on the GPU (bitwise equal to the
    host generator, test_gpu_boundary.py); shared by every test of this module."""
    m = M_SHARE
    dt = {"bf16": torch.int16}
    g = {n: torch.empty(bi.tensor_shape(m, n), dtype=torch.int16, device="cuda")
         for n in bi.global_field_names(m)}
    layers = [{f: torch.empty(bi.tensor_shape(m, f), dtype=dt["bf16"], device="cuda")
               for f in bi.layer_field_names(m)} for _ in range(m.n_layer)]
    dw = tb.DeviceWeights(g, layers)
    tb.bloom_init_weights(tb.make_config(m), dw, seed=0)
    torch.cuda.synchronize()
    yield dw
    del dw, g, layers
    torch.cuda.empty_cache()


def _generate(dw, act, n_new, want_graph=False):
    m = dataclasses.replace(M_SHARE, activations=act)
    cfg = tb.make_config(m)
    prompt, valid = bi.prompts(m, 1, P)
    kv = tb.KVCache(cfg, 1, P + n_new, fill=float("nan"))
    ws = tb.workspace(cfg, 1, P + n_new)
    tok = torch.from_numpy(prompt).cuda()
    vl = torch.from_numpy(valid).cuda()
    ids, hid = tb.greedy_generate(cfg, dw, kv, tok, vl, n_new, ws)
    torch.cuda.synchronize()
    return m, cfg, prompt, valid, kv, ws, ids.cpu().numpy().T.copy(), hid.cpu().numpy()


def _oracle_states(ids, n_new, rounded):
    """Final-LayerNorm states of positions P-1 .. P+n_new-2 from one causal pass over the
    prompt and the given tokens: exact, and (rounded=True) with bf16-rounded
    activations too."""
    m = M_SHARE
    prompt, valid = bi.prompts(m, 1, P)
    tokens = np.concatenate([prompt, ids[:, :n_new - 1]], axis=1)
    pad = P - np.asarray(valid, dtype=np.int64)
    glob = {n: bi.tensor(m, n) for n in bi.global_field_names(m)}
    om = oracle.OracleModel.from_storage(dataclasses.replace(m, n_layer=0),
                                         dict(glob, layers=[]))
    x = np.asarray(om.embed[tokens], dtype=np.float64)
    x = oracle.layer_norm(x, om.emb_ln[0], om.emb_ln[1], om.ln_eps)
    xr = x.copy() if rounded else None
    empty = np.zeros((1, m.n_head_local, 0, m.head_dim))
    t0 = time.perf_counter()
    for l in range(m.n_layer):
        lw = oracle.layer_from_storage(m, {f: bi.tensor(m, f, l) for f in bi.layer_field_names(m)})
        x = oracle.decoder_layer(om, lw, x, pad, 0, {"k": empty, "v": empty})
        if rounded:
            xr = oracle.decoder_layer(om, lw, xr, pad, 0, {"k": empty, "v": empty},
                                      act=oracle.round_bf16)
        if (l + 1) % 10 == 0:
            _log(f"oracle layer {l + 1}/{m.n_layer} ({time.perf_counter() - t0:.0f}s)")
    h = oracle.layer_norm(x, om.lnf[0], om.lnf[1], om.ln_eps)[0, P - 1:]
    hr = oracle.layer_norm(xr, om.lnf[0], om.lnf[1], om.ln_eps)[0, P - 1:] if rounded else None
    return om, h, hr


def _ids_ok(om, h, ids, n_new, tol):
    logits = oracle.lm_logits(om, h)
    top1 = logits.max(axis=-1)
    rms = np.sqrt(np.mean(logits ** 2, axis=-1))
    chosen = logits[np.arange(n_new), ids[0]]
    exact = ids[0] == oracle.greedy_argmax(logits)
    return bool(np.all(chosen >= top1 - 3 * tol * rms)), float(exact.mean())


def test_tp_share_176b_full_depth_parity(share_weights):
    n_new = 4
    *_, ids32, hid32 = _generate(share_weights, "f32", n_new)
    *_, idsh, hidh = _generate(share_weights, "f16", n_new)
    *_, ids16, hid16 = _generate(share_weights, "bf16", n_new)
    # fp16 with the LayerNorms of the decode steps folded into the QKV / MLP-up GEMVs
    # (the benchmarked configuration)
    share_weights.fold_layernorm(tb.make_config(dataclasses.replace(M_SHARE, activations="f16")))
    *_, idsf, hidf = _generate(share_weights, "f16", n_new)
    share_weights.unfold_layernorm()
    torch.cuda.empty_cache()
    assert np.array_equal(ids32, idsh) and np.array_equal(ids32, idsf)
    om, h, hr = _oracle_states(ids32, n_new, rounded=np.array_equal(ids32, ids16))
    rel32 = float(np.linalg.norm(hid32[:, 0] - h) / np.linalg.norm(h))
    ok32, ex32 = _ids_ok(om, h, ids32, n_new, 1e-2)
    relh = float(np.linalg.norm(hidh[:, 0] - h) / np.linalg.norm(h))
    okh, exh = _ids_ok(om, h, idsh, n_new, 1e-2)
    relf = float(np.linalg.norm(hidf[:, 0] - h) / np.linalg.norm(h))
    okf, exf = _ids_ok(om, h, idsf, n_new, 1e-2)
    if hr is None:   # the bf16 run chose other tokens: its own teacher-forced pass
        om, h, hr = _oracle_states(ids16, n_new, rounded=True)
    rel16 = float(np.linalg.norm(hid16[:, 0] - h) / np.linalg.norm(h))
    rel_ref = float(np.linalg.norm(hr - h) / np.linalg.norm(h))
    ok16, ex16 = _ids_ok(om, h, ids16, n_new, 1e-2)
    _log(f"176b share, 70 layers: float32 activations hidden rel {rel32:.2e} (exact ids "
         f"{ex32:.2f}); fp16 {relh:.2e} (exact ids {exh:.2f}), with folded LayerNorms "
         f"{relf:.2e} (exact ids {exf:.2f}); bf16 activations "
         f"{rel16:.2e} against the bf16-activation oracle's {rel_ref:.2e} (exact ids "
         f"{ex16:.2f})")
    assert rel32 <= 1e-2 and rel32 <= 1e-3 and ok32          # the gate, float32 activations
    assert relh <= 1e-2 and okh                               # the gate, fp16 activations
    assert relf <= 1e-2 and okf                               # the gate, folded LayerNorms
    assert rel16 <= 1.25 * rel_ref and ok16                   # bf16 activations: regression


def test_tp_share_176b_decode_step_equals_prompt_pass(share_weights):
    """The decode step that produced token t (t = 1..3; input ids[t-1] at position
    P + t - 1) against a prompt pass over the P + t tokens prompt + ids[0..t-1] (all
    real: the prompt is unpadded), compared on the final-LayerNorm state of that last
    position, and on the greedy token it gives."""
    n_new = 4
    m, cfg, prompt, valid, kv, ws, ids, hid = _generate(share_weights, "f32", n_new)
    assert int(valid[0]) == P
    worst, same = 0.0, 0
    for t in range(1, n_new):
        toks = np.concatenate([prompt, ids[:, :t]], axis=1).astype(np.int32)
        vl = torch.tensor([P + t], dtype=torch.int32, device="cuda")
        kv2 = tb.KVCache(cfg, 1, P + n_new)
        out = torch.empty((1, cfg.hidden), dtype=torch.float32, device="cuda")
        nxt = torch.empty(1, dtype=torch.int32, device="cuda")
        tb.bloom_prefill(cfg, share_weights, kv2, 1, P + t, torch.from_numpy(toks).cuda(),
                         vl, nxt, out, ws)
        torch.cuda.synchronize()
        ref = hid[t, 0]
        rel = float(np.linalg.norm(out.cpu().numpy()[0] - ref) / np.linalg.norm(ref))
        worst = max(worst, rel)
        same += int(int(nxt.item()) == int(ids[0, t]))
        del kv2
    _log(f"176b share, 70 layers: decode steps vs prompt passes over the prefix: max rel "
         f"{worst:.2e}, same greedy token {same}/{n_new - 1}")
    assert worst <= 1e-3


def test_tp_share_176b_kv_save_restore_reproduces_the_continuation(share_weights):
    n_new, t0 = 6, 3
    m = dataclasses.replace(M_SHARE, activations="f32")
    cfg = tb.make_config(m)
    prompt, valid = bi.prompts(m, 1, P)
    kv = tb.KVCache(cfg, 1, P + n_new)
    ws = tb.workspace(cfg, 1, P)
    tok = torch.from_numpy(prompt).cuda()
    vl = torch.from_numpy(valid).cuda()
    ids = torch.empty((n_new, 1), dtype=torch.int32, device="cuda")
    hid = torch.empty((n_new, 1, cfg.hidden), dtype=torch.float32, device="cuda")
    tb.bloom_prefill(cfg, share_weights, kv, 1, P, tok, vl, ids[0], hid[0], ws)
    for t in range(1, t0):
        tb.bloom_decode_step(cfg, share_weights, kv, 1, ids[t - 1], vl, ids[t], hid[t], ws)
    torch.cuda.synchronize()
    saved = (kv.k.clone(), kv.v.clone(), kv.struct.len, kv.struct.prompt_len)
    for t in range(t0, n_new):
        tb.bloom_decode_step(cfg, share_weights, kv, 1, ids[t - 1], vl, ids[t], hid[t], ws)
    torch.cuda.synchronize()
    ids_a, hid_a = ids.clone(), hid.clone()
    # something else uses the cache in between, then the saved state comes back
    kv.k.normal_(); kv.v.normal_()
    kv.k.copy_(saved[0]); kv.v.copy_(saved[1])
    kv.struct.len, kv.struct.prompt_len = saved[2], saved[3]
    for t in range(t0, n_new):
        tb.bloom_decode_step(cfg, share_weights, kv, 1, ids[t - 1], vl, ids[t], hid[t], ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_a)
    assert torch.equal(hid.view(torch.int32), hid_a.view(torch.int32))
