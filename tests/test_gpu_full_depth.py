"""Full-depth parity of the 176B tensor-parallel rank-0 share (70 layers, the workload
bench.py times at batch 1): the HIP path's prompt pass and first decode steps against
the oracle, teacher-forced.

The oracle does not hold the 70 layers at once (≈ 86 GB in float64).  Teacher forcing
fixes every input token, so the KV-cached steps equal one causal pass over the prompt
followed by the GPU's tokens; the oracle runs that pass layer by layer, regenerating
and widening one layer's weights at a time, and compares the final-LayerNorm states of
the prompt's last position and of each decode step.

Tolerance at this depth.  The 1e-2 hidden-state gate is met on the 2-layer truncations
(test_gpu_model.py).  Over 70 layers of these random N(0, 0.02) weights the stack
amplifies rounding: attention scores have a spread of ≈ 6, so a bf16 rounding of q / k
moves the softmax by ≈ 1%, and two computations that differ only in rounding drift
apart layer after layer.  The oracle run a second time with the activations the path
stores in bf16 rounded to bf16 (oracle.round_bf16 at LN outputs, new K/V, attention and
GeLU outputs) is itself 2.5e-2 from the exact oracle at 70 layers.  The test therefore
requires the GPU to be no further from the exact oracle than 1.5x that bf16-activation
reference (and never beyond 5e-2), and every greedy id to pass the teacher-forced rule
of the other parity tests (oracle logit within 3 * 1e-2 * RMS(row) of the best).
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
from gpu_util import run_gpu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def test_tp_share_176b_full_depth_teacher_forced():
    m = bi.BLOOM_176B_TP8_RANK0
    n_new, tol = 4, 1e-2
    t0 = time.perf_counter()
    g = {name: tb.to_device(bi.tensor(m, name)) for name in bi.global_field_names(m)}
    layers = [{f: tb.to_device(bi.tensor(m, f, l)) for f in bi.layer_field_names(m)}
              for l in range(m.n_layer)]
    dw, cfg = tb.DeviceWeights(g, layers), tb.make_config(m)
    _log(f"uploaded {m.n_layer} layers ({time.perf_counter() - t0:.0f}s)")
    prompt, valid = bi.prompts(m, 1, 16)
    run = run_gpu(cfg, dw, prompt, valid, n_new)
    del dw, layers, g
    torch.cuda.empty_cache()

    P = prompt.shape[1]
    tokens = np.concatenate([prompt, run.ids[:, :n_new - 1]], axis=1)   # [1, P + n_new - 1]
    pad = P - np.asarray(valid, dtype=np.int64)
    glob = {name: bi.tensor(m, name) for name in bi.global_field_names(m)}
    om = oracle.OracleModel.from_storage(dataclasses.replace(m, n_layer=0),
                                         dict(glob, layers=[]))
    x = np.asarray(om.embed[tokens], dtype=np.float64)
    if om.embed_ln:
        x = oracle.layer_norm(x, om.emb_ln[0], om.emb_ln[1], om.ln_eps)
    xr = x.copy()
    empty = np.zeros((1, m.n_head_local, 0, m.head_dim))
    for l in range(m.n_layer):
        lw = oracle.layer_from_storage(m, {f: bi.tensor(m, f, l) for f in bi.layer_field_names(m)})
        x = oracle.decoder_layer(om, lw, x, pad, 0, {"k": empty, "v": empty})
        xr = oracle.decoder_layer(om, lw, xr, pad, 0, {"k": empty, "v": empty},
                                  act=oracle.round_bf16)
        if (l + 1) % 10 == 0:
            _log(f"oracle layer {l + 1}/{m.n_layer} ({time.perf_counter() - t0:.0f}s)")
    h = oracle.layer_norm(x, om.lnf[0], om.lnf[1], om.ln_eps)[0, P - 1:]   # [n_new, hidden]
    hr = oracle.layer_norm(xr, om.lnf[0], om.lnf[1], om.ln_eps)[0, P - 1:]
    got = run.hidden[:, 0]
    rel = float(np.linalg.norm(got - h) / np.linalg.norm(h))
    rel_ref = float(np.linalg.norm(hr - h) / np.linalg.norm(h))
    logits = oracle.lm_logits(om, h)                                       # [n_new, vocab]
    top1 = logits.max(axis=-1)
    rms = np.sqrt(np.mean(logits ** 2, axis=-1))
    chosen = logits[np.arange(n_new), run.ids[0]]
    exact = run.ids[0] == oracle.greedy_argmax(logits)
    _log(f"176b share, 70 layers: hidden rel {rel:.2e} (bf16-activation oracle {rel_ref:.2e}), "
         f"exact ids {exact.mean():.2f} ({time.perf_counter() - t0:.0f}s)")
    assert rel <= min(1.5 * rel_ref, 5e-2)
    assert np.all(chosen >= top1 - 3 * tol * rms)
