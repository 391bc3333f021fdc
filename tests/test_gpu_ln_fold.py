"""The LayerNorm fold of one-row passes (bloom_ln_fold; include/bloom.h): with the fold
vectors c_n = sum_k W[n][k] g_k and d_n = sum_k W[n][k] b_k + bias_n, the QKV and MLP-up
GEMVs of a batch-1 decode step read g * x (stored by the residual epilogue of the
previous projection, whose blocks also add their sums of x and x^2 to integer
accumulators) and finish rstd (acc - mean c_n) + d_n, and the separate LayerNorm
launches go away ("DeepSpeed Inference ...", Section III.D fuses each LayerNorm with the
GeMM that follows it).

* The fold vectors equal float64 sums of the stored weights (float32 rounding).
* Batch 1 at the 176B share's width (hidden 14336), 2 layers, fp16, bf16 and float32
  activations: against the oracle within the same bound as the unfolded path (1e-2),
  greedy ids by the teacher-forced rule, and close to the unfolded run (the two round
  different values to the activation type: g * x here, the LayerNorm output there).
* Graph replays equal the eager loop bit for bit (the accumulated sums do not depend on
  the order in which blocks add them); where the fold does not apply (batch 2, or hidden
  <= 4096, where the LayerNorm already runs inside the GEMV) a folded weight set gives
  the unfolded results bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb
from gpu_util import compare, run_gpu, upload

pytestmark = pytest.mark.gpu

M2 = bi.BLOOM_176B_TP8_RANK0.truncated(2)


def test_fold_vectors_equal_float64_sums():
    T, dw, cfg = upload(M2)
    dw.fold_layernorm(cfg)
    torch.cuda.synchronize()
    fold = dw.fold.cpu().numpy().astype(np.float64)
    hd3 = 3 * M2.n_head_local * M2.head_dim
    F = M2.ffn
    per = 2 * (hd3 + F)
    assert fold.size == M2.n_layer * per

    for l in range(M2.n_layer):
        lw = oracle.layer_from_storage(M2, T["layers"][l])
        for (w, b, (g, beta), off, n) in ((lw["qkv"], lw["b_qkv"], lw["ln1"], 0, hd3),
                                          (lw["up"], lw["b_up"], lw["ln2"], 2 * hd3, F)):
            c_ref = w @ g
            d_ref = w @ beta + b
            c = fold[l * per + off: l * per + off + n]
            d = fold[l * per + off + n: l * per + off + 2 * n]
            # one float32 rounding of a float64 sum (summation order: ~1e-16 of the
            # terms' magnitudes)
            tc = 2.0 ** -22 * np.abs(c_ref) + 1e-12 * (np.abs(w) @ np.abs(g))
            td = 2.0 ** -22 * np.abs(d_ref) + 1e-12 * (np.abs(w) @ np.abs(beta) + np.abs(b))
            assert np.all(np.abs(c - c_ref) <= tc) and np.all(np.abs(d - d_ref) <= td)
            print(f"layer {l} fold {n} rows: max |c - c_ref| / tol "
                  f"{np.max(np.abs(c - c_ref) / tc):.2f}")


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
def test_fold_batch1_two_layers_matches_oracle(act):
    m = dataclasses.replace(M2, activations=act)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, 1, 16)
    plain = run_gpu(cfg, dw, prompt, vl, 6)
    dw.fold_layernorm(cfg)
    run = run_gpu(cfg, dw, prompt, vl, 6)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    vp = compare(m, T, prompt, vl, plain, 1e-2, widen_embed=True)
    diff = float(np.linalg.norm(run.hidden - plain.hidden) / np.linalg.norm(plain.hidden))
    print(f"176b share L2 B1 act {act}: folded hidden rel {v.hidden_rel:.2e} (exact ids "
          f"{v.exact_frac:.3f}), unfolded {vp.hidden_rel:.2e}, folded vs unfolded {diff:.2e}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    # the prompt pass (16 rows) is not folded: the first token's state is shared
    assert np.array_equal(run.hidden[0], plain.hidden[0])
    # two paths that round at different points, each about as far from the exact result
    assert diff <= 2.5 * max(vp.hidden_rel, v.hidden_rel)


def test_fold_graph_loop_equals_eager():
    m = dataclasses.replace(M2, activations="f16")
    T, dw, cfg = upload(m)
    dw.fold_layernorm(cfg)
    prompt, valid = bi.prompts(m, 1, 16)
    tok = torch.from_numpy(prompt.astype(np.int32)).cuda()
    vl = torch.from_numpy(np.asarray(valid, dtype=np.int32)).cuda()
    outs = []
    for graph in (False, True):
        kv = tb.KVCache(cfg, 1, 16 + 8, fill=float("nan"))
        ws = tb.workspace(cfg, 1, 16)
        ids, hid = tb.greedy_generate(cfg, dw, kv, tok, vl, 8, ws, graph=graph)
        torch.cuda.synchronize()
        outs.append((ids.cpu(), hid.cpu()))
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1].view(torch.int32), outs[1][1].view(torch.int32))


@pytest.mark.parametrize("shape, batch", [(M2, 2), (bi.BLOOM_560M.truncated(2), 1)])
def test_fold_not_applied_gives_unfolded_results(shape, batch):
    """Batch 2 (two activation rows) and hidden 1024 (the LayerNorm already runs as the
    GEMV prologue) do not fold: the same bits with and without the fold vectors."""
    m = dataclasses.replace(shape, activations="f16")
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16)
    plain = run_gpu(cfg, dw, prompt, vl, 4)
    dw.fold_layernorm(cfg)
    run = run_gpu(cfg, dw, prompt, vl, 4)
    assert np.array_equal(run.ids, plain.ids)
    assert np.array_equal(run.hidden.view(np.uint32), plain.hidden.view(np.uint32))
