"""Parity of the float32- and fp16-activation paths (bloom_config.act_dtype =
BLOOM_F32 / BLOOM_F16: activations and KV cache in that type; the MFMA GEMM reads them
as two bf16 planes) against the CPU oracle, and greedy generation whose tokens change
from step to step.

Tolerance.  The path keeps every activation to within 2^-17 of its float32 value
(2^-24 where it is stored as float32), against 2^-9 for bf16 storage.  The float64
oracle with its activations rounded to bf16 is 8.5e-3 from the exact one after two
layers of the 176B share and 2.5e-2 after 70; rounded to float32 it is 1.6e-7 and
5e-7.  Scaled by the 2^8 ratio of the bf16-pair rounding to float32 rounding, that
is <= 1.3e-4 at any depth, so these tests require 1e-3 (the spec gate is
1e-2), and ids equal to the oracle's, free-running, where the oracle's top-2 logit
gap exceeds 1e-3 of the row's RMS.  fp16 storage rounds to 2^-11: the float64 oracle
with fp16-rounded activations and KV is 9.6e-4 from the exact one after two layers of
the 176B share and 3.0e-3 after 70, so fp16 runs are held to the 1e-2 gate.

Varied tokens.  With N(0, 0.02) weights each row repeats one token (the embedding
dominates the final state); with a larger init scale the attention and MLP branches
dominate and the greedy token changes from step to step, which exercises the
feedback of each step's token into the next.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
from gpu_util import compare, kv_numpy, run_gpu, upload

pytestmark = pytest.mark.gpu

TOL_F32ACT = 1e-3


def _free_running(m, T, prompt, valid, run, gap_frac=1e-3):
    """Oracle free-running; GPU ids must equal it at every step up to the first whose
    top-2 gap is within gap_frac of the row RMS (none in practice); returns the
    oracle result and the number of distinct tokens per row."""
    om = oracle.OracleModel.from_storage(m, T)
    res = oracle.greedy_generate(om, prompt, valid, run.ids.shape[1])
    gap = (res.top1 - res.top2) / res.rms          # [n_new, B]
    for b in range(prompt.shape[0]):
        close = np.nonzero(gap[:, b] <= gap_frac)[0]
        upto = close[0] + 1 if close.size else run.ids.shape[1]
        np.testing.assert_array_equal(run.ids[b, :upto], res.tokens[b, :upto])
    return res


@pytest.mark.parametrize("wdt, std, min_distinct", [("f32", 0.3, 8), ("bf16", 0.3, 8),
                                                     ("int8", 0.4, 4)])
def test_tiny_varied_tokens_free_running(wdt, std, min_distinct):
    """Tiny shape at a large init scale (oracle: 11-13 distinct greedy tokens per row in
    24 steps at 0.3 for float32 / bf16 weights, 4-6 at 0.4 for the int8 weights, which
    are drawn differently); float32 weights must match exactly, bf16 / int8 weights
    with float32 activations within TOL_F32ACT and the same free-running ids."""
    m = dataclasses.replace(bi.TINY, weight_dtype=wdt, init_std=std, activations="f32",
                            name=f"tiny-{wdt}-std{std}")
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, 2, 8, (8, 5))
    run = run_gpu(cfg, dw, prompt, valid, 24)
    res = _free_running(m, T, prompt, valid, run)
    rel = np.linalg.norm(run.hidden - res.hidden) / np.linalg.norm(res.hidden)
    distinct = [len(set(r)) for r in run.ids]
    print(f"tiny {wdt} std {std}: distinct tokens {distinct}, hidden rel {rel:.2e}")
    assert min(distinct) >= min_distinct
    assert rel <= (1e-5 if wdt == "f32" else TOL_F32ACT)


@pytest.mark.parametrize("B", [2, 6])
def test_tiny_varied_tokens_bf16_activations_teacher_forced(B):
    """bf16 weights and bf16 activations on the varied-token tiny model (init scale 0.3;
    the float64 oracle with its activations rounded to bf16 is 8.2e-3 from the exact
    one there): hidden rel <= 1e-2 and every id by the teacher-forced near-tie rule,
    with the near-tie count reported.  Batch 2 runs the vector-ALU GEMV, batch 6 the
    MFMA GEMM."""
    m = dataclasses.replace(bi.TINY, weight_dtype="bf16", init_std=0.3,
                            name="tiny-bf16-std0.3")
    T, dw, cfg = upload(m)
    valid = (8, 5, 8, 3, 8, 6)[:B]
    prompt, vl = bi.prompts(m, B, 8, valid)
    run = run_gpu(cfg, dw, prompt, vl, 24)
    v = compare(m, T, prompt, vl, run, 1e-2)
    distinct = [len(set(r)) for r in run.ids]
    print(f"tiny bf16 act bf16 std 0.3 B{B}: distinct {distinct}, hidden rel "
          f"{v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}, near-ties {v.near_ties}")
    assert sum(distinct) >= 4 * B         # the token stream changes from step to step
    assert v.hidden_rel <= 1e-2 and v.tokens_ok


@pytest.mark.parametrize("B", [2, 6])
def test_560m_varied_tokens_f32_activations(B):
    """BLOOM-560m width, 4 layers, init scale 0.08 (8-10 distinct tokens per row in 12
    steps; bf16 activations are 1.5e-2 from the oracle here, the float64 oracle with
    bf16-rounded activations 1.48e-2): float32 activations within TOL_F32ACT and
    free-running ids; batch 2 on the vector-ALU GEMV, batch 6 on the MFMA GEMM."""
    m = dataclasses.replace(bi.BLOOM_560M.truncated(4), init_std=0.08, activations="f32")
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, B, 16)
    run = run_gpu(cfg, dw, prompt, valid, 12)
    v = compare(m, T, prompt, valid, run, 1e-2, widen_embed=True)
    distinct = [len(set(r)) for r in run.ids]
    print(f"560m L4 std 0.08 act f32 B{B}: distinct {distinct}, hidden rel "
          f"{v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}, near-ties {v.near_ties}")
    assert sum(distinct) >= 4 * B
    assert v.hidden_rel <= TOL_F32ACT and v.tokens_ok
    _free_running(m, T, prompt, valid, run)


TOL = {"f32": TOL_F32ACT, "f16": 1e-2}


@pytest.mark.parametrize("act", ["f32", "f16"])
@pytest.mark.parametrize("batch, valid", [(1, None), (3, (16, 9, 2)), (8, None)])
def test_tp_share_176b_two_layers_precise_activations(batch, valid, act):
    m = dataclasses.replace(bi.BLOOM_176B_TP8_RANK0.truncated(2), activations=act)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16, valid)
    run = run_gpu(cfg, dw, prompt, vl, 4)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"176b share L2 act {act} B{batch}: hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= TOL[act] and v.tokens_ok
    # KV slots hold the keys / values in the activation type, unwritten slots NaN
    for layer in range(2):
        k, vv = kv_numpy(run.kv, layer)
        for got, ref in ((k, v.oracle.cache[layer]["k"]), (vv, v.oracle.cache[layer]["v"])):
            L = ref.shape[2]
            assert np.isnan(got[:batch, :, L:]).all()
            err = np.linalg.norm(got[:batch, :, :L] - ref) / np.linalg.norm(ref)
            assert err <= TOL[act], (layer, err)


@pytest.mark.parametrize("act", ["f32", "f16"])
@pytest.mark.parametrize("batch", [1, 16])
def test_full_176b_int8_two_layers_precise_activations(batch, act):
    m = dataclasses.replace(bi.BLOOM_176B_INT8.truncated(2), activations=act)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16)
    run = run_gpu(cfg, dw, prompt, vl, 3)
    del dw
    torch.cuda.empty_cache()
    v = compare(m, T, prompt, vl, run, 2e-2)
    print(f"176b int8 L2 act {act} B{batch}: hidden rel {v.hidden_rel:.2e}")
    assert v.hidden_rel <= TOL[act] and v.tokens_ok
