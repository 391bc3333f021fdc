"""GPU parity of the whole greedy-decode path (bloom_prefill + bloom_decode_step)
against the CPU oracle, on the pages' workload shapes.

Gates (float32 model: exact; bf16 weights: hidden rel-L2 <= 1e-2; int8 weights:
<= 2e-2), greedy ids by the teacher-forced rule in gpu_util, and KV-cache indexing
checked bit-exactly against a NaN sentinel: every slot below the cache length holds
the oracle's key/value, every slot above it is still the sentinel.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
from gpu_util import compare, kv_numpy, run_gpu, upload

pytestmark = pytest.mark.gpu


def _kv_check(run, res, B, length, rtol):
    H = run.cfg.n_head_local
    for layer in range(run.cfg.n_layer):
        k, v = kv_numpy(run.kv, layer)
        ok, ov = res.cache[layer]["k"], res.cache[layer]["v"]
        assert ok.shape[2] == length
        for got, ref in ((k, ok), (v, ov)):
            assert not np.isnan(got[:B, :, :length]).any()
            assert np.isnan(got[:B, :, length:]).all()          # untouched slots
            err = np.linalg.norm(got[:B, :, :length] - ref) / np.linalg.norm(ref)
            assert err <= rtol, (layer, err)
    assert run.kv.len == length


def test_tiny_fp32_matches_oracle_exactly_free_running():
    w = bi.WORKLOADS["tiny"]
    m = w.model
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, 2, w.prompt_len, w.valid_lens)
    run = run_gpu(cfg, dw, prompt, valid, w.new_tokens)
    om = oracle.OracleModel.from_storage(m, T)
    res = oracle.greedy_generate(om, prompt, valid, w.new_tokens)
    np.testing.assert_array_equal(run.ids, res.tokens)
    rel = np.linalg.norm(run.hidden - res.hidden) / np.linalg.norm(res.hidden)
    print(f"tiny fp32: ids equal, hidden rel {rel:.2e}")
    assert rel <= 1e-5
    _kv_check(run, res, 2, w.prompt_len + w.new_tokens - 1, 1e-5)
    assert run.kv.prompt_len == w.prompt_len


@pytest.mark.parametrize("wdt, tol", [("bf16", 1e-2), ("int8", 2e-2)])
def test_tiny_shape_low_precision(wdt, tol):
    m = dataclasses.replace(bi.TINY, weight_dtype=wdt)
    T, dw, cfg = upload(m, seed=3)
    prompt, valid = bi.prompts(m, 3, 8, (8, 5, 1), seed=4)
    run = run_gpu(cfg, dw, prompt, valid, 12)
    v = compare(m, T, prompt, valid, run, tol)
    print(f"tiny {wdt}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= tol and v.tokens_ok
    _kv_check(run, v.oracle, 3, 8 + 11, 2 * tol)


@pytest.mark.parametrize("valid", [(16, 11, 3), (16, 7), (5,)])
def test_bloom560m_truncated_ragged_batch(valid):
    m = bi.BLOOM_560M.truncated(4)
    T, dw, cfg = upload(m)
    B = len(valid)
    prompt, valid = bi.prompts(m, B, 16, valid)
    run = run_gpu(cfg, dw, prompt, valid, 12)
    v = compare(m, T, prompt, valid, run, 1e-2, widen_embed=True)
    print(f"560m L4 B{B}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    _kv_check(run, v.oracle, B, 16 + 11, 2e-2)


@pytest.mark.parametrize("batch, n_new", [(1, 100), (8, 30)])
def test_bloom560m_full_depth(batch, n_new):
    w = bi.WORKLOADS["bloom-560m"]
    m = w.model
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, batch, w.prompt_len)
    run = run_gpu(cfg, dw, prompt, valid, n_new)
    v = compare(m, T, prompt, valid, run, 1e-2, widen_embed=True)
    print(f"560m B{batch} {n_new} tokens: hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f} ({v.near_ties} accepted near-ties)")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok


@pytest.mark.parametrize("batch, valid", [(1, None), (3, (16, 9, 2))])
def test_tp_share_176b_two_layers(batch, valid):
    m = bi.BLOOM_176B_TP8_RANK0.truncated(2)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16, valid)
    run = run_gpu(cfg, dw, prompt, vl, 4)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"176b rank-0 share L2 B{batch}: hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    _kv_check(run, v.oracle, batch, 16 + 3, 2e-2)


@pytest.mark.parametrize("batch", [1, 16])
def test_full_176b_int8_two_layers(batch):
    """Full 176B width with int8 weights: batch 1 runs the vector-ALU GEMV, batch 16 the
    direct-to-LDS GEMM (256-row prompt pass, 16-row decode steps)."""
    m = bi.BLOOM_176B_INT8.truncated(2)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16)
    run = run_gpu(cfg, dw, prompt, vl, 3)
    del dw
    torch.cuda.empty_cache()
    v = compare(m, T, prompt, vl, run, 2e-2)
    print(f"176b int8 L2 B{batch}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 2e-2 and v.tokens_ok


def test_bloom560m_wide_batch_direct_to_lds_tiles():
    """72 rows: the 1152-row prompt pass takes the 256 x 256 tiles, the decode steps and
    the LM head (argmax epilogue) the 128-row decode tiles."""
    m = bi.BLOOM_560M.truncated(2)
    T, dw, cfg = upload(m, seed=9)
    prompt, valid = bi.prompts(m, 72, 16, np.arange(72) % 16 + 1, seed=10)
    run = run_gpu(cfg, dw, prompt, valid, 3)
    v = compare(m, T, prompt, valid, run, 1e-2, widen_embed=True)
    print(f"560m L2 B72: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok


@pytest.mark.parametrize("d, P, valid", [
    (128, 100, (100, 37)),                                          # per-row prompt kernel
    (128, 100, (100, 37, 1, 64, 99, 100, 2, 50, 77, 13)),           # 280 prompt blocks
    (256, 70, (70, 1, 33, 8, 69, 70, 2, 40, 9, 16, 55, 3, 64, 17, 70)),
    (64, 130, (130, 129, 64, 1, 33, 100, 7))])
def test_long_rows_cross_attention_batches(d, P, valid):
    """Long prompts and up to P + 59 visible keys.  With >= 256 (sequence, head, chunk)
    blocks the prompt pass runs the chunked prompt kernel: several chunks of query rows
    per sequence and several LDS key tiles (32 keys per tile at d = 256, 64 otherwise),
    with padding that leaves whole chunks without a visible key; with fewer it runs one
    block per (row, head).  The decode steps see more keys than one batch of the decode
    kernel (16 lane groups x 8 keys at d = 128), so the running-max rescale across
    batches runs."""
    H = 512 // d
    m = dataclasses.replace(bi.BLOOM_560M, name=f"d{d}", n_layer=1, hidden=512, n_head_total=H,
                            n_head_local=H, head_dim=d, ffn=1024, vocab=512)
    T, dw, cfg = upload(m, seed=21)
    B = len(valid)
    prompt, valid = bi.prompts(m, B, P, valid, seed=22)
    run = run_gpu(cfg, dw, prompt, valid, 60)
    v = compare(m, T, prompt, valid, run, 1e-2)
    print(f"d{d} L1 P{P}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    _kv_check(run, v.oracle, B, P + 59, 2e-2)


@pytest.mark.parametrize("hidden, ffn, n_new", [(2112, 4224, 24), (3072, 8192, 12)])
def test_batch1_whole_row_gemv_widths(hidden, ffn, n_new):
    """Batch 1: QKV, MLP-up, MLP-down and the LM head (rows of 4-16 KB; the LM head with
    the argmax epilogue) run the GEMV that issues a wave's whole weight row at once, the
    dense projection (2 KB rows) the two-rows-per-wave GEMV.  Hidden 2112 leaves a partial
    last 1 KB piece in every row."""
    m = dataclasses.replace(bi.BLOOM_560M, name=f"h{hidden}", n_layer=2, hidden=hidden,
                            n_head_total=32, n_head_local=16, head_dim=64, ffn=ffn, vocab=8192)
    T, dw, cfg = upload(m, seed=31)
    prompt, valid = bi.prompts(m, 1, 16, seed=32)
    run = run_gpu(cfg, dw, prompt, valid, n_new)
    v = compare(m, T, prompt, valid, run, 1e-2)
    print(f"h{hidden} L2 B1: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    _kv_check(run, v.oracle, 1, 16 + n_new - 1, 2e-2)


@pytest.mark.parametrize("wdt, tol", [("bf16", 1e-2), ("int8", 2e-2)])
@pytest.mark.parametrize("batch, hidden, ffn", [(20, 1088, 4160), (40, 1088, 4160),
                                                (70, 1088, 4160)])
def test_prompt_pass_direct_to_lds_gemm_ragged(batch, hidden, ffn, wdt, tol):
    """Prompt passes of 320, 640 and 1120 rows run the direct-to-LDS MFMA GEMM (128 x
    128, 256 x 128 and 256 x 256 tiles, split-K) with M and N that are not multiples of
    the tile, and ragged left padding; the decode steps (20, 40 and 70 rows) its skinny
    tiles (32 x 256 for int8 weights at 20 rows); int8 weights are widened from LDS and
    scaled per row in the epilogue."""
    m = dataclasses.replace(bi.BLOOM_560M, name=f"lg{batch}", n_layer=2, hidden=hidden,
                            n_head_total=16, n_head_local=16, head_dim=64, ffn=ffn, vocab=4096,
                            weight_dtype=wdt)
    T, dw, cfg = upload(m, seed=41)
    prompt, valid = bi.prompts(m, batch, 16, np.arange(batch) % 16 + 1, seed=42)
    run = run_gpu(cfg, dw, prompt, valid, 3)
    v = compare(m, T, prompt, valid, run, tol)
    print(f"lg {wdt} B{batch} h{hidden}: hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= tol and v.tokens_ok
    _kv_check(run, v.oracle, batch, 16 + 2, 2e-2)


@pytest.mark.parametrize("batch", [48, 100])
def test_int8_wide_ffn_decode_tiles(batch):
    """int8 weights with a 32832-wide MLP (not a multiple of 256): decode steps of 48
    rows run the MLP-up with 64 x 256 tiles and the other linears with 64 x 128 tiles,
    100 rows the 128-row tile with all four waves side by side; splits from the
    rounds-of-resident-blocks rule."""
    m = dataclasses.replace(bi.BLOOM_560M, name=f"i8w{batch}", n_layer=2, hidden=1088,
                            n_head_total=16, n_head_local=16, head_dim=64, ffn=32832,
                            vocab=4096, weight_dtype="int8")
    T, dw, cfg = upload(m, seed=51)
    prompt, valid = bi.prompts(m, batch, 4, np.arange(batch) % 4 + 1, seed=52)
    run = run_gpu(cfg, dw, prompt, valid, 3)
    v = compare(m, T, prompt, valid, run, 2e-2)
    print(f"int8 ffn 32832 B{batch}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 2e-2 and v.tokens_ok
    _kv_check(run, v.oracle, batch, 4 + 2, 4e-2)


def test_four_way_split_residual_layernorm():
    """Hidden 6656 at 8 rows: dense and MLP-down split K four ways, so their partials go
    through the fused split-K + bias + residual + LayerNorm kernel with four partials
    (LN2 after dense, the second layer's LN1 after the first layer's down)."""
    m = dataclasses.replace(bi.BLOOM_560M, name="h6656", n_layer=2, hidden=6656,
                            n_head_total=52, n_head_local=52, head_dim=128, ffn=6656,
                            vocab=4096)
    T, dw, cfg = upload(m, seed=61)
    prompt, valid = bi.prompts(m, 8, 4, (4, 3, 2, 1, 4, 4, 2, 3), seed=62)
    run = run_gpu(cfg, dw, prompt, valid, 4)
    v = compare(m, T, prompt, valid, run, 1e-2)
    print(f"h6656 B8: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
    _kv_check(run, v.oracle, 8, 4 + 3, 2e-2)


def test_tp_share_176b_prompt_pass_batch32():
    """The 176B rank-0 share at full width, batch 32: the 512-row prompt pass runs the
    direct-to-LDS GEMM with split-K on the real layer shapes."""
    m = bi.BLOOM_176B_TP8_RANK0.truncated(2)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, 32, 16)
    run = run_gpu(cfg, dw, prompt, vl, 2)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"176b rank-0 share L2 B32: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok


@pytest.mark.parametrize("act, batch", [("f16", 8), ("f16", 128), ("bf16", 128)])
def test_tp_share_176b_two_layers_benchmarked_batches(act, batch):
    """The 176B rank-0 share at the batches the benchmark runs (8: 32-row decode tiles;
    128: 128-row decode tiles with split-K and the fused split-K residual LayerNorm, and
    the 2048-row prompt pass on the large prompt tiles), 2 layers, compared on sampled
    rows (the oracle runs those rows alone)."""
    m = dataclasses.replace(bi.BLOOM_176B_TP8_RANK0.truncated(2), activations=act)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16)
    run = run_gpu(cfg, dw, prompt, vl, 4)
    del dw
    torch.cuda.empty_cache()
    rows = list(range(batch)) if batch <= 8 else [0, 57, batch - 1]
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True, rows=rows)
    print(f"176b share L2 act {act} B{batch} (rows {rows}): hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok


@pytest.mark.parametrize("batch", [64, 128])
def test_full_176b_int8_two_layers_benchmarked_batches(batch):
    """The full 176B model with int8 weights and bf16 activations at the benchmarked
    batches 64 and 128 (int8 decode tiles 64 x 256 / 128 x 128, the 1024- and 2048-row
    int8 prompt passes), 2 layers, sampled rows against the oracle at 2e-2."""
    m = bi.BLOOM_176B_INT8.truncated(2)
    T, dw, cfg = upload(m)
    prompt, vl = bi.prompts(m, batch, 16)
    run = run_gpu(cfg, dw, prompt, vl, 3)
    del dw
    torch.cuda.empty_cache()
    rows = [0, 31, batch - 1]
    v = compare(m, T, prompt, vl, run, 2e-2, rows=rows)
    print(f"176b int8 L2 B{batch} (rows {rows}): hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 2e-2 and v.tokens_ok


def test_bloom560m_full_depth_batch32_100_tokens():
    """BLOOM-560m, 24 layers, batch 32, 100 greedy tokens (the benchmarked configuration
    of that model), fp16 activations, sampled rows against the oracle."""
    w = bi.WORKLOADS["bloom-560m"]
    m = dataclasses.replace(w.model, activations="f16")
    T, dw, cfg = upload(m)
    prompt, valid = bi.prompts(m, 32, w.prompt_len)
    run = run_gpu(cfg, dw, prompt, valid, 100)
    rows = [0, 13, 31]
    v = compare(m, T, prompt, valid, run, 1e-2, widen_embed=True, rows=rows)
    print(f"560m B32 100 tokens (rows {rows}): hidden rel {v.hidden_rel:.2e}, "
          f"exact ids {v.exact_frac:.3f} ({v.near_ties} accepted near-ties)")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
