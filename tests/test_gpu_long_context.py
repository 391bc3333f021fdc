"""Decode attention over a long cache (split over the keys): the decode step's attention
takes one block per (row, head, key range) when the cache is long and the (row, head)
blocks alone would leave the chip idle, and a merge kernel combines the ranges' partial
softmax sums in range order ("Hugging Face BLOOM Inference Optimization", Custom CUDA
Kernels and Hardware Acceleration: the fused masked softmax in float32).  Compared with
the oracle, teacher-forced, at a KV length of 2048: left-padded rows (whole key ranges
masked), a batch whose rows each split, the captured decode step of bloom_generate
(its position from device memory), and the int8 cache."""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import transformer_bloom_decode_amd as tb
from gpu_util import GpuRun, compare, run_gpu, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batch, valid", [(1, None), (3, (2000, 1500, 900))])
def test_560m_kv2048(batch, valid):
    m = dataclasses.replace(bi.BLOOM_560M.truncated(2), activations="f32")
    T, dw, cfg = upload(m)
    P, n_new = 2000, 48
    prompt, vl = bi.prompts(m, batch, P, valid)
    run = run_gpu(cfg, dw, prompt, vl, n_new, max_len=2048)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"560m L2 kv2048 B{batch}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-3 and v.tokens_ok


def test_560m_kv2048_graph_equals_eager():
    m = dataclasses.replace(bi.BLOOM_560M.truncated(2), activations="f32")
    T, dw, cfg = upload(m)
    B, P, n_new = 2, 2030, 18
    prompt, vl = bi.prompts(m, B, P, (2030, 1200))
    tok = torch.from_numpy(prompt.astype(np.int32)).cuda()
    val = torch.from_numpy(np.asarray(vl, dtype=np.int32)).cuda()
    outs = []
    for graph in (False, True):
        kv = tb.KVCache(cfg, B, 2048, fill=float("nan"))
        ws = tb.workspace(cfg, B, P)
        ids, hid = tb.greedy_generate(cfg, dw, kv, tok, val, n_new, ws, graph=graph)
        torch.cuda.synchronize()
        outs.append((ids.cpu().numpy(), hid.cpu().numpy(), kv))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.int32), outs[1][1].view(np.int32))
    run = GpuRun(outs[1][0].T.copy(), outs[1][1], outs[1][2], cfg)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"560m L2 kv2048 graph B{B}: hidden rel {v.hidden_rel:.2e}")
    assert v.hidden_rel <= 1e-3 and v.tokens_ok


def test_tp_share_176b_kv2048():
    """The 176B rank-0 share (14 heads of 128), one layer, fp16 activations and cache,
    batch 1: 2040 prompt tokens, then decode steps up to a KV length of 2048."""
    m = dataclasses.replace(bi.BLOOM_176B_TP8_RANK0.truncated(1), activations="f16")
    T, dw, cfg = upload(m)
    P, n_new = 2040, 9
    prompt, vl = bi.prompts(m, 1, P)
    run = run_gpu(cfg, dw, prompt, vl, n_new, max_len=2048)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"176b share L1 kv2048: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok


@pytest.mark.parametrize("shape, act, batch, valid", [
    (bi.BLOOM_560M.truncated(2), "f32", 3, (2000, 1500, 900)),
    (bi.BLOOM_176B_TP8_RANK0.truncated(1), "f16", 1, None)])
def test_int8_cache_kv2048(shape, act, batch, valid):
    """The int8 cache over a long cache: each lane reads 16 codes of a key or value row
    (head dims 64 and 128), the key ranges split and merge as for the other caches; the
    oracle rounds the cached keys and values to int8 per (row, head, slot)."""
    m = dataclasses.replace(shape, activations=act, kv_cache="int8")
    T, dw, cfg = upload(m)
    P, n_new = (2000, 48) if valid else (2040, 9)
    prompt, vl = bi.prompts(m, batch, P, valid)
    run = run_gpu(cfg, dw, prompt, vl, n_new, max_len=2048)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True)
    print(f"{m.name} L{m.n_layer} {act} int8 KV kv2048 B{batch}: hidden rel "
          f"{v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
