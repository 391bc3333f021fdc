"""Decode attention with one wave per (row, head) pair (k_attention_wave), which decode
steps of at least 1024 pairs use: ALiBi-biased scores over the row's visible slots,
left-padded rows masked, float32 softmax and P.V ("Hugging Face BLOOM Inference
Optimization", Custom CUDA Kernels and Hardware Acceleration: the fused masked softmax
in float32).  BLOOM-560m on 2 layers at batch 64 (64 x 16 = 1024 pairs) with ragged
valid lengths, teacher-forced against the oracle on sampled rows: float32 activations
and cache, and the int8 cache (codes and per-slot scales); bf16 activations at head dims 128 and
256 on one layer of the same width (8 heads at batch 136, 4 heads at batch 264)."""
import dataclasses

import numpy as np
import pytest

import bloom_inputs as bi
from gpu_util import compare, run_gpu, upload

pytestmark = pytest.mark.gpu

ROWS = [0, 5, 17, 40, 63]


def _valid(batch, P):
    # ragged left padding: full rows, single-token rows and everything between
    v = np.array([P, 1, P // 2, 3, P - 1, 7, P, 2], dtype=np.int32)
    return np.resize(v, batch)


@pytest.mark.parametrize("kv, tol", [("auto", 1e-5), ("int8", 1e-3)])
def test_560m_batch64_ragged(kv, tol):
    m = dataclasses.replace(bi.BLOOM_560M.truncated(2), activations="f32", kv_cache=kv)
    assert 64 * m.n_head_local >= 1024
    T, dw, cfg = upload(m)
    P = 24
    prompt, vl = bi.prompts(m, 64, P, _valid(64, P))
    run = run_gpu(cfg, dw, prompt, vl, 12)
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True, rows=ROWS)
    print(f"560m L2 B64 ragged kv {kv}: hidden rel {v.hidden_rel:.2e}, exact ids "
          f"{v.exact_frac:.3f}")
    assert v.hidden_rel <= tol and v.tokens_ok


@pytest.mark.parametrize("head_dim", [128, 256])
def test_head_dims_batch128(head_dim):
    base = bi.BLOOM_560M.truncated(1)
    heads = 1024 // head_dim
    m = dataclasses.replace(base, n_head_total=heads, n_head_local=heads, head_dim=head_dim,
                            activations="bf16", name=f"d{head_dim}")
    B = 1024 // heads + 8   # at least 1024 pairs
    T, dw, cfg = upload(m)
    P = 16
    prompt, vl = bi.prompts(m, B, P, _valid(B, P))
    run = run_gpu(cfg, dw, prompt, vl, 6)
    rows = [0, 1, 3, B // 2, B - 1]
    v = compare(m, T, prompt, vl, run, 1e-2, widen_embed=True, rows=rows)
    print(f"d{head_dim} L1 B{B}: hidden rel {v.hidden_rel:.2e}, exact ids {v.exact_frac:.3f}")
    assert v.hidden_rel <= 1e-2 and v.tokens_ok
