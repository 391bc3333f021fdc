"""GPU test of kv_cache_append: new key/value vectors land bit-exactly in the requested
slots of the requested layer; every other slot keeps its NaN sentinel ("Hugging Face
BLOOM Inference Optimization", Efficient PyTorch Implementation: the KV "past" kept in
a layout that needs no reshape)."""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wdt", ["bf16", "f32"])
@pytest.mark.parametrize("layer, batch, pos, n_new", [(0, 2, 0, 8), (1, 3, 5, 1), (1, 1, 27, 1),
                                                      (0, 3, 10, 18)])
def test_kv_append_writes_exactly_the_slots(wdt, layer, batch, pos, n_new):
    import transformer_bloom_decode_amd as tb

    m = dataclasses.replace(bi.TINY, weight_dtype=wdt)
    cfg = tb.make_config(m)
    max_batch, max_len = 3, 28
    kv = tb.KVCache(cfg, max_batch, max_len, fill=float("nan"))
    dt = kv.k.dtype
    H, d = m.n_head_local, m.head_dim
    g = torch.Generator().manual_seed(layer * 100 + pos)
    k = torch.randn((batch, H, n_new, d), generator=g).to(dt).cuda()
    v = torch.randn((batch, H, n_new, d), generator=g).to(dt).cuda()
    tb.kv_cache_append(cfg, kv, layer, batch, pos, k, v, n_new)
    torch.cuda.synchronize()
    K = kv.k.float().cpu()
    V = kv.v.float().cpu()
    assert torch.equal(K[layer, :batch, :, pos: pos + n_new], k.float().cpu())
    assert torch.equal(V[layer, :batch, :, pos: pos + n_new], v.float().cpu())
    mask = torch.ones_like(K, dtype=torch.bool)
    mask[layer, :batch, :, pos: pos + n_new] = False
    assert torch.isnan(K[mask]).all() and torch.isnan(V[mask]).all()
    assert kv.len == 0          # appending does not move the cache length


def test_kv_append_capacity_is_checked_before_launch():
    import transformer_bloom_decode_amd as tb

    cfg = tb.make_config(bi.TINY)
    kv = tb.KVCache(cfg, 2, 8, fill=float("nan"))
    k = torch.zeros((1, 8, 2, 8), device="cuda")
    with pytest.raises(tb.BloomError) as ei:
        tb.kv_cache_append(cfg, kv, 0, 1, 7, k, k, 2)
    assert ei.value.code == tb.BLOOM_ECAPACITY
    torch.cuda.synchronize()
    assert torch.isnan(kv.k).all()
