"""The C-ABI boundary pieces around the forward pass, on the GPU:

* bloom_init_weights (the seeded weight specification, computed on the GPU) is bitwise
  equal to the host generator of the test inputs (bloom_inputs/gen.c), which
  implements the same specification independently: whole tensors for the small
  shapes, and every tensor kind (float32, bf16, int8 weights with fp16 row scales);
* a device-resident KV length (bloom_kv_cache.d_len): a caller captures one
  bloom_decode_step call in a graph and replays it; every replay gives the tokens,
  final-LayerNorm states and KV slots of the eager loop bit for bit, and the device
  length advances by one per replay;
* the device guard: a step that finds the device length at the cache's end writes no
  slot and leaves the length there.
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import transformer_bloom_decode_amd as tb

pytestmark = pytest.mark.gpu


def _empty_weights(m):
    """Device buffers of the model's storage shapes (uninitialised) and the struct."""
    dt = {"f32": torch.float32, "bf16": torch.int16, "int8": torch.int8}
    def buf(name, layer=None):
        shape = bi.tensor_shape(m, name)
        if name.startswith("s_"):
            return torch.empty(shape, dtype=torch.int16, device="cuda")
        kind = m.weight_dtype if name.startswith("w_") else m.param_dtype
        return torch.empty(shape, dtype=dt[kind], device="cuda")
    g = {n: buf(n) for n in bi.global_field_names(m)}
    layers = [{f: buf(f, l) for f in bi.layer_field_names(m)} for l in range(m.n_layer)]
    return tb.DeviceWeights(g, layers)


def _host_view(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


@pytest.mark.parametrize("shape", [
    bi.TINY,
    dataclasses.replace(bi.TINY, weight_dtype="bf16", name="tiny-bf16"),
    dataclasses.replace(bi.TINY, weight_dtype="int8", name="tiny-int8"),
    dataclasses.replace(bi.TINY, init_std=0.3, name="tiny-std0.3"),
    bi.BLOOM_560M.truncated(2),
])
def test_init_weights_equals_the_host_generator(shape):
    dw = _empty_weights(shape)
    cfg = tb.make_config(shape)
    tb.bloom_init_weights(cfg, dw, seed=0, sigma=shape.init_std)
    torch.cuda.synchronize()
    for name in bi.global_field_names(shape):
        np.testing.assert_array_equal(_host_view(dw.tensors["globals"][name]),
                                      bi.tensor(shape, name), err_msg=name)
    for l in range(shape.n_layer):
        for f in bi.layer_field_names(shape):
            np.testing.assert_array_equal(_host_view(dw.tensors["layers"][l][f]),
                                          bi.tensor(shape, f, l), err_msg=f"{f} layer {l}")


def test_init_weights_full_width_int8_layer_sampled():
    """One layer of the full 176B int8 model (2.5 G weights): sampled rows of every tensor."""
    m = bi.BLOOM_176B_INT8.truncated(1)
    dw = _empty_weights(m)
    tb.bloom_init_weights(tb.make_config(m), dw, seed=7)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4097, 14335])
    for f in bi.layer_field_names(m):
        ref = bi.tensor(m, f, 0, seed=7)
        got = dw.tensors["layers"][0][f]
        if ref.ndim == 2:
            r = rows[rows < ref.shape[0]]
            np.testing.assert_array_equal(_host_view(got[torch.from_numpy(r).cuda()]), ref[r],
                                          err_msg=f)
        else:
            np.testing.assert_array_equal(_host_view(got), ref, err_msg=f)
        del got


def _decode_setup(m, B, P, n_new, seed=0):
    T = bi.model_tensors(m)
    dw = tb.DeviceWeights.from_arrays(T)
    cfg = tb.make_config(m)
    prompt, valid = bi.prompts(m, B, P, seed=seed)
    tok = torch.from_numpy(prompt).cuda()
    vl = torch.from_numpy(valid).cuda()
    return dw, cfg, tok, vl


def test_captured_decode_step_replays_equal_the_eager_loop():
    m = bi.BLOOM_560M.truncated(3)
    B, P, n_new = 2, 16, 12
    dw, cfg, tok, vl = _decode_setup(m, B, P, n_new)
    ws = tb.workspace(cfg, B, P)
    h = cfg.hidden

    # eager loop, host-side length
    kv_e = tb.KVCache(cfg, B, P + n_new, fill=float("nan"))
    ids_e, hid_e = tb.greedy_generate(cfg, dw, kv_e, tok, vl, n_new, ws)
    torch.cuda.synchronize()

    # device length: prompt pass and one eager step, then one step captured and replayed
    kv = tb.KVCache(cfg, B, P + n_new, fill=float("nan"), device_len=True)
    ids = torch.full((n_new, B), -1, dtype=torch.int32, device="cuda")
    hid = torch.zeros((n_new, B, h), dtype=torch.float32, device="cuda")
    cur = torch.empty(B, dtype=torch.int32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    hstep = torch.empty((B, h), dtype=torch.float32, device="cuda")
    tb.bloom_prefill(cfg, dw, kv, B, P, tok, vl, ids[0], hid[0], ws)
    torch.cuda.synchronize()
    assert int(kv.d_len.item()) == P
    cur.copy_(ids[0])
    tb.bloom_decode_step(cfg, dw, kv, B, cur, vl, nxt, hstep, ws)
    ids[1].copy_(nxt); hid[1].copy_(hstep); cur.copy_(nxt)
    torch.cuda.synchronize()
    assert int(kv.d_len.item()) == P + 1

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            tb.bloom_decode_step(cfg, dw, kv, B, cur, vl, nxt, hstep, ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    # the capture itself ran nothing: the device length is unchanged
    torch.cuda.synchronize()
    assert int(kv.d_len.item()) == P + 1
    for t in range(2, n_new):
        g.replay()
        # the caller's own eager work between replays: record and feed back the token
        ids[t].copy_(nxt); hid[t].copy_(hstep); cur.copy_(nxt)
        torch.cuda.synchronize()
        assert int(kv.d_len.item()) == P + t, t
        np.testing.assert_array_equal(ids[t].cpu().numpy(), ids_e[t].cpu().numpy())
        np.testing.assert_array_equal(hid[t].cpu().numpy(), hid_e[t].cpu().numpy())
    np.testing.assert_array_equal(ids.cpu().numpy(), ids_e.cpu().numpy())
    L = P + n_new - 1
    np.testing.assert_array_equal(kv.k[:, :, :, :L].float().cpu().numpy(),
                                  kv_e.k[:, :, :, :L].float().cpu().numpy())
    np.testing.assert_array_equal(kv.v[:, :, :, :L].float().cpu().numpy(),
                                  kv_e.v[:, :, :, :L].float().cpu().numpy())
    assert torch.isnan(kv.k[:, :, :, L:].float()).all()


def test_device_length_at_the_cache_end_writes_no_slot():
    m = bi.BLOOM_560M.truncated(2)
    B, P, n_new = 1, 16, 4
    dw, cfg, tok, vl = _decode_setup(m, B, P, n_new)
    ws = tb.workspace(cfg, B, P)
    max_len = P + n_new
    kv = tb.KVCache(cfg, B, max_len, fill=float("nan"), device_len=True)
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    tb.bloom_prefill(cfg, dw, kv, B, P, tok, vl, nxt, None, ws)
    torch.cuda.synchronize()
    # the device length says the cache is full (a caller's replays ran ahead of the
    # host's count): the step must leave every slot and the length as they are
    kv.d_len.fill_(max_len)
    k0, v0 = kv.k.clone(), kv.v.clone()
    tb.bloom_decode_step(cfg, dw, kv, B, nxt, vl, nxt, None, ws)
    torch.cuda.synchronize()
    assert int(kv.d_len.item()) == max_len
    assert torch.equal(kv.k.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(kv.v.view(torch.int16), v0.view(torch.int16))
    assert 0 <= int(nxt.item()) < m.vocab
