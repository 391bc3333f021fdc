"""The C-ABI library loads, exports every function include/bloom.h declares, and its
synchronous validation returns the documented status codes.  Nothing here launches
a kernel: every call fails (or is a no-op) before touching the device, so these run
without a GPU."""
import ctypes
import dataclasses
import re

import pytest

import bloom_inputs as bi
import transformer_bloom_decode_amd as tb


def _declared_functions():
    text = open(tb.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names) - {"if", "return"})


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("bloom_prefill", "bloom_decode_step", "bloom_generate", "alibi_masked_softmax",
                     "kv_cache_append", "bloom_workspace_bytes", "bloom_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(tb.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(so, n)]
    assert not missing, missing


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert tb.bloom_status_string(code)
    assert tb.bloom_status_string(-99) == "unknown status"


def test_struct_layout_matches_header():
    # 12 int32 + 1 float; 16 pointers; 5 pointers + 1 pointer; 2 pointers + 4 int32 +
    # 3 pointers; 2 int32 + 7 pointers + 1 size_t
    assert ctypes.sizeof(tb.bloom_gen_control) == 8 + 7 * 8 + 8
    assert ctypes.sizeof(tb.bloom_config) == 52
    assert ctypes.sizeof(tb.bloom_layer_weights) == 16 * 8
    assert ctypes.sizeof(tb.bloom_weights) == 7 * 8
    assert ctypes.sizeof(tb.bloom_kv_cache) == 2 * 8 + 4 * 4 + 3 * 8


def _cfg(**kw):
    return tb.make_config(dataclasses.replace(bi.BLOOM_560M, **kw))


def _err(fn, *a):
    with pytest.raises(tb.BloomError) as ei:
        fn(*a)
    return ei.value.code


@pytest.mark.parametrize("change, code", [
    (dict(head_dim=96), tb.BLOOM_EINVAL),           # not a power of two
    (dict(head_dim=512), tb.BLOOM_EINVAL),
    (dict(hidden=1000), tb.BLOOM_EINVAL),           # bf16 needs multiples of 64
    (dict(n_layer=0), tb.BLOOM_EINVAL),
    (dict(head_offset=10), tb.BLOOM_EINVAL),        # 10 + 16 heads > 16
    (dict(ln_eps=float("nan")), tb.BLOOM_EINVAL),
])
def test_workspace_rejects_bad_config(change, code):
    assert _err(tb.bloom_workspace_bytes, _cfg(**change), 1, 16) == code


def test_workspace_rejects_bad_dtype():
    c = _cfg()
    c.weight_dtype = 7
    assert _err(tb.bloom_workspace_bytes, c, 1, 16) == tb.BLOOM_EDTYPE


@pytest.mark.parametrize("weights, act, kv, code", [
    ("int8", "int8", "int8", tb.BLOOM_OK),       # W8A8 with an int8 cache
    ("int8", "int8", "f16", tb.BLOOM_EDTYPE),    # the cache holds act_dtype or int8
    ("int8", "f16", "int8", tb.BLOOM_OK),        # int8 cache under fp16 activations
    ("bf16", "bf16", "int8", tb.BLOOM_OK),
    ("bf16", "int8", "int8", tb.BLOOM_EDTYPE),   # int8 activations need int8 weights
    ("f32", "f32", "int8", tb.BLOOM_EDTYPE),     # the float32 model is float32 throughout
])
def test_int8_activation_and_cache_types(weights, act, kv, code):
    shape = dataclasses.replace(bi.BLOOM_176B_INT8.truncated(2), weight_dtype=weights,
                                activations=act, kv_cache=kv)
    c = tb.make_config(shape)
    if code == tb.BLOOM_OK:
        assert tb.bloom_workspace_bytes(c, 4, 16) > 0
    else:
        assert _err(tb.bloom_workspace_bytes, c, 4, 16) == code


def test_int8_cache_requires_scale_buffers():
    shape = dataclasses.replace(bi.BLOOM_176B_INT8.truncated(2), activations="int8",
                                kv_cache="int8")
    f = _Fake(shape)
    assert _prefill(f) == tb.BLOOM_EINVAL                          # no k_scale / v_scale
    f.kv.k_scale = 0x1000
    assert _prefill(f) == tb.BLOOM_EINVAL                          # v_scale still missing
    f.kv.v_scale = 0x1002                                          # not 4-byte aligned
    assert _prefill(f) == tb.BLOOM_EINVAL
    f.kv.v_scale = 0x1000
    assert _prefill(f, ws_bytes=1024) == tb.BLOOM_EWORKSPACE       # checks passed


def test_workspace_grows_with_batch_and_prompt():
    c = _cfg()
    a = tb.bloom_workspace_bytes(c, 1, 1)
    b = tb.bloom_workspace_bytes(c, 8, 16)
    assert 0 < a < b
    assert tb.bloom_workspace_bytes(_cfg(weight_dtype="f32"), 0, 0) >= 0


class _Fake:
    """Non-null dummy device pointers: validation must fail before any use."""

    def __init__(self, shape):
        self.cfg = tb.make_config(shape)
        self.layers = (tb.bloom_layer_weights * shape.n_layer)()
        for lw in self.layers:
            for f in tb.LAYER_FIELDS:
                if not f.startswith("s_") or shape.weight_dtype == "int8":
                    setattr(lw, f, 0x1000)
        self.w = tb.bloom_weights(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, self.layers)
        self.kv = tb.bloom_kv_cache(0x1000, 0x1000, 4, 32, 0, 0)


def _prefill(f, batch=2, prompt=8, ws_bytes=1 << 40, tokens=0x1000):
    return tb.lib.bloom_prefill(ctypes.byref(f.cfg), ctypes.byref(f.w), ctypes.byref(f.kv), batch,
                                prompt, tokens, 0x1000, 0x1000, None, 0x1000, ws_bytes, None)


def _decode(f, batch=2, ws_bytes=1 << 40):
    return tb.lib.bloom_decode_step(ctypes.byref(f.cfg), ctypes.byref(f.w), ctypes.byref(f.kv),
                                    batch, 0x1000, 0x1000, 0x1000, None, 0x1000, ws_bytes, None)


def test_prefill_validation_paths():
    f = _Fake(bi.BLOOM_560M)
    assert _prefill(f, batch=5) == tb.BLOOM_ECAPACITY           # > max_batch
    assert _prefill(f, prompt=33) == tb.BLOOM_ECAPACITY         # > max_len
    assert _prefill(f, prompt=0) == tb.BLOOM_EINVAL
    assert _prefill(f, batch=-1) == tb.BLOOM_EINVAL
    assert _prefill(f, ws_bytes=1024) == tb.BLOOM_EWORKSPACE
    assert _prefill(f, tokens=None) == tb.BLOOM_EINVAL
    assert _prefill(f, batch=0) == tb.BLOOM_OK                   # empty batch: no-op
    assert f.kv.len == 0 and f.kv.prompt_len == 0                # state untouched
    f.layers[3].w_up = None
    assert _prefill(f) == tb.BLOOM_EINVAL
    f.layers[3].w_up = 0x1000
    f.layers[0].s_up = 0x1000                                    # scales on bf16 weights
    assert _prefill(f) == tb.BLOOM_EINVAL


def test_int8_requires_row_scales():
    f = _Fake(bi.BLOOM_176B_INT8.truncated(2))
    f.kv.max_len = 32
    f.layers[1].s_down = None
    assert _prefill(f) == tb.BLOOM_EINVAL


def test_decode_validation_paths():
    f = _Fake(bi.BLOOM_560M)
    assert _decode(f) == tb.BLOOM_EINVAL                         # no prompt pass yet
    f.kv.prompt_len = 8
    f.kv.len = 32
    assert _decode(f) == tb.BLOOM_ECAPACITY                      # cache full
    f.kv.len = 20
    assert _decode(f, batch=9) == tb.BLOOM_ECAPACITY
    assert _decode(f, ws_bytes=10) == tb.BLOOM_EWORKSPACE
    assert _decode(f, batch=0) == tb.BLOOM_OK
    assert f.kv.len == 20
    f.kv.len = 4                                                  # len < prompt_len
    assert _decode(f) == tb.BLOOM_EINVAL
    f.kv.max_len = (1 << 20) + 1                                  # beyond the supported 2^20
    f.kv.len = 20
    assert _decode(f) == tb.BLOOM_EINVAL


def _generate(f, batch=2, prompt=8, n_new=4, ws_bytes=1 << 40, ids=0x1000, ctl=None):
    return tb.lib.bloom_generate(ctypes.byref(f.cfg), ctypes.byref(f.w), ctypes.byref(f.kv),
                                 batch, prompt, 0x1000, 0x1000, n_new, ids, None,
                                 None if ctl is None else ctypes.byref(ctl), 0x1000, ws_bytes,
                                 None)


def test_generate_validation_paths():
    f = _Fake(bi.BLOOM_560M)
    assert _generate(f, prompt=8, n_new=26) == tb.BLOOM_ECAPACITY   # 8 + 25 > 32
    assert _generate(f, batch=5) == tb.BLOOM_ECAPACITY
    assert _generate(f, n_new=0) == tb.BLOOM_EINVAL
    assert _generate(f, prompt=0) == tb.BLOOM_EINVAL
    assert _generate(f, ids=None) == tb.BLOOM_EINVAL
    assert _generate(f, ws_bytes=1024) == tb.BLOOM_EWORKSPACE
    assert _generate(f, batch=0) == tb.BLOOM_OK
    assert _generate(f, ctl=tb.bloom_gen_control(250880, 0, None, None)) == tb.BLOOM_EINVAL
    assert _generate(f, ctl=tb.bloom_gen_control(5, 0, None, None), ws_bytes=16) == \
        tb.BLOOM_EWORKSPACE
    # sampling fields: all or none; the sampling workspace must be large enough
    part = tb.bloom_gen_control(-1, 0, None, None, 0x10, 0x10, None, 0x10, 0x10, 1 << 30)
    assert _generate(f, ctl=part) == tb.BLOOM_EINVAL
    full = tb.bloom_gen_control(-1, 0, None, None, 0x10, 0x10, 0x10, 0x10, 0x10, 64)
    assert _generate(f, ctl=full) == tb.BLOOM_EWORKSPACE
    assert f.kv.len == 0 and f.kv.prompt_len == 0


def test_kv_append_validation_paths():
    f = _Fake(bi.BLOOM_560M)
    app = lambda layer, batch, pos, n: tb.lib.kv_cache_append(
        ctypes.byref(f.cfg), ctypes.byref(f.kv), layer, batch, pos, 0x1000, 0x1000, n, None)
    assert app(24, 1, 0, 1) == tb.BLOOM_EINVAL        # layer out of range
    assert app(0, 5, 0, 1) == tb.BLOOM_ECAPACITY      # batch > max_batch
    assert app(0, 1, 30, 3) == tb.BLOOM_ECAPACITY     # 30 + 3 > 32
    assert app(0, 1, 0, 0) == tb.BLOOM_OK             # nothing to copy
    assert app(0, 1, -1, 1) == tb.BLOOM_EINVAL


def test_kv_compact_validation_paths():
    f = _Fake(bi.BLOOM_560M)
    f.kv.len = 8
    comp = lambda batch, keep: tb.lib.kv_cache_compact(
        ctypes.byref(f.cfg), ctypes.byref(f.kv), batch, (ctypes.c_int32 * max(1, len(keep)))(*keep),
        len(keep), None)
    assert comp(4, [2, 2]) == tb.BLOOM_EINVAL               # not strictly increasing
    assert comp(4, [1, 0]) == tb.BLOOM_EINVAL
    assert comp(4, [0, 4]) == tb.BLOOM_EINVAL               # index >= batch
    assert comp(4, [-1]) == tb.BLOOM_EINVAL
    assert comp(2, [0, 1, 1]) == tb.BLOOM_EINVAL            # n_keep > batch
    assert comp(5, [0]) == tb.BLOOM_ECAPACITY               # batch > max_batch
    assert comp(4, []) == tb.BLOOM_OK                       # nothing kept: no-op
    assert f.kv.len == 8


def test_softmax_validation_paths():
    sm = lambda *a: tb.lib.alibi_masked_softmax(*a)
    assert sm(0x10, 1, 0x10, 1, 1, 3, 2, 8, 0, 0x10, 0, None) == tb.BLOOM_EINVAL   # Q > K
    assert sm(0x10, 9, 0x10, 1, 1, 1, 2, 8, 0, 0x10, 0, None) == tb.BLOOM_EDTYPE
    assert sm(0x10, 1, 0x10, 1, 1, 1, 2, 8, 0, 0x10, 5, None) == tb.BLOOM_EDTYPE
    assert sm(0x10, 1, 0x10, 1, 4, 1, 2, 8, 6, 0x10, 0, None) == tb.BLOOM_EINVAL   # heads > total
    assert sm(None, 1, None, 1, 1, 1, 2, 8, 0, None, 0, None) == tb.BLOOM_EINVAL
    assert sm(None, 1, None, 0, 1, 1, 2, 8, 0, None, 0, None) == tb.BLOOM_OK       # empty


def test_timer_read_without_launches():
    tb.bloom_timer_disable()
    for cls in (-1, 1, 2, 3):
        ms, n, b = tb.bloom_timer_read(cls)
        assert (ms, n, b) == (0.0, 0, 0.0)


def test_prefill_and_decode_need_tokens_or_hidden_out():
    f = _Fake(bi.BLOOM_560M)
    call = lambda nxt, hid: tb.lib.bloom_prefill(
        ctypes.byref(f.cfg), ctypes.byref(f.w), ctypes.byref(f.kv), 2, 8, 0x1000, 0x1000, nxt,
        hid, 0x1000, 1024, None)
    # neither output: EINVAL; either one passes that check (and then fails the workspace)
    assert call(None, None) == tb.BLOOM_EINVAL
    assert call(None, 0x1000) == tb.BLOOM_EWORKSPACE
    assert call(0x1000, None) == tb.BLOOM_EWORKSPACE
    f.kv.prompt_len = f.kv.len = 8
    dec = lambda nxt, hid: tb.lib.bloom_decode_step(
        ctypes.byref(f.cfg), ctypes.byref(f.w), ctypes.byref(f.kv), 2, 0x1000, 0x1000, nxt, hid,
        0x1000, 1024, None)
    assert dec(None, None) == tb.BLOOM_EINVAL
    assert dec(None, 0x1000) == tb.BLOOM_EWORKSPACE


def test_sampling_and_lm_logits_validation_paths():
    smp = lambda *a: tb.lib.bloom_sample_tokens(*a[:7], 0x10 if len(a) < 8 else a[7],
                                                 1 << 30 if len(a) < 9 else a[8], None)
    assert smp(0x10, -1, 8, 0x10, 0x10, 0x10, 0x10) == tb.BLOOM_EINVAL
    assert smp(0x10, 2, 0, 0x10, 0x10, 0x10, 0x10) == tb.BLOOM_EINVAL
    assert smp(0x10, 2, (1 << 23) + 1, 0x10, 0x10, 0x10, 0x10) == tb.BLOOM_EINVAL
    assert smp(0x10, 2, 8, None, 0x10, 0x10, 0x10) == tb.BLOOM_EINVAL
    assert smp(0x10, 2, 8, 0x10, 0x10, 0x10, None) == tb.BLOOM_EINVAL
    assert smp(0x10, 2, 8, 0x10, 0x10, 0x10, 0x10, None) == tb.BLOOM_EINVAL   # no workspace
    need = tb.bloom_sample_workspace_bytes(2, 250880)
    assert need > 0 and tb.bloom_sample_workspace_bytes(128, 250880) > need
    assert smp(0x10, 2, 250880, 0x10, 0x10, 0x10, 0x10, 0x10, need - 1) == tb.BLOOM_EWORKSPACE
    assert smp(None, 0, 8, None, None, None, None) == tb.BLOOM_OK              # empty batch
    f = _Fake(bi.BLOOM_560M)
    lg = lambda w, b, h, out, wsb: tb.lib.bloom_lm_logits(ctypes.byref(f.cfg), w, b, h, out,
                                                          0x1000, wsb, None)
    assert lg(None, 2, 0x10, 0x10, 1 << 40) == tb.BLOOM_EINVAL                  # no weights
    assert lg(ctypes.byref(f.w), -1, 0x10, 0x10, 1 << 40) == tb.BLOOM_EINVAL
    assert lg(ctypes.byref(f.w), 2, None, 0x10, 1 << 40) == tb.BLOOM_EINVAL
    assert lg(ctypes.byref(f.w), 2, 0x10, 0x10, 16) == tb.BLOOM_EWORKSPACE
    assert lg(ctypes.byref(f.w), 0, None, None, 0) == tb.BLOOM_OK


def test_ln_fold_sizes_and_validation_paths():
    """bloom_ln_fold_bytes: per layer 2 (3 Hd + F) float32; bloom_ln_fold rejects non-bf16
    weights, a short buffer, a null buffer and missing weight pointers before launching."""
    m = bi.BLOOM_176B_TP8_RANK0.truncated(2)
    f = _Fake(m)
    n = ctypes.c_size_t(0)
    assert tb.lib.bloom_ln_fold_bytes(ctypes.byref(f.cfg), ctypes.byref(n)) == tb.BLOOM_OK
    hd = m.n_head_local * m.head_dim
    assert n.value == 2 * 2 * (3 * hd + m.ffn) * 4

    def fold(ff, buf=0x1000, nbytes=1 << 40):
        return tb.lib.bloom_ln_fold(ctypes.byref(ff.cfg), ctypes.byref(ff.w), buf, nbytes, None)

    assert fold(f, nbytes=n.value - 4) == tb.BLOOM_EWORKSPACE
    assert fold(f, buf=None) == tb.BLOOM_EINVAL
    f.layers[1].w_up = None
    assert fold(f) == tb.BLOOM_EINVAL
    g = _Fake(bi.BLOOM_176B_INT8.truncated(2))
    assert fold(g) == tb.BLOOM_EDTYPE
