"""Python binding of the MI355X (gfx950) BLOOM greedy-decode library.

Argument marshalling only: torch tensors supply device memory and the HIP stream,
and every step of the hot path runs in the HIP kernels of ``libbloom_mi355x.so``
(declared in ``include/bloom.h``).  The functions below carry the C names
(``bloom_prefill``, ``bloom_decode_step``, ``alibi_masked_softmax``,
``kv_cache_append``, ...) and raise ``BloomError`` on a non-zero status.

Importing this package loads the shared library and fails loudly if it has not been
built (``python transformer_bloom_decode_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbloom_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "bloom.h")

BLOOM_OK, BLOOM_EINVAL, BLOOM_EDTYPE, BLOOM_ECAPACITY, BLOOM_EWORKSPACE, BLOOM_EHIP = (
    0, -1, -2, -3, -4, -5)
BLOOM_F32, BLOOM_BF16, BLOOM_INT8_ROWSCALE, BLOOM_F16 = 0, 1, 2, 3
DTYPE_CODES = {"f32": BLOOM_F32, "bf16": BLOOM_BF16, "int8": BLOOM_INT8_ROWSCALE,
               "f16": BLOOM_F16}

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32


class bloom_config(ctypes.Structure):
    _fields_ = [("n_layer", _i32), ("hidden", _i32), ("n_head_total", _i32),
                ("head_offset", _i32), ("n_head_local", _i32), ("head_dim", _i32),
                ("ffn", _i32), ("vocab", _i32), ("weight_dtype", _i32), ("embed_ln", _i32),
                ("ln_eps", ctypes.c_float), ("act_dtype", _i32), ("kv_dtype", _i32)]


LAYER_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "s_qkv", "w_dense", "b_dense", "s_dense",
                "ln2_g", "ln2_b", "w_up", "b_up", "s_up", "w_down", "b_down", "s_down")


class bloom_layer_weights(ctypes.Structure):
    _fields_ = [(f, _c_void_p) for f in LAYER_FIELDS]


class bloom_weights(ctypes.Structure):
    _fields_ = [("embed", _c_void_p), ("emb_ln_g", _c_void_p), ("emb_ln_b", _c_void_p),
                ("lnf_g", _c_void_p), ("lnf_b", _c_void_p),
                ("layers", ctypes.POINTER(bloom_layer_weights)), ("ln_fold", _c_void_p)]


class bloom_kv_cache(ctypes.Structure):
    _fields_ = [("k", _c_void_p), ("v", _c_void_p), ("max_batch", _i32), ("max_len", _i32),
                ("len", _i32), ("prompt_len", _i32), ("d_len", _c_void_p),
                ("k_scale", _c_void_p), ("v_scale", _c_void_p)]


class bloom_gen_control(ctypes.Structure):
    _fields_ = [("eos_id", _i32), ("pad_id", _i32), ("d_max_new", _c_void_p),
                ("d_out_len", _c_void_p), ("d_temperature", _c_void_p), ("d_top_p", _c_void_p),
                ("d_uniform", _c_void_p), ("d_logits", _c_void_p), ("d_sample_ws", _c_void_p),
                ("sample_ws_bytes", ctypes.c_size_t)]


class BloomError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = f"{where}: {bloom_status_string(code)} ({code})"
        if code == BLOOM_EHIP:
            msg += f": {lib.bloom_last_hip_error().decode()}"
        super().__init__(msg)


def _load():
    # torch ships its own HIP runtime (libamdhip64.so.7 + libhsa-runtime64.so).  Loading
    # torch first makes the dynamic loader bind this library's libamdhip64.so.7
    # dependency to that same, already-loaded runtime; loading this library first
    # would bring in a second HSA runtime next to torch's, which can fail to open the
    # device.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run transformer_bloom_decode_amd/build.py "
                          "(the HIP library is required: there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = _c_void_p
    lib.bloom_status_string.argtypes = [ctypes.c_int]
    lib.bloom_status_string.restype = ctypes.c_char_p
    lib.bloom_last_hip_error.argtypes = []
    lib.bloom_last_hip_error.restype = ctypes.c_char_p
    lib.bloom_workspace_bytes.argtypes = [P(bloom_config), _i32, _i32, P(ctypes.c_size_t)]
    lib.bloom_prefill.argtypes = [P(bloom_config), P(bloom_weights), P(bloom_kv_cache), _i32, _i32,
                                  vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bloom_decode_step.argtypes = [P(bloom_config), P(bloom_weights), P(bloom_kv_cache), _i32,
                                      vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.bloom_generate.argtypes = [P(bloom_config), P(bloom_weights), P(bloom_kv_cache), _i32,
                                   _i32, vp, vp, _i32, vp, vp, P(bloom_gen_control), vp,
                                   ctypes.c_size_t, vp]
    lib.alibi_masked_softmax.argtypes = [vp, _i32, vp, _i32, _i32, _i32, _i32, _i32, _i32, vp,
                                         _i32, vp]
    lib.kv_cache_append.argtypes = [P(bloom_config), P(bloom_kv_cache), _i32, _i32, _i32, vp, vp,
                                    _i32, vp]
    lib.kv_cache_compact.argtypes = [P(bloom_config), P(bloom_kv_cache), _i32, P(_i32), _i32, vp]
    lib.bloom_lm_logits.argtypes = [P(bloom_config), P(bloom_weights), _i32, vp, vp, vp,
                                    ctypes.c_size_t, vp]
    lib.bloom_sample_tokens.argtypes = [vp, _i32, _i32, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                        vp]
    lib.bloom_sample_workspace_bytes.argtypes = [_i32, _i32, P(ctypes.c_size_t)]
    lib.bloom_init_weights.argtypes = [P(bloom_config), P(bloom_weights), ctypes.c_uint64,
                                       ctypes.c_double, vp]
    lib.bloom_ln_fold_bytes.argtypes = [P(bloom_config), P(ctypes.c_size_t)]
    lib.bloom_ln_fold.argtypes = [P(bloom_config), P(bloom_weights), vp, ctypes.c_size_t, vp]
    lib.bloom_sample_tokens_static.argtypes = [vp, _i32, _i32, vp, vp, vp, vp, vp]
    lib.bloom_sample_scratch_limit.argtypes = [_i32, _i32, P(_i32), P(ctypes.c_size_t)]
    lib.bloom_linear_workspace_bytes.argtypes = [P(bloom_config), _i32, _i32, _i32,
                                                 P(ctypes.c_size_t)]
    lib.bloom_linear.argtypes = [P(bloom_config), _i32, _i32, _i32, vp, vp, vp, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    lib.bloom_timer_enable.argtypes = [_i32]
    lib.bloom_timer_disable.argtypes = []
    lib.bloom_timer_read.argtypes = [_i32, P(ctypes.c_double), P(_i32), P(ctypes.c_double)]
    lib.bloom_timer_pause.argtypes = [_i32]
    for name in ("bloom_workspace_bytes", "bloom_prefill", "bloom_decode_step", "bloom_generate",
                 "alibi_masked_softmax", "kv_cache_append", "kv_cache_compact",
                 "bloom_lm_logits", "bloom_sample_tokens", "bloom_sample_workspace_bytes",
                 "bloom_sample_tokens_static", "bloom_sample_scratch_limit",
                 "bloom_init_weights", "bloom_linear", "bloom_linear_workspace_bytes",
                 "bloom_ln_fold_bytes", "bloom_ln_fold", "bloom_timer_enable",
                 "bloom_timer_disable", "bloom_timer_read", "bloom_timer_pause"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _check(code: int, where: str):
    if code != BLOOM_OK:
        raise BloomError(code, where)


def _ptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# C functions, same names
# ---------------------------------------------------------------------------

def _require(t, numel: int, dtype, name: str, device=None):
    """Raise ValueError unless ``t`` is a contiguous device tensor of ``numel``
    elements of ``dtype`` (on ``device`` when given): the kernels index such buffers
    directly, so a short or mistyped one would be read out of bounds."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: a device tensor is required")
    if t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name}: need a contiguous {dtype} tensor on the GPU, got "
                         f"{t.dtype} on {t.device} (contiguous={t.is_contiguous()})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")


def bloom_status_string(code: int) -> str:
    return lib.bloom_status_string(code).decode()


def bloom_workspace_bytes(cfg: bloom_config, max_batch: int, max_prompt: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.bloom_workspace_bytes(ctypes.byref(cfg), max_batch, max_prompt, ctypes.byref(out)),
           "bloom_workspace_bytes")
    return out.value


def bloom_prefill(cfg, weights, kv, batch: int, prompt_len: int, tokens, valid_len, next_tokens,
                  hidden_out, ws, stream=None):
    w = weights.struct if hasattr(weights, "struct") else weights
    k = kv.struct if hasattr(kv, "struct") else kv
    _check(lib.bloom_prefill(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(k), batch,
                             prompt_len, _ptr(tokens), _ptr(valid_len), _ptr(next_tokens),
                             _ptr(hidden_out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "bloom_prefill")


def bloom_decode_step(cfg, weights, kv, batch: int, tokens, valid_len, next_tokens, hidden_out,
                      ws, stream=None):
    w = weights.struct if hasattr(weights, "struct") else weights
    k = kv.struct if hasattr(kv, "struct") else kv
    _check(lib.bloom_decode_step(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(k), batch,
                                 _ptr(tokens), _ptr(valid_len), _ptr(next_tokens),
                                 _ptr(hidden_out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "bloom_decode_step")


def bloom_generate(cfg, weights, kv, batch: int, prompt_len: int, tokens, valid_len, n_new: int,
                   ids, hidden_out, ws, stream=None, eos_id: Optional[int] = None, pad_id: int = 0,
                   max_new=None, out_len=None, temperature=None, top_p=None, uniform=None,
                   logits=None, sample_ws=None):
    """bloom_generate; eos_id / max_new (device int32 [batch]) / out_len (device int32
    [batch]) and the sampling inputs (temperature, top_p: device float32 [batch];
    uniform: device float32 [n_new, batch]; logits: device float32 [batch, vocab]
    scratch; sample_ws: device bytes) fill a bloom_gen_control when any is given.
    With temperature given and logits / sample_ws not, those are allocated here."""
    w = weights.struct if hasattr(weights, "struct") else weights
    k = kv.struct if hasattr(kv, "struct") else kv
    ctl = None
    if temperature is not None or top_p is not None or uniform is not None:
        import torch
        if temperature is None or top_p is None or uniform is None:
            raise ValueError("temperature, top_p and uniform go together")
        dev = temperature.device
        _require(temperature, batch, torch.float32, "temperature")
        _require(top_p, batch, torch.float32, "top_p", dev)
        _require(uniform, n_new * batch, torch.float32, "uniform", dev)
        if logits is None:
            logits = torch.empty((batch, cfg.vocab), dtype=torch.float32, device=dev)
        _require(logits, batch * cfg.vocab, torch.float32, "logits", dev)
        if sample_ws is None:
            sample_ws = torch.empty(bloom_sample_workspace_bytes(batch, cfg.vocab),
                                    dtype=torch.uint8, device=dev)
    for t, name in ((max_new, "max_new"), (out_len, "out_len")):
        if t is not None:
            import torch
            _require(t, batch, torch.int32, name)
    if (eos_id is not None or max_new is not None or out_len is not None
            or temperature is not None):
        ctl = ctypes.byref(bloom_gen_control(
            -1 if eos_id is None else eos_id, pad_id, _ptr(max_new), _ptr(out_len),
            _ptr(temperature), _ptr(top_p), _ptr(uniform), _ptr(logits), _ptr(sample_ws),
            _nbytes(sample_ws)))
    _check(lib.bloom_generate(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(k), batch,
                              prompt_len, _ptr(tokens), _ptr(valid_len), n_new, _ptr(ids),
                              _ptr(hidden_out), ctl, _ptr(ws), _nbytes(ws), _stream(stream)),
           "bloom_generate")


def alibi_masked_softmax(scores, in_dtype: int, valid_len, B: int, H: int, Q: int, K: int,
                         n_head_total: int, head_offset: int, probs, out_dtype: int, stream=None):
    _check(lib.alibi_masked_softmax(_ptr(scores), in_dtype, _ptr(valid_len), B, H, Q, K,
                                    n_head_total, head_offset, _ptr(probs), out_dtype,
                                    _stream(stream)), "alibi_masked_softmax")


def kv_cache_append(cfg, kv, layer: int, batch: int, pos: int, k, v, n_new: int, stream=None):
    s = kv.struct if hasattr(kv, "struct") else kv
    _check(lib.kv_cache_append(ctypes.byref(cfg), ctypes.byref(s), layer, batch, pos, _ptr(k),
                               _ptr(v), n_new, _stream(stream)), "kv_cache_append")


def kv_cache_compact(cfg, kv, batch: int, keep, stream=None):
    """Rows keep[i] of the cache -> row i (keep: host sequence of strictly increasing ints)."""
    s = kv.struct if hasattr(kv, "struct") else kv
    arr = (_i32 * max(1, len(keep)))(*[int(k) for k in keep])
    _check(lib.kv_cache_compact(ctypes.byref(cfg), ctypes.byref(s), batch, arr, len(keep),
                                _stream(stream)), "kv_cache_compact")


def bloom_lm_logits(cfg, weights, batch: int, hidden, logits, ws, stream=None):
    w = weights.struct if hasattr(weights, "struct") else weights
    _check(lib.bloom_lm_logits(ctypes.byref(cfg), ctypes.byref(w), batch, _ptr(hidden),
                               _ptr(logits), _ptr(ws), _nbytes(ws), _stream(stream)),
           "bloom_lm_logits")


def bloom_linear_workspace_bytes(cfg, M: int, N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.bloom_linear_workspace_bytes(ctypes.byref(cfg), M, N, K, ctypes.byref(out)),
           "bloom_linear_workspace_bytes")
    return out.value


def bloom_linear(cfg, M: int, N: int, K: int, x, w, s, b, y, ws, stream=None):
    """y = x W^T (* s) (+ b) with the library's linear kernels (bloom.h, bloom_linear)."""
    _check(lib.bloom_linear(ctypes.byref(cfg), M, N, K, _ptr(x), _ptr(w), _ptr(s), _ptr(b),
                            _ptr(y), _ptr(ws), _nbytes(ws), _stream(stream)), "bloom_linear")


def bloom_sample_workspace_bytes(batch: int, vocab: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.bloom_sample_workspace_bytes(batch, vocab, ctypes.byref(out)),
           "bloom_sample_workspace_bytes")
    return out.value


def bloom_sample_tokens(logits, batch: int, vocab: int, temperature, top_p, uniform, tokens,
                        ws=None, stream=None):
    """bloom_sample_tokens; without `ws` a workspace of the required size is allocated
    on the logits' device for this call."""
    if batch > 0:
        import torch
        _require(logits, batch * vocab, torch.float32, "logits")
        for t, name in ((temperature, "temperature"), (top_p, "top_p"),
                        (uniform, "uniform")):
            _require(t, batch, torch.float32, name, logits.device)
        _require(tokens, batch, torch.int32, "tokens", logits.device)
    if ws is None and batch > 0:
        import torch
        ws = torch.empty(bloom_sample_workspace_bytes(batch, vocab), dtype=torch.uint8,
                         device=logits.device)
    _check(lib.bloom_sample_tokens(_ptr(logits), batch, vocab, _ptr(temperature), _ptr(top_p),
                                   _ptr(uniform), _ptr(tokens), _ptr(ws), _nbytes(ws),
                                   _stream(stream)), "bloom_sample_tokens")


def bloom_sample_tokens_static(logits, batch: int, vocab: int, temperature, top_p, uniform,
                               tokens, stream=None):
    """bloom_sample_tokens_static: the library's per-GPU scratch array, no workspace."""
    if batch > 0:
        import torch
        _require(logits, batch * vocab, torch.float32, "logits")
        for t, name in ((temperature, "temperature"), (top_p, "top_p"),
                        (uniform, "uniform")):
            _require(t, batch, torch.float32, name, logits.device)
        _require(tokens, batch, torch.int32, "tokens", logits.device)
    _check(lib.bloom_sample_tokens_static(_ptr(logits), batch, vocab, _ptr(temperature),
                                          _ptr(top_p), _ptr(uniform), _ptr(tokens),
                                          _stream(stream)), "bloom_sample_tokens_static")


def bloom_sample_scratch_limit(batch: int, vocab: int):
    """(fits, scratch bytes) of bloom_sample_tokens_static for these rows."""
    fits, nbytes = _i32(0), ctypes.c_size_t(0)
    _check(lib.bloom_sample_scratch_limit(batch, vocab, ctypes.byref(fits), ctypes.byref(nbytes)),
           "bloom_sample_scratch_limit")
    return bool(fits.value), nbytes.value


def bloom_timer_enable(max_launches: int):
    _check(lib.bloom_timer_enable(max_launches), "bloom_timer_enable")


def bloom_timer_disable():
    _check(lib.bloom_timer_disable(), "bloom_timer_disable")


def bloom_timer_pause(paused: bool):
    _check(lib.bloom_timer_pause(int(bool(paused))), "bloom_timer_pause")


KERNEL_CLASSES = {2: "k_gemv_valu", 5: "k_gemm_f32", 6: "k_gemm_lg"}


def bloom_timer_read(kernel_class: int = -1):
    """(total ms, launches, weight bytes) of the timed launches of one kernel class."""
    ms, n, b = ctypes.c_double(0), _i32(0), ctypes.c_double(0)
    _check(lib.bloom_timer_read(kernel_class, ctypes.byref(ms), ctypes.byref(n),
                                ctypes.byref(b)), "bloom_timer_read")
    return ms.value, n.value, b.value


def _nbytes(t) -> int:
    if t is None:
        return 0
    return t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# marshalling helpers: build the C structs from torch device tensors
# ---------------------------------------------------------------------------

def make_config(shape) -> bloom_config:
    """bloom_config from any object with the shape attributes (n_layer, hidden, ...;
    act_dtype 'f32', 'f16', 'bf16' or 'int8'; kv_dtype, default the activation type)."""
    act = DTYPE_CODES[getattr(shape, "act_dtype", "f32" if shape.weight_dtype == "f32"
                              else "bf16")]
    kv = DTYPE_CODES[getattr(shape, "kv_dtype", None) or
                     getattr(shape, "act_dtype", "f32" if shape.weight_dtype == "f32"
                             else "bf16")]
    return bloom_config(shape.n_layer, shape.hidden, shape.n_head_total, shape.head_offset,
                        shape.n_head_local, shape.head_dim, shape.ffn, shape.vocab,
                        DTYPE_CODES[shape.weight_dtype], int(bool(shape.embed_ln)),
                        float(shape.ln_eps), act, kv)


def bloom_init_weights(cfg, weights, seed: int = 0, sigma: float = 0.02, stream=None):
    """Fill the weights' device buffers with the seeded synthetic values (bloom.h)."""
    w = weights.struct if hasattr(weights, "struct") else weights
    _check(lib.bloom_init_weights(ctypes.byref(cfg), ctypes.byref(w), seed, sigma,
                                  _stream(stream)), "bloom_init_weights")


def bloom_ln_fold_bytes(cfg) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.bloom_ln_fold_bytes(ctypes.byref(cfg), ctypes.byref(n)), "bloom_ln_fold_bytes")
    return n.value


def bloom_ln_fold(cfg, weights, fold, stream=None):
    """Write the LayerNorm fold vectors of the weights into `fold` (float32 device tensor of
    bloom_ln_fold_bytes(cfg) bytes; bloom.h)."""
    import torch
    w = weights.struct if hasattr(weights, "struct") else weights
    _require(fold, bloom_ln_fold_bytes(cfg) // 4, torch.float32, "fold")
    _check(lib.bloom_ln_fold(ctypes.byref(cfg), ctypes.byref(w), _ptr(fold), _nbytes(fold),
                             _stream(stream)), "bloom_ln_fold")


def to_device(a, device="cuda"):
    """numpy array (float32, int8, or uint16 bit patterns) -> torch device tensor, same bytes."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceWeights:
    """Device tensors of one model plus the bloom_weights struct pointing at them."""

    def __init__(self, globals_: dict, layers: Sequence[dict]):
        self.tensors = {"globals": globals_, "layers": list(layers)}
        self._layer_arr = (bloom_layer_weights * len(layers))()
        for i, lw in enumerate(layers):
            for f in LAYER_FIELDS:
                setattr(self._layer_arr[i], f, _ptr(lw.get(f)))
        g = globals_
        self.struct = bloom_weights(_ptr(g["embed"]), _ptr(g.get("emb_ln_g")),
                                    _ptr(g.get("emb_ln_b")), _ptr(g["lnf_g"]), _ptr(g["lnf_b"]),
                                    self._layer_arr)

    def fold_layernorm(self, cfg, stream=None):
        """Compute the LayerNorm fold vectors (bloom_ln_fold) into a new device buffer and
        point the struct at it: one-row passes then fold LN1 / LN2 into the QKV / MLP-up
        GEMVs where the library supports it.  Only for BF16 weights; a no-op otherwise."""
        import torch
        if cfg.weight_dtype != BLOOM_BF16:
            return self
        self.fold = torch.empty(bloom_ln_fold_bytes(cfg) // 4, dtype=torch.float32,
                                device="cuda")
        bloom_ln_fold(cfg, self, self.fold, stream)
        self.struct.ln_fold = _ptr(self.fold)
        return self

    def unfold_layernorm(self):
        """Stop folding (the struct's ln_fold back to NULL)."""
        self.struct.ln_fold = None
        return self

    @classmethod
    def from_arrays(cls, tensors: dict, device="cuda"):
        """From {'embed': ..., 'lnf_g': ..., 'layers': [{field: array}]} host arrays."""
        g = {k: to_device(v, device) for k, v in tensors.items() if k != "layers"}
        layers = [{k: to_device(v, device) for k, v in lw.items()} for lw in tensors["layers"]]
        return cls(g, layers)


class KVCache:
    """Caller-owned KV cache buffers ([n_layer][max_batch][H][max_len][d]) and the struct.
    device_len=True also keeps the length in device memory (bloom_kv_cache.d_len).  An
    int8 cache also holds float32 scales k_scale / v_scale [n_layer][max_batch][H][max_len];
    with `fill` given, the scales take that value and the int8 codes -128."""

    def __init__(self, cfg: bloom_config, max_batch: int, max_len: int, device="cuda",
                 fill: Optional[float] = None, device_len: bool = False):
        import torch
        dt = {BLOOM_F32: torch.float32, BLOOM_F16: torch.float16,
              BLOOM_INT8_ROWSCALE: torch.int8}.get(cfg.kv_dtype, torch.bfloat16)
        shape = (cfg.n_layer, max_batch, cfg.n_head_local, max_len, cfg.head_dim)

        def buf(shp, dtype, value):
            if fill is None:
                return torch.empty(shp, dtype=dtype, device=device)
            return torch.full(shp, value, dtype=dtype, device=device)

        # int8 codes lie in [-127, 127]: a filled int8 cache holds -128, never a code
        code_fill = -128 if dt == torch.int8 else fill
        self.k = buf(shape, dt, code_fill)
        self.v = buf(shape, dt, code_fill)
        self.k_scale = self.v_scale = None
        if cfg.kv_dtype == BLOOM_INT8_ROWSCALE:
            self.k_scale = buf(shape[:-1], torch.float32, fill)
            self.v_scale = buf(shape[:-1], torch.float32, fill)
        self.d_len = torch.zeros(1, dtype=torch.int32, device=device) if device_len else None
        self.struct = bloom_kv_cache(_ptr(self.k), _ptr(self.v), max_batch, max_len, 0, 0,
                                     _ptr(self.d_len), _ptr(self.k_scale), _ptr(self.v_scale))

    @property
    def len(self) -> int:
        return self.struct.len

    @property
    def prompt_len(self) -> int:
        return self.struct.prompt_len


def workspace(cfg: bloom_config, max_batch: int, max_prompt: int, device="cuda"):
    import torch
    return torch.empty(bloom_workspace_bytes(cfg, max_batch, max_prompt), dtype=torch.uint8,
                       device=device)


def greedy_generate(cfg: bloom_config, weights: DeviceWeights, kv: KVCache, tokens, valid_len,
                    n_new: int, ws, want_hidden: bool = True, stream=None, graph: bool = False):
    """Greedy generation loop ("Incredibly Fast BLOOM Inference with DeepSpeed and
    Accelerate", Benchmark Environment): one bloom_prefill over the left-padded prompt
    (which yields the first new token), then n_new - 1 bloom_decode_step calls.  Token
    ids stay on the device between steps.  With graph=True the whole loop is one
    bloom_generate call, which replays a captured decode step.

    tokens [batch, prompt_len] int32 and valid_len [batch] int32 are device tensors.
    Returns (ids [n_new, batch] int32, hidden [n_new, batch, hidden] float32 or None),
    both on the device; nothing is synchronised in the eager loop (bloom_generate
    returns after its replays have finished).
    """
    import torch
    batch, prompt_len = tokens.shape
    dev = tokens.device
    ids = torch.empty((n_new, batch), dtype=torch.int32, device=dev)
    hid = (torch.empty((n_new, batch, cfg.hidden), dtype=torch.float32, device=dev)
           if want_hidden else None)
    if graph:
        bloom_generate(cfg, weights, kv, batch, prompt_len, tokens, valid_len, n_new, ids, hid,
                       ws, stream)
        return ids, hid
    bloom_prefill(cfg, weights, kv, batch, prompt_len, tokens, valid_len, ids[0],
                  None if hid is None else hid[0], ws, stream)
    for t in range(1, n_new):
        bloom_decode_step(cfg, weights, kv, batch, ids[t - 1], valid_len, ids[t],
                          None if hid is None else hid[t], ws, stream)
    return ids, hid
