"""Plain float64 CPU oracle of BLOOM greedy KV-cached generation.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product.  Shares no code
with the HIP path.

What it computes, and where the pages say so:

* greedy generation of new tokens with a KV cache ("Incredibly Fast BLOOM Inference
  with DeepSpeed and Accelerate", Benchmark Environment: do_sample=False, KV cache on);
* a pre-LayerNorm decoder layer: input LayerNorm feeding the fused QKV projection,
  attention, the output projection with bias and residual, the post-attention
  LayerNorm feeding the MLP ("DeepSpeed Inference ...", Section III.D, Putting It
  Together: the four fused groups name exactly these steps);
* ALiBi positional bias ("Hugging Face BLOOM Inference Optimization", Efficient
  PyTorch Implementation), with the slopes of the ALiBi paper (Press, Smith and
  Lewis, "Train Short, Test Long", ICLR 2022, Section 3), since the pages give none;
* masked fill of the attention scores followed by a softmax ("Hugging Face BLOOM
  Inference Optimization", Custom CUDA Kernels and Hardware Acceleration); masked
  keys get probability exactly 0;
* the tanh form of GeLU (same page, Kernel Fusion with torch.jit.script, which names
  ``bloom_gelu_forward``), with the Hendrycks-Gimpel constants sqrt(2/pi), 0.044715;
* tied embeddings: the LM head is the embedding matrix.

Readings where the pages are silent (all in float64 unless a caller asks otherwise):
LayerNorm uses the biased variance with eps from the model shape (1e-5); the
ALiBi bias is slope * (key position - left padding), i.e. positions counted over
real tokens only; the bias is added after the 1/sqrt(head_dim) score scale; the
fused QKV rows are ordered [head][q, k, v][head_dim]; every linear has a bias;
int8 weights mean W[r, k] = scale[r] * q[r, k]; a query with no valid key gives a
zero attention output; greedy ties go to the lowest token id, taken on logits
rounded to float32 (the precision the GPU path decides in).

No blocking, fusion or reordering beyond the definitions above, except that the
LM-head product is evaluated over slices of the vocabulary (each logit is still
one dot product) so that a 250880 x 14336 embedding is never widened at once.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# elementary operations
# ---------------------------------------------------------------------------

def alibi_slopes(n_head_total: int, dtype=F64) -> np.ndarray:
    """Per-head ALiBi slopes for a model with ``n_head_total`` heads.

    ALiBi paper, Section 3: for n heads (n a power of two) the slopes are the
    geometric sequence starting at 2^(-8/n) with that same ratio.  For other n, the
    first c = 2^floor(log2 n) heads take the c-head sequence and the remaining
    n - c heads take every other term (the 1st, 3rd, 5th, ...) of the 2c-head
    sequence.
    """
    n = int(n_head_total)
    if n < 1:
        raise ValueError("n_head_total must be >= 1")
    c = 1 << (n.bit_length() - 1)
    seq_c = [2.0 ** (-8.0 * k / c) for k in range(1, c + 1)]
    seq_2c = [2.0 ** (-8.0 * k / (2 * c)) for k in range(1, 2 * c + 1)]
    rest = seq_2c[0::2][: n - c]
    return np.array(seq_c + rest, dtype=dtype)


def layer_norm(x: np.ndarray, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis: gamma * (x - mean) / sqrt(biased var + eps) + beta."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma + beta


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def masked_softmax(s: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """Softmax over the last axis restricted to ``valid`` entries.

    Masked entries get probability exactly 0 (masked_fill with -inf before the
    softmax).  A row with no valid entry is all zeros.
    """
    valid = np.broadcast_to(valid, s.shape)
    filled = np.where(valid, s, -np.inf)
    m = filled.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(valid, np.exp(np.where(valid, filled - m, 0.0)), 0.0)
    z = e.sum(axis=-1, keepdims=True)
    return np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)


def alibi_masked_softmax(scores: np.ndarray, valid_len, n_head_total: int,
                         head_offset: int = 0, dtype=F64) -> np.ndarray:
    """The standalone fused op: ALiBi bias, left-pad + causal mask, softmax.

    ``scores`` [B, H, Q, K] are already scaled by 1/sqrt(head_dim).  Row b has
    ``valid_len[b]`` real keys at the right end (keys j >= K - valid_len[b]); query i
    sits at key position K - Q + i and sees keys up to that position.  Heads are
    global heads head_offset .. head_offset + H - 1 of an n_head_total-head model.
    """
    s = np.asarray(scores, dtype)
    B, H, Q, K = s.shape
    slopes = alibi_slopes(n_head_total, dtype)[head_offset: head_offset + H]
    pad = K - np.asarray(valid_len, dtype=np.int64).reshape(B)
    j = np.arange(K)
    qpos = K - Q + np.arange(Q)
    rel = (j[None, :] - pad[:, None]).astype(dtype)                       # [B, K]
    bias = slopes[None, :, None, None] * rel[:, None, None, :]            # [B, H, 1, K]
    valid = (j[None, None, None, :] >= pad[:, None, None, None]) & \
            (j[None, None, None, :] <= qpos[None, None, :, None])         # [B, 1, Q, K]
    return masked_softmax(s + bias, valid)


class Int8RowScale:
    """Weight-only int8 matrix: W[r, k] = scale[r] * q[r, k]."""

    def __init__(self, q: np.ndarray, scale: np.ndarray):
        self.q = np.asarray(q, dtype=np.int8)
        self.scale = np.asarray(scale)
        if self.scale.shape != (self.q.shape[0],):
            raise ValueError("one scale per output row")

    @property
    def shape(self):
        return self.q.shape

    def dense(self, dtype=F64) -> np.ndarray:
        return self.scale.astype(dtype)[:, None] * self.q.astype(dtype)


def _dense(w, dtype):
    return w.dense(dtype) if isinstance(w, Int8RowScale) else np.asarray(w, dtype=dtype)


def linear(x: np.ndarray, w, b=None, dtype=F64) -> np.ndarray:
    """y = x W^T + b with W stored [out, in]."""
    y = x @ _dense(w, dtype).T
    return y if b is None else y + np.asarray(b, dtype=dtype)


def attention(q: np.ndarray, k_all: np.ndarray, v_all: np.ndarray, slopes: np.ndarray,
              pad: np.ndarray, start: int) -> np.ndarray:
    """ALiBi attention of S new queries over the cached keys.

    q [B, S, H, d] (query s at absolute position start + s); k_all, v_all [B, H, T, d]
    hold positions 0 .. T-1.  Key j is visible to the query at position p iff
    pad[b] <= j <= p.  score = q.k / sqrt(d) + slope_h * (j - pad[b]).
    Returns o [B, S, H, d].
    """
    B, S, H, d = q.shape
    T = k_all.shape[2]
    scores = np.einsum("bshd,bhtd->bhst", q, k_all) / math.sqrt(d)
    j = np.arange(T)
    p = start + np.arange(S)
    rel = (j[None, :] - pad[:, None]).astype(q.dtype)                      # [B, T]
    bias = slopes[None, :, None, None] * rel[:, None, None, :]
    valid = (j[None, None, None, :] >= pad[:, None, None, None]) & \
            (j[None, None, None, :] <= p[None, None, :, None])
    probs = masked_softmax(scores + bias, valid)
    return np.einsum("bhst,bhtd->bshd", probs, v_all)


# ---------------------------------------------------------------------------
# model
# ---------------------------------------------------------------------------

def _widen(a: np.ndarray, storage: str) -> np.ndarray:
    """Exact value of a stored tensor: bf16 / fp16 bit patterns (uint16) or floats."""
    a = np.asarray(a)
    if storage == "bf16" and a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    if storage == "f16" and a.dtype == np.uint16:
        return a.view(np.float16).astype(np.float32)
    return a


def layer_from_storage(shape, lw: dict, dtype=F64, widen_weights: bool = True) -> dict:
    """One decoder layer's parameters from their storage form (see
    OracleModel.from_storage), as the dict that ``decoder_layer`` takes."""
    wd = shape.weight_dtype
    pd = "f32" if wd == "f32" else "bf16"

    def par(a):
        return _widen(a, pd).astype(dtype)

    def mat(field):
        if wd == "int8":
            w8 = Int8RowScale(lw["w_" + field], _widen(lw["s_" + field], "f16"))
            return w8.dense(dtype) if widen_weights else w8
        w = _widen(lw["w_" + field], wd)
        return w.astype(dtype) if widen_weights else w

    return {
        "ln1": (par(lw["ln1_g"]), par(lw["ln1_b"])),
        "qkv": mat("qkv"), "b_qkv": par(lw["b_qkv"]),
        "dense": mat("dense"), "b_dense": par(lw["b_dense"]),
        "ln2": (par(lw["ln2_g"]), par(lw["ln2_b"])),
        "up": mat("up"), "b_up": par(lw["b_up"]),
        "down": mat("down"), "b_down": par(lw["b_down"]),
    }


@dataclasses.dataclass
class OracleModel:
    """Shape plus weight values of one BLOOM stack (whole model or one TP share)."""
    n_layer: int
    hidden: int
    n_head_total: int
    head_offset: int
    n_head_local: int
    head_dim: int
    ffn: int
    vocab: int
    embed_ln: bool
    ln_eps: float
    embed: np.ndarray
    emb_ln: Optional[tuple]
    lnf: tuple
    layers: List[dict]
    dtype: type = F64
    act_round: Optional[object] = None   # the four linears' inputs (int8 activations)
    kv_round: Optional[object] = None    # new keys / values (int8 KV cache)

    @classmethod
    def from_storage(cls, shape, tensors: dict, dtype=F64, widen_weights: bool = True):
        """Build from a shape (attributes as in the workload description) and tensors in
        storage form: bf16 as uint16 bits, fp16 scales as uint16 bits, int8, float32.

        widen_weights=True converts every layer matrix to ``dtype`` once (int8 ones are
        dequantised, W = s q); False keeps the stored form and widens at each use.
        Either way the arithmetic is the same."""
        wd = shape.weight_dtype
        pd = "f32" if wd == "f32" else "bf16"

        def par(a):
            return _widen(a, pd).astype(dtype)

        layers = [layer_from_storage(shape, lw, dtype, widen_weights)
                  for lw in tensors["layers"]]
        emb_ln = None
        if shape.embed_ln:
            emb_ln = (par(tensors["emb_ln_g"]), par(tensors["emb_ln_b"]))
        # int8 activations (W8A8) and an int8 KV cache are part of what those modes
        # compute; every other storage type is an implementation precision, and the
        # oracle stays exact for it
        act_int8 = getattr(shape, "act_dtype", None) == "int8"
        kv_int8 = getattr(shape, "kv_dtype", None) == "int8"
        return cls(n_layer=len(layers), hidden=shape.hidden, n_head_total=shape.n_head_total,
                   head_offset=shape.head_offset, n_head_local=shape.n_head_local,
                   head_dim=shape.head_dim, ffn=shape.ffn, vocab=shape.vocab,
                   embed_ln=bool(shape.embed_ln), ln_eps=float(shape.ln_eps),
                   embed=_widen(tensors["embed"], pd), emb_ln=emb_ln,
                   lnf=(par(tensors["lnf_g"]), par(tensors["lnf_b"])), layers=layers,
                   dtype=dtype, act_round=int8_rows if act_int8 else None,
                   kv_round=int8_rows if kv_int8 else None)

    @property
    def slopes(self) -> np.ndarray:
        all_slopes = alibi_slopes(self.n_head_total, self.dtype)
        return all_slopes[self.head_offset: self.head_offset + self.n_head_local]


def new_cache(model: OracleModel, batch: int) -> list:
    H, d = model.n_head_local, model.head_dim
    empty = np.zeros((batch, H, 0, d), dtype=model.dtype)
    return [{"k": empty, "v": empty} for _ in range(model.n_layer)]


def forward(model: OracleModel, tokens: np.ndarray, start: int, pad: np.ndarray,
            cache: list, trace: Optional[list] = None) -> np.ndarray:
    """Run S new tokens per row through the stack, appending their K/V to ``cache``.

    tokens [B, S] sit at absolute positions start .. start+S-1; ``cache`` already holds
    positions 0 .. start-1.  pad[b] = number of left-pad slots of row b.  Returns the
    final-LayerNorm hidden state [B, S, hidden].  If ``trace`` is a list, the residual
    stream after every layer is appended to it.
    """
    dt = model.dtype
    tokens = np.asarray(tokens)
    pad = np.asarray(pad, dtype=np.int64)
    if cache[0]["k"].shape[2] != start:
        raise ValueError("cache length does not match start position")
    x = np.asarray(model.embed[tokens], dtype=dt)
    if model.embed_ln:
        x = layer_norm(x, model.emb_ln[0], model.emb_ln[1], model.ln_eps)
    for li, lw in enumerate(model.layers):
        x = decoder_layer(model, lw, x, pad, start, cache[li], act=model.act_round,
                          kv=model.kv_round)
        if trace is not None:
            trace.append(x.copy())
    return layer_norm(x, model.lnf[0], model.lnf[1], model.ln_eps)


def quantize_int8(a: np.ndarray):
    """Symmetric int8 quantisation with one scale per slice along the last axis (the
    pages name DeepSpeed's INT8 inference, "DeepSpeed Inference ...", Section VII.B,
    without its scheme; this is the plain symmetric per-slice form): with
    amax = max |a| over the slice, the code of each value is the nearest integer (ties
    to even) to a * (127 / amax), clamped to [-127, 127], and the scale is amax / 127; a
    slice of zeros has codes 0 and scale 0.  The decisions are taken in float32, the
    precision the kernels take them in: a is rounded to float32, 127 / amax and the
    product are float32 operations.  Returns (codes int8, scale float32 with a trailing
    axis of 1)."""
    f = np.asarray(a, dtype=np.float32)
    amax = np.max(np.abs(f), axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(127.0) / amax, np.float32(0.0)).astype(np.float32)
    codes = np.clip(np.rint(f * inv), -127, 127).astype(np.int8)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    return codes, scale


def dequantize_int8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """The value an int8 code stands for: code * scale, exact in float64."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)


def int8_rows(a: np.ndarray) -> np.ndarray:
    """The values an int8 path carries for a: quantize_int8 then dequantize_int8 (per
    slice along the last axis)."""
    return dequantize_int8(*quantize_int8(a))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, returned as float64: the
    value is first rounded to float32, then its low 16 bits are rounded away."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def decoder_layer(model: OracleModel, lw: dict, x: np.ndarray, pad: np.ndarray, start: int,
                  c: dict, act=None, kv=None) -> np.ndarray:
    """One pre-LayerNorm decoder layer ("DeepSpeed Inference ...", Section III.D) on the
    residual stream x [B, S, hidden] at positions start .. start+S-1, appending the
    layer's K/V to the cache entry ``c`` ({"k", "v"}: [B, H, start, d]).  Only the shape
    fields, ln_eps and the ALiBi slopes of ``model`` are used.

    ``act`` (optional) is applied to the input of each of the four linears (both
    LayerNorm outputs, the attention output [B, S, H*d], the GeLU output), and ``kv``
    (optional; default ``act``) to the new keys and values [B, S, H, d], before they
    enter the cache; the residual stream and q are left exact.  Either is a rounding to
    a narrower type (e.g. round_bf16, a yardstick of a path's storage precision) or, for
    the int8 modes, part of the method itself (int8_rows: W8A8 per-token activations;
    per-(token, head) int8 keys and values).  Without them every value stays in
    ``model.dtype``."""
    dt = model.dtype
    r = act if act is not None else (lambda t: t)
    rk = kv if kv is not None else r
    pad = np.asarray(pad, dtype=np.int64)
    B, S = x.shape[:2]
    H, d = model.n_head_local, model.head_dim
    a = r(layer_norm(x, lw["ln1"][0], lw["ln1"][1], model.ln_eps))
    qkv = linear(a, lw["qkv"], lw["b_qkv"], dt).reshape(B, S, H, 3, d)
    q, k, v = qkv[:, :, :, 0, :], rk(qkv[:, :, :, 1, :]), rk(qkv[:, :, :, 2, :])
    c["k"] = np.concatenate([c["k"], k.transpose(0, 2, 1, 3)], axis=2)
    c["v"] = np.concatenate([c["v"], v.transpose(0, 2, 1, 3)], axis=2)
    o = r(attention(q, c["k"], c["v"], model.slopes, pad, start).reshape(B, S, H * d))
    x = x + linear(o, lw["dense"], lw["b_dense"], dt)
    a2 = r(layer_norm(x, lw["ln2"][0], lw["ln2"][1], model.ln_eps))
    u = r(gelu_tanh(linear(a2, lw["up"], lw["b_up"], dt)))
    return x + linear(u, lw["down"], lw["b_down"], dt)


def lm_logits(model: OracleModel, hidden: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """Tied LM head: logits = hidden E^T, one dot product per logit (vocab taken in slices)."""
    hidden = np.asarray(hidden, dtype=model.dtype)
    out = np.empty(hidden.shape[:-1] + (model.vocab,), dtype=model.dtype)
    for v0 in range(0, model.vocab, chunk):
        e = np.asarray(model.embed[v0: v0 + chunk], dtype=model.dtype)
        out[..., v0: v0 + chunk] = hidden @ e.T
    return out


@dataclasses.dataclass
class GenerateResult:
    tokens: np.ndarray        # [B, n_new] oracle greedy choice at each step
    hidden: np.ndarray        # [n_new, B, hidden] final-LN state that produced each token
    top1: np.ndarray          # [n_new, B] largest logit
    top2: np.ndarray          # [n_new, B] second largest logit
    rms: np.ndarray           # [n_new, B] root-mean-square of the logits row
    chosen: Optional[np.ndarray]  # [n_new, B] oracle logit of the forced token (teacher forcing)
    cache: list


def stop_rule(tokens: np.ndarray, eos_id: int, max_new, pad_id: int):
    """Per-row end of generation ("Hugging Face BLOOM Inference Optimization", Webserver
    Architecture and Request Handling: requests in one batch end at their own limits).
    Row b ends at its first step t whose token is eos_id (kept) or at t = max_new[b] - 1;
    later tokens become pad_id.  tokens [B, n]; eos_id < 0 for none; max_new None or [B].
    Returns (tokens with the rule applied, tokens per row)."""
    tokens = np.array(tokens, copy=True)
    B, n = tokens.shape
    lengths = np.full(B, n, dtype=np.int64)
    for b in range(B):
        limit = n if max_new is None else max(1, min(n, int(max_new[b])))
        end = limit
        for t in range(limit):
            if eos_id >= 0 and tokens[b, t] == eos_id:
                end = t + 1
                break
        tokens[b, end:] = pad_id
        lengths[b] = end
    return tokens, lengths


def greedy_argmax(logits: np.ndarray) -> np.ndarray:
    """Lowest token id among the maxima, decided on float32-rounded logits."""
    return np.argmax(logits.astype(np.float32), axis=-1).astype(np.int32)


def greedy_generate(model: OracleModel, prompt: np.ndarray, valid_len, n_new: int,
                    forced: Optional[np.ndarray] = None) -> GenerateResult:
    """Greedy generation of ``n_new`` tokens: one forward over the left-padded prompt
    (which yields token 1), then one single-token forward per further token.

    With ``forced`` [B, n_new] (teacher forcing) the token fed back at step t is
    forced[:, t] instead of the oracle's own choice; the oracle's choice and the
    logit of the forced token are still recorded.
    """
    prompt = np.asarray(prompt)
    B, P = prompt.shape
    pad = P - np.asarray(valid_len, dtype=np.int64).reshape(B)
    cache = new_cache(model, B)
    toks = np.zeros((B, n_new), dtype=np.int32)
    hid = np.zeros((n_new, B, model.hidden), dtype=model.dtype)
    top1 = np.zeros((n_new, B)); top2 = np.zeros((n_new, B)); rms = np.zeros((n_new, B))
    chosen = None if forced is None else np.zeros((n_new, B))
    h = forward(model, prompt, 0, pad, cache)[:, -1]
    for t in range(n_new):
        logits = lm_logits(model, h)
        toks[:, t] = greedy_argmax(logits)
        hid[t] = h
        part = np.partition(logits, -2, axis=-1)
        top1[t], top2[t] = part[:, -1], part[:, -2]
        rms[t] = np.sqrt(np.mean(logits ** 2, axis=-1))
        nxt = toks[:, t]
        if forced is not None:
            nxt = np.asarray(forced[:, t], dtype=np.int32)
            chosen[t] = logits[np.arange(B), nxt]
        if t + 1 < n_new:
            h = forward(model, nxt[:, None], P + t, pad, cache)[:, 0]
    return GenerateResult(toks, hid, top1, top2, rms, chosen, cache)


# ---------------------------------------------------------------------------
# per-row sampling (temperature, nucleus / top-p)
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class SampleResult:
    tokens: np.ndarray        # [B] chosen token ids
    keep_margin: np.ndarray   # [B] distance of top_p from the nucleus' cumulative-mass bounds
    draw_margin: np.ndarray   # [B] distance of u from the chosen token's CDF interval bounds
    nucleus_size: np.ndarray  # [B] tokens in the nucleus


def sample_tokens(logits: np.ndarray, temperature, top_p, uniform) -> SampleResult:
    """One sampled token per row ("Hugging Face BLOOM Inference Optimization", Webserver
    Architecture and Request Handling: the custom generation loop applies its own
    sampling parameters, e.g. top-p, to each member of a batch).  The pages define
    neither step, so the textbook definitions are used (float64):

    * temperature T <= 0: greedy, the lowest id among the largest logits (decided on
      float32-rounded logits, as ``greedy_argmax``); so is a positive T whose
      reciprocal overflows float32 (T below about 2.9e-39): softmax(logits / T) tends
      to the largest logits as T -> 0, and the temperature is an input of float32
      precision, so the limit is taken once 1/T has no float32 value;
    * otherwise q = softmax(logits / T);
    * nucleus (Holtzman et al., "The Curious Case of Neural Text Degeneration", ICLR
      2020, Section 3.1): sort q in decreasing order and take the shortest prefix whose
      mass reaches top_p; every token whose q equals the last one taken is kept too
      (ties are not broken by id).  top_p >= 1 keeps every token; top_p <= 0 keeps the
      tokens of the largest q only;
    * the draw: the kept tokens in increasing id order, with cumulative mass F (over the
      kept mass M), give the first id whose F exceeds u * M; u in [0, 1) is an input.

    The margins say how far the decisions are from their rounding-sensitive edges, in
    units of the (normalised) mass: keep_margin = distance of top_p from the cumulative
    mass just before and just after the last kept group of equal q; draw_margin =
    distance of u * M / M from the ends of the chosen token's interval.
    """
    logits = np.asarray(logits, dtype=F64)
    B, V = logits.shape
    T = np.asarray(temperature, dtype=F64).reshape(B)
    P = np.asarray(top_p, dtype=F64).reshape(B)
    U = np.asarray(uniform, dtype=F64).reshape(B)
    toks = np.zeros(B, dtype=np.int32)
    keep_m = np.full(B, np.inf)
    draw_m = np.full(B, np.inf)
    size = np.zeros(B, dtype=np.int64)
    for b in range(B):
        with np.errstate(over="ignore", divide="ignore"):
            inv_t32 = np.float32(1.0) / np.float32(T[b]) if T[b] > 0 else np.float32(0)
        if not T[b] > 0 or not np.isfinite(inv_t32):
            toks[b] = int(np.argmax(logits[b].astype(np.float32)))
            size[b] = 1
            continue
        z = logits[b] / T[b]
        q = np.exp(z - z.max())
        q = q / q.sum()
        if P[b] >= 1:
            keep = q > 0
        else:
            order = np.argsort(-q, kind="stable")
            qs = q[order]
            cum = np.cumsum(qs)
            # shortest prefix whose mass reaches top_p (at least one token)
            k = int(np.searchsorted(cum, P[b], side="left")) if P[b] > 0 else 0
            k = min(k, V - 1)
            last = qs[k]
            keep = q >= last
            # mass before the group of values equal to `last`, and with it
            before = float(q[q > last].sum())
            upto = float(q[keep].sum())
            keep_m[b] = min(P[b] - before, upto - P[b]) if P[b] > 0 else upto
        idx = np.nonzero(keep)[0]
        mass = q[idx]
        M = mass.sum()
        F = np.cumsum(mass) / M
        j = int(np.searchsorted(F, U[b], side="right"))
        j = min(j, len(idx) - 1)
        toks[b] = int(idx[j])
        lo = F[j - 1] if j > 0 else 0.0
        draw_m[b] = min(U[b] - lo, F[j] - U[b])
        size[b] = len(idx)
    return SampleResult(toks, keep_m, draw_m, size)
