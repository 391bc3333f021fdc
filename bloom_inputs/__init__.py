"""Seeded synthetic inputs for the BLOOM greedy-decode workloads.

This module only produces inputs (weights, prompt ids, attention scores, left-pad
lengths) and describes the workload shapes.  It holds none of the model's
arithmetic.  The CPU oracle and the GPU library are both fed from here, so they see
bit-identical inputs; neither of them imports the other.

Workload shapes follow the pages' problem statement: BLOOM with ALiBi, pre-LN, a
tanh-GeLU MLP and tied embeddings, decoded greedily with a KV cache for 100 new
tokens ("Incredibly Fast BLOOM Inference with DeepSpeed and Accelerate",
Benchmark Environment).  There are no trained weights: every tensor is drawn from
the counter hash in ``gen.c`` (SplitMix64 + Irwin-Hall(4) normals), so any slice
of any tensor can be regenerated alone, on any host, with the same bits.

Seeds: 0 weights, 1 prompt ids, 2 attention scores, 3 left-pad lengths.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libbloom_inputs.so")
_lib = None

SEED_WEIGHTS, SEED_PROMPTS, SEED_SCORES, SEED_LENGTHS = 0, 1, 2, 3
INIT_STD = 0.02
_KIND = {"f32": 0, "bf16": 1, "f16": 2}


def build(verbose: bool = False) -> str:
    """Compile gen.c into libbloom_inputs.so with gcc (IEEE fp32, no fast-math)."""
    import subprocess

    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c99", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, f64, f32 = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int,
                               ctypes.c_double, ctypes.c_float)
    vp = ctypes.c_void_p
    lib.bi_fill_normal.argtypes = [u64, u64, u64, f64, f32, i32, vp, i32]
    lib.bi_fill_int8.argtypes = [u64, u64, u64, vp, i32]
    lib.bi_fill_scale_f16.argtypes = [u64, u64, u64, f32, vp, i32]
    lib.bi_fill_ids.argtypes = [u64, u64, u64, i64, u64, vp]
    lib.bi_hash.argtypes = [u64, u64, u64]
    lib.bi_hash.restype = u64
    lib.bi_f32_to_bf16.argtypes = [f32]
    lib.bi_f32_to_bf16.restype = ctypes.c_uint16
    lib.bi_f32_to_f16.argtypes = [f32]
    lib.bi_f32_to_f16.restype = ctypes.c_uint16
    for name in ("bi_fill_normal", "bi_fill_int8", "bi_fill_scale_f16", "bi_fill_ids"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ---------------------------------------------------------------------------
# raw generators
# ---------------------------------------------------------------------------

def hash64(seed: int, tid: int, index: int) -> int:
    return int(_load().bi_hash(seed, tid, index))


def normal(seed: int, tid: int, shape, sigma: float, mean: float = 0.0,
           kind: str = "bf16", out: Optional[np.ndarray] = None,
           threads: Optional[int] = None) -> np.ndarray:
    """Irwin-Hall(4) approximate N(mean, sigma^2); 'bf16'/'f16' return uint16 bit arrays."""
    dt = np.float32 if kind == "f32" else np.uint16
    if out is None:
        out = np.empty(shape, dtype=dt)
    assert out.dtype == dt and out.flags.c_contiguous
    _load().bi_fill_normal(seed, tid, out.size, float(sigma), float(mean), _KIND[kind],
                           out.ctypes.data, threads or default_threads())
    return out


def uniform_int8(seed: int, tid: int, shape, out: Optional[np.ndarray] = None,
                 threads: Optional[int] = None) -> np.ndarray:
    if out is None:
        out = np.empty(shape, dtype=np.int8)
    assert out.dtype == np.int8 and out.flags.c_contiguous
    _load().bi_fill_int8(seed, tid, out.size, out.ctypes.data, threads or default_threads())
    return out


def row_scales_f16(seed: int, tid: int, n: int, s0: float) -> np.ndarray:
    out = np.empty((n,), dtype=np.uint16)
    _load().bi_fill_scale_f16(seed, tid, n, float(s0), out.ctypes.data, default_threads())
    return out


def ids(seed: int, tid: int, shape, lo: int, modulus: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.int32)
    _load().bi_fill_ids(seed, tid, out.size, int(lo), int(modulus), out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits (vectorised; same rule as gen.c)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class ModelShape:
    """Shape of one BLOOM stack on one GPU (a whole model or one tensor-parallel share)."""
    name: str
    n_layer: int
    hidden: int
    n_head_total: int       # heads of the whole model (sets the ALiBi slopes)
    head_offset: int        # first global head held here
    n_head_local: int       # heads held here
    head_dim: int
    ffn: int                # MLP width held here
    vocab: int
    weight_dtype: str       # 'f32' | 'bf16' | 'int8'
    embed_ln: bool = True
    ln_eps: float = 1e-5
    activations: str = "auto"   # 'auto' (float32 for f32 weights, else bf16) | 'f32' | 'f16'
                                # | 'bf16' | 'int8' (per-token int8 inputs of the linears,
                                # with int8 weights)
    kv_cache: str = "auto"      # 'auto' (the activation type) | 'f32' | 'f16' | 'bf16' | 'int8'
    init_std: float = 0.02      # standard deviation of the synthetic weights

    @property
    def param_dtype(self) -> str:
        """Storage type of embeddings, biases and LayerNorm parameters."""
        return "f32" if self.weight_dtype == "f32" else "bf16"

    @property
    def act_dtype(self) -> str:
        """Type of the stored activations and of the KV cache."""
        if self.activations != "auto":
            return self.activations
        return "f32" if self.weight_dtype == "f32" else "bf16"

    @property
    def kv_dtype(self) -> str:
        """Element type of the KV cache (int8: one float32 scale per token and head)."""
        return self.act_dtype if self.kv_cache == "auto" else self.kv_cache

    @property
    def kv_bytes(self) -> float:
        """Bytes per cached key / value element (an int8 cache's scales included)."""
        return {"f32": 4, "f16": 2, "bf16": 2, "int8": 1 + 4.0 / self.head_dim}[self.kv_dtype]

    @property
    def qkv_rows(self) -> int:
        return 3 * self.n_head_local * self.head_dim

    @property
    def attn_width(self) -> int:
        return self.n_head_local * self.head_dim

    def truncated(self, n_layer: int) -> "ModelShape":
        return dataclasses.replace(self, name=f"{self.name}-L{n_layer}", n_layer=n_layer)

    def linear_shapes(self):
        """(field, rows, cols) of the four per-layer linears, [out, in] row-major."""
        h, F = self.hidden, self.ffn
        return (("qkv", self.qkv_rows, h), ("dense", h, self.attn_width),
                ("up", F, h), ("down", h, F))

    def layer_weight_bytes(self) -> int:
        wb = {"f32": 4, "bf16": 2, "int8": 1}[self.weight_dtype]
        pb = 4 if self.param_dtype == "f32" else 2
        total = 0
        for _, r, c in self.linear_shapes():
            total += r * c * wb + r * pb + (2 * r if self.weight_dtype == "int8" else 0)
        total += 4 * self.hidden * pb  # ln1, ln2 gamma/beta
        return total

    def head_bytes(self) -> int:
        pb = 4 if self.param_dtype == "f32" else 2
        return self.vocab * self.hidden * pb + 2 * self.hidden * pb


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelShape
    batches: tuple
    prompt_len: int
    new_tokens: int
    valid_lens: Optional[tuple] = None   # per-row valid prompt lengths (None: no padding)


TINY = ModelShape("tiny", 2, 64, 8, 0, 8, 8, 256, 1024, "f32")
BLOOM_560M = ModelShape("bloom-560m", 24, 1024, 16, 0, 16, 64, 4096, 250880, "bf16")
BLOOM_176B_TP8_RANK0 = ModelShape("bloom-176b-tp8-rank0", 70, 14336, 112, 0, 14, 128, 7168,
                                  250880, "bf16")
BLOOM_176B_INT8 = ModelShape("bloom-176b-int8", 70, 14336, 112, 0, 112, 128, 57344, 250880,
                             "int8")

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, (2,), 8, 20, (8, 5)),
    "bloom-560m": Workload("bloom-560m", BLOOM_560M, (1, 8, 32), 16, 100),
    "bloom-176b-tp8-rank0": Workload("bloom-176b-tp8-rank0", BLOOM_176B_TP8_RANK0,
                                     (1, 8, 32, 128), 16, 100),
    "bloom-176b-int8": Workload("bloom-176b-int8", BLOOM_176B_INT8, (1, 16, 64, 128), 16, 100),
}


@dataclasses.dataclass(frozen=True)
class SoftmaxWorkload:
    """Standalone ALiBi + left-pad mask + softmax over one query row per (batch, head)."""
    batch: int = 32
    heads: int = 14
    q_len: int = 1
    kv_len: int = 2048
    n_head_total: int = 112
    head_offset: int = 0
    score_std: float = 4.0
    min_valid: int = 64


SOFTMAX = SoftmaxWorkload()

# ---------------------------------------------------------------------------
# tensors
# ---------------------------------------------------------------------------

_GLOBAL_TID = {"embed": 1, "emb_ln_g": 2, "emb_ln_b": 3, "lnf_g": 4, "lnf_b": 5}
_LAYER_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_dense", "b_dense", "ln2_g", "ln2_b",
                 "w_up", "b_up", "w_down", "b_down", "s_qkv", "s_dense", "s_up", "s_down")
LINEAR_FIELDS = ("qkv", "dense", "up", "down")
INT8_S0 = INIT_STD / float(np.sqrt((255.0 ** 2 - 1.0) / 12.0))


def tensor_id(name: str, layer: Optional[int] = None) -> int:
    if layer is None:
        return _GLOBAL_TID[name]
    return 1024 + 16 * layer + _LAYER_FIELDS.index(name)


def tensor_shape(m: ModelShape, name: str):
    h = m.hidden
    if name == "embed":
        return (m.vocab, h)
    if name in ("emb_ln_g", "emb_ln_b", "lnf_g", "lnf_b", "ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        return (h,)
    rows = {"qkv": m.qkv_rows, "dense": h, "up": m.ffn, "down": h}
    cols = {"qkv": h, "dense": m.attn_width, "up": h, "down": m.ffn}
    kind, field = name.split("_", 1)
    if kind == "w":
        return (rows[field], cols[field])
    if kind in ("b", "s"):
        return (rows[field],)
    raise KeyError(name)


def tensor(m: ModelShape, name: str, layer: Optional[int] = None, seed: int = SEED_WEIGHTS,
           out: Optional[np.ndarray] = None) -> np.ndarray:
    """One parameter tensor in storage form.

    bf16 and fp16 tensors are uint16 bit arrays, fp32 tensors float32, int8 weights int8.
    Distributions: weights and embeddings N(0, 0.02); biases and LayerNorm beta
    N(0, 0.02); LayerNorm gamma 1 + N(0, 0.02); int8 weights uniform on {-127..127}
    with per-row fp16 scales s0 * U[0.5, 1.5) (s0 chosen so s0 * q has std 0.02).
    """
    tid = tensor_id(name, layer)
    shape = tensor_shape(m, name)
    if name.startswith("w_") and m.weight_dtype == "int8":
        return uniform_int8(seed, tid, shape, out=out)
    if name.startswith("s_"):
        if m.weight_dtype != "int8":
            raise KeyError(f"{name}: row scales exist only for int8 weights")
        s0 = m.init_std / float(np.sqrt((255.0 ** 2 - 1.0) / 12.0))
        return row_scales_f16(seed, tid, shape[0], s0)
    if name.startswith("w_") or name == "embed":
        kind = m.weight_dtype if name.startswith("w_") else m.param_dtype
    else:
        kind = m.param_dtype
    mean = 1.0 if name.endswith("_g") else 0.0
    return normal(seed, tid, shape, m.init_std, mean=mean, kind=kind, out=out)


def layer_field_names(m: ModelShape) -> tuple:
    names = ["ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_dense", "b_dense", "ln2_g", "ln2_b",
             "w_up", "b_up", "w_down", "b_down"]
    if m.weight_dtype == "int8":
        names += ["s_qkv", "s_dense", "s_up", "s_down"]
    return tuple(names)


def global_field_names(m: ModelShape) -> tuple:
    names = ["embed", "lnf_g", "lnf_b"]
    if m.embed_ln:
        names += ["emb_ln_g", "emb_ln_b"]
    return tuple(names)


def model_tensors(m: ModelShape, seed: int = SEED_WEIGHTS,
                  layers: Optional[Iterable[int]] = None) -> dict:
    """All tensors of a (possibly truncated) model in storage form.

    Returns {'embed': ..., 'lnf_g': ..., ..., 'layers': [ {field: array}, ... ]}.
    """
    layers = range(m.n_layer) if layers is None else layers
    out = {name: tensor(m, name, seed=seed) for name in global_field_names(m)}
    out["layers"] = [{f: tensor(m, f, l, seed=seed) for f in layer_field_names(m)}
                     for l in layers]
    return out


def prompts(m: ModelShape, batch: int, prompt_len: int, valid_lens=None,
            seed: int = SEED_PROMPTS, pad_id: int = 0) -> tuple:
    """Left-padded random prompts: (ids int32 [batch, prompt_len], valid_len int32 [batch])."""
    tok = ids(seed, 0, (batch, prompt_len), 0, m.vocab)
    if valid_lens is None:
        valid = np.full((batch,), prompt_len, dtype=np.int32)
    else:
        valid = np.asarray(valid_lens, dtype=np.int32).reshape(batch)
    for b in range(batch):
        tok[b, : prompt_len - valid[b]] = pad_id
    return tok, valid


def softmax_inputs(w: SoftmaxWorkload = SOFTMAX, std: Optional[float] = None,
                   seed_scores: int = SEED_SCORES, seed_lengths: int = SEED_LENGTHS) -> tuple:
    """bf16 score bits [B, H, Q, K] ~ N(0, std) and valid lengths uniform in [min_valid, K]."""
    std = w.score_std if std is None else std
    scores = normal(seed_scores, 0, (w.batch, w.heads, w.q_len, w.kv_len), std, kind="bf16")
    lengths = ids(seed_lengths, 0, (w.batch,), w.min_valid, w.kv_len - w.min_valid + 1)
    return scores, lengths


SEED_SAMPLING = 4


def sampling_inputs(batch: int, vocab: int, sigmas=(3.0, 4.0, 5.0, 6.0),
                    temperatures=(0.5, 0.8, 1.0, 1.3), top_ps=(0.3, 0.8, 0.9, 0.95, 1.0),
                    seed: int = SEED_SAMPLING) -> tuple:
    """Per-row sampling inputs: float32 logits [batch, vocab], row b ~ N(0, sigma_b^2)
    with sigma_b cycling through `sigmas` (peaked enough that the nucleus boundary and
    the draw sit well clear of float32 rounding for most rows), temperatures and top-p
    values cycling through the given lists (offset so the combinations mix), and one
    uniform number in [0, 1) per row."""
    logits = np.empty((batch, vocab), dtype=np.float32)
    for b in range(batch):
        normal(seed, 16 + b, (vocab,), sigmas[b % len(sigmas)], kind="f32", out=logits[b])
    T = np.array([temperatures[(b // len(sigmas)) % len(temperatures)] for b in range(batch)],
                 dtype=np.float32)
    P = np.array([top_ps[(b * 3 + 1) % len(top_ps)] for b in range(batch)], dtype=np.float32)
    u = (ids(seed, 15, (batch,), 0, 1 << 24).astype(np.float64) / float(1 << 24)).astype(np.float32)
    return logits, T, P, u
