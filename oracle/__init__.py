"""CPU oracle for BLOOM greedy KV-cached decoding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this package: only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
use it.  It shares no code with the HIP library (``transformer_bloom_decode_amd``).

Every function is pinned by tests against things other than itself (the Hugging
Face ``transformers`` BLOOM implementation run in float64, closed forms, special
cases that reduce to textbook routines, invariants); see ``tests/test_oracle_*.py``.
"""
from .bloom_oracle import (  # noqa: F401
    Int8RowScale,
    OracleModel,
    alibi_masked_softmax,
    alibi_slopes,
    attention,
    decoder_layer,
    dequantize_int8,
    int8_rows,
    forward,
    gelu_tanh,
    greedy_argmax,
    greedy_generate,
    layer_from_storage,
    layer_norm,
    linear,
    lm_logits,
    masked_softmax,
    new_cache,
    quantize_int8,
    round_bf16,
    sample_tokens,
    stop_rule,
)
