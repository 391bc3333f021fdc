"""Build a Hugging Face ``transformers`` BLOOM model (float64, CPU) from generated tensors.

Used only as an independent library implementation that pins the CPU oracle.  The
tensors are widened with the input module's own helpers, not the oracle's.
"""
import numpy as np
import torch

import bloom_inputs as bi


def _val(a, storage):
    a = np.asarray(a)
    if storage == "bf16":
        return bi.bf16_to_f32(a).astype(np.float64)
    if storage == "f16":
        return bi.f16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def weight_values(shape, lw, field):
    """Dense float64 value of one linear's weight (int8 weights dequantised per row)."""
    if shape.weight_dtype == "int8":
        return _val(lw["s_" + field], "f16")[:, None] * lw["w_" + field].astype(np.float64)
    return _val(lw["w_" + field], shape.weight_dtype)


def hf_bloom(shape, tensors):
    from transformers import BloomConfig, BloomForCausalLM

    assert shape.ffn == 4 * shape.hidden and shape.n_head_local == shape.n_head_total
    assert shape.embed_ln, "the HF model always has the embedding LayerNorm"
    cfg = BloomConfig(vocab_size=shape.vocab, hidden_size=shape.hidden, n_layer=len(tensors["layers"]),
                      n_head=shape.n_head_total, layer_norm_epsilon=shape.ln_eps,
                      bos_token_id=None, eos_token_id=None, pad_token_id=0)
    torch.manual_seed(0)
    model = BloomForCausalLM(cfg).to(torch.float64).eval()
    pd = shape.param_dtype
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    sd = {
        "transformer.word_embeddings.weight": t(_val(tensors["embed"], pd)),
        "transformer.word_embeddings_layernorm.weight": t(_val(tensors["emb_ln_g"], pd)),
        "transformer.word_embeddings_layernorm.bias": t(_val(tensors["emb_ln_b"], pd)),
        "transformer.ln_f.weight": t(_val(tensors["lnf_g"], pd)),
        "transformer.ln_f.bias": t(_val(tensors["lnf_b"], pd)),
    }
    names = {"qkv": "self_attention.query_key_value", "dense": "self_attention.dense",
             "up": "mlp.dense_h_to_4h", "down": "mlp.dense_4h_to_h"}
    for l, lw in enumerate(tensors["layers"]):
        p = f"transformer.h.{l}."
        sd[p + "input_layernorm.weight"] = t(_val(lw["ln1_g"], pd))
        sd[p + "input_layernorm.bias"] = t(_val(lw["ln1_b"], pd))
        sd[p + "post_attention_layernorm.weight"] = t(_val(lw["ln2_g"], pd))
        sd[p + "post_attention_layernorm.bias"] = t(_val(lw["ln2_b"], pd))
        for f, n in names.items():
            sd[p + n + ".weight"] = t(weight_values(shape, lw, f))
            sd[p + n + ".bias"] = t(_val(lw["b_" + f], pd))
    missing, unexpected = model.load_state_dict(sd, strict=False)
    assert not unexpected, unexpected
    assert all(m == "lm_head.weight" for m in missing), missing
    model.tie_weights()
    assert torch.equal(model.lm_head.weight, model.transformer.word_embeddings.weight)
    model.generation_config.eos_token_id = None
    model.generation_config.bos_token_id = None
    model.generation_config.pad_token_id = 0
    return model


def hf_hidden(model, ids, valid_len):
    """Final-LayerNorm hidden states [B, S, h] for left-padded ids."""
    B, S = ids.shape
    mask = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        mask[b, S - valid_len[b]:] = 1
    with torch.no_grad():
        out = model.transformer(input_ids=torch.from_numpy(ids.astype(np.int64)),
                                attention_mask=torch.from_numpy(mask))
    return out.last_hidden_state.numpy()


def hf_generate(model, ids, valid_len, n_new):
    B, S = ids.shape
    mask = np.zeros((B, S), dtype=np.int64)
    for b in range(B):
        mask[b, S - valid_len[b]:] = 1
    with torch.no_grad():
        out = model.generate(input_ids=torch.from_numpy(ids.astype(np.int64)),
                             attention_mask=torch.from_numpy(mask), max_new_tokens=n_new,
                             min_new_tokens=n_new, do_sample=False, num_beams=1,
                             use_cache=True)
    return out[:, S:].numpy()
