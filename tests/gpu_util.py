"""Helpers shared by the GPU parity tests: upload generated weights, run the HIP
generation loop, and compare with the CPU oracle teacher-forced.

Acceptance rule for greedy ids (the pages ask for greedy, do_sample=False, decoding;
a bf16 path cannot reproduce an fp64 argmax when two logits are closer than its own
rounding): the oracle replays the GPU's tokens (teacher forcing); at every step the
GPU's token must have an oracle logit within delta of the oracle's best, with
delta = 3 * tol * RMS(oracle logits row); steps where it is not the oracle's own
argmax are counted and reported.  The fp32 model must match free-running, exactly.
"""
import dataclasses

import numpy as np
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb


@dataclasses.dataclass
class GpuRun:
    ids: np.ndarray      # [B, n_new]
    hidden: np.ndarray   # [n_new, B, h]
    kv: object
    cfg: object


def upload(shape, seed=0):
    T = bi.model_tensors(shape, seed=seed)
    return T, tb.DeviceWeights.from_arrays(T), tb.make_config(shape)


def run_gpu(cfg, dw, prompt, valid, n_new, kv_fill=float("nan"), max_len=None):
    B, P = prompt.shape
    kv = tb.KVCache(cfg, B, max_len or (P + n_new), fill=kv_fill)
    ws = tb.workspace(cfg, B, P)
    tok = torch.from_numpy(np.ascontiguousarray(prompt, dtype=np.int32)).cuda()
    vl = torch.from_numpy(np.ascontiguousarray(valid, dtype=np.int32)).cuda()
    ids, hid = tb.greedy_generate(cfg, dw, kv, tok, vl, n_new, ws)
    torch.cuda.synchronize()
    return GpuRun(ids.cpu().numpy().T.copy(), hid.cpu().numpy(), kv, cfg)


@dataclasses.dataclass
class Verdict:
    hidden_rel: float
    tokens_ok: bool
    exact_frac: float
    near_ties: int
    oracle: object


def compare(shape, tensors, prompt, valid, run: GpuRun, tol_logit: float, widen_embed=False,
            rows=None):
    """Teacher-forced comparison of a GPU run with the oracle.  rows (optional): the
    batch rows to compare; the sequences of a batch never interact (each attends to its
    own keys only), so the oracle runs on those rows alone while the GPU ran the whole
    batch with the kernels of its size."""
    om = oracle.OracleModel.from_storage(shape, tensors)
    if widen_embed:
        om.embed = np.asarray(om.embed, dtype=np.float64)
    ids, hidden = run.ids, run.hidden
    if rows is not None:
        rows = np.asarray(rows)
        prompt, valid = np.asarray(prompt)[rows], np.asarray(valid)[rows]
        ids, hidden = ids[rows], hidden[:, rows]
    n_new = ids.shape[1]
    res = oracle.greedy_generate(om, prompt, valid, n_new, forced=ids)
    rel = float(np.linalg.norm(hidden - res.hidden) / np.linalg.norm(res.hidden))
    delta = 3.0 * tol_logit * res.rms
    ok = bool(np.all(res.chosen >= res.top1 - delta))
    exact = ids == res.tokens
    return Verdict(rel, ok, float(exact.mean()), int((~exact).sum()), res)


def kv_numpy(kv, layer):
    k = kv.k[layer].float().cpu().numpy()
    v = kv.v[layer].float().cpu().numpy()
    return k, v
