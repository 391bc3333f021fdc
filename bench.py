#!/usr/bin/env python3
"""ms/token of BLOOM greedy KV-cached generation on one MI355X.

The metric is the pages' (ms/token = wall time / (batch x tokens); "Incredibly Fast
BLOOM Inference with DeepSpeed and Accelerate", Benchmark Environment): greedy
generation of 100 new tokens from a 16-token prompt with the KV cache on.  One
"step" is one whole generation for the batch: bloom_prefill, then 99
bloom_decode_step calls.  Default workload: one tensor-parallel rank's share of the
BLOOM-176B layer stack (70 layers, hidden 14336, 14 of 112 heads, MLP share 7168,
bf16) with the full 250880-token tied LM head, batch 1.  Weights are random
(seeded), inputs synthetic; everything is resident in HBM before timing starts.

Printed: one JSON line with the metric, the roofline of the dominant kernel (the
weight-streaming GEMV, timed per launch with HIP events on the library's stream in
one extra generation after the timed steps) and the CPU oracle timed on a bounded
sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, vendor peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (no sparsity)
MFMA_INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 matrix peak (W8A8 prompt passes)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3, help="timed generations")
    ap.add_argument("--warmup", type=int, default=1, help="untimed generations")
    ap.add_argument("--workload", default="bloom-176b-tp8-rank0",
                    help="a decode workload, 'softmax' for the standalone fused ALiBi + "
                         "masked softmax, or 'sample' for per-row top-p sampling (each its "
                         "own JSON line)")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--new-tokens", type=int, default=None)
    ap.add_argument("--no-ln-fold", action="store_true",
                    help="keep the LayerNorms of batch-1 steps as launches of their own "
                         "(by default bf16-weight batch-1 runs fold them into the QKV / "
                         "MLP-up GEMVs with bloom_ln_fold)")
    ap.add_argument("--prompt-len", type=int, default=None,
                    help="prompt tokens per row (default: the workload's; long prompts run "
                         "the decode attention split over the keys)")
    ap.add_argument("--layers", type=int, default=None, help="truncate the stack (development)")
    ap.add_argument("--act", choices=("f32", "f16", "bf16", "int8"), default=None,
                    help="activation type of bf16 / int8 models: float32, fp16, bf16, or int8 "
                         "(W8A8, int8 weights only) (default: fp16 for bf16 weights; bf16 for "
                         "the int8 model, whose configuration states bf16 activations)")
    ap.add_argument("--kv", choices=("auto", "f32", "f16", "bf16", "int8"), default="auto",
                    help="KV-cache type (auto: the activation type)")
    ap.add_argument("--loop", choices=("eager", "graph"), default="eager",
                    help="decode loop: one bloom_decode_step call per token, or bloom_generate "
                         "(replays of a captured decode step)")
    ap.add_argument("--sample", action="store_true",
                    help="with --loop graph: per-row sampling (temperature 0.8, top-p 0.9, "
                         "seeded uniform numbers) instead of greedy tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-kernel-timer", action="store_true",
                    help="do not time the linear-layer launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device-to-device copies of 1 GiB (a known-size stream "
                         "to scale hardware traffic counters against), then exit")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 5}), flush=True)


def device_weights(m, cfg, seed=0):
    """Allocate the model's tensors in HBM and fill them on the GPU with the seeded
    generator (bloom_init_weights; bitwise equal to the host generator of the tests)."""
    import torch

    import bloom_inputs as bi
    import transformer_bloom_decode_amd as tb

    dt = {"f32": torch.float32, "bf16": torch.int16, "int8": torch.int8}

    def buf(name):
        if name.startswith("s_"):
            return torch.empty(bi.tensor_shape(m, name), dtype=torch.int16, device="cuda")
        kind = m.weight_dtype if name.startswith("w_") else m.param_dtype
        return torch.empty(bi.tensor_shape(m, name), dtype=dt[kind], device="cuda")

    t0 = time.perf_counter()
    g = {name: buf(name) for name in bi.global_field_names(m)}
    layers = [{f: buf(f) for f in bi.layer_field_names(m)} for _ in range(m.n_layer)]
    dw = tb.DeviceWeights(g, layers)
    tb.bloom_init_weights(cfg, dw, seed=seed, sigma=m.init_std)
    torch.cuda.synchronize()
    log(f"  generated {m.n_layer} layers on the GPU ({time.perf_counter() - t0:.1f}s)")
    return dw


def kernel_source_digest():
    """Hash of the sources that define the batch-1 GEMV as launched: its kernel, planner
    and launcher (gemv.hip) and the fused epilogues it calls (common.hpp)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("gemv.hip", "common.hpp"):
        h.update(open(os.path.join(ROOT, "transformer_bloom_decode_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def counted_traffic(kernel, workload, batch):
    """HBM bytes per launch of `kernel` measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a plain-copy calibration), from the committed summary in profiles/; None
    when there is no summary for this kernel and workload or the kernel source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}_b{batch}_decode.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", "`")):
            k, _, v = line.partition(":")
            fields[k.strip()] = v.strip()
    if fields.get("kernel") != kernel or fields.get("source_sha256_16") != kernel_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def step_bytes(m, B, P, n_new):
    """Algorithmic HBM bytes of one decode step averaged over the generation: every
    weight byte once (layers + tied LM head + LayerNorm/bias/scales) plus the KV cache
    read (T keys and values per head) and the new key/value written."""
    act = m.kv_bytes
    weights = m.n_layer * m.layer_weight_bytes() + m.head_bytes()
    if m.embed_ln:
        weights += 2 * m.hidden * (4 if m.param_dtype == "f32" else 2)
    T_avg = sum(P + t for t in range(1, n_new)) / max(1, n_new - 1)  # keys seen per step
    kv_read = 2 * m.n_layer * B * m.n_head_local * T_avg * m.head_dim * act
    kv_write = 2 * m.n_layer * B * m.n_head_local * m.head_dim * act
    return weights + kv_read + kv_write, weights


def prefill_flops(m, B, P):
    """Flops of the prompt pass: the four linears on B*P rows, causal attention over P
    keys, and the LM head on the last position of each row."""
    params = m.qkv_rows * m.hidden + m.hidden * m.attn_width + 2 * m.ffn * m.hidden
    lin = 2.0 * B * P * m.n_layer * params
    attn = 4.0 * m.n_layer * B * m.n_head_local * m.head_dim * P * (P + 1) / 2
    head = 2.0 * B * m.vocab * m.hidden
    return lin + attn + head


def cpu_baseline(m, B, P, n_new, budget_s):
    """The CPU oracle, as it stands, on a bounded sample: a 2-layer full-width slice of
    the same model, its prompt pass and as many single-token steps as fit the budget;
    per-layer and LM-head times are scaled to the full stack and the full generation."""
    import numpy as np

    import bloom_inputs as bi
    import oracle
    from oracle import bloom_oracle as bo

    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in blas] or [1])
        blas_name = ", ".join(f"{i.get('internal_api')} {i.get('version')}" for i in blas)
    except Exception:  # pragma: no cover
        cores, blas_name = os.cpu_count() or 1, "unknown"
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    Ls = min(2, m.n_layer)
    ms = m.truncated(Ls)
    tensors = bi.model_tensors(ms)
    om = oracle.OracleModel.from_storage(ms, tensors)
    prompt, valid = bi.prompts(ms, B, P)
    pad = P - valid
    cache = oracle.new_cache(om, B)
    t0 = time.perf_counter()
    h = oracle.forward(om, prompt, 0, pad, cache)[:, -1]
    t_prompt_layers = time.perf_counter() - t0
    t0 = time.perf_counter()
    logits = bo.lm_logits(om, h)
    t_head = time.perf_counter() - t0
    nxt = bo.greedy_argmax(logits)
    steps, t_step_layers = 0, 0.0
    start = time.perf_counter()
    while steps < n_new - 1 and (time.perf_counter() - start) < budget_s * 0.5:
        t0 = time.perf_counter()
        h = oracle.forward(om, nxt[:, None], P + steps, pad, cache)[:, 0]
        t_step_layers += time.perf_counter() - t0
        t0 = time.perf_counter()
        nxt = bo.greedy_argmax(bo.lm_logits(om, h))
        t_head += time.perf_counter() - t0
        steps += 1
    per_layer_prompt = t_prompt_layers / Ls
    per_layer_step = t_step_layers / max(1, steps) / Ls
    per_head = t_head / (steps + 1)
    total_s = m.n_layer * (per_layer_prompt + (n_new - 1) * per_layer_step) + n_new * per_head
    return {
        "value": round(total_s * 1e3 / (B * n_new), 3),
        "unit": "ms/token",
        "cores": int(cores),
        "host_cpus_available": int(affinity),
        "cpu_model": cpu_model,
        "blas": blas_name,
        "kind": "oracle",
        "sample": (f"float64 numpy oracle on {Ls} of {m.n_layer} layers at full width, batch {B}: "
                   f"{P}-token prompt pass + {steps} single-token steps, each with the full "
                   f"{m.vocab}-row LM head; per-layer time x {m.n_layer} and LM-head time x "
                   f"{n_new} scaled to the {n_new}-token generation"),
    }


def softmax_bench(args):
    """Standalone alibi_masked_softmax on its workload shape (bf16 scores [32, 14, 1, 2048],
    left-pad valid lengths uniform in [64, 2048], fp32 probabilities): the kernel time on
    one resident buffer set (it fits the 256 MB MALL), and the rate over 80 rotating sets
    (> 350 MB, so the scores and probabilities come from and go to HBM)."""
    import numpy as np
    import torch

    import bloom_inputs as bi
    import transformer_bloom_decode_amd as tb

    w = bi.SOFTMAX
    scores, lengths = bi.softmax_inputs(w)
    B, H, Q, K = w.batch, w.heads, w.q_len, w.kv_len
    n_sets = 80
    s_dev = torch.from_numpy(scores.view(np.int16)).cuda()
    sets = [s_dev.clone() for _ in range(n_sets)]
    vl = torch.from_numpy(lengths.astype(np.int32)).cuda()
    outs = [torch.empty((B, H, Q, K), dtype=torch.float32, device="cuda") for _ in range(n_sets)]
    stream = torch.cuda.current_stream()
    # algorithmic bytes: the valid scores read, every probability written, the lengths
    valid_keys = int(np.minimum(lengths, K).sum()) * H * Q
    nbytes = valid_keys * 2 + B * H * Q * K * 4 + B * 4

    def call(i):
        tb.alibi_masked_softmax(sets[i], tb.BLOOM_BF16, vl, B, H, Q, K, w.n_head_total,
                                w.head_offset, outs[i], tb.BLOOM_F32, stream)

    def timed(reps, rotate):
        for i in range(3):
            call(i % n_sets if rotate else 0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i % n_sets if rotate else 0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    us_res = timed(400, False)
    us_rot = timed(400, True)
    out = {
        "metric": "fused ALiBi + masked softmax kernel time",
        "value": round(us_res, 2), "unit": "us", "higher_is_better": False,
        "n_gpus": 1, "dtype": "bf16 in, f32 softmax and out", "data": "synthetic",
        "config": {"workload": "alibi_masked_softmax", "batch": B, "heads": H, "q_len": Q,
                   "kv_len": K, "valid_len": f"uniform [{w.min_valid}, {K}]",
                   "score_std": w.score_std},
        "algorithmic_bytes": nbytes,
        "resident_gb_per_s": round(nbytes / (us_res * 1e-6) / 1e9, 1),
        "hbm_resident": {"sets": n_sets, "us": round(us_rot, 2),
                         "gb_per_s": round(nbytes / (us_rot * 1e-6) / 1e9, 1),
                         "frac": round(nbytes / (us_rot * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    print(json.dumps(out), flush=True)


def sample_bench(args):
    """bloom_sample_tokens on float32 logits [batch, 250880] (per-row temperature and
    top-p, one uniform number per row; seeded synthetic logits): time per call (its
    seven launches), and the oracle's time on the same rows.  The kernels read each row
    up to six times (max, mass, three radix levels, segment masses) from cache; the
    algorithmic traffic is one read of the logits."""
    import numpy as np
    import torch

    import bloom_inputs as bi
    import transformer_bloom_decode_amd as tb

    B, V = args.batch, 250880
    logits, T, P, u = bi.sampling_inputs(B, V)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    lg, Td, Pd, ud = d(logits), d(T), d(P), d(u)
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(tb.bloom_sample_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        tb.bloom_sample_tokens(lg, B, V, Td, Pd, ud, out, ws, stream)
    torch.cuda.synchronize()
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        tb.bloom_sample_tokens(lg, B, V, Td, Pd, ud, out, ws, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = B * V * 4 + B * 16
    res = {
        "metric": "per-row temperature + top-p sampling kernel time",
        "value": round(us, 2), "unit": "us", "higher_is_better": False, "n_gpus": 1,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "bloom_sample_tokens", "batch": B, "vocab": V,
                   "logit_std": "3-6 by row", "temperature": "0.5-1.3", "top_p": "0.3-1.0"},
        "algorithmic_bytes": nbytes,
        "gb_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        oracle.sample_tokens(logits, T, P, u)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "us", "cores": 1,
                               "kind": "oracle", "sample": f"the same {B} rows, float64 numpy"}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (no "
              "multi-GPU path is implemented: the library runs one GPU's share of the model).",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.workload == "sample":
        sample_bench(args)
        return
    if args.workload == "softmax":
        softmax_bench(args)
        return

    import numpy as np
    import torch

    import bloom_inputs as bi
    import transformer_bloom_decode_amd as tb

    import dataclasses
    wl = bi.WORKLOADS[args.workload]
    m = wl.model if args.layers is None else wl.model.truncated(args.layers)
    if m.weight_dtype != "f32":
        act = args.act or ("bf16" if m.weight_dtype == "int8" else "f16")
        m = dataclasses.replace(m, activations=act, kv_cache=args.kv)
    B = args.batch
    P = args.prompt_len or wl.prompt_len
    n_new = args.new_tokens or wl.new_tokens
    torch.cuda.set_device(0)

    t0 = time.perf_counter()
    cfg = tb.make_config(m)
    dw = device_weights(m, cfg)
    ln_fold = m.weight_dtype == "bf16" and B == 1 and not args.no_ln_fold
    if ln_fold:
        # LayerNorm fold vectors, computed once per model (used by one-row passes)
        dw.fold_layernorm(cfg)
        torch.cuda.synchronize()
    prompt, valid = bi.prompts(m, B, P)
    tok = torch.from_numpy(prompt).cuda()
    vl = torch.from_numpy(valid).cuda()
    kv = tb.KVCache(cfg, B, P + n_new)
    ws = tb.workspace(cfg, B, P)
    ids = torch.empty((n_new, B), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t0:.1f}s: {m.name} L={m.n_layer} B={B} P={P} new={n_new}")

    graph = args.loop == "graph"
    if args.sample and not graph:
        log("--sample needs --loop graph")
        sys.exit(2)
    smp = {}
    if args.sample:
        import numpy as np
        u = (bi.ids(bi.SEED_SAMPLING, 99, (n_new, B), 0, 1 << 24).astype(np.float64)
             / (1 << 24)).astype(np.float32)
        smp = dict(temperature=torch.full((B,), 0.8, device="cuda"),
                   top_p=torch.full((B,), 0.9, device="cuda"),
                   uniform=torch.from_numpy(u).cuda(),
                   logits=torch.empty((B, m.vocab), dtype=torch.float32, device="cuda"),
                   sample_ws=torch.empty(tb.bloom_sample_workspace_bytes(B, m.vocab),
                                         dtype=torch.uint8, device="cuda"))

    def generation(ev_mid=None, timed=False):
        kv.struct.len = 0
        kv.struct.prompt_len = 0
        if graph and not timed:
            tb.bloom_generate(cfg, dw, kv, B, P, tok, vl, n_new, ids, None, ws, stream, **smp)
            return
        if timed:
            tb.bloom_timer_pause(True)
        tb.bloom_prefill(cfg, dw, kv, B, P, tok, vl, ids[0], None, ws, stream)
        if ev_mid is not None:
            ev_mid.record(stream)
        if timed:
            tb.bloom_timer_pause(False)
        for t in range(1, n_new):
            tb.bloom_decode_step(cfg, dw, kv, B, ids[t - 1], vl, ids[t], None, ws, stream)

    for _ in range(args.warmup):
        generation()
    torch.cuda.synchronize()

    # timed region: K whole generations, no per-launch instrumentation
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        generation(None if graph else ev[k][1])
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gen_ms = [a.elapsed_time(c) for a, _, c in ev]
    if graph:
        # bloom_generate is one call: time its prompt pass on its own, outside the
        # timed region, and take the decode steps as the rest of each generation
        for k in range(K):
            kv.struct.len = kv.struct.prompt_len = 0
            ev[k][0].record(stream)
            tb.bloom_prefill(cfg, dw, kv, B, P, tok, vl, ids[0], None, ws, stream)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        prefill_ms = [a.elapsed_time(b) for a, b, _ in ev]
        decode_ms = [(g - p) / (n_new - 1) for g, p in zip(gen_ms, prefill_ms)]
    else:
        prefill_ms = [a.elapsed_time(b) for a, b, _ in ev]
        decode_ms = [b.elapsed_time(c) / (n_new - 1) for _, b, c in ev]

    ms_per_step = wall * 1e3 / K
    ms_per_token = ms_per_step / (B * n_new)
    sb, wbytes = step_bytes(m, B, P, n_new)
    dec_step_ms = float(np.median(decode_ms))

    # kernel pass: one more identical generation whose decode-step GEMV launches are
    # bracketed by HIP events on the library's stream (the events themselves cost a few
    # percent, so this pass is kept out of the timed region above)
    roofline = None
    kernels = {}
    if not args.no_kernel_timer:
        launches_per_gen = (n_new - 1) * (4 * m.n_layer + 1 + (B - 1) // 128)
        tb.bloom_timer_enable(launches_per_gen)
        generation(timed=True)
        for cls, name in tb.KERNEL_CLASSES.items():
            k_ms, k_n, k_bytes = tb.bloom_timer_read(cls)
            if k_n:
                kernels[name] = {"launches": k_n, "total_ms": round(k_ms, 3),
                                 "avg_launch_us": round(k_ms * 1e3 / k_n, 2),
                                 "gb_per_s": round(k_bytes / (k_ms * 1e-3) / 1e9, 1),
                                 "bytes_per_launch": round(k_bytes / k_n)}
        tb.bloom_timer_disable()
        if kernels:
            # the dominant kernel: largest share of the decode-step time
            name = max(kernels, key=lambda k: kernels[k]["total_ms"])
            kd = kernels[name]
            achieved = kd["gb_per_s"]
            roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": counted_traffic(name, m.name, B), "kernel": name,
                        "launches": kd["launches"],
                        "avg_launch_us": kd["avg_launch_us"],
                        "bytes_per_launch": kd["bytes_per_launch"]}
    ids_host = ids.cpu().numpy()

    out = {
        "metric": "ms/token (wall/(batch*tokens)), BLOOM-176B-shape greedy decode",
        "value": round(ms_per_token, 4),
        "unit": "ms/token",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (f"{m.weight_dtype} weights, {m.act_dtype} activations, {m.kv_dtype} KV"
                  if m.weight_dtype != "f32" else "f32"),
        "data": "synthetic (seeded random weights and prompt ids)",
        "config": {"workload": m.name, "batch": B, "prompt_len": P, "new_tokens": n_new,
                   "layers": m.n_layer, "hidden": m.hidden, "heads_local": m.n_head_local,
                   "heads_total": m.n_head_total, "ffn_local": m.ffn, "vocab": m.vocab,
                   "weights": m.weight_dtype, "activations": m.act_dtype,
                   "kv_cache": m.kv_dtype, "ln_fold": ln_fold, "greedy": not args.sample,
                   "parallelism": "none (1 GPU)", "loop": args.loop,
                   "tokens": "sampled (temperature 0.8, top-p 0.9)" if args.sample else "greedy"},
        "tokens_per_s": round(B * n_new / (ms_per_step * 1e-3), 2),
        "prefill_ms": round(float(np.median(prefill_ms)), 3),
        "prefill_tflops": round(prefill_flops(m, B, P) / (float(np.median(prefill_ms)) * 1e-3)
                                / 1e12, 1),
        "prefill_mfma_frac": round(prefill_flops(m, B, P) / (float(np.median(prefill_ms)) * 1e-3)
                                   / 1e12 / (MFMA_INT8_PEAK_TOPS if m.act_dtype == "int8"
                                             else MFMA_BF16_PEAK_TFLOPS), 4),
        "decode_step_ms": round(dec_step_ms, 4),
        "decode_step_gb": round(sb / 1e9, 3),
        "decode_step_hbm_frac": round(sb / (dec_step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "event_ms_per_step": round(float(np.median(gen_ms)), 3),
        "roofline": roofline,
        "decode_kernels": kernels,
        "checksum_ids": int(ids_host.astype(np.int64).sum()),
    }
    if not args.no_cpu_baseline:
        del dw, kv, ws
        torch.cuda.empty_cache()
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(m, B, P, n_new, args.cpu_budget_s)
        log(f"cpu baseline {time.perf_counter() - t0:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
