"""Decision noise of W8A8 (int8 activations with one scale per row, int8 KV cache with one
scale per row, head and slot) on the 176B int8 model: how far the oracle itself moves
when every value it quantises is perturbed by a relative N(0, (2^-23)^2), about one
float32 rounding.  Each quantisation rounds to a grid of amax / 127; a perturbation that
moves a value across a rounding boundary changes its code by one step, and that change
reaches every later layer.  Two correct float32 implementations differ by roundings of
this size, so their hidden states differ by about this much; the W8A8 GPU parity test
takes its bound from the largest value found here.

Calls only the oracle and the input generators.  Writes w8a8_decision_noise.json:
  python tests/golden/w8a8_decision_noise.py [--layers 2] [--seeds 4] [--rows 4]
"""
import argparse
import dataclasses
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import bloom_inputs as bi  # noqa: E402
import oracle  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--layers", type=int, default=2)
    ap.add_argument("--seeds", type=int, default=4)
    ap.add_argument("--rows", type=int, default=4, help="rows of the batch-16 prompts")
    ap.add_argument("--new", type=int, default=3)
    ap.add_argument("--rel", type=float, default=2.0 ** -23)
    args = ap.parse_args()
    m = dataclasses.replace(bi.BLOOM_176B_INT8.truncated(args.layers), activations="int8",
                            kv_cache="int8")
    T = bi.model_tensors(m, seed=0)
    prompt, valid = bi.prompts(m, 16, 16)
    prompt, valid = prompt[: args.rows], valid[: args.rows]
    om = oracle.OracleModel.from_storage(m, T, widen_weights=False)
    ref = oracle.greedy_generate(om, prompt, valid, args.new)
    exact_act, exact_kv = om.act_round, om.kv_round
    runs = []
    for s in range(args.seeds):
        rng = np.random.default_rng(1000 + s)

        def perturbed(f):
            return lambda a: f(np.asarray(a) * (1.0 + args.rel * rng.standard_normal(np.shape(a))))

        om.act_round, om.kv_round = perturbed(exact_act), perturbed(exact_kv)
        res = oracle.greedy_generate(om, prompt, valid, args.new, forced=ref.tokens)
        # relative L2 distance of the final hidden states per row, over all steps
        per_row = [float(np.linalg.norm(res.hidden[:, b] - ref.hidden[:, b])
                         / np.linalg.norm(ref.hidden[:, b])) for b in range(args.rows)]
        runs.append({"seed": 1000 + s, "hidden_rel_per_row": per_row})
        print(f"seed {1000 + s}: {['%.2e' % v for v in per_row]}", flush=True)
    out = {"model": m.name, "layers": args.layers, "prompt_rows": args.rows,
           "new_tokens": args.new, "perturbation_rel": args.rel, "runs": runs,
           "max_hidden_rel": max(max(r["hidden_rel_per_row"]) for r in runs)}
    with open(os.path.join(HERE, "w8a8_decision_noise.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("max", out["max_hidden_rel"])


if __name__ == "__main__":
    main()
