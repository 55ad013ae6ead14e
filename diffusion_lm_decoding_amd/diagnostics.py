"""Cache-staleness sweep over a decode (reading notes sec. 14 and Algorithm 4,
steps 4-5): before every denoising step, dllm_staleness compares the cached
and the fresh evaluation of the block and the cached K/V against fresh ones;
the records are grouped by cache age (steps since the last refresh).

The decode itself is unchanged by the probes (the library restores the cache
after each).  Summary statistics are host-side analysis of the returned
arrays.

    python -m diffusion_lm_decoding_amd.diagnostics --workload llada8b_p512_g256 --blocks 2
"""
from __future__ import annotations

import argparse
import json
import sys
import time
from collections import defaultdict

import numpy as np


def staleness_sweep(eng, cv, cfg, blocks=None):
    """Decode `cv` block by block (DualCache / PrefixCache: refresh at each
    block start) and probe before every step.  Returns one record per step:
    block, age, agreement of cached and fresh argmax over the masked rows,
    mean / max |c_cached - c_fresh|, and per-layer mean K and V cosines over
    the cached positions (outside the block) and inside the block."""
    mask_id = eng.shape.mask_id
    P, B = cfg.prompt_len, cfg.block_len
    nb = cfg.gen_len // B
    eng.begin(cv, cfg)
    recs = []
    for j in range(nb if blocks is None else min(blocks, nb)):
        eng.refresh(cv, cfg, 0)
        s, e = P + j * B, P + (j + 1) * B
        age = 0
        while (cv.tokens[:, s:e] == mask_id).any().item():
            t0 = time.perf_counter()
            g = eng.staleness(cv, cfg, j)
            ms = 1e3 * (time.perf_counter() - t0)
            g = {k: v.cpu().numpy() for k, v in g.items()}
            live = g["tok_cached"] >= 0
            kc, vc = g["k_cos"], g["v_cos"]            # [layers, batch, N]
            inside = np.zeros(kc.shape[-1], bool)
            inside[s:e] = True
            recs.append({
                "block": j, "age": age, "masked": int(live.sum()),
                "argmax_agree": float((g["tok_cached"][live] == g["tok_fresh"][live]).mean()),
                "conf_shift_mean": float(np.abs(g["conf_cached"][live] - g["conf_fresh"][live]).mean()),
                "conf_shift_max": float(np.abs(g["conf_cached"][live] - g["conf_fresh"][live]).max()),
                "k_cos_cached_by_layer": kc[:, :, ~inside].mean(axis=(1, 2)).tolist(),
                "v_cos_cached_by_layer": vc[:, :, ~inside].mean(axis=(1, 2)).tolist(),
                "k_cos_block_by_layer": kc[:, :, inside].mean(axis=(1, 2)).tolist(),
                "probe_ms": ms,
            })
            eng.step(cv, cfg, j)
            age += 1
    return recs


def by_age(recs):
    """Mean of each scalar statistic over records of equal cache age."""
    groups = defaultdict(list)
    for r in recs:
        groups[r["age"]].append(r)
    out = []
    for age in sorted(groups):
        g = groups[age]
        out.append({"age": age, "n": len(g),
                    "argmax_agree": float(np.mean([r["argmax_agree"] for r in g])),
                    "conf_shift_mean": float(np.mean([r["conf_shift_mean"] for r in g])),
                    "k_cos_cached_min_layer": float(np.mean([min(r["k_cos_cached_by_layer"]) for r in g])),
                    "k_cos_cached_mean": float(np.mean([np.mean(r["k_cos_cached_by_layer"]) for r in g])),
                    "v_cos_cached_mean": float(np.mean([np.mean(r["v_cos_cached_by_layer"]) for r in g]))})
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llada8b_p512_g256")
    ap.add_argument("--blocks", type=int, default=2)
    ap.add_argument("--cache", default="dual")
    ap.add_argument("--alpha-max", type=float, default=0.0, help="override the workload's alpha_max")
    args = ap.parse_args(argv)
    from workloads import gen_bias, gen_prompt, gen_tensor, workload

    from .engine import Engine
    w = workload(args.workload, cache=args.cache)
    shape = w.model
    eng = Engine(shape, lambda n: gen_tensor(shape, n, w.weight_seed), max_batch=w.batch, max_seq=w.seq_len)
    prompt = gen_prompt(shape, w.batch, w.prompt_len, w.prompt_seed)
    target, alpha = gen_bias(shape, w.batch, w.gen_len, w.bias_seed, args.alpha_max or w.alpha_max)
    cv = eng.canvas(prompt, target, alpha, w.gen_len)
    recs = staleness_sweep(eng, cv, Engine.cfg_from_workload(w), blocks=args.blocks)
    for row in by_age(recs):
        print(json.dumps(row), flush=True)
    print(json.dumps({"workload": w.name, "cache": args.cache, "steps_probed": len(recs),
                      "probe_ms_mean": float(np.mean([r["probe_ms"] for r in recs]))}), flush=True)
    eng.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
