"""Benchmark: committed tokens/s of block-wise masked-diffusion decoding on one
MI355X (LLaDA-8B-shaped random model, DualCache, block 32, tau 0.9).

One timed "step" is one whole dllm_decode of the workload: every block's
cache refresh (whose whole-canvas forward also evaluates the block's first
denoising step), every other denoising step (block forward, LM-head reduce,
select/commit) and the per-step readback.  Inputs (weights, prompt, planted
bias) are synthetic and already resident in HBM when timing starts.

Prints one JSON line.  `roofline` is computed for the kernel class with the
largest device time in the denoising steps, from the library's algorithmic
byte/flop counts and the HIP-event durations of that class's launches inside
the timed region (events on the library's stream, on every 31st launch of the
class: 31 is coprime to the 32 layers, so the sample rotates over them, and
the events' own few-microsecond cost stays out of the throughput).  `cpu_baseline` times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TIMED_SAMPLE_EVERY = 31
# HBM bytes per launch of the dominant kernel from two rocprofv3 --pmc runs
# (FETCH_SIZE, WRITE_SIZE, calibrated on a copy of known size), valid only
# while the kernel sources hash to the value recorded with them
TRAFFIC_PROFILES = {("llada8b_p512_g256", "gateup"): "profiles/gateup_projection_llada8b_p512_g256.md"}
# dense MFMA peaks (TFLOP/s): fp16/bf16 inputs, fp32 inputs
PEAKS_TFLOPS = {"f16": 2500.0, "f32": 157.3}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--workload", default="llada8b_p512_g256")
    p.add_argument("--batch", type=int, default=0, help="override the workload batch")
    p.add_argument("--cache", default="", help="override the cache mode")
    p.add_argument("--rule", default="", help="override the rule")
    p.add_argument("--factor", type=float, default=0.0, help="override the factor-rule f")
    p.add_argument("--k", type=int, default=0, help="override the tokens per step of the top-k rule")
    p.add_argument("--cpu-steps", type=int, default=8, help="oracle denoising steps timed for cpu_baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-b16", action="store_true", help="skip the batch-16 projection MFMA-fraction measurement")
    p.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak microkernels")
    p.add_argument("--probe", type=int, default=0, metavar="STEPS",
                   help="counter-collection mode: one cache pass, STEPS denoising steps of block 0 and a "
                        "copy of COPY_MIB MiB (read once, written once) that calibrates the byte counters; "
                        "prints one JSON line describing what ran")
    return p.parse_args()


COPY_MIB = 256


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_table(title, prof):
    tot = sum(v["ms"] for v in prof.values()) or 1.0
    log(f"[bench] {title}: {tot:.1f} ms of timed kernels")
    for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["ms"]):
        if v["launches"]:
            ms = max(v["ms"], 1e-9)
            log(f"[bench]   {k:8s} {v['launches']:6d} launches {v['ms']:9.2f} ms ({100 * v['ms'] / tot:5.1f}%) "
                f"{1e3 * v['ms'] / v['launches']:8.1f} us/launch {v['bytes'] / ms / 1e6:8.1f} GB/s "
                f"{v['flops'] / ms / 1e9:8.1f} TFLOP/s")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library runs the "
              f"decoding path on a single GPU (batch rows or heads would be split across GPUs, one "
              f"process each, but no multi-GPU path is implemented).", file=sys.stderr)
        sys.exit(2)
    import torch

    from diffusion_lm_decoding_amd import _lib as L
    from diffusion_lm_decoding_amd.engine import Engine
    from workloads import gen_bias, gen_prompt, gen_tensor, workload

    over = {k: v for k, v in (("batch", args.batch), ("cache", args.cache), ("rule", args.rule),
                              ("factor", args.factor), ("k", args.k)) if v}
    w = workload(args.workload, **over)
    shape = w.model
    dev = torch.device("cuda:0")
    t0 = time.time()
    host_weights = {}

    def get(name):
        a = gen_tensor(shape, name, w.weight_seed)
        if not args.no_cpu_baseline:
            host_weights[name] = a
        return a

    peaks = None
    if not args.no_peaks and not args.probe:
        hbm, mfma = L.dllm_probe_peaks(8 << 30)
        peaks = {"hbm_gbs": hbm, "mfma_f16_tflops": mfma,
                 "how": "library microkernels: streaming read of 8 GiB; 32x32x16 fp16 MFMA chains from registers"}
        if shape.name == "llada8b":
            # one cold streaming read of each step projection's weight bytes: the ceiling of a kernel that
            # reads them once, launch ramp and drain included
            d, f, v = shape.d_model, shape.d_ffn, shape.vocab
            sizes = {"gateup": 2 * 2 * f * d, "qkv": 2 * 3 * d * d, "down": 2 * d * f, "oproj": 2 * d * d,
                     "lmhead": 2 * v * d}
            peaks["read_gbs_at_weight_bytes"] = {k: L.dllm_probe_read(b) for k, b in sizes.items()}
            peaks["read_bytes"] = sizes
        # what a large-M projection's main loop leaves of the MFMA rate: the same MFMA stream with the LDS
        # reads (8 KiB per 16 MFMAs: a 128x128 wave tile) and DMA copies into LDS (4 KiB per wave per 16
        # MFMAs: a 256x256 workgroup tile; 2: half of that) beside it, at one and two waves per SIMD
        mix = {}
        for wps in (1, 2):
            for name, rd, dm in (("mfma", 0, 0), ("lds_reads", 8, 0), ("copies", 0, 4), ("reads_and_copies", 8, 4),
                                 ("reads_and_half_copies", 8, 2)):
                mix[f"{wps}_wave_per_simd_{name}"] = L.dllm_probe_mfma_mix(wps, rd, dm)
        peaks["mfma_tflops_beside_lds_traffic"] = mix
        log(f"[bench] achievable: HBM read {hbm:.0f} GB/s, fp16 MFMA {mfma:.0f} TFLOP/s; streaming read at the "
            f"projections' weight bytes: {peaks.get('read_gbs_at_weight_bytes')}; MFMA TFLOP/s beside LDS "
            f"reads / copies: {', '.join(f'{k} {v:.0f}' for k, v in mix.items())}")
    b16 = None if (args.no_b16 or args.probe) else workload("llada8b_p128_g128")
    max_batch = max(w.batch, b16.batch if b16 else 0)
    max_seq = max(w.seq_len, b16.seq_len if b16 else 0)
    eng = Engine(shape, get, max_batch=max_batch, max_seq=max_seq, device="cuda:0")
    log(f"[bench] weights generated and packed in {time.time() - t0:.1f} s")
    prompt = gen_prompt(shape, w.batch, w.prompt_len, w.prompt_seed)
    target, alpha = gen_bias(shape, w.batch, w.gen_len, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    if args.probe:
        probe(eng, w, prompt, target, alpha, args.probe, dev)
        return
    canvases = [eng.canvas(prompt, target, alpha, w.gen_len) for _ in range(args.warmup + args.steps)]

    # warmup; the warmup decodes also time every kernel class
    L.dllm_set_timing(eng.ctx, L.KERNEL_CLASSES)
    for i in range(args.warmup):
        st = eng.decode(canvases[i], cfg)
        log(f"[bench] warmup {i}: {st.steps} steps, {st.committed} tokens, {st.ms_total:.1f} ms "
            f"(refresh {st.ms_refresh:.1f} ms)")
    prof = L.dllm_get_timing(eng.ctx, reset=True)
    kernel_table("denoising-step kernels (warmup)", prof["step"])
    kernel_table("cache-pass kernels (warmup)", prof["cache"])
    dom = max(prof["step"], key=lambda k: prof["step"][k]["ms"])

    # timed region: a rotating sample of the dominant class's launches is
    # bracketed by events
    L.dllm_set_timing(eng.ctx, [dom], TIMED_SAMPLE_EVERY)
    torch.cuda.synchronize(dev)
    t_start = time.perf_counter()
    stats = [eng.decode(canvases[args.warmup + i], cfg) for i in range(args.steps)]
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t_start
    L.dllm_set_timing(eng.ctx, [])
    kt = L.dllm_get_timing(eng.ctx, reset=True)["step"][dom]

    committed = sum(s.committed for s in stats)
    steps = sum(s.steps for s in stats)
    refresh_ms = sum(s.ms_refresh for s in stats)
    # under DualCache/PrefixCache the decode runs every refresh as the forward
    # of the step after it: those steps count as steps and their time as
    # refresh time, so the time per step from the cache leaves them out
    cached = w.cache in ("dual", "prefix")
    cache_steps = steps - sum(s.refreshes for s in stats) if cached else steps
    dtype = "f16" if shape.dtype == "bf16" else "f32"
    n = max(kt["launches"], 1)
    intensity = kt["flops"] / max(kt["bytes"], 1.0)
    ridge = PEAKS_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        roof = {"bound": "hbm", "achieved": kt["bytes"] / kt["ms"] / 1e6, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kt["flops"] / kt["ms"] / 1e9, "peak": PEAKS_TFLOPS[dtype],
                "unit": "TFLOP/s"}
    roof.update(frac=roof["achieved"] / roof["peak"], traffic=stored_traffic(w.name, dom),
                traffic_unit="HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                kernel=f"{dom} projection (denoising step)",
                launches=kt["launches"], sampled_every=TIMED_SAMPLE_EVERY, us_per_launch=1e3 * kt["ms"] / n,
                bytes_per_launch=kt["bytes"] / n, flops_per_launch=kt["flops"] / n)

    out = {
        "metric": "committed tokens/s, LLaDA-8B-shape DualCache B=32 tau=0.9; % of HBM/MFMA peak",
        "value": committed / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (counter-hash random weights, uniform random prompt, planted logit bias)",
        "config": {"workload": w.name, "batch": w.batch, "prompt_len": w.prompt_len, "gen_len": w.gen_len,
                   "block_len": w.block_len, "cache": w.cache, "rule": w.rule, "tau": w.tau,
                   **({"factor": w.factor} if w.rule == "factor" else {}),
                   **({"k": w.k} if w.rule == "topk" else {}),
                   "alpha_max": w.alpha_max, "weights": shape.dtype},
        "denoise_steps_per_s": steps / elapsed,
        "tokens_per_denoise_step": committed / max(steps, 1),
        "ms_per_denoise_step": (elapsed * 1e3 - refresh_ms) / max(cache_steps, 1),
        "steps_with_refresh_per_decode": (steps - cache_steps) / args.steps,
        "ms_refresh_per_decode": refresh_ms / args.steps,
        # eq. (15) of the reading notes: S C_active + R + T_selection (device time per decode)
        "cost_split_ms_per_decode": {"steps_forward": sum(s.ms_step for s in stats) / args.steps,
                                     "refresh": refresh_ms / args.steps,
                                     "selection": sum(s.ms_select for s in stats) / args.steps,
                                     "host": sum(s.ms_total - s.ms_step - s.ms_select - s.ms_refresh
                                                 for s in stats) / args.steps},
        "roofline": roof,
    }
    ms_step = (elapsed * 1e3 - refresh_ms) / max(cache_steps, 1)
    if shape.name == "llada8b" and w.batch == 1 and w.cache == "dual":
        # whole denoising step against HBM: weights (layers + LM head) read once,
        # the canvas's K/V read, the block's K/V written
        n_params = shape.n_layers * (4 * shape.d_model ** 2 + 3 * shape.d_model * shape.d_ffn) + \
            shape.vocab * shape.d_model
        kv_pos = 2 * shape.n_layers * shape.d_model * 2
        alg = 2 * n_params + kv_pos * w.seq_len + kv_pos * w.block_len
        out["step_hbm_fraction"] = {"value": alg / (HBM_PEAK_GBS * 1e9) / (ms_step / 1e3),
                                    "algorithmic_bytes": alg, "ms_per_step": ms_step, "peak_gbs": HBM_PEAK_GBS}
        if peaks:
            out["step_hbm_fraction"]["vs_achievable"] = alg / (peaks["hbm_gbs"] * 1e9) / (ms_step / 1e3)
    if peaks:
        out["achievable"] = peaks
        at = peaks.get("read_gbs_at_weight_bytes", {}).get(dom)
        if at and roof["unit"] == "GB/s":
            roof["frac_of_read_at_same_bytes"] = roof["achieved"] / at
    if b16 is not None:
        out["b16_projection_mfma_fraction"] = b16_projections(eng, b16, L)
    eng.close()
    del eng
    if b16 is not None and shape.name == "llada8b":
        out["b16_projection_mfma_fraction"]["library_yardstick"] = library_yardstick(shape)
    if not args.no_cpu_baseline:
        sample = cpu_baseline(shape, host_weights, w, prompt, target, alpha, args.cpu_steps)
        out["cpu_baseline"] = cpu_baseline_record(sample, w, steps / args.steps, committed / args.steps,
                                                  args.cpu_steps)
    print(json.dumps(out), flush=True)


def probe(eng, w, prompt, target, alpha, n_steps, dev):
    """A short, fixed sequence of launches for hardware-counter runs: the
    block-0 cache pass, n_steps denoising steps, then torch.neg over a
    float32 tensor of COPY_MIB MiB (a plain streaming kernel that reads and
    writes exactly that many bytes once each)."""
    import torch

    from diffusion_lm_decoding_amd.engine import Engine
    cfg = Engine.cfg_from_workload(w)
    cv = eng.canvas(prompt, target, alpha, w.gen_len)
    eng.refresh(cv, cfg, 0)
    for _ in range(n_steps):
        eng.step(cv, cfg, 0)
    n = COPY_MIB * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize(dev)
    torch.neg(src, out=dst)
    torch.cuda.synchronize(dev)
    print(json.dumps({"probe": w.name, "denoising_steps": n_steps, "copy_bytes_read": n * 4,
                      "copy_bytes_written": n * 4}), flush=True)
    eng.close()


def library_yardstick(shape, reps=10):
    """Context for the large-M projections: the vendor library's fp16 GEMM
    (torch.nn.functional.linear -> hipBLASLt, weights [out, in] as a
    projection stores them, fp32 accumulation, plain output, no fused
    epilogue) at the projections' shapes with 512 rows (batch-16 step) and 768
    rows (cache refresh), TFLOP/s from the best of `reps` timed calls with cold
    weights (two weight copies alternate)."""
    import torch
    import torch.nn.functional as F
    d, f = shape.d_model, shape.d_ffn
    out = {}
    for m in (512, 768):
        for name, n, k in (("qkv", 3 * d, d), ("oproj", d, d), ("gateup", 2 * f, d), ("down", d, f)):
            x = torch.randn(m, k, dtype=torch.float16, device="cuda")
            ws = [torch.randn(n, k, dtype=torch.float16, device="cuda") * 0.02 for _ in range(2)]
            F.linear(x, ws[0])
            torch.cuda.synchronize()
            best = 1e30
            for i in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                F.linear(x, ws[i % 2])
                e1.record()
                e1.synchronize()
                best = min(best, e0.elapsed_time(e1))
            out[f"{name}_m{m}"] = {"us": best * 1e3, "tflops": 2.0 * m * n * k / (best * 1e-3) / 1e12}
            del x, ws
    torch.cuda.empty_cache()
    log("[bench] library fp16 GEMM yardstick: " + ", ".join(f"{k} {v['us']:.0f} us ({v['tflops']:.0f} TF)"
                                                             for k, v in out.items()))
    return out


def b16_projections(eng, w, L, n_steps=3):
    """MFMA fraction of the batch-16 projection GEMMs: the projection flops of
    one denoising step (2 x rows x layer parameters) over their summed kernel
    time, against the dense fp16 peak.  Block 0 of the batch-16 DualCache
    workload, one refresh then n_steps steps."""
    from diffusion_lm_decoding_amd.engine import Engine
    from workloads import gen_bias, gen_prompt
    shape = w.model
    prompt = gen_prompt(shape, w.batch, w.prompt_len, w.prompt_seed)
    target, alpha = gen_bias(shape, w.batch, w.gen_len, w.bias_seed, w.alpha_max)
    cfg = Engine.cfg_from_workload(w)
    cv = eng.canvas(prompt, target, alpha, w.gen_len)
    eng.begin(cv, cfg)
    eng.refresh(cv, cfg, 0)
    gemms = ["qkv", "oproj", "gateup", "down"]
    L.dllm_get_timing(eng.ctx, reset=True)
    L.dllm_set_timing(eng.ctx, gemms)
    for _ in range(n_steps):
        eng.step(cv, cfg, 0)
    L.dllm_set_timing(eng.ctx, [])
    kt = L.dllm_get_timing(eng.ctx, reset=True)["step"]
    ms = sum(kt[g]["ms"] for g in gemms) / n_steps
    rows = w.batch * w.block_len
    flops = 2.0 * rows * shape.n_layers * (4 * shape.d_model ** 2 + 3 * shape.d_model * shape.d_ffn)
    frac = flops / (ms / 1e3) / (PEAKS_TFLOPS["f16"] * 1e12)
    log(f"[bench] batch-16 projections: {ms:.3f} ms per step, {flops / ms / 1e9:.0f} TFLOP/s, {100 * frac:.1f}% of peak")
    return {"value": frac, "flops_per_step": flops, "gemm_ms_per_step": ms, "peak_tflops": PEAKS_TFLOPS["f16"],
            "workload": w.name, "steps": n_steps}


def stored_traffic(workload, cls):
    """Measured HBM bytes per launch recorded for (workload, kernel class), or
    None when there is no record or the kernel sources changed since."""
    import hashlib
    rel = TRAFFIC_PROFILES.get((workload, cls))
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    fields = {}
    for line in open(os.path.join(ROOT, rel)):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in fields["sources"].split(","):
            with open(os.path.join(ROOT, f.strip()), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != fields["sources_sha256"]:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_baseline(shape, weights, w, prompt, target, alpha, n_steps):
    """The float64 oracle on a bounded sample of the workload, reported in the
    unit of `value`: one cache refresh over the whole canvas and n_steps
    DualCache denoising steps of block 0 (sequence 0) are timed, and the time
    of a whole decode is extrapolated as (blocks x refresh) + (denoising steps
    x step), with the step count the GPU decode took.  The weights are widened
    to float64 before timing."""
    import psutil
    from threadpoolctl import threadpool_info

    from oracle import OracleDecoder, OracleModel
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    om = OracleModel(shape, weights)
    om.materialize()
    dec = OracleDecoder(om, w.prompt_len, w.gen_len, w.block_len, cache=w.cache, rule=w.rule,
                        tau=w.tau, factor=w.factor, k=w.k)
    st = dec.new_state(prompt[0], target[0], alpha[0])
    t0 = time.perf_counter()
    dec.refresh(st)
    t_refresh = time.perf_counter() - t0
    t0 = time.perf_counter()
    committed = 0
    for _ in range(n_steps):
        committed += len(dec.step(st, 0).selected)
    t_step = (time.perf_counter() - t0) / n_steps
    return t_refresh, t_step, committed, threads, psutil.cpu_count(logical=False), psutil.cpu_count()


def cpu_baseline_record(sample, w, gpu_steps_per_decode, gpu_tokens_per_decode, n_steps):
    t_refresh, t_step, committed, threads, phys, logical = sample
    refreshes = w.n_blocks if w.cache in ("dual", "prefix") else 0
    decode_s = refreshes * t_refresh + gpu_steps_per_decode * t_step
    log(f"[bench] oracle: refresh {t_refresh:.1f} s, {n_steps} steps at {t_step:.2f} s each, "
        f"{threads} BLAS threads; whole decode ~{decode_s:.0f} s")
    return {"value": gpu_tokens_per_decode / decode_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 NumPy oracle on {w.name}, sequence 0: one refresh over all {w.seq_len} canvas "
                      f"positions ({t_refresh:.1f} s) and {n_steps} DualCache denoising steps of block 0 "
                      f"({t_step:.2f} s each); whole-decode time extrapolated as {refreshes} refreshes + "
                      f"{gpu_steps_per_decode:.0f} steps (the GPU decode's count)",
            "seconds_measured": t_refresh + n_steps * t_step, "extrapolated_decode_s": decode_s,
            "host_physical_cores": phys, "host_logical_cpus": logical}


if __name__ == "__main__":
    main()
